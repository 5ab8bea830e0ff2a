// Grouped Newton-Schulz GEMMs on gfx950 MFMA.
//
// One iteration of the odd polynomial X <- aX + (bA + cA^2)X, A = X X^T, on
// every matrix of an effective-shape group (the "several matrix products at
// parameter-update time" of page "きみはNanoGPT speedrunを知っているか？",
// section "おまけ"; the orthogonalisation itself is described in section
// "Muonとは").  Three grouped launches per iteration:
//   GRAM : A = alpha * X X^T             (alpha = s^2 on the first iteration)
//   POLY : B = b A + c A A               (skipped when c == 0)
//   APPLY: X' = scale * (a X + beta B X) (scale = s on the first iteration)
// where s = 1 / (||U||_F + eps) folds the Frobenius normalisation of the
// first iterate into the products.
//
// Tiling: square TS x TS output tiles, 256 threads as a 2 x 2 grid of waves,
// each wave (TS/2) x (TS/2) built from 32x32 MFMA blocks.  Every operand tile
// goes from global memory to LDS by buffer loads with the LDS-DMA bit (no
// register staging), two LDS stages, one barrier per K step.
//   * Operands whose contraction index is contiguous in memory (both GRAM
//     operands, both POLY operands, the B operand of APPLY) are stored as
//     128-byte rows of 16-byte chunks, the chunk index XOR-swizzled by the row
//     so that the 32 rows read by one MFMA operand load hit distinct banks.
//   * APPLY contracts over the rows of X, so its X tile is stored row-major
//     (contraction index = LDS row) and the bf16 MFMA operand is assembled by
//     the LDS transpose read (each 16-lane group turns a 4 x 16 block into four
//     consecutive contraction values per column).
// GRAM and POLY are symmetric: only tiles on or above the diagonal run, and
// off-diagonal tiles also store their mirror image.  The MFMA output layout
// gives each lane four consecutive rows of one column; the tiles are arranged
// so that those four values are contiguous in memory (row Q, columns P..P+3).
#include "muon_common.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

enum { GRAM = 0, POLY = 1, APPLY = 2 };

// Buffer descriptor word 3 for raw (untyped) loads.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

template <int XDT> struct Ty;
template <> struct Ty<kBF16> {
  using T = uint16_t;
  static constexpr int ES = 2;   // element bytes
  static constexpr int BK = 64;  // contraction elements per K step (128-byte rows)
};
template <> struct Ty<kF32> {
  using T = float;
  static constexpr int ES = 4;
  static constexpr int BK = 32;
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row << 7) + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four consecutive elements <-> floats.
__device__ __forceinline__ void ld4(const uint16_t* p, float* v) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void ld4(const float* p, float* v) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void st4(uint16_t* p, const float* v) {
  uint2 q;
  q.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
  q.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = q;
}
__device__ __forceinline__ void st4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st1(uint16_t* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }

// 1 / (sqrt(sum of the matrix's norm partials) + eps), same summation order in
// every block of the matrix.
// Summation order: 256-strided per-thread sums over the first four waves'
// lanes, then the butterfly, then the wave totals in order -- the same in
// every kernel and block size, so every block of a matrix gets the same s.
template <int NW>
__device__ __forceinline__ float matrix_scale(const float* partials, int count, float eps,
                                              float* red) {
  float acc = 0.f;
  if (threadIdx.x < 256)
    for (int i = threadIdx.x; i < count; i += 256) acc += partials[i];
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  const float s = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return 1.0f / (sqrtf(s) + eps);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, uint32_t voff,
                                      uint32_t soff) {
#if __HIP_DEVICE_COMPILE__   // the LDS-DMA builtin exists only in the device pass
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, soff, 0, 0);
#else
  (void)rs; (void)lds; (void)voff; (void)soff;
#endif
}

// Per-block load plan of one operand: buffer descriptor, per-lane offsets
// (fixed across K steps) and the uniform byte offset of the tile's origin.
struct OpLoad {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[2];
  uint32_t origin;     // bytes: first row of the tile (and first column for row-major X)
  uint32_t ld_bytes;
};

// K-contiguous operand: wave instruction j moves rows 8j..8j+7 (1 KiB); lane L
// fills physical chunk L & 7 of row 8j + L/8 with the logical chunk that the
// swizzle maps there.  Rows handled by one of NW waves are j = wave + NW u,
// whose low three bits take at most two values (wave, wave + NW).
template <int NW>
__device__ __forceinline__ void plan_kc(OpLoad& o, int lane, int wave) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int jl = (wave + NW * x) & 7;
    const int c = (lane & 7) ^ (((lane >> 3) ^ jl) & 7);
    o.voff[x] = static_cast<uint32_t>(lane >> 3) * o.ld_bytes + 16u * c;
  }
}

template <int TS, int NW>
__device__ __forceinline__ void load_kc(const OpLoad& o, uint32_t kbytes, int wave, uint8_t* dst) {
#pragma unroll
  for (int u = 0; u < TS / (8 * NW); ++u) {
    const int j = wave + NW * u;
    dma16(o.rs, dst + j * 1024, o.voff[NW < 8 ? (u & 1) : 0], o.origin + 8u * j * o.ld_bytes + kbytes);
  }
}

// Row-major X tile of APPLY: BK rows (contraction) of TS elements; instruction
// j moves RPI = 1024 / (TS * ES) rows; the 16-byte chunk index of row r is
// XOR-ed with 4 * (r & 1).
template <int TS, int ES>
__device__ __forceinline__ void plan_rm(OpLoad& o, int lane) {
  constexpr int RB = TS * ES, RPI = 1024 / RB, CPR = RB / 16;
  const int rr = lane / CPR, ch = lane % CPR;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int par = RPI > 1 ? (rr & 1) : p;    // row parity
    o.voff[p] = static_cast<uint32_t>(rr) * o.ld_bytes + 16u * (ch ^ (4 * par));
  }
}

template <int TS, int ES, int BK, int NW>
__device__ __forceinline__ void load_rm(const OpLoad& o, uint32_t k0, int wave, uint8_t* dst) {
  constexpr int RB = TS * ES, RPI = 1024 / RB, NI = BK / RPI;
#pragma unroll
  for (int u = 0; u < NI / NW; ++u) {
    const int j = wave + NW * u;
    dma16(o.rs, dst + j * 1024, o.voff[RPI > 1 ? 0 : (j & 1)],
          o.origin + (k0 + static_cast<uint32_t>(RPI * j)) * o.ld_bytes);
  }
}

// Byte address of element (k, p) in the row-major X tile.
template <int TS, int ES>
__device__ __forceinline__ int rm_off(int k, int p) {
  constexpr int RB = TS * ES, EPC = 16 / ES;
  return k * RB + (((p / EPC) ^ (4 * (k & 1))) << 4) + (p % EPC) * ES;
}

// MFMA over one LDS stage; the wave at (wr, wc) of a WGP x WGQ grid owns a
// (TS/WGP) x (TS/WGQ) sub-tile made of FP x FQ 32x32 blocks.
template <int XDT, int MODE, int TS, int WGP, int WGQ>
__device__ __forceinline__ void gemm_compute(const uint8_t* sa, const uint8_t* sbp, int lane,
                                             int wr, int wc,
                                             f32x16_t (&acc)[TS / WGP / 32][TS / WGQ / 32]) {
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ, FP = WTP / 32, FQ = WTQ / 32;
  const int l32 = lane & 31, hl = lane >> 5;
  if constexpr (XDT == kBF16) {
    // lane halves hold contraction elements 0-7 and 8-15 of each 16-step.
    // Fragments of step kk+1 are read while the MFMAs of step kk run.
    const int g = lane >> 4, i = lane & 15;
    bf16x8_t fa[2][FP], fb[2][FQ];
    auto load = [&](int kk, int buf) {
#pragma unroll
      for (int f = 0; f < FP; ++f) {
        if constexpr (MODE == APPLY) {
          const int kb = 16 * kk + 8 * (g >> 1) + (i >> 2);
          const int p = wr * WTP + f * 32 + 16 * (g & 1) + 4 * (i & 3);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(sa + rm_off<TS, 2>(kb, p)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(sa + rm_off<TS, 2>(kb + 4, p)));
          fa[buf][f] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          fa[buf][f] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off(wr * WTP + f * 32 + l32, 2 * kk + hl));
        }
      }
#pragma unroll
      for (int f = 0; f < FQ; ++f)
        fb[buf][f] = *reinterpret_cast<const bf16x8_t*>(sbp + lds_off(wc * WTQ + f * 32 + l32, 2 * kk + hl));
    };
    constexpr int NR = (MODE == APPLY ? 2 : 1) * FP + FQ;   // LDS reads per step
    constexpr int NM = FP * FQ;                             // MFMAs per step
    load(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk < 3) load(kk + 1, cur ^ 1);
#pragma unroll
      for (int a = 0; a < FP; ++a)
#pragma unroll
        for (int b = 0; b < FQ; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], acc[a][b], 0, 0, 0);
    }
#if __HIP_DEVICE_COMPILE__
    // schedule: first step's reads, then for each step one MFMA per read of
    // the following step, then the remaining MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int r = 0; r < (NR < NM ? NR : NM); ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
      if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
#endif
  } else {
    // lane half h feeds contraction elements 8h..8h+7 of each 16-step over
    // eight 32x32x2 instructions
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int ch = 4 * g2 + 2 * hl;
      float fa[FP][8], fb[FQ][8];
#pragma unroll
      for (int f = 0; f < FQ; ++f) {
        const int rb_ = wc * WTQ + f * 32 + l32;
        const float4 b0 = *reinterpret_cast<const float4*>(sbp + lds_off(rb_, ch));
        const float4 b1 = *reinterpret_cast<const float4*>(sbp + lds_off(rb_, ch + 1));
        fb[f][0] = b0.x; fb[f][1] = b0.y; fb[f][2] = b0.z; fb[f][3] = b0.w;
        fb[f][4] = b1.x; fb[f][5] = b1.y; fb[f][6] = b1.z; fb[f][7] = b1.w;
      }
#pragma unroll
      for (int f = 0; f < FP; ++f) {
        if constexpr (MODE == APPLY) {
          const int p = wr * WTP + f * 32 + l32;
#pragma unroll
          for (int s = 0; s < 8; ++s)
            fa[f][s] = *reinterpret_cast<const float*>(sa + rm_off<TS, 4>(16 * g2 + 8 * hl + s, p));
        } else {
          const int ra_ = wr * WTP + f * 32 + l32;
          const float4 a0 = *reinterpret_cast<const float4*>(sa + lds_off(ra_, ch));
          const float4 a1 = *reinterpret_cast<const float4*>(sa + lds_off(ra_, ch + 1));
          fa[f][0] = a0.x; fa[f][1] = a0.y; fa[f][2] = a0.z; fa[f][3] = a0.w;
          fa[f][4] = a1.x; fa[f][5] = a1.y; fa[f][6] = a1.z; fa[f][7] = a1.w;
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int a = 0; a < FP; ++a)
#pragma unroll
          for (int b = 0; b < FQ; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a][s], fb[b][s], acc[a][b], 0, 0, 0);
    }
  }
}

// One K step: start filling `fill` with step kt+1, multiply from `cur`.
template <int XDT, int MODE, int TS, int WGP, int WGQ>
__device__ __forceinline__ void gemm_stage(const OpLoad& la, const OpLoad& lb, int kt, int nk,
                                           int wave, int lane, int wr, int wc, uint8_t* cur,
                                           uint8_t* fill,
                                           f32x16_t (&acc)[TS / WGP / 32][TS / WGQ / 32]) {
  constexpr int ES = Ty<XDT>::ES, BK = Ty<XDT>::BK, OPB = TS * 128, NW = WGP * WGQ;
  if (kt + 1 < nk) {
    const uint32_t k1 = static_cast<uint32_t>(kt + 1) * BK;
    if constexpr (MODE == APPLY) load_rm<TS, ES, BK, NW>(la, k1, wave, fill);
    else load_kc<TS, NW>(la, k1 * ES, wave, fill);
    load_kc<TS, NW>(lb, k1 * ES, wave, fill + OPB);
  }
  gemm_compute<XDT, MODE, TS, WGP, WGQ>(cur, cur + OPB, lane, wr, wc, acc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Logical block index: blocks are dealt round-robin to the eight XCDs; this
// gives each XCD a contiguous range of logical tiles, so tiles that share
// operand panels run on the same L2.
__device__ __forceinline__ int xcd_block() {
  const int nb = gridDim.x, b = blockIdx.x;
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

template <int XDT, int MODE, int TS, int WGP, int WGQ>
__global__ __launch_bounds__(64 * WGP * WGQ, 1) void k_gemm(GemmArgs args) {
  using T = typename Ty<XDT>::T;
  constexpr int ES = Ty<XDT>::ES;
  constexpr int BK = Ty<XDT>::BK;
  constexpr int NW = WGP * WGQ;       // waves per block
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ;
  constexpr int FP = WTP / 32, FQ = WTQ / 32;
  constexpr int OPB = TS * 128;       // LDS bytes per operand per stage

  __shared__ __attribute__((aligned(1024))) uint8_t smem0[2 * OPB];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[2 * OPB];
  __shared__ float red[NW];

  // ---- locate group, matrix and tile
  const int bid = xcd_block();
  // constant-index selection keeps the group table in kernel-argument space
  GemmGroup G = args.g[0];
#pragma unroll
  for (int k = 1; k < kMaxGroups; ++k)
    if (k < args.ngroups && bid >= args.g[k].block_base) G = args.g[k];
  const int local = bid - G.block_base;
  const int mat = local / G.tiles;
  const int tile = local - mat * G.tiles;
  int tP, tQ;
  if (MODE == APPLY) {
    // groups of up to four row panels (Q), column panels (P) outer
    const int tn = G.np / TS, tm = G.mp / TS;
    const int grp = tile / (4 * tn), q0 = 4 * grp;
    const int gq = tm - q0 < 4 ? tm - q0 : 4;
    const int in = tile - grp * 4 * tn;
    tQ = q0 + in % gq;
    tP = in / gq;
  } else {
    const int tm = G.mp / TS;
    int bi = 0, rem = tile;
    while (rem >= tm - bi) { rem -= tm - bi; ++bi; }
    tP = bi;
    tQ = bi + rem;
  }

  const T* xin = static_cast<const T*>(G.xin) + static_cast<int64_t>(mat) * G.in_stride;
  T* out = static_cast<T*>(G.out) + static_cast<int64_t>(mat) * G.out_stride;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave / WGQ, wc = wave % WGQ;

  OpLoad la, lb;
  int K;
  if (MODE == GRAM || MODE == POLY) {
    const int ld = MODE == GRAM ? G.np : G.mp;
    K = ld;
    const uint32_t bytes = static_cast<uint32_t>(G.mp) * ld * ES;
    la.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(xin), 0, bytes, kRsrcWord3);
    lb.rs = la.rs;
    la.ld_bytes = lb.ld_bytes = static_cast<uint32_t>(ld) * ES;
    la.origin = static_cast<uint32_t>(tP) * TS * la.ld_bytes;
    lb.origin = static_cast<uint32_t>(tQ) * TS * lb.ld_bytes;
    plan_kc<NW>(la, lane, wave);
    plan_kc<NW>(lb, lane, wave);
  } else {
    K = G.mp;
    la.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(xin), 0,
                                              static_cast<uint32_t>(G.mp) * G.np * ES, kRsrcWord3);
    la.ld_bytes = static_cast<uint32_t>(G.np) * ES;
    la.origin = static_cast<uint32_t>(tP) * TS * ES;
    plan_rm<TS, ES>(la, lane);
    const T* bm = static_cast<const T*>(G.bop) + static_cast<int64_t>(mat) * G.b_stride;
    lb.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(bm), 0,
                                              static_cast<uint32_t>(G.mp) * G.mp * ES, kRsrcWord3);
    lb.ld_bytes = static_cast<uint32_t>(G.mp) * ES;
    lb.origin = static_cast<uint32_t>(tQ) * TS * lb.ld_bytes;
    plan_kc<NW>(lb, lane, wave);
  }

  float scale = 1.f;
  if (args.first) scale = matrix_scale<NW>(G.partials + static_cast<int64_t>(mat) * G.p_stride,
                                           G.npartials, args.eps, red);

  f32x16_t acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  if constexpr (MODE == APPLY) load_rm<TS, ES, BK, NW>(la, 0, wave, smem0);
  else load_kc<TS, NW>(la, 0, wave, smem0);
  load_kc<TS, NW>(lb, 0, wave, smem0 + OPB);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // two K steps per trip: the stage being read and the stage being filled are
  // always different __shared__ objects
  // (the planner pads every dimension so that nk is even)
#pragma unroll 1
  for (int kt = 0; kt < nk; kt += 2) {
    gemm_stage<XDT, MODE, TS, WGP, WGQ>(la, lb, kt, nk, wave, lane, wr, wc, smem0, smem1, acc);
    gemm_stage<XDT, MODE, TS, WGP, WGQ>(la, lb, kt + 1, nk, wave, lane, wr, wc, smem1, smem0, acc);
  }

  // ---- epilogue
  const int ld_out = MODE == APPLY ? G.np : G.mp;
  const float alpha = MODE == GRAM ? scale * scale : 1.f;
  // off-diagonal symmetric tiles also store the transposed tile; bf16 tiles
  // stage it in the (now idle) LDS so that it leaves as 16-byte rows
  const bool mirror = MODE != APPLY && tP != tQ;
  constexpr bool kStage = XDT == kBF16 && MODE != APPLY;
  constexpr int SP = TS * 2;                 // staged row pitch (bytes)
  // staged row r (= P - tP*TS) lives in smem0 for r < TS/2, else in smem1
  static_assert(!kStage || (TS / 2) * SP <= 2 * OPB, "mirror staging does not fit");
  auto srow = [&](int r) -> uint8_t* {
    return (r < TS / 2 ? smem0 : smem1) + (r % (TS / 2)) * SP;
  };
#pragma unroll
  for (int i = 0; i < FP; ++i) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int ql = wc * WTQ + j * 32 + (lane & 31);
      const int Q = tQ * TS + ql;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int pl = wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
        const int P = tP * TS + pl;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][rg * 4 + e];
        const int64_t qp = static_cast<int64_t>(Q) * ld_out + P;
        if (MODE == GRAM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= alpha;
        } else if (MODE == POLY) {
          float av[4];
          ld4(xin + qp, av);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = args.cb * av[e] + args.cc * v[e];
        } else {
          float xv[4];
          ld4(xin + qp, xv);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = scale * (args.ca * xv[e] + args.cbb * v[e]);
        }
        st4(out + qp, v);
        if (mirror) {
          if constexpr (kStage) {
            // row pl+e, column ql; 16-byte chunks XOR 4 on every fourth row
            // group so the two lane halves land on different banks
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = pl + e;
              const int off = ((((ql >> 3) ^ (4 * ((r >> 2) & 1)))) << 4) + (ql & 7) * 2;
              *reinterpret_cast<uint16_t*>(srow(r) + off) = f2bf(v[e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) st1(out + static_cast<int64_t>(P + e) * ld_out + Q, v[e]);
          }
        }
      }
    }
  }
  if constexpr (kStage) {
    if (mirror) {
      __syncthreads();
      constexpr int CPRW = TS / 8;           // 16-byte chunks per staged row
      for (int c = t; c < TS * CPRW; c += 64 * NW) {
        const int r = c / CPRW, ch = c % CPRW;
        const int pch = ch ^ (4 * ((r >> 2) & 1));
        const uint4 vv = *reinterpret_cast<const uint4*>(srow(r) + (pch << 4));
        *reinterpret_cast<uint4*>(out + static_cast<int64_t>(tP * TS + r) * ld_out + tQ * TS + ch * 8) = vv;
      }
    }
  }
}

template <int XDT, int MODE>
hipError_t launch_ts(int ts, int waves, const GemmArgs& a, int64_t blocks, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (ts == 256 && waves == 8)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 256, 2, 4>), grid, dim3(512), 0, s, a);
  else if (ts == 256)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 256, 2, 2>), grid, dim3(256), 0, s, a);
  else if (ts == 128)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 128, 2, 2>), grid, dim3(256), 0, s, a);
  else if (ts == 64)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 64, 2, 2>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int phase, int xdt, int ts, int waves, const GemmArgs& a,
                       int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (xdt == kBF16) {
    if (phase == GRAM) return launch_ts<kBF16, GRAM>(ts, waves, a, blocks, s);
    if (phase == POLY) return launch_ts<kBF16, POLY>(ts, waves, a, blocks, s);
    return launch_ts<kBF16, APPLY>(ts, waves, a, blocks, s);
  }
  // the fp32 path keeps four waves
  if (phase == GRAM) return launch_ts<kF32, GRAM>(ts, 4, a, blocks, s);
  if (phase == POLY) return launch_ts<kF32, POLY>(ts, 4, a, blocks, s);
  return launch_ts<kF32, APPLY>(ts, 4, a, blocks, s);
}

}  // namespace muon
