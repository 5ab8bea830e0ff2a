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
// Tiling: square TS x TS output tiles, a WGP x WGQ grid of waves, each wave
// a sub-tile of 32x32 MFMA blocks.  Every operand tile goes from global memory
// to LDS by buffer loads with the LDS-DMA bit (no register staging).
//   * bf16: two LDS stages of 128 bytes of contraction per operand row (one
//     full cache line per row and load), the next stage loading while the
//     current one is multiplied; one barrier per stage.
//   * fp32: a ring of four stages of 64 bytes per row, loads three stages
//     ahead.
// Operands whose contraction index is contiguous in memory (both GRAM
// operands, both POLY operands, the B operand of APPLY) are stored as rows of
// 16-byte chunks with the chunk index XOR-ed with a function of the row, so
// the 16 rows read by each 16-lane slice of an MFMA operand load cover all 64
// banks.  APPLY contracts over the rows of X, so its X tile is stored
// row-major (contraction index = LDS row) and the bf16 MFMA operand is
// assembled by the LDS transpose read (each 16-lane group turns a 4 x 16
// block into four consecutive contraction values per column).
// GRAM and POLY are symmetric: only tiles on or above the diagonal run, and
// off-diagonal tiles also store their mirror image.  The MFMA output layout
// gives each lane four consecutive rows of one column; the tiles are arranged
// so that those four values are contiguous in memory (row Q, columns P..P+3).
#include <type_traits>

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
  static constexpr int ES = 2;    // element bytes
  static constexpr int BK = 64;   // contraction elements per stage (128-byte rows)
  static constexpr int CPR = 8;   // 16-byte chunks per operand row per stage
  static constexpr int NST = 2;   // LDS stages
};
template <> struct Ty<kF32> {
  using T = float;
  static constexpr int ES = 4;
  static constexpr int BK = 16;
  static constexpr int CPR = 4;
  static constexpr int NST = 4;
};
// LDS stages of a tile's ring.  64-wide bf16 tiles (small problems: few
// tiles, short K loops, each stage waiting on load latency) keep three stages
// in flight in a four-stage ring of 64 KB (measured on one 256 x 512 matrix:
// step 10 % faster than two stages; eight stages, 128 KB, 1 % faster).
template <int XDT, int TS>
constexpr int stages() {
  return XDT == kBF16 && TS == 64 ? 4 : Ty<XDT>::NST;
}

// LDS bank model: 64 four-byte banks; a 16-byte-per-lane read is served 16
// lanes (256 bytes) at a time, an 8-byte read 32 lanes at a time.
//
// K-contiguous tile: row r, logical 16-byte chunk c.  With four chunks per
// row (64 bytes) four rows share a 256-byte bank line and the chunk is XOR-ed
// with (r >> 2) & 3; with eight (128 bytes) two rows share a line and the
// chunk is XOR-ed with (r >> 1) & 7.  Either way the 16 rows read by one
// 16-lane slice land on 16 distinct 16-byte slots.
template <int CPR>
__device__ __forceinline__ int kc_off(int r, int c) {
  if constexpr (CPR == 4) return (r << 6) + ((c ^ ((r >> 2) & 3)) << 4);
  else return (r << 7) + ((c ^ ((r >> 1) & 7)) << 4);
}
// Row-major X tile: contraction row k, column p.  The chunk index is XOR-ed
// with 4 (k & 3), so the four rows read by two transpose groups (64 bytes
// each) fall in four different quarters of the bank line.
template <int TS, int ES>
__device__ __forceinline__ int rm_off(int k, int p) {
  constexpr int RB = TS * ES, EPC = 16 / ES, CPR = RB / 16;
  return k * RB + (((p / EPC) ^ ((4 * (k & 3)) & (CPR - 1))) << 4) + (p % EPC) * ES;
}

// fp32 -> bf16, round to nearest even: gfx950 converts a pair per
// instruction (v_cvt_pk_bf16_f32); NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Four consecutive elements <-> floats.
__device__ __forceinline__ void unpack4(const uint2 q, float* v) {
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack4(const float4 q, float* v) {
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void st4(uint16_t* p, const float* v) {
  uint2 q;
  q.x = pack_bf16(v[0], v[1]);
  q.y = pack_bf16(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = q;
}
__device__ __forceinline__ void st4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st1(uint16_t* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }

// 1 / (sqrt(sum of the matrix's norm partials) + eps).  Summation order:
// 256-strided per-thread sums over the first four waves' lanes, the
// butterfly, then the wave totals in order -- the same in every kernel and
// block size, so every block of a matrix gets the same s.
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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes at `base` (reads past the end
// return zero).  All fields are block-uniform and live in SGPRs.
__device__ __forceinline__ u32x4_t make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t d;
  d[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  d[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = kRsrcWord3;
  return d;
}

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  // the low half of a flat address in the LDS aperture is the LDS address (an
  // address-space cast here adds a null check that one compiler release
  // fails to select in the single-launch kernel)
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// One 1 KiB LDS-DMA load: lane L copies 16 bytes from global offset
// voff + soff of the descriptor's buffer to LDS address lds + 16 L.  It is
// issued as inline assembly so that the compiler does not order later LDS
// reads of *other* stage buffers behind it; wait_vm orders it explicitly.
// It has no result register.
// (M0 is reserved for the compiler's own M0 users, which set it right before
// each use; the clobber keeps it from assuming a value survives.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4_t& d, uint32_t lds, uint32_t voff,
                                      uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(d), "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most n of this wave's vector loads are outstanding (loads
// complete in issue order); LDS and export counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until a stage has landed when min(ahead, MAXA) later stages of PER
// loads each were issued after it.
template <int MAXA, int PER>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= MAXA) wait_vm<MAXA * PER>();
    else wait_ahead<MAXA - 1, PER>(ahead);
  }
}

// Workgroup barrier without a memory fence.  Stage data arrive by LDS DMA
// and are covered by wait_vm before it.  The wave's own LDS reads must have
// returned before it: the compiler is free to sink the MFMAs of the previous
// stage, and the waits for their operands, below a bare s_barrier, and a
// wave past the barrier may then refill (or stage output into) a buffer that
// a slower wave is still reading.  The wait sits in the same statement so
// that nothing can separate the two.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-block load plan of one operand: buffer descriptor, per-lane offset
// (fixed across stages) and the uniform byte offset of the tile's origin.
struct OpLoad {
  u32x4_t rs;
  uint32_t kstep;      // bytes from one stage of 64 contraction elements to the next
  uint32_t voff;
  uint32_t origin;     // bytes: first row of the tile (and first column for row-major X)
  uint32_t ld_bytes;
};

// K-contiguous operand, one 1 KiB instruction j per 64 / CPR rows.  Four
// chunks: rows 16j..16j+15, lane L fills physical chunk L & 3 of row
// 16j + L/4 with logical chunk (L & 3) ^ ((L >> 4) & 3) for every j.  Eight
// chunks: rows 8j..8j+7, lane L fills physical chunk L & 7 of row 8j + L/8
// with logical chunk (L & 7) ^ ((4 (j & 1) + L/16) & 7); j = wave (mod 2)
// because the wave count is even, so the offset is fixed per lane.
template <int CPR>
__device__ __forceinline__ void plan_kc(OpLoad& o, int lane, int wave) {
  if constexpr (CPR == 4)
    o.voff = static_cast<uint32_t>(lane >> 2) * o.ld_bytes + 16u * ((lane & 3) ^ ((lane >> 4) & 3));
  else
    o.voff = static_cast<uint32_t>(lane >> 3) * o.ld_bytes +
             16u * ((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7));
}

template <int TS, int NW, int CPR>
__device__ __forceinline__ void load_kc(const OpLoad& o, uint32_t kbytes, int wave, uint8_t* dst) {
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int u = 0; u < TS / (RPI * NW); ++u) {
    const int j = wave + NW * u;
    dma16(o.rs, lds_addr(dst) + j * 1024, o.voff, o.origin + RPI * j * o.ld_bytes + kbytes);
  }
}

// Row-major X tile of APPLY: BK rows of TS elements; instruction j moves
// RPI = 1024 / (TS ES) rows.  With NW a multiple of four every instruction
// of a wave has j = wave (mod 4), so the row's low two bits -- and the lane's
// offset -- are fixed per lane.
template <int TS, int ES, int NW>
__device__ __forceinline__ void plan_rm(OpLoad& o, int lane, int wave) {
  static_assert(NW % 4 == 0, "wave count");
  constexpr int RB = TS * ES, RPI = 1024 / RB, CPR = RB / 16;
  const int rr = lane / CPR, ch = lane % CPR;
  const int r3 = (RPI * wave + rr) & 3;
  o.voff = static_cast<uint32_t>(rr) * o.ld_bytes + 16u * (ch ^ ((4 * r3) & (CPR - 1)));
}

template <int TS, int ES, int BK, int NW>
__device__ __forceinline__ void load_rm(const OpLoad& o, uint32_t k0, int wave, uint8_t* dst) {
  constexpr int RB = TS * ES, RPI = 1024 / RB, NI = BK / RPI;
  static_assert(NI % NW == 0, "row-major load split");
#pragma unroll
  for (int u = 0; u < NI / NW; ++u) {
    const int j = wave + NW * u;
    dma16(o.rs, lds_addr(dst) + j * 1024, o.voff,
          o.origin + (k0 + static_cast<uint32_t>(RPI * j)) * o.ld_bytes);
  }
}

// MFMA over one LDS stage; the wave at (wr, wc) of a WGP x WGQ grid owns a
// (TS/WGP) x (TS/WGQ) sub-tile made of FP x FQ 32x32 blocks.
template <int XDT, int MODE, int TS, int WGP, int WGQ, int H>
__device__ __forceinline__ void gemm_compute(const uint8_t* sa, const uint8_t* sbp, int lane,
                                             int wr, int wc,
                                             f32x16_t (&acc)[TS / WGP / 32][TS / WGQ / 32]) {
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ, FP = WTP / 32, FQ = WTQ / 32;
  const int l32 = lane & 31, hl = lane >> 5;
  if constexpr (XDT == kBF16) {
    // lane halves hold contraction elements 0-7 and 8-15 of each 16-step;
    // the fragments of the second step are read while the first step's
    // MFMAs run
    const int g = lane >> 4, i = lane & 15;
    bf16x8_t fa[2][FP], fb[2][FQ];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int f = 0; f < FP; ++f) {
        if constexpr (MODE == APPLY) {
          const int kb = 32 * H + 16 * kk + 8 * (g >> 1) + (i >> 2);
          const int p = wr * WTP + f * 32 + 16 * (g & 1) + 4 * (i & 3);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(sa + rm_off<TS, 2>(kb, p)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(sa + rm_off<TS, 2>(kb + 4, p)));
          fa[kk][f] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          fa[kk][f] = *reinterpret_cast<const bf16x8_t*>(sa + kc_off<8>(wr * WTP + f * 32 + l32, 4 * H + 2 * kk + hl));
        }
      }
#pragma unroll
      for (int f = 0; f < FQ; ++f)
        fb[kk][f] = *reinterpret_cast<const bf16x8_t*>(sbp + kc_off<8>(wc * WTQ + f * 32 + l32, 4 * H + 2 * kk + hl));
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int a = 0; a < FP; ++a)
#pragma unroll
        for (int b = 0; b < FQ; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][a], fb[kk][b], acc[a][b], 0, 0, 0);
#if __HIP_DEVICE_COMPILE__
    constexpr int NR = (MODE == APPLY ? 2 : 1) * FP + FQ;   // LDS reads per 16-step
    constexpr int NM = FP * FQ;                             // MFMAs per 16-step
    constexpr int NI = NR < NM ? NR : NM;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
    if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
#endif
  } else {
    // lane half h feeds contraction elements 8h..8h+7 over eight 32x32x2
    // instructions
    float fa[FP][8], fb[FQ][8];
#pragma unroll
    for (int f = 0; f < FQ; ++f) {
      const int rb_ = wc * WTQ + f * 32 + l32;
      const float4 b0 = *reinterpret_cast<const float4*>(sbp + kc_off<4>(rb_, 2 * hl));
      const float4 b1 = *reinterpret_cast<const float4*>(sbp + kc_off<4>(rb_, 2 * hl + 1));
      fb[f][0] = b0.x; fb[f][1] = b0.y; fb[f][2] = b0.z; fb[f][3] = b0.w;
      fb[f][4] = b1.x; fb[f][5] = b1.y; fb[f][6] = b1.z; fb[f][7] = b1.w;
    }
#pragma unroll
    for (int f = 0; f < FP; ++f) {
      if constexpr (MODE == APPLY) {
        const int p = wr * WTP + f * 32 + l32;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          fa[f][s] = *reinterpret_cast<const float*>(sa + rm_off<TS, 4>(8 * hl + s, p));
      } else {
        const int ra_ = wr * WTP + f * 32 + l32;
        const float4 a0 = *reinterpret_cast<const float4*>(sa + kc_off<4>(ra_, 2 * hl));
        const float4 a1 = *reinterpret_cast<const float4*>(sa + kc_off<4>(ra_, 2 * hl + 1));
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

// Issue the loads of stage k into buffer `dst` ([A | B]).
// share: a diagonal GRAM/POLY tile, whose two operands are the same row
// panel, loads it once (the B half of the buffer is not used).
template <int XDT, int MODE, int TS, int NW>
__device__ __forceinline__ void gemm_issue(const OpLoad& la, const OpLoad& lb, int k, int wave,
                                           uint8_t* dst, bool share) {
  constexpr int ES = Ty<XDT>::ES, BK = Ty<XDT>::BK, CPR = Ty<XDT>::CPR, OPB = TS * CPR * 16;
  const uint32_t k0 = static_cast<uint32_t>(k) * BK;
  if constexpr (MODE == APPLY) load_rm<TS, ES, BK, NW>(la, k0, wave, dst);
  else load_kc<TS, NW, CPR>(la, static_cast<uint32_t>(k) * la.kstep, wave, dst);
  if (!share) load_kc<TS, NW, CPR>(lb, static_cast<uint32_t>(k) * lb.kstep, wave, dst + OPB);
}

// One stage: wait for stage k, refill the buffer of stage k-1 with stage
// k + NST - 1, multiply from stage k.  share (two-stage ring only: its wait
// does not count loads): both operands from the A half of the buffer.
// NWL: the waves [0, NWL) that issue the stage loads (the others multiply
// straight after the barrier).
template <int XDT, int MODE, int TS, int WGP, int WGQ, int NWL = WGP * WGQ>
__device__ __forceinline__ void gemm_step(const OpLoad& la, const OpLoad& lb, int k, int nk,
                                          int wave, int lane, int wr, int wc, uint8_t* cur,
                                          uint8_t* fill, bool share,
                                          f32x16_t (&acc)[TS / WGP / 32][TS / WGQ / 32]) {
  constexpr int ES = Ty<XDT>::ES, BK = Ty<XDT>::BK, CPR = Ty<XDT>::CPR, NST = stages<XDT, TS>();
  constexpr int NW = WGP * WGQ, OPB = TS * CPR * 16, RPI = 64 / CPR;
  constexpr int NA = MODE == APPLY ? BK / (1024 / (TS * ES)) / NW : TS / (RPI * NW);
  constexpr int PER = NA + TS / (RPI * NW);   // loads per wave per stage
  if constexpr (NST > 2) {
    // stages issued after this one: min(NST - 2, nk - 1 - k)
    wait_ahead<NST - 2, PER>(nk - 1 - k);
  } else {
    if (NWL == NW || wave < NWL) wait_vm<0>();
  }
  // bare barrier: a fenced __syncthreads would also wait for the loads of the
  // stages still in flight
  lds_barrier();
  if (k + NST - 1 < nk && (NWL == NW || wave < NWL))
    gemm_issue<XDT, MODE, TS, NWL>(la, lb, k + NST - 1, wave, fill, share);
  // GRAM: the wave in its MFMA run takes issue priority over the other wave
  // of its SIMD (measured: GRAM 2.5 % faster; neutral for POLY, APPLY)
  if constexpr (MODE == GRAM) __builtin_amdgcn_s_setprio(1);
  const uint8_t* const bop = share ? cur : cur + OPB;
  gemm_compute<XDT, MODE, TS, WGP, WGQ, 0>(cur, bop, lane, wr, wc, acc);
  if constexpr (XDT == kBF16)
    gemm_compute<XDT, MODE, TS, WGP, WGQ, 1>(cur, bop, lane, wr, wc, acc);
  if constexpr (MODE == GRAM) __builtin_amdgcn_s_setprio(0);
}

// ---- input term and staged output of 256-wide bf16 tiles
//
// POLY (B = b A + c A A) and APPLY (X' = s (a X + beta B X)) add a multiple of
// their input at the output positions.  That input tile passes through LDS
// during the K loop anyway (APPLY: rows Q of X are the contraction rows of one
// stage; POLY: A[Q][P] = A[P][Q] is part of the stage whose contraction range
// covers P), so each wave folds coef * input into its accumulators there:
// acc = product + coef * input, output = mult * acc, with coef = a / beta,
// mult = s beta (APPLY) and coef = b / c, mult = c (POLY).
template <int MODE, int TS, int WGP, int WGQ>
__device__ __forceinline__ void capture_input(int k, const uint8_t* stage, int lane, int wr,
                                              int wc, int tP, int tQ, float coef, bool share,
                                              f32x16_t (&acc)[TS / WGP / 32][TS / WGQ / 32]) {
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ, FP = WTP / 32, FQ = WTQ / 32;
  constexpr int BK = Ty<kBF16>::BK, OPB = TS * Ty<kBF16>::CPR * 16;
  const int k0 = k * BK;
  const uint8_t* const bst = share ? stage : stage + OPB;   // POLY: the B operand's rows
  if constexpr (MODE == APPLY) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q0 = tQ * TS + wc * WTQ + j * 32;   // first X row of fragment j
      if (q0 >= k0 && q0 < k0 + BK) {
        const int r = q0 - k0 + (lane & 31);
#pragma unroll
        for (int i = 0; i < FP; ++i)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int p = wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
            float x[4];
            unpack4(*reinterpret_cast<const uint2*>(stage + rm_off<TS, 2>(r, p)), x);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][rg * 4 + e] += coef * x[e];
          }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      const int p0 = tP * TS + wr * WTP + i * 32;   // first column of fragment i
      if (p0 >= k0 && p0 < k0 + BK) {
#pragma unroll
        for (int j = 0; j < FQ; ++j) {
          const int row = wc * WTQ + j * 32 + (lane & 31);
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int kk = p0 - k0 + rg * 8 + (lane >> 5) * 4;
            float x[4];
            unpack4(*reinterpret_cast<const uint2*>(bst + kc_off<8>(row, kk >> 3) +
                                                    (kk & 7) * 2), x);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][rg * 4 + e] += coef * x[e];
          }
        }
      }
    }
  }
}

// Staging tile of a 256 x 256 bf16 output in LDS: row Q (512 bytes), 8-byte
// slot s = P / 4 stored at s ^ stg_sw(Q).  The 32 rows written by one
// half-wave (same P) land on 32 distinct bank pairs, and the two slots of a
// 16-byte chunk stay together (chunk c at c ^ (Q & 15), halves swapped when
// bit 4 of Q is set).
__device__ __forceinline__ int stg_sw(int q) { return (2 * (q & 15)) ^ ((q >> 4) & 1); }

// Write mult * acc to the tile at (tQ, tP) through the LDS staging tile:
// 16-byte row stores, and for off-diagonal GRAM/POLY tiles the mirror image
// from transposing LDS reads (each 16-lane group turns 16 rows x 4 columns
// into 4 rows x 16 columns).
// Element offset of (r, c) in an m x m matrix stored tile-contiguous: blocks
// of 256 rows x 64 columns (32 KB of bf16, rows of 128 bytes), block
// (c / 64) * nbr + r / 256 for nbr = m / 256 row panels.  A stage of a row
// panel is then one contiguous block for the LDS-DMA loads.
__device__ __forceinline__ int64_t blk_off(int r, int c, int nbr) {
  return (static_cast<int64_t>((c >> 6) * nbr + (r >> 8)) << 14) + ((r & 255) << 6) + (c & 63);
}

// nbr > 0: `out` is tile-contiguous with nbr row panels (ld unused).
template <int MODE, int WGP, int WGQ>
__device__ __forceinline__ void staged_store(uint8_t* stg, uint16_t* out, int64_t ld, int nbr,
                                             int tP, int tQ, bool mirror, float mult, int wave,
                                             int lane, int wr, int wc,
                                             f32x16_t (&acc)[256 / WGP / 32][256 / WGQ / 32]) {
  constexpr int TS = 256, NW = WGP * WGQ;
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ, FP = WTP / 32, FQ = WTQ / 32;
  // every wave is past its last read of the stage buffers
  lds_barrier();
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = wc * WTQ + j * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int p = wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
        uint2 v;
        v.x = pack_bf16(mult * acc[i][j][rg * 4], mult * acc[i][j][rg * 4 + 1]);
        v.y = pack_bf16(mult * acc[i][j][rg * 4 + 2], mult * acc[i][j][rg * 4 + 3]);
        *reinterpret_cast<uint2*>(stg + q * 512 + (((p >> 2) ^ stg_sw(q)) << 3)) = v;
      }
    }
  __syncthreads();
  // rows: two per instruction, 32 lanes x 16 bytes each
#pragma unroll
  for (int u = 0; u < TS / (2 * NW); ++u) {
    const int q = 2 * (wave + NW * u) + (lane >> 5), c = lane & 31, sw = stg_sw(q);
    uint4 v = *reinterpret_cast<const uint4*>(stg + q * 512 + ((c ^ (sw >> 1)) << 4));
    if (sw & 1) v = make_uint4(v.z, v.w, v.x, v.y);
    const int64_t o = nbr ? blk_off(tQ * TS + q, tP * TS + 8 * c, nbr)
                          : static_cast<int64_t>(tQ * TS + q) * ld + tP * TS + 8 * c;
    *reinterpret_cast<uint4*>(out + o) = v;
  }
  if (!mirror) return;
  // mirror: a pair of transposing reads gives lane j of group g eight
  // consecutive rows Q0 + 8 (j / 4) + 0..7 of column 4 pq + j % 4, where the
  // group's quad pq is qb + {0, 8, 1, 9}[g] (groups 0 and 1 read disjoint
  // bank sets)
  const int g = lane >> 4, i = lane & 15;
  const int goff = (g & 1) * 8 + (g >> 1);
#pragma unroll 4
  for (int t = wave; t < 128; t += NW) {
    const int n = t & 7, h = (t >> 3) & 3, m = t >> 5;
    const int q0 = 32 * n, pq = 16 * m + 2 * h + goff;
    i16x4_t r[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int q = q0 + 8 * (i & 3) + (i >> 2) + 4 * rr;
      r[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(stg + q * 512 + ((pq ^ stg_sw(q)) << 3)));
    }
    const int p = 4 * pq + (i & 3);
    uint4 v;
    v.x = static_cast<uint16_t>(r[0][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[0][1])) << 16);
    v.y = static_cast<uint16_t>(r[0][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[0][3])) << 16);
    v.z = static_cast<uint16_t>(r[1][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[1][1])) << 16);
    v.w = static_cast<uint16_t>(r[1][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[1][3])) << 16);
    const int64_t o = nbr ? blk_off(tP * TS + p, tQ * TS + q0 + 8 * (i >> 2), nbr)
                          : static_cast<int64_t>(tP * TS + p) * ld + tQ * TS + q0 + 8 * (i >> 2);
    *reinterpret_cast<uint4*>(out + o) = v;
  }
}

// Last APPLY of a plain step: instead of storing the iterate, update the
// parameter matrix W <- (W - lrwd W) - lr O, with O = bf16(mult * acc) (the
// value the iterate would be stored as) and the fp32 operation order of the
// separate finish kernel, so W is bit for bit what that kernel writes.  The
// tile goes through the staging tile as in staged_store; W rows are the
// iterate's rows (16-byte row reads), or for a tall W its columns (the
// transposing reads of the mirror path).  Each lane loads all of its W
// chunks before it reads the staging tile, so their latency overlaps.
// Shapes are multiples of 8, so an 8-element chunk is wholly inside W or
// wholly in the padding.
template <int WGP, int WGQ>
__device__ __forceinline__ void staged_finish(uint8_t* stg, const FinDesc& f, int tP, int tQ,
                                              float mult, float lr, float lrwd, int wave,
                                              int lane, int wr, int wc,
                                              f32x16_t (&acc)[256 / WGP / 32][256 / WGQ / 32]) {
#pragma clang fp contract(off)
  constexpr int TS = 256, NW = WGP * WGQ;
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ, FP = WTP / 32, FQ = WTQ / 32;
  constexpr int NU = TS / (2 * NW);   // 16-byte chunks per lane
  static_assert(NU == 128 / NW, "row and column passes move the same chunk count");
  lds_barrier();
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = wc * WTQ + j * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int p = wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
        uint2 v;
        v.x = pack_bf16(mult * acc[i][j][rg * 4], mult * acc[i][j][rg * 4 + 1]);
        v.y = pack_bf16(mult * acc[i][j][rg * 4 + 2], mult * acc[i][j][rg * 4 + 3]);
        *reinterpret_cast<uint2*>(stg + q * 512 + (((p >> 2) ^ stg_sw(q)) << 3)) = v;
      }
    }
  lds_barrier();
  uint16_t* const w = static_cast<uint16_t*>(f.w);
  const int g = lane >> 4, i = lane & 15;
  const int goff = (g & 1) * 8 + (g >> 1);
  int64_t off[NU];
  bool ok[NU];
  uint4 wv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    int R, C;
    if (!f.tall) {
      const int q = 2 * (wave + NW * u) + (lane >> 5);
      R = tQ * TS + q;
      C = tP * TS + 8 * (lane & 31);
    } else {
      const int t = wave + NW * u;
      const int n = t & 7, h = (t >> 3) & 3, m = t >> 5;
      R = tP * TS + 4 * (16 * m + 2 * h + goff) + (i & 3);
      C = tQ * TS + 32 * n + 8 * (i >> 2);
    }
    ok[u] = R < f.rows && C < f.cols;
    off[u] = static_cast<int64_t>(R) * f.ldw + C;
    if (ok[u]) wv[u] = *reinterpret_cast<const uint4*>(w + off[u]);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    uint4 o;
    if (!f.tall) {
      const int q = 2 * (wave + NW * u) + (lane >> 5), c = lane & 31, sw = stg_sw(q);
      o = *reinterpret_cast<const uint4*>(stg + q * 512 + ((c ^ (sw >> 1)) << 4));
      if (sw & 1) o = make_uint4(o.z, o.w, o.x, o.y);
    } else {
      const int t = wave + NW * u;
      const int n = t & 7, h = (t >> 3) & 3, m = t >> 5;
      const int q0 = 32 * n, pq = 16 * m + 2 * h + goff;
      i16x4_t r[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int q = q0 + 8 * (i & 3) + (i >> 2) + 4 * rr;
        r[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(stg + q * 512 + ((pq ^ stg_sw(q)) << 3)));
      }
      o.x = static_cast<uint16_t>(r[0][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[0][1])) << 16);
      o.y = static_cast<uint16_t>(r[0][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[0][3])) << 16);
      o.z = static_cast<uint16_t>(r[1][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[1][1])) << 16);
      o.w = static_cast<uint16_t>(r[1][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(r[1][3])) << 16);
    }
    if (!ok[u]) continue;
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
    const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
    uint32_t res[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = __uint_as_float(ow[e] << 16), o1 = __uint_as_float(ow[e] & 0xffff0000u);
      float w0 = __uint_as_float(ww[e] << 16), w1 = __uint_as_float(ww[e] & 0xffff0000u);
      w0 = (w0 - lrwd * w0) - lr * o0;
      w1 = (w1 - lrwd * w1) - lr * o1;
      res[e] = pack_bf16(w0, w1);
    }
    *reinterpret_cast<uint4*>(w + off[u]) = make_uint4(res[0], res[1], res[2], res[3]);
  }
}

// Logical block index: blocks are dealt round-robin to the eight XCDs; this
// gives each XCD a contiguous range of logical tiles, so tiles that share
// operand panels run on the same L2.
__device__ __forceinline__ int xcd_block() {
  const int nb = gridDim.x, b = blockIdx.x;
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Constants of one Newton-Schulz iteration as seen by a tile.
struct TileCoef {
  float ca, cb, cc;   // a, b, c of the iteration
  float cbb;          // APPLY: multiplier of the product (1, or b when B = bA)
  float eps;
  int first;          // first iteration: fold the norm scale s in
  float lr, lrwd;     // FIN: the update's lr and fl(lr * wd)
  int ablk;           // A and B are stored tile-contiguous (256-wide bf16 tiles)
  int nofold;         // keep the input term out of the accumulators
};

// One output tile (tP, tQ) of matrix `mat` of group G: K loop and epilogue.
// smem holds NST * 2 * OPB bytes, red NW floats.  FIN (APPLY, 256-wide bf16,
// beta != 0): update the matrix's W (G.fin) instead of storing the iterate.
template <int XDT, int MODE, int TS, int WGP, int WGQ, bool FIN>
__device__ __forceinline__ void gemm_tile(const GemmGroup& G, int mat, int tP, int tQ,
                                          const TileCoef& cf, uint8_t* smem, float* red) {
  using T = typename Ty<XDT>::T;
  constexpr int ES = Ty<XDT>::ES;
  constexpr int BK = Ty<XDT>::BK, CPR = Ty<XDT>::CPR, NST = stages<XDT, TS>();
  constexpr int NW = WGP * WGQ;       // waves per block
  constexpr int WTP = TS / WGP, WTQ = TS / WGQ;
  constexpr int FP = WTP / 32, FQ = WTQ / 32;
  constexpr int OPB = TS * CPR * 16;  // LDS bytes per operand per stage
  uint8_t* const sm0 = smem;
  uint8_t* const sm1 = smem + 2 * OPB;

  const T* xin = static_cast<const T*>(G.xin) + static_cast<int64_t>(mat) * G.in_stride;
  T* out = static_cast<T*>(G.out) + static_cast<int64_t>(mat) * G.out_stride;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave / WGQ, wc = wave % WGQ;

  // A and B (m x m) are tile-contiguous for 256-wide bf16 tiles: a stage of a
  // row panel (256 rows x 64 contraction elements) is one 32 KB block
  constexpr bool kStagedT = XDT == kBF16 && TS == 256;
  const bool blk = kStagedT && cf.ablk;
  const uint32_t blk_step = static_cast<uint32_t>(G.mp / TS) * TS * BK * ES;
  auto plan_m = [&](OpLoad& o, int panel) {   // row panel of A or B
    if (blk) {
      o.ld_bytes = BK * ES;
      o.origin = static_cast<uint32_t>(panel) * TS * BK * ES;
      o.kstep = blk_step;
    } else {
      o.ld_bytes = static_cast<uint32_t>(G.mp) * ES;
      o.origin = static_cast<uint32_t>(panel) * TS * o.ld_bytes;
      o.kstep = BK * ES;
    }
  };
  // GRAM (eight waves of 128 x 64): half of the waves issue the stage loads,
  // so on every SIMD one wave starts its MFMAs right after the barrier while
  // the other issues (measured: GRAM 2-4 % faster; neutral for POLY/APPLY)
  constexpr int NWL = (MODE == GRAM && NST == 2 && NW == 8) ? 4 : NW;
  OpLoad la, lb;
  int K;
  if (MODE == GRAM || MODE == POLY) {
    const int ld = MODE == GRAM ? G.np : G.mp;
    K = G.kdim;
    const uint32_t bytes = static_cast<uint32_t>(G.mp) * ld * ES;
    la.rs = make_desc(xin, bytes);
    lb.rs = la.rs;
    if (MODE == GRAM) {
      la.ld_bytes = lb.ld_bytes = static_cast<uint32_t>(ld) * ES;
      la.origin = static_cast<uint32_t>(tP) * TS * la.ld_bytes;
      lb.origin = static_cast<uint32_t>(tQ) * TS * lb.ld_bytes;
      la.kstep = lb.kstep = BK * ES;
    } else {
      plan_m(la, tP);
      plan_m(lb, tQ);
    }
    plan_kc<CPR>(la, lane, wave);
    plan_kc<CPR>(lb, lane, wave);
  } else {
    K = G.kdim;
    la.rs = make_desc(xin, static_cast<uint32_t>(G.mp) * G.np * ES);
    la.ld_bytes = static_cast<uint32_t>(G.np) * ES;
    la.origin = static_cast<uint32_t>(tP) * TS * ES;
    la.kstep = 0;
    plan_rm<TS, ES, NWL>(la, lane, wave);
    const T* bm = static_cast<const T*>(G.bop) + static_cast<int64_t>(mat) * G.b_stride;
    lb.rs = make_desc(bm, static_cast<uint32_t>(G.mp) * G.mp * ES);
    plan_m(lb, tQ);
    plan_kc<CPR>(lb, lane, wave);
  }

  float scale = 1.f;
  if (cf.first) scale = matrix_scale<NW>(G.partials + static_cast<int64_t>(mat) * G.p_stride,
                                           G.npartials, cf.eps, red);

  f32x16_t acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // 256-wide bf16 tiles fold the input term in during the K loop and store
  // through LDS (APPLY keeps the plain epilogue when beta == 0)
  constexpr bool kStaged = XDT == kBF16 && TS == 256;
  const bool capt = kStaged && !cf.nofold && (MODE == POLY || (MODE == APPLY && cf.cbb != 0.f));
  const float coef = MODE == POLY ? cf.cb / cf.cc : (capt ? cf.ca / cf.cbb : 0.f);

  // the planner pads every dimension to a multiple of 128, so nk is even
  // and each trip of the two-stage loop below runs its buffers in order
  const int nk = K / BK;
  if constexpr (NST > 2) {
    // ring of NST stages, NST - 1 in flight; both operands always loaded
    // (the counted waits assume a fixed number of loads per stage)
    for (int st = 0; st < NST - 1; ++st)
      if (st < nk) gemm_issue<XDT, MODE, TS, NW>(la, lb, st, wave, smem + st * 2 * OPB, false);
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt)
      gemm_step<XDT, MODE, TS, WGP, WGQ>(la, lb, kt, nk, wave, lane, wr, wc,
                                         smem + (kt % NST) * 2 * OPB,
                                         smem + ((kt + NST - 1) % NST) * 2 * OPB, false, acc);
  } else {
    // a diagonal GRAM/POLY tile loads its one row panel once per stage
    const bool share = MODE != APPLY && tP == tQ;
    if (NWL == NW || wave < NWL) gemm_issue<XDT, MODE, TS, NWL>(la, lb, 0, wave, sm0, share);
#pragma unroll 1
    for (int kt = 0; kt < nk; kt += 2) {
      gemm_step<XDT, MODE, TS, WGP, WGQ, NWL>(la, lb, kt, nk, wave, lane, wr, wc, sm0, sm1, share,
                                              acc);
      if constexpr (kStaged && MODE != GRAM)
        if (capt)
          capture_input<MODE, TS, WGP, WGQ>(kt, sm0, lane, wr, wc, tP, tQ, coef, share, acc);
      gemm_step<XDT, MODE, TS, WGP, WGQ, NWL>(la, lb, kt + 1, nk, wave, lane, wr, wc, sm1, sm0,
                                              share, acc);
      if constexpr (kStaged && MODE != GRAM)
        if (capt)
          capture_input<MODE, TS, WGP, WGQ>(kt + 1, sm1, lane, wr, wc, tP, tQ, coef, share, acc);
    }
  }

  // ---- epilogue
  const int ld_out = MODE == APPLY ? G.np : G.mp;
  const float alpha = MODE == GRAM ? scale * scale : 1.f;
  const bool mirror = MODE != APPLY && tP != tQ;
  if constexpr (FIN) {
    static_assert(kStaged && MODE == APPLY, "the update runs in the staged APPLY epilogue");
    staged_finish<WGP, WGQ>(smem, G.fin[mat], tP, tQ, scale * cf.cbb, cf.lr, cf.lrwd, wave, lane,
                            wr, wc, acc);
    return;
  }
  if constexpr (kStaged) {
    if (MODE == GRAM || capt) {
      const float mult = MODE == GRAM ? alpha : MODE == POLY ? cf.cc : scale * cf.cbb;
      // GRAM and POLY outputs (A, B) tile-contiguous when the plan says so
      const int nbr = (MODE != APPLY && blk) ? G.mp / TS : 0;
      staged_store<MODE, WGP, WGQ>(smem, reinterpret_cast<uint16_t*>(out), ld_out, nbr, tP, tQ,
                                   mirror, mult, wave, lane, wr, wc, acc);
      return;
    }
  }
  // POLY and APPLY add a multiple of their input at the output positions:
  // load all of this lane's input values first, so the loads overlap each
  // other instead of each store waiting for its own load
  constexpr int NV = MODE == GRAM ? 1 : FP * FQ * 4;
  using V4 = typename std::conditional<XDT == kBF16, uint2, float4>::type;
  V4 pre[NV];
  if constexpr (MODE != GRAM) {
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FQ; ++j) {
        const int Q = tQ * TS + wc * WTQ + j * 32 + (lane & 31);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int P = tP * TS + wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
          pre[(i * FQ + j) * 4 + rg] =
              *reinterpret_cast<const V4*>(xin + static_cast<int64_t>(Q) * ld_out + P);
        }
      }
  }
#pragma unroll
  for (int i = 0; i < FP; ++i) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int Q = tQ * TS + wc * WTQ + j * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int P = tP * TS + wr * WTP + i * 32 + rg * 8 + (lane >> 5) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][rg * 4 + e];
        const int64_t qp = static_cast<int64_t>(Q) * ld_out + P;
        if constexpr (MODE == GRAM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= alpha;
        } else {
          float xv[4];
          unpack4(pre[(i * FQ + j) * 4 + rg], xv);
          if constexpr (MODE == POLY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = cf.cb * xv[e] + cf.cc * v[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = scale * (cf.ca * xv[e] + cf.cbb * v[e]);
          }
        }
        st4(out + qp, v);
        if (mirror) {
#pragma unroll
          for (int e = 0; e < 4; ++e) st1(out + static_cast<int64_t>(P + e) * ld_out + Q, v[e]);
        }
      }
    }
  }
}


template <int XDT, int MODE, int TS, int WGP, int WGQ, bool FIN>
__global__ __launch_bounds__(64 * WGP * WGQ, 1) void k_gemm(GemmArgs args) {
  constexpr int CPR = Ty<XDT>::CPR, NST = stages<XDT, TS>();
  constexpr int NW = WGP * WGQ;       // waves per block
  constexpr int OPB = TS * CPR * 16;  // LDS bytes per operand per stage

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * 2 * OPB];
  __shared__ float red[NW];

  // ---- locate group, matrix and tile
  GemmGroup G = args.g[0];
  int mat, tile;
  if (args.order & 4) {
    // matrices dealt to XCDs: matrix j of every group runs on XCD j mod 8;
    // block b is the (b / 8)-th block dispatched to XCD b mod 8
    const int x = static_cast<int>(blockIdx.x & 7);
    int i = static_cast<int>(blockIdx.x >> 3);
    int found = 0;
    mat = 0; tile = 0;
#pragma unroll
    for (int k = 0; k < kMaxGroups; ++k) {
      if (k < args.ngroups && !found) {
        const int n = (args.g[k].count + 7 - x) >> 3;
        const int nb = n * args.g[k].tiles;
        if (i < nb) {
          G = args.g[k];
          const int jm = i / G.tiles;
          mat = x + 8 * jm;
          tile = i - jm * G.tiles;
          found = 1;
        } else {
          i -= nb;
        }
      }
    }
    if (!found) return;
  } else {
    const int bid = (args.order & 1) ? static_cast<int>(blockIdx.x) : xcd_block();
    // constant-index selection keeps the group table in kernel-argument space
#pragma unroll
    for (int k = 1; k < kMaxGroups; ++k)
      if (k < args.ngroups && bid >= args.g[k].block_base) G = args.g[k];
    const int local = bid - G.block_base;
    mat = local / G.tiles;
    tile = local - mat * G.tiles;
  }
  int tP, tQ;
  if (MODE == APPLY && (args.order & 8)) {
    // column panels in turn, all row panels of each: the blocks of an XCD then
    // share a few X column panels and every B row panel of the matrix
    const int tm = G.mp / TS;
    tQ = tile % tm;
    tP = tile / tm;
  } else if (MODE == APPLY && (args.order & 2)) {
    tP = tile % (G.np / TS);
    tQ = tile / (G.np / TS);
  } else if (MODE == APPLY) {
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

  TileCoef cf;
  cf.ca = args.ca; cf.cb = args.cb; cf.cc = args.cc; cf.cbb = args.cbb;
  cf.eps = args.eps; cf.first = args.first;
  cf.lr = args.lr; cf.lrwd = args.lrwd;
  cf.ablk = args.ablk;
  cf.nofold = args.nofold;
  gemm_tile<XDT, MODE, TS, WGP, WGQ, FIN>(G, mat, tP, tQ, cf, smem, red);
}

// ---- all Newton-Schulz iterations of a small problem in one launch
//
// Grid-wide barrier between products.  Every thread releases its global
// stores at device scope (written back past its XCD's L2), one thread per
// block counts in and polls the arrival counter, and every thread then
// acquires at device scope (stale lines in its CU's and XCD's caches are
// dropped) before it reads what other blocks wrote.  The poll is bounded: a
// block that gives up sets the failure flag (the finish kernel then writes
// NaN) and goes on, so every block reaches the end of the kernel.  A limit of
// zero fails at once (the host forces the failure path that way).
__device__ __forceinline__ void grid_barrier(uint32_t* sync, uint32_t target, uint32_t limit) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t n = 0;
    while (limit == 0u ||
           __hip_atomic_load(&sync[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (n++ >= limit) {
        __hip_atomic_store(&sync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  __threadfence();
}

// The blocks take the tiles of each product (GRAM, POLY unless c = 0, APPLY)
// of each iteration in turn, block-strided over all groups, with the tile
// code of the multi-launch path (64-wide bf16 tiles), so the results are bit
// for bit those of the separate launches.  The last block out resets the
// counters for the next launch on the stream.
template <int WGP, int WGQ>
__global__ __launch_bounds__(64 * WGP * WGQ, 1) void k_ns_small(SmallArgs args) {
  constexpr int TS = 64, CPR = Ty<kBF16>::CPR, NST = stages<kBF16, TS>(), NW = WGP * WGQ;
  constexpr int OPB = TS * CPR * 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * 2 * OPB];
  __shared__ float red[NW];
  const int nb = static_cast<int>(gridDim.x);
  uint32_t target = 0;
  int cur = 0;
  for (int j = 0; j < args.steps; ++j) {
    TileCoef cf;
    cf.ca = args.coef[j][0]; cf.cb = args.coef[j][1]; cf.cc = args.coef[j][2];
    const bool poly = cf.cc != 0.f;
    cf.cbb = poly ? 1.f : cf.cb;
    cf.eps = args.eps; cf.first = j == 0;
    cf.lr = 0.f; cf.lrwd = 0.f; cf.ablk = 0; cf.nofold = 0;
    for (int ph = GRAM; ph <= APPLY; ++ph) {
      if (ph == POLY && !poly) continue;
#pragma unroll 1
      for (int t = static_cast<int>(blockIdx.x);; t += nb) {
        // group, matrix and tile of work item t (constant-index selection
        // keeps the group table in kernel-argument space)
        SmallGroup sg = args.g[0];
        int rem = t, tiles = 0, found = 0;
#pragma unroll
        for (int k = 0; k < kMaxGroups; ++k) {
          if (k < args.ngroups && !found) {
            const int tm = args.g[k].mp / TS, tn = args.g[k].np / TS;
            const int tk = ph == APPLY ? tm * tn : tm * (tm + 1) / 2;
            if (rem < args.g[k].count * tk) {
              sg = args.g[k];
              tiles = tk;
              found = 1;
            } else {
              rem -= args.g[k].count * tk;
            }
          }
        }
        if (!found) break;
        const int mat = rem / tiles, tile = rem - mat * tiles;
        const int tm = sg.mp / TS, tn = sg.np / TS;
        GemmGroup G;
        G.count = sg.count; G.mp = sg.mp; G.np = sg.np; G.tiles = tiles; G.block_base = 0;
        G.partials = sg.partials; G.p_stride = sg.npart; G.npartials = sg.npart;
        G.fin = nullptr; G.bop = nullptr; G.b_stride = 0;
        const void* xc = cur ? sg.x1 : sg.x0;
        void* xn = const_cast<void*>(cur ? sg.x0 : sg.x1);
        int tP, tQ;
        if (ph == APPLY) {
          G.xin = xc; G.bop = poly ? sg.b : sg.a; G.out = xn;
          G.in_stride = sg.x_elems; G.b_stride = sg.a_elems; G.out_stride = sg.x_elems;
          G.kdim = sg.kp;
          tP = tile % tn;
          tQ = tile / tn;
        } else {
          if (ph == GRAM) {
            G.xin = xc; G.out = sg.a; G.in_stride = sg.x_elems; G.out_stride = sg.a_elems;
            G.kdim = sg.kg;
          } else {
            G.xin = sg.a; G.out = sg.b; G.in_stride = sg.a_elems; G.out_stride = sg.a_elems;
            G.kdim = sg.kp;
          }
          int bi = 0, r = tile;
          while (r >= tm - bi) { r -= tm - bi; ++bi; }
          tP = bi;
          tQ = bi + r;
        }
        if (ph == GRAM) gemm_tile<kBF16, GRAM, TS, WGP, WGQ, false>(G, mat, tP, tQ, cf, smem, red);
        else if (ph == POLY) gemm_tile<kBF16, POLY, TS, WGP, WGQ, false>(G, mat, tP, tQ, cf, smem, red);
        else gemm_tile<kBF16, APPLY, TS, WGP, WGQ, false>(G, mat, tP, tQ, cf, smem, red);
        // the next tile's first loads refill stage buffers that a slower wave
        // may still be reading
        __syncthreads();
      }
      if (!(j == args.steps - 1 && ph == APPLY)) {
        target += static_cast<uint32_t>(nb);
        grid_barrier(args.sync, target, args.spin_limit);
      }
    }
    cur ^= 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(&args.sync[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == static_cast<uint32_t>(nb) - 1u) {
      // every other block is past its last poll
      __hip_atomic_store(&args.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&args.sync[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int XDT, int MODE>
hipError_t launch_ts(int ts, int waves, const GemmArgs& a, int64_t blocks, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(blocks));
  if constexpr (XDT == kBF16) {
    if (ts == 256 && waves == 8) {
      // GRAM: eight waves of 128 x 64 (two per SIMD).  POLY and APPLY: sixteen
      // waves of 64 x 64 (four per SIMD), which hide more of the stage latency
      // and are 1-4 % faster there; GRAM is 1-1.5 % slower with sixteen.
      if constexpr (MODE == GRAM) {
        hipLaunchKernelGGL((k_gemm<XDT, MODE, 256, 2, 4, false>), grid, dim3(512), 0, s, a);
      } else {
        if constexpr (MODE == APPLY) {
          if (a.fin) {
            if (a.cbb == 0.f) return hipErrorInvalidValue;   // needs the staged epilogue
            hipLaunchKernelGGL((k_gemm<XDT, MODE, 256, 4, 4, true>), grid, dim3(1024), 0, s, a);
            return hipGetLastError();
          }
        }
        hipLaunchKernelGGL((k_gemm<XDT, MODE, 256, 4, 4, false>), grid, dim3(1024), 0, s, a);
      }
      return hipGetLastError();
    }
  }
  if (a.fin) return hipErrorInvalidValue;
  if (ts == 128 && waves == 4)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 128, 2, 2, false>), grid, dim3(256), 0, s, a);
  else if (ts == 64 && waves == 4)
    hipLaunchKernelGGL((k_gemm<XDT, MODE, 64, 2, 2, false>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_small(const SmallArgs& a, int blocks, hipStream_t s) {
  if (blocks <= 0 || a.steps <= 0) return hipSuccess;
  if (a.steps > kSmallMaxSteps || a.ngroups < 1 || a.ngroups > kMaxGroups || !a.sync)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_ns_small<2, 2>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int phase, int xdt, int ts, int waves, const GemmArgs& a,
                       int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (xdt == kBF16) {
    if (phase == GRAM) return launch_ts<kBF16, GRAM>(ts, waves, a, blocks, s);
    if (phase == POLY) return launch_ts<kBF16, POLY>(ts, waves, a, blocks, s);
    return launch_ts<kBF16, APPLY>(ts, waves, a, blocks, s);
  }
  if (phase == GRAM) return launch_ts<kF32, GRAM>(ts, waves, a, blocks, s);
  if (phase == POLY) return launch_ts<kF32, POLY>(ts, waves, a, blocks, s);
  return launch_ts<kF32, APPLY>(ts, waves, a, blocks, s);
}

}  // namespace muon
