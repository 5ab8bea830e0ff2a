// Grouped Newton-Schulz GEMMs on gfx950 MFMA.
//
// One iteration of the odd polynomial X <- aX + (bA + cA^2)X, A = X X^T, on
// every matrix of an effective-shape group (the "several matrix products at
// parameter-update time" of page "きみはNanoGPT speedrunを知っているか？",
// section "おまけ"; the orthogonalisation itself is described in section
// "Muonとは").  Three grouped launches per iteration:
//   GRAM : A = alpha * X X^T            (alpha = s^2 on the first iteration)
//   POLY : B = b A + c A A              (skipped when c == 0)
//   APPLY: X' = scale * (a X + beta B X) (scale = s on the first iteration)
// where s = 1 / (||U||_F + eps) folds the Frobenius normalisation of the
// first iterate into the products.
//
// Tiling: square TS x TS output tiles, 256 threads as a 2 x 2 grid of waves,
// each wave (TS/2) x (TS/2) built from 32x32 MFMA blocks.  Operands are staged
// through LDS as "rows with the contraction index contiguous" (128-byte rows,
// 16-byte chunks XOR-swizzled by row), double-buffered with one barrier per
// K step.  GRAM and POLY are symmetric: only tiles on or above the diagonal
// run, and off-diagonal tiles also store their mirror image.  APPLY contracts
// over the rows of X, so its X operand is transposed in registers on the way
// into LDS.  The MFMA output layout gives each lane four consecutive rows of
// one column; the tiles are arranged so that those four values are
// contiguous in memory (row Q, columns P..P+3 of the stored matrix).
#include "muon_common.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16-byte chunk as a native vector (plain loads and stores, promotable to registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { GRAM = 0, POLY = 1, APPLY = 2 };

template <int XDT> struct Ty;
template <> struct Ty<kBF16> {
  using T = uint16_t;
  static constexpr int E = 8;    // elements per 16-byte chunk
  static constexpr int BK = 64;  // contraction elements per K step (128-byte rows)
};
template <> struct Ty<kF32> {
  using T = float;
  static constexpr int E = 4;
  static constexpr int BK = 32;
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row << 7) + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
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
__device__ __forceinline__ float matrix_scale(const float* partials, int count, float eps,
                                              float* red) {
  float acc = 0.f;
  for (int i = threadIdx.x; i < count; i += kThreads) acc += partials[i];
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  const float s = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return 1.0f / (sqrtf(s) + eps);
}

// Transpose of an E x E block held as E rows of one 16-byte chunk each:
// in[q] = row q (E elements), out[c] = column c (E elements).
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out, uint16_t) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint32_t r[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = in[2 * h][w];
      const uint32_t hi = in[2 * h + 1][w];
      r[h] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    out[c] = u32x4{r[0], r[1], r[2], r[3]};
  }
}
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out, float) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = in[q][c];
    out[c] = u32x4{r[0], r[1], r[2], r[3]};
  }
}

template <typename T> struct Chunk { static constexpr int E = 16 / sizeof(T); };

// Global -> registers for one K step.  K-contiguous operands: thread t takes
// chunk (t & 7) of rows (t >> 3) + 32u.  The transposed APPLY operand: E x E
// sub-blocks, E rows of one chunk each.
template <typename T, int MODE, int TS>
__device__ __forceinline__ void gemm_gload(const T* pa, const T* pb, int lda, int ldb, int k0,
                                           int t, u32x4* ra, u32x4* rb) {
  constexpr int E = Chunk<T>::E;
  constexpr int NCH = TS / 32;
  constexpr int NSB = 8 * (TS / E);
  constexpr int NSBT = (NSB + kThreads - 1) / kThreads;
  if constexpr (MODE == APPLY) {
#pragma unroll
    for (int v = 0; v < NSBT; ++v) {
      const int sb = t + v * kThreads;
      if (NSB % kThreads == 0 || sb < NSB) {
        const int kc = sb / (TS / E), pc = sb - kc * (TS / E);
        const T* src = pa + static_cast<int64_t>(k0 + kc * E) * lda + pc * E;
#pragma unroll
        for (int q = 0; q < E; ++q)
          ra[v * E + q] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(q) * lda);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int row = (t >> 3) + 32 * u, c = t & 7;
      ra[u] = *reinterpret_cast<const u32x4*>(pa + static_cast<int64_t>(row) * lda + k0 + c * E);
    }
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int row = (t >> 3) + 32 * u, c = t & 7;
    rb[u] = *reinterpret_cast<const u32x4*>(pb + static_cast<int64_t>(row) * ldb + k0 + c * E);
  }
}

// Registers -> LDS stage `buf` (layout [A | B] per stage, 128-byte rows).
template <typename T, int MODE, int TS>
__device__ __forceinline__ void gemm_swrite(uint8_t* smem, int buf, int t, const u32x4* ra,
                                            const u32x4* rb) {
  constexpr int E = Chunk<T>::E;
  constexpr int NCH = TS / 32;
  constexpr int NSB = 8 * (TS / E);
  constexpr int NSBT = (NSB + kThreads - 1) / kThreads;
  constexpr int OPB = TS * 128;
  uint8_t* sa = smem + buf * 2 * OPB;
  uint8_t* sbp = sa + OPB;
  if constexpr (MODE == APPLY) {
#pragma unroll
    for (int v = 0; v < NSBT; ++v) {
      const int sb = t + v * kThreads;
      if (NSB % kThreads == 0 || sb < NSB) {
        const int kc = sb / (TS / E), pc = sb - kc * (TS / E);
        u32x4 col[E];
        transpose_block(ra + v * E, col, T());
#pragma unroll
        for (int c = 0; c < E; ++c)
          *reinterpret_cast<u32x4*>(sa + lds_off(pc * E + c, kc)) = col[c];
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int row = (t >> 3) + 32 * u, c = t & 7;
      *reinterpret_cast<u32x4*>(sa + lds_off(row, c)) = ra[u];
    }
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int row = (t >> 3) + 32 * u, c = t & 7;
    *reinterpret_cast<u32x4*>(sbp + lds_off(row, c)) = rb[u];
  }
}

// MFMA over one LDS stage.  bf16: 32x32x16, lane halves hold contraction
// elements 0-7 and 8-15 of each 16-step.  fp32: 32x32x2, lane half h feeds
// elements 8h..8h+7 of each 16-step over eight instructions.
template <int XDT, int TS>
__device__ __forceinline__ void gemm_compute(const uint8_t* sa, int lane, int wr, int wc,
                                             f32x16_t (&acc)[TS / 64][TS / 64]) {
  constexpr int WT = TS / 2, F = WT / 32, OPB = TS * 128;
  const uint8_t* sbp = sa + OPB;
  const int l32 = lane & 31, hl = lane >> 5;
  if constexpr (XDT == kBF16) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + hl;
      bf16x8_t fa[F], fb[F];
#pragma unroll
      for (int f = 0; f < F; ++f)
        fa[f] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off(wr * WT + f * 32 + l32, ch));
#pragma unroll
      for (int f = 0; f < F; ++f)
        fb[f] = *reinterpret_cast<const bf16x8_t*>(sbp + lds_off(wc * WT + f * 32 + l32, ch));
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int ch = 4 * g2 + 2 * hl;
      float fa[F][8], fb[F][8];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int ra_ = wr * WT + f * 32 + l32, rb_ = wc * WT + f * 32 + l32;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(sa + lds_off(ra_, ch));
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(sa + lds_off(ra_, ch + 1));
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(sbp + lds_off(rb_, ch));
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(sbp + lds_off(rb_, ch + 1));
        fa[f][0] = a0.x; fa[f][1] = a0.y; fa[f][2] = a0.z; fa[f][3] = a0.w;
        fa[f][4] = a1.x; fa[f][5] = a1.y; fa[f][6] = a1.z; fa[f][7] = a1.w;
        fb[f][0] = b0.x; fb[f][1] = b0.y; fb[f][2] = b0.z; fb[f][3] = b0.w;
        fb[f][4] = b1.x; fb[f][5] = b1.y; fb[f][6] = b1.z; fb[f][7] = b1.w;
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
          for (int j = 0; j < F; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
    }
  }
}

template <int XDT, int MODE, int TS>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs args) {
  using T = typename Ty<XDT>::T;
  constexpr int E = Ty<XDT>::E;
  constexpr int BK = Ty<XDT>::BK;
  constexpr int WT = TS / 2;          // wave tile edge
  constexpr int F = WT / 32;          // 32x32 MFMA blocks per wave edge
  constexpr int OPB = TS * 128;       // LDS bytes per operand per stage
  constexpr int NCH = TS / 32;        // K-contiguous chunks per thread per stage
  constexpr int NSB = 8 * (TS / E);   // transposed E x E sub-blocks per stage
  constexpr int NSBT = (NSB + kThreads - 1) / kThreads;
  constexpr int NA = MODE == APPLY ? NSBT * E : NCH;   // A-operand staging chunks

  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * OPB];
  __shared__ float red[4];

  // ---- locate group, matrix and tile
  const int bid = blockIdx.x;
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
    const int tn = G.np / TS;
    tP = tile % tn;
    tQ = tile / tn;
  } else {
    const int tm = G.mp / TS;
    int bi = 0, rem = tile;
    while (rem >= tm - bi) { rem -= tm - bi; ++bi; }
    tP = bi;
    tQ = bi + rem;
  }

  const T* xin = static_cast<const T*>(G.xin) + static_cast<int64_t>(mat) * G.in_stride;
  T* out = static_cast<T*>(G.out) + static_cast<int64_t>(mat) * G.out_stride;
  const T* pa;
  const T* pb;
  int lda, ldb, K;
  if (MODE == GRAM) {
    K = G.np; lda = ldb = G.np;
    pa = xin + static_cast<int64_t>(tP) * TS * G.np;
    pb = xin + static_cast<int64_t>(tQ) * TS * G.np;
  } else if (MODE == POLY) {
    K = G.mp; lda = ldb = G.mp;
    pa = xin + static_cast<int64_t>(tP) * TS * G.mp;
    pb = xin + static_cast<int64_t>(tQ) * TS * G.mp;
  } else {
    K = G.mp; lda = G.np; ldb = G.mp;
    pa = xin + static_cast<int64_t>(tP) * TS;     // rows are k, columns P
    pb = static_cast<const T*>(G.bop) + static_cast<int64_t>(mat) * G.b_stride +
         static_cast<int64_t>(tQ) * TS * G.mp;
  }

  float scale = 1.f;
  if (args.first) scale = matrix_scale(G.partials + static_cast<int64_t>(mat) * G.p_stride,
                                       G.npartials, args.eps, red);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  u32x4 ra[NA], rb[NCH];
  f32x16_t acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  gemm_gload<T, MODE, TS>(pa, pb, lda, ldb, 0, t, ra, rb);
  gemm_swrite<T, MODE, TS>(smem, 0, t, ra, rb);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gemm_gload<T, MODE, TS>(pa, pb, lda, ldb, (kt + 1) * BK, t, ra, rb);
    gemm_compute<XDT, TS>(smem + (kt & 1) * 2 * OPB, lane, wr, wc, acc);
    if (more) gemm_swrite<T, MODE, TS>(smem, (kt + 1) & 1, t, ra, rb);
    __syncthreads();
  }

  // ---- epilogue
  const int ld_out = MODE == APPLY ? G.np : G.mp;
  const float alpha = MODE == GRAM ? scale * scale : 1.f;
  const bool mirror = MODE != APPLY && tP != tQ;
#pragma unroll
  for (int i = 0; i < F; ++i) {
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int Q = tQ * TS + wc * WT + j * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int P = tP * TS + wr * WT + i * 32 + rg * 8 + (lane >> 5) * 4;
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
#pragma unroll
          for (int e = 0; e < 4; ++e) st1(out + static_cast<int64_t>(P + e) * ld_out + Q, v[e]);
        }
      }
    }
  }
}

template <int XDT, int MODE>
hipError_t launch_ts(int ts, const GemmArgs& a, int64_t blocks, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kThreads);
  switch (ts) {
    case 256: hipLaunchKernelGGL((k_gemm<XDT, MODE, 256>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_gemm<XDT, MODE, 128>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm<XDT, MODE, 64>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int phase, int xdt, int ts, const GemmArgs& a, int64_t blocks,
                       hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (xdt == kBF16) {
    if (phase == GRAM) return launch_ts<kBF16, GRAM>(ts, a, blocks, s);
    if (phase == POLY) return launch_ts<kBF16, POLY>(ts, a, blocks, s);
    return launch_ts<kBF16, APPLY>(ts, a, blocks, s);
  }
  if (phase == GRAM) return launch_ts<kF32, GRAM>(ts, a, blocks, s);
  if (phase == POLY) return launch_ts<kF32, POLY>(ts, a, blocks, s);
  return launch_ts<kF32, APPLY>(ts, a, blocks, s);
}

}  // namespace muon
