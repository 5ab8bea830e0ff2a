// Elementwise kernels of the Muon step on gfx950: HBM-bound, one pass each.
//
//   prepare  : momentum (moving average of the gradient; page
//              "きみはNanoGPT speedrunを知っているか？", section "Muonとは"),
//              optional slow momentum (page "Training NanoGPT in 39.9
//              Seconds", section "ANVIL II와 가중치 평균"), optional Nesterov
//              look-ahead, cast of U to the iterate type, transposition of
//              tall matrices to the wide orientation, and one partial sum of
//              squares per 64x64 tile for the Frobenius norm.
//   finish   : the update W <- W - lr*wd*mask*W - lr*O with the cautious mask
//              [W*S > 0], the weight average E <- beta E + (1-beta) W (that
//              section's displayed equation), diagnostics; or, for the
//              orthogonalise-only entry point, a store of O.
//   blend    : readout mix w_final*W + (1-w_final)*E (same section).
//
// The fp32 state recurrences must be reproducible bit for bit, so this file
// forbids contraction: every product and sum is rounded on its own.
#pragma clang fp contract(off)

#include "muon_common.h"

namespace muon {
namespace {

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN becomes a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ int find_mat(const int64_t* prefix, int n, int64_t b) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Deterministic block sum: wave butterfly, then the four wave totals in order.
__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = ((red[0] + red[1]) + red[2]) + red[3];
  return s;
}

// 16 contiguous values from a row of bf16 or fp32 data.
__device__ __forceinline__ void load16(const void* row, int dt, bool vec, int valid,
                                       float* v) {
  if (vec && valid >= 16) {
    if (dt == kBF16) {
      const uint4* p = reinterpret_cast<const uint4*>(row);
      uint4 q[2] = {p[0], p[1]};
      const uint32_t* w = reinterpret_cast<const uint32_t*>(q);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(row);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float4 q = p[k];
        v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < valid)
        v[k] = dt == kBF16 ? bf2f(static_cast<const uint16_t*>(row)[k])
                           : static_cast<const float*>(row)[k];
      else
        v[k] = 0.f;
    }
  }
}

// Store 16 values to a row of bf16 (RNE) or fp32 data; returns stored values.
__device__ __forceinline__ void store16(void* row, int dt, bool vec, int valid,
                                        float* v) {
  if (dt == kBF16) {
    uint16_t h[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) { h[k] = f2bf(v[k]); v[k] = bf2f(h[k]); }
    if (vec && valid >= 16) {
      uint4* p = reinterpret_cast<uint4*>(row);
      const uint4* q = reinterpret_cast<const uint4*>(h);
      p[0] = q[0];
      p[1] = q[1];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < valid) static_cast<uint16_t*>(row)[k] = h[k];
    }
  } else {
    if (vec && valid >= 16) {
      float4* p = reinterpret_cast<float4*>(row);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        p[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < valid) static_cast<float*>(row)[k] = v[k];
    }
  }
}

__device__ __forceinline__ void loadf16(const float* row, bool vec, int valid, float* v) {
  load16(row, kF32, vec, valid, v);
}
__device__ __forceinline__ void storef16(float* row, bool vec, int valid, float* v) {
  store16(row, kF32, vec, valid, v);
}

// Matrix scale s = 1 / (sqrt(sum of partials) + eps); same order everywhere.
__device__ __forceinline__ float matrix_scale(const float* partials, int count, float eps,
                                              float* red) {
  float acc = 0.f;
  for (int i = threadIdx.x; i < count; i += kThreads) acc += partials[i];
  float s = block_sum(acc, red);
  return 1.0f / (sqrtf(s) + eps);
}

// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_prepare(ElemArgs a) {
  __shared__ float tile[kEw][kEw + 1];
  __shared__ float red[4];
  const int64_t b = blockIdx.x;
  const int mi = find_mat(a.prefix, a.nmats, b);
  const MatDesc& d = a.mats[mi];
  const int local = static_cast<int>(b - a.prefix[mi]);
  const int tpr = d.np / kEw;
  const int ti = local / tpr, tj = local - ti * tpr;
  const int tall = d.tall;
  const int sr0 = tall ? tj * kEw : ti * kEw;
  const int sc0 = tall ? ti * kEw : tj * kEw;
  const int t = threadIdx.x, lr = t >> 2, lc0 = (t & 3) * 16;
  const int sr = sr0 + lr, sc = sc0 + lc0;
  const int valid = sr < d.rows ? max(0, min(16, d.cols - sc)) : 0;

  float u[16];
  if (a.mode == 0) {
    float g[16], m[16];
    const int64_t gi = static_cast<int64_t>(sr) * d.ldg + sc;
    const int64_t di = static_cast<int64_t>(sr) * d.cols + sc;
    const char* grow = static_cast<const char*>(d.g) + gi * (d.gdt == kBF16 ? 2 : 4);
    if (valid > 0) {
      load16(grow, d.gdt, d.gvec, valid, g);
      loadf16(d.mom + di, d.dvec, valid, m);
#pragma unroll
      for (int k = 0; k < 16; ++k) m[k] = a.beta * m[k] + a.obeta * g[k];
      storef16(d.mom + di, d.dvec, valid, m);
      if (a.use_slow) {
        float s[16];
        loadf16(d.slow + di, d.dvec, valid, s);
#pragma unroll
        for (int k = 0; k < 16; ++k) s[k] = a.bslow * s[k] + a.obslow * g[k];
        storef16(d.slow + di, d.dvec, valid, s);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        u[k] = a.nesterov ? a.beta * m[k] + a.obeta * g[k] : m[k];
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) u[k] = 0.f;
    }
  } else {
    const int64_t gi = static_cast<int64_t>(sr) * d.ldg + sc;
    const char* grow = static_cast<const char*>(d.g) + gi * (d.gdt == kBF16 ? 2 : 4);
    if (valid > 0) {
      load16(grow, d.gdt, d.gvec, valid, u);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) u[k] = 0.f;
    }
  }
  // entries past the valid run are zero already; sum of squares of U
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) ss = ss + u[k] * u[k];

  if (tall) {
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[lr][lc0 + k] = u[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = tile[lc0 + k][lr];
  }
  // X0 row (ti*64 + lr), columns (tj*64 + lc0 ...), ld = np, always in bounds
  const int64_t xi = static_cast<int64_t>(ti * kEw + lr) * d.np + tj * kEw + lc0;
  char* xrow = static_cast<char*>(d.x0) + xi * (a.xdt == kBF16 ? 2 : 4);
  store16(xrow, a.xdt, true, 16, u);

  const float tot = block_sum(ss, red);
  if (t == 0) d.partials[local] = tot;
}

// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finish(ElemArgs a) {
  __shared__ float tile[kEw][kEw + 1];
  __shared__ float red[4];
  const int64_t b = blockIdx.x;
  const int mi = find_mat(a.prefix, a.nmats, b);
  const MatDesc& d = a.mats[mi];
  const int local = static_cast<int>(b - a.prefix[mi]);
  const int tpr = (d.cols + kEw - 1) / kEw;
  const int fi = local / tpr, fj = local - fi * tpr;
  const int t = threadIdx.x, lr = t >> 2, lc0 = (t & 3) * 16;
  const int sr = fi * kEw + lr, sc = fj * kEw + lc0;
  const int esz = a.xdt == kBF16 ? 2 : 4;
  const void* xb = a.final_buf ? d.x1 : d.x0;

  float o[16];
  if (d.tall) {
    // O[sr][sc] = X[sc][sr]; stage X rows (fj*64 + lr), cols (fi*64 + lc0..)
    const int64_t xi = static_cast<int64_t>(fj * kEw + lr) * d.np + fi * kEw + lc0;
    float v[16];
    load16(static_cast<const char*>(xb) + xi * esz, a.xdt, true, 16, v);
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[lr][lc0 + k] = v[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = tile[lc0 + k][lr];
  } else {
    const int64_t xi = static_cast<int64_t>(sr) * d.np + sc;
    load16(static_cast<const char*>(xb) + xi * esz, a.xdt, true, 16, o);
  }
  if (a.scale_o) {
    const float s = matrix_scale(d.partials, d.npartials, a.eps, red);
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = s * o[k];
  }
  const int valid = sr < d.rows ? max(0, min(16, d.cols - sc)) : 0;
  if (valid <= 0) return;

  const int64_t wi = static_cast<int64_t>(sr) * d.ldw + sc;
  char* wrow = static_cast<char*>(d.w) + wi * (d.wdt == kBF16 ? 2 : 4);
  const int64_t di = static_cast<int64_t>(sr) * d.cols + sc;
  if (a.mode == 1) {            // orthogonalize: out = O
    store16(wrow, d.wdt, d.wvec, valid, o);
    return;
  }
  float w[16], mk[16];
  load16(wrow, d.wdt, d.wvec, valid, w);
  if (a.cautious) {
    float s[16];
    loadf16(d.slow + di, d.dvec, valid, s);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      mk[k] = ((w[k] > 0.f && s[k] > 0.f) || (w[k] < 0.f && s[k] < 0.f)) ? 1.f : 0.f;
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) mk[k] = 1.f;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float dk = mk[k] != 0.f ? a.lrwd : 0.f;
    w[k] = (w[k] - dk * w[k]) - a.lr * o[k];
  }
  store16(wrow, d.wdt, d.wvec, valid, w);   // w now holds the stored values
  if (a.ema_on) {
    float e[16];
    if (a.ema_first) {
#pragma unroll
      for (int k = 0; k < 16; ++k) e[k] = w[k];
    } else {
      loadf16(d.ema + di, d.dvec, valid, e);
#pragma unroll
      for (int k = 0; k < 16; ++k) e[k] = a.bema * e[k] + a.obema * w[k];
    }
    storef16(d.ema + di, d.dvec, valid, e);
  }
  if (d.mask_out) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < valid) d.mask_out[di + k] = mk[k] != 0.f ? 1 : 0;
  }
  if (d.upd_out) storef16(d.upd_out + di, d.dvec, valid, o);
}

// --------------------------------------------------------------------------
// Readout blend: w slot = output, g slot = parameters, ema = average.
__global__ __launch_bounds__(kThreads) void k_blend(ElemArgs a, float wf, float owf) {
  const int64_t b = blockIdx.x;
  const int mi = find_mat(a.prefix, a.nmats, b);
  const MatDesc& d = a.mats[mi];
  const int local = static_cast<int>(b - a.prefix[mi]);
  const int tpr = (d.cols + kEw - 1) / kEw;
  const int fi = local / tpr, fj = local - fi * tpr;
  const int t = threadIdx.x, lr = t >> 2, lc0 = (t & 3) * 16;
  const int sr = fi * kEw + lr, sc = fj * kEw + lc0;
  const int valid = sr < d.rows ? max(0, min(16, d.cols - sc)) : 0;
  if (valid <= 0) return;
  float w[16], e[16];
  const int64_t gi = static_cast<int64_t>(sr) * d.ldg + sc;
  load16(static_cast<const char*>(d.g) + gi * (d.gdt == kBF16 ? 2 : 4), d.gdt, d.gvec, valid, w);
  loadf16(d.ema + static_cast<int64_t>(sr) * d.cols + sc, d.dvec, valid, e);
#pragma unroll
  for (int k = 0; k < 16; ++k) w[k] = wf * w[k] + owf * e[k];
  const int64_t wi = static_cast<int64_t>(sr) * d.ldw + sc;
  store16(static_cast<char*>(d.w) + wi * (d.wdt == kBF16 ? 2 : 4), d.wdt, d.wvec, valid, w);
}

}  // namespace

hipError_t launch_prepare(const ElemArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepare, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finish(const ElemArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finish, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_blend(const ElemArgs& a, int64_t blocks, float wf, float owf,
                        hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_blend, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, a,
                     wf, owf);
  return hipGetLastError();
}

}  // namespace muon
