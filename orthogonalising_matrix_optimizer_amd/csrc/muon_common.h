// Shared host/device definitions of the Muon step library (gfx950).
//
// Data layout in the caller's workspace (all offsets 256-byte aligned):
//   * per matrix, the Newton-Schulz iterate X in its wide orientation
//     (m = min(rows, cols), n = max(rows, cols)), zero-padded to mp x np with
//     mp, np multiples of the group's tile edge, row-major, ld = np; two such
//     buffers (ping-pong);
//   * per matrix, the m x m Gram matrix A and polynomial B, padded to mp x mp;
//   * per matrix, one fp32 partial sum of squares per 64x64 prepare tile;
//   * the device descriptor table (MatDesc[n]) and tile prefix sums.
// Zero padding stays zero through every product (zero rows and columns of X
// give zero rows and columns of A, B and the next X), so the GEMM kernels run
// on full tiles only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kThreads = 256;     // threads per block (elementwise kernels but prepare)
constexpr int kPrepThreads = 512; // threads per block of the prepare kernel
constexpr int kEw = 64;           // edge of the elementwise (prepare/finish) tiles
// row strips of the elementwise kernels for matrices kept in their layout;
// a strip holds as many elements as a tile, so both give the same partial count
constexpr int kStripRows = 32, kStripCols = 128;
static_assert(kStripRows * kStripCols == kEw * kEw, "strip and tile sizes");
constexpr int kMaxGroups = 8;     // effective-shape groups per grouped launch

enum ElemType : int32_t { kBF16 = 0, kF32 = 1 };

// Per-matrix descriptor, resident in the workspace.
struct MatDesc {
  void* w;              // parameters (rows x cols, ldw)
  const void* g;        // gradient (rows x cols, ldg); input matrix for orthogonalize
  float* mom;           // momentum, dense rows x cols
  float* slow;          // slow momentum or null
  float* ema;           // weight average or null
  uint8_t* mask_out;    // diagnostic or null
  float* upd_out;       // diagnostic or null
  void* x0;             // ping-pong iterate buffers (mp x np, ld np)
  void* x1;
  float* partials;      // prepare-tile partial sums of squares
  int64_t ldw, ldg;
  int32_t rows, cols;   // source shape
  int32_t mp, np;       // padded effective shape
  int32_t tall;         // rows > cols: X = U^T
  int32_t wdt, gdt;     // element types of w and g
  int32_t wvec, gvec;   // 16-byte vector access allowed on w / g rows
  int32_t dvec;         // dense fp32 rows (mom, slow, ema, upd) allow float4 access
  int32_t npartials;
  int32_t _pad;
};

// Kernel arguments of the elementwise kernels.
struct ElemArgs {
  const MatDesc* mats;
  const int64_t* prefix;   // block prefix sums per matrix (n + 1 entries)
  int32_t nmats;
  int32_t xdt;             // element type of the iterate
  float beta, obeta;       // momentum and (1 - beta), fp32
  float bslow, obslow;     // slow momentum and (1 - beta_slow)
  float bema, obema;       // weight average and (1 - beta_ema)
  float lr, lrwd;          // lr and fl(lr * wd)
  float eps;
  int32_t mode;            // prepare: 0 step, 1 copy; finish: 0 step, 1 write O
  int32_t nesterov, cautious, use_slow;
  int32_t ema_on, ema_first;
  int32_t final_buf;       // iterate buffer holding O (0 -> x0, 1 -> x1)
  int32_t scale_o;         // steps == 0: O = s * X0
  const uint32_t* ns_err;  // finish: nonzero flag here = the iterations failed
                           // (single-launch path), O is taken as NaN; or null
};

// A parameter matrix updated in the last APPLY's epilogue (plain update,
// bf16 W): W <- (W - lrwd W) - lr O.
struct FinDesc {
  void* w;                // W, bf16, row-major, 16-byte aligned rows
  int64_t ldw;            // elements between W rows (multiple of 8)
  int32_t rows, cols;     // W's shape (multiples of 8)
  int32_t tall;           // the iterate is W transposed
  int32_t _pad;
};

// One effective-shape group inside a grouped GEMM launch.
struct GemmGroup {
  const void* xin;        // GRAM: X; POLY: A; APPLY: X
  const void* bop;        // APPLY: B (or A for a cubic step); otherwise unused
  void* out;              // GRAM: A; POLY: B; APPLY: next X
  const float* partials;  // first iteration: per-matrix norm partials
  int64_t in_stride;      // elements between consecutive matrices of xin
  int64_t b_stride;       // ... of bop
  int64_t out_stride;     // ... of out
  int64_t p_stride;       // floats between consecutive matrices' partials
  int32_t count;          // matrices in the group
  int32_t mp, np;
  int32_t tiles;          // tiles per matrix
  int32_t block_base;     // first block of this group in the launch
  int32_t npartials;
  int32_t kdim;           // contraction length run by the K loop: the unpadded
                          // contraction dimension rounded up to 128 (n for GRAM,
                          // m for POLY and APPLY); the zero padding beyond it
                          // contributes nothing
  const FinDesc* fin;     // fused update: one entry per matrix of the group
};

struct GemmArgs {
  GemmGroup g[kMaxGroups];
  int32_t ngroups;
  int32_t first;          // first iteration: fold the norm scale s in
  float ca, cb, cc;       // coefficients of this iteration
  float cbb;              // APPLY: multiplier of the product (1, or b when B = bA)
  float eps;
  int32_t order;          // bit 0: plain block order (no XCD grouping);
                          // bit 1: row-major APPLY tile order;
                          // bit 2: whole matrices dealt to XCDs (j on j mod 8);
                          // bit 3: APPLY tiles by column panel
  int32_t fin;            // APPLY (256-wide bf16, beta != 0): update W instead of
                          // storing the iterate (the group's fin table)
  float lr, lrwd;         // fused update: lr and fl(lr * wd)
  int32_t ablk;           // 256-wide bf16 tiles: A and B stored tile-contiguous
                          // (256 x 64 blocks, see blk_off in the GEMM source)
  int32_t nofold;         // 256-wide bf16 tiles: add the input term at the store
                          // instead of folding it into the accumulators (for
                          // coefficient ratios that could overflow them)
};

// All Newton-Schulz iterations of a small problem (64-wide bf16 tiles) in one
// launch: per effective-shape group the workspace buffers, per iteration the
// coefficients; the blocks take the tiles of each product in turn and meet at
// a grid-wide barrier between products.
constexpr int kSmallMaxSteps = 16;
struct SmallGroup {
  const void* x0;         // iterate buffers (ping-pong), bf16 mp x np
  const void* x1;
  void* a;                // Gram matrix A, bf16 mp x mp
  void* b;                // polynomial B, bf16 mp x mp
  const float* partials;  // norm partials of the first iteration
  int64_t x_elems, a_elems;
  int32_t count, mp, np, npart;
  int32_t kg, kp;         // K loop lengths: GRAM (n rounded to 128), POLY and APPLY (m)
};
struct SmallArgs {
  SmallGroup g[kMaxGroups];
  int32_t ngroups, steps;
  float eps;
  uint32_t spin_limit;        // barrier polls before a block gives up (sets the flag)
  float coef[kSmallMaxSteps][3];
  uint32_t* sync;             // [0] barrier arrivals, [1] blocks done, [2] failure flag
};

}  // namespace muon

// Launchers (defined in the .hip sources; called by the C ABI layer).
namespace muon {
// AdamW over flat tensors: descriptor per tensor (resident in the workspace)
// and kernel arguments.  Blocks take kAdamChunk consecutive elements.
constexpr int kAdamChunk = 4096;
struct VecDesc {
  void* p;              // parameters (numel elements)
  const void* g;        // gradient
  float* m;             // first moment
  float* v;             // second moment
  int64_t n;            // numel
  int32_t pdt, gdt;     // element types of p and g
  int32_t pvec, gvec;   // 16-byte aligned p / g (vector access)
  int32_t svec;         // 16-byte aligned m and v
  int32_t _pad;
};
struct AdamArgs {
  const VecDesc* vecs;
  const int64_t* prefix;   // block prefix sums per tensor (n + 1 entries)
  int32_t nvec;
  float b1, ob1, b2, ob2;  // betas and (1 - beta), fp32
  float step_size;         // lr / (1 - b1^t)
  float rsc2;              // 1 / sqrt(1 - b2^t)
  float eps, lrwd;         // eps; lr * wd
};
hipError_t launch_adamw(const AdamArgs& a, int64_t blocks, hipStream_t s);

hipError_t launch_prepare(const ElemArgs& a, int64_t blocks, hipStream_t s);
hipError_t launch_finish(const ElemArgs& a, int64_t blocks, hipStream_t s);
hipError_t launch_blend(const ElemArgs& a, int64_t blocks, float wf, float owf,
                        hipStream_t s);
// Write `n` bytes (a multiple of 4) of a host table to device memory at `dst`
// (4-byte aligned) with kernels that carry the bytes as arguments: no host
// staging memory, ordered on the stream like the launches that read it.
hipError_t launch_put_table(void* dst, const uint8_t* bytes, size_t n, hipStream_t s);
// phase: 0 GRAM, 1 POLY, 2 APPLY; ts: tile edge (64, 128; 256 for bf16 only);
// waves: 8 for 256-wide tiles, else 4.
hipError_t launch_ns_small(const SmallArgs& a, int blocks, hipStream_t s);
hipError_t launch_gemm(int phase, int xdt, int ts, int waves, const GemmArgs& a,
                       int64_t blocks, hipStream_t s);
}  // namespace muon
