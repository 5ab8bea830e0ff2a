// C ABI of the Muon step library: validation, planning, launch sequencing.
//
// The method and its options are stated in include/muon.h.  This file holds
// no arithmetic of the step; it checks arguments, groups the matrices by
// effective shape (m, n) = (min(rows, cols), max(rows, cols)), lays out the
// caller's workspace, keeps the device descriptor table current and enqueues
// the kernels on the caller's stream:
//   prepare -> [GRAM -> (POLY) -> APPLY] x steps -> finish.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <cstdio>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/muon.h"
#include "muon_common.h"

using namespace muon;

namespace {

constexpr size_t kAlign = 256;
constexpr int kCUs = 256;
// descriptor-table regions of the workspace
constexpr int kTabEager = 0, kTabCapture = 1;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int esize(int dt) { return dt == MUON_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- planning
struct GroupPlan {
  int m = 0, n = 0, mp = 0, np = 0;
  int fin_base = 0;                 // first entry of the group in the fused-update table
  std::vector<int> mats;
  size_t off_x0 = 0, off_x1 = 0, off_a = 0, off_b = 0, off_part = 0;
  int64_t x_elems = 0, a_elems = 0;
  int npart = 0;
};

struct Plan {
  int xdt = MUON_BF16;
  int ts = 256;
  int waves = 4;
  // block order per phase (GRAM, POLY, APPLY): bit 0 plain order (no per-XCD
  // tile ranges), bit 1 row-major APPLY tiles (else groups of four row
  // panels), bit 2 whole matrices dealt to XCDs (matrix j on XCD j mod 8),
  // bit 3 APPLY tiles column panel by column panel
  int order[3] = {1, 1, 1};
  std::vector<int> launch_groups;   // groups in launch order: costliest tiles first
  std::vector<GroupPlan> groups;
  std::vector<int> mat_group, mat_slot;
  // descriptor table: offsets inside one table region, and the regions
  // themselves (kTabEager: sent by every uncaptured call; kTabCapture: sent by
  // muon_step_prepare only and read by captured steps, so no eager call on the
  // same workspace can change what a replay reads)
  size_t off_desc = 0, off_pprefix = 0, off_fprefix = 0, off_fin = 0, tab_bytes = 0;
  // three words of the single-launch Newton-Schulz path (barrier arrivals,
  // blocks done, failure flag): zero in every table sent
  size_t off_sync = 0;
  size_t off_tab[2] = {0, 0};
  size_t total = 0;
  std::vector<int64_t> pprefix, fprefix;
  // every padded iterate is addressable by the GEMMs' 32-bit buffer offsets
  bool fits = true;
};

// Whether dealing whole matrices to the eight XCDs (matrix j of every group
// on XCD j mod 8) gives each XCD within 5% of the mean work in every launch
// set of a phase (0 GRAM, 1 POLY, 2 APPLY).
bool xcd_deal_balanced(const Plan& p, int phase) {
  for (size_t g0 = 0; g0 < p.groups.size(); g0 += kMaxGroups) {
    const size_t g1 = std::min(p.groups.size(), g0 + kMaxGroups);
    double cost[8] = {0, 0, 0, 0, 0, 0, 0, 0}, tot = 0;
    for (size_t gi = g0; gi < g1; ++gi) {
      const GroupPlan& g = p.groups[p.launch_groups[gi]];
      const int tm = g.mp / p.ts, tn = g.np / p.ts;
      const double unit = phase == 2 ? double(tm) * tn * g.mp
                                     : double(tm) * (tm + 1) / 2 * (phase == 0 ? g.np : g.mp);
      const int c = int(g.mats.size());
      for (int x = 0; x < 8; ++x) cost[x] += ((c + 7 - x) / 8) * unit;
      tot += c * unit;
    }
    for (int x = 0; x < 8; ++x)
      if (cost[x] > 1.05 * tot / 8) return false;
  }
  return true;
}

// Relative throughput of a tile edge (larger tiles reuse operands more).
double tile_eff(int ts) { return ts == 256 ? 1.0 : ts == 128 ? 0.75 : 0.45; }

// Estimated time units of one step's products for tile edge ts: each phase
// runs in ceil(tiles / CUs) waves of its largest tile.
double plan_cost(const std::vector<std::pair<std::pair<int, int>, int>>& shapes, int ts) {
  double gram = 0, poly = 0, apply = 0, gmax = 0, pmax = 0, amax = 0;
  int64_t gt = 0, pt = 0, at = 0;
  for (auto& s : shapes) {
    const int64_t pad = std::max(ts, 128);
    const int64_t mp = round_up(s.first.first, pad), np = round_up(s.first.second, pad);
    const int64_t cnt = s.second, tm = mp / ts, tn = np / ts;
    const double tile_g = double(ts) * ts * np, tile_p = double(ts) * ts * mp;
    gt += cnt * tm * (tm + 1) / 2; pt += cnt * tm * (tm + 1) / 2; at += cnt * tm * tn;
    gram += cnt * tm * (tm + 1) / 2 * tile_g;
    poly += cnt * tm * (tm + 1) / 2 * tile_p;
    apply += cnt * tm * tn * tile_p;
    gmax = std::max(gmax, tile_g); pmax = std::max(pmax, tile_p); amax = std::max(amax, tile_p);
  }
  auto phase = [](double work, double tmax, int64_t tiles) {
    const double waves = std::ceil(double(tiles) / kCUs);
    return std::max(work / kCUs, waves * tmax);
  };
  return (phase(gram, gmax, gt) + phase(poly, pmax, pt) + phase(apply, amax, at)) / tile_eff(ts);
}

// 256-wide tiles exist for bf16 operands only (fp32 operands would need
// twice the fragment and epilogue registers); MUON_TILE forces a size.
int choose_ts(const std::vector<std::pair<std::pair<int, int>, int>>& shapes, int xdt) {
  const int top = xdt == MUON_BF16 ? 256 : 128;
  if (const char* e = std::getenv("MUON_TILE")) {
    const int v = std::atoi(e);
    if (v == 64 || v == 128 || v == 256) return std::min(v, top);
  }
  int best = top;
  double bc = plan_cost(shapes, top);
  for (int ts : {128, 64}) {
    if (ts >= top) continue;
    const double c = plan_cost(shapes, ts);
    if (c < bc * 0.999) { bc = c; best = ts; }
  }
  return best;
}

void build_plan(const int64_t* rows, const int64_t* cols, int n, int xdt, Plan& p) {
  p = Plan();
  p.xdt = xdt;
  std::map<std::pair<int, int>, int> gidx;
  p.mat_group.resize(n);
  p.mat_slot.resize(n);
  for (int i = 0; i < n; ++i) {
    const int m = int(std::min(rows[i], cols[i])), nn = int(std::max(rows[i], cols[i]));
    auto key = std::make_pair(m, nn);
    auto it = gidx.find(key);
    int g;
    if (it == gidx.end()) {
      g = int(p.groups.size());
      gidx[key] = g;
      p.groups.emplace_back();
      p.groups.back().m = m;
      p.groups.back().n = nn;
    } else {
      g = it->second;
    }
    p.mat_group[i] = g;
    p.mat_slot[i] = int(p.groups[g].mats.size());
    p.groups[g].mats.push_back(i);
  }
  std::vector<std::pair<std::pair<int, int>, int>> shapes;
  for (auto& g : p.groups) shapes.push_back({{g.m, g.n}, int(g.mats.size())});
  p.ts = choose_ts(shapes, xdt);
  // 256-wide (bf16) tiles: GRAM runs eight waves, POLY and APPLY sixteen (the
  // launcher picks the layout per phase); smaller tiles four
  p.waves = p.ts == 256 ? 8 : 4;

  const int es = esize(xdt);
  size_t off = 0;
  p.off_desc = off;
  off = align_up(off + sizeof(MatDesc) * size_t(n), kAlign);
  p.off_pprefix = off;
  off = align_up(off + sizeof(int64_t) * size_t(n + 1), kAlign);
  p.off_fprefix = off;
  off = align_up(off + sizeof(int64_t) * size_t(n + 1), kAlign);
  p.off_sync = off;
  off = align_up(off + 4 * sizeof(uint32_t), kAlign);
  // fused update table: the parameter matrices in group order
  p.off_fin = off;
  off = align_up(off + sizeof(FinDesc) * size_t(n), kAlign);
  p.tab_bytes = off;
  p.off_tab[kTabEager] = 0;
  p.off_tab[kTabCapture] = p.tab_bytes;
  off = 2 * p.tab_bytes;
  {
    int base = 0;
    for (auto& g : p.groups) { g.fin_base = base; base += int(g.mats.size()); }
  }
  // every padded dimension is a multiple of the tile edge and of two K steps
  // of the GEMM pipeline (128 elements), so the K loop runs in pairs
  const int pad = std::max(p.ts, 128);
  for (auto& g : p.groups) {
    g.mp = int(round_up(g.m, pad));
    g.np = int(round_up(g.n, pad));
    g.x_elems = int64_t(g.mp) * g.np;
    g.a_elems = int64_t(g.mp) * g.mp;
    g.npart = (g.mp / kEw) * (g.np / kEw);
    if (uint64_t(g.mp) * uint64_t(g.np) * uint64_t(es) >= (uint64_t(1) << 32)) p.fits = false;
    const size_t cnt = g.mats.size();
    g.off_x0 = off; off = align_up(off + cnt * g.x_elems * es, kAlign);
    g.off_x1 = off; off = align_up(off + cnt * g.x_elems * es, kAlign);
    g.off_a = off;  off = align_up(off + cnt * g.a_elems * es, kAlign);
    g.off_b = off;  off = align_up(off + cnt * g.a_elems * es, kAlign);
    g.off_part = off; off = align_up(off + cnt * size_t(g.npart) * 4, kAlign);
  }
  p.total = off;
  // APPLY: when matrices are small (few tiles each) give every XCD a
  // contiguous range of tiles, row-major, so whole matrices stay in one L2;
  // large matrices run in plain block order with four-row-panel groups
  {
    int64_t tiles = 0;
    for (auto& g : p.groups) tiles += int64_t(g.mats.size()) * (g.mp / p.ts) * (g.np / p.ts);
    p.order[2] = (n > 0 && tiles <= int64_t(40) * n) ? 2 : 1;
  }
  p.launch_groups.resize(p.groups.size());
  for (size_t g = 0; g < p.groups.size(); ++g) p.launch_groups[g] = int(g);
  std::stable_sort(p.launch_groups.begin(), p.launch_groups.end(), [&](int a, int b) {
    return p.groups[a].np > p.groups[b].np;
  });
  // GRAM and POLY: whole matrices per XCD when that keeps the XCDs balanced
  // (tiles of one matrix share operand panels in that XCD's L2).  APPLY
  // likewise, walking each matrix one column panel at a time (all row panels
  // of a column in turn), so that the blocks in flight on an XCD share a few
  // X column panels and the matrix's B row panels
  for (int ph = 0; ph < 2; ++ph)
    if (xcd_deal_balanced(p, ph)) p.order[ph] = 4;
  if (xcd_deal_balanced(p, 2)) p.order[2] = 4 | 8;
  // MUON_GEMM_ORDER="g,p,a" overrides the per-phase order bits (experiments)
  if (const char* e = std::getenv("MUON_GEMM_ORDER")) {
    int v[3] = {p.order[0], p.order[1], p.order[2]};
    if (std::sscanf(e, "%d,%d,%d", &v[0], &v[1], &v[2]) == 3)
      for (int k = 0; k < 3; ++k) p.order[k] = v[k] & 15;
  }
  p.pprefix.assign(n + 1, 0);
  p.fprefix.assign(n + 1, 0);
  for (int i = 0; i < n; ++i) {
    const GroupPlan& g = p.groups[p.mat_group[i]];
    p.pprefix[i + 1] = p.pprefix[i] + g.npart;
    // finish and blend: 64 x 64 tiles for tall matrices (transposed through
    // LDS), 32 x 128 row strips otherwise
    p.fprefix[i + 1] = p.fprefix[i] + (rows[i] > cols[i]
        ? ((rows[i] + kEw - 1) / kEw) * ((cols[i] + kEw - 1) / kEw)
        : ((rows[i] + kStripRows - 1) / kStripRows) * ((cols[i] + kStripCols - 1) / kStripCols));
  }
}

// Plans cached by (shape list, iterate type, tile override).
std::mutex g_mu;
std::map<std::tuple<std::vector<int64_t>, int, std::string>, Plan> g_plans;

const Plan& get_plan(const int64_t* rows, const int64_t* cols, int n, int xdt) {
  std::vector<int64_t> key(2 * size_t(n));
  for (int i = 0; i < n; ++i) { key[2 * i] = rows[i]; key[2 * i + 1] = cols[i]; }
  const char* e = std::getenv("MUON_TILE");
  const char* o = std::getenv("MUON_GEMM_ORDER");
  const std::string tile_env = std::string(e ? e : "-") + "/" + (o ? o : "-");
  auto k = std::make_tuple(std::move(key), xdt, tile_env);
  auto it = g_plans.find(k);
  if (it != g_plans.end()) return it->second;
  Plan p;
  build_plan(rows, cols, n, xdt, p);
  if (g_plans.size() > 64) g_plans.clear();
  return g_plans.emplace(std::move(k), std::move(p)).first->second;
}

// Host -> device uploads of the per-call tables (matrix descriptors and tile
// prefix sums).  The workspace is caller memory that
// may be freed and handed out again at the same address, so a table is sent on
// every call instead of being trusted to still be there.  Each copy goes from
// one slot of a ring of pinned staging buffers; a slot is reused only once the
// event recorded behind its previous copy has completed, so the stream is
// never synchronised.  Under graph capture nothing is sent: the table must
// equal what the last uncaptured call (or muon_step_prepare) sent to that
// address, and stays resident for the replays as long as no other call on the
// workspace sends different tables.
struct StageSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool used = false;
};
constexpr int kStageRing = 16;
StageSlot g_stage[kStageRing];
int g_stage_next = 0;
std::map<void*, std::vector<uint8_t>> g_sent;   // last content sent to each address

int upload_table(void* dst, const std::vector<uint8_t>& bytes, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MUON_E_HIP;
  if (cs != hipStreamCaptureStatusNone) {
    auto it = g_sent.find(dst);
    return (it != g_sent.end() && it->second == bytes) ? MUON_OK : MUON_E_CAPTURE;
  }
  StageSlot& sl = g_stage[g_stage_next];
  g_stage_next = (g_stage_next + 1) % kStageRing;
  if (sl.used && hipEventSynchronize(sl.ev) != hipSuccess) return MUON_E_HIP;
  if (!sl.ev && hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming) != hipSuccess)
    return MUON_E_HIP;
  if (sl.cap < bytes.size()) {
    if (sl.host) (void)hipHostFree(sl.host);   // its last copy has completed
    sl.host = nullptr;
    sl.cap = 0;
    const size_t want = std::max<size_t>(bytes.size(), size_t(64) << 10);
    if (hipHostMalloc(&sl.host, want, hipHostMallocDefault) != hipSuccess) return MUON_E_HIP;
    sl.cap = want;
  }
  std::memcpy(sl.host, bytes.data(), bytes.size());
  if (hipMemcpyAsync(dst, sl.host, bytes.size(), hipMemcpyHostToDevice, s) != hipSuccess)
    return MUON_E_HIP;
  if (hipEventRecord(sl.ev, s) != hipSuccess) return MUON_E_HIP;
  sl.used = true;
  if (g_sent.size() > 256) g_sent.clear();
  g_sent[dst] = bytes;
  return MUON_OK;
}

// ---------------------------------------------------------------- probes
struct Probe {
  int phase = -1;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev0, ev1;
} g_probe;

void probe_begin(int phase, hipStream_t s) {
  if (g_probe.phase == phase && g_probe.used < g_probe.cap)
    (void)hipEventRecord(g_probe.ev0[g_probe.used], s);
}
void probe_end(int phase, hipStream_t s) {
  if (g_probe.phase == phase && g_probe.used < g_probe.cap)
    (void)hipEventRecord(g_probe.ev1[g_probe.used++], s);
}

// ---------------------------------------------------------------- validation
bool finite(float v) { return std::isfinite(v); }

int check_mat(const muon_mat& m) {
  if (!m.ptr) return MUON_E_NULL;
  if (m.dtype != MUON_BF16 && m.dtype != MUON_F32) return MUON_E_DTYPE;
  if (m.rows < 1 || m.cols < 1 || m.ld < m.cols) return MUON_E_SHAPE;
  if (m.rows > (int64_t(1) << 30) || m.cols > (int64_t(1) << 30)) return MUON_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(m.ptr) % esize(m.dtype)) return MUON_E_ALIGN;
  return MUON_OK;
}

size_t mat_bytes(const muon_mat& m) {
  return size_t((m.rows - 1) * m.ld + m.cols) * esize(m.dtype);
}

bool vec_ok(const void* p, int64_t ld, int es) {
  return reinterpret_cast<uintptr_t>(p) % 16 == 0 && (ld * es) % 16 == 0;
}

struct Range { uintptr_t lo, hi; };

bool overlaps(std::vector<Range>& r) {
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi) return true;
  return false;
}

void add_range(std::vector<Range>& r, const void* p, size_t bytes) {
  if (p && bytes) r.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes});
}

int check_opt(const muon_options& o) {
  if (!finite(o.eps) || o.eps < 0.f) return MUON_E_HPARAM;
  if (o.beta_slow >= 0.f && !(o.beta_slow < 1.f)) return MUON_E_HPARAM;
  if (o.beta_ema >= 0.f && !(o.beta_ema < 1.f)) return MUON_E_HPARAM;
  if (!finite(o.beta_slow) || !finite(o.beta_ema)) return MUON_E_HPARAM;
  if (o.ns_dtype != MUON_BF16 && o.ns_dtype != MUON_F32) return MUON_E_DTYPE;
  if (o.cautious && o.beta_slow < 0.f) return MUON_E_HPARAM;
  if (o.nesterov != 0 && o.nesterov != 1) return MUON_E_HPARAM;
  if (o.cautious != 0 && o.cautious != 1) return MUON_E_HPARAM;
  if (o.avg_mode != MUON_AVG_EMA && o.avg_mode != MUON_AVG_WEIGHTED) return MUON_E_HPARAM;
  return MUON_OK;
}

int check_coeffs(const float* c, int steps) {
  if (steps < 0 || steps > MUON_MAX_STEPS) return MUON_E_COEFFS;
  if (steps > 0 && !c) return MUON_E_NULL;
  for (int i = 0; i < 3 * steps; ++i)
    if (!finite(c[i])) return MUON_E_COEFFS;
  return MUON_OK;
}

// ---------------------------------------------------------------- launches
void fill_desc(MatDesc& d, const Plan& p, int i, const muon_mat& src_shape, char* ws) {
  const GroupPlan& g = p.groups[p.mat_group[i]];
  const int slot = p.mat_slot[i];
  const int es = esize(p.xdt);
  d.rows = int(src_shape.rows);
  d.cols = int(src_shape.cols);
  d.mp = g.mp;
  d.np = g.np;
  d.tall = src_shape.rows > src_shape.cols;
  d.x0 = ws + g.off_x0 + size_t(slot) * g.x_elems * es;
  d.x1 = ws + g.off_x1 + size_t(slot) * g.x_elems * es;
  d.partials = reinterpret_cast<float*>(ws + g.off_part) + size_t(slot) * g.npart;
  d.npartials = g.npart;
  d.dvec = (src_shape.cols % 4) == 0;
}

void table_bytes(const Plan& p, const std::vector<MatDesc>& desc, std::vector<uint8_t>& out) {
  const int n = int(desc.size());
  out.assign(p.off_fin + sizeof(FinDesc) * size_t(n), 0);
  std::memcpy(out.data() + p.off_desc, desc.data(), sizeof(MatDesc) * size_t(n));
  std::memcpy(out.data() + p.off_pprefix, p.pprefix.data(), sizeof(int64_t) * size_t(n + 1));
  std::memcpy(out.data() + p.off_fprefix, p.fprefix.data(), sizeof(int64_t) * size_t(n + 1));
  // the fused-update table depends on the matrices only (not on the options
  // of a call), so the table a capture compares against stays the same
  for (int i = 0; i < n; ++i) {
    FinDesc f;
    std::memset(&f, 0, sizeof(f));
    f.w = desc[i].w;
    f.ldw = desc[i].ldw;
    f.rows = desc[i].rows;
    f.cols = desc[i].cols;
    f.tall = desc[i].tall;
    const GroupPlan& g = p.groups[p.mat_group[i]];
    std::memcpy(out.data() + p.off_fin + sizeof(FinDesc) * size_t(g.fin_base + p.mat_slot[i]), &f,
                sizeof(f));
  }
}

// Whether a step's plain update (no cautious mask, no average, no diagnostic
// outputs) runs in the epilogue of its last APPLY instead of the finish
// kernel: every parameter matrix bf16 with shapes, row pitch and base fit for
// 16-byte chunks of 8 elements, 256-wide bf16 tiles, and a last iteration
// that keeps the staged epilogue (b or c nonzero).  coeffs NULL: quintic.
// The staged epilogue of 256-wide bf16 tiles folds the input term into the
// product during the K loop: POLY keeps acc = A A + (b/c) A and stores c acc,
// a cubic APPLY keeps acc = A X + (a/b) X and stores s b acc.  A ratio or a
// multiplier far from one could overflow the fp32 accumulators where the
// unfolded sum is finite, so a coefficient table with such a row runs the
// plain epilogue (input term added at the store, A and B row-major) in every
// launch of the call.  The ratio is formed in fp32, as the kernels form it.
bool fold_ok(float num, float den) {
  const float r = num / den;
  return std::isfinite(r) && std::fabs(r) <= 0x1p32f && std::fabs(den) >= 0x1p-32f;
}

// Most tiles of any one product (GRAM, POLY, APPLY) of a plan.
int64_t max_phase_tiles(const Plan& p) {
  int64_t most = 0;
  for (int ph = 0; ph < 3; ++ph) {
    int64_t t = 0;
    for (auto& g : p.groups) {
      const int64_t tm = g.mp / p.ts, tn = g.np / p.ts;
      t += int64_t(g.mats.size()) * (ph == 2 ? tm * tn : tm * (tm + 1) / 2);
    }
    most = std::max(most, t);
  }
  return most;
}

// Small problems (64-wide bf16 tiles, at most four tiles per block and
// product) can run all iterations in one launch, on request
// (MUON_NS_SINGLE_LAUNCH=1): on MI355X its grid-wide barriers cost more than
// the kernel boundaries they replace (one 256 x 512 matrix: 0.150 ms per step
// against 0.082 ms with one launch per product), so it is not the default.
bool single_launch_ok(const Plan& p, int steps, bool fin) {
  if (fin || steps <= 0 || steps > kSmallMaxSteps || p.ts != 64 || p.xdt != MUON_BF16 ||
      p.groups.size() > size_t(kMaxGroups))
    return false;
  const char* e = std::getenv("MUON_NS_SINGLE_LAUNCH");
  if (!e || std::strcmp(e, "1") != 0) return false;
  return max_phase_tiles(p) <= 4 * int64_t(kCUs);
}

// Polls of the single launch's barrier before a block gives up; the
// MUON_NS_SPIN_LIMIT override exists to force the failure path (0: fail at
// once).
uint32_t spin_limit() {
  if (const char* e = std::getenv("MUON_NS_SPIN_LIMIT")) return uint32_t(std::strtoul(e, nullptr, 10));
  return 1u << 20;
}

bool folding_safe(const float* coeffs, int steps) {
  if (!coeffs) return true;   // quintic
  for (int j = 0; j < steps; ++j) {
    const float a = coeffs[3 * j], b = coeffs[3 * j + 1], c = coeffs[3 * j + 2];
    if (c != 0.f ? !fold_ok(b, c) : (b != 0.f && !fold_ok(a, b))) return false;
  }
  return true;
}

bool update_fusable(const Plan& p, const muon_mat* params, int n, bool cautious, bool avg,
                    bool diag, const float* coeffs, int steps) {
  if (n <= 0 || steps <= 0 || p.xdt != MUON_BF16 || p.ts != 256 || p.waves != 8 || cautious ||
      avg || diag || !folding_safe(coeffs, steps))
    return false;
  if (coeffs && coeffs[3 * (steps - 1) + 1] == 0.f && coeffs[3 * (steps - 1) + 2] == 0.f)
    return false;
  for (int i = 0; i < n; ++i)
    if (params[i].dtype != MUON_BF16 || params[i].rows % 8 || params[i].cols % 8 ||
        params[i].ld % 8 || reinterpret_cast<uintptr_t>(params[i].ptr) % 16)
      return false;
  return true;
}

// Newton-Schulz iterations; returns the buffer index holding the result.
// tab: the descriptor-table region the launches read.
hipError_t run_ns(const Plan& p, char* ws, const char* tab, const float* coeffs, int steps,
                  float eps, hipStream_t s, int* final_buf, bool fin = false, float lr = 0.f,
                  float lrwd = 0.f) {
  if (single_launch_ok(p, steps, fin)) {
    SmallArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.ngroups = int(p.groups.size());
    sa.steps = steps;
    sa.eps = eps;
    sa.spin_limit = spin_limit();
    for (int j = 0; j < steps; ++j)
      for (int c = 0; c < 3; ++c) sa.coef[j][c] = coeffs[3 * j + c];
    sa.sync = reinterpret_cast<uint32_t*>(const_cast<char*>(tab) + p.off_sync);
    for (size_t gi = 0; gi < p.groups.size(); ++gi) {
      const GroupPlan& g = p.groups[gi];
      SmallGroup& d = sa.g[gi];
      d.x0 = ws + g.off_x0; d.x1 = ws + g.off_x1; d.a = ws + g.off_a; d.b = ws + g.off_b;
      d.partials = reinterpret_cast<const float*>(ws + g.off_part);
      d.x_elems = g.x_elems; d.a_elems = g.a_elems;
      d.count = int(g.mats.size()); d.mp = g.mp; d.np = g.np; d.npart = g.npart;
      d.kg = int(round_up(g.n, 128));
      d.kp = int(round_up(g.m, 128));
    }
    // at most one block per CU: every block must be resident for the barriers
    probe_begin(MUON_PHASE_NS_SINGLE, s);
    const hipError_t err = launch_ns_small(sa, int(std::min<int64_t>(max_phase_tiles(p), kCUs)), s);
    probe_end(MUON_PHASE_NS_SINGLE, s);
    if (err != hipSuccess) return err;
    *final_buf = steps & 1;
    return hipSuccess;
  }
  int cur = 0;
  const bool fold = folding_safe(coeffs, steps);
  for (int j = 0; j < steps; ++j) {
    const float a = coeffs[3 * j], b = coeffs[3 * j + 1], c = coeffs[3 * j + 2];
    const bool poly = c != 0.f;
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.first = j == 0;
    ga.ca = a; ga.cb = b; ga.cc = c;
    ga.cbb = poly ? 1.f : b;
    ga.eps = eps;
    const int es = esize(p.xdt);
    // groups are processed in launch sets of at most kMaxGroups
    for (size_t g0 = 0; g0 < p.groups.size(); g0 += kMaxGroups) {
      const size_t g1 = std::min(p.groups.size(), g0 + kMaxGroups);
      for (int phase = 0; phase < 3; ++phase) {
        if (phase == 1 && !poly) continue;
        int64_t blocks = 0;
        ga.ngroups = int(g1 - g0);
        ga.order = p.order[phase];
        // last APPLY of a fused step: update the parameters instead of storing X
        ga.fin = fin && phase == 2 && j == steps - 1;
        ga.ablk = fold && p.ts == 256 && p.xdt == MUON_BF16 && p.waves == 8;
        ga.nofold = !fold;
        ga.lr = lr;
        ga.lrwd = lrwd;
        for (size_t gi = g0; gi < g1; ++gi) {
          const GroupPlan& g = p.groups[p.launch_groups[gi]];
          GemmGroup& d = ga.g[gi - g0];
          const int tm = g.mp / p.ts, tn = g.np / p.ts;
          char* xin = ws + (cur ? g.off_x1 : g.off_x0);
          char* xout = ws + (cur ? g.off_x0 : g.off_x1);
          d.count = int(g.mats.size());
          // K loops stop at the real contraction length (rounded to the
          // two-stage pipeline's 128): a 1408-row group padded to 1536 for
          // 256-wide tiles runs 22 stages of 64, not 24
          d.kdim = int(round_up(phase == 0 ? g.n : g.m, 128));
          d.mp = g.mp; d.np = g.np;
          d.partials = reinterpret_cast<const float*>(ws + g.off_part);
          d.p_stride = g.npart;
          d.npartials = g.npart;
          d.block_base = int(blocks);
          d.fin = reinterpret_cast<const FinDesc*>(tab + p.off_fin) + g.fin_base;
          if (phase == 0) {
            d.xin = xin; d.out = ws + g.off_a;
            d.in_stride = g.x_elems; d.out_stride = g.a_elems;
            d.tiles = tm * (tm + 1) / 2;
          } else if (phase == 1) {
            d.xin = ws + g.off_a; d.out = ws + g.off_b;
            d.in_stride = g.a_elems; d.out_stride = g.a_elems;
            d.tiles = tm * (tm + 1) / 2;
          } else {
            d.xin = xin; d.bop = ws + (poly ? g.off_b : g.off_a); d.out = xout;
            d.in_stride = g.x_elems; d.b_stride = g.a_elems; d.out_stride = g.x_elems;
            d.tiles = tm * tn;
          }
          blocks += int64_t(d.count) * d.tiles;
        }
        (void)es;
        const int ph = phase == 0 ? MUON_PHASE_GRAM : phase == 1 ? MUON_PHASE_POLY
                     : ga.fin ? MUON_PHASE_APPLY_UPDATE : MUON_PHASE_APPLY;
        probe_begin(ph, s);
        if (ga.order & 4) {
          // every XCD gets as many blocks as the one with the most matrices;
          // the surplus blocks of the others exit at once
          int64_t per = 0;
          for (int k = 0; k < ga.ngroups; ++k)
            per += int64_t((ga.g[k].count + 7) / 8) * ga.g[k].tiles;
          blocks = 8 * per;
        }
        hipError_t err = launch_gemm(phase, p.xdt, p.ts, p.waves, ga, blocks, s);
        probe_end(ph, s);
        if (err != hipSuccess) return err;
      }
    }
    cur ^= 1;
  }
  *final_buf = cur;
  return hipSuccess;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

void muon_default_options(muon_options* o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->beta_slow = -1.f;
  o->beta_ema = -1.f;
  o->eps = 1e-7f;
  o->ema_start = 1;
  o->nesterov = 0;
  o->cautious = 0;
  o->ns_dtype = MUON_BF16;
  o->avg_mode = MUON_AVG_EMA;
}

const char* muon_status_str(int s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_E_NULL: return "null pointer";
    case MUON_E_SHAPE: return "invalid shape";
    case MUON_E_DTYPE: return "invalid element type";
    case MUON_E_COEFFS: return "invalid coefficients or step count";
    case MUON_E_HPARAM: return "invalid hyperparameter or option";
    case MUON_E_WORKSPACE: return "workspace missing or too small";
    case MUON_E_ALIAS: return "overlapping buffers";
    case MUON_E_ALIGN: return "misaligned pointer";
    case MUON_E_HIP: return "HIP runtime error";
    case MUON_E_STATE: return "state inconsistent with the call";
    case MUON_E_CAPTURE: return "descriptor table not resident for a call under stream capture";
    default: return "unknown status";
  }
}

size_t muon_workspace_bytes(const muon_mat* params, int32_t n, const muon_options* opt,
                            int32_t steps) {
  (void)steps;
  if (n < 0 || (n > 0 && !params)) return 0;
  const int xdt = opt ? opt->ns_dtype : MUON_BF16;
  if (xdt != MUON_BF16 && xdt != MUON_F32) return 0;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if (params[i].rows < 1 || params[i].cols < 1) return 0;
    if (params[i].rows > (int64_t(1) << 30) || params[i].cols > (int64_t(1) << 30)) return 0;
    rows[i] = params[i].rows;
    cols[i] = params[i].cols;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, xdt);
  return p.fits ? p.total : 0;
}

namespace {
// A workspace that is not the state's: the library's static scratch of the
// allocation-free entry point.  Its descriptor table is written by kernels
// (launch_put_table) instead of a copy from pinned staging memory.
struct FixedWorkspace {
  void* ptr;
  size_t bytes;
};

// muon_step, or with prepare_only its validation and descriptor-table upload
// alone (no launch, counters unchanged).  fixed: use that workspace instead
// of st->workspace (never with prepare_only).
int step_impl(const muon_mat* params, const muon_mat* grads, muon_state* st, const float* coeffs,
              int32_t steps, float lr, float wd, float beta, void* stream, bool prepare_only,
              const FixedWorkspace* fixed = nullptr) {
  if (!st) return MUON_E_NULL;
  const int n = st->n;
  if (n < 0) return MUON_E_SHAPE;
  int rc;
  if ((rc = check_coeffs(coeffs, steps)) != MUON_OK) return rc;
  if (!finite(lr) || !finite(wd) || !(beta >= 0.f && beta < 1.f)) return MUON_E_HPARAM;
  const muon_options& o = st->opt;
  if ((rc = check_opt(o)) != MUON_OK) return rc;
  const bool ema_on = o.beta_ema >= 0.f && st->step + 1 >= o.ema_start;
  // weighted running mean: b = S/(S+w), ob = w/(S+w) in double, then fp32
  const bool weighted = ema_on && o.avg_mode == MUON_AVG_WEIGHTED;
  double avg_sum = st->avg_weight_sum;
  float avg_b = 0.f, avg_ob = 0.f;
  if (weighted) {
    const double w = st->avg_weight;
    const double s0 = st->ema_count == 0 ? 0.0 : st->avg_weight_sum;
    if (!std::isfinite(w) || w < 0.0 || !std::isfinite(s0) || s0 < 0.0 || !(s0 + w > 0.0))
      return MUON_E_HPARAM;
    avg_sum = s0 + w;
    avg_b = static_cast<float>(s0 / avg_sum);
    avg_ob = static_cast<float>(w / avg_sum);
  }
  if (n == 0) {
    if (prepare_only) return MUON_OK;
    st->step += 1;
    if (ema_on) st->ema_count += 1;
    if (weighted) st->avg_weight_sum = avg_sum;
    return MUON_OK;
  }
  if (!params || !grads || !st->mom) return MUON_E_NULL;
  if (o.beta_slow >= 0.f && !st->mom_slow) return MUON_E_STATE;
  if (o.beta_ema >= 0.f && !st->ema) return MUON_E_STATE;
  std::vector<Range> ranges;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if ((rc = check_mat(params[i])) != MUON_OK) return rc;
    if ((rc = check_mat(grads[i])) != MUON_OK) return rc;
    if (grads[i].rows != params[i].rows || grads[i].cols != params[i].cols) return MUON_E_SHAPE;
    if (!st->mom[i]) return MUON_E_STATE;
    if (o.beta_slow >= 0.f && !st->mom_slow[i]) return MUON_E_STATE;
    if (o.beta_ema >= 0.f && !st->ema[i]) return MUON_E_STATE;
    const size_t dense = size_t(params[i].rows * params[i].cols);
    const void* dps[3] = {st->mom[i], o.beta_slow >= 0.f ? st->mom_slow[i] : nullptr,
                          o.beta_ema >= 0.f ? st->ema[i] : nullptr};
    for (const void* q : dps)
      if (q && reinterpret_cast<uintptr_t>(q) % 4) return MUON_E_ALIGN;
    if (st->update_out && st->update_out[i] && reinterpret_cast<uintptr_t>(st->update_out[i]) % 4)
      return MUON_E_ALIGN;
    add_range(ranges, params[i].ptr, mat_bytes(params[i]));
    add_range(ranges, grads[i].ptr, mat_bytes(grads[i]));
    for (const void* q : dps) add_range(ranges, q, dense * 4);
    if (st->mask_out) add_range(ranges, st->mask_out[i], dense);
    if (st->update_out) add_range(ranges, st->update_out[i], dense * 4);
    rows[i] = params[i].rows;
    cols[i] = params[i].cols;
  }
  void* const wsp = fixed ? fixed->ptr : st->workspace;
  const size_t ws_bytes = fixed ? fixed->bytes : st->workspace_bytes;
  if (!wsp) return MUON_E_WORKSPACE;
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, o.ns_dtype);
  if (!p.fits) return MUON_E_SHAPE;
  if (ws_bytes < p.total) return MUON_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(wsp) % kAlign) return MUON_E_ALIGN;
  add_range(ranges, wsp, p.total);
  if (overlaps(ranges)) return MUON_E_ALIAS;

  // ---- descriptor table
  char* ws = static_cast<char*>(wsp);
  std::vector<MatDesc> desc(n);
  for (int i = 0; i < n; ++i) {
    MatDesc& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    fill_desc(d, p, i, params[i], ws);
    d.w = params[i].ptr; d.ldw = params[i].ld; d.wdt = params[i].dtype;
    d.g = grads[i].ptr; d.ldg = grads[i].ld; d.gdt = grads[i].dtype;
    d.wvec = vec_ok(d.w, d.ldw, esize(d.wdt));
    d.gvec = vec_ok(d.g, d.ldg, esize(d.gdt));
    d.mom = st->mom[i];
    d.slow = o.beta_slow >= 0.f ? st->mom_slow[i] : nullptr;
    d.ema = o.beta_ema >= 0.f ? st->ema[i] : nullptr;
    d.mask_out = st->mask_out ? st->mask_out[i] : nullptr;
    d.upd_out = st->update_out ? st->update_out[i] : nullptr;
    const bool dv = (params[i].cols % 4) == 0 && reinterpret_cast<uintptr_t>(d.mom) % 16 == 0 &&
                    (!d.slow || reinterpret_cast<uintptr_t>(d.slow) % 16 == 0) &&
                    (!d.ema || reinterpret_cast<uintptr_t>(d.ema) % 16 == 0) &&
                    (!d.upd_out || reinterpret_cast<uintptr_t>(d.upd_out) % 16 == 0);
    d.dvec = dv;
  }
  std::vector<uint8_t> bytes;
  table_bytes(p, desc, bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MUON_E_HIP;
  const bool capturing = cs != hipStreamCaptureStatusNone;
  // the weighted average's coefficients change with every step: a replayed
  // capture would repeat stale ones
  if (weighted && capturing && !prepare_only) return MUON_E_CAPTURE;
  const char* tab;
  if (fixed) {
    // the static scratch: the table is written by kernels on the stream (part
    // of a capture when the stream is capturing)
    tab = ws + p.off_tab[kTabEager];
    if (launch_put_table(const_cast<char*>(tab), bytes.data(), bytes.size(), s) != hipSuccess)
      return MUON_E_HIP;
  } else {
    // muon_step_prepare fills the capture region, which captured steps read;
    // uncaptured steps send and read the eager region
    tab = ws + p.off_tab[(prepare_only || capturing) ? kTabCapture : kTabEager];
    if ((rc = upload_table(const_cast<char*>(tab), bytes, s)) != MUON_OK) return rc;
    if (prepare_only) return MUON_OK;
  }

  ElemArgs ea;
  std::memset(&ea, 0, sizeof(ea));
  ea.mats = reinterpret_cast<const MatDesc*>(tab + p.off_desc);
  ea.prefix = reinterpret_cast<const int64_t*>(tab + p.off_pprefix);
  ea.nmats = n;
  ea.xdt = p.xdt;
  ea.beta = beta;
  ea.obeta = 1.0f - beta;
  if (o.beta_slow >= 0.f) { ea.bslow = o.beta_slow; ea.obslow = 1.0f - o.beta_slow; }
  if (weighted) {
    ea.bema = avg_b;
    ea.obema = avg_ob;
  } else if (o.beta_ema >= 0.f) {
    ea.bema = o.beta_ema;
    ea.obema = 1.0f - o.beta_ema;
  }
  ea.lr = lr;
  {
    volatile float lrwd = lr * wd;   // one fp32 rounding
    ea.lrwd = lrwd;
  }
  ea.eps = o.eps;
  ea.mode = 0;
  ea.nesterov = o.nesterov;
  ea.cautious = o.cautious;
  ea.use_slow = o.beta_slow >= 0.f;
  ea.ema_on = ema_on;
  ea.ema_first = ema_on && st->ema_count == 0;
  ea.scale_o = steps == 0;

  const bool fused = update_fusable(p, params, n, o.cautious, ema_on,
                                    st->mask_out || st->update_out, coeffs, steps);

  probe_begin(MUON_PHASE_PREPARE, s);
  hipError_t err = launch_prepare(ea, p.pprefix[n], s);
  probe_end(MUON_PHASE_PREPARE, s);
  if (err != hipSuccess) return MUON_E_HIP;
  int fb = 0;
  if (run_ns(p, ws, tab, coeffs, steps, o.eps, s, &fb, fused, ea.lr, ea.lrwd) != hipSuccess)
    return MUON_E_HIP;
  if (!fused) {
    ea.final_buf = fb;
    ea.ns_err = reinterpret_cast<const uint32_t*>(tab + p.off_sync) + 2;
    ea.prefix = reinterpret_cast<const int64_t*>(tab + p.off_fprefix);
    probe_begin(MUON_PHASE_FINISH, s);
    err = launch_finish(ea, p.fprefix[n], s);
    probe_end(MUON_PHASE_FINISH, s);
    if (err != hipSuccess) return MUON_E_HIP;
  }
  st->step += 1;
  if (ema_on) st->ema_count += 1;
  if (weighted) st->avg_weight_sum = avg_sum;
  return MUON_OK;
}
}  // namespace

int muon_step(const muon_mat* params, const muon_mat* grads, muon_state* st, const float* coeffs,
              int32_t steps, float lr, float wd, float beta, void* stream) {
  return step_impl(params, grads, st, coeffs, steps, lr, wd, beta, stream, false);
}

int muon_step_prepare(const muon_mat* params, const muon_mat* grads, muon_state* st,
                      void* stream) {
  return step_impl(params, grads, st, nullptr, 0, 0.f, 0.f, 0.f, stream, true);
}

}  // extern "C"

namespace muon {
int step_fixed_workspace(const muon_mat* params, const muon_mat* grads, muon_state* st,
                         const float* coeffs, int32_t steps, float lr, float wd, float beta,
                         void* stream, void* ws, size_t ws_bytes) {
  const FixedWorkspace f{ws, ws_bytes};
  return step_impl(params, grads, st, coeffs, steps, lr, wd, beta, stream, false, &f);
}
}  // namespace muon

extern "C" {

int muon_state_advance(muon_state* st, int32_t replays) {
  if (!st) return MUON_E_NULL;
  if (replays < 0) return MUON_E_HPARAM;
  int rc;
  if ((rc = check_opt(st->opt)) != MUON_OK) return rc;
  const muon_options& o = st->opt;
  // a replayed step repeats the captured weight-average flags: averaging must
  // be off or an exponential average already started (the capture rules)
  if (o.beta_ema >= 0.f) {
    if (o.avg_mode != MUON_AVG_EMA) return MUON_E_CAPTURE;
    if (st->ema_count == 0 || st->step + 1 < o.ema_start) return MUON_E_CAPTURE;
  }
  for (int32_t r = 0; r < replays; ++r) {
    st->step += 1;
    if (o.beta_ema >= 0.f && st->step >= o.ema_start) st->ema_count += 1;
  }
  return MUON_OK;
}

int muon_workspace_layout(const muon_mat* params, int32_t n, const muon_options* opt,
                          size_t* eager_table, size_t* capture_table, size_t* table_bytes,
                          size_t* buffers) {
  if (n < 0) return MUON_E_SHAPE;
  if ((n > 0 && !params) || !eager_table || !capture_table || !table_bytes || !buffers)
    return MUON_E_NULL;
  const int xdt = opt ? opt->ns_dtype : MUON_BF16;
  if (xdt != MUON_BF16 && xdt != MUON_F32) return MUON_E_DTYPE;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if (params[i].rows < 1 || params[i].cols < 1) return MUON_E_SHAPE;
    if (params[i].rows > (int64_t(1) << 30) || params[i].cols > (int64_t(1) << 30))
      return MUON_E_SHAPE;
    rows[i] = params[i].rows;
    cols[i] = params[i].cols;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, xdt);
  if (!p.fits) return MUON_E_SHAPE;
  *eager_table = p.off_tab[kTabEager];
  *capture_table = p.off_tab[kTabCapture];
  *table_bytes = p.tab_bytes;
  *buffers = p.groups.empty() ? p.total : p.groups[0].off_x0;
  return MUON_OK;
}

int muon_orthogonalize(const muon_mat* in, const muon_mat* out, int32_t n, const float* coeffs,
                       int32_t steps, const muon_options* opt, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (n < 0) return MUON_E_SHAPE;
  int rc;
  if ((rc = check_coeffs(coeffs, steps)) != MUON_OK) return rc;
  muon_options o;
  muon_default_options(&o);
  if (opt) {
    o.eps = opt->eps;
    o.ns_dtype = opt->ns_dtype;
  }
  if ((rc = check_opt(o)) != MUON_OK) return rc;
  if (n == 0) return MUON_OK;
  if (!in || !out) return MUON_E_NULL;
  std::vector<Range> ranges;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if ((rc = check_mat(in[i])) != MUON_OK) return rc;
    if ((rc = check_mat(out[i])) != MUON_OK) return rc;
    if (in[i].rows != out[i].rows || in[i].cols != out[i].cols) return MUON_E_SHAPE;
    add_range(ranges, in[i].ptr, mat_bytes(in[i]));
    add_range(ranges, out[i].ptr, mat_bytes(out[i]));
    rows[i] = in[i].rows;
    cols[i] = in[i].cols;
  }
  if (!workspace) return MUON_E_WORKSPACE;
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, o.ns_dtype);
  if (!p.fits) return MUON_E_SHAPE;
  if (workspace_bytes < p.total) return MUON_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return MUON_E_ALIGN;
  add_range(ranges, workspace, p.total);
  if (overlaps(ranges)) return MUON_E_ALIAS;

  char* ws = static_cast<char*>(workspace);
  std::vector<MatDesc> desc(n);
  for (int i = 0; i < n; ++i) {
    MatDesc& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    fill_desc(d, p, i, in[i], ws);
    d.g = in[i].ptr; d.ldg = in[i].ld; d.gdt = in[i].dtype;
    d.w = out[i].ptr; d.ldw = out[i].ld; d.wdt = out[i].dtype;
    d.gvec = vec_ok(d.g, d.ldg, esize(d.gdt));
    d.wvec = vec_ok(d.w, d.ldw, esize(d.wdt));
    d.dvec = 0;
  }
  std::vector<uint8_t> bytes;
  table_bytes(p, desc, bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* tab = ws + p.off_tab[kTabEager];
  if ((rc = upload_table(tab, bytes, s)) != MUON_OK) return rc;
  ElemArgs ea;
  std::memset(&ea, 0, sizeof(ea));
  ea.mats = reinterpret_cast<const MatDesc*>(tab + p.off_desc);
  ea.prefix = reinterpret_cast<const int64_t*>(tab + p.off_pprefix);
  ea.nmats = n;
  ea.xdt = p.xdt;
  ea.eps = o.eps;
  ea.mode = 1;
  ea.scale_o = steps == 0;
  probe_begin(MUON_PHASE_PREPARE, s);
  hipError_t err = launch_prepare(ea, p.pprefix[n], s);
  probe_end(MUON_PHASE_PREPARE, s);
  if (err != hipSuccess) return MUON_E_HIP;
  int fb = 0;
  if (run_ns(p, ws, tab, coeffs, steps, o.eps, s, &fb) != hipSuccess) return MUON_E_HIP;
  ea.final_buf = fb;
  ea.ns_err = reinterpret_cast<const uint32_t*>(tab + p.off_sync) + 2;
  ea.prefix = reinterpret_cast<const int64_t*>(tab + p.off_fprefix);
  probe_begin(MUON_PHASE_FINISH, s);
  err = launch_finish(ea, p.fprefix[n], s);
  probe_end(MUON_PHASE_FINISH, s);
  return err == hipSuccess ? MUON_OK : MUON_E_HIP;
}

int muon_ema_blend(const muon_mat* out, const muon_mat* params, const muon_state* st,
                   float w_final, void* stream) {
  if (!st) return MUON_E_NULL;
  const int n = st->n;
  if (n < 0) return MUON_E_SHAPE;
  if (!(w_final >= 0.f && w_final <= 1.f)) return MUON_E_HPARAM;
  if (n == 0) return MUON_OK;
  if (!out || !params) return MUON_E_NULL;
  if (!st->ema) return MUON_E_STATE;
  int rc;
  std::vector<Range> ranges;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if ((rc = check_mat(out[i])) != MUON_OK) return rc;
    if ((rc = check_mat(params[i])) != MUON_OK) return rc;
    if (out[i].rows != params[i].rows || out[i].cols != params[i].cols) return MUON_E_SHAPE;
    if (!st->ema[i]) return MUON_E_STATE;
    if (reinterpret_cast<uintptr_t>(st->ema[i]) % 4) return MUON_E_ALIGN;
    const bool same = out[i].ptr == params[i].ptr && out[i].ld == params[i].ld &&
                      out[i].dtype == params[i].dtype;
    add_range(ranges, out[i].ptr, mat_bytes(out[i]));
    if (!same) add_range(ranges, params[i].ptr, mat_bytes(params[i]));
    add_range(ranges, st->ema[i], size_t(out[i].rows * out[i].cols) * 4);
    rows[i] = out[i].rows;
    cols[i] = out[i].cols;
  }
  if (!st->workspace) return MUON_E_WORKSPACE;
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, st->opt.ns_dtype == MUON_F32 ? MUON_F32 : MUON_BF16);
  if (!p.fits) return MUON_E_SHAPE;
  if (st->workspace_bytes < p.total) return MUON_E_WORKSPACE;
  add_range(ranges, st->workspace, p.total);
  if (overlaps(ranges)) return MUON_E_ALIAS;
  char* ws = static_cast<char*>(st->workspace);
  std::vector<MatDesc> desc(n);
  for (int i = 0; i < n; ++i) {
    MatDesc& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    fill_desc(d, p, i, out[i], ws);
    d.w = out[i].ptr; d.ldw = out[i].ld; d.wdt = out[i].dtype;
    d.g = params[i].ptr; d.ldg = params[i].ld; d.gdt = params[i].dtype;
    d.wvec = vec_ok(d.w, d.ldw, esize(d.wdt));
    d.gvec = vec_ok(d.g, d.ldg, esize(d.gdt));
    d.ema = st->ema[i];
    d.dvec = (out[i].cols % 4) == 0 && reinterpret_cast<uintptr_t>(d.ema) % 16 == 0;
  }
  std::vector<uint8_t> bytes;
  table_bytes(p, desc, bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the eager region: a captured step reads the capture region, which only
  // muon_step_prepare writes
  char* tab = ws + p.off_tab[kTabEager];
  if ((rc = upload_table(tab, bytes, s)) != MUON_OK) return rc;
  ElemArgs ea;
  std::memset(&ea, 0, sizeof(ea));
  ea.mats = reinterpret_cast<const MatDesc*>(tab + p.off_desc);
  ea.prefix = reinterpret_cast<const int64_t*>(tab + p.off_fprefix);
  ea.nmats = n;
  const float wf = w_final;
  volatile float owf = 1.0f - wf;
  return launch_blend(ea, p.fprefix[n], wf, owf, s) == hipSuccess ? MUON_OK : MUON_E_HIP;
}

int muon_probe_arm(int32_t phase, int32_t capacity) {
  if (phase < 0 || phase > MUON_PHASE_NS_SINGLE || capacity < 1 || capacity > 65536)
    return MUON_E_HPARAM;
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto e : g_probe.ev0) (void)hipEventDestroy(e);
  for (auto e : g_probe.ev1) (void)hipEventDestroy(e);
  g_probe = Probe();
  g_probe.ev0.resize(capacity);
  g_probe.ev1.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&g_probe.ev0[i]) != hipSuccess || hipEventCreate(&g_probe.ev1[i]) != hipSuccess)
      return MUON_E_HIP;
  }
  g_probe.cap = capacity;
  g_probe.phase = phase;
  return MUON_OK;
}

int muon_probe_read(float* ms, int32_t capacity, int32_t* count) {
  if (!ms || !count) return MUON_E_NULL;
  std::lock_guard<std::mutex> lk(g_mu);
  const int k = std::min(capacity, g_probe.used);
  for (int i = 0; i < k; ++i) {
    if (hipEventSynchronize(g_probe.ev1[i]) != hipSuccess) return MUON_E_HIP;
    if (hipEventElapsedTime(&ms[i], g_probe.ev0[i], g_probe.ev1[i]) != hipSuccess) return MUON_E_HIP;
  }
  *count = k;
  return MUON_OK;
}

int muon_probe_disarm(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto e : g_probe.ev0) (void)hipEventDestroy(e);
  for (auto e : g_probe.ev1) (void)hipEventDestroy(e);
  g_probe = Probe();
  return MUON_OK;
}

int muon_plan_info(const muon_mat* params, int32_t n, const muon_options* opt, int32_t steps,
                   const float* coeffs, int32_t* n_groups, int32_t* tiles, int32_t cap,
                   int32_t* launches_per_step) {
  if (n < 0 || steps < 0 || steps > MUON_MAX_STEPS) return MUON_E_SHAPE;
  if (n > 0 && !params) return MUON_E_NULL;
  const int xdt = opt ? opt->ns_dtype : MUON_BF16;
  if (xdt != MUON_BF16 && xdt != MUON_F32) return MUON_E_DTYPE;
  std::vector<int64_t> rows(n), cols(n);
  for (int i = 0; i < n; ++i) {
    if (params[i].rows < 1 || params[i].cols < 1) return MUON_E_SHAPE;
    rows[i] = params[i].rows;
    cols[i] = params[i].cols;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  const Plan& p = get_plan(rows.data(), cols.data(), n, xdt);
  if (!p.fits) return MUON_E_SHAPE;
  if (n_groups) *n_groups = int(p.groups.size());
  if (tiles)
    for (int i = 0; i < std::min<int>(cap, int(p.groups.size())); ++i) tiles[i] = p.ts;
  if (launches_per_step) {
    const int sets = int((p.groups.size() + kMaxGroups - 1) / kMaxGroups);
    // prepare and finish; the finish runs inside the last APPLY when the
    // update is fused (decided here without averaging or diagnostics)
    const bool fused = update_fusable(p, params, n, opt && opt->cautious,
                                      opt && opt->beta_ema >= 0.f, false, coeffs, steps);
    int l = n > 0 ? (fused ? 1 : 2) : 0;
    if (n > 0 && single_launch_ok(p, steps, fused)) {
      l += 1;
    } else {
      for (int j = 0; j < steps && n > 0; ++j) {
        const bool poly = !coeffs || coeffs[3 * j + 2] != 0.f;
        l += sets * (poly ? 3 : 2);
      }
    }
    *launches_per_step = l;
  }
  return MUON_OK;
}


// ---------------------------------------------------------------- AdamW
// Workspace of muon_adamw_step: descriptor table, then block prefix sums.
size_t adamw_off_prefix(int n) { return align_up(sizeof(VecDesc) * size_t(n), kAlign); }
size_t adamw_total(int n) { return adamw_off_prefix(n) + align_up(sizeof(int64_t) * size_t(n + 1), kAlign); }

size_t muon_adamw_workspace_bytes(int32_t n) { return n < 0 ? 0 : adamw_total(n); }

int muon_adamw_step(const muon_vec* params, const muon_vec* grads, muon_adamw_state* st,
                    const muon_adamw_hparams* hp, void* stream) {
  if (!st || !hp) return MUON_E_NULL;
  if (st->n < 0) return MUON_E_SHAPE;
  const float lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps, wd = hp->wd;
  if (!finite(lr) || !finite(wd) || !finite(eps) || eps < 0.f) return MUON_E_HPARAM;
  if (!(b1 >= 0.f && b1 < 1.f) || !(b2 >= 0.f && b2 < 1.f)) return MUON_E_HPARAM;
  const int n = st->n;
  if (n == 0) {
    st->step += 1;
    return MUON_OK;
  }
  if (!params || !grads || !st->m || !st->v) return MUON_E_NULL;
  std::vector<Range> ranges;
  std::vector<VecDesc> desc(n);
  std::vector<int64_t> prefix(n + 1, 0);
  for (int i = 0; i < n; ++i) {
    const muon_vec& P = params[i];
    const muon_vec& G = grads[i];
    if (P.numel < 0 || G.numel != P.numel) return MUON_E_SHAPE;
    if ((P.dtype != MUON_BF16 && P.dtype != MUON_F32) ||
        (G.dtype != MUON_BF16 && G.dtype != MUON_F32))
      return MUON_E_DTYPE;
    const int64_t ne = P.numel;
    float* m = st->m[i];
    float* v = st->v[i];
    if (ne > 0) {
      if (!P.ptr || !G.ptr || !m || !v) return MUON_E_NULL;
      if (reinterpret_cast<uintptr_t>(P.ptr) % esize(P.dtype) ||
          reinterpret_cast<uintptr_t>(G.ptr) % esize(G.dtype) ||
          reinterpret_cast<uintptr_t>(m) % 4 || reinterpret_cast<uintptr_t>(v) % 4)
        return MUON_E_ALIGN;
      add_range(ranges, P.ptr, size_t(ne) * esize(P.dtype));
      add_range(ranges, G.ptr, size_t(ne) * esize(G.dtype));
      add_range(ranges, m, size_t(ne) * 4);
      add_range(ranges, v, size_t(ne) * 4);
    }
    VecDesc& d = desc[i];
    std::memset(&d, 0, sizeof(d));
    d.p = P.ptr; d.g = G.ptr; d.m = m; d.v = v; d.n = ne;
    d.pdt = P.dtype; d.gdt = G.dtype;
    d.pvec = reinterpret_cast<uintptr_t>(P.ptr) % 16 == 0;
    d.gvec = reinterpret_cast<uintptr_t>(G.ptr) % 16 == 0;
    d.svec = reinterpret_cast<uintptr_t>(m) % 16 == 0 && reinterpret_cast<uintptr_t>(v) % 16 == 0;
    prefix[i + 1] = prefix[i] + (ne + kAdamChunk - 1) / kAdamChunk;
  }
  if (prefix[n] > int64_t(INT32_MAX)) return MUON_E_SHAPE;
  if (!st->workspace) return MUON_E_WORKSPACE;
  const size_t need = adamw_total(n);
  if (st->workspace_bytes < need) return MUON_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(st->workspace) % kAlign) return MUON_E_ALIGN;
  add_range(ranges, st->workspace, need);
  if (overlaps(ranges)) return MUON_E_ALIAS;

  std::vector<uint8_t> bytes(need, 0);
  std::memcpy(bytes.data(), desc.data(), sizeof(VecDesc) * size_t(n));
  std::memcpy(bytes.data() + adamw_off_prefix(n), prefix.data(), sizeof(int64_t) * size_t(n + 1));
  std::lock_guard<std::mutex> lk(g_mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the bias terms change with every step, so a replayed capture would
  // repeat stale ones: refuse capture
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MUON_E_HIP;
  if (cs != hipStreamCaptureStatusNone) return MUON_E_CAPTURE;
  int rc;
  if ((rc = upload_table(st->workspace, bytes, s)) != MUON_OK) return rc;

  // bias terms in double from the fp32 betas; (1 - b) in fp32
  const double t = double(st->step + 1);
  const double c1 = 1.0 - std::pow(double(b1), t);
  const double c2 = 1.0 - std::pow(double(b2), t);
  AdamArgs a;
  std::memset(&a, 0, sizeof(a));
  a.vecs = static_cast<const VecDesc*>(st->workspace);
  a.prefix = reinterpret_cast<const int64_t*>(static_cast<char*>(st->workspace) +
                                              adamw_off_prefix(n));
  a.nvec = n;
  a.b1 = b1;
  a.b2 = b2;
  {
    volatile float o1 = 1.0f - b1, o2 = 1.0f - b2, lrwd = lr * wd;   // fp32 roundings
    a.ob1 = o1;
    a.ob2 = o2;
    a.lrwd = lrwd;
  }
  a.step_size = static_cast<float>(double(lr) / c1);
  a.rsc2 = static_cast<float>(1.0 / std::sqrt(c2));
  a.eps = eps;
  probe_begin(MUON_PHASE_ADAMW, s);
  const hipError_t err = launch_adamw(a, prefix[n], s);
  probe_end(MUON_PHASE_ADAMW, s);
  if (err != hipSuccess) return MUON_E_HIP;
  st->step += 1;
  return MUON_OK;
}

}  // extern "C"
