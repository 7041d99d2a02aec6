// C ABI of the Muon step: argument validation, workspace layout and the
// launch sequence on the caller's stream.  Every argument is checked before
// the first HIP call, so every error status is returned without touching the
// device.
//
// Launch sequence for one set of up to MUON_GROUPS_PER_LAUNCH shape groups
// (each phase is ONE launch over the tiles of every matrix of every group):
//   head            M' = mu M + G, U = G + mu M', X0 = U (short side first),
//                   per-tile sums of u^2
//   norm_finalize   ||U||_F and 1/(||U||_F + 1e-7) per matrix
//   ns_steps x { gram, poly, update }   (plain Muon on bf16 weights: the last
//                   update applies the step itself; MuonGS, MuonH or stats:
//                   it also writes per-tile <W,O>, ||W||^2, ||O||^2 partials)
//   [tail_reduce] + tail_finalize   (variants and stats) the per-matrix sums
//                   (tail_reduce only where the last update did not write them:
//                   NorMuon, MeqMuon, fp32, odd row lengths)
//   tail_apply      W' = (1 - lr wd) W - lr s O~   (where not applied already)
// Update order: "[Deep Learning] Muon — 행렬 업데이트를 직교화하는 옵티마이저",
// section 3 "Muon의 업데이트 순서".
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <dlfcn.h>
#include <mutex>
#include <vector>

#include "muon_internal.h"

using namespace muon;

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
constexpr int64_t kMaxBlocks = (int64_t(1) << 24) - 1;

inline bool mul_ok(size_t a, size_t b, size_t* out) { return !__builtin_mul_overflow(a, b, out); }
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char* e = std::getenv("MUON_DEBUG");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

bool dtype_ok(int dtype) { return dtype == MUON_DTYPE_F32 || dtype == MUON_DTYPE_BF16; }

struct Layout {
  int64_t p, q, p_pad, q_pad;
  int trans;
  int64_t head_tiles, tail_tiles, tail_tiles_c;
  int64_t tile;             // NS GEMM block tile edge along p
  int64_t tile_n;           // update GEMM block tile edge along q
  size_t x_bytes, a_bytes, head_bytes, tail_bytes, scal_bytes;
  size_t rc_bytes, rcs_bytes, rcst_bytes;  // row/column partials, norms, chunk statistics
  size_t total;             // 0 on overflow
};

Layout make_layout(int64_t count, int64_t rows, int64_t cols, int dtype) {
  Layout L{};
  const size_t es = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  L.tile = dtype == MUON_DTYPE_BF16 ? kBf16PadP : kF32Tile;
  L.trans = rows > cols ? 1 : 0;
  L.p = rows < cols ? rows : cols;
  L.q = rows < cols ? cols : rows;
  L.p_pad = round_up(L.p, L.tile);
  // bf16: the long side is padded to the update's column tile, 256, or 128
  // for a padded short side of 512 (the 512x128 update tiles)
  L.tile_n = dtype != MUON_DTYPE_BF16 ? kF32Tile : (L.p_pad == kUpd512P ? kUpd512TileN : kBf16PadQ);
  L.q_pad = round_up(L.q, L.tile_n);
  L.head_tiles = (L.p_pad / kEwTile) * (L.q_pad / kEwTile);
  L.tail_tiles_c = cdiv(cols, kEwTile);
  L.tail_tiles = cdiv(rows, kEwTile) * L.tail_tiles_c;
  size_t x, a, h, t, s;
  const size_t c = size_t(count);
  if (!mul_ok(c, size_t(L.p_pad * L.q_pad) * es, &x) || !mul_ok(c, size_t(L.p_pad * L.p_pad) * es, &a) ||
      !mul_ok(c, size_t(L.head_tiles) * 8, &h) || !mul_ok(c, size_t(L.tail_tiles) * 24, &t) ||
      !mul_ok(c, size_t(kScal) * 4, &s))
    return L;  // total stays 0
  size_t rc, rcs, rcst;
  if (!mul_ok(c, size_t(L.tail_tiles) * 2 * kEwTile * 4, &rc) ||
      !mul_ok(c, size_t(rows + cols) * 4, &rcs) ||
      !mul_ok(c, size_t(rc_chunks(int(rows), int(cols))) * 5 * 4, &rcst))
    return L;
  L.x_bytes = align_up(x);
  L.a_bytes = align_up(a);
  L.head_bytes = align_up(h);
  L.tail_bytes = align_up(t);
  L.scal_bytes = align_up(s);
  L.rc_bytes = align_up(rc);
  L.rcs_bytes = align_up(rcs);
  L.rcst_bytes = align_up(rcst);
  L.total = 2 * L.x_bytes + 2 * L.a_bytes + L.head_bytes + L.tail_bytes + L.scal_bytes +
            L.rc_bytes + L.rcs_bytes + L.rcst_bytes;
  if (L.total < L.x_bytes) L.total = 0;
  return L;
}

int check_scalars(double lr, double momentum, double wd, int ns_steps, double a, double b,
                  double c, int variant) {
  if (!std::isfinite(lr) || !std::isfinite(momentum) || !std::isfinite(wd) ||
      !std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
    return MUON_ERR_INVALID_ARGUMENT;
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS) return MUON_ERR_INVALID_ARGUMENT;
  const int base = variant & 0xff;
  if ((variant & ~(0xff | MUON_SCALE_KELLER)) != 0 || base < MUON_VARIANT_MUON ||
      base > MUON_VARIANT_MEQMUON)
    return MUON_ERR_INVALID_ARGUMENT;
  return MUON_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_group(const muon_group& g, int dtype) {
  if (g.count < 0) return MUON_ERR_INVALID_ARGUMENT;
  if (g.count == 0) return MUON_OK;
  if (g.rows < 1 || g.cols < 1 || g.rows > MUON_MAX_DIM || g.cols > MUON_MAX_DIM)
    return MUON_ERR_INVALID_SHAPE;
  const bool any_tab = g.W_table || g.G_table || g.M_table;
  const bool any_stk = g.W || g.G || g.M;
  if (any_tab == any_stk) return MUON_ERR_INVALID_ARGUMENT;  // neither form, or both
  if (any_tab && !(g.W_table && g.G_table && g.M_table)) return MUON_ERR_INVALID_ARGUMENT;
  if (any_stk) {
    if (!(g.W && g.G && g.M)) return MUON_ERR_INVALID_ARGUMENT;
    const size_t es = dtype == MUON_DTYPE_BF16 ? 2 : 4;
    size_t n;
    if (!mul_ok(size_t(g.count), size_t(g.rows) * size_t(g.cols), &n)) return MUON_ERR_INVALID_SHAPE;
    if (ranges_overlap(g.W, n * es, g.G, n * es) || ranges_overlap(g.W, n * es, g.M, n * 4) ||
        ranges_overlap(g.G, n * es, g.M, n * 4))
      return MUON_ERR_INVALID_ARGUMENT;
  }
  return MUON_OK;
}

// Blocks per matrix of each phase.
struct PhaseTiles {
  int64_t head, gram, update, tail;
};
// bf16 matrices whose symmetric products may take 256x256 tiles (whether
// they do depends on the launch: see the tile lists in run_groups).
bool syrk_big_eligible(const Layout& L, bool bf16) {
  return bf16 && L.p >= kBigMinP && L.p_pad % kBigTile == 0;
}
// bf16 matrices whose update takes the 512x128 tiles (always: their long
// side is padded to a multiple of 128 only).
bool upd512(const Layout& L, bool bf16) { return bf16 && L.p_pad == kUpd512P; }
// bf16 matrices whose update may take 256x256 tiles.
bool upd_big_eligible(const Layout& L, bool bf16) {
  return syrk_big_eligible(L, bf16) && !upd512(L, bf16) && L.q_pad % kBigTile == 0;
}
PhaseTiles phase_tiles(const Layout& L, bool bf16) {
  PhaseTiles t;
  const int64_t ts = bf16 ? kSyrkTile : kF32Tile;
  const int64_t nt = L.p_pad / ts;
  t.head = L.head_tiles;
  t.gram = nt * (nt + 1) / 2;
  t.update = !bf16 ? nt * (L.q_pad / kF32Tile)
                   : upd512(L, bf16) ? L.q_pad / kUpd512TileN
                                     : (L.p_pad / kUpdTileM) * (L.q_pad / kUpdTileN);
  t.tail = L.tail_tiles;
  return t;
}

const char* kPhaseNames[] = {"head",        "norm_finalize", "gram",       "poly",  "update",
                             "tail_reduce", "tail_finalize", "tail_apply", "adamw", "update_tail"};
static_assert(sizeof(kPhaseNames) / sizeof(kPhaseNames[0]) == MUON_NUM_PHASES,
              "one name per phase");
constexpr int kPhaseAdamw = 8;
constexpr int kPhaseUpdateTail = 9;  // last update launch with the step fused in

// ---- optional roctx ranges (MUON_TRACE=1): one range per entry-point call
// and one per launch, named by its phase, on the calling thread's timeline
// (rocprofv3 --marker-trace). The roctx library is opened at run time, so
// the library does not depend on it when tracing is off.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx* roctx() {
  static Roctx r;
  static std::once_flag once;
  std::call_once(once, [] {
    const char* e = std::getenv("MUON_TRACE");
    if (!e || !*e || *e == '0') return;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (!h) {
      std::fprintf(stderr, "muon: MUON_TRACE is set but no roctx library loads: %s\n", dlerror());
      return;
    }
    Roctx t;
    t.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    t.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (t.push && t.pop) r = t;
  });
  return r.push ? &r : nullptr;
}

struct TraceRange {
  explicit TraceRange(const char* name) : t(roctx()) {
    if (t) t->push(name);
  }
  ~TraceRange() {
    if (t) t->pop();
  }
  const Roctx* t;
};

// ---- optional phase timing (HIP events around each launch)
struct ProfRecord {
  int phase;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Opens the launch's trace range and records its start event when
// profiling is on; finish_launch closes both.
hipEvent_t prof_start(hipStream_t s, int phase) {
  if (const Roctx* t = roctx()) t->push(kPhaseNames[phase]);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return nullptr;
  hipEvent_t e = pooled_event();
  if (e && hipEventRecord(e, s) != hipSuccess) {
    g_event_pool.push_back(e);
    return nullptr;
  }
  return e;
}

void prof_stop(hipEvent_t start, int phase, hipStream_t s) {
  if (!start) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t e = pooled_event();
  if (!e || hipEventRecord(e, s) != hipSuccess) {
    g_event_pool.push_back(start);
    if (e) g_event_pool.push_back(e);
    return;
  }
  g_prof_records.push_back({phase, start, e});
}

int finish_launch(hipError_t e, int phase, hipStream_t s, hipEvent_t t0 = nullptr) {
  prof_stop(t0, phase, s);
  if (const Roctx* t = roctx()) t->pop();
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    g_last_hip_error = int(e);
    if (debug_sync())
      std::fprintf(stderr, "muon: %s failed: %s\n", kPhaseNames[phase], hipGetErrorString(e));
    return MUON_ERR_HIP;
  }
  return MUON_OK;
}

// Compute units per XCD of the current device (0 on a HIP error), cached.
int cus_per_xcd() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
    return 0;
  if (dev >= 0 && dev < 64) cache[dev] = n / 8;
  return n / 8;
}

// Static tile list of one persistent Newton-Schulz launch over the groups
// with tiles in it (tiles_per_matrix > 0): groups with more K steps per tile
// first (they finish last otherwise), up to the given number of resident
// blocks per XCD.  An empty list (ngroups 0) is not launched.
TileList make_tile_list(const Batch& bt, const int64_t* tiles_per_matrix, const int64_t* k_len,
                        int blocks_per_xcd_max) {
  TileList tl{};
  int order[kMaxGroups];
  int n = 0;
  for (int k = 0; k < bt.ngroups; ++k)
    if (tiles_per_matrix[k] > 0) order[n++] = k;
  std::stable_sort(order, order + n, [&](int a, int b) { return k_len[a] > k_len[b]; });
  tl.ngroups = n;
  int64_t per_xcd = 0;
  for (int i = 0; i < n; ++i) {
    const int k = order[i];
    tl.group[i] = k;
    tl.tiles[i] = int(tiles_per_matrix[k]);
    tl.n[i] = bt.g[k].count * tiles_per_matrix[k];
    per_xcd += (tl.n[i] + 7) / 8;
  }
  tl.blocks_per_xcd = int(std::max<int64_t>(1, std::min<int64_t>(blocks_per_xcd_max, per_xcd)));
  return tl;
}

struct Sel {
  const muon_group* g;
  Layout L;
  int64_t stats_index;  // first matrix of the group in the stats array
};

// Every check that needs no workspace: dtype, scalars, groups and the launch
// size limits.  Sets the workspace bytes the call needs (0 for an empty
// batch) and the number of matrices.
int validate_groups(const muon_group* groups, int ngroups, int dtype, double lr, double momentum,
                    double wd, int ns_steps, double a, double b, double c, int variant,
                    size_t* need_out, int64_t* n_out) {
  if (!dtype_ok(dtype)) return MUON_ERR_UNSUPPORTED_DTYPE;
  int st = check_scalars(lr, momentum, wd, ns_steps, a, b, c, variant);
  if (st != MUON_OK) return st;
  if (ngroups < 0 || (ngroups > 0 && !groups)) return MUON_ERR_INVALID_ARGUMENT;

  size_t need = 0;
  int64_t n_matrices = 0;
  int64_t blocks = 0;
  for (int i = 0; i < ngroups; ++i) {
    st = check_group(groups[i], dtype);
    if (st != MUON_OK) return st;
    if (groups[i].count == 0) continue;
    const Layout L = make_layout(groups[i].count, groups[i].rows, groups[i].cols, dtype);
    if (L.total == 0) return MUON_ERR_INVALID_SHAPE;
    const PhaseTiles pt = phase_tiles(L, dtype == MUON_DTYPE_BF16);
    int64_t most = pt.head > pt.update ? pt.head : pt.update;
    most = most > pt.tail ? most : pt.tail;
    // The dispatch grid is counted in work-items (32 bits): at 256 threads a
    // block, one launch holds fewer than 2^24 blocks.
    if (groups[i].count > kMaxBlocks / most) return MUON_ERR_INVALID_SHAPE;
    blocks += groups[i].count * most;
    if (blocks > kMaxBlocks) return MUON_ERR_INVALID_SHAPE;
    need += L.total;
    n_matrices += groups[i].count;
  }
  *need_out = n_matrices ? need + kAlign : 0;
  *n_out = n_matrices;
  return MUON_OK;
}

int run_groups(const muon_group* groups, int ngroups, int dtype, double lr, double momentum,
               double wd, int ns_steps, double a, double b, double c, int variant,
               void* workspace, size_t workspace_bytes, float* stats, void* stream) {
  TraceRange range("muon_step");
  size_t need = 0;
  int64_t n_matrices = 0;
  int st = validate_groups(groups, ngroups, dtype, lr, momentum, wd, ns_steps, a, b, c, variant,
                           &need, &n_matrices);
  if (st != MUON_OK) return st;
  if (n_matrices == 0) return MUON_OK;  // empty batch: nothing to do
  if (!workspace) return MUON_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return MUON_ERR_WORKSPACE_TOO_SMALL;
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& g = groups[i];
    if (g.count == 0 || !g.W) continue;
    const size_t es = dtype == MUON_DTYPE_BF16 ? 2 : 4;
    const size_t n = size_t(g.count) * size_t(g.rows) * size_t(g.cols);
    if (ranges_overlap(workspace, workspace_bytes, g.W, n * es) ||
        ranges_overlap(workspace, workspace_bytes, g.G, n * es) ||
        ranges_overlap(workspace, workspace_bytes, g.M, n * 4))
      return MUON_ERR_INVALID_ARGUMENT;
  }

  // ---- all arguments valid: enqueue work
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear an unrelated earlier error
  const bool bf16 = dtype == MUON_DTYPE_BF16;
  char* base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(workspace)));
  Hyper h;
  h.lr = float(lr);
  h.momentum = float(momentum);
  h.wd = float(wd);
  h.a = float(a);
  h.b = float(b);
  h.c = float(c);
  h.ns_steps = ns_steps;
  h.variant = variant & 0xff;
  const bool keller = (variant & MUON_SCALE_KELLER) != 0;
  const bool reduce = h.variant != MUON_VARIANT_MUON || stats != nullptr;
  const bool rc_variant = h.variant == MUON_VARIANT_NORMUON || h.variant == MUON_VARIANT_MEQMUON;

  Sel sel[kMaxGroups];
  int nsel = 0;
  int64_t stats_index = 0;
  int gi = 0;
  while (gi < ngroups) {
    nsel = 0;
    for (; gi < ngroups && nsel < kMaxGroups; ++gi) {
      if (groups[gi].count == 0) continue;
      sel[nsel].g = &groups[gi];
      sel[nsel].L = make_layout(groups[gi].count, groups[gi].rows, groups[gi].cols, dtype);
      sel[nsel].stats_index = stats_index;
      stats_index += groups[gi].count;
      ++nsel;
    }
    if (nsel == 0) break;

    Batch bt;
    std::memset(&bt, 0, sizeof(bt));
    bt.ngroups = nsel;
    Work w_head{}, w_one{}, w_gram{}, w_upd{}, w_tail{}, w_red{};
    w_head.ngroups = w_one.ngroups = w_gram.ngroups = w_upd.ngroups = w_tail.ngroups = nsel;
    w_red.ngroups = nsel;
    for (int k = 0; k < nsel; ++k) {
      const muon_group& u = *sel[k].g;
      const Layout& L = sel[k].L;
      MatGroup& m = bt.g[k];
      m.W_tab = u.W_table;
      m.G_tab = u.G_table;
      m.M_tab = u.M_table;
      m.W = static_cast<char*>(u.W);
      m.G = static_cast<const char*>(u.G);
      m.M = u.M;
      m.count = u.count;
      m.rows = int(u.rows);
      m.cols = int(u.cols);
      m.p = int(L.p);
      m.q = int(L.q);
      m.p_pad = int(L.p_pad);
      m.q_pad = int(L.q_pad);
      m.trans = L.trans;
      m.head_tiles = int(L.head_tiles);
      m.tail_tiles = int(L.tail_tiles);
      m.tail_tiles_c = int(L.tail_tiles_c);
      m.X0 = base;
      base += L.x_bytes;
      m.X1 = base;
      base += L.x_bytes;
      m.A = base;
      base += L.a_bytes;
      m.B = base;
      base += L.a_bytes;
      m.x_stride = L.p_pad * L.q_pad;
      m.a_stride = L.p_pad * L.p_pad;
      m.head_part = reinterpret_cast<double*>(base);
      base += L.head_bytes;
      m.tail_part = reinterpret_cast<double*>(base);
      base += L.tail_bytes;
      m.scal = reinterpret_cast<float*>(base);
      base += L.scal_bytes;
      m.rc_part = reinterpret_cast<float*>(base);
      base += L.rc_bytes;
      m.rc_norm2 = reinterpret_cast<float*>(base);
      base += L.rcs_bytes;
      m.rc_stat = reinterpret_cast<float*>(base);
      base += L.rcst_bytes;
      m.stats = stats ? stats + sel[k].stats_index * MUON_STATS_PER_MATRIX : nullptr;
      m.decay = float(1.0 - lr * wd);
      // Shape factor: Moonlight 0.2*sqrt(max(rows, cols)), or Keller
      // max(1, rows/cols)^0.5.
      const double sfac = keller ? std::sqrt(std::max(1.0, double(u.rows) / double(u.cols)))
                                 : 0.2 * std::sqrt(double(L.q));
      m.step = float(lr * sfac);
      // Plain Muon without statistics needs no reduction over the finished O,
      // so the last Newton-Schulz update applies the step to W itself (bf16
      // weights whose row length allows whole 16-byte chunks).
      m.fuse = (bf16 && !reduce && ns_steps >= 1 && (u.cols % 8) == 0) ? 1 : 0;
      // MuonGS, MuonH and statistics need the per-matrix sums of <W,O>,
      // ||W||^2 and ||O||^2 before W' can be written: the last update writes
      // their per-tile partials itself (same row-length rule), so no separate
      // reduction pass reads W and O (NorMuon and MeqMuon also need row and
      // column sums, which the reduction pass provides).
      m.red = (bf16 && reduce && !rc_variant && ns_steps >= 1 && (u.cols % 8) == 0) ? 1 : 0;
      m.red_tiles = int(L.tail_tiles);   // set to the update tiles below when red

      const PhaseTiles pt = phase_tiles(L, dtype == MUON_DTYPE_BF16);
      w_head.tiles[k] = int(pt.head);
      w_one.tiles[k] = 1;
      w_gram.tiles[k] = int(pt.gram);
      w_upd.tiles[k] = int(pt.update);
      w_tail.tiles[k] = m.fuse ? 0 : int(pt.tail);
      w_red.tiles[k] = (m.fuse || m.red) ? 0 : int(pt.tail);
    }
    bool any_fused = false, any_red = false;
    for (int k = 0; k < nsel; ++k) {
      any_fused = any_fused || bt.g[k].fuse;
      any_red = any_red || bt.g[k].red;
    }
    // Symmetric products: one launch over the groups in 128x128 tiles and
    // one over the large groups in 256x256 tiles (each only if non-empty).
    TileList tl_gram{}, tl_poly{}, tl_gram_big{}, tl_poly_big{}, tl_upd{}, tl_upd_big{},
        tl_upd_512{};
    if (bf16) {
      const int cpx = cus_per_xcd();
      if (cpx == 0) {
        g_last_hip_error = int(hipErrorInvalidDevice);
        return MUON_ERR_HIP;
      }
      // 256x256 tiles where the launch has enough of them: measured, they
      // are faster on a GPT-400M model (short side 1024) and on MoE experts
      // (512), slower on GPT-160M (768: 1.7 rounds of symmetric tiles, 5 of
      // update tiles).
      int64_t big_syrk = 0, big_upd = 0;
      for (int k = 0; k < nsel; ++k) {
        if (!syrk_big_eligible(sel[k].L, true)) continue;
        const int64_t nb = sel[k].L.p_pad / kBigTile;
        big_syrk += bt.g[k].count * (nb * (nb + 1) / 2);
        if (upd_big_eligible(sel[k].L, true))
          big_upd += bt.g[k].count * nb * (sel[k].L.q_pad / kBigTile);
      }
      const bool use_big_syrk = big_syrk >= int64_t(kSyrkBigMinRounds) * 8 * cpx;
      const bool use_big_upd = big_upd >= int64_t(kUpdBigMinRounds) * 8 * cpx;
      int64_t nt[kMaxGroups], ntb[kMaxGroups], npt[kMaxGroups], nptb[kMaxGroups], nu[kMaxGroups],
          nub[kMaxGroups], nu5[kMaxGroups], kq[kMaxGroups], kp[kMaxGroups];
      for (int k = 0; k < nsel; ++k) {
        const Layout& L = sel[k].L;
        const bool big = use_big_syrk && syrk_big_eligible(L, true);
        const bool ubig = use_big_upd && upd_big_eligible(L, true);
        const bool u512 = upd512(L, true);
        const int64_t nb = L.p_pad / kBigTile;
        nt[k] = big ? 0 : w_gram.tiles[k];
        ntb[k] = big ? nb * (nb + 1) / 2 : 0;
        // the polynomial (K = p) keeps 128-wide tiles below kPolyBigMinP:
        // one 256x256 tile's epilogue moves 512 KiB (B, its mirror, b*A
        // for both) with no second block on the CU to overlap it, which
        // short contractions do not amortise (measured: p = 512 and 1024
        // faster in 128-wide tiles, p = 2048 in 256-wide)
        const bool pbig = big && L.p >= kPolyBigMinP;
        npt[k] = pbig ? 0 : w_gram.tiles[k];
        nptb[k] = pbig ? nb * (nb + 1) / 2 : 0;
        nu[k] = (ubig || u512) ? 0 : w_upd.tiles[k];
        nub[k] = ubig ? nb * (L.q_pad / kBigTile) : 0;
        nu5[k] = u512 ? w_upd.tiles[k] : 0;
        if (bt.g[k].red) bt.g[k].red_tiles = int(nu5[k] ? nu5[k] : nub[k] ? nub[k] : nu[k]);
        kq[k] = bt.g[k].q_pad;
        kp[k] = bt.g[k].p_pad;
      }
      tl_gram = make_tile_list(bt, nt, kq, kSyrkBlocksPerCU * cpx);
      tl_poly = make_tile_list(bt, npt, kp, kSyrkBlocksPerCU * cpx);
      tl_gram_big = make_tile_list(bt, ntb, kq, kBigBlocksPerCU * cpx);
      tl_poly_big = make_tile_list(bt, nptb, kp, kBigBlocksPerCU * cpx);
      tl_upd = make_tile_list(bt, nu, kp, kUpdBlocksPerCU * cpx);
      tl_upd_big = make_tile_list(bt, nub, kp, kBigBlocksPerCU * cpx);
      tl_upd_512 = make_tile_list(bt, nu5, kp, kBigBlocksPerCU * cpx);
    }
    hipEvent_t t0 = nullptr;
    Work* ws[] = {&w_head, &w_one, &w_gram, &w_upd, &w_tail, &w_red};
    for (Work* w : ws) {
      w->begin[0] = 0;
      for (int k = 0; k < nsel; ++k) w->begin[k + 1] = w->begin[k] + bt.g[k].count * w->tiles[k];
    }

    if ((t0 = prof_start(s, 0)), (st = finish_launch(launch_head(bt, w_head, bf16, h.momentum, s), 0, s, t0))) return st;
    if ((t0 = prof_start(s, 1)), (st = finish_launch(launch_norm_finalize(bt, w_one, s), 1, s, t0))) return st;
    for (int it = 0; it < ns_steps; ++it) {
      if (bf16) {
        if (tl_gram.ngroups &&
            ((t0 = prof_start(s, 2)), (st = finish_launch(launch_gram_bf16(bt, tl_gram, it, false, s), 2, s, t0))))
          return st;
        if (tl_gram_big.ngroups &&
            ((t0 = prof_start(s, 2)), (st = finish_launch(launch_gram_bf16(bt, tl_gram_big, it, true, s), 2, s, t0))))
          return st;
        if (tl_poly.ngroups &&
            ((t0 = prof_start(s, 3)), (st = finish_launch(launch_poly_bf16(bt, tl_poly, h.a, h.b, h.c, false, s), 3, s, t0))))
          return st;
        if (tl_poly_big.ngroups &&
            ((t0 = prof_start(s, 3)),
             (st = finish_launch(launch_poly_bf16(bt, tl_poly_big, h.a, h.b, h.c, true, s), 3, s, t0))))
          return st;
        // (a call applies the step only when it reduces nothing: never both)
        const int fuse_tail = it != ns_steps - 1 ? 0 : any_fused ? kLastApply : any_red ? kLastReduce : 0;
        const int ph = fuse_tail ? kPhaseUpdateTail : 4;
        for (int cfg = kUpdCfg128; cfg <= kUpdCfg512; ++cfg) {
          TileList tl = cfg == kUpdCfg512 ? tl_upd_512 : cfg == kUpdCfg256 ? tl_upd_big : tl_upd;
          if (!tl.ngroups) continue;
          tl.fuse_tail = fuse_tail;
          if ((t0 = prof_start(s, ph)), (st = finish_launch(launch_update_bf16(bt, tl, it, cfg, s), ph, s, t0)))
            return st;
        }
      } else {
        if ((t0 = prof_start(s, 2)), (st = finish_launch(launch_gram_f32(bt, w_gram, it, s), 2, s, t0))) return st;
        if ((t0 = prof_start(s, 3)), (st = finish_launch(launch_poly_f32(bt, w_gram, h.b, h.c, s), 3, s, t0))) return st;
        if ((t0 = prof_start(s, 4)), (st = finish_launch(launch_update_f32(bt, w_upd, it, h.a, s), 4, s, t0))) return st;
      }
    }
    if (reduce) {
      const bool rc = h.variant == MUON_VARIANT_NORMUON || h.variant == MUON_VARIANT_MEQMUON;
      if (w_red.begin[nsel] > 0 &&  // every group may have been reduced by its last update
          ((t0 = prof_start(s, 5)),
           (st = finish_launch(launch_tail_reduce(bt, w_red, bf16, ns_steps, rc, s), 5, s, t0))))
        return st;
      if (rc) {
        // row and column norms in blocks of kRcChunk rows or columns
        Work w_rc{};
        w_rc.ngroups = nsel;
        w_rc.begin[0] = 0;
        for (int k = 0; k < nsel; ++k) {
          w_rc.tiles[k] = rc_chunks(bt.g[k].rows, bt.g[k].cols);
          w_rc.begin[k + 1] = w_rc.begin[k] + bt.g[k].count * w_rc.tiles[k];
        }
        if ((t0 = prof_start(s, 6)), (st = finish_launch(launch_rc_sum(bt, w_rc, s), 6, s, t0))) return st;
      }
      if ((t0 = prof_start(s, 6)), (st = finish_launch(launch_tail_finalize(bt, w_one, h.variant, rc, s), 6, s, t0))) return st;
    }
    if (w_tail.begin[nsel] > 0 &&  // every group may have been finished by its last update
        ((t0 = prof_start(s, 7)), (st = finish_launch(launch_tail_apply(bt, w_tail, bf16, h, reduce, s),
                                                    7, s, t0))))
      return st;
  }
  return MUON_OK;
}

// ---- AdamW over many tensors
// A tensor is split into segments of at most kAdamSegMaxBlocks blocks, and a
// launch takes up to kAdamSegs segments and at most kMaxBlocks blocks.
constexpr int64_t kAdamSegMaxBlocks = int64_t(1) << 22;

int check_adamw_scalars(double beta1, double beta2, double eps, int64_t step) {
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0)) return MUON_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(eps) || eps < 0.0) return MUON_ERR_INVALID_ARGUMENT;
  if (step < 1) return MUON_ERR_INVALID_ARGUMENT;
  return MUON_OK;
}

int check_adamw_tensors(const muon_adamw_tensor* t, int64_t count, int dtype) {
  if (count < 0 || (count > 0 && !t)) return MUON_ERR_INVALID_ARGUMENT;
  const size_t es = dtype == MUON_DTYPE_BF16 ? 2 : 4;
  struct Range {
    uintptr_t lo, hi;
  };
  std::vector<Range> r;
  r.reserve(size_t(count) * 4);
  for (int64_t i = 0; i < count; ++i) {
    const muon_adamw_tensor& x = t[i];
    if (!std::isfinite(x.lr) || !std::isfinite(x.weight_decay)) return MUON_ERR_INVALID_ARGUMENT;
    if (x.n < 0 || x.n > MUON_ADAMW_MAX_ELEMENTS) return MUON_ERR_INVALID_SHAPE;
    if (x.n == 0) continue;
    if (!x.P || !x.G || !x.m || !x.v) return MUON_ERR_INVALID_ARGUMENT;
    const size_t n = size_t(x.n);
    r.push_back({reinterpret_cast<uintptr_t>(x.P), reinterpret_cast<uintptr_t>(x.P) + n * es});
    r.push_back({reinterpret_cast<uintptr_t>(x.G), reinterpret_cast<uintptr_t>(x.G) + n * es});
    r.push_back({reinterpret_cast<uintptr_t>(x.m), reinterpret_cast<uintptr_t>(x.m) + n * 4});
    r.push_back({reinterpret_cast<uintptr_t>(x.v), reinterpret_cast<uintptr_t>(x.v) + n * 4});
  }
  // No buffer of any tensor may overlap another buffer (of the same or of
  // another tensor): sorted by start, each range must end before the next.
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi) return MUON_ERR_INVALID_ARGUMENT;
  return MUON_OK;
}

int run_adamw(const muon_adamw_tensor* t, int64_t count, int dtype, double beta1, double beta2,
              double eps, int64_t step, void* stream) {
  TraceRange range("muon_adamw_step");
  if (!dtype_ok(dtype)) return MUON_ERR_UNSUPPORTED_DTYPE;
  int st = check_adamw_scalars(beta1, beta2, eps, step);
  if (st != MUON_OK) return st;
  st = check_adamw_tensors(t, count, dtype);
  if (st != MUON_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool bf16 = dtype == MUON_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  // Bias corrections in double: 1 - beta^t.
  const double bc1 = 1.0 - std::pow(beta1, double(step));
  const double bc2 = 1.0 - std::pow(beta2, double(step));
  AdamBatch bt;
  std::memset(&bt, 0, sizeof(bt));
  bt.beta1 = float(beta1);
  bt.beta2 = float(beta2);
  bt.one_minus_beta1 = float(1.0 - beta1);
  bt.one_minus_beta2 = float(1.0 - beta2);
  bt.eps = float(eps);
  bt.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));

  auto flush = [&]() -> int {
    if (bt.nseg == 0) return MUON_OK;
    hipEvent_t t0 = prof_start(s, kPhaseAdamw);
    const int r = finish_launch(launch_adamw(bt, bf16, s), kPhaseAdamw, s, t0);
    bt.nseg = 0;
    bt.begin[0] = 0;
    return r;
  };
  for (int64_t i = 0; i < count; ++i) {
    const muon_adamw_tensor& x = t[i];
    if (x.n == 0) continue;
    const uintptr_t vp = reinterpret_cast<uintptr_t>(x.P), vg = reinterpret_cast<uintptr_t>(x.G);
    const uintptr_t vm = reinterpret_cast<uintptr_t>(x.m), vv = reinterpret_cast<uintptr_t>(x.v);
    const size_t va = es * kAdamVec;
    const int vec = (vp % va == 0 && vg % va == 0 && vm % 16 == 0 && vv % 16 == 0) ? 1 : 0;
    const float decay = float(1.0 - x.lr * x.weight_decay);
    const float step_size = float(x.lr / bc1);
    for (int64_t off = 0; off < x.n;) {
      const int64_t blocks = std::min(cdiv(x.n - off, kAdamChunk), kAdamSegMaxBlocks);
      if (bt.nseg == kAdamSegs || bt.begin[bt.nseg] + blocks > kMaxBlocks) {
        if ((st = flush()) != MUON_OK) return st;
      }
      const int64_t n = std::min(x.n - off, blocks * int64_t(kAdamChunk));
      AdamSeg& g = bt.seg[bt.nseg];
      g.P = static_cast<char*>(x.P) + size_t(off) * es;
      g.G = static_cast<const char*>(x.G) + size_t(off) * es;
      g.m = x.m + off;
      g.v = x.v + off;
      g.n = n;
      g.decay = decay;
      g.step_size = step_size;
      g.vec = vec;
      bt.begin[bt.nseg + 1] = bt.begin[bt.nseg] + blocks;
      ++bt.nseg;
      off += n;
    }
  }
  return flush();
}

// ---- the workspace of muon_step_grouped_noalloc: one static array per GPU
// (each device holds its own copy while the process lives).  Host code never
// uses the array's name as an address: its device address is looked up once
// per device with hipGetSymbolAddress (with that device current) and kept.
constexpr size_t kScratchBytes = MUON_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of the current device's scratch array (null on a HIP error,
// which is then kept for muon_last_hip_error).
void* scratch_on_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    g_last_hip_error = int(e != hipSuccess ? e : hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = int(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int muon_adamw_step(void* P, const void* G, float* m, float* v, int64_t n, int dtype, double lr,
                    double beta1, double beta2, double eps, double weight_decay, int64_t step,
                    void* stream) {
  muon_adamw_tensor t{};
  t.P = P;
  t.G = G;
  t.m = m;
  t.v = v;
  t.n = n;
  t.lr = lr;
  t.weight_decay = weight_decay;
  return run_adamw(&t, 1, dtype, beta1, beta2, eps, step, stream);
}

int muon_adamw_step_grouped(const muon_adamw_tensor* tensors, int64_t count, int dtype,
                            double beta1, double beta2, double eps, int64_t step, void* stream) {
  return run_adamw(tensors, count, dtype, beta1, beta2, eps, step, stream);
}

size_t muon_workspace_bytes(int64_t count, int64_t rows, int64_t cols, int dtype) {
  if (!dtype_ok(dtype) || count < 0) return 0;
  if (count == 0) return 0;
  if (rows < 1 || cols < 1 || rows > MUON_MAX_DIM || cols > MUON_MAX_DIM) return 0;
  const Layout L = make_layout(count, rows, cols, dtype);
  return L.total ? L.total + kAlign : 0;
}

size_t muon_workspace_bytes_grouped(const muon_group* groups, int ngroups, int dtype) {
  if (!dtype_ok(dtype) || ngroups < 0 || (ngroups > 0 && !groups)) return 0;
  size_t need = 0;
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& g = groups[i];
    if (g.count < 0) return 0;
    if (g.count == 0) continue;
    if (g.rows < 1 || g.cols < 1 || g.rows > MUON_MAX_DIM || g.cols > MUON_MAX_DIM) return 0;
    const Layout L = make_layout(g.count, g.rows, g.cols, dtype);
    if (!L.total) return 0;
    need += L.total;
  }
  return need ? need + kAlign : 0;
}

int muon_step(void* W, const void* G, float* M, int64_t rows, int64_t cols, int dtype, double lr,
              double momentum, double weight_decay, int ns_steps, double a, double b, double c,
              int variant, void* workspace, size_t workspace_bytes, float* stats, void* stream) {
  if (!W || !G || !M) return MUON_ERR_INVALID_ARGUMENT;
  muon_group g{};
  g.count = 1;
  g.rows = rows;
  g.cols = cols;
  g.W = W;
  g.G = G;
  g.M = M;
  return run_groups(&g, 1, dtype, lr, momentum, weight_decay, ns_steps, a, b, c, variant,
                    workspace, workspace_bytes, stats, stream);
}

int muon_step_batched(void* const* W, const void* const* G, float* const* M, int64_t count,
                      int64_t rows, int64_t cols, int dtype, double lr, double momentum,
                      double weight_decay, int ns_steps, double a, double b, double c, int variant,
                      void* workspace, size_t workspace_bytes, float* stats, void* stream) {
  if (count < 0) return MUON_ERR_INVALID_ARGUMENT;
  if (count > 0 && (!W || !G || !M)) return MUON_ERR_INVALID_ARGUMENT;
  muon_group g{};
  g.count = count;
  g.rows = rows;
  g.cols = cols;
  g.W_table = W;
  g.G_table = G;
  g.M_table = M;
  return run_groups(&g, 1, dtype, lr, momentum, weight_decay, ns_steps, a, b, c, variant,
                    workspace, workspace_bytes, stats, stream);
}

int muon_step_grouped(const muon_group* groups, int ngroups, int dtype, double lr, double momentum,
                      double weight_decay, int ns_steps, double a, double b, double c, int variant,
                      void* workspace, size_t workspace_bytes, float* stats, void* stream) {
  return run_groups(groups, ngroups, dtype, lr, momentum, weight_decay, ns_steps, a, b, c,
                    variant, workspace, workspace_bytes, stats, stream);
}

int muon_step_grouped_noalloc(const muon_group* groups, int ngroups, int dtype, double lr,
                              double momentum, double weight_decay, int ns_steps, double a,
                              double b, double c, int variant, float* stats, void* stream) {
  size_t need = 0;
  int64_t n_matrices = 0;
  const int st = validate_groups(groups, ngroups, dtype, lr, momentum, weight_decay, ns_steps, a, b,
                                 c, variant, &need, &n_matrices);
  if (st != MUON_OK) return st;
  if (n_matrices == 0) return MUON_OK;
  if (need > kScratchBytes) return MUON_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_on_current_device();
  if (!ws) return MUON_ERR_HIP;
  return run_groups(groups, ngroups, dtype, lr, momentum, weight_decay, ns_steps, a, b, c, variant,
                    ws, kScratchBytes, stats, stream);
}

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MUON_ERR_INVALID_SHAPE: return "invalid shape";
    case MUON_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MUON_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int muon_last_hip_error(void) { return g_last_hip_error; }

int muon_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  return MUON_OK;
}

int muon_profile_read(double* ms_total, int64_t* launches, int nphases) {
  if (!ms_total || !launches || nphases < 1) return MUON_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int status = MUON_OK;
  for (const ProfRecord& r : g_prof_records) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) {
      g_last_hip_error = int(e);
      status = MUON_ERR_HIP;
    } else if (r.phase < nphases) {
      ms_total[r.phase] += ms;
      launches[r.phase] += 1;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof_records.clear();
  return status;
}

const char* muon_phase_name(int phase) {
  return (phase >= 0 && phase < MUON_NUM_PHASES) ? kPhaseNames[phase] : "?";
}

}  // extern "C"
