// C ABI of the fused chunked KL loss: argument checks, chunk planner,
// workspace cache and the chunk loop that enqueues the kernels, for the fused
// call and for the forward / recomputing-backward pair.
#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/ckl.h"
#include "launch.hpp"

using namespace ckl;

// Workspace of ckl_fwd_bwd_noalloc, for callers that cannot allocate device
// memory.  Each GPU the library runs on holds its own copy of this array until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: kernels get the address that hipGetSymbolAddress returns
// for the current device (scratch_ptr below).
static __device__ __align__(256) char scratch[CKL_NOALLOC_MAX_BYTES];

namespace {

constexpr uint64_t kScratchBytes = CKL_NOALLOC_MAX_BYTES;

constexpr uint64_t kDefaultBudget = 6ull << 30;
constexpr int64_t kRowStep = 256;
// Rows per chunk at most: keeps every grid dimension and tile count of a
// chunk's launches far inside 32 bits.
constexpr int64_t kMaxChunk = (int64_t)1 << 20;

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
inline int64_t roundup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Which call a chunk loop serves: the fused forward + backward, the forward
// alone (loss and log-normalisers), or the backward that recomputes the logits.
enum Pass : int { PASS_FUSED = CKL_PASS_FUSED, PASS_FWD = CKL_PASS_FWD, PASS_BWD = CKL_PASS_BWD };

// Device workspace of one call with chunks of C rows.
struct Layout {
  int64_t C = 0;
  int64_t pblk = 0;     // elements between tile rows of the exp / gradient tiles
  int n_slices = 0;     // (max, sum exp) pairs per row
  int splits = 0;       // k-splits of the dH contraction
  int64_t cpad = 0;     // rows of the id tables (C rounded up to 256)
  uint64_t w_off = 0, p_off = 0, part_off = 0, scat_off = 0, slab_off = 0, kl_off = 0, lse_off = 0, scal_off = 0,
           hc_off = 0, idc_off = 0, tlc_off = 0, vidx_off = 0, pos_off = 0, bits_off = 0, pre_off = 0, rank_off = 0,
           zs_off = 0, total = 0;
};

Layout make_layout(Pass pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t C, size_t esz) {
  Layout L;
  L.C = C;
  L.pblk = tile_row_stride(V);
  L.n_slices = (int)((V + 127) / 128);
  L.splits = pass == PASS_FWD ? 0 : dh_splits(esz == 2 ? DT_BF16 : DT_F32, C, d, V);
  const int64_t tile_rows = (C + 63) / 64;
  uint64_t off = 0;
  L.w_off = off;  // tiled copy of W
  off += align256((uint64_t)((V + 63) / 64) * tile_row_stride(d) * esz);
  L.p_off = off;  // the forward alone keeps no exp values
  if (pass != PASS_FWD) off += align256((uint64_t)tile_rows * L.pblk * esz);
  L.part_off = off;
  off += align256((uint64_t)C * L.n_slices * 8);
  L.scat_off = off;
  off += align256((uint64_t)C * K * 4);
  L.slab_off = off;
  off += align256((uint64_t)L.splits * C * d * 4);
  L.kl_off = off;
  off += align256((uint64_t)N * 4);
  L.lse_off = off;
  off += align256((uint64_t)N * 4);
  L.scal_off = off;
  off += 256;
  // compacted chunk (calls with a mask): valid rows of H, ids and teacher
  // logits, and the index maps
  L.hc_off = off;
  off += align256((uint64_t)C * d * esz);
  L.idc_off = off;
  off += align256((uint64_t)C * K * 4);
  L.tlc_off = off;
  off += align256((uint64_t)C * K * 4);
  L.vidx_off = off;
  off += align256((uint64_t)C * 4);
  L.pos_off = off;
  off += align256((uint64_t)C * 4);
  // id tables of the chunk's cached ids: per (row, slice) a 128-bit mask and
  // a uint16 count, per cached id its rank, and the exact logits by rank
  L.cpad = roundup(C, 256);
  L.bits_off = off;
  off += align256((uint64_t)id_table_pairs(V) * L.cpad * 32);
  L.pre_off = off;
  off += align256((uint64_t)id_table_pairs(V) * L.cpad * 4);
  L.rank_off = off;
  off += align256((uint64_t)C * K * 4);
  L.zs_off = off;
  off += align256((uint64_t)C * K * 4);
  L.total = off;
  return L;
}

uint64_t budget_from_env(uint64_t b) {
  if (b) return b;
  const char* e = std::getenv("CKL_WORKSPACE_BYTES");
  if (e && *e) {
    char* end = nullptr;
    unsigned long long v = std::strtoull(e, &end, 10);
    if (end != e && v > 0) return (uint64_t)v;
  }
  return kDefaultBudget;
}

int plan_impl(Pass pass, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, uint64_t budget, size_t esz,
              Layout* out) {
  if (N < 0 || d <= 0 || V <= 0 || K <= 0 || chunk < 0) return CKL_EINVAL;
  if (K > V) return CKL_EINVAL;
  if (d % 8 != 0 || K > kMaxK) return CKL_EUNSUPPORTED;
  if (V > (int64_t)1 << 26 || N > (int64_t)1 << 31 || d > (int64_t)1 << 20) return CKL_EUNSUPPORTED;
  if (N == 0) {  // an empty batch: no chunk, no workspace
    *out = Layout{};
    return CKL_OK;
  }
  budget = budget_from_env(budget);
  if (chunk > 0) {
    const int64_t C = chunk < N ? chunk : N;
    if (C > kMaxChunk) return CKL_EUNSUPPORTED;
    Layout L = make_layout(pass, N, d, V, K, C, esz);
    if (L.total > budget) return CKL_EBUDGET;
    *out = L;
    return CKL_OK;
  }
  // largest fitting multiple of 256 rows (or N itself when smaller)
  int64_t cmax = 0;
  if (N <= kRowStep) {
    if (make_layout(pass, N, d, V, K, N, esz).total <= budget) cmax = N;
  } else {
    int64_t lo = 1, hi = roundup(N < kMaxChunk ? N : kMaxChunk, kRowStep) / kRowStep;  // in units of 256 rows
    if (make_layout(pass, N, d, V, K, kRowStep, esz).total > budget) return CKL_EBUDGET;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (make_layout(pass, N, d, V, K, mid * kRowStep, esz).total <= budget)
        lo = mid;
      else
        hi = mid - 1;
    }
    cmax = lo * kRowStep;
    if (cmax > N) cmax = N;
  }
  if (cmax == 0) return CKL_EBUDGET;
  // even out: same number of chunks, the smallest 256-multiple that covers N
  const int64_t nch = (N + cmax - 1) / cmax;
  int64_t C = roundup((N + nch - 1) / nch, kRowStep);
  if (C > cmax) C = cmax;
  if (C > N) C = N;
  // The dH split count, and with it the slab bytes, depends on the chunk, so
  // the workspace is not monotonic in C: the search above only guarantees a
  // fitting multiple of 256 below the one it returns.  Step down until the
  // chunk really fits.
  for (int64_t c = C; c > 0; c = (c % kRowStep) ? c - c % kRowStep : c - kRowStep) {
    const Layout L = make_layout(pass, N, d, V, K, c, esz);
    if (L.total <= budget) {
      *out = L;
      return CKL_OK;
    }
  }
  return CKL_EBUDGET;
}

// ------------------------------------------------------------------ workspace cache
struct WsKey {
  int dev;
  hipStream_t stream;
  bool operator<(const WsKey& o) const { return dev != o.dev ? dev < o.dev : stream < o.stream; }
};
struct WsBuf {
  void* ptr = nullptr;
  uint64_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<WsKey, WsBuf> g_ws;

int get_workspace(int dev, hipStream_t s, uint64_t bytes, void** ptr) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsBuf& b = g_ws[WsKey{dev, s}];
  if (b.bytes >= bytes) {
    *ptr = b.ptr;
    return CKL_OK;
  }
  if (b.ptr) {
    // the previous call on this stream may still be using the old buffer
    if (hipStreamSynchronize(s) != hipSuccess) return CKL_EHIP;
    if (hipFree(b.ptr) != hipSuccess) return CKL_EHIP;
    b.ptr = nullptr;
    b.bytes = 0;
  }
  const char* fail = std::getenv("CKL_TEST_FAIL_ALLOC");
  if (fail && fail[0] == '1') return CKL_ENOMEM;
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return CKL_ENOMEM;
  }
  b.ptr = p;
  b.bytes = bytes;
  *ptr = p;
  return CKL_OK;
}

// ------------------------------------------------------------------ fixed scratch
// Address of this device's copy of `scratch` (defined at file scope above),
// taken once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scr_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return CKL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scr_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return CKL_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CKL_OK;
}

// ------------------------------------------------------------------ tracing
// CKL_TRACE=1: roctx ranges around each loss call and around each chunk's
// launches (host enqueue time; `rocprofv3 --marker-trace` records them next to
// the kernels).  The roctx library is opened at run time, so the library has
// no link-time dependency on the profiler; without it the ranges are skipped.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
  bool tried = false;
};
Roctx g_roctx;
std::mutex g_roctx_mu;

bool trace_requested() {
  const char* e = std::getenv("CKL_TRACE");
  return e && e[0] == '1';
}

const Roctx* roctx_api() {
  std::lock_guard<std::mutex> lk(g_roctx_mu);
  if (!g_roctx.tried) {
    g_roctx.tried = true;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (h) {
      g_roctx.push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
      g_roctx.pop = (int (*)())dlsym(h, "roctxRangePop");
      if (!g_roctx.push || !g_roctx.pop) g_roctx.push = nullptr;
    }
  }
  return g_roctx.push ? &g_roctx : nullptr;
}

struct TraceRange {
  const Roctx* api = nullptr;
  explicit TraceRange(const char* fmt, ...) __attribute__((format(printf, 2, 3))) {
    if (!trace_requested()) return;
    api = roctx_api();
    if (!api) return;
    char buf[192];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    api->push(buf);
  }
  ~TraceRange() {
    if (api) api->pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

// ------------------------------------------------------------------ timing
enum Kind { T_LOGITS = 0, T_ROWS, T_DH, T_DHRED, T_DW, T_OTHER, T_TOPK, T_KINDS };
struct TimingState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  std::vector<std::pair<int, int>> recs;  // (kind, pool index)
};
TimingState g_tm;

struct Timed {
  int idx = -1;
  hipStream_t s;
  Timed(int kind, hipStream_t st, bool enabled = true) : s(st) {
    if (!g_tm.on || !enabled) return;
    const int i = (int)g_tm.recs.size();
    if (i >= (int)g_tm.pool.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) return;
      g_tm.pool.push_back({a, b});
    }
    g_tm.recs.push_back({kind, i});
    idx = i;
    (void)hipEventRecord(g_tm.pool[i].first, s);
  }
  ~Timed() {
    if (idx >= 0) (void)hipEventRecord(g_tm.pool[idx].second, s);
  }
};

#define CKL_TRY(expr)                     \
  do {                                    \
    hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return CKL_EHIP; \
  } while (0)

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool debug_checks() {
  const char* e = std::getenv("CKL_DEBUG");
  return e && e[0] == '1';
}

// One call of any pass.  Inputs common to all: H, W, ids, tlogit, mask.
//   PASS_FUSED: out_loss, dH, dW (+ optional row_kl, row_lse)
//   PASS_FWD:   out_loss, row_lse (+ optional row_kl); no exp values are kept
//   PASS_BWD:   lse_in (the forward's row_lse), optional gscale; dH, dW; the
//               logits epilogue writes the gradient, so no dense pass runs
// With fixed_ws set, the call runs in the fixed scratch array of this device
// (budget kScratchBytes) and allocates nothing: no workspace cache, no timing
// events.
int run_impl(Pass pass, Dtype dt, const void* H, const void* W, const int32_t* ids, const float* tlogit,
             const uint8_t* mask, const float* lse_in, const float* gscale, int64_t N, int64_t d, int64_t V,
             int64_t K, int64_t chunk, float* out_loss, void* dH, float* dW, float* row_kl, float* row_lse,
             hipStream_t stream, bool fixed_ws = false) {
  const bool want_loss = pass != PASS_BWD, want_grad = pass != PASS_FWD;
  if (N == 0) {
    // An empty batch reads no row (its row arrays may be null) and has no
    // valid position: the loss is 0 and dW is 0.
    if (!W || (want_loss && !out_loss) || (want_grad && !dW)) return CKL_EINVAL;
    if (!aligned(W, 16) || !aligned(dW, 16) || !aligned(out_loss, 4)) return CKL_EINVAL;
    Layout L;
    const int st = plan_impl(pass, 0, d, V, K, chunk, 0, dt == DT_BF16 ? 2 : 4, &L);
    if (st != CKL_OK) return st;
    if (want_loss) CKL_TRY(launch_fill_f32(out_loss, 1, 0.f, stream));
    if (want_grad) CKL_TRY(launch_fill_f32(dW, V * d, 0.f, stream));
    return CKL_OK;
  }
  if (!H || !W || !ids || !tlogit) return CKL_EINVAL;
  if (want_loss && !out_loss) return CKL_EINVAL;
  if (want_grad && (!dH || !dW)) return CKL_EINVAL;
  if (pass == PASS_FWD && !row_lse) return CKL_EINVAL;
  if (pass == PASS_BWD && !lse_in) return CKL_EINVAL;
  if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16)) return CKL_EINVAL;
  if (!aligned(ids, 4) || !aligned(tlogit, 4) || !aligned(out_loss, 4)) return CKL_EINVAL;
  if (!aligned(row_kl, 4) || !aligned(row_lse, 4) || !aligned(lse_in, 4) || !aligned(gscale, 4)) return CKL_EINVAL;
  const size_t esz = dt == DT_BF16 ? 2 : 4;
  Layout L;
  int st = plan_impl(pass, N, d, V, K, chunk, fixed_ws ? kScratchBytes : 0, esz, &L);
  if (st != CKL_OK) return st;
  if ((N + L.C - 1) / L.C > (int64_t)1 << 24) return CKL_EUNSUPPORTED;

  int dev = 0;
  CKL_TRY(hipGetDevice(&dev));
  void* ws = nullptr;
  st = fixed_ws ? scratch_ptr(dev, &ws) : get_workspace(dev, stream, L.total, &ws);
  if (st != CKL_OK) return st;
  const bool tm = !fixed_ws;
  static const char* const kPassName[] = {"ckl fused", "ckl forward", "ckl backward"};
  TraceRange call_range("%s N=%lld d=%lld V=%lld K=%lld chunk=%lld%s%s", kPassName[pass], (long long)N, (long long)d,
                        (long long)V, (long long)K, (long long)L.C, mask ? " masked" : "", fixed_ws ? " noalloc" : "");
  char* base = (char*)ws;
  void* Wt = base + L.w_off;
  void* P = pass == PASS_FWD ? nullptr : base + L.p_off;
  float2* part = (float2*)(base + L.part_off);
  float* scat = (float*)(base + L.scat_off);
  float* slab = (float*)(base + L.slab_off);
  float* kl = row_kl ? row_kl : (float*)(base + L.kl_off);
  float* lse = row_lse ? row_lse : (float*)(base + L.lse_off);
  void* scal = base + L.scal_off;
  // with a mask, every chunk is compacted to its valid rows; their count lives
  // in the scalar block, after the valid count and scale
  int* live = mask ? (int*)((char*)scal + 64) : nullptr;
  void* Hcc = base + L.hc_off;
  int32_t* idc = (int32_t*)(base + L.idc_off);
  float* tlc = (float*)(base + L.tlc_off);
  int* vidx = (int*)(base + L.vidx_off);
  int* pos = (int*)(base + L.pos_off);
  IdTables tab{};
  tab.bits = base + L.bits_off;
  tab.pre = base + L.pre_off;
  tab.cpad = L.cpad;
  tab.rank = (const int32_t*)(base + L.rank_off);
  tab.zs = (float*)(base + L.zs_off);
  tab.K = (int)K;
  unsigned* err = (unsigned*)((char*)scal + kErrOffset);

  {
    Timed t(T_OTHER, stream, tm);
    CKL_TRY(launch_mask_count(mask, N, scal, stream));
    CKL_TRY(launch_tile_copy(dt, W, V, d, Wt, stream));
  }
  for (int64_t r0 = 0; r0 < N; r0 += L.C) {
    const int64_t rows = (N - r0) < L.C ? (N - r0) : L.C;
    TraceRange chunk_range("chunk %lld: rows %lld-%lld", (long long)(r0 / L.C), (long long)r0,
                           (long long)(r0 + rows - 1));
    const void* Hc = (const char*)H + (size_t)r0 * d * esz;
    const int32_t* ids_c = ids + r0 * K;
    const float* tl_c = tlogit + r0 * K;
    float* lse_c = pass == PASS_BWD ? nullptr : lse + r0;
    if (live) {
      Timed t(T_OTHER, stream, tm);
      CKL_TRY(launch_compact(dt, mask + r0, rows, L.C, Hc, d, ids_c, tl_c, (int)K, vidx, pos, live, kl + r0, lse_c,
                             Hcc, idc, tlc, stream));
      Hc = Hcc;
      ids_c = idc;
      tl_c = tlc;
    }
    {
      Timed t(T_ROWS, stream, tm);
      CKL_TRY(launch_id_tables(ids_c, (int)K, rows, V, live, base + L.bits_off, base + L.pre_off, L.cpad,
                               (int32_t*)(base + L.rank_off), err, stream));
    }
    // The recomputing backward knows the log-normalisers before the logits:
    // their epilogue stores the gradient's dense part, and no dense pass runs.
    GradTerms gt{};
    if (pass == PASS_BWD) {
      gt.lse = lse_in + r0;
      gt.rowmap = live ? vidx : nullptr;
      gt.scale = (const float*)((const char*)scal + kScaleOffset);
      gt.gscale = gscale;
    }
    {
      Timed t(T_LOGITS, stream, tm);
      CKL_TRY(launch_logits(dt, Wt, Hc, V, d, rows, P, L.pblk, part, L.n_slices, &tab,
                            pass == PASS_BWD ? &gt : nullptr, live, stream));
    }
    {
      RowArgs a{};
      a.P = P;
      a.pblk = L.pblk;
      a.part = part;
      a.n_slices = L.n_slices;
      a.ids = ids_c;
      a.tlogit = tl_c;
      a.mask = nullptr;  // without a mask every row counts; with one, the compacted rows all do
      a.scal = scal;
      a.V = V;
      a.K = (int)K;
      a.rows = rows;
      a.scat = scat;
      a.kl_out = kl + r0;
      a.lse_out = lse_c;
      a.lse_in = pass == PASS_BWD ? lse_in + r0 : nullptr;
      a.gscale = pass == PASS_BWD ? gscale : nullptr;
      a.live = live;
      a.vidx = live ? vidx : nullptr;
      a.rank = tab.rank;
      a.zs = tab.zs;
      Timed t(T_ROWS, stream, tm);
      CKL_TRY(launch_row_stats(dt, a, stream));
      if (want_grad) {
        if (pass != PASS_BWD) CKL_TRY(launch_dense(dt, a, stream));
        CKL_TRY(launch_scatter(dt, a, stream));
      }
    }
    if (!want_grad) continue;
    int splits = dh_splits(dt, rows, d, V);
    const int64_t cap = (int64_t)L.splits * L.C / rows;  // slab capacity in splits of this chunk
    if (splits > cap) splits = dh_fit_splits(dt, V, (int)cap);
    {
      Timed t(T_DH, stream, tm);
      CKL_TRY(launch_dh(dt, P, L.pblk, Wt, V, d, rows, slab, splits, live, stream));
    }
    {
      Timed t(T_DHRED, stream, tm);
      CKL_TRY(launch_dh_reduce(dt, slab, splits, rows, d, live ? pos : nullptr, (char*)dH + (size_t)r0 * d * esz,
                               stream));
    }
    {
      Timed t(T_DW, stream, tm);
      CKL_TRY(launch_dw(dt, P, L.pblk, Hc, V, d, rows, dW, r0 > 0 ? 1 : 0, live, stream));
    }
  }
  if (want_loss) {
    Timed t(T_OTHER, stream, tm);
    CKL_TRY(launch_finalize(kl, N, scal, out_loss, stream));
  }
  // CKL_DEBUG=1: wait for the call and report cached ids outside [0, V) or
  // repeated within a row (the kernels leave them out, so nothing outside the
  // buffers was touched, but the results are not those of the definition)
  if (debug_checks()) {
    unsigned flags = 0;
    CKL_TRY(hipMemcpyAsync(&flags, err, sizeof(flags), hipMemcpyDeviceToHost, stream));
    CKL_TRY(hipStreamSynchronize(stream));
    if (flags != 0) return CKL_EINVAL;
  }
  return CKL_OK;
}

inline bool dtype_ok(int dtype) { return dtype == CKL_DTYPE_BF16 || dtype == CKL_DTYPE_F32; }
inline Dtype to_dt(int dtype) { return dtype == CKL_DTYPE_BF16 ? DT_BF16 : DT_F32; }

}  // namespace

extern "C" {

int ckl_fwd_bwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
                const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, float* out_loss,
                void* dH, float* dW, hipStream_t stream) {
  try {
    return run_impl(PASS_FUSED, DT_BF16, H, W, topk_idx, topk_logit, mask, nullptr, nullptr, N, d, V, K, chunk,
                    out_loss, dH, dW, nullptr, nullptr, stream);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_fwd_bwd_f32(const float* H, const float* W, const int32_t* topk_idx, const float* topk_logit,
                    const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                    float* out_loss, float* dH, float* dW, hipStream_t stream) {
  try {
    return run_impl(PASS_FUSED, DT_F32, H, W, topk_idx, topk_logit, mask, nullptr, nullptr, N, d, V, K, chunk,
                    out_loss, dH, dW, nullptr, nullptr, stream);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_fwd_bwd_ex(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
                   const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, float* out_loss,
                   void* dH, float* dW, float* row_kl, float* row_lse, hipStream_t stream) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  try {
    return run_impl(PASS_FUSED, to_dt(dtype), H, W, topk_idx, topk_logit, mask, nullptr, nullptr, N, d, V, K, chunk,
                    out_loss, dH, dW, row_kl, row_lse, stream);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_fwd_bwd_noalloc(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                        const float* topk_logit, const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K,
                        int64_t chunk, float* out_loss, void* dH, float* dW, float* row_kl, float* row_lse,
                        hipStream_t stream) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  try {
    return run_impl(PASS_FUSED, to_dt(dtype), H, W, topk_idx, topk_logit, mask, nullptr, nullptr, N, d, V, K, chunk,
                    out_loss, dH, dW, row_kl, row_lse, stream, true);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
            const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, float* out_loss,
            float* row_lse, float* row_kl, hipStream_t stream) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  try {
    return run_impl(PASS_FWD, to_dt(dtype), H, W, topk_idx, topk_logit, mask, nullptr, nullptr, N, d, V, K, chunk,
                    out_loss, nullptr, nullptr, row_kl, row_lse, stream);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
            const uint8_t* mask, const float* row_lse, const float* grad_loss, int64_t N, int64_t d, int64_t V,
            int64_t K, int64_t chunk, void* dH, float* dW, hipStream_t stream) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  try {
    return run_impl(PASS_BWD, to_dt(dtype), H, W, topk_idx, topk_logit, mask, row_lse, grad_loss, N, d, V, K, chunk,
                    nullptr, dH, dW, nullptr, nullptr, stream);
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_topk(int dtype, const void* logits, int64_t N, int64_t V, int64_t K, int32_t* ids_out, float* vals_out,
             hipStream_t stream) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  const size_t esz = dtype == CKL_DTYPE_BF16 ? 2 : 4;
  if (N < 0 || V <= 0 || K <= 0 || K > V) return CKL_EINVAL;
  if (N == 0) return K > kMaxK ? CKL_EUNSUPPORTED : CKL_OK;  // no rows: nothing to write
  if (!logits || !ids_out || !vals_out) return CKL_EINVAL;
  if (!aligned(logits, esz) || !aligned(ids_out, 4) || !aligned(vals_out, 4)) return CKL_EINVAL;
  if (K > kMaxK || V > 0x7FFFFFFFll || N > (int64_t)(0xFFFFFFFFull / 512)) return CKL_EUNSUPPORTED;
  try {
    Timed t(T_TOPK, stream);
    CKL_TRY(launch_topk(to_dt(dtype), logits, N, V, K, ids_out, vals_out, stream));
    return CKL_OK;
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_plan_pass(int pass, int64_t N, int64_t d, int64_t V, int64_t K, int dtype, int64_t chunk,
                  uint64_t budget_bytes, int64_t* chunk_out, uint64_t* workspace_bytes_out) {
  if (!dtype_ok(dtype)) return CKL_EINVAL;
  if (pass != CKL_PASS_FUSED && pass != CKL_PASS_FWD && pass != CKL_PASS_BWD) return CKL_EINVAL;
  try {
    Layout L;
    const int st = plan_impl((Pass)pass, N, d, V, K, chunk, budget_bytes, dtype == CKL_DTYPE_BF16 ? 2 : 4, &L);
    if (st != CKL_OK) return st;
    if (chunk_out) *chunk_out = L.C;
    if (workspace_bytes_out) *workspace_bytes_out = L.total;
    return CKL_OK;
  } catch (...) {
    return CKL_EINVAL;
  }
}

int ckl_plan(int64_t N, int64_t d, int64_t V, int64_t K, int dtype, uint64_t budget_bytes, int64_t* chunk_out,
             uint64_t* workspace_bytes_out) {
  return ckl_plan_pass(CKL_PASS_FUSED, N, d, V, K, dtype, 0, budget_bytes, chunk_out, workspace_bytes_out);
}

void ckl_release_workspace(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(kv.first.dev);
      (void)hipDeviceSynchronize();
      (void)hipFree(kv.second.ptr);
      (void)hipSetDevice(cur);
    }
  }
  g_ws.clear();
}

uint64_t ckl_workspace_bytes_held(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  uint64_t t = 0;
  for (auto& kv : g_ws) t += kv.second.bytes;
  return t;
}

const char* ckl_strerror(int status) {
  switch (status) {
    case CKL_OK: return "ok";
    case CKL_EINVAL: return "invalid argument";
    case CKL_ENOMEM: return "device workspace allocation failed";
    case CKL_EBUDGET: return "no chunk size fits the workspace budget";
    case CKL_EHIP: return "HIP runtime error";
    case CKL_EUNSUPPORTED: return "unsupported shape";
    default: return "unknown status";
  }
}

int ckl_debug_rows(const float* Z, const int32_t* idx, const float* tlogit, const uint8_t* mask, int64_t R,
                   int64_t V, int64_t K, float scale, int g_bf16, float* zg_out, int32_t* scatter_ids_out,
                   void* G_out, float* kl_out, float* lse_out, hipStream_t stream) {
  try {
    if (!Z || !idx || !tlogit || !zg_out || !scatter_ids_out || !G_out || !kl_out || !lse_out) return CKL_EINVAL;
    if (R <= 0 || V <= 0 || K <= 0 || K > V) return CKL_EINVAL;
    if (K > kMaxK) return CKL_EUNSUPPORTED;
    if (R > (int64_t)1 << 20 || V > (int64_t)1 << 26) return CKL_EUNSUPPORTED;
    const Dtype gdt = g_bf16 ? DT_BF16 : DT_F32;
    const size_t esz = g_bf16 ? 2 : 4;
    const int64_t pblk = tile_row_stride(V);
    const int n_slices = (int)((V + 127) / 128);
    const int64_t cpad = roundup(R, 256);
    const uint64_t pb = align256((uint64_t)((R + 63) / 64) * pblk * esz);
    const uint64_t qb = align256((uint64_t)R * n_slices * 8);
    const uint64_t sb = align256((uint64_t)R * K * 4);
    const uint64_t bb = align256((uint64_t)id_table_pairs(V) * cpad * 32);
    const uint64_t cb = align256((uint64_t)id_table_pairs(V) * cpad * 4);
    int dev = 0;
    CKL_TRY(hipGetDevice(&dev));
    void* ws = nullptr;
    int st = get_workspace(dev, stream, pb + qb + 3 * sb + bb + cb, &ws);
    if (st != CKL_OK) return st;
    char* wsb = (char*)ws;
    void* P = wsb;
    float2* part = (float2*)(wsb + pb);
    float* scat = (float*)(wsb + pb + qb);
    int32_t* rank = (int32_t*)(wsb + pb + qb + sb);
    float* zs = (float*)(wsb + pb + qb + 2 * sb);
    void* bits = wsb + pb + qb + 3 * sb;
    void* pre = wsb + pb + qb + 3 * sb + bb;
    // the id tables the chunk loop builds, and the logits at the cached ids
    // copied from Z as the logits contraction copies them from its accumulators
    CKL_TRY(launch_id_tables(idx, (int)K, R, V, nullptr, bits, pre, cpad, rank, nullptr, stream));
    CKL_TRY(launch_zs_from_z(Z, V, idx, rank, R, (int)K, zs, stream));
    CKL_TRY(launch_partials_from_z(gdt, Z, V, R, V, part, n_slices, P, pblk, stream));
    RowArgs a{};
    a.P = P;
    a.pblk = pblk;
    a.part = part;
    a.n_slices = n_slices;
    a.ids = idx;
    a.tlogit = tlogit;
    a.mask = mask;
    a.scal = nullptr;
    a.scale_value = scale;
    a.V = V;
    a.K = (int)K;
    a.rows = R;
    a.scat = scat;
    a.kl_out = kl_out;
    a.lse_out = lse_out;
    a.rank = rank;
    a.zs = zs;
    a.zg_dbg = zg_out;
    a.sid_dbg = scatter_ids_out;
    CKL_TRY(launch_row_stats(gdt, a, stream));
    CKL_TRY(launch_dense(gdt, a, stream));
    CKL_TRY(launch_scatter(gdt, a, stream));
    CKL_TRY(launch_untile(gdt, P, pblk, R, V, G_out, stream));
    CKL_TRY(hipStreamSynchronize(stream));
    return CKL_OK;
  } catch (...) {
    return CKL_EHIP;
  }
}

int ckl_timing_enable(int on) {
  g_tm.on = on != 0;
  g_tm.recs.clear();
  return CKL_OK;
}

int ckl_timing_query(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= T_KINDS || !total_ms || !launches) return CKL_EINVAL;
  double t = 0.0;
  int64_t n = 0;
  for (auto& r : g_tm.recs) {
    if (r.first != kind) continue;
    auto& ev = g_tm.pool[r.second];
    if (hipEventSynchronize(ev.second) != hipSuccess) return CKL_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess) return CKL_EHIP;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return CKL_OK;
}

}  // extern "C"
