// Host runtime of the GCA library: the C ABI of include/gca.h.
//
// Every device call validates against the host planner first (no device
// sync), enqueues its kernels on the caller's stream, and only then commits
// the planner state, so a rejected call changes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gca.h"
#include "gca_kernels.h"
#include "gca_plan.h"

namespace {

thread_local std::string g_last_error;

int hip_fail(hipError_t e, const char* what) {
  char buf[256];
  std::snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  g_last_error = buf;
  return GCA_ERR_HIP;
}

#define GCA_HIP(call, what)                 \
  do {                                      \
    hipError_t e_ = (call);                 \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15) == 0; }

constexpr int kMaxSplits = 16;

// Per-call scratch of gca_step_static (prepared queries, split partials): a
// fixed array in device memory, one copy per GPU the library runs on, held
// until the process ends.  Host code never uses the name `scratch` as an
// address: each device's copy is looked up once (hipGetSymbolAddress, with
// that device current) and passed to the kernels as a plain pointer.
constexpr size_t kStaticScratchBytes = (size_t)GCA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // by device index; null until looked up

// This device's copy of `scratch` (the device must be current).
hipError_t static_scratch(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0) return hipErrorInvalidDevice;
  if ((size_t)device >= g_scratch_ptr.size()) g_scratch_ptr.resize(device + 1, nullptr);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Where one attention call keeps its scratch: the prepared queries and the
// split-KV partials.
struct Work {
  void* qrot;
  float* o_part;
  float* lse_part;
};

struct ProfRec {
  int kind;
  hipEvent_t a, b;
};

}  // namespace

struct gca_cache {
  gca::Geometry g;
  gca::Planner plan;
  int device = 0;
  int num_cu = 256;
  size_t esize = 2;
  void* kpool = nullptr;
  void* vpool = nullptr;
  int32_t* ring = nullptr;
  int32_t* ring_init = nullptr;  // device copy of a caller order, or null
  void* raw_k = nullptr;  // windowed inference: raw K/V of the last keyframes, [overlap][T][H][D]
  void* raw_v = nullptr;
  int32_t* rec_pages = nullptr;
  int32_t* traj_pages = nullptr;
  int32_t* compact = nullptr;
  int32_t* sel_page = nullptr;
  int32_t* sel_len = nullptr;
  double2* rope_t = nullptr;
  double2* rope_h = nullptr;
  double2* rope_w = nullptr;
  gca::RopeTabs tabs{};
  float* o_part = nullptr;
  float* lse_part = nullptr;
  void* qrot = nullptr;  // prepared (rotated) queries of the current attention call
  void* static_scratch = nullptr;  // this device's copy of `scratch` (gca_step_static)
  // tiles of a first-dispatched split per tile of a second-dispatched one
  float split_ratio = 1.7f;
  bool sel_valid = false;
  int sel_n = 0;
  int64_t sel_ctx = 0;
  // profiling
  int prof_cap = 0;
  uint32_t prof_kinds = 0;
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> prof_pool;

  explicit gca_cache(const gca::Geometry& geo) : g(geo), plan(geo) {}
};

namespace {

void free_all(gca_cache* c) {
  void* ptrs[] = {c->kpool, c->vpool, c->ring, c->ring_init, c->raw_k, c->raw_v, c->rec_pages, c->traj_pages,
                  c->compact, c->sel_page, c->sel_len, c->rope_t, c->rope_h, c->rope_w,
                  c->o_part, c->lse_part, c->qrot};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  for (auto& r : c->prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : c->prof_pool) (void)hipEventDestroy(e);
}

template <typename T>
hipError_t dmalloc(T** p, size_t bytes) {
  return hipMalloc((void**)p, std::max<size_t>(bytes, 16));
}

// Rotary tables for the [t | h | w] split of the head dim: d_h = d_w =
// 2 * (D / 6), d_t = D - d_h - d_w; pair j of an axis block of width d turns
// by pos * theta^(-2j/d).  (cos, sin) evaluated and stored in double.
void build_rope(const gca::Geometry& g, std::vector<double2>* t, std::vector<double2>* h,
                std::vector<double2>* w, int* nt, int* nh, int* nw) {
  int dh = 2 * (g.D / 6), dw = dh, dt = g.D - dh - dw;
  *nt = dt / 2;
  *nh = dh / 2;
  *nw = dw / 2;
  auto fill = [&](std::vector<double2>* out, int64_t npos, int width) {
    int npairs = width / 2;
    out->resize((size_t)npos * npairs);
    for (int64_t p = 0; p < npos; ++p)
      for (int j = 0; j < npairs; ++j) {
        double ang = (double)p * std::pow((double)g.theta, -(double)(2 * j) / width);
        (*out)[(size_t)p * npairs + j] = make_double2(std::cos(ang), std::sin(ang));
      }
  };
  fill(t, g.rope_pos, dt);
  fill(h, g.grid_h, dh);
  fill(w, g.grid_w, dw);
}

void prof_begin(gca_cache* c, int kind, hipStream_t s, ProfRec* r) {
  r->kind = -1;
  if (c->prof_cap <= 0 || !(c->prof_kinds & (1u << kind)) || (int)c->prof.size() >= c->prof_cap ||
      c->prof_pool.size() < 2)
    return;
  r->kind = kind;
  r->b = c->prof_pool.back();
  c->prof_pool.pop_back();
  r->a = c->prof_pool.back();
  c->prof_pool.pop_back();
  (void)hipEventRecord(r->a, s);
}

void prof_end(gca_cache* c, hipStream_t s, ProfRec* r) {
  if (r->kind < 0) return;
  (void)hipEventRecord(r->b, s);
  c->prof.push_back(*r);
}

struct Prof {
  gca_cache* c;
  hipStream_t s;
  ProfRec r;
  Prof(gca_cache* c_, int kind, hipStream_t s_) : c(c_), s(s_) { prof_begin(c, kind, s, &r); }
  ~Prof() { prof_end(c, s, &r); }
};

gca::SelectArgs select_args(gca_cache* c, const gca::SelectStep& st) {
  gca::SelectArgs a;
  a.rec_pages = c->rec_pages;
  a.traj_pages = c->traj_pages;
  a.sel_page = c->sel_page;
  a.sel_len = c->sel_len;
  a.traj_len = st.traj_len;
  a.ppf = c->g.ppf;
  a.P = c->g.P;
  a.last_len = c->g.last_len;
  a.A = c->g.A;
  a.Wr = c->g.Wr;
  a.n_anchor = st.n_anchor;
  a.win_first = st.win_first;
  a.win_count = st.win_count;
  a.n_traj_pages = st.n_traj_pages;
  a.n_sel = st.n_sel;
  a.n_write = gca::padded_sel(st.n_sel, c->g.P);
  a.zero_page = c->g.N;
  a.ring = c->ring;
  a.N = c->g.N;
  a.newest_pos = -1;  // all page ids are in the page tables
  a.traj_known = st.n_traj_pages;
  a.traj_pos = 0;
  return a;
}

size_t frame_bytes(const gca_cache* c) { return (size_t)c->g.T * c->g.H * c->g.D * c->esize; }

gca::AppendArgs append_args(gca_cache* c, const gca::AppendStep& st, const void* k, const void* v) {
  gca::AppendArgs a;
  a.k = k;
  a.v = v;
  a.raw_k = st.raw_slot >= 0 ? (char*)c->raw_k + st.raw_slot * frame_bytes(c) : nullptr;
  a.raw_v = st.raw_slot >= 0 ? (char*)c->raw_v + st.raw_slot * frame_bytes(c) : nullptr;
  a.kpool = c->kpool;
  a.vpool = c->vpool;
  a.ring = c->ring;
  a.rec_pages = c->rec_pages;
  a.ring_pos = st.ring_pos % c->g.N;
  a.tpos = st.rope;
  a.N = c->g.N;
  a.slot = st.slot;
  a.ppf = c->g.ppf;
  a.T = c->g.T;
  a.H = c->g.H;
  a.P = c->g.P;
  a.rope = c->g.rope;
  a.tabs = c->tabs;
  return a;
}

gca::EvictArgs evict_args(gca_cache* c, const gca::EvictStep& st) {
  gca::EvictArgs a;
  a.kpool = c->kpool;
  a.vpool = c->vpool;
  a.ring = c->ring;
  a.rec_pages = c->rec_pages;
  a.traj_pages = c->traj_pages;
  a.compact = c->compact;
  a.traj_len = st.traj_len;
  a.ring_head = st.ring_head % c->g.N;
  a.ring_tail = st.ring_tail % c->g.N;
  a.N = c->g.N;
  a.slot = st.slot;
  a.ppf = c->g.ppf;
  a.n_traj_pages = st.n_traj_pages;
  a.new_pages = st.new_pages;
  a.C = c->g.C;
  a.H = c->g.H;
  a.P = c->g.P;
  return a;
}

// The attention's queries: rotated when rope = 1 (rounded once to the cache
// dtype) at temporal position tpos (the frame index, window-relative in
// windowed inference), else copied, into the query workspace.
gca::RopeArgs query_args(gca_cache* c, int64_t tpos, const void* q, void* dst, int nf = 1) {
  gca::RopeArgs ra;
  ra.x = q;
  ra.y = dst;
  ra.tpos = tpos;
  ra.nf = nf;
  ra.T = c->g.T;
  ra.H = c->g.H;
  ra.rotate = c->g.rope;
  ra.tabs = c->tabs;
  return ra;
}

// Split count of an attention call over n_sel gather entries for nf frames of
// queries: about two workgroups per compute unit, at most kMaxSplits / nf
// (the cache's split workspace holds kMaxSplits partials of one frame's rows),
// at least two tiles per split.
struct Split {
  int n_tiles, qtiles, S, tps;
};
Split split_of(const gca_cache* c, int n_sel, int nf) {
  const gca::Geometry& g = c->g;
  Split sp;
  const int ept = gca::kKeysPerTile / g.P;
  sp.n_tiles = (n_sel + ept - 1) / ept;
  sp.qtiles = (nf * g.T + gca::queries_per_wg(g.dtype) - 1) / gca::queries_per_wg(g.dtype);
  const int base = sp.qtiles * g.H;
  int S = (2 * c->num_cu + base - 1) / base;
  S = std::min(S, kMaxSplits / nf);
  S = std::min(S, std::max(1, sp.n_tiles / 2));
  S = std::max(S, 1);
  sp.tps = (sp.n_tiles + S - 1) / S;
  sp.S = (sp.n_tiles + sp.tps - 1) / sp.tps;
  return sp;
}

// Scratch bytes of one attention call: the prepared queries of nf frames and,
// when split, the partials.
size_t work_bytes(const gca_cache* c, const Split& sp, int nf) {
  const gca::Geometry& g = c->g;
  const size_t rows = (size_t)nf * g.T * g.H;
  size_t b = align256(rows * g.D * c->esize);
  if (sp.S > 1) b += align256(sizeof(float) * rows * g.D * sp.S) + align256(sizeof(float) * rows * sp.S);
  return b;
}

// The scratch of one call laid out in the static array: queries, partials,
// partial LSEs, each 256-byte aligned.
Work static_work(const gca_cache* c, const Split& sp, int nf) {
  const gca::Geometry& g = c->g;
  const size_t rows = (size_t)nf * g.T * g.H;
  char* p = (char*)c->static_scratch;
  Work w;
  w.qrot = p;
  p += align256(rows * g.D * c->esize);
  w.o_part = (float*)p;
  p += align256(sizeof(float) * rows * g.D * std::max(sp.S, 1));
  w.lse_part = (float*)p;
  return w;
}

Work own_work(const gca_cache* c) { return Work{c->qrot, c->o_part, c->lse_part}; }

// Attention over the gather list already built for `st` (queries of nf
// stacked frames already prepared into w.qrot by query_args), then the split
// merge.
int attend_launch(gca_cache* c, int64_t frame_idx, void* out, float* lse, const gca::SelectStep& st,
                  hipStream_t s, const Work& w, int nf = 1) {
  const gca::Geometry& g = c->g;
  const int Tq = nf * g.T;
  const Split sp = split_of(c, st.n_sel, nf);
  const int n_tiles = sp.n_tiles, S = sp.S;
  gca::AttnArgs a;
  a.q = w.qrot;
  a.qk_scale = (float)((double)g.scale * 1.4426950408889634);
  a.kpool = c->kpool;
  a.vpool = c->vpool;
  a.sel_page = c->sel_page;
  a.sel_len = c->sel_len;
  a.o_part = w.o_part;
  a.lse_part = w.lse_part;
  a.out = out;
  a.lse = lse;
  a.frame = frame_idx;
  a.Tq = Tq;
  a.H = g.H;
  a.P = g.P;
  a.n_sel = st.n_sel;
  a.n_tiles = n_tiles;
  a.tiles_per_split = sp.tps;
  a.S = S;
  a.n_qtiles = sp.qtiles;
  a.n_units = g.H * S;
  a.out_bf16 = g.out_dtype == GCA_BF16;
  a.head_major = g.H % gca::kNumXcd == 0;
  a.t_odd = 0;
  if (a.head_major && S % 2 == 0 && c->split_ratio > 1.0f) {
    // pairs of splits: the first dispatched (even) split takes ratio / (1 + ratio)
    const int pair = (2 * n_tiles + S - 1) / S;
    int te = (int)((float)pair * c->split_ratio / (1.0f + c->split_ratio) + 0.5f);
    te = std::min(std::max(te, 1), pair);
    if (pair - te >= 1) {
      a.tiles_per_split = te;
      a.t_odd = pair - te;
    }
  }
  {
    Prof p(c, 3, s);
    GCA_HIP(gca::launch_attn(g.dtype, a, s), "attention kernel launch");
  }
  if (S > 1) {
    gca::MergeArgs m;
    m.o_part = w.o_part;
    m.lse_part = w.lse_part;
    m.out = out;
    m.lse = lse;
    m.rows = Tq * g.H;
    m.S = S;
    m.out_bf16 = a.out_bf16;
    Prof p(c, 4, s);
    GCA_HIP(gca::launch_merge(m, s), "merge kernel launch");
  }
  return GCA_OK;
}

// Windowed inference: the start of the next window on the device.  The ring
// back in its initial order, then the kept keyframes appended again from
// their raw copies in one launch.
int enqueue_restart(gca_cache* c, const gca::RestartStep& r, hipStream_t s) {
  Prof p(c, 0, s);
  GCA_HIP(gca::launch_ring_init(c->ring, c->ring_init, c->g.N, s), "ring init launch");
  if (r.n == 0) return GCA_OK;
  gca::AppendBatch b{};
  b.a = append_args(c, r.step[0], nullptr, nullptr);
  b.a.raw_k = b.a.raw_v = nullptr;
  b.n = r.n;
  for (int j = 0; j < r.n; ++j) {
    const gca::AppendStep& st = r.step[j];
    b.slot[j] = st.slot;
    b.tpos[j] = st.rope;
    b.k[j] = (const char*)c->raw_k + st.raw_slot * frame_bytes(c);
    b.v[j] = (const char*)c->raw_v + st.raw_slot * frame_bytes(c);
    b.rk[j] = b.rv[j] = nullptr;
  }
  GCA_HIP(gca::launch_append_batch(c->g.dtype, b, s), "append kernel launch");
  return GCA_OK;
}

// On planner p: the restart due before appending `frame`, if any (r->n = -1
// when none).
int plan_restart(gca::Planner& p, int64_t frame, gca::RestartStep* r) {
  r->n = -1;
  if (!p.restart_due(frame)) return GCA_OK;
  int rc = p.check_restart(frame, r);
  if (rc) return rc;
  p.commit_restart(*r);
  return GCA_OK;
}

int do_select(gca_cache* c, hipStream_t s, gca::SelectStep* out) {
  gca::SelectStep st = c->plan.select();
  gca::SelectArgs a = select_args(c, st);
  {
    Prof p(c, 2, s);
    GCA_HIP(gca::launch_select(a, s), "select kernel launch");
  }
  c->sel_valid = true;
  c->sel_n = st.n_sel;
  c->sel_ctx = st.n_ctx;
  if (out) *out = st;
  return GCA_OK;
}

}  // namespace

extern "C" {

const char* gca_last_error(void) { return g_last_error.c_str(); }

int gca_cache_create(const gca_config* cfg, gca_cache** out) {
  if (!out) return GCA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  gca::Geometry g;
  int rc = gca::make_geometry(cfg, &g);
  if (rc) return rc;
  gca_cache* c = new gca_cache(g);
  auto fail = [&](hipError_t e, const char* what) {
    int r = hip_fail(e, what);
    free_all(c);
    delete c;
    return r;
  };
  hipError_t e;
  if ((e = hipGetDevice(&c->device)) != hipSuccess) return fail(e, "hipGetDevice");
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess &&
      cus > 0)
    c->num_cu = cus;
  c->esize = g.dtype == GCA_BF16 ? 2 : 4;
  // the first-dispatched workgroup of a CU issues ahead of the second, and
  // speeds up once it runs alone; sweeps of the ratio from 1.4 to 2.5 were
  // best from 2.2 on, within 1.5 % over the whole range
  c->split_ratio = g.P >= 64 ? 2.3f : 2.2f;
  size_t page_elems = (size_t)g.H * g.P * g.D;
  // pages [0, N) are handed out by the ring; page N stays zero forever and
  // pads the gather list
  size_t pool_bytes = ((size_t)g.N + 1) * page_elems * c->esize;
  size_t rows = (size_t)g.T * g.H;
  if ((e = dmalloc(&c->kpool, pool_bytes)) != hipSuccess) return fail(e, "hipMalloc K pool");
  if ((e = dmalloc(&c->vpool, pool_bytes)) != hipSuccess) return fail(e, "hipMalloc V pool");
  if ((e = dmalloc(&c->ring, sizeof(int32_t) * g.N)) != hipSuccess) return fail(e, "hipMalloc ring");
  if ((e = dmalloc(&c->rec_pages, sizeof(int32_t) * (size_t)(g.A + g.Wr) * g.ppf)) != hipSuccess)
    return fail(e, "hipMalloc records");
  if ((e = dmalloc(&c->traj_pages, sizeof(int32_t) * (size_t)g.traj_cap)) != hipSuccess)
    return fail(e, "hipMalloc trajectory");
  if ((e = dmalloc(&c->compact, sizeof(int32_t) * (size_t)g.C)) != hipSuccess)
    return fail(e, "hipMalloc compact list");
  if ((e = dmalloc(&c->sel_page, sizeof(int32_t) * ((size_t)g.sel_cap + gca::kSelPad))) != hipSuccess)
    return fail(e, "hipMalloc gather list");
  if ((e = dmalloc(&c->sel_len, sizeof(int32_t) * ((size_t)g.sel_cap + gca::kSelPad))) != hipSuccess)
    return fail(e, "hipMalloc gather list");
  if ((e = dmalloc(&c->o_part, sizeof(float) * rows * g.D * kMaxSplits)) != hipSuccess)
    return fail(e, "hipMalloc split workspace");
  if ((e = dmalloc(&c->lse_part, sizeof(float) * rows * kMaxSplits)) != hipSuccess)
    return fail(e, "hipMalloc split workspace");
  // prepared queries: one frame, or the A anchor frames of a joint call
  if ((e = dmalloc(&c->qrot, rows * g.D * c->esize * std::max(1, g.A))) != hipSuccess)
    return fail(e, "hipMalloc query workspace");
  if (g.window > 0) {
    const size_t rb = (size_t)g.overlap * rows * g.D * c->esize;
    if ((e = dmalloc(&c->raw_k, rb)) != hipSuccess) return fail(e, "hipMalloc raw keyframes");
    if ((e = dmalloc(&c->raw_v, rb)) != hipSuccess) return fail(e, "hipMalloc raw keyframes");
  }
  if ((e = hipMemset(c->kpool, 0, pool_bytes)) != hipSuccess) return fail(e, "hipMemset K pool");
  if ((e = hipMemset(c->vpool, 0, pool_bytes)) != hipSuccess) return fail(e, "hipMemset V pool");
  if (g.C) {
    if ((e = hipMemcpy(c->compact, g.compact.data(), sizeof(int32_t) * g.C, hipMemcpyHostToDevice)) !=
        hipSuccess)
      return fail(e, "upload compact list");
  }
  std::vector<int32_t> ring(g.N);
  for (int i = 0; i < g.N; ++i) ring[i] = g.ring_init.empty() ? i : g.ring_init[i];
  if (!g.ring_init.empty()) {
    if ((e = dmalloc(&c->ring_init, sizeof(int32_t) * g.N)) != hipSuccess) return fail(e, "hipMalloc ring order");
    if ((e = hipMemcpy(c->ring_init, ring.data(), sizeof(int32_t) * g.N, hipMemcpyHostToDevice)) != hipSuccess)
      return fail(e, "upload ring order");
  }
  if ((e = hipMemcpy(c->ring, ring.data(), sizeof(int32_t) * g.N, hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e, "upload ring");
  if (g.rope) {
    std::vector<double2> t, h, w;
    int nt, nh, nw;
    build_rope(g, &t, &h, &w, &nt, &nh, &nw);
    // the kernels load the cos/sin of two pairs at once (12, 10, 10 pairs for D = 64)
    if ((nt | nh | nw) & 1) return fail(hipErrorInvalidValue, "rotary split with an odd pair count");
    if ((e = dmalloc(&c->rope_t, sizeof(double2) * t.size())) != hipSuccess) return fail(e, "hipMalloc rope");
    if ((e = dmalloc(&c->rope_h, sizeof(double2) * h.size())) != hipSuccess) return fail(e, "hipMalloc rope");
    if ((e = dmalloc(&c->rope_w, sizeof(double2) * w.size())) != hipSuccess) return fail(e, "hipMalloc rope");
    if ((e = hipMemcpy(c->rope_t, t.data(), sizeof(double2) * t.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return fail(e, "upload rope");
    if ((e = hipMemcpy(c->rope_h, h.data(), sizeof(double2) * h.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return fail(e, "upload rope");
    if ((e = hipMemcpy(c->rope_w, w.data(), sizeof(double2) * w.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return fail(e, "upload rope");
    c->tabs.t = c->rope_t;
    c->tabs.h = c->rope_h;
    c->tabs.w = c->rope_w;
    c->tabs.nt = nt;
    c->tabs.nh = nh;
    c->tabs.nw = nw;
    c->tabs.num_special = g.num_special;
    c->tabs.grid_w = g.grid_w;
  }
  if ((e = static_scratch(c->device, &c->static_scratch)) != hipSuccess)
    return fail(e, "static scratch address");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e, "create sync");
  *out = c;
  return GCA_OK;
}

int gca_cache_destroy(gca_cache* c) {
  if (!c) return GCA_OK;
  (void)hipSetDevice(c->device);
  hipError_t e = hipDeviceSynchronize();
  free_all(c);
  delete c;
  return e == hipSuccess ? GCA_OK : hip_fail(e, "destroy sync");
}

int gca_cache_reset(gca_cache* c, gca_stream_t stream) {
  if (!c) return GCA_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  GCA_HIP(gca::launch_ring_init(c->ring, c->ring_init, c->g.N, s), "ring init launch");
  c->plan.reset();
  c->sel_valid = false;
  return GCA_OK;
}

int gca_append_frame(gca_cache* c, int64_t frame_idx, const void* k, const void* v, uint32_t flags,
                     gca_stream_t stream) {
  if (!c || !aligned16(k) || !aligned16(v) || (flags & ~GCA_APPEND_TEMP))
    return GCA_ERR_INVALID_ARGUMENT;
  bool temp = flags & GCA_APPEND_TEMP;
  gca::Planner p = c->plan;
  gca::RestartStep r;
  int rc = plan_restart(p, frame_idx, &r);
  if (rc) return rc;
  gca::AppendStep st;
  if ((rc = p.check_append(frame_idx, temp, &st))) return rc;
  p.commit_append(st, temp);
  hipStream_t s = (hipStream_t)stream;
  if (r.n >= 0 && (rc = enqueue_restart(c, r, s))) return rc;
  gca::AppendArgs a = append_args(c, st, k, v);
  {
    Prof pr(c, 0, s);
    GCA_HIP(gca::launch_append(c->g.dtype, a, s), "append kernel launch");
  }
  c->plan = p;
  c->sel_valid = false;
  return GCA_OK;
}

int gca_append_frames(gca_cache* c, int64_t first_frame, int32_t n_frames, const void* k, const void* v,
                      gca_stream_t stream) {
  if (!c || !aligned16(k) || !aligned16(v) || first_frame < 0 || n_frames < 1)
    return GCA_ERR_INVALID_ARGUMENT;
  if (n_frames > gca::kMaxAppendBatch) return GCA_ERR_CAPACITY;
  // every append on a copy of the planner first, as the individual calls
  // would run them; nothing is enqueued or changed unless all are valid
  gca::Planner p = c->plan;
  gca::RestartStep r;
  int rc = plan_restart(p, first_frame, &r);
  if (rc) return rc;
  gca::AppendBatch b{};
  int64_t pos0 = 0;
  const size_t fb = frame_bytes(c);
  for (int j = 0; j < n_frames; ++j) {
    gca::AppendStep st;
    // windowed inference: a batch does not cross into the next window
    if (j > 0 && p.restart_due(first_frame + j)) return GCA_ERR_SEQUENCE;
    if ((rc = p.check_append(first_frame + j, false, &st))) return rc;
    const gca::AppendArgs aj = append_args(c, st, (const char*)k + j * fb, (const char*)v + j * fb);
    if (j == 0) {
      b.a = aj;
      pos0 = st.ring_pos;
    } else if (st.ring_pos != pos0 + (int64_t)j * c->g.ppf) {
      return GCA_ERR_SEQUENCE;  // not reached: with no eviction between them the pops are consecutive
    }
    b.slot[j] = st.slot;
    b.tpos[j] = aj.tpos;
    b.k[j] = aj.k;
    b.v[j] = aj.v;
    b.rk[j] = aj.raw_k;
    b.rv[j] = aj.raw_v;
    p.commit_append(st, false);
  }
  b.n = n_frames;
  hipStream_t s = (hipStream_t)stream;
  if (r.n >= 0 && (rc = enqueue_restart(c, r, s))) return rc;
  {
    Prof pr(c, 0, s);
    GCA_HIP(gca::launch_append_batch(c->g.dtype, b, s), "append kernel launch");
  }
  c->plan = p;
  c->sel_valid = false;
  return GCA_OK;
}

int gca_evict_compact(gca_cache* c, gca_stream_t stream) {
  if (!c) return GCA_ERR_INVALID_ARGUMENT;
  std::vector<gca::EvictStep> steps;
  int rc = c->plan.check_evict(&steps);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  for (const gca::EvictStep& st : steps) {
    gca::EvictArgs a = evict_args(c, st);
    Prof p(c, 1, s);
    GCA_HIP(gca::launch_evict(c->g.dtype, a, s), "evict kernel launch");
  }
  c->plan.commit_evict(steps);
  if (!steps.empty()) c->sel_valid = false;
  return GCA_OK;
}

int gca_select(gca_cache* c, gca_stream_t stream) {
  if (!c) return GCA_ERR_INVALID_ARGUMENT;
  if (c->plan.empty()) return GCA_ERR_SEQUENCE;
  return do_select(c, (hipStream_t)stream, nullptr);
}

int gca_attend(gca_cache* c, int64_t frame_idx, const void* q, void* out, float* lse,
               gca_stream_t stream) {
  if (!c || !aligned16(q) || !aligned16(out) || (lse && ((uintptr_t)lse & 3)))
    return GCA_ERR_INVALID_ARGUMENT;
  int rc = c->plan.check_attend(frame_idx);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const gca::Geometry& g = c->g;
  gca::SelectStep st = c->plan.select();
  {
    // gather list and prepared queries from one launch
    Prof p(c, 2, s);
    GCA_HIP(gca::launch_prepare(g.dtype, select_args(c, st),
                                query_args(c, c->plan.rope_of(frame_idx), q, c->qrot), s),
            "prepare kernel launch");
  }
  c->sel_valid = true;
  c->sel_n = st.n_sel;
  c->sel_ctx = st.n_ctx;
  return attend_launch(c, frame_idx, out, lse, st, s, own_work(c));
}

int gca_attend_frames(gca_cache* c, int64_t first_frame, int32_t n_frames, const void* q, void* out,
                      float* lse, gca_stream_t stream) {
  if (!c || !aligned16(q) || !aligned16(out) || (lse && ((uintptr_t)lse & 3)) || first_frame < 0 ||
      n_frames < 1)
    return GCA_ERR_INVALID_ARGUMENT;
  if (n_frames > std::max(1, c->g.A)) return GCA_ERR_CAPACITY;
  int rc = c->plan.check_attend(first_frame + n_frames - 1);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const gca::Geometry& g = c->g;
  gca::SelectStep st = c->plan.select();
  {
    Prof p(c, 2, s);
    GCA_HIP(gca::launch_prepare(g.dtype, select_args(c, st),
                                query_args(c, c->plan.rope_of(first_frame), q, c->qrot, n_frames), s),
            "prepare kernel launch");
  }
  c->sel_valid = true;
  c->sel_n = st.n_sel;
  c->sel_ctx = st.n_ctx;
  return attend_launch(c, first_frame + n_frames - 1, out, lse, st, s, own_work(c), n_frames);
}

int gca_rollback_last_frame(gca_cache* c, int64_t frame_idx, gca_stream_t stream) {
  (void)stream;
  if (!c) return GCA_ERR_INVALID_ARGUMENT;
  int rc = c->plan.check_rollback(frame_idx);
  if (rc) return rc;
  // The popped ring slots still hold the page ids: moving the head back
  // returns them, and the frame's record slot is simply no longer live.
  c->plan.commit_rollback();
  c->sel_valid = false;
  return GCA_OK;
}

}  // extern "C"

namespace {

// One frame of the loop (gca_step), its attention scratch in the cache's own
// workspace or, with use_static, in this device's copy of `scratch`.
int step_impl(gca_cache* c, int64_t frame_idx, const void* k, const void* v, const void* q, void* out,
              float* lse, uint32_t flags, gca_stream_t stream, bool use_static) {
  if (!c || !aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) ||
      (lse && ((uintptr_t)lse & 3)) || (flags & ~GCA_STEP_KEYFRAME))
    return GCA_ERR_INVALID_ARGUMENT;
  const bool key = flags & GCA_STEP_KEYFRAME;
  const gca::Geometry& g = c->g;
  // the whole step on a copy of the planner first: nothing is enqueued or
  // changed unless every part is valid
  gca::Planner p = c->plan;
  gca::RestartStep rs;
  int rc = plan_restart(p, frame_idx, &rs);
  if (rc) return rc;
  gca::AppendStep as;
  if ((rc = p.check_append(frame_idx, !key, &as))) return rc;
  p.commit_append(as, !key);
  std::vector<gca::EvictStep> ev;
  if (key) {
    if ((rc = p.check_evict(&ev))) return rc;
    p.commit_evict(ev);
  }
  if ((rc = p.check_attend(frame_idx))) return rc;
  if (!key && (rc = p.check_rollback(frame_idx))) return rc;
  const gca::SelectStep st = p.select();
  Work w = own_work(c);
  if (use_static) {
    const Split sp = split_of(c, st.n_sel, 1);
    const size_t need = work_bytes(c, sp, 1);
    if (need > kStaticScratchBytes) {
      char buf[192];
      std::snprintf(buf, sizeof buf, "gca_step_static: the step needs %zu bytes of scratch, the static array holds %zu",
                    need, kStaticScratchBytes);
      g_last_error = buf;
      return GCA_ERR_CAPACITY;
    }
    w = static_work(c, sp, 1);
  }

  hipStream_t s = (hipStream_t)stream;
  if (ev.size() > 1) {
    // several evictions depend on one another: the individual calls, then the
    // attention with this step's scratch
    if ((rc = gca_append_frame(c, frame_idx, k, v, 0, stream))) return rc;
    if ((rc = gca_evict_compact(c, stream))) return rc;
    const gca::SelectStep st2 = c->plan.select();
    {
      Prof pr(c, 2, s);
      GCA_HIP(gca::launch_prepare(g.dtype, select_args(c, st2),
                                  query_args(c, c->plan.rope_of(frame_idx), q, w.qrot), s),
              "prepare kernel launch");
    }
    c->sel_valid = true;
    c->sel_n = st2.n_sel;
    c->sel_ctx = st2.n_ctx;
    return attend_launch(c, frame_idx, out, lse, st2, s, w);
  }
  if (rs.n >= 0 && (rc = enqueue_restart(c, rs, s))) return rc;
  gca::AppendArgs aa = append_args(c, as, k, v);
  gca::EvictArgs ea{};
  if (!ev.empty()) ea = evict_args(c, ev[0]);
  gca::RopeArgs ra = query_args(c, p.rope_of(frame_idx), q, w.qrot);
  gca::SelectArgs sa = select_args(c, st);
  sa.newest_pos = as.ring_pos % g.N;
  if (!ev.empty()) {
    sa.traj_known = ev[0].n_traj_pages;
    sa.traj_pos = ev[0].ring_head % g.N;
  }
  {
    Prof pr(c, 6, s);
    GCA_HIP(gca::launch_update(g.dtype, &aa, ev.empty() ? nullptr : &ea, &ra, &sa, s),
            "update kernel launch");
  }
  c->plan = p;
  c->sel_valid = true;
  c->sel_n = st.n_sel;
  c->sel_ctx = st.n_ctx;
  rc = attend_launch(c, frame_idx, out, lse, st, s, w);
  if (rc) return rc;
  if (!key) {
    c->plan.commit_rollback();
    c->sel_valid = false;
  }
  return GCA_OK;
}

}  // namespace

extern "C" {

int gca_step(gca_cache* c, int64_t frame_idx, const void* k, const void* v, const void* q, void* out,
             float* lse, uint32_t flags, gca_stream_t stream) {
  return step_impl(c, frame_idx, k, v, q, out, lse, flags, stream, false);
}

int gca_step_static(gca_cache* c, int64_t frame_idx, const void* k, const void* v, const void* q, void* out,
                    float* lse, uint32_t flags, gca_stream_t stream) {
  return step_impl(c, frame_idx, k, v, q, out, lse, flags, stream, true);
}

int gca_rope3d(gca_cache* c, int64_t frame_idx, const void* x, void* y, gca_stream_t stream) {
  if (!c || !aligned16(x) || !aligned16(y) || frame_idx < 0) return GCA_ERR_INVALID_ARGUMENT;
  if (!c->g.rope) return GCA_ERR_UNSUPPORTED;
  if (frame_idx >= c->g.rope_pos) return GCA_ERR_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  gca::RopeArgs a;
  a.x = x;
  a.y = y;
  a.tpos = frame_idx;
  a.nf = 1;
  a.T = c->g.T;
  a.H = c->g.H;
  a.rotate = 1;
  a.tabs = c->tabs;
  Prof p(c, 5, s);
  GCA_HIP(gca::launch_rope(c->g.dtype, a, s), "rope kernel launch");
  return GCA_OK;
}

int gca_query(const gca_cache* c, gca_info* out) {
  if (!c || !out) return GCA_ERR_INVALID_ARGUMENT;
  c->plan.info(out);
  out->max_splits = kMaxSplits;
  return GCA_OK;
}

int gca_export_state(gca_cache* c, gca_state_view* v, gca_stream_t stream) {
  if (!c || !v) return GCA_ERR_INVALID_ARGUMENT;
  GCA_HIP(hipStreamSynchronize((hipStream_t)stream), "export sync");
  const gca::Geometry& g = c->g;
  std::vector<int32_t> ring(g.N);
  GCA_HIP(hipMemcpy(ring.data(), c->ring, sizeof(int32_t) * g.N, hipMemcpyDeviceToHost), "export ring");
  int64_t head = c->plan.ring_head(), tail = c->plan.ring_tail();
  v->n_free = (int32_t)(tail - head);
  if (v->free_ring)
    for (int64_t i = 0; i < tail - head; ++i) v->free_ring[i] = ring[(size_t)((head + i) % g.N)];
  std::vector<int> slots;
  std::vector<int64_t> frames;
  c->plan.live_frames(&slots, &frames);
  v->n_frames = (int32_t)slots.size();
  std::vector<int32_t> rec((size_t)(g.A + g.Wr) * g.ppf);
  GCA_HIP(hipMemcpy(rec.data(), c->rec_pages, sizeof(int32_t) * rec.size(), hipMemcpyDeviceToHost),
          "export records");
  for (size_t i = 0; i < slots.size(); ++i) {
    if (v->frame_idx) v->frame_idx[i] = frames[i];
    if (v->frame_pages)
      std::memcpy(v->frame_pages + i * g.ppf, rec.data() + (size_t)slots[i] * g.ppf, sizeof(int32_t) * g.ppf);
  }
  gca_info inf;
  c->plan.info(&inf);
  v->n_traj_pages = inf.traj_pages;
  v->traj_tokens = inf.traj_tokens;
  if (v->traj_pages && inf.traj_pages)
    GCA_HIP(hipMemcpy(v->traj_pages, c->traj_pages, sizeof(int32_t) * inf.traj_pages, hipMemcpyDeviceToHost),
            "export trajectory");
  v->n_sel = c->sel_valid ? c->sel_n : 0;
  v->n_ctx = c->sel_valid ? c->sel_ctx : 0;
  if (v->n_sel) {
    if (v->sel_page)
      GCA_HIP(hipMemcpy(v->sel_page, c->sel_page, sizeof(int32_t) * v->n_sel, hipMemcpyDeviceToHost),
              "export gather list");
    if (v->sel_len)
      GCA_HIP(hipMemcpy(v->sel_len, c->sel_len, sizeof(int32_t) * v->n_sel, hipMemcpyDeviceToHost),
              "export gather list");
  }
  return GCA_OK;
}

int gca_read_page(gca_cache* c, int32_t page, void* host_k, void* host_v, gca_stream_t stream) {
  if (!c || page < 0 || page >= c->g.N || !host_k || !host_v) return GCA_ERR_INVALID_ARGUMENT;
  GCA_HIP(hipStreamSynchronize((hipStream_t)stream), "read_page sync");
  const gca::Geometry& g = c->g;
  size_t n = (size_t)g.H * g.P * g.D;
  size_t off = (size_t)page * n * c->esize;
  GCA_HIP(hipMemcpy(host_k, (char*)c->kpool + off, n * c->esize, hipMemcpyDeviceToHost), "read K page");
  std::vector<char> vt(n * c->esize);
  GCA_HIP(hipMemcpy(vt.data(), (char*)c->vpool + off, n * c->esize, hipMemcpyDeviceToHost), "read V page");
  // device V page is [H][D][P] (bf16: slots in operand order, vslot); hand
  // it out as [H][P][D] in slot order
  char* dst = (char*)host_v;
  for (int h = 0; h < g.H; ++h)
    for (int d = 0; d < g.D; ++d)
      for (int s = 0; s < g.P; ++s) {
        const int pos = g.dtype == GCA_BF16 ? gca::vslot(s) : s;
        std::memcpy(dst + (((size_t)h * g.P + s) * g.D + d) * c->esize,
                    vt.data() + (((size_t)h * g.D + d) * g.P + pos) * c->esize, c->esize);
      }
  return GCA_OK;
}

int gca_profile_enable(gca_cache* c, int32_t capacity, uint32_t kinds) {
  if (!c || capacity < 0) return GCA_ERR_INVALID_ARGUMENT;
  c->prof_kinds = kinds;
  GCA_HIP(hipDeviceSynchronize(), "profile sync");
  for (auto& r : c->prof) {
    c->prof_pool.push_back(r.a);
    c->prof_pool.push_back(r.b);
  }
  c->prof.clear();
  c->prof_cap = capacity;
  while ((int)c->prof_pool.size() < 2 * capacity) {
    hipEvent_t e;
    GCA_HIP(hipEventCreate(&e), "hipEventCreate");
    c->prof_pool.push_back(e);
  }
  return GCA_OK;
}

int gca_profile_read(gca_cache* c, int32_t kind, double* total_ms, int32_t* count) {
  if (!c || !total_ms || !count) return GCA_ERR_INVALID_ARGUMENT;
  double sum = 0.0;
  int n = 0;
  std::vector<ProfRec> keep;
  for (auto& r : c->prof) {
    if (r.kind != kind) {
      keep.push_back(r);
      continue;
    }
    GCA_HIP(hipEventSynchronize(r.b), "profile event sync");
    float ms = 0.f;
    GCA_HIP(hipEventElapsedTime(&ms, r.a, r.b), "profile elapsed");
    sum += ms;
    n++;
    c->prof_pool.push_back(r.a);
    c->prof_pool.push_back(r.b);
  }
  c->prof.swap(keep);
  *total_ms = sum;
  *count = n;
  return GCA_OK;
}

}  // extern "C"
