// CPU oracle for Geometric Context Attention (GCA) over a three-pool KV cache.
//
// TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the package smoke check
// and the benchmark's CPU-baseline leg may load this library.  It shares no code,
// header, table or constant with the HIP library: every rule below is written
// out again here from the pages, in plain loops and float64 arithmetic.
//
// What it computes (lingbot-map pages):
//  * Three context pools per attention step ("How the Geometric Context
//    Transformer Enables Streaming 3D Reconstruction", section "Causal
//    Aggregation with KV-Cache Management"; and "LingBot-Map runs 10,000 frames
//    on monocular video", section "How GCT's Anchor-Pose-Trajectory Pools Make
//    Monocular 3D Tractable"): an anchor context, a local window of recent
//    frames, and a trajectory memory that keeps only a few compact tokens of
//    every frame pushed out of the window.
//  * Per-frame call order append -> evict -> attend; a non-keyframe does
//    append -> attend -> rollback and leaves no trace (FlashInferBlock listing,
//    section "Attention Blocks: FlashInfer vs. SDPA").
//  * 3D rotary embedding over (t, h, w) with t = global frame index (section
//    "3D Rotary Positional Embeddings").
//  * Attention = dense softmax attention of the current frame's queries over the
//    selected context; the current frame sees all of its own tokens, earlier
//    frames only through the pools (FAQ "Why are scale frames processed
//    differently", causal across frames).
//  * Scale frames: the first few frames are processed together, each one's
//    queries attending over all of them (bidirectional), before causal
//    streaming starts (section "Streaming Inference API" and the same FAQ).
//    Read as: append those frames, then every one of their queries, rotated
//    at its own frame index, attends over the context that then exists.
//  * Windowed inference ("LingBot-Map runs 10,000 frames on monocular video",
//    section "Cloning and Installing"; the project summary's "Main features"
//    table): past the range the video rotary embedding was trained on, the
//    memory slides as fixed-size windows that overlap by a few keyframes.
//    Read as: a window spans `window` frames from its origin, and a frame's
//    temporal rotary position is its index relative to that origin.  The
//    first frame outside the window starts the next one: the cache is reset,
//    the last `overlap` keyframes that fit in a window with the new frame are
//    appended again from their raw K/V (oldest first, at positions relative
//    to the new origin, which is the oldest of them), then the frame itself.
//    The pages give no restart rule: parity unpinned by the pages (pinned to
//    this reading by hand-derived sizes, positions and live frames in the
//    tests, and by a restarted window equalling a fresh cache).
//
// Readings where the pages are silent (each is a choice, mirrored by the HIP
// library's own independent code):
//  * RoPE split of head_dim D into [t | h | w] blocks with d_h = d_w = 2*(D/6),
//    d_t = D - d_h - d_w; pair j of a block of width d uses frequency
//    theta^(-2j/d); adjacent pairs (2j, 2j+1) rotate; special tokens sit at
//    (t, 0, 0), patch p at (t, p / grid_w, p % grid_w).  Parity unpinned by the
//    pages (only pinned by the rotary invariants in the tests).
//  * Compact tokens: a fixed list of token offsets per frame; default is the
//    special tokens first, then evenly spaced patch tokens.  Parity unpinned by
//    the pages.
//  * Window W counts cached non-anchor keyframes including the newest one.
//  * Page allocator: FIFO ring of N page ids; allocation pops from the head,
//    freeing pushes to the tail in the frame's page order; during an eviction the
//    trajectory page(s) are popped before the evicted frame's pages are pushed;
//    a rollback returns the popped ids to the head.  Frames own ceil(T/P) pages
//    (the last one partial); trajectory tokens pack densely into their own pages.
//  * Gather order: anchor frames, window frames oldest to newest (the pending
//    frame last), then trajectory pages oldest first.
//  * Q' and K' (after rotation) are stored in the cache dtype (bf16 rounding to
//    nearest even, or float32); attention itself is evaluated in float64.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <thread>
#include <vector>

namespace {

enum { OK = 0, E_ARG = -1, E_SEQ = -2, E_PAGES = -3, E_CAP = -4 };

struct Cfg {
  int T, H, D, P;
  int bf16;             // 1: bfloat16 storage, 0: float32 storage
  int A, W, C;
  std::vector<int> compact;
  int num_special, grid_h, grid_w;
  int rope;
  double theta;
  double scale;
  long long max_frames;
  int num_pages;
  std::vector<int> ring_init;
  int window, overlap;  // windowed inference: frames per window (0 = off), overlap keyframes
};

// ---- rounding to the storage type -----------------------------------------

// Round a double to the nearest bfloat16 value (8 significant bits, ties to even).
double round_bf16(double x) {
  if (x == 0.0 || std::isnan(x) || std::isinf(x)) return x;
  int e;
  double m = std::frexp(x, &e);          // x = m * 2^e, 0.5 <= |m| < 1
  double q = std::nearbyint(m * 256.0);  // 8 significant bits, ties to even
  return std::ldexp(q, e - 8);
}

double round_store(const Cfg& c, double x) {
  return c.bf16 ? round_bf16(x) : (double)(float)x;
}

// ---- 3D rotary embedding ----------------------------------------------------

// Angle of rotation pair j (0 <= j < D/2) for token `tok` of frame `frame`.
double rope_angle(const Cfg& c, long long frame, int tok, int j) {
  int dh = 2 * (c.D / 6), dw = dh, dt = c.D - dh - dw;
  long long pt = frame, ph = 0, pw = 0;
  if (tok >= c.num_special) {
    int p = tok - c.num_special;
    ph = p / c.grid_w;
    pw = p % c.grid_w;
  }
  int d = 2 * j;  // first dim of the pair
  if (d < dt) return (double)pt * std::pow(c.theta, -(double)d / dt);
  d -= dt;
  if (d < dh) return (double)ph * std::pow(c.theta, -(double)d / dh);
  d -= dh;
  return (double)pw * std::pow(c.theta, -(double)d / dw);
}

// y = R(frame, tok) x for one head vector of length D (float64, unrounded).
void rope_vec(const Cfg& c, long long frame, int tok, const double* x, double* y) {
  for (int j = 0; j < c.D / 2; ++j) {
    double a = rope_angle(c, frame, tok, j);
    double cs = std::cos(a), sn = std::sin(a);
    y[2 * j] = x[2 * j] * cs - x[2 * j + 1] * sn;
    y[2 * j + 1] = x[2 * j] * sn + x[2 * j + 1] * cs;
  }
}

// Rotate (if enabled) and round a whole frame [T][H][D] into storage values.
// The rotation of a token is the same for every head: its cos/sin are
// evaluated once per token (the values rope_vec would use).  Tokens are
// independent, so blocks of them go to separate threads.
std::vector<float> prepare(const Cfg& c, long long frame, const float* x, bool rotate) {
  size_t n = (size_t)c.T * c.H * c.D;
  std::vector<float> out(n);
  const bool rot = rotate && c.rope;
  auto tokens = [&](int t0, int t1) {
    std::vector<double> a(c.D), b(c.D), cs(c.D / 2), sn(c.D / 2);
    for (int t = t0; t < t1; ++t) {
      if (rot)
        for (int j = 0; j < c.D / 2; ++j) {
          double ang = rope_angle(c, frame, t, j);
          cs[j] = std::cos(ang);
          sn[j] = std::sin(ang);
        }
      for (int h = 0; h < c.H; ++h) {
        const float* src = x + ((size_t)t * c.H + h) * c.D;
        for (int d = 0; d < c.D; ++d) a[d] = src[d];
        if (rot) {
          for (int j = 0; j < c.D / 2; ++j) {
            b[2 * j] = a[2 * j] * cs[j] - a[2 * j + 1] * sn[j];
            b[2 * j + 1] = a[2 * j] * sn[j] + a[2 * j + 1] * cs[j];
          }
        } else {
          b = a;
        }
        float* dst = out.data() + ((size_t)t * c.H + h) * c.D;
        for (int d = 0; d < c.D; ++d) dst[d] = (float)round_store(c, b[d]);
      }
    }
  };
  const int nt = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (nt == 1 || (size_t)c.T * c.H < 4096) {
    tokens(0, c.T);
  } else {
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) pool.emplace_back(tokens, c.T * i / nt, c.T * (i + 1) / nt);
    for (auto& th : pool) th.join();
  }
  return out;
}

// ---- the non-paged cache store and the allocator model -------------------

struct Frame {
  long long idx;
  std::vector<float> k, v;  // [T][H][D], storage values (K rotated)
  std::vector<int> pages;   // allocator model: ceil(T/P) page ids
};

// a keyframe's raw (un-rotated) K/V, kept for the next window's overlap
struct RawFrame {
  long long idx;
  std::vector<float> k, v;  // empty for a frame appended without data
};

struct Cache {
  Cfg c;
  int ppf;
  int N;
  // token store
  std::vector<Frame> anchors;
  std::deque<Frame> window;      // oldest first; a pending TEMP frame is last
  std::vector<float> traj_k, traj_v;  // [len][H][D]
  std::vector<long long> traj_frame;  // provenance tags of trajectory tokens
  std::vector<int> traj_tok;
  long long traj_len = 0;
  bool temp_pending = false;
  bool data_less = false;  // some frame was appended without K/V
  bool has_last = false;
  long long last_frame = -1;
  // allocator model
  std::vector<int> ring;  // size N
  long long head = 0, tail = 0;  // monotonic counters, slot = counter mod N
  std::vector<int> traj_pages;
  // windowed inference
  long long origin = 0;          // frame index of the window's temporal position 0
  std::deque<RawFrame> overlap;  // raw K/V of the window's last keyframes (at most `overlap`)
};

int pop_page(Cache& s) {
  int id = s.ring[(size_t)(s.head % s.N)];
  s.head++;
  return id;
}
void push_page(Cache& s, int id) {
  s.ring[(size_t)(s.tail % s.N)] = id;
  s.tail++;
}
long long free_pages(const Cache& s) { return s.tail - s.head; }

void reset(Cache& s) {
  s.anchors.clear();
  s.window.clear();
  s.traj_k.clear();
  s.traj_v.clear();
  s.traj_frame.clear();
  s.traj_tok.clear();
  s.traj_len = 0;
  s.temp_pending = false;
  s.data_less = false;
  s.has_last = false;
  s.last_frame = -1;
  s.ring.assign(s.N, 0);
  for (int i = 0; i < s.N; ++i) s.ring[i] = s.c.ring_init.empty() ? i : s.c.ring_init[i];
  s.head = 0;
  s.tail = s.N;
  s.traj_pages.clear();
  s.origin = 0;
  s.overlap.clear();
}

int page_len_frame(const Cache& s, int i) {
  return (i == s.ppf - 1) ? s.c.T - (s.ppf - 1) * s.c.P : s.c.P;
}

}  // namespace

extern "C" {

// Configuration as passed from Python (field meaning mirrors the library's, but
// this struct is the oracle's own).
struct orc_config {
  int32_t T, H, D, P;
  int32_t bf16;
  int32_t A, W, C;
  const int32_t* compact_idx;  // NULL -> default rule
  int32_t num_special, grid_h, grid_w;
  int32_t rope;
  double rope_theta;
  double sm_scale;
  int64_t max_frames;
  int32_t num_pages;           // 0 -> peak occupancy of a keyframe stream
  const int32_t* ring_init;    // NULL -> identity order
  int32_t window;              // windowed inference: frames per window (0 = off)
  int32_t overlap;             // keyframes carried into the next window
};

// Default compact offsets: special tokens first, then C - S evenly spaced patches.
void orc_default_compact(int32_t T, int32_t num_special, int32_t C, int32_t* out) {
  int S = std::min(C, num_special);
  for (int j = 0; j < S; ++j) out[j] = j;
  int rest = C - S, npatch = T - num_special;
  for (int j = 0; j < rest; ++j) out[S + j] = num_special + (int)(((long long)j * npatch) / rest);
}

// Pages needed at the peak of a keyframe stream: anchors, W+1 window frames
// (append precedes evict), and the trajectory pages of every possible eviction
// (in windowed mode at most a window's frames are cached between resets).
int64_t orc_default_num_pages(const orc_config* c) {
  long long ppf = (c->T + c->P - 1) / c->P;
  long long span = c->window > 0 ? std::min<long long>(c->max_frames, c->window) : c->max_frames;
  long long evictions = std::max<long long>(0, span - c->A - c->W);
  long long traj_tokens = (long long)c->C * evictions;
  long long traj_pages = (traj_tokens + c->P - 1) / c->P;
  return (long long)c->A * ppf + (long long)(c->W + 1) * ppf + traj_pages;
}

void* orc_create(const orc_config* in) {
  if (!in || in->T <= 0 || in->H <= 0 || in->D <= 0 || in->D % 2 || in->P <= 0 || in->W < 1 ||
      in->A < 0 || in->C < 0 || in->C > in->T || in->max_frames <= 0 || in->window < 0 || in->overlap < 0 ||
      (in->window > 0 && (in->overlap < 1 || in->overlap > in->A + in->W || in->overlap >= in->window)))
    return nullptr;
  Cache* s = new Cache();
  Cfg& c = s->c;
  c.T = in->T; c.H = in->H; c.D = in->D; c.P = in->P; c.bf16 = in->bf16;
  c.A = in->A; c.W = in->W; c.C = in->C;
  c.compact.resize(c.C);
  if (in->compact_idx) for (int j = 0; j < c.C; ++j) c.compact[j] = in->compact_idx[j];
  else if (c.C) orc_default_compact(c.T, in->num_special, c.C, c.compact.data());
  c.num_special = in->num_special; c.grid_h = in->grid_h; c.grid_w = in->grid_w;
  c.rope = in->rope; c.theta = in->rope_theta; c.scale = in->sm_scale;
  c.max_frames = in->max_frames;
  c.window = in->window;
  c.overlap = in->window > 0 ? in->overlap : 0;
  c.num_pages = in->num_pages > 0 ? in->num_pages : (int)orc_default_num_pages(in);
  if (in->ring_init) c.ring_init.assign(in->ring_init, in->ring_init + c.num_pages);
  s->ppf = (c.T + c.P - 1) / c.P;
  s->N = c.num_pages;
  reset(*s);
  return s;
}

void orc_destroy(void* h) { delete (Cache*)h; }
void orc_reset(void* h) { reset(*(Cache*)h); }
int32_t orc_num_pages(void* h) { return ((Cache*)h)->N; }
int32_t orc_pages_per_frame(void* h) { return ((Cache*)h)->ppf; }

// Append one frame at temporal rotary position t (the global frame index, or
// in windowed mode the index relative to the window's origin).
static int append_at(Cache& s, int64_t frame, long long t, const float* k, const float* v, int32_t temp) {
  if (free_pages(s) < s.ppf) return E_PAGES;
  Frame f;
  f.idx = frame;
  // k == v == NULL appends a frame for bookkeeping only (page tables, gather
  // lists); such a cache cannot attend or materialise its context.
  if (k) {
    f.k = prepare(s.c, t, k, true);
    f.v = prepare(s.c, t, v, false);
  } else {
    s.data_less = true;
  }
  for (int i = 0; i < s.ppf; ++i) f.pages.push_back(pop_page(s));
  s.has_last = true;
  s.last_frame = frame;
  if (temp) {
    s.temp_pending = true;
    s.window.push_back(std::move(f));
  } else if ((int)s.anchors.size() < s.c.A) {
    s.anchors.push_back(std::move(f));
  } else {
    s.window.push_back(std::move(f));
  }
  return OK;
}

// Append one frame (raw, un-rotated K and V of shape [T][H][D]).  temp != 0
// marks a non-keyframe that will be rolled back after attention.  In windowed
// mode the first frame outside the window starts the next window first.
int orc_append(void* h, int64_t frame, const float* k, const float* v, int32_t temp) {
  Cache& s = *(Cache*)h;
  if (s.temp_pending) return E_SEQ;
  if (s.has_last && frame <= s.last_frame) return E_SEQ;
  if (frame < 0 || frame >= s.c.max_frames) return E_CAP;
  if ((k == nullptr) != (v == nullptr)) return E_ARG;
  if (s.c.window > 0 && !s.has_last) s.origin = frame;  // the first frame opens the first window
  if (s.c.window > 0 && s.has_last && frame - s.origin >= s.c.window) {
    // the next window: the last keyframes that fit in one window with this
    // frame, oldest first; the oldest of them (or the frame) is the origin
    std::vector<RawFrame> keep;
    for (auto& r : s.overlap)
      if (frame - r.idx < s.c.window) keep.push_back(std::move(r));
    const bool dl = s.data_less;
    reset(s);
    s.data_less = dl;
    s.origin = keep.empty() ? frame : keep.front().idx;
    for (auto& r : keep) {
      int rc = append_at(s, r.idx, r.idx - s.origin, r.k.empty() ? nullptr : r.k.data(),
                         r.v.empty() ? nullptr : r.v.data(), 0);
      if (rc) return rc;
      s.overlap.push_back(std::move(r));
    }
  }
  int rc = append_at(s, frame, s.c.window > 0 ? frame - s.origin : frame, k, v, temp);
  if (rc) return rc;
  if (s.c.window > 0 && !temp) {
    RawFrame r;
    r.idx = frame;
    if (k) {
      size_t n = (size_t)s.c.T * s.c.H * s.c.D;
      r.k.assign(k, k + n);
      r.v.assign(v, v + n);
    }
    s.overlap.push_back(std::move(r));
    while ((int)s.overlap.size() > s.c.overlap) s.overlap.pop_front();
  }
  return OK;
}

// Temporal rotary position of a frame: its global index, or in windowed mode
// its index relative to the window's origin.
int64_t orc_rope_position(void* h, int64_t frame) {
  Cache& s = *(Cache*)h;
  return s.c.window > 0 ? frame - s.origin : frame;
}

// Evict window frames beyond W: keep their compact tokens in the trajectory and
// free their pages.
int orc_evict(void* h) {
  Cache& s = *(Cache*)h;
  if (s.temp_pending) return E_SEQ;
  while ((int)s.window.size() > s.c.W) {
    // capacity check for the whole eviction before touching state
    long long need = 0;
    for (int j = 0; j < s.c.C; ++j)
      if ((s.traj_len + j) % s.c.P == 0) need++;
    if (free_pages(s) < need) return E_PAGES;
    Frame f = std::move(s.window.front());
    s.window.pop_front();
    size_t hd = (size_t)s.c.H * s.c.D;
    for (int j = 0; j < s.c.C; ++j) {
      if (s.traj_len % s.c.P == 0) s.traj_pages.push_back(pop_page(s));
      int tok = s.c.compact[j];
      s.traj_frame.push_back(f.idx);
      s.traj_tok.push_back(tok);
      s.traj_len++;
      if (f.k.empty()) continue;
      s.traj_k.insert(s.traj_k.end(), f.k.begin() + tok * hd, f.k.begin() + (tok + 1) * hd);
      s.traj_v.insert(s.traj_v.end(), f.v.begin() + tok * hd, f.v.begin() + (tok + 1) * hd);
    }
    for (int i = 0; i < s.ppf; ++i) push_page(s, f.pages[i]);
  }
  return OK;
}

// Undo the pending non-keyframe: its pages go back to the ring head.
int orc_rollback(void* h, int64_t frame) {
  Cache& s = *(Cache*)h;
  if (!s.temp_pending || s.window.empty() || s.window.back().idx != frame) return E_SEQ;
  s.head -= s.ppf;
  s.window.pop_back();
  s.temp_pending = false;
  return OK;
}

// Context length (tokens) of the next attention step.
int64_t orc_n_ctx(void* h) {
  Cache& s = *(Cache*)h;
  return (long long)(s.anchors.size() + s.window.size()) * s.c.T + s.traj_len;
}

// Expected gather list (page id, valid tokens) in canonical order.
int orc_select(void* h, int32_t* page, int32_t* len, int32_t cap, int32_t* n_sel, int64_t* n_ctx) {
  Cache& s = *(Cache*)h;
  std::vector<std::pair<int, int>> e;
  for (auto& f : s.anchors)
    for (int i = 0; i < s.ppf; ++i) e.push_back({f.pages[i], page_len_frame(s, i)});
  for (auto& f : s.window)
    for (int i = 0; i < s.ppf; ++i) e.push_back({f.pages[i], page_len_frame(s, i)});
  for (size_t i = 0; i < s.traj_pages.size(); ++i) {
    long long l = std::min<long long>(s.c.P, s.traj_len - (long long)i * s.c.P);
    e.push_back({s.traj_pages[i], (int)l});
  }
  *n_sel = (int)e.size();
  long long tot = 0;
  for (auto& x : e) tot += x.second;
  *n_ctx = tot;
  if ((int)e.size() > cap) return E_ARG;
  for (size_t i = 0; i < e.size(); ++i) { page[i] = e[i].first; len[i] = e[i].second; }
  return OK;
}

// Allocator state: free ring from head (oldest free first), live frames in
// gather order with their pages, trajectory pages.
int orc_state(void* h, int32_t* free_out, int32_t* n_free, int64_t* frame_idx, int32_t* frame_pages,
              int32_t* n_frames, int32_t* traj_pages, int32_t* n_traj_pages, int64_t* traj_len) {
  Cache& s = *(Cache*)h;
  long long nf = free_pages(s);
  *n_free = (int)nf;
  for (long long i = 0; i < nf; ++i) free_out[i] = s.ring[(size_t)((s.head + i) % s.N)];
  int k = 0;
  auto put = [&](const Frame& f) {
    frame_idx[k] = f.idx;
    for (int i = 0; i < s.ppf; ++i) frame_pages[(size_t)k * s.ppf + i] = f.pages[i];
    k++;
  };
  for (auto& f : s.anchors) put(f);
  for (auto& f : s.window) put(f);
  *n_frames = k;
  for (size_t i = 0; i < s.traj_pages.size(); ++i) traj_pages[i] = s.traj_pages[i];
  *n_traj_pages = (int)s.traj_pages.size();
  *traj_len = s.traj_len;
  return OK;
}

// Materialise the context contiguously in canonical order: K'/V rows of
// [n_ctx][H][D] plus provenance (frame index, token offset) of every row.
int orc_context(void* h, float* k_ctx, float* v_ctx, int64_t* tag_frame, int32_t* tag_tok, int64_t cap) {
  Cache& s = *(Cache*)h;
  long long n = orc_n_ctx(h);
  if (n > cap) return E_ARG;
  if (s.data_less && (k_ctx || v_ctx)) return E_ARG;
  size_t hd = (size_t)s.c.H * s.c.D;
  long long r = 0;
  auto put_frame = [&](const Frame& f) {
    if (k_ctx) std::memcpy(k_ctx + r * hd, f.k.data(), sizeof(float) * hd * s.c.T);
    if (v_ctx) std::memcpy(v_ctx + r * hd, f.v.data(), sizeof(float) * hd * s.c.T);
    for (int t = 0; t < s.c.T; ++t) {
      if (tag_frame) tag_frame[r + t] = f.idx;
      if (tag_tok) tag_tok[r + t] = t;
    }
    r += s.c.T;
  };
  for (auto& f : s.anchors) put_frame(f);
  for (auto& f : s.window) put_frame(f);
  if (s.traj_len) {
    if (k_ctx) std::memcpy(k_ctx + r * hd, s.traj_k.data(), sizeof(float) * hd * s.traj_len);
    if (v_ctx) std::memcpy(v_ctx + r * hd, s.traj_v.data(), sizeof(float) * hd * s.traj_len);
    for (long long i = 0; i < s.traj_len; ++i) {
      if (tag_frame) tag_frame[r + i] = s.traj_frame[i];
      if (tag_tok) tag_tok[r + i] = s.traj_tok[i];
    }
  }
  return OK;
}

// Expected content of one physical page: K' and V of its tokens as [H][P][D]
// (storage values) and a validity mask [P].  Returns E_ARG for a free page.
int orc_page(void* h, int32_t page, float* k, float* v, uint8_t* valid) {
  Cache& s = *(Cache*)h;
  if (s.data_less) return E_ARG;
  int P = s.c.P, H = s.c.H, D = s.c.D;
  std::memset(valid, 0, P);
  auto from_frame = [&](const Frame& f) -> bool {
    for (int i = 0; i < s.ppf; ++i) {
      if (f.pages[i] != page) continue;
      for (int slot = 0; slot < P; ++slot) {
        int t = i * P + slot;
        if (t >= s.c.T) break;
        valid[slot] = 1;
        for (int hh = 0; hh < H; ++hh)
          for (int d = 0; d < D; ++d) {
            size_t src = ((size_t)t * H + hh) * D + d;
            size_t dst = ((size_t)hh * P + slot) * D + d;
            k[dst] = f.k[src];
            v[dst] = f.v[src];
          }
      }
      return true;
    }
    return false;
  };
  for (auto& f : s.anchors) if (from_frame(f)) return OK;
  for (auto& f : s.window) if (from_frame(f)) return OK;
  for (size_t i = 0; i < s.traj_pages.size(); ++i) {
    if (s.traj_pages[i] != page) continue;
    for (int slot = 0; slot < P; ++slot) {
      long long t = (long long)i * P + slot;
      if (t >= s.traj_len) break;
      valid[slot] = 1;
      for (int hh = 0; hh < H; ++hh)
        for (int d = 0; d < D; ++d) {
          size_t src = ((size_t)t * H + hh) * D + d;
          size_t dst = ((size_t)hh * P + slot) * D + d;
          k[dst] = s.traj_k[src];
          v[dst] = s.traj_v[src];
        }
    }
    return OK;
  }
  return E_ARG;
}

// Rotary embedding of one frame [T][H][D] in float64 (not rounded).
void orc_rope(const orc_config* in, int64_t frame, const float* x, double* y) {
  Cfg c;
  c.T = in->T; c.H = in->H; c.D = in->D; c.num_special = in->num_special;
  c.grid_h = in->grid_h; c.grid_w = in->grid_w; c.rope = 1; c.theta = in->rope_theta;
  std::vector<double> a(c.D);
  for (int t = 0; t < c.T; ++t)
    for (int hh = 0; hh < c.H; ++hh) {
      size_t o = ((size_t)t * c.H + hh) * c.D;
      for (int d = 0; d < c.D; ++d) a[d] = x[o + d];
      rope_vec(c, frame, t, a.data(), y + o);
    }
}

double orc_rope_angle(const orc_config* in, int64_t frame, int32_t tok, int32_t pair) {
  Cfg c;
  c.D = in->D; c.num_special = in->num_special; c.grid_h = in->grid_h; c.grid_w = in->grid_w;
  c.theta = in->rope_theta;
  return rope_angle(c, frame, tok, pair);
}

double orc_round_bf16(double x) { return round_bf16(x); }

// Dense softmax attention, float64, of prepared queries Qp [T][H][D] (rows
// `rows`) over a materialised context K, V [n][H][D]; out[n_rows][H][D],
// natural-log lse[n_rows][H].
static void attend_over(const Cfg& c, const std::vector<float>& K, const std::vector<float>& V,
                        long long n, const std::vector<float>& Qp, const int32_t* rows,
                        int32_t n_rows, double* out, double* lse, int32_t threads) {
  size_t hd = (size_t)c.H * c.D;
  // one (row, head): two passes over the context (max, then exponentials,
  // row sum and the weighted sum of V)
  auto one = [&](int ri, int hh, std::vector<double>& sc) {
    int t = rows[ri];
    const float* qv = Qp.data() + ((size_t)t * c.H + hh) * c.D;
    double m = -INFINITY;
    for (long long j = 0; j < n; ++j) {
      const float* kv = K.data() + (size_t)j * hd + (size_t)hh * c.D;
      double dot = 0.0;
      for (int d = 0; d < c.D; ++d) dot += (double)qv[d] * (double)kv[d];
      sc[j] = c.scale * dot;
      m = std::max(m, sc[j]);
    }
    double l = 0.0;
    for (long long j = 0; j < n; ++j) {
      sc[j] = std::exp(sc[j] - m);
      l += sc[j];
    }
    double* o = out + ((size_t)ri * c.H + hh) * c.D;
    for (int d = 0; d < c.D; ++d) o[d] = 0.0;
    for (long long j = 0; j < n; ++j) {
      const float* vv = V.data() + (size_t)j * hd + (size_t)hh * c.D;
      for (int d = 0; d < c.D; ++d) o[d] += sc[j] * (double)vv[d];
    }
    for (int d = 0; d < c.D; ++d) o[d] /= l;
    if (lse) lse[(size_t)ri * c.H + hh] = m + std::log(l);
  };
  // work units (head, block of 64 rows), taken in turn by the threads; each
  // (row, head) is computed the same way whatever the thread count
  const int RB = 64;
  const int nrb = (n_rows + RB - 1) / RB;
  const int units = c.H * nrb;
  std::atomic<int> next{0};
  auto work = [&]() {
    std::vector<double> sc(n);
    for (int u = next++; u < units; u = next++) {
      int hh = u / nrb, r0 = (u % nrb) * RB, r1 = std::min<int>(n_rows, r0 + RB);
      for (int ri = r0; ri < r1; ++ri) one(ri, hh, sc);
    }
  };
  int nt = std::max(1, std::min<int>(threads > 0 ? threads : 1, units));
  std::vector<std::thread> pool;
  for (int i = 0; i < nt; ++i) pool.emplace_back(work);
  for (auto& th : pool) th.join();
}

// Attention of frame `frame`'s queries (raw Q [T][H][D]) over the current
// context, for the query rows listed in `rows`.  Output float64
// out[n_rows][H][D] and natural-log LSE lse[n_rows][H].
int orc_attend(void* h, int64_t frame, const float* q, const int32_t* rows, int32_t n_rows,
               double* out, double* lse, int32_t threads) {
  Cache& s = *(Cache*)h;
  if (!s.has_last || frame != s.last_frame) return E_SEQ;
  if (s.data_less) return E_ARG;
  const Cfg& c = s.c;
  long long n = orc_n_ctx(h);
  size_t hd = (size_t)c.H * c.D;
  // 1. materialise the selected context contiguously
  std::vector<float> K((size_t)n * hd), V((size_t)n * hd);
  orc_context(h, K.data(), V.data(), nullptr, nullptr, n);
  // 2. rotate and round the queries (window-relative position in windowed mode)
  std::vector<float> Qp = prepare(c, orc_rope_position(h, frame), q, true);
  // 3. softmax attention per (row, head), float64
  attend_over(c, K, V, n, Qp, rows, n_rows, out, lse, threads);
  return OK;
}

// Scale frames processed together: the queries of frames first .. first +
// nf - 1 (raw Q [nf][T][H][D], the last of them the newest appended frame),
// each rotated at its own frame index, attend over the one current context.
// out[nf][n_rows][H][D], lse[nf][n_rows][H].
int orc_attend_frames(void* h, int64_t first, int32_t nf, const float* q, const int32_t* rows,
                      int32_t n_rows, double* out, double* lse, int32_t threads) {
  Cache& s = *(Cache*)h;
  if (first < 0 || nf < 1) return E_ARG;
  if (!s.has_last || first + nf - 1 != s.last_frame) return E_SEQ;
  if (s.data_less) return E_ARG;
  const Cfg& c = s.c;
  long long n = orc_n_ctx(h);
  size_t hd = (size_t)c.H * c.D;
  std::vector<float> K((size_t)n * hd), V((size_t)n * hd);
  orc_context(h, K.data(), V.data(), nullptr, nullptr, n);
  for (int i = 0; i < nf; ++i) {
    std::vector<float> Qp = prepare(c, orc_rope_position(h, first + i), q + (size_t)i * c.T * hd, true);
    attend_over(c, K, V, n, Qp, rows, n_rows, out + (size_t)i * n_rows * hd,
                lse ? lse + (size_t)i * n_rows * c.H : nullptr, threads);
  }
  return OK;
}

}  // extern "C"
