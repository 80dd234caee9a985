// Host planner under AddressSanitizer and UndefinedBehaviorSanitizer: every
// entry point of the host-only planner (gca_plan_*), over seeded random call
// sequences of several geometries (keyframes, non-keyframes rolled back,
// evictions, ring wrap-around, error paths), with the occupancy it reports
// checked against the pool rules' closed form for the context size:
//   n_ctx = A' T + w T + C e + (T if a non-keyframe is pending),
// A' anchors so far, w window keyframes, e evictions.
// Windowed inference is checked against a model of its window starts.
// Exits non-zero on the first mismatch; a sanitizer report aborts the run.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "../../include/gca.h"

static int fails = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static gca_config base(int T, int H, int P, int A, int W, int C, int64_t frames) {
  gca_config c{};
  c.tokens_per_frame = T;
  c.num_heads = H;
  c.head_dim = 64;
  c.page_size = P;
  c.dtype = GCA_BF16;
  c.out_dtype = GCA_F32;
  c.num_anchor_frames = A;
  c.window_frames = W;
  c.num_compact = C;
  c.compact_idx = nullptr;
  c.num_special = T > 5 ? 5 : 0;
  c.grid_h = 1;
  c.grid_w = T - c.num_special;
  c.rope = 1;
  c.rope_theta = 10000.f;
  c.sm_scale = 0.125f;
  c.max_frames = frames;
  c.num_pages = 0;
  c.ring_init = nullptr;
  return c;
}

static void stream(const gca_config& cfg, int interval, uint64_t seed) {
  gca_plan* p = nullptr;
  EXPECT(gca_plan_create(&cfg, &p) == GCA_OK);
  if (!p) return;
  std::mt19937_64 rng(seed);
  int32_t offs[64];
  int32_t n = 0;
  EXPECT(gca_plan_compact(p, nullptr, 0, &n) == (cfg.num_compact ? GCA_ERR_CAPACITY : GCA_OK));
  EXPECT(n == cfg.num_compact);
  EXPECT(gca_plan_compact(p, offs, 64, &n) == GCA_OK);
  for (int j = 1; j < n; ++j) EXPECT(offs[j] > offs[j - 1]);
  const int64_t T = cfg.tokens_per_frame;
  int64_t anchors = 0, window = 0, evictions = 0;
  for (int64_t f = 0; f < cfg.max_frames; ++f) {
    const bool key = f % interval == 0;
    // an occasional out-of-order call first: refused, changes nothing
    if (rng() % 7 == 0) {
      gca_info a, b;
      gca_plan_query(p, &a);
      EXPECT(gca_plan_append(p, f > 0 ? f - 1 : -1, 0) != GCA_OK);
      EXPECT(gca_plan_rollback(p, f) == GCA_ERR_SEQUENCE);
      gca_plan_query(p, &b);
      EXPECT(a.n_ctx == b.n_ctx && a.free_pages == b.free_pages && a.last_frame == b.last_frame);
    }
    EXPECT(gca_plan_append(p, f, key ? 0u : (uint32_t)GCA_APPEND_TEMP) == GCA_OK);
    if (key) {
      if (anchors < cfg.num_anchor_frames) anchors++;
      else window++;
      EXPECT(gca_plan_evict(p) == GCA_OK);
      while (window > cfg.window_frames) {
        window--;
        evictions++;
      }
    } else {
      EXPECT(gca_plan_evict(p) == GCA_ERR_SEQUENCE);
    }
    EXPECT(gca_plan_attend(p, f) == GCA_OK);
    gca_info inf;
    EXPECT(gca_plan_query(p, &inf) == GCA_OK);
    const int64_t want = (anchors + window + (key ? 0 : 1)) * T + (int64_t)cfg.num_compact * evictions;
    EXPECT(inf.n_ctx == want);
    EXPECT(inf.traj_tokens == (int64_t)cfg.num_compact * evictions);
    if (!key) EXPECT(gca_plan_rollback(p, f) == GCA_OK);
  }
  EXPECT(gca_plan_append(p, cfg.max_frames, 0) == GCA_ERR_CAPACITY);
  EXPECT(gca_plan_reset(p) == GCA_OK);
  gca_info inf;
  EXPECT(gca_plan_query(p, &inf) == GCA_OK && inf.n_ctx == 0);
  EXPECT(gca_plan_destroy(p) == GCA_OK);
}

// Windowed inference: a model of the window starts (the last `overlap`
// keyframes that fit in a window with the new frame are kept, the oldest kept
// one becomes the origin) checked against the planner's context size and
// origin at every frame.
static void windowed(gca_config cfg, int window, int overlap, int interval) {
  cfg.infer_window = window;
  cfg.infer_overlap = overlap;
  gca_plan* p = nullptr;
  EXPECT(gca_plan_create(&cfg, &p) == GCA_OK);
  if (!p) return;
  const int64_t T = cfg.tokens_per_frame;
  const int A = cfg.num_anchor_frames, W = cfg.window_frames;
  int64_t anchors = 0, win = 0, evictions = 0, origin = 0;
  std::vector<int64_t> keys;  // the last `overlap` keyframes
  int starts = 0;
  for (int64_t f = 0; f < cfg.max_frames; ++f) {
    const bool key = f % interval == 0;
    if (f > 0 && f - origin >= window) {
      std::vector<int64_t> kept;
      for (int64_t k : keys)
        if (f - k < window) kept.push_back(k);
      keys = kept;
      origin = kept.empty() ? f : kept.front();
      anchors = std::min<int64_t>(A, (int64_t)kept.size());
      win = (int64_t)kept.size() - anchors;
      evictions = 0;
      starts++;
    }
    EXPECT(gca_plan_append(p, f, key ? 0u : (uint32_t)GCA_APPEND_TEMP) == GCA_OK);
    if (key) {
      if (anchors < A) anchors++;
      else win++;
      keys.push_back(f);
      if ((int)keys.size() > overlap) keys.erase(keys.begin());
      EXPECT(gca_plan_evict(p) == GCA_OK);
      while (win > W) {
        win--;
        evictions++;
      }
    }
    EXPECT(gca_plan_attend(p, f) == GCA_OK);
    gca_info inf;
    EXPECT(gca_plan_query(p, &inf) == GCA_OK);
    EXPECT(inf.n_ctx == (anchors + win + (key ? 0 : 1)) * T + (int64_t)cfg.num_compact * evictions);
    EXPECT(inf.window_origin == origin);
    if (!key) EXPECT(gca_plan_rollback(p, f) == GCA_OK);
  }
  EXPECT(starts > 0);
  EXPECT(gca_plan_destroy(p) == GCA_OK);
}

int main() {
  // bad configs are refused without leaks
  gca_config bad = base(64, 2, 16, 1, 2, 1, 6);
  bad.page_size = 24;
  gca_plan* p = nullptr;
  EXPECT(gca_plan_create(&bad, &p) == GCA_ERR_INVALID_ARGUMENT && p == nullptr);
  bad = base(64, 2, 16, 1, 2, 2, 6);
  int32_t dup[2] = {3, 3};
  bad.compact_idx = dup;
  EXPECT(gca_plan_create(&bad, &p) == GCA_ERR_INVALID_ARGUMENT);
  EXPECT(gca_plan_create(nullptr, &p) == GCA_ERR_INVALID_ARGUMENT);
  EXPECT(gca_plan_query(nullptr, nullptr) == GCA_ERR_INVALID_ARGUMENT);
  // the workloads' geometries, shortened, and small ones with fast wrap-around
  stream(base(1004, 16, 16, 1, 16, 13, 64), 1, 1);
  stream(base(1004, 16, 64, 1, 64, 13, 300), 1, 2);
  stream(base(1004, 16, 64, 1, 32, 13, 800), 4, 3);
  stream(base(1004, 16, 64, 0, 12, 0, 500), 1, 4);
  stream(base(64, 2, 16, 1, 2, 1, 200), 2, 5);
  stream(base(1, 16, 16, 1, 32, 1, 300), 1, 6);
  stream(base(300, 4, 32, 3, 2, 7, 150), 3, 7);
  windowed(base(1004, 16, 64, 1, 32, 13, 1200), 128, 8, 2);
  windowed(base(66, 2, 16, 1, 3, 3, 200), 8, 3, 3);
  windowed(base(70, 2, 32, 1, 2, 5, 200), 6, 2, 1);
  windowed(base(64, 2, 16, 2, 3, 2, 300), 5, 4, 2);
  if (fails) {
    std::fprintf(stderr, "%d expectations failed\n", fails);
    return 1;
  }
  std::printf("plan driver ok\n");
  return 0;
}
