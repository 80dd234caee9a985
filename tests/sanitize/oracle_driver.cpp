// The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
// entry point over seeded tiny streams with keyframes, non-keyframes rolled
// back, evictions into the trajectory, scale frames, page and context
// exports.  Only memory and undefined-behaviour errors are looked for here
// (the values are pinned by the Python tests); a sanitizer report aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
struct orc_config {
  int32_t T, H, D, P;
  int32_t bf16;
  int32_t A, W, C;
  const int32_t* compact_idx;
  int32_t num_special, grid_h, grid_w;
  int32_t rope;
  double rope_theta;
  double sm_scale;
  int64_t max_frames;
  int32_t num_pages;
  const int32_t* ring_init;
  int32_t window, overlap;
};
void* orc_create(const orc_config*);
void orc_destroy(void*);
void orc_reset(void*);
int32_t orc_num_pages(void*);
int32_t orc_pages_per_frame(void*);
int orc_append(void*, int64_t, const float*, const float*, int32_t);
int orc_evict(void*);
int orc_rollback(void*, int64_t);
int64_t orc_n_ctx(void*);
int orc_select(void*, int32_t*, int32_t*, int32_t, int32_t*, int64_t*);
int orc_state(void*, int32_t*, int32_t*, int64_t*, int32_t*, int32_t*, int32_t*, int32_t*, int64_t*);
int orc_context(void*, float*, float*, int64_t*, int32_t*, int64_t);
int orc_page(void*, int32_t, float*, float*, uint8_t*);
void orc_rope(const orc_config*, int64_t, const float*, double*);
int orc_attend(void*, int64_t, const float*, const int32_t*, int32_t, double*, double*, int32_t);
int orc_attend_frames(void*, int64_t, int32_t, const float*, const int32_t*, int32_t, double*, double*,
                      int32_t);
int64_t orc_rope_position(void*, int64_t);
void orc_default_compact(int32_t, int32_t, int32_t, int32_t*);
}

static int fails = 0;
#define EXPECT(c)                                                                          \
  do {                                                                                     \
    if (!(c)) {                                                                            \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c);     \
      ++fails;                                                                             \
    }                                                                                      \
  } while (0)

static void run(orc_config c, int frames, int interval, int scale_frames, uint64_t seed) {
  c.max_frames = frames;
  void* h = orc_create(&c);
  EXPECT(h != nullptr);
  if (!h) return;
  std::mt19937_64 rng(seed);
  std::normal_distribution<float> nd(0.f, 1.f);
  const size_t fe = (size_t)c.T * c.H * c.D;
  std::vector<float> q(fe * (scale_frames > 0 ? scale_frames : 1)), k(fe), v(fe);
  std::vector<int32_t> rows(c.T);
  for (int t = 0; t < c.T; ++t) rows[t] = t;
  const int N = orc_num_pages(h), ppf = orc_pages_per_frame(h);
  std::vector<int32_t> sp(N + 8), sl(N + 8), fr(N), fp((size_t)N * ppf + 8), tp(N + 8);
  std::vector<int64_t> fi(N + 8);
  std::vector<float> pk((size_t)c.H * c.P * c.D), pv(pk.size());
  std::vector<uint8_t> valid(c.P);
  for (int f = 0; f < frames; ++f) {
    const bool key = f % interval == 0 || f < scale_frames;
    for (auto& x : k) x = nd(rng);
    for (auto& x : v) x = nd(rng);
    for (auto& x : q) x = nd(rng);
    EXPECT(orc_append(h, f, k.data(), v.data(), key ? 0 : 1) == 0);
    if (key) EXPECT(orc_evict(h) == 0);
    else EXPECT(orc_evict(h) == -2);
    const int64_t n = orc_n_ctx(h);
    std::vector<double> o((size_t)c.T * c.H * c.D * (scale_frames > 0 ? scale_frames : 1));
    std::vector<double> l((size_t)c.T * c.H * (scale_frames > 0 ? scale_frames : 1));
    if (scale_frames > 0 && f == scale_frames - 1) {
      EXPECT(orc_attend_frames(h, 0, scale_frames, q.data(), rows.data(), c.T, o.data(), l.data(), 3) == 0);
    } else {
      EXPECT(orc_attend(h, f, q.data(), rows.data(), c.T, o.data(), l.data(), 3) == 0);
    }
    for (double x : o) EXPECT(std::isfinite(x));
    int32_t ns = 0;
    int64_t nc = 0;
    EXPECT(orc_select(h, sp.data(), sl.data(), (int32_t)sp.size(), &ns, &nc) == 0 && nc == n);
    int32_t nfree = 0, nfr = 0, ntp = 0;
    int64_t tl = 0;
    EXPECT(orc_state(h, fr.data(), &nfree, fi.data(), fp.data(), &nfr, tp.data(), &ntp, &tl) == 0);
    std::vector<float> kc((size_t)n * c.H * c.D), vc(kc.size());
    std::vector<int64_t> tf(n);
    std::vector<int32_t> tt(n);
    EXPECT(orc_context(h, kc.data(), vc.data(), tf.data(), tt.data(), n) == 0);
    EXPECT(orc_context(h, kc.data(), vc.data(), tf.data(), tt.data(), n - 1) == -1);
    for (int i = 0; i < ns; ++i) EXPECT(orc_page(h, sp[i], pk.data(), pv.data(), valid.data()) == 0);
    if (!key) EXPECT(orc_rollback(h, f) == 0);
  }
  EXPECT(orc_append(h, frames, k.data(), v.data(), 0) == -4);
  orc_reset(h);
  EXPECT(orc_n_ctx(h) == 0);
  orc_destroy(h);
}

int main() {
  orc_config c{};
  c.T = 64; c.H = 2; c.D = 64; c.P = 16; c.bf16 = 0;
  c.A = 1; c.W = 2; c.C = 1; c.compact_idx = nullptr;
  c.num_special = 0; c.grid_h = 8; c.grid_w = 8; c.rope = 0;
  c.rope_theta = 10000.0; c.sm_scale = 0.125; c.num_pages = 0; c.ring_init = nullptr;
  c.window = 0; c.overlap = 0;
  run(c, 8, 1, 0, 1);
  c.bf16 = 1; c.rope = 1; c.T = 36; c.num_special = 3; c.grid_h = 3; c.grid_w = 11; c.C = 5; c.P = 32;
  run(c, 12, 3, 0, 2);
  c.A = 3; c.W = 2;
  run(c, 7, 2, 3, 3);
  c.A = 0; c.W = 3; c.C = 0;
  run(c, 10, 1, 0, 4);
  // windowed inference: windows of 5 frames overlapping by 2 keyframes
  c.A = 1; c.W = 2; c.C = 3; c.window = 5; c.overlap = 2;
  run(c, 17, 1, 0, 5);
  run(c, 17, 2, 0, 6);
  c.window = 0; c.overlap = 0;
  std::vector<double> y((size_t)c.T * c.H * c.D);
  std::vector<float> x(y.size(), 1.f);
  orc_rope(&c, 5, x.data(), y.data());
  int32_t out[13];
  orc_default_compact(1004, 5, 13, out);
  EXPECT(out[12] == 879);
  orc_config bad = c;
  bad.W = 0;
  EXPECT(orc_create(&bad) == nullptr);
  if (fails) {
    std::fprintf(stderr, "%d expectations failed\n", fails);
    return 1;
  }
  std::printf("oracle driver ok\n");
  return 0;
}
