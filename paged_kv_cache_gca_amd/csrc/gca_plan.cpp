// Host-side occupancy state machine of a GCA cache (see gca_plan.h).
#include "gca_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <new>

namespace gca {

int make_geometry(const gca_config* c, Geometry* g) {
  if (!c || !g) return GCA_ERR_INVALID_ARGUMENT;
  if (c->tokens_per_frame < 1 || c->num_heads < 1 || c->head_dim < 1 || c->page_size < 1)
    return GCA_ERR_INVALID_ARGUMENT;
  if (c->page_size % 16) return GCA_ERR_INVALID_ARGUMENT;
  if ((c->dtype != GCA_F32 && c->dtype != GCA_BF16) ||
      (c->out_dtype != GCA_F32 && c->out_dtype != GCA_BF16))
    return GCA_ERR_INVALID_ARGUMENT;
  if (c->num_anchor_frames < 0 || c->window_frames < 1 || c->num_compact < 0 ||
      c->num_compact > c->tokens_per_frame || c->max_frames < 1 || c->num_pages < 0 ||
      c->num_special < 0 || c->num_special > c->tokens_per_frame)
    return GCA_ERR_INVALID_ARGUMENT;
  if (c->rope != 0 && c->rope != 1) return GCA_ERR_INVALID_ARGUMENT;
  if (c->rope == 1) {
    if (c->grid_h < 1 || c->grid_w < 1 || !(c->rope_theta > 0.f) ||
        (int64_t)c->num_special + (int64_t)c->grid_h * c->grid_w != c->tokens_per_frame)
      return GCA_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(c->sm_scale) || !(c->sm_scale > 0.f)) return GCA_ERR_INVALID_ARGUMENT;
  if (c->infer_window < 0 || c->infer_overlap < 0) return GCA_ERR_INVALID_ARGUMENT;
  if (c->infer_window > 0 &&
      (c->infer_overlap < 1 || c->infer_overlap > kMaxOverlap ||
       c->infer_overlap > c->num_anchor_frames + c->window_frames || c->infer_overlap >= c->infer_window))
    return GCA_ERR_INVALID_ARGUMENT;
  if (c->head_dim != 64) return GCA_ERR_UNSUPPORTED;
  if (c->page_size != 16 && c->page_size != 32 && c->page_size != 64) return GCA_ERR_UNSUPPORTED;

  Geometry& o = *g;
  o.T = c->tokens_per_frame; o.H = c->num_heads; o.D = c->head_dim; o.P = c->page_size;
  o.dtype = c->dtype; o.out_dtype = c->out_dtype;
  o.A = c->num_anchor_frames; o.W = c->window_frames; o.C = c->num_compact;
  o.num_special = c->num_special; o.grid_h = c->grid_h; o.grid_w = c->grid_w;
  o.rope = c->rope; o.theta = c->rope_theta; o.scale = c->sm_scale;
  o.max_frames = c->max_frames;
  o.window = c->infer_window;
  o.overlap = c->infer_window > 0 ? c->infer_overlap : 0;
  o.rope_pos = o.window > 0 ? std::min<int64_t>(o.max_frames, o.window) : o.max_frames;
  o.ppf = (o.T + o.P - 1) / o.P;
  o.last_len = o.T - (o.ppf - 1) * o.P;
  o.Wr = o.W + 1;

  // compact offsets: given (distinct, in range) or the default rule
  o.compact.assign(o.C, 0);
  if (c->compact_idx) {
    std::vector<char> seen(o.T, 0);
    for (int j = 0; j < o.C; ++j) {
      int t = c->compact_idx[j];
      if (t < 0 || t >= o.T || seen[t]) return GCA_ERR_INVALID_ARGUMENT;
      seen[t] = 1;
      o.compact[j] = t;
    }
  } else {
    // the frame's special tokens first, then C - S patch tokens spread evenly
    int s = std::min(o.C, o.num_special);
    for (int j = 0; j < s; ++j) o.compact[j] = j;
    int rest = o.C - s;
    int npatch = o.T - o.num_special;
    for (int j = 0; j < rest; ++j)
      o.compact[s + j] = o.num_special + (int)(((int64_t)j * npatch) / rest);
  }

  // at most one window's frames are cached between the resets of windowed inference
  int64_t evictions = std::max<int64_t>(0, o.rope_pos - o.A - o.W);
  int64_t traj_pages = ((int64_t)o.C * evictions + o.P - 1) / o.P;
  int64_t n = c->num_pages > 0
                  ? (int64_t)c->num_pages
                  : (int64_t)o.A * o.ppf + (int64_t)o.Wr * o.ppf + traj_pages;
  if (n < 1 || n > (1ll << 30)) return GCA_ERR_INVALID_ARGUMENT;
  o.N = (int)n;
  o.traj_cap = (int)std::min<int64_t>(traj_pages, n);
  int64_t sel = (int64_t)(o.A + o.Wr) * o.ppf + o.traj_cap;
  if (sel > (1ll << 30)) return GCA_ERR_INVALID_ARGUMENT;
  o.sel_cap = (int)sel;

  o.ring_init.clear();
  if (c->ring_init) {
    std::vector<char> seen(o.N, 0);
    o.ring_init.resize(o.N);
    for (int i = 0; i < o.N; ++i) {
      int p = c->ring_init[i];
      if (p < 0 || p >= o.N || seen[p]) return GCA_ERR_INVALID_ARGUMENT;
      seen[p] = 1;
      o.ring_init[i] = p;
    }
  }
  return GCA_OK;
}

void Planner::reset() {
  head_ = 0;
  tail_ = g_.N;
  n_anchor_ = 0;
  win_first_ = 0;
  win_count_ = 0;
  temp_ = false;
  has_last_ = false;
  last_ = -1;
  traj_len_ = 0;
  n_traj_pages_ = 0;
  slot_frame_.assign(g_.A + g_.Wr, -1);
  origin_ = 0;
  raw_next_ = 0;
  ov_frame_.clear();
  ov_slot_.clear();
}

bool Planner::restart_due(int64_t frame) const {
  return g_.window > 0 && has_last_ && frame >= 0 && frame - origin_ >= g_.window;
}

// The next window before frame `frame`: the last keyframes (at most
// `overlap`, oldest first) that fit in one window with it, re-appended into a
// freshly reset cache at positions relative to the oldest of them.
int Planner::check_restart(int64_t frame, RestartStep* out) const {
  if (temp_) return GCA_ERR_SEQUENCE;
  if (frame <= last_) return GCA_ERR_SEQUENCE;
  if (frame >= g_.max_frames) return GCA_ERR_CAPACITY;
  out->n = 0;
  out->origin = frame;
  for (size_t i = 0; i < ov_frame_.size(); ++i)
    if (frame - ov_frame_[i] < g_.window) {
      if (out->n == 0) out->origin = ov_frame_[i];
      AppendStep& a = out->step[out->n++];
      a.frame = ov_frame_[i];
      a.raw_slot = ov_slot_[i];
    }
  // a fresh cache: ring from its initial order, anchors first
  for (int j = 0; j < out->n; ++j) {
    AppendStep& a = out->step[j];
    a.rope = a.frame - out->origin;
    a.ring_pos = (int64_t)j * g_.ppf;
    a.slot = j < g_.A ? j : g_.A + (j - g_.A) % g_.Wr;
  }
  if ((int64_t)out->n * g_.ppf > g_.N) return GCA_ERR_OUT_OF_PAGES;
  return GCA_OK;
}

void Planner::commit_restart(const RestartStep& r) {
  std::vector<int64_t> fr;
  std::vector<int> sl;
  for (int j = 0; j < r.n; ++j) {
    fr.push_back(r.step[j].frame);
    sl.push_back(r.step[j].raw_slot);
  }
  const int64_t rn = raw_next_;
  reset();
  raw_next_ = rn;
  for (int j = 0; j < r.n; ++j) place(r.step[j], false);
  origin_ = r.origin;
  ov_frame_ = fr;
  ov_slot_ = sl;
}

int Planner::check_append(int64_t frame, bool temp, AppendStep* out) const {
  if (frame < 0) return GCA_ERR_INVALID_ARGUMENT;
  if (temp_) return GCA_ERR_SEQUENCE;
  if (has_last_ && frame <= last_) return GCA_ERR_SEQUENCE;
  bool anchor = !temp && n_anchor_ < g_.A;
  if (!anchor && win_count_ >= g_.Wr) return GCA_ERR_SEQUENCE;  // eviction is due
  if (frame >= g_.max_frames) return GCA_ERR_CAPACITY;
  if (tail_ - head_ < g_.ppf) return GCA_ERR_OUT_OF_PAGES;
  // windowed inference: a frame outside the window needs the restart first
  if (g_.window > 0 && has_last_ && frame - origin_ >= g_.window) return GCA_ERR_SEQUENCE;
  out->frame = frame;
  out->rope = g_.window > 0 ? (has_last_ ? frame - origin_ : 0) : frame;
  out->ring_pos = head_;
  out->slot = anchor ? n_anchor_ : g_.A + (win_first_ + win_count_) % g_.Wr;
  out->raw_slot = g_.window > 0 && !temp ? (int)(raw_next_ % g_.overlap) : -1;
  return GCA_OK;
}

void Planner::commit_append(const AppendStep& s, bool temp) {
  place(s, temp);
  if (g_.window > 0 && !temp) {
    // a keyframe appended by the caller: its raw copy went to the next raw slot
    raw_next_++;
    ov_frame_.push_back(s.frame);
    ov_slot_.push_back(s.raw_slot);
    if ((int)ov_frame_.size() > g_.overlap) {
      ov_frame_.erase(ov_frame_.begin());
      ov_slot_.erase(ov_slot_.begin());
    }
  }
}

void Planner::place(const AppendStep& s, bool temp) {
  if (g_.window > 0 && !has_last_) origin_ = s.frame;  // the first frame opens the first window
  head_ += g_.ppf;
  slot_frame_[s.slot] = s.frame;
  if (s.slot < g_.A) n_anchor_++;
  else win_count_++;
  temp_ = temp;
  has_last_ = true;
  last_ = s.frame;
}

int Planner::check_evict(std::vector<EvictStep>* out) const {
  out->clear();
  if (temp_) return GCA_ERR_SEQUENCE;
  int wc = win_count_, wf = win_first_, ntp = n_traj_pages_;
  int64_t tl = traj_len_, h = head_, t = tail_;
  while (wc > g_.W) {
    int fresh = 0;
    for (int j = 0; j < g_.C; ++j)
      if ((tl + j) % g_.P == 0) fresh++;
    if (t - h < fresh) return GCA_ERR_OUT_OF_PAGES;
    if (ntp + fresh > g_.traj_cap) return GCA_ERR_CAPACITY;
    EvictStep e;
    e.slot = g_.A + wf;
    e.traj_len = tl;
    e.n_traj_pages = ntp;
    e.new_pages = fresh;
    e.ring_head = h;
    e.ring_tail = t;
    out->push_back(e);
    h += fresh;
    t += g_.ppf;
    tl += g_.C;
    ntp += fresh;
    wf = (wf + 1) % g_.Wr;
    wc--;
  }
  return GCA_OK;
}

void Planner::commit_evict(const std::vector<EvictStep>& steps) {
  for (const EvictStep& e : steps) {
    head_ += e.new_pages;
    tail_ += g_.ppf;
    traj_len_ += g_.C;
    n_traj_pages_ += e.new_pages;
    slot_frame_[g_.A + win_first_] = -1;
    win_first_ = (win_first_ + 1) % g_.Wr;
    win_count_--;
  }
}

int Planner::check_attend(int64_t frame) const {
  if (!has_last_ || frame != last_ || empty()) return GCA_ERR_SEQUENCE;
  return GCA_OK;
}

int Planner::check_rollback(int64_t frame) const {
  if (!temp_ || frame != last_) return GCA_ERR_SEQUENCE;
  return GCA_OK;
}

void Planner::commit_rollback() {
  head_ -= g_.ppf;
  win_count_--;
  slot_frame_[g_.A + (win_first_ + win_count_) % g_.Wr] = -1;
  temp_ = false;
}

SelectStep Planner::select() const {
  SelectStep s;
  s.n_anchor = n_anchor_;
  s.win_first = win_first_;
  s.win_count = win_count_;
  s.n_traj_pages = n_traj_pages_;
  s.traj_len = traj_len_;
  s.n_sel = (n_anchor_ + win_count_) * g_.ppf + n_traj_pages_;
  s.n_ctx = (int64_t)(n_anchor_ + win_count_) * g_.T + traj_len_;
  return s;
}

void Planner::info(gca_info* o) const {
  SelectStep s = select();
  o->pages_per_frame = g_.ppf;
  o->num_pages = g_.N;
  o->free_pages = (int32_t)(tail_ - head_);
  o->anchor_frames = n_anchor_;
  o->window_frames = win_count_;
  o->temp_pending = temp_ ? 1 : 0;
  o->traj_pages = n_traj_pages_;
  o->n_sel = s.n_sel;
  o->traj_tokens = traj_len_;
  o->n_ctx = s.n_ctx;
  o->last_frame = has_last_ ? last_ : -1;
  o->max_splits = 0;
  o->reserved = 0;
  o->window_origin = g_.window > 0 ? origin_ : 0;
}

void Planner::live_frames(std::vector<int>* slots, std::vector<int64_t>* frames) const {
  slots->clear();
  frames->clear();
  for (int i = 0; i < n_anchor_; ++i) {
    slots->push_back(i);
    frames->push_back(slot_frame_[i]);
  }
  for (int i = 0; i < win_count_; ++i) {
    int s = g_.A + (win_first_ + i) % g_.Wr;
    slots->push_back(s);
    frames->push_back(slot_frame_[s]);
  }
}

}  // namespace gca

// ---- C ABI of the host-only planner ------------------------------------------

struct gca_plan {
  gca::Planner p;
  explicit gca_plan(const gca::Geometry& g) : p(g) {}
};

extern "C" {

int gca_plan_create(const gca_config* cfg, gca_plan** out) {
  if (!out) return GCA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  gca::Geometry g;
  int rc = gca::make_geometry(cfg, &g);
  if (rc) return rc;
  *out = new (std::nothrow) gca_plan(g);
  return *out ? GCA_OK : GCA_ERR_INVALID_ARGUMENT;
}

int gca_plan_destroy(gca_plan* plan) {
  delete plan;
  return GCA_OK;
}

int gca_plan_reset(gca_plan* plan) {
  if (!plan) return GCA_ERR_INVALID_ARGUMENT;
  plan->p.reset();
  return GCA_OK;
}

int gca_plan_append(gca_plan* plan, int64_t frame_idx, uint32_t flags) {
  if (!plan || (flags & ~GCA_APPEND_TEMP)) return GCA_ERR_INVALID_ARGUMENT;
  gca::AppendStep s;
  bool temp = flags & GCA_APPEND_TEMP;
  gca::Planner p = plan->p;
  int rc;
  if (p.restart_due(frame_idx)) {
    gca::RestartStep r;
    if ((rc = p.check_restart(frame_idx, &r))) return rc;
    p.commit_restart(r);
  }
  if ((rc = p.check_append(frame_idx, temp, &s))) return rc;
  p.commit_append(s, temp);
  plan->p = p;
  return GCA_OK;
}

int gca_plan_evict(gca_plan* plan) {
  if (!plan) return GCA_ERR_INVALID_ARGUMENT;
  std::vector<gca::EvictStep> steps;
  int rc = plan->p.check_evict(&steps);
  if (rc) return rc;
  plan->p.commit_evict(steps);
  return GCA_OK;
}

int gca_plan_attend(gca_plan* plan, int64_t frame_idx) {
  if (!plan) return GCA_ERR_INVALID_ARGUMENT;
  return plan->p.check_attend(frame_idx);
}

int gca_plan_rollback(gca_plan* plan, int64_t frame_idx) {
  if (!plan) return GCA_ERR_INVALID_ARGUMENT;
  int rc = plan->p.check_rollback(frame_idx);
  if (rc) return rc;
  plan->p.commit_rollback();
  return GCA_OK;
}

int gca_plan_query(const gca_plan* plan, gca_info* out) {
  if (!plan || !out) return GCA_ERR_INVALID_ARGUMENT;
  plan->p.info(out);
  return GCA_OK;
}

int gca_plan_compact(const gca_plan* plan, int32_t* out, int32_t cap, int32_t* n) {
  if (!plan || !n || cap < 0 || (cap > 0 && !out)) return GCA_ERR_INVALID_ARGUMENT;
  const std::vector<int>& c = plan->p.geometry().compact;
  *n = (int32_t)c.size();
  if ((int32_t)c.size() > cap) return GCA_ERR_CAPACITY;
  for (size_t j = 0; j < c.size(); ++j) out[j] = c[j];
  return GCA_OK;
}

const char* gca_status_string(int s) {
  switch (s) {
    case GCA_OK: return "ok";
    case GCA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GCA_ERR_SEQUENCE: return "call out of protocol order";
    case GCA_ERR_OUT_OF_PAGES: return "out of pages";
    case GCA_ERR_CAPACITY: return "capacity exceeded";
    case GCA_ERR_HIP: return "HIP runtime error";
    case GCA_ERR_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

}  // extern "C"
