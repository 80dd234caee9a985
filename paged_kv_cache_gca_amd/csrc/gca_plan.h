// Host-side occupancy state machine of a GCA cache.
//
// Cache occupancy (which ring positions are popped or pushed, which record
// slots hold which frames, how long the trajectory is) depends only on the
// configuration and the call sequence, never on tensor values.  The planner
// tracks it exactly on the host, so every device kernel gets its ring
// positions and record slots as launch arguments and host-side errors need no
// device sync.  Page *ids* are never known here: they live in the device ring
// and page tables.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/gca.h"

namespace gca {

struct Geometry {
  int T, H, D, P;
  int dtype, out_dtype;
  int A, W, C;
  std::vector<int32_t> compact;   // resolved compact offsets
  std::vector<int32_t> ring_init;  // empty: identity
  int num_special, grid_h, grid_w;
  int rope;
  float theta, scale;
  int64_t max_frames;
  int ppf;          // pages per frame = ceil(T / P)
  int N;            // ring size
  int window;       // windowed inference: frames per window (0 = off)
  int overlap;      // keyframes carried into the next window
  int64_t rope_pos; // temporal rotary positions in the table
  int Wr;           // window record slots = W + 1
  int traj_cap;     // trajectory page capacity
  int sel_cap;      // gather-list capacity
  int last_len;     // valid tokens in a frame's last page
};

// Validate a config and derive the geometry.  Returns a gca status code.
int make_geometry(const gca_config* cfg, Geometry* g);

// Launch parameters of one append.
struct AppendStep {
  int64_t frame;
  int64_t rope;      // temporal rotary position (window-relative when windowed)
  int64_t ring_pos;  // ring counter of the first popped page
  int slot;          // record slot receiving the frame's pages
  int raw_slot;      // windowed keyframe: its raw-copy slot, else -1
};

// Windowed inference: the start of the next window, before appending frame
// `frame`: reset, then these keyframes appended again from their raw copies.
constexpr int kMaxOverlap = 16;
struct RestartStep {
  int64_t origin;
  int n;
  AppendStep step[kMaxOverlap];  // raw_slot: where each one's raw copy is
};

// Launch parameters of one eviction.
struct EvictStep {
  int slot;             // record slot of the evicted frame
  int64_t traj_len;     // trajectory tokens before this eviction
  int n_traj_pages;     // trajectory pages before this eviction
  int new_pages;        // trajectory pages popped by this eviction
  int64_t ring_head;    // ring counter of the first popped page
  int64_t ring_tail;    // ring counter where the freed pages are pushed
};

// Layout of the gather list for the current state.
struct SelectStep {
  int n_anchor;
  int win_first, win_count;
  int n_traj_pages;
  int64_t traj_len;
  int n_sel;
  int64_t n_ctx;
};

class Planner {
 public:
  explicit Planner(const Geometry& g) : g_(g) { reset(); }
  void reset();

  // Each check_* validates without changing state; commit_* applies it.
  // Windowed inference: whether appending `frame` starts the next window,
  // and that restart (call before check_append of the frame).
  bool restart_due(int64_t frame) const;
  int check_restart(int64_t frame, RestartStep* out) const;
  void commit_restart(const RestartStep& r);
  int check_append(int64_t frame, bool temp, AppendStep* out) const;
  void commit_append(const AppendStep& s, bool temp);
  int check_evict(std::vector<EvictStep>* out) const;
  void commit_evict(const std::vector<EvictStep>& steps);
  int check_attend(int64_t frame) const;
  int check_rollback(int64_t frame) const;
  void commit_rollback();

  SelectStep select() const;
  void info(gca_info* out) const;
  // Record slots of the live frames in gather order and their frame indices.
  void live_frames(std::vector<int>* slots, std::vector<int64_t>* frames) const;
  int64_t ring_head() const { return head_; }
  int64_t origin() const { return origin_; }
  // temporal rotary position of frame index f
  int64_t rope_of(int64_t f) const { return g_.window > 0 ? f - origin_ : f; }
  int64_t ring_tail() const { return tail_; }
  bool empty() const { return n_anchor_ + win_count_ == 0; }
  const Geometry& geometry() const { return g_; }

 private:
  // the page and slot bookkeeping of an append
  void place(const AppendStep& s, bool temp);

  Geometry g_;
  int64_t head_ = 0, tail_ = 0;  // ring counters; slot = counter mod N
  int n_anchor_ = 0;
  int win_first_ = 0, win_count_ = 0;
  bool temp_ = false;
  bool has_last_ = false;
  int64_t last_ = -1;
  int64_t traj_len_ = 0;
  int n_traj_pages_ = 0;
  std::vector<int64_t> slot_frame_;  // frame index held by each record slot
  // windowed inference
  int64_t origin_ = 0;
  int64_t raw_next_ = 0;                // raw-copy slot of the next keyframe: raw_next_ % overlap
  std::vector<int64_t> ov_frame_;       // the window's last keyframes, oldest first ...
  std::vector<int> ov_slot_;            // ... and their raw-copy slots
};

}  // namespace gca
