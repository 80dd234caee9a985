// Kernel argument blocks and launchers shared by the GCA runtime and kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gca {

constexpr int kHeadDim = 64;    // D
constexpr int kKeysPerTile = 64;  // keys staged in LDS per attention step
constexpr int kWaves = 4;       // waves per attention workgroup
// queries per attention workgroup: 4 waves x 64 (bf16) or x 32 (float32)
inline int queries_per_wg(int dtype) { return kWaves * (dtype ? 64 : 32); }
constexpr int kNumXcd = 8;      // MI355X: 8 accelerator complex dies, round-robin dispatch
// The gather list is written out to (ceil(n_sel / EPT) + 4) * EPT entries, EPT =
// kKeysPerTile / P entries per tile: entries past n_sel name the zero page (page
// N, never handed out) with length 0, so the attention loader can fetch page ids
// up to four tiles ahead unchecked.
//
// Pool invariant: every slot of a live page past its entry's valid length holds
// zeros (append zeroes the frame's last page past T, evict zeroes the last
// trajectory page past the tokens it wrote).  Masked keys get P = 0 and meet a
// zero V row, so stale non-finite data can never reach an output.
constexpr int kSelPad = 5 * (kKeysPerTile / 16);
inline int padded_sel(int n_sel, int P) {
  int ept = kKeysPerTile / P;
  return ((n_sel + ept - 1) / ept + 4) * ept;
}

// Rotary tables: (cos, sin) in float64, evaluated on the host.
struct RopeTabs {
  const double2* t;  // [max_frames][nt]
  const double2* h;  // [grid_h][nh]
  const double2* w;  // [grid_w][nw]
  int nt, nh, nw;   // rotation pairs per axis block (time, row, column)
  int num_special, grid_w;
};

struct AppendArgs {
  const void* k;  // [T][H][D], raw
  const void* v;
  void* raw_k;    // non-null: the raw K and V are also copied here ([T][H][D])
  void* raw_v;
  void* kpool;  // [N][H][P][D]
  void* vpool;  // [N][H][D][P]
  const int32_t* ring;
  int32_t* rec_pages;  // [slots][ppf]
  int64_t ring_pos;
  int64_t tpos;        // temporal rotary position of the frame
  int N, slot, ppf, T, H, P;
  int rope;
  RopeTabs tabs;
};

// Several frames appended in one launch: frame j (0 <= j < n) reads its
// inputs at k[j], v[j] (copying them to rk[j], rv[j] when those are
// non-null), is rotated at temporal position tpos[j], pops ring positions
// ring_pos + j * ppf onwards and fills record slot slot[j]; `a` holds the
// arguments common to all.
constexpr int kMaxAppendBatch = 16;
struct AppendBatch {
  AppendArgs a;
  int n;
  int slot[kMaxAppendBatch];
  int64_t tpos[kMaxAppendBatch];
  const void* k[kMaxAppendBatch];
  const void* v[kMaxAppendBatch];
  void* rk[kMaxAppendBatch];
  void* rv[kMaxAppendBatch];
};

struct EvictArgs {
  void* kpool;
  void* vpool;
  int32_t* ring;
  const int32_t* rec_pages;
  int32_t* traj_pages;
  const int32_t* compact;
  int64_t traj_len, ring_head, ring_tail;
  int N, slot, ppf, n_traj_pages, new_pages, C, H, P;
};

struct SelectArgs {
  const int32_t* rec_pages;
  const int32_t* traj_pages;
  int32_t* sel_page;
  int32_t* sel_len;
  int64_t traj_len;
  int ppf, P, last_len, A, Wr, n_anchor, win_first, win_count, n_traj_pages, n_sel;
  int n_write;    // padded_sel(n_sel, P): entries written, the tail as (zero_page, 0)
  int zero_page;  // N
  // Built in the same launch as an append / eviction: page ids not yet in the
  // page tables are read from the ring where that launch pops them.
  const int32_t* ring;
  int N;
  int64_t newest_pos;  // >= 0: ring position of the newest frame's first page
  int traj_known;      // trajectory pages whose ids are in traj_pages; the
  int64_t traj_pos;    // rest start at this ring position
};

struct AttnArgs {
  const void* q;       // [Tq][H][D], rotated (3D RoPE) and rounded to the cache dtype
  float qk_scale;      // sm_scale * log2(e): scores q'.k' times this are base-2 logits
  const void* kpool;   // [N][H][P][D]
  const void* vpool;   // [N][H][D][P]
  const int32_t* sel_page;
  const int32_t* sel_len;
  float* o_part;       // [S][Tq][H][D] (S > 1)
  float* lse_part;     // [S][Tq][H]
  void* out;           // [Tq][H][D] (S == 1)
  float* lse;          // [Tq][H] or null (S == 1)
  int64_t frame;
  int Tq, H, P, n_sel, n_tiles, tiles_per_split, S, n_qtiles, n_units;
  int t_odd;           // > 0: even splits hold tiles_per_split tiles, odd ones t_odd
  int out_bf16;
  int head_major;      // H % 8 == 0: all workgroups of a head on one XCD
};

struct MergeArgs {
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse;
  int rows;  // Tq * H
  int S;
  int out_bf16;
};

// bf16 V pools hold each 16-slot group of a page row in P-operand order:
// slots 0-3, 8-11, 4-7, 12-15 (storage position s holds slot vslot(s); the
// map swaps bits 2 and 3 and is its own inverse), so that a 16-byte chunk of
// a V^T row is one MFMA operand.  fp32 pools keep slot order.
__host__ __device__ inline int vslot(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

struct RopeArgs {
  const void* x;  // [nf][T][H][D]: temporal positions tpos, tpos + 1, ..., tpos + nf - 1
  void* y;
  int64_t tpos;
  int nf;
  int T, H;
  int rotate;   // 0: y = x
  RopeTabs tabs;
};

// Launchers (defined in gca_kernels.hip).  dtype: 0 float32, 1 bfloat16.
hipError_t launch_append(int dtype, const AppendArgs& a, hipStream_t s);
hipError_t launch_append_batch(int dtype, const AppendBatch& b, hipStream_t s);
hipError_t launch_evict(int dtype, const EvictArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
// gather list and query rotation (into ra.y) in one launch
hipError_t launch_prepare(int dtype, const SelectArgs& sa, const RopeArgs& ra, hipStream_t s);
// One launch: append (if ap), eviction (if ev), query rotation (if ra) and the
// gather list (if sa) of the state after them; their accesses are disjoint.
hipError_t launch_update(int dtype, const AppendArgs* ap, const EvictArgs* ev, const RopeArgs* ra,
                         const SelectArgs* sa, hipStream_t s);
hipError_t launch_attn(int dtype, const AttnArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_rope(int dtype, const RopeArgs& a, hipStream_t s);
hipError_t launch_ring_init(int32_t* ring, const int32_t* init, int N, hipStream_t s);

}  // namespace gca
