// HIP kernels of the GCA path for CDNA4 (gfx950, MI355X).
//
//   k_rope    3D (t, h, w) rotary embedding of [nf][T][H][D] (frames
//             frame .. frame + nf - 1)
//   k_append  pop a frame's pages, rotate K, scatter K into [page][H][P][D]
//             and V into dim-major pages (16-slot groups in operand order)
//   k_evict   copy an evicted frame's compact tokens into trajectory pages
//             and push the frame's pages to the ring tail
//   k_select  gather list (page, valid tokens): anchor, window, trajectory
//   k_prepare gather list plus the attention's prepared queries (rotated,
//             rounded once) in one launch
//   k_update  one frame's append, eviction, query preparation and gather
//             list in one launch (the per-frame step)
//   k_attn    paged flash attention: K/V pages staged in LDS, S^T = K Q^T and
//             O^T = V^T P^T on MFMA (bf16 32x32x16, or f32 32x32x2), online
//             softmax in float32, split over the context (split-KV)
//   k_merge   log-sum-exp merge of the split partials
//
// Ring positions, record slots and sizes arrive as launch arguments computed by
// the host planner; page ids are read from and written to device memory only.
#include "gca_kernels.h"

namespace gca {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename T>
union Vec16 {
  uint4 u;
  T e[16 / sizeof(T)];
};

__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(bf16 x) { return (float)x; }
template <typename T>
__device__ inline T from_f(float x);
template <>
__device__ inline float from_f<float>(float x) { return x; }
template <>
__device__ inline bf16 from_f<bf16>(float x) { return (bf16)x; }  // round to nearest even

// ---------------------------------------------------------------------------
// 3D rotary embedding.  Pair j rotates dims (2j, 2j+1); pairs [0, nt) use the
// frame index, [nt, nt+nh) the patch row, the rest the patch column; special
// tokens sit at row 0, column 0.  The rotation is evaluated in float64 from
// float64 (cos, sin) and rounded once to the storage type: y0 = x0 c - x1 s,
// y1 = x0 s + x1 c, each product and the sum rounded in float64 (no fused
// multiply-add), then round to nearest even.

// cos/sin of pairs `pair` and `pair` + 1 (pair even): the axis blocks have an
// even number of pairs (12, 10, 10 for D = 64), so both lie next to each
// other in one table.
__device__ inline void rope_cs2(const RopeTabs& R, int64_t frame, int tok, int pair, double2& c0,
                                double2& c1) {
  const double2* p;
  if (pair < R.nt) {
    p = R.t + frame * R.nt + pair;
  } else {
    int row = 0, col = 0;
    if (tok >= R.num_special) {
      int q = tok - R.num_special;
      row = q / R.grid_w;
      col = q - row * R.grid_w;
    }
    pair -= R.nt;
    p = pair < R.nh ? R.h + row * R.nh + pair : R.w + col * R.nw + (pair - R.nh);
  }
  c0 = p[0];
  c1 = p[1];
}

__device__ inline void rotate(double x0, double x1, double2 cs, double& y0, double& y1) {
  y0 = __dsub_rn(__dmul_rn(x0, cs.x), __dmul_rn(x1, cs.y));
  y1 = __dadd_rn(__dmul_rn(x0, cs.y), __dmul_rn(x1, cs.x));
}

// A float64 value rounded to the storage type, round to nearest even: for
// bfloat16, to 8 significant bits (frexp, rint, ldexp), which a float holds
// exactly and then converts to bfloat16 unchanged.
template <typename T>
__device__ inline T round_store(double y);
template <>
__device__ inline float round_store<float>(double y) { return (float)y; }
template <>
__device__ inline bf16 round_store<bf16>(double y) {
  if (y == 0.0 || !__builtin_isfinite(y)) return (bf16)(float)y;
  int e;
  const double m = __builtin_frexp(y, &e);
  return (bf16)(float)__builtin_ldexp(__builtin_rint(m * 256.0), e - 8);
}

template <typename T>
__device__ inline void rotate_chunk(Vec16<T>& v, const RopeTabs& R, int64_t frame, int tok, int first_pair) {
  constexpr int EPC = 16 / sizeof(T);
#pragma unroll
  for (int m = 0; m < EPC / 2; m += 2) {
    double2 cs[2];
    rope_cs2(R, frame, tok, first_pair + m, cs[0], cs[1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      double y0, y1;
      rotate((double)to_f(v.e[2 * (m + u)]), (double)to_f(v.e[2 * (m + u) + 1]), cs[u], y0, y1);
      v.e[2 * (m + u)] = round_store<T>(y0);
      v.e[2 * (m + u) + 1] = round_store<T>(y1);
    }
  }
}

// 16-byte chunk c of x -> y: rotated when a.rotate, else copied; chunks past
// the tensor are ignored
template <typename T>
__device__ inline void rope_chunk(const RopeArgs& a, size_t c) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = kHeadDim / EPC;
  size_t total = (size_t)a.nf * a.T * a.H * CPR;
  if (c >= total) return;
  int part = (int)(c % CPR);
  int row = (int)(c / CPR / a.H);  // token of the nf stacked frames
  int tok = row % a.T;
  Vec16<T> v;
  v.u = ((const uint4*)a.x)[c];
  if (a.rotate) rotate_chunk<T>(v, a.tabs, a.tpos + row / a.T, tok, part * EPC / 2);
  ((uint4*)a.y)[c] = v.u;
}
template <typename T>
inline size_t rope_chunks(const RopeArgs& a) {
  return (size_t)a.nf * a.T * a.H * (kHeadDim / (16 / sizeof(T)));
}

template <typename T>
__global__ __launch_bounds__(256) void k_rope(RopeArgs a) {
  rope_chunk<T>(a, (size_t)blockIdx.x * 256 + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Append: workgroup (i, h) fills page i of the frame for head h.  K rows are
// rotated and written token-major; V goes through LDS and is written
// dim-major (V^T), the operand layout of the P.V contraction.  Slots past the
// frame's last token are zeroed.

template <typename T>
__device__ inline void append_block(const AppendArgs& a, int i, int h) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = kHeadDim / EPC;
  constexpr int LP = kHeadDim + EPC;  // LDS row pitch
  __shared__ __attribute__((aligned(16))) T lds[64 * LP];
  const int tid = threadIdx.x;
  const int page = a.ring[(a.ring_pos + i) % a.N];
  if (h == 0 && tid == 0) a.rec_pages[a.slot * a.ppf + i] = page;
  const T* K = (const T*)a.k;
  const T* V = (const T*)a.v;
  T* kp = (T*)a.kpool + ((size_t)page * a.H + h) * a.P * kHeadDim;
  T* vp = (T*)a.vpool + ((size_t)page * a.H + h) * kHeadDim * a.P;
  const int tok0 = i * a.P;
  for (int c = tid; c < a.P * CPR; c += 256) {
    int s = c / CPR, part = c - s * CPR;
    int tok = tok0 + s;
    Vec16<T> kv, vv;
    kv.u = make_uint4(0, 0, 0, 0);
    vv.u = kv.u;
    if (tok < a.T) {
      size_t off = ((size_t)tok * a.H + h) * kHeadDim + part * EPC;
      kv.u = *(const uint4*)(K + off);
      vv.u = *(const uint4*)(V + off);
      if (a.raw_k) {
        *(uint4*)((T*)a.raw_k + off) = kv.u;
        *(uint4*)((T*)a.raw_v + off) = vv.u;
      }
      if (a.rope) rotate_chunk<T>(kv, a.tabs, a.tpos, tok, part * EPC / 2);
    }
    *(uint4*)(kp + (size_t)s * kHeadDim + part * EPC) = kv.u;
    *(uint4*)(lds + s * LP + part * EPC) = vv.u;
  }
  __syncthreads();
  const int cpk = a.P / EPC;  // 16-byte chunks per V^T row
  for (int c = tid; c < kHeadDim * cpk; c += 256) {
    int d = c / cpk, kc = c - d * cpk;
    Vec16<T> o;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int slot = sizeof(T) == 2 ? vslot(kc * EPC + e) : kc * EPC + e;
      o.e[e] = lds[slot * LP + d];
    }
    *(uint4*)(vp + (size_t)d * a.P + kc * EPC) = o.u;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  append_block<T>(a, blockIdx.x, blockIdx.y);
}

// workgroup (j * ppf + i, h): page i of frame j of the batch, head h
template <typename T>
__global__ __launch_bounds__(256) void k_append_batch(AppendBatch b) {
  const int j = blockIdx.x / b.a.ppf, i = blockIdx.x - j * b.a.ppf;
  AppendArgs a = b.a;
  a.k = b.k[j];
  a.v = b.v[j];
  a.raw_k = b.rk[j];
  a.raw_v = b.rv[j];
  a.ring_pos = (b.a.ring_pos + (int64_t)j * a.ppf) % a.N;
  a.tpos = b.tpos[j];
  a.slot = b.slot[j];
  append_block<T>(a, i, blockIdx.y);
}

// ---------------------------------------------------------------------------
// Evict one frame: workgroup h copies the C compact tokens of head h; block 0
// also records the trajectory pages it pops and pushes the frame's pages to
// the ring tail.  The popped positions [ring_head, ring_head + new_pages) and
// pushed positions [ring_tail, ring_tail + ppf) never overlap modulo N because
// the evicted frame's own pages are live while it is evicted.

// Workgroup b of an eviction: head h = b / evict_groups(C), compact tokens
// [4g, 4g + 4) with g = b % evict_groups(C), one (token, dim) element per
// thread, so every element's chain of dependent loads (compact offset, source
// page, element) runs in parallel.  Group 0 of each head also zeroes its last
// trajectory page past the new end; group 0 of head 0 records the popped
// trajectory pages and pushes the evicted frame's pages to the ring tail.
__host__ __device__ inline int evict_groups(int C) { return C > 4 ? (C + 3) / 4 : 1; }

template <typename T>
__device__ inline void evict_block(const EvictArgs& a, int b) {
  const int tid = threadIdx.x;
  const int ng = evict_groups(a.C);
  const int h = b / ng, grp = b % ng;
  T* kp = (T*)a.kpool;
  T* vp = (T*)a.vpool;
  const int j = grp * 4 + (tid >> 6), d = tid & 63;
  if (j < a.C) {
    int tok = a.compact[j];
    int src = a.rec_pages[a.slot * a.ppf + tok / a.P];
    int ss = tok % a.P;
    int64_t tt = a.traj_len + j;
    int pi = (int)(tt / a.P);
    int ds = (int)(tt % a.P);
    int dst = pi < a.n_traj_pages ? a.traj_pages[pi]
                                  : a.ring[(a.ring_head + (pi - a.n_traj_pages)) % a.N];
    kp[(((size_t)dst * a.H + h) * a.P + ds) * kHeadDim + d] =
        kp[(((size_t)src * a.H + h) * a.P + ss) * kHeadDim + d];
    const int vd = sizeof(T) == 2 ? vslot(ds) : ds, vs = sizeof(T) == 2 ? vslot(ss) : ss;
    vp[(((size_t)dst * a.H + h) * kHeadDim + d) * a.P + vd] =
        vp[(((size_t)src * a.H + h) * kHeadDim + d) * a.P + vs];
  }
  if (grp != 0) return;
  // slots of the last written trajectory page past the new end stay zero (a
  // popped page holds stale data); they are disjoint from the slots copied above
  const int64_t end = a.traj_len + a.C;
  const int fill = (int)(end % a.P);
  if (a.C > 0 && fill != 0) {
    int pi = (int)((end - 1) / a.P);
    int dst = pi < a.n_traj_pages ? a.traj_pages[pi]
                                  : a.ring[(a.ring_head + (pi - a.n_traj_pages)) % a.N];
    const int n = (a.P - fill) * kHeadDim;
    for (int idx = tid; idx < n; idx += 256) {
      int jj = idx / kHeadDim, dd = idx - jj * kHeadDim;
      kp[(((size_t)dst * a.H + h) * a.P + fill + jj) * kHeadDim + dd] = from_f<T>(0.f);
      const int vz = sizeof(T) == 2 ? vslot(fill + jj) : fill + jj;
      vp[(((size_t)dst * a.H + h) * kHeadDim + dd) * a.P + vz] = from_f<T>(0.f);
    }
  }
  if (h == 0) {
    for (int i = tid; i < a.new_pages; i += 256)
      a.traj_pages[a.n_traj_pages + i] = a.ring[(a.ring_head + i) % a.N];
    for (int i = tid; i < a.ppf; i += 256)
      a.ring[(a.ring_tail + i) % a.N] = a.rec_pages[a.slot * a.ppf + i];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_evict(EvictArgs a) {
  evict_block<T>(a, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Gather list in canonical order: anchors, window oldest -> newest, trajectory.

__device__ inline void gather_entry(const SelectArgs& a, int e) {
  int page = a.zero_page, len = 0;
  const int nfr = a.n_anchor + a.win_count;
  int nf = nfr * a.ppf;
  if (e < nf) {
    int f = e / a.ppf, i = e - f * a.ppf;
    int slot = f < a.n_anchor ? f : a.A + (a.win_first + (f - a.n_anchor)) % a.Wr;
    page = (a.newest_pos >= 0 && f == nfr - 1) ? a.ring[(a.newest_pos + i) % a.N]
                                               : a.rec_pages[slot * a.ppf + i];
    len = (i == a.ppf - 1) ? a.last_len : a.P;
  } else if (e < a.n_sel) {
    int ti = e - nf;
    page = ti < a.traj_known ? a.traj_pages[ti] : a.ring[(a.traj_pos + (ti - a.traj_known)) % a.N];
    int64_t rem = a.traj_len - (int64_t)ti * a.P;
    len = rem < a.P ? (int)rem : a.P;
  }
  a.sel_page[e] = page;
  a.sel_len[e] = len;
}

__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
  int e = blockIdx.x * 256 + threadIdx.x;
  if (e < a.n_write) gather_entry(a, e);
}

// One launch per attention call: blocks [0, sel_blocks) build the gather
// list, the remaining blocks rotate the queries (one frame's, or the scale
// frames' together) into a workspace.
template <typename T>
__global__ __launch_bounds__(256) void k_prepare(SelectArgs sa, RopeArgs ra, int sel_blocks) {
  if ((int)blockIdx.x < sel_blocks) {
    int e = blockIdx.x * 256 + threadIdx.x;
    if (e < sa.n_write) gather_entry(sa, e);
    return;
  }
  rope_chunk<T>(ra, (size_t)(blockIdx.x - sel_blocks) * 256 + threadIdx.x);
}

// The per-frame update as one launch.  Block ranges: [0, na) append blocks
// (page i = b % ppf, head b / ppf), [na, na + ne) eviction blocks (head, token group),
// [.., + nr) query rotation chunks, [.., + ns) gather-list entries.  The
// append writes the new frame's pages and record slot; the eviction reads
// the oldest window frame's pages, writes trajectory pages popped after the
// append's and pushes to the ring tail; the gather list reads page ids that
// are not in the page tables yet from the ring positions those pops use.
template <typename T>
__global__ __launch_bounds__(256) void k_update(AppendArgs ap, EvictArgs ev, RopeArgs ra, SelectArgs sa,
                                                 int na, int ne, int nr) {
  int b = blockIdx.x;
  if (b < na) {
    append_block<T>(ap, b % ap.ppf, b / ap.ppf);
    return;
  }
  b -= na;
  if (b < ne) {
    evict_block<T>(ev, b);
    return;
  }
  b -= ne;
  if (b < nr) {
    rope_chunk<T>(ra, (size_t)b * 256 + threadIdx.x);
    return;
  }
  b -= nr;
  const int e = b * 256 + threadIdx.x;
  if (e < sa.n_write) gather_entry(sa, e);
}

__global__ void k_ring_init(int32_t* ring, const int32_t* init, int N) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < N) ring[i] = init ? init[i] : i;
}

// ---------------------------------------------------------------------------
// Paged attention.
//
// Workgroup = 4 waves x 64 queries (32 with the fp32 cache) of one head,
// over one split of the gather list.  Per 64-key tile: K (64 keys x 64 dims)
// and V^T (64 dims x 64 keys) are staged in LDS, then each wave computes
// S^T = K Q^T (keys x queries) with 32x32 MFMA blocks, so that each lane owns
// one query column: the softmax max and scaling are per lane plus one
// exchange with lane ^ 32.  P^T is fed
// straight from the S^T accumulators as the B operand of O^T = V^T P^T; the
// key order inside each 16-key chunk follows the accumulator layout, and the
// V^T operand is read in the same order.  Row sums add the same rounded P
// that P.V uses (on the matrix cores in the bf16 kernel), so sum(P) and P.V
// use identical weights (they sum to one, so an offset common to all V rows
// passes through).

template <typename T>
struct Mfma;

__device__ inline floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// A 32-key block with a masked key gets a rank-1 mask product in its S^T
// accumulators (the fp32 kernel starts from it, the bf16 kernel adds it after
// K.Q^T): A holds, per key row, 1 for a key past its gather entry's valid
// length (else 0) in column 0; B holds -1e30 in row 0 for every query column.
// A masked key's score is then about -1e30, its logit -inf in effect, its P
// exactly 0.
constexpr float kMaskedScore = -1e30f;
typedef short shortx4 __attribute__((ext_vector_type(4)));

template <>
struct Mfma<bf16> {
  static constexpr int NQB = 2;  // 32-query blocks per wave
  static constexpr int KPL = 8;  // operand elements per lane
  typedef bf16x8 Frag;
  typedef shortx4 Seed;          // 32x32x8 operand: lane (l32, hi) holds k = 4*hi .. 4*hi+3
  __device__ static inline floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline short bits(float x) { return __builtin_bit_cast(short, (bf16)x); }
  __device__ static inline Seed mask_a(bool masked, int hi) {
    Seed r = {0, 0, 0, 0};
    if (hi == 0) r[0] = bits(masked ? 1.f : 0.f);
    return r;
  }
  __device__ static inline Seed mask_b(int hi) {
    Seed r = {0, 0, 0, 0};
    if (hi == 0) r[0] = bits(kMaskedScore);
    return r;
  }
  __device__ static inline floatx16 mma_seed(Seed a, Seed b) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, zero16(), 0, 0, 0);
  }
  __device__ static inline floatx16 mma_seed_acc(Seed a, Seed b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  static constexpr int NQB = 1;
  static constexpr int KPL = 1;
  typedef float Frag;
  typedef float Seed;            // 32x32x2 operand: lane (l32, hi) holds k = hi
  __device__ static inline floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline Seed mask_a(bool masked, int hi) { return hi == 0 && masked ? 1.f : 0.f; }
  __device__ static inline Seed mask_b(int hi) { return hi == 0 ? kMaskedScore : 0.f; }
  __device__ static inline floatx16 mma_seed(Seed a, Seed b) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, zero16(), 0, 0, 0);
  }
};

// bf16 tiles in LDS: 64 rows of 128 bytes (K: key rows of 64 dims; V^T: dim
// rows of 64 keys), no padding.  A 128-bit LDS read serves 16 lanes per
// cycle from 64 four-byte banks (256 bytes), and an operand read gives those
// lanes 16 consecutive rows at one logical chunk.  Two consecutive rows span
// all 64 banks, so the 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 1) & 7): the 8 row pairs of a lane group use 8 different
// positions, each row of a pair its own half of the banks.
__device__ inline int swz(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// fp32 K operand: key row `row`, dim 2 dc + hi.
__device__ inline float read_k(const float* lk, int pitch, int row, int dc, int hi) {
  return lk[row * pitch + dc * 2 + hi];
}

// bf16 V^T tile in LDS: the 16-byte chunk q of dim row d holds key slots
// 8q .. 8q + 7 of the tile.  The tile is stored page by page, as the pool
// holds it: page q / (P / 8) of the tile is one block of 64 dim rows of P / 8
// chunks (128 P bytes), so that one DMA load instruction (1 KB) fills part of
// one page only.  Inside a block the chunk u of row d sits at position
// u ^ ((d / R) mod (P / 8)), R = 16 / (P / 8) rows per 256 bytes: the 16
// rows that one operand read serves together then cover all 64 banks.  At
// P = 64 this is the K tile's swizzle.
//
// Operand reads of the bf16 tiles, from lane offsets computed once.
// K: key row 32 kb + l32, dims [16 dc + 8 hi, +8) (swz; the row's XOR term
// does not depend on kb).  V^T: dim row 32 db + l32, chunk 4 kb + 2 ch + hi,
// i.e. the keys whose S^T accumulator registers form the matching P^T
// operand, keys 16*ch + 4*hi + {0..3} and 16*ch + 8 + 4*hi + {0..3} of the
// block; the V^T tile holds each 16-key group in that order (keys 0-3, 8-11,
// 4-7, 12-15), so the operand is one 16-byte read.  In the V^T layout the
// row's XOR term does not depend on db, and the chunk splits into a page and
// an in-page chunk without carries, so only the in-page chunk's XOR takes a
// lane offset of its own: one at P = 16, two at P = 32, four at P = 64.  The
// offsets are kept opaque, so that each read is one register plus an
// immediate.
template <int P>
struct TileAddr {
  static constexpr int CPP = P / 8, R = 16 / CPP, NV = CPP / 2;
  int k[4], v[NV];
  __device__ void init(int l32, int hi) {
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      k[dc] = swz(l32, dc * 2 + hi);
      asm volatile("" : "+v"(k[dc]));
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      v[i] = l32 * (CPP * 16) + (((2 * i + hi) ^ ((l32 / R) % CPP)) << 4);
      asm volatile("" : "+v"(v[i]));
    }
  }
  __device__ bf16x8 kop(const char* t, int kb, int dc) const {
    return *(const bf16x8*)(t + kb * 32 * 128 + k[dc]);
  }
  __device__ bf16x8 vop(const char* t, int db, int kb, int ch) const {
    const int q0 = kb * 4 + ch * 2;
    return *(const bf16x8*)(t + (q0 / CPP) * (128 * P) + db * (32 * CPP * 16) + v[(q0 % CPP) / 2]);
  }
};

// fp32 V^T operand
__device__ inline float read_v(const float* lv, int pitch, int d, int kb, int ch, int hi) {
  return lv[d * pitch + kb * 32 + (ch >> 2) * 8 + hi * 4 + (ch & 3)];
}

__device__ inline bf16x8 pack_p(const floatx16& s, int ch, bf16) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)s[ch * 8 + i];
  return r;
}
__device__ inline float pack_p(const floatx16& s, int ch, float) { return s[ch]; }

// Queries (already rotated) as B operands: lane holds query qb*32 + l32,
// dims [dc*2*KPL + hi*KPL, +KPL).  Lanes past the last query read the last
// one (no branch, so no load waits for another): their columns are computed
// and never written.
__device__ inline void load_q(const AttnArgs& a, int qbase, int h, int l32, int hi, bf16x8 (&qf)[2][4]) {
  const bf16* Q = (const bf16*)a.q;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = min(qbase + qb * 32 + l32, a.Tq - 1);
#pragma unroll
    for (int dc = 0; dc < 4; ++dc)
      qf[qb][dc] = *(const bf16x8*)(Q + ((size_t)q * a.H + h) * kHeadDim + dc * 16 + hi * 8);
  }
}
__device__ inline void load_q(const AttnArgs& a, int qbase, int h, int l32, int hi, float (&qf)[1][32]) {
  const float* Q = (const float*)a.q;
  int q = qbase + l32;
#pragma unroll
  for (int dc = 0; dc < 32; ++dc)
    qf[0][dc] = q < a.Tq ? Q[((size_t)q * a.H + h) * kHeadDim + dc * 2 + hi] : 0.f;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// The EPT (= 1, 2 or 4) valid lengths of one tile's gather entries.
template <int N>
__device__ inline i32x4 load_lens(const int32_t* p) {
  i32x4 v = {0, 0, 0, 0};
  if constexpr (N == 4) {
    v = *(const i32x4*)p;
  } else if constexpr (N == 2) {
    const i32x2 u = *(const i32x2*)p;
    v.x = u.x;
    v.y = u.y;
  } else {
    v.x = *p;
  }
  return v;
}

// The same, for a wave-uniform address: scalar loads.
template <int N>
__device__ inline i32x4 load_uniform(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  typedef const __attribute__((address_space(4))) i32x2 cint2;
  typedef const __attribute__((address_space(4))) i32x4 cint4;
  i32x4 v = {0, 0, 0, 0};
  if constexpr (N == 4) {
    v = *(cint4*)(const void*)p;
  } else if constexpr (N == 2) {
    const i32x2 u = *(cint2*)(const void*)p;
    v.x = u.x;
    v.y = u.y;
  } else {
    v.x = *(cint*)(const void*)p;
  }
  return v;
}

// element j of v (a per-lane index): straight-line selects, no divergent branches
__device__ inline int pick(i32x4 v, int j) {
  int r = v.x;
  r = j == 1 ? v.y : r;
  r = j == 2 ? v.z : r;
  r = j == 3 ? v.w : r;
  return r;
}

// Key `key` of a tile is masked when its slot lies past its gather entry's
// valid length (a partial page, or padding).
template <int P>
__device__ inline bool key_masked(const i32x4& tl, int key) {
  return (key % P) >= pick(tl, key / P);
}

// Whether any entry of the tile is partial (the same in every lane: made
// wave-uniform so that full tiles skip the masks).
template <int P>
__device__ inline bool tile_partial(const i32x4& tl) {
  constexpr int EPT = kKeysPerTile / P;
  int any = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) any |= pick(tl, e) < P;
  return __builtin_amdgcn_readfirstlane(any) != 0;
}

// Whether 32-key block kb of a tile holds a masked key, from the entry
// lengths in scalar registers (wave-uniform).
template <int P>
__device__ inline bool block_masked(const i32x4& tl, int kb) {
  if constexpr (P <= 32) {
    bool m = false;
#pragma unroll
    for (int e = kb * 32 / P; e < (kb + 1) * 32 / P; ++e) m = m || pick(tl, e) < P;
    return m;
  } else {
    return tl.x < (kb + 1) * 32;
  }
}

template <typename T, int P>
struct TileLoader {
  static constexpr int EPC = 16 / sizeof(T);           // elements per 16-byte chunk
  static constexpr int EPT = kKeysPerTile / P;         // gather entries per tile
  static constexpr int CPRK = kHeadDim / EPC;          // chunks per K row
  static constexpr int CPRV = kKeysPerTile / EPC;      // chunks per V^T row
  static constexpr int NC = kKeysPerTile * CPRK / 256; // chunks per thread (K and V alike)
  // LDS layout: bf16 as the swizzled 128-byte rows the operand reads expect
  // (swz); fp32 rows padded by 16 bytes
  static constexpr bool SWZ = sizeof(T) == 2;
  static constexpr int KP = SWZ ? kHeadDim : kHeadDim + EPC;
  static constexpr int VP = SWZ ? kKeysPerTile : kKeysPerTile + EPC;
  static constexpr int TILE_ELEMS = kKeysPerTile * KP + kHeadDim * VP;

  // chunk i of thread t: K row r = c / CPRK, part c % CPRK; V^T row d = c / CPRV,
  // keys (c % CPRV) * EPC.. with c = t + 256 i.  c % CPRV does not depend on i.
  __device__ static int k_row(int tid, int i) { return (tid + 256 * i) / CPRK; }
  __device__ static int k_part(int tid) { return tid % CPRK; }
  __device__ static int v_row(int tid, int i) { return (tid + 256 * i) / CPRV; }
  __device__ static int v_key0(int tid) { return (tid % CPRV) * EPC; }

  const char* kaddr[NC];     // this thread's K chunks inside page 0 (bytes)
  const char* vaddr;         // its first V^T chunk inside page 0; chunk i is VSTEP bytes on
  static constexpr int VSTEP = (256 / CPRV) * P * (int)sizeof(T);
  uint32_t page_bytes;
  int pg_k[NC], pg_v;         // page ids of the next tile
  u32x4 kr[NC], vr[NC];       // 16-byte chunks of the next tile (native vectors: plain loads)
  i32x4 tlen;                 // valid lengths of the EPT entries of the tile whose page ids are held
  i32x4 dlen;                 // the same for the tile held in kr / vr

  __device__ void init(const T* kpool, const T* vpool, int h, int H, int tid) {
    page_bytes = (uint32_t)(H * P * kHeadDim * sizeof(T));
#pragma unroll
    for (int i = 0; i < NC; ++i)
      kaddr[i] = (const char*)(kpool + ((h * P) + (k_row(tid, i) % P)) * kHeadDim + k_part(tid) * EPC);
    vaddr = (const char*)(vpool + (h * kHeadDim + v_row(tid, 0)) * P + (v_key0(tid) % P));
  }
  // page ids and lengths of tile `tile` (the gather list is padded past its
  // end).  With several entries per tile each thread loads those of its own
  // chunks with plain loads and all EPT lengths with one vector load,
  // consumed a whole tile later when that tile's data loads are issued; with
  // one entry per tile (P = 64) a scalar load through the constant address
  // space (the list is not written during the launch) serves the whole wave.
  __device__ void fetch_pages(const AttnArgs& a, int tile, int tid) {
    if constexpr (EPT == 1) {
      typedef const __attribute__((address_space(4))) int32_t cint;
      const int pg = *(cint*)(const void*)(a.sel_page + tile);
      const int ln = *(cint*)(const void*)(a.sel_len + tile);
#pragma unroll
      for (int i = 0; i < NC; ++i) pg_k[i] = pg;
      pg_v = pg;
      tlen = i32x4{ln, ln, ln, ln};
    } else {
      const int32_t* sp = a.sel_page + tile * EPT;
#pragma unroll
      for (int i = 0; i < NC; ++i) pg_k[i] = sp[k_row(tid, i) / P];
      pg_v = sp[v_key0(tid) / P];
      tlen = load_lens<EPT>(a.sel_len + tile * EPT);
    }
  }
  __device__ void fetch_data(int tid) {
    dlen = tlen;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      kr[i] = *(const u32x4*)(kaddr[i] + (uint64_t)(uint32_t)pg_k[i] * page_bytes);
      vr[i] = *(const u32x4*)(vaddr + (uint64_t)(uint32_t)pg_v * page_bytes + i * VSTEP);
    }
  }
  __device__ void store(T* tileb, int tid) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if constexpr (SWZ) {
        char* kt = (char*)tileb;
        *(u32x4*)(kt + swz(k_row(tid, i), k_part(tid))) = kr[i];
        *(u32x4*)(kt + kKeysPerTile * KP * 2 + swz(v_row(tid, i), v_key0(tid) / EPC)) = vr[i];
      } else {
        *(u32x4*)(tileb + k_row(tid, i) * KP + k_part(tid) * EPC) = kr[i];
        *(u32x4*)(tileb + kKeysPerTile * KP + v_row(tid, i) * VP + v_key0(tid)) = vr[i];
      }
    }
  }
};

// bf16 tiles go straight from HBM/L2 into LDS (global_load_lds: each lane's
// 16 bytes land at the instruction's LDS base + lane * 16), three buffers
// deep, so a tile's loads have two tiles of math to land and no registers
// hold tile data.  Each lane loads the 16-byte piece that belongs at its
// (swizzled) LDS position: 2 instructions per wave for K and 2 for V^T, whose
// pool rows are already in operand order (vslot).  Page ids and entry
// lengths are loaded one tile before the tile's data, with plain per-lane
// vector loads.
template <int P>
struct DmaLoader {
  static constexpr int EPT = kKeysPerTile / P;
  static constexpr int KBYTES = kKeysPerTile * kHeadDim * 2;  // 8 KB, then V^T 8 KB
  static constexpr int BUF_BYTES = 2 * KBYTES;
  static constexpr int NISSUE = 4;  // DMA loads per wave and tile
  // the EPT page ids and lengths of a tile: wave-uniform, in scalar
  // registers
  struct Ids {
    i32x4 pg, ln;
  };
  uint32_t page_bytes, head_off;
  int w, pw;
  uint32_t koff[2], voff[2];

  // Wave w fills tile bytes [2 KB w, 2 KB (w + 1)) of K and of V^T with its two
  // loads each: key rows 16 w .. 16 w + 15 and their V^T chunks, all in the
  // tile's page pw = 16 w / P.  koff and voff are this lane's byte offsets
  // inside that page's (page, head) block, the same for every tile.
  __device__ void init(int h, int H, int tid) {
    w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the LDS destinations need no waterfall
    pw = 16 * w / P;
    const int lane = tid & 63;
    page_bytes = (uint32_t)(H * P * kHeadDim * 2);
    head_off = (uint32_t)(h * P * kHeadDim * 2);
    constexpr int CPP = P / 8, R = 16 / CPP;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = (w * 2 + j) * 64 + lane;  // 16-byte position in the tile
      // K: key row r, logical chunk c (the swizzle of swz)
      const int r = pos >> 3, c = (pos & 7) ^ ((r >> 1) & 7);
      koff[j] = (uint32_t)(((r % P) * kHeadDim + c * 8) * 2);
      // V^T: dim row d, chunk u of the page block (the inverse of the V^T layout)
      const int e = pos % (CPP * 64), d = e / CPP, u = (e % CPP) ^ ((d / R) % CPP);
      voff[j] = (uint32_t)((d * P + u * 8) * 2);
    }
  }
  // scalar loads through the constant address space (the gather list is
  // not written during the launch): no vector registers, and nothing for the
  // vector-memory counter, which then tracks the tile data alone
  __device__ void fetch(const AttnArgs& a, int tile, Ids& x) const {
    x.pg = load_uniform<EPT>(a.sel_page + tile * EPT);
    x.ln = load_uniform<EPT>(a.sel_len + tile * EPT);
  }
  // the tile's data: one scalar base per pool, lane offsets from init
  __device__ void issue(const char* kpool, const char* vpool, const Ids& x, char* buf, int /*wave*/) {
    typedef __attribute__((address_space(3))) void lds_t;
    const uint64_t off = (uint64_t)(uint32_t)pick(x.pg, pw) * page_bytes + head_off;
    const char* kb = kpool + off;
    const char* vb = vpool + off;
    // (the 32-bit offsets are pinned here so that each load takes the scalar
    // base and the offset as they are, not a 64-bit sum made in vector registers)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      asm volatile("" : "+v"(koff[j]));
      __builtin_amdgcn_global_load_lds(kb + koff[j], (lds_t*)(buf + (w * 2 + j) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      asm volatile("" : "+v"(voff[j]));
      __builtin_amdgcn_global_load_lds(vb + voff[j], (lds_t*)(buf + KBYTES + (w * 2 + j) * 1024), 16, 0, 0);
    }
  }
};

// Row sums of P on the matrix cores, from the same rounded values the P.V
// product uses.  A P^T operand (16 keys x 32 queries) gives lane (l32, hi)
// eight keys of query l32.  In a 16x16x32 product lane l supplies row l % 16
// (A) or column l % 16 (B) of lane group l / 16, and holds rows
// 4 * (l / 16) .. + 3 of column l % 16 of the result.  With A row m set to
// one over lane groups g where g % 2 == (m / 4) % 2, column n of result row m
// sums the keys of query n + 16 * ((m / 4) % 2) held by both halves of the
// wave, so every lane's result (all four registers alike) is the sum over
// the operand's 16 keys of its own query l32.
__device__ inline bf16x8 rowsum_selector(int lane) {
  const bf16 v = (bf16)((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 1.f : 0.f);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = v;
  return r;
}
__device__ inline floatx4 rowsum_mma(bf16x8 sel, bf16x8 p, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p, acc, 0, 0, 0);
}

// s_waitcnt on the vector-memory count only (vmcnt <= N, N < 16): bits 3:0
// vmcnt, 6:4 expcnt (7: no wait), 11:8 lgkmcnt (15: no wait), 15:14 the high
// vmcnt bits (0 here)
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// s_waitcnt on the scalar-memory / LDS count only (lgkmcnt 0; vmcnt 63 and
// expcnt 7: no wait)
__device__ inline void wait_smem() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// max over the two 32-lane halves of the wave
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup -> (head, split, q tile) and its tile range [t0, t1); false for a
// workgroup past the work.  Dispatch is round-robin over the XCDs, each with
// its own L2.  With H a multiple of 8, all workgroups of a head run on one XCD
// (XCD = h % 8), so both its K/V pages and each q tile's queries come from HBM
// once and are shared through that L2; the q tiles of one split are
// dispatched consecutively.  Otherwise the q tiles of one (head, split) share
// an XCD.
//
// Split sizes (head-major, S even): the even splits of every (head, q tile)
// are dispatched first, as the first workgroup of their CU, and hold
// tiles_per_split tiles; the odd ones come second and hold t_odd.  Two
// workgroups share a CU and the first one dispatched issues ahead of the
// other, so uneven splits let both finish together.  Boundaries depend only
// on the launch parameters: results stay deterministic.
__device__ inline bool attn_place(const AttnArgs& a, int& h, int& split, int& qt, int& t0, int& t1) {
  const int b = blockIdx.x;
  const int xcd = b % kNumXcd, kx = b / kNumXcd;
  if (a.head_major) {
    const int per = a.S * a.n_qtiles;              // workgroups of one head
    const int nh = (a.H + kNumXcd - 1) / kNumXcd;  // heads on this XCD
    if (a.t_odd > 0) {
      const int halfw = nh * per / 2;              // even (then odd) splits of all those heads
      const int odd = kx / halfw, r = kx % halfw, j = r % (per / 2);
      h = xcd + kNumXcd * (r / (per / 2));
      split = 2 * (j / a.n_qtiles) + odd;
      qt = j % a.n_qtiles;
    } else {
      const int j = kx % per;
      h = xcd + kNumXcd * (kx / per);
      split = j / a.n_qtiles;
      qt = j % a.n_qtiles;
    }
    if (h >= a.H) return false;
  } else {
    const int unit = (kx / a.n_qtiles) * kNumXcd + xcd;
    if (unit >= a.n_units) return false;
    qt = kx % a.n_qtiles;
    h = unit / a.S;
    split = unit % a.S;
  }
  t0 = a.t_odd > 0 ? (split >> 1) * (a.tiles_per_split + a.t_odd) + (split & 1) * a.tiles_per_split
                   : split * a.tiles_per_split;
  t1 = min(a.n_tiles, t0 + ((split & 1) && a.t_odd > 0 ? a.t_odd : a.tiles_per_split));
  return true;
}

// float32 paged attention (the float32 cache): 4 waves x 32 queries of one
// head per workgroup, over one split of the gather list.  Per 64-key tile, K
// (64 keys x 64 dims) and V^T (64 dims x 64 keys) are staged in LDS (two
// buffers, each thread's next chunks held in registers), then each wave
// computes S^T = K Q^T with 32x32x2 MFMAs, one query column per lane, and
// O^T += V^T P^T from the S^T accumulators.  Scores, lazy offsets and masks as
// described in k_attn_bf.
template <int P>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  using M = Mfma<float>;
  using Frag = float;
  using L = TileLoader<float, P>;
  constexpr int NDC = kHeadDim / 2;  // MFMAs along the head dim
  constexpr int NCH = 16;            // P^T operands per 32-key block
  constexpr int QPW = 32;            // queries per wave
  constexpr int VOFF = kKeysPerTile * L::KP;  // V^T within a buffer
  __shared__ __attribute__((aligned(16))) float lt[2][L::TILE_ELEMS];

  int h, split, qt, t0, t1;
  if (!attn_place(a, h, split, qt, t0, t1)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qbase = (qt * kWaves + wave) * QPW;

  Frag qf[1][NDC];
  load_q(a, qbase, h, l32, hi, qf);
  floatx16 o[2] = {zero16(), zero16()};
  const float qs = a.qk_scale;
  constexpr float kNoKey = -1e20f;
  constexpr float kMaxBlockSum = 65536.f;
  constexpr float kRaise = 8.f;
  float m = kNoKey, nm = -kNoKey, l = 0.f;

  // one 32-key block kb of the tile in LDS: K at ck, V^T at cv, entry lengths tl
  auto block = [&](const float* ck, const float* cv, const i32x4& tl, int kb) {
    const bool partial = tile_partial<P>(tl);
    auto qk = [&]() {
      floatx16 s = partial ? M::mma_seed(M::mask_a(key_masked<P>(tl, kb * 32 + l32), hi), M::mask_b(hi))
                           : zero16();
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) s = M::mma(read_k(ck, L::KP, kb * 32 + l32, dc, hi), qf[0][dc], s);
      return s;
    };
    auto expo = [&](floatx16& s) {
      float ts = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], qs, nm));
        ts += s[r];
      }
      return ts;
    };
    floatx16 s = qk();
    float ts = expo(s);
    if (__any(!(ts <= kMaxBlockSum))) {
      s = qk();
      float x = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, s[r]);
      const float mx = half_swap_max(x) * qs;
      if (mx > m + kRaise) {
        const float alpha = __builtin_amdgcn_exp2f(m - mx);
        m = mx;
        nm = -mx;
        o[0] *= alpha;
        o[1] *= alpha;
        l *= alpha;
      }
      ts = expo(s);
    }
    l += ts;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] = M::mma(read_v(cv, L::VP, db * 32 + l32, kb, ch, hi), s[ch], o[db]);
  };

  const int n = max(t1 - t0, 0);
  L ld;
  ld.init((const float*)a.kpool, (const float*)a.vpool, h, a.H, tid);
  if (n > 0) {
    ld.fetch_pages(a, t0, tid);
    ld.fetch_data(tid);
    ld.fetch_pages(a, t0 + 1, tid);
    ld.store(lt[t0 & 1], tid);
  }
  i32x4 cur_lens = ld.dlen;  // entry lengths of the tile in LDS
  __syncthreads();
  for (int tile = t0; tile < t1; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < t1;
    if (more) {
      ld.fetch_data(tid);                         // tile + 1, lands during this tile's math
      ld.fetch_pages(a, tile + 2, tid);           // page ids two tiles ahead
    }
    block(lt[buf], lt[buf] + VOFF, cur_lens, 0);
    block(lt[buf], lt[buf] + VOFF, cur_lens, 1);
    // the other buffer was last read in the previous tile, before its barrier
    if (more) ld.store(lt[buf ^ 1], tid);
    cur_lens = ld.dlen;
    __syncthreads();
  }

  // each lane summed P over its own half of the keys; both halves share m
  l += __shfl_xor(l, 32);
  const int q = qbase + l32;
  if (q >= a.Tq) return;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse = empty ? -INFINITY : m * 0.69314718f + __logf(l);  // m is in log2 units
  const size_t row = (size_t)q * a.H + h;
  // O^T accumulators hold dims db*32 + 8*(r/4) + 4*hi + r%4
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + hi * 4;
      floatx4 v;
      v[0] = o[db][g * 4 + 0] * inv;
      v[1] = o[db][g * 4 + 1] * inv;
      v[2] = o[db][g * 4 + 2] * inv;
      v[3] = o[db][g * 4 + 3] * inv;
      if (a.S > 1) {
        *(floatx4*)(a.o_part + ((size_t)split * a.Tq * a.H + row) * kHeadDim + d) = v;
      } else if (a.out_bf16) {
        bf16x4 w;
        w[0] = (bf16)v[0]; w[1] = (bf16)v[1]; w[2] = (bf16)v[2]; w[3] = (bf16)v[3];
        *(bf16x4*)((bf16*)a.out + row * kHeadDim + d) = w;
      } else {
        *(floatx4*)((float*)a.out + row * kHeadDim + d) = v;
      }
    }
  if (hi == 0) {
    if (a.S > 1) a.lse_part[(size_t)split * a.Tq * a.H + row] = lse;
    else if (a.lse) a.lse[row] = lse;
  }
}

// Epilogue of the bf16 attention: O normalized by the row sum l (each lane
// holds both halves' sums), written to the output with the LSE, or, with
// S > 1, to this split's partial.  Partials go out through LDS (free once
// every wave is past its last tile and no tile load is still landing): each
// wave stages its 64 queries x 32 dims of one half of the head dim as
// swizzled 128-byte rows, then every store instruction writes 8 whole
// 128-byte lines instead of 32-byte pieces of 32 rows.
__device__ inline void attn_epilogue_bf(const AttnArgs& a, const floatx16 (&o)[2][2], const float (&m)[2],
                                        const float (&l)[2], int split, int qbase, int h, int l32, int hi,
                                        int lane, int wave, char* lds) {
  constexpr int NQB = 2, QPW = 64;
  float inv[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) inv[qb] = l[qb] > 0.f ? 1.f / l[qb] : 0.f;
  if (a.S > 1) {
    __syncthreads();
    char* st = lds + wave * (QPW * 32 * 4);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          floatx4 v;
          v[0] = o[db][qb][g * 4 + 0] * inv[qb];
          v[1] = o[db][qb][g * 4 + 1] * inv[qb];
          v[2] = o[db][qb][g * 4 + 2] * inv[qb];
          v[3] = o[db][qb][g * 4 + 3] * inv[qb];
          *(floatx4*)(st + swz(qb * 32 + l32, 2 * g + hi)) = v;
        }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int it = 0; it < QPW / 8; ++it) {
        const int row = it * 8 + (lane >> 3), c = lane & 7;
        const floatx4 v = *(const floatx4*)(st + swz(row, c));
        const int q = qbase + row;
        if (q < a.Tq)
          *(floatx4*)(a.o_part + (((size_t)split * a.Tq + q) * a.H + h) * kHeadDim + db * 32 + c * 4) = v;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int q = qbase + qb * 32 + l32;
      if (q < a.Tq && hi == 0)
        a.lse_part[((size_t)split * a.Tq + q) * a.H + h] =
            l[qb] > 0.f ? m[qb] * 0.69314718f + __logf(l[qb]) : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int q = qbase + qb * 32 + l32;
    if (q >= a.Tq) continue;
    const float lse = l[qb] > 0.f ? m[qb] * 0.69314718f + __logf(l[qb]) : -INFINITY;  // m in log2 units
    const size_t row = (size_t)q * a.H + h;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hi * 4;
        floatx4 v;
        v[0] = o[db][qb][g * 4 + 0] * inv[qb];
        v[1] = o[db][qb][g * 4 + 1] * inv[qb];
        v[2] = o[db][qb][g * 4 + 2] * inv[qb];
        v[3] = o[db][qb][g * 4 + 3] * inv[qb];
        if (a.out_bf16) {
          bf16x4 w;
          w[0] = (bf16)v[0]; w[1] = (bf16)v[1]; w[2] = (bf16)v[2]; w[3] = (bf16)v[3];
          *(bf16x4*)((bf16*)a.out + row * kHeadDim + d) = w;
        } else {
          *(floatx4*)((float*)a.out + row * kHeadDim + d) = v;
        }
      }
    if (hi == 0 && a.lse) a.lse[row] = lse;
  }
}

// ---------------------------------------------------------------------------
// bf16 paged attention, software-pipelined over 32-key blocks.
//
// Workgroup shape, mapping and splits as in k_attn.  Step j of a wave issues,
// independently of one another, the P.V MFMAs of key block j - 1, the
// softmax of block j (scaling, exponentials and packing on the VALU, the row
// sums on the matrix cores) and the K.Q^T MFMAs of block j + 1, interleaved
// one MFMA to five VALU instructions, so that the matrix and vector pipes of
// a SIMD stay busy together.  Every LDS
// operand is read at least four groups before its MFMA: the step's K
// fragments at its start (the P.V MFMAs come first), the V^T fragments of the
// next step's P.V during this step's K.Q^T.  Block j's sums are checked at
// the end of step j, before its P.V in step j + 1.  A 64-key tile (two
// blocks) is read for its K from the step before its first block's softmax
// and for its V^T until the step of its last one: two tiles are in use, one
// is landing and a fourth buffer is being filled.  Tiles go straight from
// memory into four LDS buffers (global_load_lds), issued three tiles ahead,
// with one barrier per tile.
template <int P>
__global__ __launch_bounds__(256, 2) void k_attn_bf(AttnArgs a) {
  using M = Mfma<bf16>;
  using Frag = bf16x8;
  using DL = DmaLoader<P>;
  constexpr int NQB = 2, NDC = 4, NCH = 2;
  constexpr int BB = DL::BUF_BYTES;
  __shared__ __attribute__((aligned(16))) char lt[4 * BB];

  int h, split, qt, t0, t1;
  if (!attn_place(a, h, split, qt, t0, t1)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qbase = (qt * kWaves + wave) * 64;
  // bf16 1.0 in the lanes that hold column 0 of a mask-product A operand, else
  // 0: that operand is the key's mask bit times this (M::mask_a in two instructions)
  const int one_hi = hi == 0 ? M::bits(1.f) : 0;
  const Frag sel = rowsum_selector(lane);
  TileAddr<P> ta;
  ta.init(l32, hi);

  Frag qf[NQB][NDC];
  load_q(a, qbase, h, l32, hi, qf);
  floatx16 o[2][NQB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NQB; ++j) o[i][j] = zero16();
  // scores, lazy offsets and masks as in k_attn
  const float qs = a.qk_scale;
  constexpr float kNoKey = -1e20f;
  constexpr float kMaxBlockSum = 65536.f;
  constexpr float kRaise = 8.f;
  float m[NQB], l[NQB], nm[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = kNoKey;
    nm[qb] = -kNoKey;
    l[qb] = 0.f;
  }

  const int n = max(t1 - t0, 0);
  if (n > 0) {
    DL ld;
    ld.init(h, a.H, tid);
    const char* kp = (const char*)a.kpool;
    const char* vp = (const char*)a.vpool;
    // buffer of the split's i-th tile (i counted from t0): with the tile
    // loop unrolled four times every buffer offset is a constant
    auto buf = [&](int i) __attribute__((always_inline)) { return lt + (i & 3) * BB; };
    // mask bits of a tile: bit kb set when key kb*32 + l32 is masked
    // the same per block for the whole wave: bit kb set when block kb has a masked key
    auto sminfo = [&](const typename DL::Ids& x) __attribute__((always_inline)) {
      return (block_masked<P>(x.ln, 0) ? 1 : 0) | (block_masked<P>(x.ln, 1) ? 2 : 0);
    };
    auto minfo = [&](const typename DL::Ids& x) __attribute__((always_inline)) {
      int r = 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) r |= key_masked<P>(x.ln, kb * 32 + l32) ? 1 << kb : 0;
      return r;
    };
    auto ready = [](typename DL::Ids& x) __attribute__((always_inline)) { asm volatile("" : "+s"(x.pg), "+s"(x.ln)); };

    // raw scores of key block kb of the tile in buffer b (mask bits mi)
    auto qk_raw = [&](const char* b, int kb, int mi, floatx16 (&s)[NQB]) __attribute__((always_inline)) {
      Frag kf[NDC];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) kf[dc] = ta.kop(b, kb, dc);
      u32x2 sw = {(uint32_t)(-((mi >> kb) & 1) & one_hi), 0u};
      const floatx16 s0 = M::mma_seed(__builtin_bit_cast(typename M::Seed, sw), M::mask_b(hi));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = M::mma(kf[0], qf[qb][0], s0);
#pragma unroll
        for (int dc = 1; dc < NDC; ++dc) s[qb] = M::mma(kf[dc], qf[qb][dc], s[qb]);
      }
    };
    auto softmax = [&](floatx16 (&s)[NQB], Frag (&p)[NCH][NQB], floatx4 (&ts)[NQB]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], qs, nm[qb]));
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) p[ch][qb] = pack_p(s[qb], ch, bf16());
        ts[qb] = rowsum_mma(sel, p[1][qb], rowsum_mma(sel, p[0][qb], floatx4{0.f, 0.f, 0.f, 0.f}));
      }
    };
    // One step: P.V of pV with the V^T fragments vfc (read during the
    // previous step), softmax of sS into pS, K.Q^T of block qkb of buffer
    // qbuf into sQ (mask bits qmi per lane, smi per wave), and the V^T
    // fragments of the next step's P.V (block nvkb of buffer nvbuf) into vfn.
    // Issued in 17 groups of five VALU instructions of the softmax (two
    // elements: their scaled logits and exponentials, one bf16 pack), each but
    // group 8 with an MFMA, kept in this order by scheduling barriers: the
    // eight P.V MFMAs first, while this step's K fragments land, then the
    // K.Q^T MFMAs while the next V^T fragments land.  The row sums of the new
    // P go to the matrix cores as well, one 16x16x32 product per packed
    // operand, a group after its last pack.  A block with a masked key adds
    // the mask product to its scores at the end.
    auto step = [&](const char* qbuf, int qkb, int qmi, int smi, const Frag (&vfc)[NCH][2], const char* nvbuf, int nvkb,
                    Frag (&vfn)[NCH][2], floatx16 (&sQ)[NQB], floatx16 (&sS)[NQB], Frag (&pS)[NCH][NQB],
                    const Frag (&pV)[NCH][NQB], floatx4 (&ts)[NQB]) __attribute__((always_inline)) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      Frag kf[NDC];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) kf[dc] = ta.kop(qbuf, qkb, dc);
      // softmax work of group g: the scaled logits and exponentials of
      // elements 2i, 2i + 1 of query block qb = g / 8 (pair g) and the bf16
      // pack of pair g - 1 (its exponentials issued a group earlier), so that
      // no instruction waits on the one before it; pair 15's pack closes the step
      float xe[2];
      bf16x2 pk;
      auto valu = [&](int g) __attribute__((always_inline)) {
        float xn[2];
        if (g < 16) {
          const int qb = g >> 3, i = g & 7;
          xn[0] = __builtin_fmaf(sS[qb][2 * i], qs, nm[qb]);
          xn[1] = __builtin_fmaf(sS[qb][2 * i + 1], qs, nm[qb]);
        }
        if (g > 0 && g < 17) {
          const int gp = g - 1, qb = gp >> 3, i = gp & 7, ch = i >> 2, k = i & 3;
          bf16x2 pr;
          pr[0] = (bf16)xe[0];
          pr[1] = (bf16)xe[1];
          // the pack stays in this group (it would otherwise sink to the
          // end of the step, past the sum check)
          uint32_t u = __builtin_bit_cast(uint32_t, pr);
          asm volatile("" : "+v"(u));
          pk = __builtin_bit_cast(bf16x2, u);
          pS[ch][qb][2 * k] = pk[0];
          pS[ch][qb][2 * k + 1] = pk[1];
        }
        if (g < 16) {
          xe[0] = __builtin_amdgcn_exp2f(xn[0]);
          xe[1] = __builtin_amdgcn_exp2f(xn[1]);
        }
      };
      // groups 0 .. 7: P.V
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int c = g >> 2, db = (g >> 1) & 1, qb = g & 1;
        o[db][qb] = M::mma(vfc[c][db], pV[c][qb], o[db][qb]);
        // pairs 0-3 (query block 0, keys of chunk 0) were packed in group 4
        if (g == 5) ts[0] = rowsum_mma(sel, pS[0][0], floatx4{0.f, 0.f, 0.f, 0.f});
        valu(g);
        __builtin_amdgcn_sched_barrier(0);
      }
      // group 8: softmax work only
      valu(8);
      __builtin_amdgcn_sched_barrier(0);
      // groups 9 .. 16: K.Q^T from zero, the next V^T fragments read in the first four
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int dc = g >> 1, qb = g & 1;
        sQ[qb] = dc == 0 ? M::mma(kf[dc], qf[qb][dc], zero16()) : M::mma(kf[dc], qf[qb][dc], sQ[qb]);
        if (g == 0) ts[0] = rowsum_mma(sel, pS[1][0], ts[0]);
        if (g == 4) ts[1] = rowsum_mma(sel, pS[0][1], floatx4{0.f, 0.f, 0.f, 0.f});
        if (g < 7) valu(g + 9);
        if (g < 4) {
          const int c = g >> 1, db = g & 1;
          vfn[c][db] = ta.vop(nvbuf + DL::KBYTES, db, nvkb, c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      valu(16);
      __builtin_amdgcn_sched_barrier(0);
      ts[1] = rowsum_mma(sel, pS[1][1], ts[1]);
      // a block with masked keys (wave-uniform): the mask product added to
      // both query blocks' scores, pushing masked keys to about -1e30
      if ((smi >> qkb) & 1) {
        u32x2 sw = {(uint32_t)(-((qmi >> qkb) & 1) & one_hi), 0u};
        const typename M::Seed sa = __builtin_bit_cast(typename M::Seed, sw), sb = M::mask_b(hi);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sQ[qb] = M::mma_seed_acc(sa, sb, sQ[qb]);
      }
    };
    // the sum check of block kb of buffer b after its softmax: if the sum of
    // some query's P over the block exceeds 2^16, the block's raw scores again (its tile is still in
    // LDS), m raised to the block max where that exceeds it by more than
    // kRaise (O and l rescaled), then the softmax again
    auto settle = [&](const char* b, int kb, int mi, floatx16 (&s)[NQB], Frag (&p)[NCH][NQB], floatx4 (&ts)[NQB])
        __attribute__((always_inline)) {
      bool bad = false;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) bad = bad || !(ts[qb][0] <= kMaxBlockSum);
      if (__any(bad)) {
        qk_raw(b, kb, mi, s);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float x = s[qb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) x = fmaxf(x, s[qb][r]);
          const float mx = half_swap_max(x) * qs;  // masked keys sit near -1e30 * qs < kNoKey
          if (mx > m[qb] + kRaise) {
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mx);
            m[qb] = mx;
            nm[qb] = -mx;
            o[0][qb] *= alpha;
            o[1][qb] *= alpha;
            l[qb] *= alpha;
          }
        }
        softmax(s, p, ts);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) l[qb] += ts[qb][0];
    };

    // Prologue: page ids and lengths of tiles t0 .. t0 + 3, then the data of
    // t0 .. t0 + 2.  From then on every tile period issues the ids of tile
    // t + 4 (scalar loads, used a period later) and then tile t + 3's data
    // (four vector-memory loads) after its barrier, so waiting for all but
    // the last four vector-memory operations before the next barrier leaves
    // only the newest tile's data in flight: the tile needed next has landed.
    typename DL::Ids ida, idb, idc, idd;
    ld.fetch(a, t0, ida);
    ld.fetch(a, t0 + 1, idb);
    ld.fetch(a, t0 + 2, idc);
    ld.fetch(a, t0 + 3, idd);
    // the ids only: the queries' vector loads land with tile t0's (loads
    // return in order, and the queries were issued first)
    wait_smem();
    ready(ida);
    ready(idb);
    ready(idc);
    ready(idd);
    asm volatile("" ::: "memory");
    ld.issue(kp, vp, ida, buf(0), wave);
    ld.issue(kp, vp, idb, buf(1), wave);
    ld.issue(kp, vp, idc, buf(2), wave);
    // mask bits of tiles t, t + 1, t + 2 in bits 0-1, 2-3, 4-5
    int mr = minfo(ida) | minfo(idb) << 2 | minfo(idc) << 4;
    int smr = sminfo(ida) | sminfo(idb) << 2 | sminfo(idc) << 4;
    idb = idd;  // the ids of tile t0 + 3, used in the first period
    asm volatile("" ::: "memory");
    wait_vmem<2 * DL::NISSUE>();  // the queries and tile t0 have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    floatx16 s0[NQB], s1[NQB];
    Frag p0[NCH][NQB], p1[NCH][NQB];
    Frag va[NCH][2], vb[NCH][2];  // V^T fragments of the next P.V, read a step ahead
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) p1[ch][qb] = Frag{};  // the P.V of step 0 adds nothing
    floatx4 ts[NQB];
    qk_raw(buf(0), 0, mr & 3, s0);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int db = 0; db < 2; ++db) va[c][db] = ta.vop(buf(0) + DL::KBYTES, db, 1, c);

    // one tile period; `use` holds the ids of tile t + 3, `next` receives those of t + 4
    auto period = [&](int i, typename DL::Ids& use, typename DL::Ids& next) __attribute__((always_inline)) {
      const int t = t0 + i;
      // step 2i: P.V of block 1 of tile t - 1 (of tile t with P = 0 in the
      // first step), softmax of block 0 of tile t, QK of block 1 of tile t;
      // reads the V^T of block 0 of tile t for the next step
      step(buf(i), 1, mr & 3, smr & 3, va, buf(i), 0, vb, s1, s0, p0, p1, ts);
      settle(buf(i), 0, mr & 3, s0, p0, ts);
      // tile t + 1 has landed; tile t - 1's buffer is free: ids of tile t + 4,
      // data of tile t + 3 (past the split's end they are read and unused)
      asm volatile("" ::: "memory");
      wait_vmem<DL::NISSUE>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      ready(use);
      ld.fetch(a, t + 4, next);
      ld.issue(kp, vp, use, buf(i + 3), wave);
      mr |= minfo(use) << 6;
      smr |= sminfo(use) << 6;
      asm volatile("" ::: "memory");
      // step 2i + 1: P.V of block 0 of tile t, softmax of block 1 of tile t,
      // QK of block 0 of tile t + 1; reads the V^T of block 1 of tile t
      step(buf(i + 1), 0, (mr >> 2) & 3, (smr >> 2) & 3, vb, buf(i), 1, va, s0, s1, p1, p0, ts);
      settle(buf(i), 1, mr & 3, s1, p1, ts);
      mr >>= 2;
      smr >>= 2;
    };
    // after the prologue idb holds the ids of tile t0 + 3
    for (int i = 0; i < n; i += 4) {
      period(i, idb, ida);
      if (i + 1 < n) period(i + 1, ida, idb);
      if (i + 2 < n) period(i + 2, idb, ida);
      if (i + 3 < n) period(i + 3, ida, idb);
    }
    // the last block's P.V (its V^T fragments read by the last step)
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) o[db][qb] = M::mma(va[ch][db], p1[ch][qb], o[db][qb]);
    // the loads issued past the last tile land before the workgroup's LDS is reused
    wait_vmem<0>();
  }

  attn_epilogue_bf(a, o, m, l, split, qbase, h, l32, hi, lane, wave, lt);
}

// Split merge: 16 threads per (token, head) row, 4 dims each; all partial
// loads of a thread are independent and issued together.
constexpr int kMaxSplitsDev = 16;

__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  int d = (threadIdx.x & 15) * 4;
  if (row >= a.rows) return;
  // every split's lse and partial are loaded at once (one memory round
  // trip); an empty split (lse = -inf, partial 0) gets weight 0
  float ls[kMaxSplitsDev];
  floatx4 v[kMaxSplitsDev];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplitsDev; ++s) {
    if (s < a.S) {
      ls[s] = a.lse_part[(size_t)s * a.rows + row];
      v[s] = *(const floatx4*)(a.o_part + ((size_t)s * a.rows + row) * kHeadDim + d);
    } else {
      ls[s] = -INFINITY;
      v[s] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int s = 0; s < kMaxSplitsDev; ++s) mx = fmaxf(mx, ls[s]);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplitsDev; ++s) {
    const float w = ls[s] == -INFINITY ? 0.f : __expf(ls[s] - mx);
    sum += w;
    acc[0] = __builtin_fmaf(w, v[s][0], acc[0]);
    acc[1] = __builtin_fmaf(w, v[s][1], acc[1]);
    acc[2] = __builtin_fmaf(w, v[s][2], acc[2]);
    acc[3] = __builtin_fmaf(w, v[s][3], acc[3]);
  }
  float inv = 1.f / sum;
  acc[0] *= inv; acc[1] *= inv; acc[2] *= inv; acc[3] *= inv;
  if (a.out_bf16) {
    bf16x4 w;
    w[0] = (bf16)acc[0]; w[1] = (bf16)acc[1]; w[2] = (bf16)acc[2]; w[3] = (bf16)acc[3];
    *(bf16x4*)((bf16*)a.out + (size_t)row * kHeadDim + d) = w;
  } else {
    *(floatx4*)((float*)a.out + (size_t)row * kHeadDim + d) = acc;
  }
  if (d == 0 && a.lse) a.lse[row] = mx + __logf(sum);
}

}  // namespace

hipError_t launch_append(int dtype, const AppendArgs& a, hipStream_t s) {
  dim3 grid(a.ppf, a.H);
  if (dtype) hipLaunchKernelGGL(k_append<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_append<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_batch(int dtype, const AppendBatch& b, hipStream_t s) {
  if (b.n < 1 || b.n > kMaxAppendBatch) return hipErrorInvalidValue;
  dim3 grid(b.a.ppf * b.n, b.a.H);
  if (dtype) hipLaunchKernelGGL(k_append_batch<bf16>, grid, dim3(256), 0, s, b);
  else hipLaunchKernelGGL(k_append_batch<float>, grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_evict(int dtype, const EvictArgs& a, hipStream_t s) {
  dim3 grid(a.H * evict_groups(a.C));
  if (dtype) hipLaunchKernelGGL(k_evict<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_evict<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.n_write <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_select, dim3((a.n_write + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_update(int dtype, const AppendArgs* ap, const EvictArgs* ev, const RopeArgs* ra,
                         const SelectArgs* sa, hipStream_t s) {
  AppendArgs a0{};
  EvictArgs e0{};
  RopeArgs r0{};
  SelectArgs s0{};
  const int na = ap ? ap->ppf * ap->H : 0;
  const int ne = ev ? ev->H * evict_groups(ev->C) : 0;
  const int nr = ra ? (int)(((dtype ? rope_chunks<bf16>(*ra) : rope_chunks<float>(*ra)) + 255) / 256) : 0;
  const int ns = sa ? (sa->n_write + 255) / 256 : 0;
  const int nb = na + ne + nr + ns;
  if (nb == 0) return hipSuccess;
  if (dtype)
    hipLaunchKernelGGL(k_update<bf16>, dim3(nb), dim3(256), 0, s, ap ? *ap : a0, ev ? *ev : e0, ra ? *ra : r0,
                       sa ? *sa : s0, na, ne, nr);
  else
    hipLaunchKernelGGL(k_update<float>, dim3(nb), dim3(256), 0, s, ap ? *ap : a0, ev ? *ev : e0, ra ? *ra : r0,
                       sa ? *sa : s0, na, ne, nr);
  return hipGetLastError();
}

hipError_t launch_prepare(int dtype, const SelectArgs& sa, const RopeArgs& ra, hipStream_t s) {
  int sel_blocks = (sa.n_write + 255) / 256;
  size_t chunks = dtype ? rope_chunks<bf16>(ra) : rope_chunks<float>(ra);
  int rope_blocks = (int)((chunks + 255) / 256);
  dim3 grid(sel_blocks + rope_blocks);
  if (dtype) hipLaunchKernelGGL(k_prepare<bf16>, grid, dim3(256), 0, s, sa, ra, sel_blocks);
  else hipLaunchKernelGGL(k_prepare<float>, grid, dim3(256), 0, s, sa, ra, sel_blocks);
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, const AttnArgs& a, hipStream_t s) {
  int groups = (a.n_units + kNumXcd - 1) / kNumXcd;
  dim3 grid(groups * kNumXcd * a.n_qtiles);
  switch (dtype * 100 + a.P) {
    case 116: hipLaunchKernelGGL((k_attn_bf<16>), grid, dim3(256), 0, s, a); break;
    case 132: hipLaunchKernelGGL((k_attn_bf<32>), grid, dim3(256), 0, s, a); break;
    case 164: hipLaunchKernelGGL((k_attn_bf<64>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_attn<16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_attn<32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_attn<64>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.S > kMaxSplitsDev) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_merge, dim3((a.rows + 15) / 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope(int dtype, const RopeArgs& a, hipStream_t s) {
  size_t chunks = dtype ? rope_chunks<bf16>(a) : rope_chunks<float>(a);
  dim3 grid((unsigned)((chunks + 255) / 256));
  if (dtype) hipLaunchKernelGGL(k_rope<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_rope<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ring_init(int32_t* ring, const int32_t* init, int N, hipStream_t s) {
  hipLaunchKernelGGL(k_ring_init, dim3((N + 255) / 256), dim3(256), 0, s, ring, init, N);
  return hipGetLastError();
}

}  // namespace gca
