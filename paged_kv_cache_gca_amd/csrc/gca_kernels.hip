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
//             scaled to base-2 logits, rounded once) in one launch
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
// tokens sit at row 0, column 0.

// cos/sin of pairs `pair` and `pair` + 1 (pair even) in one 16-byte load: the
// axis blocks have an even number of pairs (12, 10, 10 for D = 64), so both
// lie next to each other in one table, at a 16-byte aligned offset.
__device__ inline float4 rope_cs2(const RopeTabs& R, int64_t frame, int tok, int pair) {
  const float2* p;
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
  return *(const float4*)p;
}

// One fixed operation sequence, so every kernel that rotates gives the same bits.
__device__ inline void rotate(float x0, float x1, float2 cs, float& y0, float& y1) {
  float a = x1 * cs.y;
  float b = x1 * cs.x;
  y0 = __builtin_fmaf(x0, cs.x, -a);
  y1 = __builtin_fmaf(x0, cs.y, b);
}

// Rotated values times `scale` (exact for scale = 1), rounded once to T.
template <typename T>
__device__ inline void rotate_chunk(Vec16<T>& v, const RopeTabs& R, int64_t frame, int tok,
                                    int first_pair, float scale = 1.f) {
  constexpr int EPC = 16 / sizeof(T);
#pragma unroll
  for (int m = 0; m < EPC / 2; m += 2) {
    const float4 c4 = rope_cs2(R, frame, tok, first_pair + m);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float2 cs = u ? make_float2(c4.z, c4.w) : make_float2(c4.x, c4.y);
      float y0, y1;
      rotate(to_f(v.e[2 * (m + u)]), to_f(v.e[2 * (m + u) + 1]), cs, y0, y1);
      v.e[2 * (m + u)] = from_f<T>(y0 * scale);
      v.e[2 * (m + u) + 1] = from_f<T>(y1 * scale);
    }
  }
}

// 16-byte chunk c of x -> y: rotated when a.rotate, times a.scale, rounded
// once; chunks past the tensor are ignored
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
  if (a.rotate) {
    rotate_chunk<T>(v, a.tabs, a.frame + row / a.T, tok, part * EPC / 2, a.scale);
  } else {
#pragma unroll
    for (int i = 0; i < EPC; ++i) v.e[i] = from_f<T>(to_f(v.e[i]) * a.scale);
  }
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
      if (a.rope) rotate_chunk<T>(kv, a.tabs, a.frame, tok, part * EPC / 2);
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
  const size_t fe = (size_t)a.T * a.H * kHeadDim;
  a.k = (const T*)b.a.k + j * fe;
  a.v = (const T*)b.a.v + j * fe;
  a.ring_pos = b.a.ring_pos + (int64_t)j * a.ppf;
  a.frame = b.a.frame + j;
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
// Workgroup = 4 waves x 64 queries of one head, over one split of the gather
// list.  Per 64-key tile: K (64 keys x 64 dims) and V^T (64 dims x 64 keys)
// are staged in LDS, then each wave computes S^T = K Q^T (keys x queries) with
// 32x32 MFMA blocks, so that each lane owns one query column: the softmax max
// and scaling are per lane plus one exchange with lane ^ 32.  P^T is fed
// straight from the S^T accumulators as the B operand of O^T = V^T P^T; the
// key order inside each 16-key chunk follows the accumulator layout, and the
// V^T operand is read in the same order.  Row sums are dot products of the
// same rounded P with ones, so sum(P) and P.V use identical weights.

template <typename T>
struct Mfma;
typedef short shortx4 __attribute__((ext_vector_type(4)));

// Seed operands: a rank-2 product fills a 32x32 S^T accumulator before the
// K.Q^T MFMAs.  A holds, per key row, 1 in column 0 and the key's mask (1 for
// a key past its page's valid length, else 0) in column 1; B holds, per query
// column, the offset x in row 0 and -1e30 in row 1.  The product is x for a
// valid key and x - 1e30 (exp2 of which is 0) for a masked one.
constexpr float kMaskedScore = -1e30f;

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
  __device__ static inline Seed seed_a(float mask, int hi) {
    Seed r = {0, 0, 0, 0};
    if (hi == 0) {
      r[0] = bits(1.f);
      r[1] = bits(mask);
    }
    return r;
  }
  __device__ static inline Seed seed_b(float x, int hi) {
    Seed r = {0, 0, 0, 0};
    if (hi == 0) {
      r[0] = bits(x);
      r[1] = bits(kMaskedScore);
    }
    return r;
  }
  __device__ static inline floatx16 mma_seed(Seed a, Seed b) {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, z, 0, 0, 0);
  }
  // nearest value the seed operand holds exactly
  __device__ static inline float exact(float x) { return (float)(bf16)x; }
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
  __device__ static inline Seed seed_a(float mask, int hi) { return hi == 0 ? 1.f : mask; }
  __device__ static inline Seed seed_b(float x, int hi) { return hi == 0 ? x : kMaskedScore; }
  __device__ static inline floatx16 mma_seed(Seed a, Seed b) {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, z, 0, 0, 0);
  }
  __device__ static inline float exact(float x) { return x; }
};

// bf16 tiles in LDS: 64 rows of 128 bytes (K: key rows of 64 dims; V^T: dim
// rows of 64 keys), no padding.  A 128-bit LDS read serves 16 lanes per
// cycle from 64 four-byte banks (256 bytes), and an operand read gives those
// lanes 16 consecutive rows at one logical chunk.  Two consecutive rows span
// all 64 banks, so the 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 1) & 7): the 8 row pairs of a lane group use 8 different
// positions, each row of a pair its own half of the banks.
__device__ inline int swz(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// K operand: key row `row`, dims [dc*2*KPL + hi*KPL, +KPL).
__device__ inline bf16x8 read_k(const bf16* lk, int pitch, int row, int dc, int hi) {
  (void)pitch;
  return *(const bf16x8*)((const char*)lk + swz(row, dc * 2 + hi));
}
__device__ inline float read_k(const float* lk, int pitch, int row, int dc, int hi) {
  return lk[row * pitch + dc * 2 + hi];
}

// V^T operand for dim row d and chunk ch of key block kb: the keys whose S^T
// accumulator registers form the matching P^T operand, i.e. keys
// 16*ch + 4*hi + {0..3} and 16*ch + 8 + 4*hi + {0..3} of the block.  The bf16
// V^T tile holds each 16-key group in that order (keys 0-3, 8-11, 4-7,
// 12-15), so the operand is one 16-byte read, laid out like the K reads.
__device__ inline bf16x8 read_v(const bf16* lv, int pitch, int d, int kb, int ch, int hi) {
  (void)pitch;
  return *(const bf16x8*)((const char*)lv + swz(d, kb * 4 + ch * 2 + hi));
}
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
// dims [dc*2*KPL + hi*KPL, +KPL).
__device__ inline void load_q(const AttnArgs& a, int qbase, int h, int l32, int hi, bf16x8 (&qf)[2][4]) {
  const bf16* Q = (const bf16*)a.q;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int q = qbase + qb * 32 + l32;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      Vec16<bf16> v;
      v.u = make_uint4(0, 0, 0, 0);
      if (q < a.Tq) v.u = *(const uint4*)(Q + ((size_t)q * a.H + h) * kHeadDim + dc * 16 + hi * 8);
      bf16x8 f;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = v.e[i];
      qf[qb][dc] = f;
    }
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
  int lens[2];                // valid lengths of the entries of keys l32 and 32 + l32 of the
                              // tile whose page ids are held
  int dlens[2];               // the same for the tile held in kr / vr

  __device__ void init(const T* kpool, const T* vpool, int h, int H, int tid) {
    page_bytes = (uint32_t)(H * P * kHeadDim * sizeof(T));
#pragma unroll
    for (int i = 0; i < NC; ++i)
      kaddr[i] = (const char*)(kpool + ((h * P) + (k_row(tid, i) % P)) * kHeadDim + k_part(tid) * EPC);
    vaddr = (const char*)(vpool + (h * kHeadDim + v_row(tid, 0)) * P + (v_key0(tid) % P));
  }
  // page ids and lengths of tile `tile` (the gather list is padded past its
  // end).  With several entries per tile each thread loads those of its own
  // chunks and keys with plain vector loads, consumed a whole tile later when
  // that tile's data loads are issued; with one entry per tile (P = 64) a
  // scalar load through the constant address space (the list is not written
  // during the launch) serves the whole wave.
  __device__ void fetch_pages(const AttnArgs& a, int tile, int tid) {
    if constexpr (EPT == 1) {
      typedef const __attribute__((address_space(4))) int32_t cint;
      const int pg = *(cint*)(const void*)(a.sel_page + tile);
      const int ln = *(cint*)(const void*)(a.sel_len + tile);
#pragma unroll
      for (int i = 0; i < NC; ++i) pg_k[i] = pg;
      pg_v = pg;
      lens[0] = ln;
      lens[1] = ln;
    } else {
      const int32_t* sp = a.sel_page + tile * EPT;
      const int32_t* sl = a.sel_len + tile * EPT;
#pragma unroll
      for (int i = 0; i < NC; ++i) pg_k[i] = sp[k_row(tid, i) / P];
      pg_v = sp[v_key0(tid) / P];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) lens[kb] = sl[(kb * 32 + (tid & 31)) / P];
    }
  }
  __device__ void fetch_data(int tid) {
    dlens[0] = lens[0];
    dlens[1] = lens[1];
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

__device__ inline int pick(i32x4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

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
  static constexpr int NFETCH = 2;  // vector loads per fetch: the tile's page ids, its lengths
  static constexpr int NISSUE = 4;  // DMA loads per wave and tile
  // the EPT page ids and lengths of a tile, as loaded (every lane loads the
  // same 4 to 16 bytes); each lane picks its pieces' entries when it issues
  struct Ids {
    i32x4 pg, ln;
  };
  uint32_t koff[2], voff[2];  // piece offsets inside a (page, head) block (bytes)
  int kent[2], vent[2];       // their gather entries within a tile
  uint32_t page_bytes, head_off;

  __device__ void init(int h, int H, int tid) {
    const int w = tid >> 6, lane = tid & 63;
    page_bytes = (uint32_t)(H * P * kHeadDim * 2);
    head_off = (uint32_t)(h * P * kHeadDim * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = (w * 2 + j) * 64 + lane;        // 16-byte position in the K tile
      const int r = pos >> 3, c = (pos & 7) ^ ((r >> 1) & 7);  // key row, logical chunk (swz)
      kent[j] = r / P;
      koff[j] = (uint32_t)(((r % P) * kHeadDim + c * 8) * 2);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = (w * 2 + j) * 64 + lane;        // 16-byte position in the V^T tile
      const int d = pos >> 3, c = (pos & 7) ^ ((d >> 1) & 7);  // dim row, chunk (8 stored slots)
      vent[j] = (8 * c) / P;
      voff[j] = (uint32_t)((d * P + (8 * c) % P) * 2);
    }
  }
  template <int N>
  __device__ static i32x4 load_n(const int32_t* p) {
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
  __device__ void fetch(const AttnArgs& a, int tile, Ids& x) const {
    x.pg = load_n<EPT>(a.sel_page + tile * EPT);
    x.ln = load_n<EPT>(a.sel_len + tile * EPT);
  }
  // entry lengths of keys l32 and 32 + l32
  __device__ static void lens_of(const Ids& x, int l32, int (&out)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) out[kb] = pick(x.ln, (kb * 32 + l32) / P);
  }
  __device__ void issue(const char* kpool, const char* vpool, const Ids& x, char* buf, int w) const {
    typedef __attribute__((address_space(3))) void lds_t;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(kpool + (uint64_t)(uint32_t)pick(x.pg, kent[j]) * page_bytes + head_off +
                                           koff[j],
                                       (lds_t*)(buf + (w * 2 + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(vpool + (uint64_t)(uint32_t)pick(x.pg, vent[j]) * page_bytes + head_off +
                                           voff[j],
                                       (lds_t*)(buf + KBYTES + (w * 2 + j) * 1024), 16, 0, 0);
  }
};

// s_waitcnt on the vector-memory count only (vmcnt <= N, N < 16): bits 3:0
// vmcnt, 6:4 expcnt (7: no wait), 11:8 lgkmcnt (15: no wait), 15:14 the high
// vmcnt bits (0 here)
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Row sums of P from the same rounded values the P.V product uses (this
// lane's keys only; the lane pair l, l ^ 32 covers the whole tile).
__device__ inline float rowsum_add(float l, bf16x8 p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 one;
  one[0] = (bf16)1.0f;
  one[1] = (bf16)1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x2 pr;
    pr[0] = p[2 * i];
    pr[1] = p[2 * i + 1];
    l = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l, false);
  }
  return l;
}
__device__ inline float rowsum_add(float l, float p) { return l + p; }

// max over the two 32-lane halves of the wave
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <typename T, int P>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
  using M = Mfma<T>;
  using Frag = typename M::Frag;
  using L = TileLoader<T, P>;   // fp32: through registers, two buffers
  using DL = DmaLoader<P>;      // bf16: straight into LDS, three buffers
  // bf16 tiles: straight into LDS at P = 64, through registers at P = 16/32
  // (measured faster each way)
  constexpr bool DMA = sizeof(T) == 2 && P == 64;
  constexpr int NQB = M::NQB;
  constexpr int KPL = M::KPL;
  constexpr int NDC = kHeadDim / (2 * KPL);  // MFMAs along the head dim
  constexpr int NCH = 16 / KPL;              // P^T operands per 32-key block
  constexpr int QPW = NQB * 32;              // queries per wave
  constexpr int NBUF = DMA ? 3 : 2;
  constexpr int BUF_ELEMS = DMA ? DL::BUF_BYTES / (int)sizeof(T) : L::TILE_ELEMS;
  constexpr int VOFF = DMA ? kKeysPerTile * kHeadDim : kKeysPerTile * L::KP;  // V^T within a buffer
  __shared__ __attribute__((aligned(16))) T lt[NBUF][BUF_ELEMS];

  // workgroup -> (head, split, q tile).  Dispatch is round-robin over the
  // XCDs, each with its own L2.  With H a multiple of 8, all workgroups of a
  // head run on one XCD (XCD = h % 8), so both its K/V pages and each q
  // tile's queries come from HBM once and are shared through that L2; the q
  // tiles of one split are dispatched consecutively.  Otherwise the q tiles
  // of one (head, split) share an XCD.
  //
  // Split sizes (head-major, S even): the even splits of every (head, q tile)
  // are dispatched first, as the first workgroup of their CU, and hold
  // t_even tiles; the odd ones come second and hold t_odd.  Two workgroups
  // share a CU and the first one dispatched issues ahead of the other, so
  // uneven splits let both finish together.  Boundaries depend only on the
  // launch parameters: results stay deterministic.
  const int b = blockIdx.x;
  const int xcd = b % kNumXcd, kx = b / kNumXcd;
  int h, split, qt;
  if (a.head_major) {
    const int per = a.S * a.n_qtiles;           // workgroups of one head
    const int nh = (a.H + kNumXcd - 1) / kNumXcd;  // heads on this XCD
    if (a.t_odd > 0) {
      const int halfw = nh * per / 2;             // even (then odd) splits of all those heads
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
    if (h >= a.H) return;
  } else {
    const int unit = (kx / a.n_qtiles) * kNumXcd + xcd;
    if (unit >= a.n_units) return;
    qt = kx % a.n_qtiles;
    h = unit / a.S;
    split = unit % a.S;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int t0 = a.t_odd > 0 ? (split >> 1) * (a.tiles_per_split + a.t_odd) + (split & 1) * a.tiles_per_split
                             : split * a.tiles_per_split;
  const int t1 = min(a.n_tiles, t0 + ((split & 1) && a.t_odd > 0 ? a.t_odd : a.tiles_per_split));
  const int qbase = (qt * kWaves + wave) * QPW;
  const T* kpool = (const T*)a.kpool;
  const T* vpool = (const T*)a.vpool;

  // the wave's query fragments stay in registers (B operands)
  Frag qf[NQB][NDC];
  load_q(a, qbase, h, l32, hi, qf);

  floatx16 o[2][NQB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][j][r] = 0.f;
  // Scores are in log2 units: the queries arrive scaled by sm_scale*log2(e).
  // m is each query column's running offset, a value the seed operand holds
  // exactly.  Every 32-key block's S^T accumulators start from the seed
  // product, -m for a valid key and -m - 1e30 for a masked one, so
  // P = exp2(S^T) directly and masked keys get P = 0.  m is raised lazily: a
  // block is accepted while the sum of each lane's P over it stays <= 2^16
  // (then no P exceeds 2^16 and nothing can overflow); otherwise (the first
  // block, or a max that rose by more than 16) the block is redone from its
  // raw scores, with m raised to the block max where that exceeds m by more
  // than 8, and O and l rescaled.
  float m[NQB], l[NQB];
  typename M::Seed nm[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
    nm[qb] = M::seed_b(INFINITY, hi);
  }
  constexpr float kMaxBlockSum = 65536.f;
  constexpr float kRaise = 8.f;

  // one 64-key tile from LDS: K at ck, V^T at cv, entry lengths of keys l32
  // and 32 + l32 in cur_lens
  auto compute_tile = [&](const T* ck, const T* cv, const int (&cur_lens)[2]) {
    // seed A operands: key kb*32 + l32 is masked when past its gather
    // entry's valid length (partial pages)
    typename M::Seed sa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sa[kb] = M::seed_a((kb * 32 + l32) % P >= cur_lens[kb] ? 1.f : 0.f, hi);
    }
    // seed of key block kb: offset scores, or raw (offset 0) for a redo
    auto seed = [&](int kb, bool raw, floatx16 (&init)[NQB]) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) init[qb] = M::mma_seed(sa[kb], raw ? M::seed_b(0.f, hi) : nm[qb]);
    };
    // S^T of the whole tile (both key blocks): s[kb][qb] holds keys
    // kb*32 + 8*(r/4) + 4*hi + r%4 of query column l32
    auto qk_tile = [&](floatx16 (&s)[2][NQB], bool raw) {
      seed(0, raw, s[0]);
      seed(1, raw, s[1]);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          Frag kf = read_k(ck, L::KP, kb * 32 + l32, dc, hi);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = M::mma(kf, qf[qb][dc], s[kb][qb]);
        }
    };
    // exponentials, packing and this lane's sums of key block kb
    auto exp_block = [&](int kb, floatx16 (&s)[2][NQB], Frag (&pf)[2][NCH][NQB], float (&ts)[NQB]) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        ts[qb] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = __builtin_amdgcn_exp2f(s[kb][qb][r]);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          pf[kb][ch][qb] = pack_p(s[kb][qb], ch, T());
          ts[qb] = rowsum_add(ts[qb], pf[kb][ch][qb]);
        }
      }
    };
    auto sums_ok = [&](const float (&ts)[NQB]) {
      bool bad = false;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) bad = bad || !(ts[qb] <= kMaxBlockSum);
      return !__any(bad);
    };
    // the redo of key blocks kb0..kb1 from raw scores already in s: m raised
    // to their max where that exceeds it by more than kRaise (O and l
    // rescaled), then offset scores and exponentials again
    auto redo = [&](int kb0, int kb1, floatx16 (&s)[2][NQB], Frag (&pf)[2][NCH][NQB], float (&ts)[NQB]) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float x = s[kb0][qb][0];
#pragma unroll
        for (int kb = kb0; kb <= kb1; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) x = fmaxf(x, s[kb][qb][r]);
        const float mx = half_swap_max(x);
        if (mx > m[qb] + kRaise) {
          const float mn = M::exact(mx);
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);  // 0 while m = -inf
          m[qb] = mn;
          nm[qb] = M::seed_b(-mn, hi);
          o[0][qb] *= alpha;
          o[1][qb] *= alpha;
          l[qb] *= alpha;
        }
        // a column with no valid key so far keeps m = -inf: its P is 0
        const float off = m[qb] == -INFINITY ? 0.f : m[qb];
#pragma unroll
        for (int kb = kb0; kb <= kb1; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] -= off;
      }
      exp_block(kb0, s, pf, ts);
    };
    // O^T += V^T P^T over key block kb
    auto pv_block = [&](int kb, const Frag (&pf)[2][NCH][NQB]) {
      Frag vf[NCH][2];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int db = 0; db < 2; ++db) vf[ch][db] = read_v(cv, L::VP, db * 32 + l32, kb, ch, hi);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) o[db][qb] = M::mma(vf[ch][db], pf[kb][ch][qb], o[db][qb]);
    };

    floatx16 s[2][NQB];
    Frag pf[2][NCH][NQB];
    float ts[NQB];
    if constexpr (sizeof(T) == 2) {
      // Two 32-key blocks in flight: block 0's exponentials run beside block
      // 1's QK MFMAs, block 1's beside block 0's PV MFMAs.  Each block's sums
      // are checked before its PV; block 0's redo covers both blocks (block
      // 1's scores carry the old offset), block 1's only itself.
      Frag kf[2][NDC];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) kf[kb][dc] = read_k(ck, L::KP, kb * 32 + l32, dc, hi);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        seed(kb, false, s[kb]);
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = M::mma(kf[kb][dc], qf[qb][dc], s[kb][qb]);
      }
      exp_block(0, s, pf, ts);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDC, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NQB * (NDC + 2), 0);
#pragma unroll
      for (int i = 0; i < NDC * NQB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      if (!sums_ok(ts)) {
        qk_tile(s, true);
        redo(0, 1, s, pf, ts);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) l[qb] += ts[qb];

      pv_block(0, pf);
      exp_block(1, s, pf, ts);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NCH, 0);
#pragma unroll
      for (int i = 0; i < 2 * NCH * NQB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      if (!sums_ok(ts)) {
        seed(1, true, s[1]);
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const Frag kf1 = read_k(ck, L::KP, 32 + l32, dc, hi);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[1][qb] = M::mma(kf1, qf[qb][dc], s[1][qb]);
        }
        redo(1, 1, s, pf, ts);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) l[qb] += ts[qb];
      pv_block(1, pf);
    } else {
      // fp32: the whole tile at once
      qk_tile(s, false);
      float t1s[NQB];
      exp_block(0, s, pf, ts);
      exp_block(1, s, pf, t1s);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) ts[qb] += t1s[qb];
      if (!sums_ok(ts)) {
        qk_tile(s, true);
        redo(0, 1, s, pf, ts);
        exp_block(1, s, pf, t1s);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) ts[qb] += t1s[qb];
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) l[qb] += ts[qb];
      pv_block(0, pf);
      pv_block(1, pf);
    }

  };

  const int n = max(t1 - t0, 0);
  if constexpr (DMA) {
   if (n > 0) {
    // Every iteration fetches and issues unconditionally: a split that has
    // tiles reads at most three tiles past its end, which the gather list's
    // padding covers (pad entries name the zero page).  So
    // each iteration adds the same vector-memory operations, in the same
    // order: the ids of tile i + 3 (NFETCH), then tile i + 2's data (NISSUE).
    // Waiting until at most NISSUE are in flight at the end of iteration i
    // leaves only tile i + 2's data outstanding: tile i + 1 has landed and
    // the ids of tile i + 3 are in registers (the compiler counts the same
    // way and adds no wait before they are used).
    DL ld;
    ld.init(h, a.H, tid);
    typename DL::Ids ide, ido;  // ids of the tiles at even / odd distance from t0
    int lc[2], l1[2], l2[2];    // lengths: this tile, next, next but one
    const char* kp = (const char*)a.kpool;
    const char* vp = (const char*)a.vpool;
    char* lbase = (char*)&lt[0][0];
    constexpr int BB = DL::BUF_BYTES;
    auto ready = [](typename DL::Ids& x) {
      asm volatile("" : "+v"(x.pg), "+v"(x.ln));
    };
    ld.fetch(a, t0, ide);
    ld.fetch(a, t0 + 1, ido);
    __builtin_amdgcn_s_waitcnt(0);  // the queries and the first ids
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) asm volatile("" : "+v"(qf[qb][dc]));
    ready(ide);
    ready(ido);
    asm volatile("" ::: "memory");
    ld.issue(kp, vp, ide, lbase, wave);
    DL::lens_of(ide, l32, lc);
    ld.fetch(a, t0 + 2, ide);
    ld.issue(kp, vp, ido, lbase + BB, wave);
    DL::lens_of(ido, l32, l1);
    asm volatile("" ::: "memory");
    wait_vmem<DL::NISSUE>();  // tile t0 and the ids of tile t0 + 2 have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    auto step = [&](int i, typename DL::Ids& fx, const typename DL::Ids& iy) {
      ld.fetch(a, t0 + i + 3, fx);
      ld.issue(kp, vp, iy, lbase + ((i + 2) % 3) * BB, wave);
      DL::lens_of(iy, l32, l2);
      asm volatile("" ::: "memory");  // the loads above stay ahead of the count below
      const T* ck = lt[i % 3];
      compute_tile(ck, ck + VOFF, lc);
      asm volatile("" ::: "memory");
      wait_vmem<DL::NISSUE>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();  // buffer i % 3 is free, tile i + 1 visible to all waves
      asm volatile("" ::: "memory");
      lc[0] = l1[0];
      lc[1] = l1[1];
      l1[0] = l2[0];
      l1[1] = l2[1];
    };
    for (int i = 0; i < n; i += 2) {
      step(i, ido, ide);
      if (i + 1 < n) step(i + 1, ide, ido);
    }
    // the loads issued past the last tile land before the workgroup's LDS is released
    wait_vmem<0>();
   }
  } else {
    L ld;
    ld.init(kpool, vpool, h, a.H, tid);
    if (n > 0) {
      ld.fetch_pages(a, t0, tid);
      ld.fetch_data(tid);
      ld.fetch_pages(a, t0 + 1, tid);
      ld.store(lt[t0 & 1], tid);
    }
    int cur_lens[2] = {ld.dlens[0], ld.dlens[1]};  // entry lengths of the tile in LDS
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
      const int buf = tile & 1;
      const bool more = tile + 1 < t1;
      if (more) {
        ld.fetch_data(tid);                         // tile + 1, lands during this tile's math
        ld.fetch_pages(a, tile + 2, tid);           // page ids two tiles ahead
      }
      compute_tile(lt[buf], lt[buf] + VOFF, cur_lens);
      // the other buffer was last read in the previous tile, before its barrier
      if (more) ld.store(lt[buf ^ 1], tid);
      cur_lens[0] = ld.dlens[0];
      cur_lens[1] = ld.dlens[1];
      __syncthreads();
    }
  }

  // Each lane summed P over its own half of the keys (rows 4*hi + ...); both
  // halves share the running max, so the two partial sums simply add.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) l[qb] += __shfl_xor(l[qb], 32);

  // epilogue: O^T accumulators hold dims db*32 + 8*(r/4) + 4*hi + r%4
  if constexpr (sizeof(T) == 2) {
    if (a.S > 1) {
      // split partials go out through LDS (free once every wave is past its
      // last tile and no tile load is still landing): each wave stages its
      // 64 queries x 32 dims of one half of the head dim as 128-byte rows
      // (swizzled like the tiles), then every store instruction writes 8
      // whole 128-byte lines instead of 32-byte pieces of 32 rows
      static_assert(NBUF * BUF_ELEMS * sizeof(T) >= kWaves * QPW * 32 * 4, "staging fits the tile buffers");
      wait_vmem<0>();
      __syncthreads();
      char* st = (char*)&lt[0][0] + wave * (QPW * 32 * 4);
      float inv[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) inv[qb] = l[qb] > 0.f ? 1.f / l[qb] : 0.f;
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
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    int q = qbase + qb * 32 + l32;
    if (q >= a.Tq) continue;
    bool empty = !(l[qb] > 0.f);
    float inv = empty ? 0.f : 1.f / l[qb];
    float lse = empty ? -INFINITY : m[qb] * 0.69314718f + __logf(l[qb]);  // m is in log2 units
    size_t row = (size_t)q * a.H + h;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d = db * 32 + g * 8 + hi * 4;
        floatx4 v;
        v[0] = o[db][qb][g * 4 + 0] * inv;
        v[1] = o[db][qb][g * 4 + 1] * inv;
        v[2] = o[db][qb][g * 4 + 2] * inv;
        v[3] = o[db][qb][g * 4 + 3] * inv;
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
    case 116: hipLaunchKernelGGL((k_attn<bf16, 16>), grid, dim3(256), 0, s, a); break;
    case 132: hipLaunchKernelGGL((k_attn<bf16, 32>), grid, dim3(256), 0, s, a); break;
    case 164: hipLaunchKernelGGL((k_attn<bf16, 64>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_attn<float, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_attn<float, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_attn<float, 64>), grid, dim3(256), 0, s, a); break;
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
