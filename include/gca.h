/*
 * gca.h — C ABI of the MI355X (gfx950) Geometric Context Attention library.
 *
 * Geometric Context Attention (GCA) is the streaming attention of LingBot-Map's
 * Geometric Context Transformer: every new frame's tokens attend over a paged
 * KV cache made of three pools (page "LingBot-Map runs 10,000 frames on
 * monocular video", section "How GCT's Anchor-Pose-Trajectory Pools Make
 * Monocular 3D Tractable"):
 *   - an anchor context (the first A keyframes), which grounds the coordinate
 *     frame and scale;
 *   - a local pose-reference window (the newest W keyframes, the current one
 *     included);
 *   - a compressed trajectory memory: each frame pushed out of the window keeps
 *     only C compact tokens there.
 *
 * The calls follow the cache-manager protocol of the streaming global block
 * (page "How the Geometric Context Transformer Enables Streaming 3D
 * Reconstruction", section "FlashInferBlock (GPU-Accelerated)"):
 *   keyframe:      gca_append_frame -> gca_evict_compact -> gca_attend
 *   non-keyframe:  gca_append_frame(GCA_APPEND_TEMP) -> gca_attend ->
 *                  gca_rollback_last_frame   (keyframe-only caching)
 * and gca_cache_reset clears the cache between videos (same page, section
 * "KV-Cache Initialization").
 *
 * Tensors.  Q, K, V and O are dense [T][H][D] row-major ("NHD": token, head,
 * dim), D = 64, in the cache dtype (float32 or bfloat16); out may be float32
 * or bfloat16 (config.out_dtype); lse is float32 [T][H].  Q and K are passed
 * BEFORE the rotary embedding: with config.rope = 1 the library applies the
 * 3D (t, h, w) rotary embedding itself, t being the global frame index
 * (section "3D Rotary Positional Embeddings").
 *
 * Device pointers.  q, k, v, out and lse are device pointers owned by the
 * caller, 16-byte aligned, valid until the work enqueued on `stream` has
 * completed.  The library keeps no caller pointer after a call returns.  The
 * library owns everything else (page pools, page tables, ring, gather list,
 * rotary tables, split workspace).
 *
 * Streams.  Every device call enqueues work on `stream` (a hipStream_t; NULL
 * is the null stream) and returns without synchronising, except
 * gca_export_state, gca_read_page, gca_profile_read and gca_cache_destroy,
 * which synchronise.  A handle is not thread safe; calls on different streams
 * must be ordered by the caller.
 *
 * Errors.  Every call returns GCA_OK (0) or a negative code.  An error
 * detected on the host (arguments, call sequence, capacity) enqueues nothing
 * and changes no state.  Cache occupancy is a data-independent function of the
 * configuration and the call sequence, so these checks need no device sync.
 * GCA_ERR_HIP reports a HIP runtime failure; gca_last_error() gives its text.
 */
#ifndef GCA_H_
#define GCA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* gca_stream_t; /* a hipStream_t */
typedef struct gca_cache gca_cache;
typedef struct gca_plan gca_plan;

enum {
  GCA_OK = 0,
  GCA_ERR_INVALID_ARGUMENT = -1, /* null/misaligned pointer, bad config or frame index */
  GCA_ERR_SEQUENCE = -2,         /* call out of protocol order (see each call) */
  GCA_ERR_OUT_OF_PAGES = -3,     /* the ring holds too few free pages */
  GCA_ERR_CAPACITY = -4,         /* frame_idx >= max_frames, or trajectory full */
  GCA_ERR_HIP = -5,              /* HIP runtime error (text: gca_last_error) */
  GCA_ERR_UNSUPPORTED = -6       /* valid but not built for (e.g. head_dim != 64) */
};

enum { GCA_F32 = 0, GCA_BF16 = 1 };

enum { GCA_APPEND_TEMP = 1u }; /* non-keyframe: attend, then roll back */

typedef struct {
  int32_t tokens_per_frame;  /* T >= 1 */
  int32_t num_heads;         /* H >= 1 (MHA: as many K/V heads as Q heads) */
  int32_t head_dim;          /* D: 64 only (else GCA_ERR_UNSUPPORTED) */
  int32_t page_size;         /* P: 16, 32 or 64 tokens (else GCA_ERR_UNSUPPORTED) */
  int32_t dtype;             /* GCA_F32 | GCA_BF16: Q, K, V and the page pools */
  int32_t out_dtype;         /* GCA_F32 | GCA_BF16: attention output */
  int32_t num_anchor_frames; /* A >= 0: the first A keyframes are kept whole */
  int32_t window_frames;     /* W >= 1: newest keyframes kept whole, current included */
  int32_t num_compact;       /* C in [0, T]: tokens kept per frame evicted from the window */
  const int32_t* compact_idx;/* C distinct offsets in [0, T) (copied); NULL: special
                                tokens first, then evenly spaced patch tokens */
  int32_t num_special;       /* special tokens at the start of each frame */
  int32_t grid_h, grid_w;    /* patch grid; T = num_special + grid_h * grid_w when rope = 1 */
  int32_t rope;              /* 0: none; 1: 3D rotary embedding over (t, h, w) */
  float rope_theta;          /* rotary base, e.g. 10000 */
  float sm_scale;            /* softmax scale, e.g. 1/sqrt(D) */
  int64_t max_frames;        /* frame indices are < max_frames (sizes the rotary
                                table and the trajectory) */
  int32_t num_pages;         /* ring size N; 0: peak of a keyframe stream,
                                A*ceil(T/P) + (W+1)*ceil(T/P) +
                                ceil(C*max(0, F-A-W)/P), F = max_frames, or
                                min(max_frames, infer_window) when windowed */
  const int32_t* ring_init;  /* N distinct page ids giving the initial free order
                                (copied); NULL: 0, 1, ..., N-1 */
  /* Windowed inference ("LingBot-Map runs 10,000 frames on monocular video",
   * section "Cloning and Installing"; the project summary's "Main features"
   * table: past the frame range the video rotary embedding was trained on,
   * the memory slides as fixed-size windows overlapping by a few keyframes).
   * With infer_window > 0 a window spans infer_window frames from its origin
   * and the temporal rotary position of a frame (keys and queries) is its
   * index relative to that origin.  The first frame appended outside the
   * window starts the next one: the cache is reset and the last
   * infer_overlap keyframes that fit in one window with that frame are
   * appended again, oldest first, from raw copies the library keeps (their
   * positions now relative to the oldest of them, the new origin); then the
   * frame itself.  Requires 1 <= infer_overlap <= min(16, A + W) and
   * infer_overlap < infer_window.  0 (the default) disables it. */
  int32_t infer_window;
  int32_t infer_overlap;
} gca_config;

/* Host-side occupancy (no device access). */
typedef struct {
  int32_t pages_per_frame;   /* ceil(T/P) */
  int32_t num_pages;         /* N */
  int32_t free_pages;        /* pages in the ring */
  int32_t anchor_frames;     /* live anchor frames */
  int32_t window_frames;     /* live window frames, a pending non-keyframe included */
  int32_t temp_pending;      /* 1 while a GCA_APPEND_TEMP frame awaits rollback */
  int32_t traj_pages;        /* pages holding trajectory tokens */
  int32_t n_sel;             /* gather-list entries of the next attention */
  int64_t traj_tokens;       /* compact tokens in the trajectory */
  int64_t n_ctx;             /* context tokens of the next attention */
  int64_t last_frame;        /* last appended frame index, -1 if none */
  int32_t max_splits;        /* split-KV workspace depth */
  int32_t reserved;
  int64_t window_origin;     /* windowed inference: frame index of temporal position 0 */
} gca_info;

/* Device state copied to host buffers by gca_export_state.  Inputs: host
 * buffers, each may be NULL to skip; sizes from gca_query.  Outputs: counts. */
typedef struct {
  int32_t* free_ring;   /* [N] free page ids from the ring head (next allocated first) */
  int64_t* frame_idx;   /* [anchor_frames + window_frames] live frames in gather order */
  int32_t* frame_pages; /* [same][pages_per_frame] their page ids */
  int32_t* traj_pages;  /* [traj_pages] trajectory pages, oldest first */
  int32_t* sel_page;    /* [n_sel] last built gather list: page ids */
  int32_t* sel_len;     /* [n_sel] valid tokens per entry */
  int32_t n_free, n_frames, n_traj_pages, n_sel;
  int64_t traj_tokens, n_ctx;
} gca_state_view;

/* ---- cache lifecycle ------------------------------------------------------ */

/* Validate the config, allocate the page pools (N * H * P * D elements each for
 * K and V), page tables, ring, gather list, rotary tables and split workspace
 * with hipMalloc on the current device, and initialise the ring.  Synchronous.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, HIP. */
int gca_cache_create(const gca_config* cfg, gca_cache** out);

/* Synchronise the device and free everything.  NULL is accepted. */
int gca_cache_destroy(gca_cache* cache);

/* Forget every frame and restore the initial ring (clean_kv_cache). */
int gca_cache_reset(gca_cache* cache, gca_stream_t stream);

/* ---- per-frame protocol ---------------------------------------------------- */

/* append_frame(global_idx, k_nhd, v_nhd): pop ceil(T/P) pages from the ring
 * head, record the frame (as an anchor while fewer than A anchors exist, else
 * as the newest window frame; a GCA_APPEND_TEMP frame always as the pending
 * newest window frame), rotate K (rope = 1) and scatter K' and V into the
 * pages: token n goes to page n / P, slot n % P.  k, v: raw [T][H][D].
 * Errors: INVALID_ARGUMENT (null/misaligned, frame_idx < 0); SEQUENCE (a TEMP
 * frame is pending, frame_idx not above the last appended one, or W+1 window
 * frames are live and gca_evict_compact is due); CAPACITY (frame_idx >=
 * max_frames); OUT_OF_PAGES.
 * Windowed inference (infer_window > 0): K is rotated at frame_idx minus the
 * window origin; a keyframe's raw K and V are also copied into the library's
 * overlap store; a frame_idx outside the window first restarts the cache as
 * gca_config describes (ring back to its initial order, the kept keyframes
 * appended again, enqueued on `stream` before this frame's append). */
int gca_append_frame(gca_cache* cache, int64_t frame_idx, const void* k, const void* v,
                     uint32_t flags, gca_stream_t stream);

/* Several keyframes appended in one launch: append_frame for frames
 * first_frame .. first_frame + n_frames - 1 in that order, k and v raw
 * [n_frames][T][H][D].  Meant for the scale frames (a stream's first frames,
 * processed together and kept as the anchor: "How the Geometric Context
 * Transformer Enables Streaming 3D Reconstruction in LingBot-Map", section
 * "Streaming Inference API"), or any burst of keyframes with no eviction due
 * in between.  Results are bit for bit those of the individual calls.  The
 * whole batch is validated first; an error leaves the cache unchanged.
 * Errors: INVALID_ARGUMENT (null/misaligned, first_frame < 0, n_frames < 1);
 * CAPACITY (n_frames > 16, or a frame index >= max_frames); SEQUENCE (as
 * gca_append_frame for any frame of the batch, including an eviction coming
 * due inside it, or in windowed inference a frame past the first one that
 * would start the next window); OUT_OF_PAGES. */
int gca_append_frames(gca_cache* cache, int64_t first_frame, int32_t n_frames, const void* k,
                      const void* v, gca_stream_t stream);

/* evict_frames: while more than W window frames are live, take the oldest,
 * copy its C compact tokens (K' and V) to the end of the trajectory (popping a
 * new trajectory page from the ring head whenever the trajectory length is a
 * multiple of P), then push its pages to the ring tail.  No-op if nothing to
 * evict.  Errors: SEQUENCE (TEMP pending), OUT_OF_PAGES, CAPACITY. */
int gca_evict_compact(gca_cache* cache, gca_stream_t stream);

/* compute_attention(global_idx, q_nhd): build the gather list (anchor pages,
 * window pages oldest to newest with the current frame last, trajectory
 * pages), rotate Q at frame_idx (rope = 1; minus the window origin in
 * windowed inference) and write, for every token n and
 * head h, out[n][h] = sum_i softmax_i(sm_scale * q'.k'_i) v_i over the n_ctx
 * context tokens (no other mask: the current frame sees all of its own
 * tokens) and, if lse != NULL, lse[n][h] = natural log of the softmax
 * denominator including the scale.  frame_idx must be the last appended
 * frame.  Errors: INVALID_ARGUMENT, SEQUENCE. */
int gca_attend(gca_cache* cache, int64_t frame_idx, const void* q, void* out, float* lse,
               gca_stream_t stream);

/* Scale frames processed together: a stream starts with a few frames that are
 * handled jointly, each attending over all of them (bidirectional), before
 * causal streaming begins ("How the Geometric Context Transformer Enables
 * Streaming 3D Reconstruction in LingBot-Map", section "Streaming Inference
 * API" and the FAQ on why scale frames are processed differently).  Appended
 * as the anchor frames, they are attended to here in one call:
 * compute_attention for the queries of the n_frames frames first_frame ..
 * first_frame + n_frames - 1, q raw [n_frames][T][H][D], each frame's queries
 * rotated at its own frame index (rope = 1), all over the one current context
 * (the gather list of gca_attend).  out [n_frames][T][H][D] (out_dtype), lse
 * [n_frames][T][H] or NULL.  The last of the frames must be the last appended
 * frame, as for gca_attend; n_frames = 1 is gca_attend.  Errors:
 * INVALID_ARGUMENT (null/misaligned, first_frame < 0, n_frames < 1); CAPACITY
 * (n_frames above max(1, num_anchor_frames), the frames the query workspace
 * holds); SEQUENCE. */
int gca_attend_frames(gca_cache* cache, int64_t first_frame, int32_t n_frames, const void* q,
                      void* out, float* lse, gca_stream_t stream);

/* rollback_last_frame(global_idx): drop the pending GCA_APPEND_TEMP frame and
 * return its pages to the ring head; the cache is as before its append.
 * Errors: SEQUENCE (no TEMP pending or another frame index). */
int gca_rollback_last_frame(gca_cache* cache, int64_t frame_idx, gca_stream_t stream);

/* One frame of the loop above in a single call: append_frame (as a keyframe
 * with GCA_STEP_KEYFRAME, then evict_frames; otherwise as GCA_APPEND_TEMP),
 * compute_attention at frame_idx, and for a non-keyframe
 * rollback_last_frame.  Results are bit for bit those of the individual calls
 * in that order.  The whole step is validated on the host before anything is
 * enqueued, so an error leaves the cache unchanged.  The append, the
 * eviction, the query rotation and the gather list are enqueued as one
 * launch, followed by the attention.  k, v, q, out, lse as for
 * gca_append_frame and gca_attend.  Errors: the union of theirs. */
enum { GCA_STEP_KEYFRAME = 1u };
int gca_step(gca_cache* cache, int64_t frame_idx, const void* k, const void* v, const void* q,
             void* out, float* lse, uint32_t flags, gca_stream_t stream);

/* gca_step for callers that cannot allocate device memory while they run:
 * code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  Same arguments, validation, errors and results as gca_step
 * (bit for bit), and it calls no allocating routine: the step's scratch (the
 * prepared queries, then the split-KV partials of the attention) comes from a
 * fixed library-wide device array of GCA_STATIC_SCRATCH_BYTES instead of the
 * cache's workspace.  The cache itself is allocated once, by
 * gca_cache_create, which also looks the array up on its device.
 * Limit: the step needs T*H*64*esize bytes of queries plus, when the context
 * is split S ways (about two workgroups per compute unit), S*T*H*65*4 bytes of
 * partials, each rounded up to 256 bytes (about 36 MB for 1004 tokens x 16
 * heads at S = 8); a step needing more returns GCA_ERR_CAPACITY, enqueues
 * nothing and changes nothing (gca_last_error says how much it needed).
 * Sharing: each GPU holds one copy of the array, from the first cache created
 * on it until the process ends, shared by every cache and stream on that GPU
 * and keeping the last call's contents (every byte a step reads it has
 * written first, so nothing needs clearing).  Calls that may overlap on one
 * GPU (other streams, other threads) race on it: order them, or use
 * gca_step. */
#define GCA_STATIC_SCRATCH_BYTES (64u << 20)
int gca_step_static(gca_cache* cache, int64_t frame_idx, const void* k, const void* v, const void* q,
                    void* out, float* lse, uint32_t flags, gca_stream_t stream);

/* ---- pieces of the path, for tests and tools ------------------------------- */

/* Build the gather list of the current context on the device (gca_attend does
 * this itself).  Errors: SEQUENCE (empty cache). */
int gca_select(gca_cache* cache, gca_stream_t stream);

/* y = rotary embedding of x ([T][H][D], cache dtype) at temporal position
 * frame_idx, the same arithmetic gca_append_frame applies to K and gca_attend
 * to Q (in windowed inference frame_idx is the window-relative position).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (rope = 0), CAPACITY (frame_idx >=
 * max_frames, or >= infer_window in windowed inference). */
int gca_rope3d(gca_cache* cache, int64_t frame_idx, const void* x, void* y, gca_stream_t stream);

/* Host-side occupancy; no device access. */
int gca_query(const gca_cache* cache, gca_info* out);

/* Synchronise `stream` and copy ring, page tables and the last gather list to
 * the host buffers of *view. */
int gca_export_state(gca_cache* cache, gca_state_view* view, gca_stream_t stream);

/* Synchronise `stream` and copy one page's K' and V to host buffers laid out
 * [H][P][D] in the cache dtype (slot order), whatever the device layout. */
int gca_read_page(gca_cache* cache, int32_t page, void* host_k, void* host_v, gca_stream_t stream);

/* Kernel timing with HIP events recorded around launches on their stream.
 * kind: 0 append, 1 evict, 2 selection (inside gca_attend it also rotates
 * the queries), 3 attention, 4 split merge, 5 rope, 6 the update launch of
 * gca_step (append, eviction, query rotation and gather list).
 * gca_profile_enable(cache, capacity, kinds) starts recording up to
 * `capacity` launches of the kinds whose bit (1 << kind) is set in `kinds`
 * (capacity 0 stops); gca_profile_read synchronises and returns the summed
 * milliseconds and launch count of one kind, then forgets them.  Each event
 * adds a little stream work, so record only the kinds to be measured. */
int gca_profile_enable(gca_cache* cache, int32_t capacity, uint32_t kinds);
int gca_profile_read(gca_cache* cache, int32_t kind, double* total_ms, int32_t* count);

/* ---- host-only planner -------------------------------------------------------
 * The occupancy state machine that gca_cache runs on the host, without a
 * device: validates a config and a call sequence and reports the occupancy it
 * would produce (page needs, context sizes), e.g. to size num_pages.  Same
 * error codes as the device calls. */
int gca_plan_create(const gca_config* cfg, gca_plan** out);
int gca_plan_destroy(gca_plan* plan);
int gca_plan_reset(gca_plan* plan);
int gca_plan_append(gca_plan* plan, int64_t frame_idx, uint32_t flags);
int gca_plan_evict(gca_plan* plan);
int gca_plan_attend(gca_plan* plan, int64_t frame_idx);
int gca_plan_rollback(gca_plan* plan, int64_t frame_idx);
int gca_plan_query(const gca_plan* plan, gca_info* out);
/* The compact token offsets the config resolves to (the given list, or the
 * default rule: special tokens first, then evenly spaced patch tokens),
 * copied to out[0 .. *n).  *n is always set; GCA_ERR_CAPACITY (nothing
 * copied) when cap < *n. */
int gca_plan_compact(const gca_plan* plan, int32_t* out, int32_t cap, int32_t* n);

/* ---- diagnostics -------------------------------------------------------------- */
const char* gca_status_string(int status);
const char* gca_last_error(void); /* text of the last GCA_ERR_HIP (or gca_step_static's
                                     GCA_ERR_CAPACITY) on this thread */

#ifdef __cplusplus
}
#endif

#endif /* GCA_H_ */
