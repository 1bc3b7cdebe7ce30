/*
 * statekv.h -- C ABI of the StateKV streaming video-prefill step on MI355X (gfx950).
 *
 * What the library computes (per transformer layer, per arriving frame n):
 *   1. the frame's T queries attend, with a softmax, over the candidate pool
 *      [compressed state C_{n-1} ; the frame's own T keys/values]; every state
 *      token is visible to every query, frame tokens are causal (t' <= t);
 *   2. the same probabilities give every candidate j an importance score
 *      sigma_j = sum over the frame's queries i and over the query heads that
 *      share j's KV head of P_ij;
 *   3. the top-B candidates by (sigma descending, original position ascending)
 *      become C_n;
 *   4. the frame's keys/values are appended to the detailed cache D_n.
 * Sources: "Linear Scaling Video VLMs for Long Video Understanding" as
 * summarised on paper.rainbus.top (method-steps section: per-layer detailed and
 * fixed-capacity compressed states, attention over their concatenation, append
 * to the detailed state, top-B of previous state plus frame by summed attention
 * weight) and on paperlayer.ai (section 3.2-3.3: the two caches and the
 * per-frame cache-builder pass; App. A "Protocol": sinks are kept per layer and
 * KV head).  The pages define no programming interface; this one is derived
 * from that description.
 *
 * Conventions for every entry point:
 *   - All tensors are device pointers (hipMalloc'd or torch CUDA memory),
 *     contiguous, 16-byte aligned.  bf16 means IEEE bfloat16 bit patterns.
 *   - Q is [T][Hq][d] bf16, K and V are [T][Hkv][d] bf16 (token-major, the
 *     natural output of a QKV projection), already rotated (RoPE) at the tokens'
 *     original positions p = position_offset + n*T + t.  The library never
 *     applies positional encoding; it only records p.
 *   - O is written as float32 [T][Hq][d].
 *   - Numeric preconditions (not checked; violating them gives inf/NaN in O,
 *     never a fault): q, k and v are finite, and |v| < 65504 -- the value
 *     side of the attention runs on fp16 matrix instructions, which hold
 *     every bf16 value of that range (exactly for |v| >= 2^-17).  NaN or inf
 *     inputs give an unspecified selection (never an out-of-range index).
 *   - `stream` is a hipStream_t (NULL = default stream).  Work is enqueued
 *     asynchronously; results are ready once the stream is synchronised.
 *   - The caller owns every device buffer, including the one workspace; the
 *     library allocates no device memory, except statekv_qkv_rope when called
 *     without a workspace (stream-ordered, freed on the same stream).  The layer handle is host memory
 *     owned by the library until statekv_free_layer.
 *   - Every argument check is done on the host before anything is enqueued; on
 *     an error return other than STATEKV_ERR_HIP nothing was enqueued and the
 *     layer is unchanged.
 *     Asynchronous device faults surface at the caller's next synchronisation.
 *   - A layer is not thread-safe; use one layer per stream.  Distinct layers are
 *     independent.
 */
#ifndef STATEKV_H_
#define STATEKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
enum {
  STATEKV_OK = 0,
  STATEKV_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad shape, misuse          */
  STATEKV_ERR_UNSUPPORTED = -2,      /* valid but not implemented (e.g. d=96)    */
  STATEKV_ERR_WORKSPACE = -3,        /* workspace too small or misaligned        */
  STATEKV_ERR_CAPACITY = -4,         /* detailed cache full and D_RING not set   */
  STATEKV_ERR_HIP = -5               /* a HIP launch reported an error           */
};

/* Layer flags. */
enum {
  /* One kept set per layer: candidates are ranked by their importance summed
   * over every query head of the layer, and every KV head keeps the same
   * positions (rainbus method steps define the importance as a sum over
   * queries without fixing whether heads share one kept set; this is the
   * per-layer reading).  The state view's score rows stay per KV head; the
   * ranked layer-wide value is their fp32 sum in head order.  The default is
   * per-KV-head selection (paperlayer App. A: sinks kept per layer and KV
   * head). */
  STATEKV_FLAG_SELECT_SHARED = 1u << 0,
  /* Wrap the detailed cache: token p goes to slot (p - position_offset) mod
   * detailed_capacity.  Without it, a frame that would overflow D fails with
   * STATEKV_ERR_CAPACITY. */
  STATEKV_FLAG_D_RING = 1u << 1,
  /* Frame tokens see every frame token, not only earlier ones. */
  STATEKV_FLAG_NONCAUSAL_FRAME = 1u << 2,
  /* Keep C as the positions of its tokens only: attention reads their K and V
   * rows from D (every token is there), and the state update moves positions
   * instead of K/V rows.  Needs a linear D (with D_RING:
   * STATEKV_ERR_UNSUPPORTED).  The state view's k and v are then NULL. */
  STATEKV_FLAG_C_IN_D = 1u << 3,
  /* Recency window instead of importance: keep the B most recent candidates
   * (the rule StateKV is compared against -- rainbus core method: ReKV keeps
   * the last R frames; paperlayer App. A.3 measures the gap).  Importance
   * scores are still computed and reported. */
  STATEKV_FLAG_SELECT_RECENT = 1u << 4,
  /* Update C in place: kept state rows stay in their rows, and the kept frame
   * tokens fill the rows that were freed (evicted rows in ascending row order,
   * then the unused rows count..B-1 while C fills up; the i-th such row takes
   * the i-th kept frame token in frame order).  At most T rows per KV head
   * move instead of every kept row (rainbus method steps: the kept set is
   * what matters, not its storage order).  C's rows are then in no particular
   * position order (the state view's pos gives each row's position); ties in
   * importance still go to the lower original position, as long as the
   * positions of the tied candidates lie within 2^32 - 3 of the newest one. */
  STATEKV_FLAG_SLOT_STABLE = 1u << 5,
  /* statekv_prefill_frame writes O as bf16 [T][Hq][d] (round to nearest even
   * from the fp32 result it would otherwise write) instead of fp32, for a
   * caller that feeds O to a bf16 output projection.  The quadratic baseline
   * (statekv_full_attention_frame) refuses such a layer. */
  STATEKV_FLAG_OUT_BF16 = 1u << 6
};

typedef struct statekv_layer statekv_layer; /* opaque, host memory */

typedef struct statekv_layer_config {
  int32_t n_q_heads;         /* Hq, multiple of n_kv_heads, G = Hq/Hkv <= 16     */
  int32_t n_kv_heads;        /* Hkv >= 1                                         */
  int32_t head_dim;          /* d: 64 or 128                                     */
  int32_t frame_tokens;      /* T, 1 .. 4096                                     */
  int32_t state_budget;      /* B >= 1 with B + T <= 32768                       */
  int32_t num_splits;        /* key splits of the attention grid; 0 = automatic  */
  int64_t detailed_capacity; /* tokens preallocated per KV head in D, >= T       */
  int64_t position_offset;   /* original position of frame 0, token 0            */
  float softmax_scale;       /* logit scale; <= 0 means 1/sqrt(d)                */
  uint32_t flags;            /* STATEKV_FLAG_*                                   */
  /* Rotary embedding inside the library.  rope_theta > 0: q and k arrive
   * unrotated and every per-frame call rotates them at the frame's original
   * positions p = position_offset + n*T + t before anything else (C and D then
   * hold rotated keys; paperlayer section 3.3: positions stay virtual although
   * C is physically shorter); statekv_rope rotates other tokens (text queries)
   * with the same parameters.  Pairing (x_i, x_{i+d/2}), angle
   * (p / rope_scaling) * rope_theta^(-2i/d); angle, cosine, sine and the
   * rotation in double precision, one rounding to bf16 (nearest, ties to
   * even).  rope_theta = 0: q and k arrive rotated.
   * rope_scaling: linear position interpolation, <= 0 means 1 (the pages
   * require one value for cache building and generation but give none). */
  float rope_theta;
  float rope_scaling;
} statekv_layer_config;

/* View of the compressed state C_n (borrowed; valid until the next
 * prefill/reset/free on the layer).  Rows [0, count) of every KV head are live,
 * in ascending original position (in any order with SLOT_STABLE).  Read after
 * synchronising the stream. */
typedef struct statekv_state_view {
  const void* k;            /* device, [Hkv][capacity][d] bf16                   */
  const void* v;            /* device, [Hkv][capacity][d] bf16                   */
  const int64_t* pos;       /* device, [Hkv][capacity] original positions        */
  const float* last_scores; /* device, [Hkv][scores_stride]: importance of each
                               candidate of the last frame's pool, pool order
                               ([C_{n-1} ; frame]); entries [0, last_pool) valid */
  int32_t count;            /* |C_n| = min(B, frames_seen * T)                   */
  int32_t capacity;         /* B                                                 */
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t last_pool;        /* c_{n-1} + T of the last frame (0 before any)      */
  int32_t scores_stride;
  int64_t frames_seen;
} statekv_state_view;

/* View of the detailed cache D_n (borrowed, same validity as above). */
typedef struct statekv_cache_view {
  const void* k;      /* device, [Hkv][capacity][d] bf16                         */
  const void* v;      /* device, [Hkv][capacity][d] bf16                         */
  int64_t length;     /* tokens held: min(frames_seen*T, capacity)               */
  int64_t capacity;   /* detailed_capacity                                      */
  int64_t start;      /* original position of the oldest token held; with
                         D_RING it lives in slot (start-position_offset) mod cap */
  int32_t n_kv_heads;
  int32_t head_dim;
} statekv_cache_view;

/* Bytes of device workspace a layer with this configuration needs.
 * Host only; returns STATEKV_ERR_INVALID_ARGUMENT / _UNSUPPORTED for bad
 * configurations. */
int statekv_workspace_bytes(const statekv_layer_config* cfg, size_t* bytes);

/* Create a layer over a caller-allocated device workspace of at least
 * statekv_workspace_bytes() bytes, 256-byte aligned, kept alive until
 * statekv_free_layer.  Host only (enqueues nothing): the layer starts with an
 * empty compressed state and an empty detailed cache. */
int statekv_init_layer(const statekv_layer_config* cfg, void* d_workspace,
                       size_t workspace_bytes, statekv_layer** out);

/* The per-frame StateKV step (the four parts listed at the top; rainbus
 * method steps; paperlayer section 3.3) for the next frame n = frames_seen:
 * reads q/k/v, writes o, updates C and D, and advances frames_seen.  The
 * numeric preconditions above apply (finite inputs, |v| < 65504).  Kernels: attention statistics pass, attention output + score
 * pass, top-B select (with the split-O reduction in the same launch),
 * gather + detailed-cache append (with SLOT_STABLE the select launch applies
 * the state update and the append itself: three launches). */
int statekv_prefill_frame(statekv_layer* layer, const void* q, const void* k,
                          const void* v, void* o, void* stream);

/* Quadratic baseline on the same layer object: full causal self-attention
 * ("Full SA"), in which every position attends to every earlier position, so
 * frame n costs O(nT^2) and a video O((TN)^2) (rainbus prerequisites, section
 * on self-attention complexity; paperlayer App. C.1-C.2 compare StateKV's
 * marginal and cumulative compute against it).  Appends the frame to D, then
 * the frame's queries attend over D[0 : (n+1)T] causally; C is never
 * touched.  Same numeric preconditions as statekv_prefill_frame.  A layer serves either this
 * or statekv_prefill_frame, not both (mixing returns INVALID_ARGUMENT).  Needs
 * a linear (non-ring) D. */
int statekv_full_attention_frame(statekv_layer* layer, const void* q, const void* k,
                                 const void* v, float* o, void* stream);

/* Decoding attention over the detailed state (the step after the video
 * prefill): once the frames are in, text generation attends over D_N, which
 * keeps every original video token (gist.science/nl, "Het Proces", decoding
 * item; rainbus core method: ordinary text decoding over all video tokens).
 * The text follows the video, so every live D token (slots [0, min(frames_seen
 * * T, detailed_capacity)), any order) is visible to every query; the queries'
 * own text context (prompt, generated tokens) is the caller's ordinary decoder
 * cache and is not included.
 *   q: device, [n_queries][Hq][d] bf16, 16-byte aligned, RoPE applied by the
 *      caller at the text positions; query head g reads KV head g / G;
 *   o: device, [n_queries][Hq][d] fp32, 16-byte aligned, written;
 *   1 <= n_queries and G * n_queries <= 32 (else STATEKV_ERR_UNSUPPORTED);
 *   frames_seen >= 1 (else STATEKV_ERR_INVALID_ARGUMENT).
 * Works after statekv_prefill_frame or statekv_full_attention_frame and
 * changes no layer state; uses the workspace's split-partial regions, so it
 * must not overlap a prefill call of the same layer.  Same numeric
 * preconditions as statekv_prefill_frame (finite q and D, |v| < 65504).  Kernels: DECODE (one
 * wave per KV head and D split), then SPLIT_SUM (split combine). */
int statekv_decode_attention(statekv_layer* layer, const void* q, int32_t n_queries, float* o,
                             void* stream);

/* statekv_decode_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split partials in a
 * fixed 8 MiB device array of the library (one per GPU, kept until the
 * process ends) instead of the layer's workspace; it calls no allocator.
 * Results are bit-identical to statekv_decode_attention whenever the split
 * count that one chooses fits the array (every G * n_queries <= 32 case of
 * up to 64 query heads of d <= 128); otherwise fewer splits are used.  All
 * calls on one GPU share the array: calls that overlap on one GPU (on
 * different streams, or from several host threads) race and must be
 * serialised by the caller.  Same arguments, preconditions and errors as
 * statekv_decode_attention, plus STATEKV_ERR_HIP if the array's device
 * address cannot be resolved. */
int statekv_decode_attention_noalloc(statekv_layer* layer, const void* q, int32_t n_queries,
                                     float* o, void* stream);

/* Rotate n_tokens x n_heads rows of d bf16 values in place (device,
 * [n_tokens][n_heads][d], 16-byte aligned) at positions first_position + i,
 * with the layer's rope_theta and rope_scaling (text queries before
 * statekv_decode_attention, so that cache building and generation share one
 * RoPE configuration).  STATEKV_ERR_INVALID_ARGUMENT if the layer has
 * rope_theta = 0 or an argument is out of range. */
int statekv_rope(statekv_layer* layer, void* x, int32_t n_tokens, int32_t n_heads,
                 int64_t first_position, void* stream);

/* The frame front end: the frame's queries, keys and values from the hidden
 * states of its visual tokens, Q_n = X_n W_Q, K_n = X_n W_K, V_n = X_n W_V
 * (rainbus method steps; no bias), with q and k rotated at the tokens'
 * original positions by the one RoPE configuration that cache building and
 * generation share (paperlayer section 3.3; rainbus prerequisites, RoPE
 * scaling).  Needs no layer; its outputs feed statekv_prefill_frame of a
 * layer made with rope_theta = 0, with first_position = position_offset +
 * n*T for frame n.
 *   x: device, [n_tokens][hidden] bf16;
 *   w: device, [(Hq + 2 Hkv) d][hidden] bf16, output-major: row r holds the
 *      weights of output feature r; rows [0, Hq d) are W_Q transposed (query
 *      head g = rows g d .. g d + d - 1), then W_K, then W_V, likewise;
 *   q: device, [n_tokens][Hq][d] bf16, k and v: [n_tokens][Hkv][d] bf16,
 *      written (must not overlap x or w);
 *   token t sits at position first_position + t; rope_theta > 0 rotates q and
 *   k (pairs (x_i, x_{i+d/2}), angle (p / rope_scaling) * rope_theta^(-2i/d),
 *   rope_scaling <= 0 means 1); rope_theta = 0 leaves them unrotated.
 * Arithmetic: fp32 accumulation of the bf16 products (in up to a few splits
 * of the hidden dimension, summed in split order: deterministic), the
 * rotation in double from the fp32 sums, one rounding to bf16 (nearest, ties
 * to even).
 * workspace: device, 256-byte aligned, at least the bytes that
 *   statekv_qkv_rope_workspace_size gives for these sizes (the splits' fp32
 *   partial sums); owned by the caller, not read across calls, and must not
 *   be in use by another call in flight.  NULL (workspace_bytes ignored): the
 *   library takes the bytes it needs, if any, with hipMallocAsync on `stream`
 *   and frees them with hipFreeAsync on `stream` after the last kernel.
 * Errors (host checks, nothing enqueued): STATEKV_ERR_INVALID_ARGUMENT for a
 * null or misaligned pointer, a non-positive size, Hq not a multiple of Hkv,
 * a negative first_position, rope_theta < 0, = 1 or not finite;
 * STATEKV_ERR_UNSUPPORTED for d other than 64/128, hidden not a multiple of
 * 64, or sizes beyond 2^20 tokens or features; STATEKV_ERR_WORKSPACE for a
 * workspace that is misaligned or smaller than needed; STATEKV_ERR_HIP if a
 * launch or the stream-ordered allocation fails.  Asynchronous on stream. */
int statekv_qkv_rope(const void* x, const void* w, int32_t n_tokens, int32_t hidden,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int64_t first_position, double rope_theta, double rope_scaling,
                     void* q, void* k, void* v, void* workspace, uint64_t workspace_bytes,
                     void* stream);

/* Bytes of the workspace statekv_qkv_rope needs for these sizes (0 if it does
 * not split the hidden dimension), written to *bytes.  Host only; the same
 * size errors as statekv_qkv_rope (STATEKV_ERR_INVALID_ARGUMENT /
 * _UNSUPPORTED), STATEKV_ERR_INVALID_ARGUMENT for a null `bytes`. */
int statekv_qkv_rope_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, uint64_t* bytes);

/* Views (host only; they enqueue nothing and never fail on a valid layer;
 * STATEKV_ERR_INVALID_ARGUMENT for a null argument).
 * statekv_state: the compressed state C_n, the fixed-capacity, importance-
 * selected temporal state that only the streaming prefill reads (rainbus
 * method steps: a compressed state of capacity B per layer; rainbus
 * technical novelty: this cache serves the video prefill only), plus the
 * importance of each candidate of the last frame's pool (the ranking that
 * chose C_n).
 * statekv_detailed_cache: the detailed state D_n, every visual token of every
 * frame so far, kept for the final text decoding (rainbus method steps: the
 * detailed state accumulates all visual tokens up to frame n; rainbus core
 * method and gist.science/nl "Het Proces": decoding runs over all video
 * tokens). */
int statekv_state(const statekv_layer* layer, statekv_state_view* out);
int statekv_detailed_cache(const statekv_layer* layer, statekv_cache_view* out);

/* Forget every frame (host only): empty C and D, frames_seen = 0. */
int statekv_reset_layer(statekv_layer* layer);

/* Resume a layer from a checkpoint (host only).  The natural checkpoint of a
 * layer after frame n-1 is (C_n rows with their positions, D[0 : n*T), n):
 * the caller writes them into the regions that statekv_state and
 * statekv_detailed_cache report (C rows [0, count) of k, v and pos in
 * ascending position, any order with SLOT_STABLE; D as the detailed view lays
 * it out), then calls this
 * so that the next statekv_prefill_frame processes frame frames_seen.
 * count must equal min(B, frames_seen * T) (STATEKV_ERR_INVALID_ARGUMENT
 * otherwise), and a linear D must hold frames_seen * T tokens
 * (STATEKV_ERR_CAPACITY).  The last frame's scores are not part of the
 * checkpoint (last_pool becomes 0). */
int statekv_restore_layer(statekv_layer* layer, int64_t frames_seen, int32_t count);

/* The App. A measurements of the last frame (paperlayer App. A.1-A.3), for a
 * layer that has kept every token so far (state_budget >= frames_seen * T;
 * STATEKV_ERR_INVALID_ARGUMENT otherwise, or before the first frame).  Such a
 * layer computes full attention, and the importance its last
 * statekv_prefill_frame left in the state view, summed over the KV heads, is
 * the pages' aggregate over the layer's heads and the frame's queries.  For
 * each budget b = budgets[i] (host array of n_budgets <= 64 values >= 1):
 *   out[3i]     share of the historical mass (tokens of earlier frames) held
 *               by the b largest historical importances (A.1);
 *   out[3i + 1] share held by the b most recent historical tokens (A.3);
 *   out[3i + 2] weighted candidate-pool recall (A.2): S_n = the b tokens
 *               through this frame with the largest importance (ties to the
 *               lower position); the share of S_n's importance inside S_{n-1}
 *               plus this frame's tokens.
 * out: device, 3 * n_budgets floats, NaN where a share is undefined (no
 * earlier frame).  sets: device, n_budgets * statekv_mass_set_words() words,
 * owned by the caller and kept between calls: S_{n-1} is read from it (when
 * frames_seen > 1) and S_n written to it (bit j of word j/32 set when token
 * j, counted from the first frame, is in the set).  Asynchronous on stream. */
int statekv_attention_mass(statekv_layer* layer, const int32_t* budgets,
                           int32_t n_budgets, uint32_t* sets, float* out, void* stream);
/* Words per budget of the sets buffer of statekv_attention_mass (host only). */
int statekv_mass_set_words(const statekv_layer* layer, int32_t* words);

/* The launch plan of the prefill step at a pool of `pool` candidates (c + T,
 * 1 <= pool <= B + T): the key splits of the output pass (each writes one fp32
 * O partial, summed in the select launch) and of the statistics pass, the row
 * tiles of one KV head's G*T query rows (256 rows each) and the pool's 64-key
 * tiles.  For callers that size or measure the step's traffic; host only, no
 * device work.  STATEKV_ERR_INVALID_ARGUMENT for a null argument or a pool out
 * of range. */
typedef struct {
  int32_t out_splits;   /* key splits of the output pass                      */
  int32_t stat_splits;  /* key splits of the statistics pass                  */
  int32_t row_tiles;    /* 256-row tiles per KV head                          */
  int32_t key_tiles;    /* ceil(pool / 64)                                    */
} statekv_launch_plan;
int statekv_launch_plan_for(const statekv_layer* layer, int32_t pool, statekv_launch_plan* out);

/* Release the host handle (the workspace stays the caller's). */
int statekv_free_layer(statekv_layer* layer);

/* Human-readable name of a status code (static storage). */
const char* statekv_status_string(int status);

/* Kernels of the per-frame and decoding calls, for the timing hooks below. */
enum {
  STATEKV_KERNEL_ATTN_STATS = 0, /* attention pass 1: row statistics           */
  STATEKV_KERNEL_ATTN_OUT = 1,   /* attention pass 2: O, importance partials   */
  STATEKV_KERNEL_SPLIT_SUM = 2,  /* split combine of the full-attention baseline
                                    and of decoding (the StateKV path sums its
                                    split O partials in the SELECT launch)      */
  STATEKV_KERNEL_SELECT = 3,     /* importance sums + top-B select + O split sum
                                    (with SLOT_STABLE also the state moves and
                                    the detailed-cache append)                  */
  STATEKV_KERNEL_GATHER = 4,     /* C_n gather + detailed-cache append (not
                                    launched with SLOT_STABLE)                  */
  STATEKV_KERNEL_DECODE = 5,     /* decoding over D: split partials            */
  STATEKV_KERNEL_ROPE = 6,       /* in-library rotary embedding of the frame   */
  STATEKV_KERNEL_MASS = 7,       /* App. A diagnostics                         */
  STATEKV_NUM_KERNELS = 8
};

/* Timing hooks for benchmarks (measurement only; results are unaffected).
 * statekv_profile_start: from now on every statekv_prefill_frame (and
 * statekv_full_attention_frame: its attention kernel counts as ATTN_OUT, its
 * split combine as SPLIT_SUM, its append as GATHER) records a
 * HIP event on its stream immediately before and after each kernel whose bit
 * is set in kernel_mask (1u << STATEKV_KERNEL_*), for at most max_records
 * kernel launches (further launches are not recorded).  The events are
 * created here, on the current device.
 * statekv_profile_stop: waits for the recorded events, writes per kernel the
 * summed event-to-event milliseconds (total_ms[STATEKV_NUM_KERNELS]) and the
 * number of recorded launches (launches[STATEKV_NUM_KERNELS]), stops
 * recording and destroys the events.  Either output may be NULL. */
int statekv_profile_start(statekv_layer* layer, uint32_t kernel_mask, int32_t max_records);
int statekv_profile_stop(statekv_layer* layer, double* total_ms, int64_t* launches);

/* The top-B select used inside the step (rainbus method steps and paperlayer
 * section 3.3: C_n = the B candidates of C_{n-1} plus the frame with the
 * largest summed attention weight; ties to the lower position are this
 * library's reading, the pages leave ties open), exposed for bit-exact
 * testing: of the n fp32 scores (device, non-negative or +0; NaN ranks lowest), keep
 * min(budget, n) indices -- larger score first, ties to the lower index -- and
 * write them in ascending index order to d_out_idx (device, >= min(budget,n)
 * int32).  1 <= n <= 32768, budget >= 1. */
int statekv_select_topb(const float* d_scores, int32_t n, int32_t budget,
                        int32_t* d_out_idx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STATEKV_H_ */
