/*
 * mor.h -- C ABI of the MI355X (gfx950) Mixture-of-Recursions forward-pass library.
 *
 * The method: a Llama-style pre-norm Transformer unrolled to L layers with
 * Middle-Cycle weight tying (a unique first layer, n_s = (L-2)/N_r shared layers
 * cycled N_r times, a unique last layer), in which a router keeps a shrinking set
 * of tokens at every recursion and attention at a recursion reads only the keys
 * and values of tokens active at that same recursion.
 * Sources: "Mixture-of-Recursions: Learning Dynamic Recursive Depths for Adaptive
 * Token-Level Computation" (Appendix A.1 sharing, A.2 routing, A.3 KV caching,
 * Appendix D FLOP accounting) and the "Mixture-of-Recursions: Adaptive Token Depth"
 * reading notes (section 1 parameter sharing, 2.1 expert-choice, 2.2 token-choice,
 * 3.1 recursion-wise caching, 3.2 recursive KV sharing, 4 depth-wise batching).
 *
 * Conventions for every call:
 *  - Every pointer named "device" is GPU memory owned by the caller. The library never
 *    allocates or frees device memory: all scratch lives in the caller's workspace.
 *  - "stream" is a hipStream_t passed as void*. All work is enqueued on it; results are
 *    valid once the stream has completed. No call synchronises the stream unless it says so.
 *  - Arguments are validated before anything is enqueued: an error status means nothing
 *    was launched. MOR_E_HIP means a HIP call failed and the stream state is undefined.
 *  - mor_last_error() returns a thread-local message for the last failing call.
 *  - A handle is not thread-safe; calls on one handle must not overlap.
 *  - Matrices are row-major. Weight matrices are [out][in] (y = x W^T), in the config dtype
 *    (fp32 or bf16). Hidden states, norm gains and router weights are fp32.
 */
#ifndef MOR_H
#define MOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOR_ABI_VERSION 3
#define MOR_MAX_REC 8
#define MOR_MAX_SHARED 64

typedef enum {
  MOR_OK = 0,
  MOR_E_INVALID = -1,   /* bad argument (null pointer, out-of-range value)              */
  MOR_E_SHAPE = -2,     /* shapes the kernels do not support, or beyond the init bounds */
  MOR_E_WORKSPACE = -3, /* workspace smaller than mor_workspace_bytes()                 */
  MOR_E_KV_FULL = -4,   /* decode KV page pool exhausted                                */
  MOR_E_HIP = -5,       /* a HIP runtime call failed                                    */
  MOR_E_STATE = -6      /* call not valid in the handle's current state                */
} mor_status;

typedef enum { MOR_F32 = 0, MOR_BF16 = 1 } mor_dtype;

/* Routing (reading notes 2.1 / 2.2):
 *  EC_TOPK:      at recursion r the router logit z = theta_r . H scores the tokens active at
 *                r-1 and the ceil(cap_r * T) best of each sequence continue (expert choice).
 *  TOKEN_CHOICE: after the first layer, z_j = Theta_j . H (j = 1..N_r), depth = argmax_j z_j
 *                (lowest j on ties); recursion r runs the tokens with depth >= r.
 *  THRESHOLD:    recursion 1 runs every token; at r >= 2 a token continues iff
 *                theta_r . H + b_r > 0 (the static sigmoid > 0.5 test used at inference). */
typedef enum { MOR_ROUTE_EC_TOPK = 0, MOR_ROUTE_TOKEN_CHOICE = 1, MOR_ROUTE_THRESHOLD = 2 } mor_routing;
/* KV caching (MoR paper A.3; reading notes 3.1 / 3.2):
 *  RECURSION_WISE: each (recursion, shared layer) keeps the K/V of the tokens active there and
 *                  attention at that recursion reads only those.
 *  SHARE_FIRST:    recursions >= 2 compute no K/V and attend to the recursion-1 K/V of the
 *                  same shared layer (all recursion-1 tokens at positions <= the query's). */
typedef enum { MOR_KV_RECURSION_WISE = 0, MOR_KV_SHARE_FIRST = 1 } mor_kv_mode;
/* Gate of the recursion update: ROUTER merges H + g (F(H) - H) with g = sigmoid(z) (expert choice,
 * threshold) or the chosen-depth softmax weight (token choice); UNIT assigns H = F(H). */
typedef enum { MOR_GATE_ROUTER = 0, MOR_GATE_UNIT = 1 } mor_gate_mode;
/* Parameter sharing (MoR paper A.1; reading notes section 1): how the L unrolled layers map onto
 * the pool of n_s shared blocks. The N_r routed recursions are consecutive spans of n_s layers.
 *  MIDDLE_CYCLE:    unique first and last layers; n_s = (L-2)/N_r; position j of every recursion
 *                   uses shared block j (the MoR default).
 *  MIDDLE_SEQUENCE: unique first and last layers; interior layer u = 0..L-3 uses block u / N_r.
 *  CYCLE:           no unique layers; n_s = L/N_r; position j of every recursion uses block j.
 *  SEQUENCE:        no unique layers; layer u = 0..L-1 uses block u / N_r.
 * Without unique layers recursion 1 routes the input H^0 and the output is H after recursion N_r.
 * Depth-wise batched decode (max_slots > 0) needs MIDDLE_CYCLE: it runs one position j for every
 * depth with the same block. Under SHARE_FIRST a recursion r >= 2 layer reads the recursion-1
 * K/V of the same position j. */
typedef enum {
  MOR_SHARE_MIDDLE_CYCLE = 0, MOR_SHARE_MIDDLE_SEQUENCE = 1, MOR_SHARE_CYCLE = 2, MOR_SHARE_SEQUENCE = 3
} mor_sharing;

typedef struct {
  int32_t d_model, n_q_heads, n_kv_heads, head_dim, d_ff;
  int32_t n_layers;              /* L, unrolled depth (unique first and last layer included)      */
  int32_t n_rec;                 /* N_r, 1..MOR_MAX_REC; (L - 2) % N_r == 0 under MIDDLE_* sharing,
                                    L % N_r == 0 otherwise                                       */
  int32_t cap_num[MOR_MAX_REC];  /* capacity of recursion r = cap_num[r-1] / cap_den, non-increasing, <= 1 */
  int32_t cap_den;
  int32_t routing;               /* mor_routing   */
  int32_t kv_mode;               /* mor_kv_mode   */
  int32_t gate_mode;             /* mor_gate_mode */
  int32_t dtype;                 /* mor_dtype     */
  float rms_eps;                 /* RMSNorm epsilon (1e-5)      */
  float rope_theta;              /* RoPE base (10000)            */
  int32_t max_batch, max_seq;    /* prefill bounds the workspace is planned for; max_seq also bounds
                                    decode positions */
  /* Depth-wise batched decode (reading notes section 4). max_slots = 0 plans no decode state. */
  int32_t max_slots;             /* concurrent sequences, 0..64 (needs THRESHOLD routing)          */
  int32_t kv_page_tokens;        /* tokens per KV page: 16, 32, 64 or 128                           */
  int32_t kv_pages;              /* pages in the pool; 0 = enough for max_slots sequences of max_seq
                                    tokens that all run every recursion                             */
  int32_t max_requests;          /* requests one mor_decode_submit may queue                       */
  int32_t sharing;               /* a mor_sharing value, 0 = MIDDLE_CYCLE                           */
} mor_config;

/* One Llama decoder layer. All device pointers. [out][in] matrices in the config dtype:
 * wq [Hq*hd][d], wk [Hkv*hd][d], wv [Hkv*hd][d], wo [d][Hq*hd], w_gate [d_ff][d],
 * w_up [d_ff][d], w_down [d][d_ff]; fp32 RMSNorm gains g_attn [d], g_ffn [d]. */
typedef struct {
  const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
  const float *g_attn, *g_ffn;
} mor_block_weights;

typedef struct {
  mor_block_weights first, last;    /* unique layers (ignored under CYCLE and SEQUENCE sharing)     */
  const mor_block_weights* shared;  /* host array of the n_s shared blocks (block j = 1..n_s)       */
  const float* router_w;            /* device fp32 [N_r][d]: row r-1 is theta_r (EC, threshold) or Theta_r (TC) */
  const float* router_b;            /* device fp32 [N_r] (threshold biases b_r), or NULL for zeros */
} mor_weights;

typedef struct mor_handle_s mor_handle;

int32_t mor_abi_version(void);
const char* mor_last_error(void);

/* Bytes of device workspace mor_init needs for this config (packed weights, activations for
 * max_batch x max_seq tokens, the per-recursion KV caches, routing state, and, with max_slots > 0,
 * the decode engine and its KV page pool). 0 if cfg is invalid. */
size_t mor_workspace_bytes(const mor_config* cfg);

/* Validate cfg, plan the workspace, copy/pack the weights into it and upload the RoPE table
 * (cos/sin of pos * theta^(-2i/hd), evaluated in double, stored fp32). Synchronises `stream`
 * once at the end. The weight buffers may be freed after this call returns.
 * Errors: MOR_E_INVALID, MOR_E_SHAPE (d_model % 64, d_ff % 64, head_dim not in {16, 32, 64} for
 * fp32 / not 64 for bf16, Hq % Hkv, Hq/Hkv > 4, max_seq > 8192), MOR_E_WORKSPACE, MOR_E_HIP. */
mor_status mor_init(const mor_config* cfg, const mor_weights* w, void* workspace,
                    size_t workspace_bytes, void* stream, mor_handle** out);

/* MoR prefill of B sequences of T tokens (MoR paper A.1-A.3; reading notes 1, 2, 3).
 *   h_in   device fp32 [B][T][d]   input hidden states H^0.
 *   h_out  device fp32 [B][T][d]   output H^L after the last layer (no final norm, no LM head).
 *                                  May equal h_in (then h_in is overwritten); must not
 *                                  otherwise overlap it. Also serves as the fp32 residual
 *                                  stream. With a unique first layer, h_in is only read by that
 *                                  layer (no copy of it is made).
 * Optional outputs (NULL to skip), all device memory:
 *   sel_pos   int32 [N_r][B][T]  positions of the tokens active at recursion r, ascending, -1 padded.
 *   counts    int32 [N_r][B]     number of active tokens per recursion and sequence.
 *   logits    fp32  [N_r][B][T]  EC/threshold: z^r_t for t active at r-1 (NaN elsewhere);
 *                                TC: Theta_r . H^1_t for every t.
 *   h_per_rec fp32  [N_r+1][B][T][d] H after the first layer (the input under CYCLE / SEQUENCE
 *                                sharing) and after each recursion.
 * Router logits are computed in fp32 in one fixed order: lane l (0..63) accumulates
 * p = p + x[i]*w[i] over i = l, l+64, ... with the product and the sum rounded separately,
 * then p = p + p[l+o] for o = 32,16,...,1; bias, if any, is added last. Expert-choice selects
 * by z descending, then position ascending; -0 counts as +0; NaN ranks last and sets
 * error flag bit 0 (mor_get_error_flags).
 * The K/V of every layer are left in the workspace cache (mor_kv_view).
 * Errors: MOR_E_INVALID (null pointers), MOR_E_SHAPE (B, T outside 1..max), MOR_E_HIP. */
mor_status mor_prefill(mor_handle* h, const float* h_in, int32_t B, int32_t T, float* h_out,
                       int32_t* sel_pos, int32_t* counts, float* logits, float* h_per_rec,
                       void* stream);

/* Routing stage alone, for testing the router kernels (the same kernels mor_prefill runs).
 * Given H^r (device fp32 [B][T][d]) and the set active at r-1 (device int32 active_in [B][T],
 * ascending positions, count in counts_in [B]), computes z^r (fixed order above, plus b_r in
 * threshold mode) into z_out [B][T] (NaN outside the active set) and the set active at r into
 * active_out [B][T] (-1 padded) and counts_out [B]. r is 1-based. EC and threshold routing only
 * (MOR_E_STATE for token choice). */
mor_status mor_route(mor_handle* h, const float* H, const int32_t* active_in,
                     const int32_t* counts_in, int32_t r, int32_t B, int32_t T,
                     int32_t* active_out, int32_t* counts_out, float* z_out, void* stream);

/* mor_route without scratch in the workspace, for callers that cannot allocate or must not touch
 * workspace memory another call may be using: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, kernels and results as mor_route (router
 * logits, selection, counts and the NaN error flag bitwise equal); the handle supplies only the
 * router weights and the error flag. Its scratch (row offsets and the row map of the active set)
 * is a static device array of (MOR_NOALLOC_MAX_BATCH + 1 + MOR_NOALLOC_MAX_TOKENS) int32 (about
 * 266 KB), one per GPU, held until the process ends and bound to its device address by mor_init.
 * The call allocates nothing. Every call on a GPU shares that GPU's array (whatever the handle),
 * so calls that may overlap on one GPU (other streams, other threads) race: serialise them.
 * Nothing in the array needs clearing between calls (each call writes what it reads).
 * Errors: those of mor_route, and MOR_E_SHAPE if B > MOR_NOALLOC_MAX_BATCH or
 * B*T > MOR_NOALLOC_MAX_TOKENS (nothing is launched then). */
#define MOR_NOALLOC_MAX_BATCH 1024
#define MOR_NOALLOC_MAX_TOKENS 65536
mor_status mor_route_noalloc(mor_handle* h, const float* H, const int32_t* active_in,
                             const int32_t* counts_in, int32_t r, int32_t B, int32_t T,
                             int32_t* active_out, int32_t* counts_out, float* z_out, void* stream);

/* Where the K/V cache of one layer stream lives after mor_prefill.
 * stream 0 = first layer, 1 + (r-1)*n_s + (j-1) = position j of recursion r, 1 + N_r*n_s = last
 * (streams 0 and 1 + N_r*n_s are not written under CYCLE / SEQUENCE sharing).
 * K is [B][kpad][Hkv][hd] (row = index of the token in that recursion's active list) and
 * V is stored transposed as [B][Hkv][hd][kpad]; kpad = max_seq rounded up to 64; dtype = config.
 * Under SHARE_FIRST the streams of recursions >= 2 are not written. */
mor_status mor_kv_view(mor_handle* h, int32_t stream, const void** k, const void** v_t,
                       int32_t* kpad);

/* Reads and clears the device error flags (bit 0: a NaN router logit). Synchronises `stream`. */
mor_status mor_get_error_flags(mor_handle* h, void* stream, uint32_t* flags);

/* Measurement hooks. mor_timing_enable makes later calls record a pair of HIP events, on the
 * call's stream, around every launch of one kernel kind of mor_prefill: 1 QKV projection,
 * 2 attention, 3 output projection, 4 gate/up projection (SwiGLU), 5 down projection, 6 router
 * logits of recursion 1 (all tokens; token-choice router included), 7 top-k / threshold
 * selection with compaction, 8 gather of the active rows, 9 gated scatter (with the next
 * recursion's router logits), 10 RMSNorm; 0 turns it off.
 * At most max_launches launches are recorded (events are created here, not during calls).
 * mor_timing_read waits for the last recorded event, returns the summed kernel time in ms and
 * the number of recorded launches, and clears the record. */
mor_status mor_timing_enable(mor_handle* h, int32_t kind, int32_t max_launches);
mor_status mor_timing_read(mor_handle* h, double* total_ms, int32_t* launches);
/* Shader clock during the recorded launches of a bf16 projection kind (1, 3, 4, 5): each such
 * launch's first workgroup counts shader cycles and constant-rate real-time ticks over its life;
 * *ghz = cycles / ticks x the real-time rate, summed over the launches recorded since
 * mor_timing_enable (which clears the sums), or 0 when none were sampled. Synchronises the
 * device. */
mor_status mor_timing_clock(mor_handle* h, double* ghz);

/* ---------------------------------------------------------------- depth-wise batched decode
 * Continuous depth-wise batching (reading notes section 4) of the threshold-routed model (reading
 * notes 2.1: at inference a token continues to recursion r >= 2 iff theta_r . H + b_r > 0, i.e.
 * sigmoid > 0.5; recursion 1 always runs). Up to max_slots requests are in flight, one token each.
 * Every decode iteration advances every occupied slot by one recursion: a token that enters runs
 * the first layer, all occupied slots run the n_s shared layers at their own recursion (one launch
 * per operation for all depths), and a token whose next logit is not positive, or that finished
 * recursion N_r, runs the last layer and writes its output. The slot then takes the request's next
 * token at the next iteration (one token per request in flight keeps the autoregressive order), or,
 * when the request is finished, the next queued request (FIFO, lowest free slot first).
 * The KV caches are paged per (request, layer stream): the first layer, the last layer, and each
 * shared layer at each recursion (recursion-wise caching, MoR paper A.3), or at recursion 1 only
 * under SHARE_FIRST (recursions >= 2 then read the recursion-1 pages). Pages are taken from a
 * device free list when a stream's token count reaches a page boundary and returned when the
 * request finishes. Results of a token do not depend on which other requests share the batch.
 *
 * mor_decode_submit resets the engine and queues n_req requests (discarding unfinished work).
 *   lengths    host int32 [n_req], each 1..max_seq; request i's tokens occupy rows
 *              off_i .. off_i + len_i - 1 of the token arrays, off_i = sum of earlier lengths.
 *   inputs     device fp32 [sum len][d]  input hidden state of every token.
 *   outputs    device fp32 [sum len][d]  hidden state after the last layer (no norm, no LM head).
 *   exit_depth device int8 [sum len]     recursions the token ran (1..N_r).
 *   h_dump     device fp32 [sum len][N_r + 1][d] or NULL: H after the first layer and after each
 *              recursion the token ran (other rows untouched).
 *   z_dump     device fp32 [sum len][N_r] or NULL: router logit z^r (bias included) for every
 *              recursion whose gate or exit test was evaluated; the rest is set to NaN.
 * The buffers must stay valid until the requests are finished.
 * Errors: MOR_E_STATE (handle planned without decode), MOR_E_INVALID, MOR_E_SHAPE (n_req >
 * max_requests, a length outside 1..max_seq), MOR_E_HIP. */
mor_status mor_decode_submit(mor_handle* h, int32_t n_req, const int32_t* lengths,
                             const float* inputs, float* outputs, int8_t* exit_depth,
                             float* h_dump, float* z_dump, void* stream);

/* Prefill -> decode hand-over: the n_req requests continue the n_req sequences of the last
 * mor_prefill on this handle (same batch B = n_req <= max_slots, threshold routing). Request b's
 * tokens take positions T .. T + lengths[b] - 1 (T = the prefill's sequence length), and its
 * attention at every layer and recursion also reads the K/V the prefill cached for sequence b at
 * that layer and recursion (the prefill's caches are copied into the request's pages; slot b
 * holds request b). With threshold routing the result equals the prefill of the whole sequence.
 * Arguments and token-array layout as mor_decode_submit (rows are the continuation tokens only).
 * Errors: MOR_E_STATE (no prefill, no decode state, or not threshold routing), MOR_E_SHAPE
 * (n_req != prefill batch, n_req > max_slots, T + length > max_seq), MOR_E_INVALID, MOR_E_HIP. */
mor_status mor_decode_continue(mor_handle* h, int32_t n_req, const int32_t* lengths,
                               const float* inputs, float* outputs, int8_t* exit_depth,
                               float* h_dump, float* z_dump, void* stream);

/* Enqueues n_iters decode iterations on `stream` (no host synchronisation). If progress is not
 * NULL it then synchronises and writes {tokens finished, requests finished, iterations run} of
 * the current submission into progress[0..2].
 * MOR_E_KV_FULL: the page pool ran out; the engine stopped at that iteration (its tokens are
 * not finished) and stays stopped until the next submit. Checked only when progress is given. */
mor_status mor_decode_step(mor_handle* h, int32_t n_iters, void* stream, int32_t* progress);

/* Synchronises `stream` and reports the current submission (measurement):
 *   out[0] tokens finished, out[1] requests finished, out[2] requests admitted from the queue,
 *   out[3] iterations run, then the algorithmic bytes of those iterations: out[4] weights (every
 *   layer that ran for at least one token, once per iteration), out[5] K/V read from the cache,
 *   out[6] K/V appended, out[7] input and output rows; out[8] the most KV pages in use at once,
 *   out[9] bytes per page. out has room for 10 values. */
mor_status mor_decode_stats(mor_handle* h, void* stream, int64_t* out);

/* Frees the host-side handle. The workspace stays the caller's. NULL is ignored. */
void mor_destroy(mor_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MOR_H */
