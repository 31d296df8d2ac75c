/*
 * gr_beam.h -- C ABI of the semantic-ID beam-search decode step on one AMD
 * Instinct MI355X (gfx950).
 *
 * The calls follow the serving pattern of generative recommendation with
 * semantic IDs as described in the zhiding.cn article on NVIDIA
 * recsys-examples, section "语义ID生成式推荐专用推理框架" (semantic-ID
 * generative-recommendation inference framework): a long user context that
 * every beam shares (ContextKV), a short per-beam decode history (BeamKV), the
 * logical ancestry of each beam (BeamPath), wide and dynamic beam widths, and
 * item-constrained generation with an item-constrained top-K; and the
 * multi-beam return of the paper-daily summary "Advancing Generative
 * Recommendation Inference", section "Background" (return every surviving
 * beam, not only the best one).
 *
 * Model stand-in.  The pages give no model for this step beyond naming
 * Qwen3-1.7B.  The library computes, per decode step s of request r and beam j
 * with code prefix c_0..c_{s-1}:
 *   - per layer l and query head hq (kv head hq / (Hq/Hkv)):
 *       query  q = q_last[r][l][hq]                 (s = 0)
 *              q = tok_q[l][s-1][c_{s-1}][hq]       (s >= 1)
 *       keys   the request's context keys, then tok_k[l][t][c_t] for t < s
 *       values likewise; o_l = softmax(q K^T / sqrt(d)) V
 *   - hidden h = sum_l o_l, head-major (hq*d + i), float32
 *   - logits = h @ w_sid[s]   (float32)
 *   - log-softmax over the codes that extend a valid item prefix (GR_NORM_VALID)
 *     or over all codes (GR_NORM_FULL), keeping only valid codes
 *   - candidate score = beam score + log-prob; the next beam set holds the
 *     min(W, #valid candidates) best candidates over all beams x codes, ordered
 *     by score descending, then by flat index j*V + c ascending.
 * The context is stored once per request; a beam's own tokens are written
 * once into BeamKV and found again through BeamPath, never copied on reorder.
 *
 * Conventions
 *   - Every call returns gr_status; on failure gr_last_error() gives a
 *     thread-local message.  No exception or abort crosses the ABI.
 *   - After a HIP runtime error the engine is poisoned: later calls on it
 *     return GR_E_DEVICE.
 *   - "device" pointers are HIP device memory (e.g. torch CUDA tensors on
 *     ROCm); "host" pointers are ordinary process memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device work
 *     of a call is enqueued on it; an engine must be used from one host thread
 *     and one stream at a time.
 *   - The caller owns every buffer it passes, including the workspace; the
 *     engine sub-allocates the workspace.  Its own allocations are a small ring
 *     of pinned host buffers for per-step work descriptors, timing and ordering
 *     events and three auxiliary streams (all at bind time), the prefill staging
 *     of gr_engine_set_prefill (a pinned token buffer, grown by gr_ctx_prefill
 *     when a longer context comes, and a small device area for the soft token),
 *     and a scheduler's pinned result buffers (gr_sched_create).  No decode-step
 *     call allocates.
 */
#ifndef GR_BEAM_H
#define GR_BEAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GR_OK = 0,
  GR_E_INVALID_ARG = 1,   /* a bad argument; nothing was changed */
  GR_E_OUT_OF_MEMORY = 2, /* workspace, request slots or context pool exhausted */
  GR_E_BAD_STATE = 3,     /* call not valid in the object's current state */
  GR_E_NOT_FOUND = 4,     /* unknown request id */
  GR_E_DEVICE = 5,        /* a HIP runtime error; the engine is poisoned */
  GR_E_UNSUPPORTED = 6    /* valid but unsupported shape (see limits below) */
} gr_status;

typedef enum { GR_DTYPE_F32 = 0, GR_DTYPE_BF16 = 1 } gr_dtype;

/* Normalisation domain of the item-constrained log-softmax. */
typedef enum {
  GR_NORM_VALID = 0, /* over the codes that extend a valid item prefix (default) */
  GR_NORM_FULL = 1   /* over the whole codebook, then restricted to valid codes */
} gr_norm;

typedef struct gr_engine gr_engine; /* opaque */

/* The layer-chain model: a pre-norm decoder of the Qwen3-1.7B shape the pages run the decode on
 * ([TRT] section "Performance"; [GR] section "语义ID生成式推荐专用推理框架"), with layer l+1's
 * new-token query, key and value computed from layer l's output.  D = n_q_heads * head_dim.  Per
 * step s and beam with codes c_0..c_{s-1}, the new token's input vector x is embed[s-1][c_{s-1}]
 * (s >= 1) or the request's x_last (s = 0; that token's key and value are the context's last
 * row, so it attends to the context only).  Per layer l, with RMSNorm(x, g) = x / sqrt(mean(x^2)
 * + rms_eps) * g and b() rounding to bf16 (nearest even):
 *   xn = b(RMSNorm(x, g_attn[l])); q = b(xn w_q[l]^T), k = b(xn w_k[l]^T), v = b(xn w_v[l]^T)
 *   o  = attention of q over the context and the beam's own tokens (k, v of each at layer l)
 *   x += b(o) w_o[l]^T
 *   xm = b(RMSNorm(x, g_mlp[l])); x += b(silu(xm w_gate[l]^T) * (xm w_up[l]^T)) w_down[l]^T
 * and the hidden vector is RMSNorm(x, g_final) (float32), projected by w_sid as in the stand-in.
 * The projections run in float32 on bf16 inputs; the residual x is float32.  Every matrix is
 * device memory, bf16, row-major "out x in" (K contiguous).  Limits: bf16; n_q_heads * head_dim
 * and n_kv_heads * head_dim multiples of 128; intermediate a positive multiple of 64. */
typedef struct {
  int32_t intermediate;      /* MLP width I */
  float rms_eps;             /* > 0 */
  const void *embed;         /* device [n_levels-1][V][D] */
  const void *w_q;           /* device [L][n_q_heads*head_dim][D] */
  const void *w_k, *w_v;     /* device [L][n_kv_heads*head_dim][D] */
  const void *w_o;           /* device [L][D][n_q_heads*head_dim] */
  const void *w_gate, *w_up; /* device [L][I][D] */
  const void *w_down;        /* device [L][D][I] */
  const float *g_attn;       /* device [L][D] */
  const float *g_mlp;        /* device [L][D] */
  const float *g_final;      /* device [D] */
} gr_chain_desc;

/* The label head for scoring given candidates by label tokens ([TRT] sections "Background" and
 * "Scoring many candidates at once": the candidates go into the prompt, each sees only the shared
 * prefix and itself, and the model's log-probabilities of label tokens such as "yes" and "no",
 * read after each candidate, rank them).  With a label head the token tables hold n_levels levels
 * instead of n_levels - 1: level n_levels - 1 gives a candidate's last code its query, key and
 * value, so that code runs as a token (attending to the context, the candidate's earlier codes and
 * itself), and its hidden vector h (as the step's hidden vector: the sum over layers of the
 * attention outputs) gives z_c = h . w_label[:, c] and the label log-probabilities z_c -
 * logsumexp(z) over the n_labels outputs.  Limits: 1 <= n_labels <= 16; not with a layer chain. */
typedef struct {
  int32_t n_labels;
  const float *w_label; /* device [n_q_heads*head_dim][n_labels] float32 */
} gr_label_desc;

/* Model description.  Limits: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0;
 * n_q_heads * head_dim a multiple of 128; 1 <= n_levels <= 8; 2 <= codebook_size <= 1024
 * and codebook_size**n_levels < 2**62.
 * All table pointers are device memory owned by the caller and must outlive
 * the engine.  Element type of tok_q/tok_k/tok_v is `dtype` (bf16 = raw 16-bit
 * patterns, f32 = float). */
typedef struct {
  int32_t n_layers, n_q_heads, n_kv_heads, head_dim;
  int32_t n_levels, codebook_size;
  int32_t dtype; /* gr_dtype: ContextKV, BeamKV and token tables */
  int32_t norm;  /* gr_norm */
  const void *tok_q;   /* device [L][T][V][Hq][d]  (the stand-in; unused by a chain); T = n_levels-1,
                          or n_levels with a label head */
  const void *tok_k;   /* device [L][T][V][Hkv][d] */
  const void *tok_v;   /* device [L][T][V][Hkv][d] */
  const float *w_sid;  /* device [n_levels][Hq*d][V] float32 */
  const gr_chain_desc *chain; /* host, read at gr_engine_create: the layer-chain model; NULL = the
                                 table stand-in above */
  const gr_label_desc *label; /* host, read at gr_engine_create: the label head; NULL = none */
} gr_model_desc;

/* The valid items: distinct code tuples (duplicates are tolerated and merged).
 * Host memory, read during gr_engine_create only. */
typedef struct {
  int64_t n_items;
  const int32_t *codes; /* host [n_items][n_levels], each code in [0, V) */
} gr_item_set;

#define GR_ENGINE_DEBUG_ATTN 1u /* keep every layer's attention output for gr_debug_attn_out */
/* One context-attention launch per layer at every level, the launch sequence of a model whose
 * layer l+1 reads layer l's output: no launch covers two layers (the first level included).  A
 * layer whose row blocks fill the chip runs each block over the whole context; otherwise the
 * context is split into token ranges whose partials the next layer's launch merges.  Without
 * this flag the engine may run several layers in one launch where every layer's query is an
 * input (the model stand-in above). */
#define GR_ENGINE_PER_LAYER 2u
/* Graph replay of decode steps ([GR] section "语义ID生成式推荐专用推理框架": the runtime replays
 * captured graphs over views of the KV pool): gr_beam_step captures the launch sequence of each
 * step shape (the request count and the per-request parameters that set every launch) once, on
 * an engine-owned stream, as a HIP graph, and replays it for every later step of that shape; the
 * step's descriptors are uploaded to one fixed device area before each replay.  A new shape costs
 * a capture and an instantiation (host time and a little device memory; up to 64 shapes are kept,
 * the oldest dropped first).  Steps with profiling enabled, debug engines and the label step are
 * launched directly.  Results are the same as without the flag, bit for bit. */
#define GR_ENGINE_GRAPH 4u

typedef struct {
  int32_t max_requests;   /* requests loaded at once (slots), >= 1 */
  int32_t max_beam_width; /* largest beam width W of any request, 1..1024 */
  int64_t max_ctx_tokens; /* context tokens the engine's own pool holds for copy loads
                             (each request takes its length rounded up to 64);
                             0 = only GR_LOAD_ADOPT loads */
  int32_t max_splits;     /* split-K partial slots per (request, kv head) at full beam width
                             (narrower steps may use proportionally more); 0 = 4 */
  uint32_t flags;         /* GR_ENGINE_DEBUG_ATTN | GR_ENGINE_PER_LAYER | GR_ENGINE_GRAPH */
  int32_t max_layers_per_launch; /* full-context steps: at most this many layers per
                             context-attention launch; 0 = automatic (about seven rounds of
                             workgroups per launch, layers split evenly over the launches);
                             GR_ENGINE_PER_LAYER forces 1 */
} gr_engine_opts;

/* ---- engine lifetime ------------------------------------------------------ */

/* Validates the description, builds the item trie (per level: a bit mask of
 * valid next codes and the index of the first child for every valid prefix)
 * on the host.  Makes no HIP call.  *out receives the engine. */
gr_status gr_engine_create(const gr_model_desc *model, const gr_item_set *items,
                           const gr_engine_opts *opts, gr_engine **out);

/* Bytes of device workspace the engine needs (trie, per-slot BeamKV,
 * BeamPath, hidden/logit/partial buffers, context pool).  0 on a NULL engine. */
size_t gr_engine_workspace_bytes(const gr_engine *eng);

/* Hands the engine its workspace (device memory, 256-byte aligned, at least
 * gr_engine_workspace_bytes bytes, owned by the caller and kept alive until
 * gr_engine_destroy) and uploads the trie on `stream`.  Once per engine. */
gr_status gr_engine_bind_workspace(gr_engine *eng, void *workspace, size_t bytes, void *stream);

/* Synchronises the engine's last stream, frees host state and pinned buffers.
 * Does not free the workspace or any caller buffer.  NULL is a no-op. */
gr_status gr_engine_destroy(gr_engine *eng);

/* Trie statistics (host): number of valid prefixes of length `level`
 * (level 0 -> 1 root, level n_levels -> number of distinct items). */
gr_status gr_engine_trie_nodes(const gr_engine *eng, int32_t level, int64_t *n_nodes);

/* ---- requests ------------------------------------------------------------- */

/* Context length padded for the native ContextKV layout (multiple of 64). */
int32_t gr_ctx_padded_len(int32_t ctx_len);

#define GR_LOAD_ADOPT 1u /* k/v already in the native layout: view them, copy nothing */

/* Admits request `request_id` with its shared context and creates its root
 * beam (empty prefix, score 0): the "long shared context loaded once" of [GR] section
 * "语义ID生成式推荐专用推理框架" (ContextKV, shared by every beam of the request).
 *   ctx_len    N >= 1 context tokens;  beam_width 1 <= W <= max_beam_width.
 *   q_last     device [L][Hq][d] (dtype): query of the last context token,
 *              used at decode step 0; copied.  Layer-chain model: device [D] float32, the
 *              last context token's input vector x_last.
 *   flags = 0: k, v are device [L][N][Hkv][d] (dtype); copied and re-laid-out
 *              into the engine's context pool (stream-ordered; the sources may be
 *              freed once the stream has passed this call).
 *   flags = GR_LOAD_ADOPT: k is K in the native layout [L][Hkv][Np][d] and v is
 *              V transposed, [L][Hkv][d][Np], Np = gr_ctx_padded_len(N); tokens
 *              N..Np-1 must be zero.  The engine only keeps the pointers: the
 *              buffers must stay alive and unchanged until gr_request_release.
 *   k and v are 16-byte aligned in both cases.  Either way one pass over the
 *   context also takes, per (layer, kv head), the largest key norm and the
 *   largest |v| (bounds that the attention kernels use).  A copy load of a bf16
 *   model with head_dim 128 also keeps V^T as float16, in the units the wide
 *   attention kernel computes in, so that kernel reads it without converting
 *   (the pool then takes 3*L*Hkv*d*2 bytes per token, else 2*L*Hkv*d*dtype
 *   size); adopted contexts are converted inside the kernel, with the same
 *   result.
 * Errors: GR_E_INVALID_ARG (bad sizes, duplicate id, misaligned k or v),
 * GR_E_OUT_OF_MEMORY (no free slot or pool space), GR_E_BAD_STATE (workspace not
 * bound). */
gr_status gr_ctx_kv_load(gr_engine *eng, int64_t request_id, int32_t ctx_len, int32_t beam_width,
                         const void *k, const void *v, const void *q_last, uint32_t flags,
                         void *stream);

/* Prefill: the step before the decode, producing a request's ContextKV from context token
 * ids, with one position optionally replaced by a soft token ([TRT] section "Getting the
 * user vector into the prompt: three approaches", the third approach: a user vector mapped
 * by one linear layer to a token-sized embedding and put in place of a placeholder position
 * before the first forward pass).  Under the model stand-in above, a context token's query,
 * key and value at layer l are rows of per-layer tables indexed by token id (standing in for
 * the projections of its embedding, as tok_q/tok_k/tok_v do for fed-back codes).  The soft
 * token has no table row: its embedding e = u * proj (u: user vector [user_dim], proj:
 * [user_dim][embed_dim]) is projected per layer, q = e * w_q[l], k = e * w_k[l],
 * v = e * w_v[l] (head-major columns hq*d + i), in float32, then rounded to the model dtype
 * (round to nearest even).  Tables are device memory (tok_k and tok_v 16-byte aligned)
 * that must stay valid while the engine
 * uses them.  Limits: vocab >= 1; user_dim = 0 (no soft token) or 1..8192 with embed_dim
 * 1..8192 and every projection pointer set. */
typedef struct {
  int32_t vocab;            /* context-token vocabulary size Vc */
  const void *tok_q;        /* device [L][Vc][Hq][d], model dtype */
  const void *tok_k;        /* device [L][Vc][Hkv][d], model dtype */
  const void *tok_v;        /* device [L][Vc][Hkv][d], model dtype */
  int32_t user_dim;         /* length of the user vector; 0 = no soft token */
  int32_t embed_dim;        /* soft embedding size */
  const float *proj;        /* device [user_dim][embed_dim] */
  const float *w_q;         /* device [L][embed_dim][Hq*d] */
  const float *w_k;         /* device [L][embed_dim][Hkv*d] */
  const float *w_v;         /* device [L][embed_dim][Hkv*d] */
} gr_prefill_desc;

/* Sets (or replaces) the prefill tables of the engine.  Allocates the engine's prefill
 * staging (a pinned token buffer and a small device area; outside any hot path).  Errors:
 * GR_E_INVALID_ARG (limits above, null pointers), GR_E_OUT_OF_MEMORY. */
gr_status gr_engine_set_prefill(gr_engine *eng, const gr_prefill_desc *desc);

/* Admits request `request_id` like gr_ctx_kv_load, its context made from tokens host
 * [ctx_len] (each in [0, vocab) except at soft_pos, whose entry is ignored).  soft_pos = -1:
 * no soft token; else 0 <= soft_pos < ctx_len takes the soft token of user_vec device
 * [user_dim] float32.  q_last is the last position's query (a table row, or the soft
 * token's q when soft_pos = ctx_len - 1).
 *   k_native, vt_native both NULL: the context goes into the engine's pool (as a copy load);
 *   both set: it is written to these caller buffers in the native layout of GR_LOAD_ADOPT
 *     (K [L][Hkv][Np][d], V^T [L][Hkv][d][Np], padding zero) and the request keeps them
 *     (alive and unchanged until gr_request_release), 16-byte aligned.
 * q_last_out: optional device [L][Hq][d] copy of the last query.  Stream-ordered; the
 * engine's prefill staging is shared, so prefills of one engine run on one stream.
 * Errors: GR_E_BAD_STATE (workspace not bound, no prefill tables, soft_pos >= 0 without
 * a soft projection), GR_E_INVALID_ARG (a token id out of range, bad soft_pos, null
 * tokens or user_vec, one of k_native / vt_native set, an id already loaded, ctx_len < 1,
 * beam_width outside [1, max_beam_width]), GR_E_OUT_OF_MEMORY (no free slot or pool space). */
gr_status gr_ctx_prefill(gr_engine *eng, int64_t request_id, const int32_t *tokens, int32_t ctx_len,
                         int32_t soft_pos, const float *user_vec, int32_t beam_width, void *k_native,
                         void *vt_native, void *q_last_out, void *stream);

/* gr_ctx_prefill for callers that cannot allocate: code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc.  The same context, bounds and last query as
 * gr_ctx_prefill (the same kernels), with two differences:
 *   tokens_dev  device [ctx_len] int32 token ids (the entry at soft_pos is ignored).  They are
 *               not checked on the host: an id outside [0, vocab) is clamped into it.
 *   the soft token's partial sums go to a fixed device array of the library, 4 MiB
 *               (kSoftSplit = 8 partial sums of embed_dim + n_layers * (Hq + 2 Hkv) * head_dim
 *               floats must fit: 28 layers of 16/8 heads of 128 with embed_dim 2048 take 3.7 MB);
 *               each GPU the library runs on holds one such array until the process ends.
 * No call here runs hipMalloc, hipHostMalloc or hipFree (only the engine's host request table is
 * updated).  Every call on one GPU shares that GPU's array and overwrites it: calls that overlap
 * on one GPU (several streams or engines prefilling soft tokens at once) race.  Errors: those of
 * gr_ctx_prefill except the token-id check, and GR_E_UNSUPPORTED when the soft token's partial
 * sums exceed the array. */
gr_status gr_ctx_prefill_noalloc(gr_engine *eng, int64_t request_id, const int32_t *tokens_dev, int32_t ctx_len,
                                 int32_t soft_pos, const float *user_vec, int32_t beam_width, void *k_native,
                                 void *vt_native, void *q_last_out, void *stream);

/* Advances each listed request by one decode step (one semantic-ID level),
 * whatever level each one is at: requests at different levels can share a
 * call (continuous batching, [GR] section "语义ID生成式推荐专用推理框架").  One step is the
 * beam-search expansion of [TRT] section "Background": every beam attends to its request's
 * ContextKV and to its own BeamKV tokens through BeamPath, its hidden vector is projected onto
 * the level's codes, the item-constrained log-softmax and the top-K over beams x codes keep
 * the best min(W, #valid) candidates, and BeamPath is updated (no KV copy).  Enqueued on `stream`; returns without waiting.
 * Errors: GR_E_INVALID_ARG (n_requests < 1, duplicate ids), GR_E_NOT_FOUND,
 * GR_E_BAD_STATE (a request already decoded all levels); nothing is enqueued
 * when an error is returned. */
gr_status gr_beam_step(gr_engine *eng, const int64_t *request_ids, int32_t n_requests, void *stream);

/* Multi-beam return after all n_levels steps ([TRT] section "Background": every surviving
 * beam is returned, not only the best).  Writes n = min(W, #valid items reachable) beams,
 * best first: codes host [capacity][n_levels], scores host
 * [capacity] (cumulative log-probability).  Synchronises `stream`.
 * Errors: GR_E_BAD_STATE before the last step, GR_E_INVALID_ARG when
 * capacity < n (then *n_beams still receives n). */
gr_status gr_beams_get(gr_engine *eng, int64_t request_id, int32_t capacity, int32_t *codes,
                       float *scores, int32_t *n_beams, void *stream);

/* gr_beams_get for several requests at once (the same multi-beam return, [GR]
 * continuous batching): one small gather kernel, one device-to-host copy
 * through engine-owned pinned memory and one synchronisation of `stream` for
 * the whole batch.  Request i (request_ids[i]) fills codes host
 * [n_requests][capacity][n_levels] at row block i, scores host
 * [n_requests][capacity] at row i and n_beams host [n_requests] at i; rows past
 * n_beams[i] are left untouched.  Errors: GR_E_INVALID_ARG (n_requests outside
 * 1..max_requests, null outputs, or some request with more beams than capacity:
 * every n_beams[i] is still written, and the rows of requests that fit),
 * GR_E_NOT_FOUND, GR_E_BAD_STATE before a request's last step; nothing is
 * copied when an id is unknown or unfinished. */
gr_status gr_beams_get_batch(gr_engine *eng, const int64_t *request_ids, int32_t n_requests, int32_t capacity,
                             int32_t *codes, float *scores, int32_t *n_beams, void *stream);

/* gr_beams_get_batch without the synchronisation, for a host that keeps enqueueing while
 * results travel (the overlap scheduling of [TRT] section "Moving all three into
 * TensorRT-LLM"): enqueues the gather and an asynchronous copy of request i's record into
 * out_host + i * gr_beams_result_bytes(eng) on `stream` and returns.  out_host: caller-owned
 * host memory of n_requests records, pinned (hipHostMalloc) for the copy to overlap.  Once
 * the stream has passed the copy (an event recorded after this call), gr_beams_unpack reads
 * the records.  The engine's staging area is reused in stream order, so later calls on the
 * same stream may follow at once; out_host must not be read before the copy is done nor
 * reused before it has been read.  Errors as gr_beams_get_batch (nothing enqueued). */
gr_status gr_beams_get_batch_async(gr_engine *eng, const int64_t *request_ids, int32_t n_requests,
                                   void *out_host, void *stream);

/* Bytes of one request's record for gr_beams_get_batch_async (0 on a NULL engine). */
size_t gr_beams_result_bytes(const gr_engine *eng);

/* Record i of a completed gr_beams_get_batch_async copy: *n_beams, then (if it fits
 * `capacity`) codes host [capacity][n_levels] and scores host [capacity] as gr_beams_get.
 * GR_E_INVALID_ARG if capacity < *n_beams (n_beams still written). */
gr_status gr_beams_unpack(const gr_engine *eng, const void *out_host, int32_t i, int32_t capacity, int32_t *codes,
                          float *scores, int32_t *n_beams);

/* Candidate scoring over a loaded request's context (the pages' second task, [TRT]
 * "Background": candidates are given and the model ranks them; here, as in [GR]
 * section "语义ID", by the model's own outputs).  Each of the n items (host
 * [n][n_levels] codes) gets its log-probability under the item-constrained decode:
 * the sum over levels of the constrained log-softmax of its code given its own
 * prefix.  The n_levels steps run as in gr_beam_step, with the candidates' codes
 * forced instead of selected (same attention kernels, BeamKV and BeamPath): level 0
 * expands the root to every candidate, beam i then carries candidate i.  scores host
 * [n], in candidate order; -inf for a code tuple that leaves the item trie.  The
 * request is rewound first and stays at its last level afterwards (gr_beams_get then
 * returns the candidates in the same order; gr_request_reset returns it to beam
 * search).  Synchronises `stream`.  Errors: GR_E_INVALID_ARG (null arrays, n outside
 * 1..max_beam_width, a code outside the codebook), GR_E_NOT_FOUND, GR_E_BAD_STATE
 * (workspace not bound). */
gr_status gr_score_items(gr_engine *eng, int64_t request_id, const int32_t *items, int32_t n, float *scores,
                         void *stream);

/* gr_score_items for several requests in the same steps (continuous batching): request
 * i (request_ids[i]) scores the n items at items host [n_requests][n][n_levels] row
 * block i into scores host [n_requests][n] row i.  Errors: as gr_score_items, plus
 * GR_E_INVALID_ARG for n_requests outside 1..max_requests or a duplicate id. */
gr_status gr_score_items_batch(gr_engine *eng, const int64_t *request_ids, int32_t n_requests, const int32_t *items,
                               int32_t n, float *scores, void *stream);

/* Candidate scoring by label tokens ([TRT] "Background", "Scoring many candidates at once"):
 * runs gr_score_items_batch (scores[i][k]: candidate k's item log-likelihood, as there), then one
 * more step in which each candidate's last code runs as a token over the context and the
 * candidate's earlier codes (each candidate sees the shared context and itself only), and the
 * label head on its hidden vector.  label_logp: host [n_requests][n][n_labels] float32, the label
 * log-probabilities of candidate k of request i.  Needs an engine with a label head
 * (GR_E_BAD_STATE otherwise); same argument rules as gr_score_items_batch.  Synchronises
 * `stream`. */
gr_status gr_score_items_labels(gr_engine *eng, const int64_t *request_ids, int32_t n_requests, const int32_t *items,
                                int32_t n, float *scores, float *label_logp, void *stream);

/* Releases a request's slot and pool space (host bookkeeping only; later work
 * on the same stream may reuse them).  Errors: GR_E_NOT_FOUND. */
gr_status gr_request_release(gr_engine *eng, int64_t request_id);

/* Rewinds a loaded request to its root beam (level 0, empty prefix, score 0),
 * keeping its ContextKV and q_last: the next gr_beam_step decodes it again from
 * the start.  Enqueued on `stream`.  Errors: GR_E_NOT_FOUND. */
gr_status gr_request_reset(gr_engine *eng, int64_t request_id, void *stream);

/* gr_request_reset for several requests with one launch.  Errors: GR_E_INVALID_ARG
 * (n_requests < 1), GR_E_NOT_FOUND (nothing is reset then). */
gr_status gr_request_reset_batch(gr_engine *eng, const int64_t *request_ids, int32_t n_requests, void *stream);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char *gr_last_error(void);

/* ---- continuous batching: host scheduler ---------------------------------- */
/* A scheduler drives one engine on one stream in the continuous-batching pattern of the
 * zhiding.cn article's semantic-ID inference framework (section "语义ID生成式推荐专用推理
 * 框架": requests join and leave the running batch between decode steps) and prepares the
 * next step while the GPU runs the current one: the overlap scheduling of the paper-daily
 * TensorRT-LLM summary, section "Moving all three into TensorRT-LLM" (the GPU keeps working
 * while the CPU prepares the next step).  Requests wait in a FIFO queue until a slot frees;
 * each gr_sched_advance then
 *   1. loads queued requests (gr_ctx_kv_load) while fewer than max_active decode,
 *   2. enqueues one gr_beam_step over every decoding request (each at its own level),
 *   3. enqueues the result gather and a copy into pinned host memory for the requests that
 *      this step finished, and releases their slots (later work on the stream reuses them
 *      only after the gather),
 *   4. waits for the copy enqueued by the PREVIOUS call (the GPU meanwhile runs this call's
 *      step) and moves those results into the scheduler's result store.
 * So the host stays one step ahead and never waits for the step it just enqueued.  A
 * request's result is available from the call after the one whose step finished it (or
 * after gr_sched_flush).  Not thread-safe; one scheduler per engine, and nothing else may
 * load, step or release requests of that engine while the scheduler is in use. */
typedef struct gr_sched gr_sched; /* opaque */

/* max_active: requests decoding at once, 1..max_requests of the engine.  Allocates the
 * scheduler's two pinned result buffers (outside any hot path).  stream: hipStream_t every
 * call of the scheduler enqueues on. */
gr_status gr_sched_create(gr_engine *eng, int32_t max_active, void *stream, gr_sched **out);

/* Waits for the stream, frees the pinned buffers.  Requests still queued or decoding are
 * released from the engine. */
gr_status gr_sched_destroy(gr_sched *sched);

/* Queues a request: the arguments of gr_ctx_kv_load (k, v, q_last device or host memory as
 * there; with device sources they must stay valid until the request's load has run on the
 * stream, i.e. until a later gr_sched_advance returns).  GR_E_INVALID_ARG for an id that is
 * queued, decoding or holds an unfetched result; the load's own checks run at admission. */
gr_status gr_sched_submit(gr_sched *sched, int64_t request_id, int32_t ctx_len, int32_t beam_width,
                          const void *k, const void *v, const void *q_last, uint32_t load_flags);

/* One scheduling round (above).  *n_completed = results that became available in this call
 * (those of the previous call's step).  With nothing queued or decoding it only collects. */
gr_status gr_sched_advance(gr_sched *sched, int32_t *n_completed);

/* Collects every result still in flight (synchronises the stream); *n_completed as above. */
gr_status gr_sched_flush(gr_sched *sched, int32_t *n_completed);

/* Ids of available results, oldest first, up to `capacity` (host [capacity]);
 * *n = how many are available in all. */
gr_status gr_sched_completed(gr_sched *sched, int32_t capacity, int64_t *request_ids, int32_t *n);

/* Takes a request's result out of the store: as gr_beams_get (codes host [capacity][n_levels],
 * scores host [capacity], sorted by score).  GR_E_NOT_FOUND if the id holds no result (yet);
 * GR_E_INVALID_ARG (result kept) if capacity < its beam count. */
gr_status gr_sched_result(gr_sched *sched, int64_t request_id, int32_t capacity, int32_t *codes,
                          float *scores, int32_t *n_beams);

/* Requests queued, decoding, and holding unfetched results; batched steps enqueued so far. */
gr_status gr_sched_counts(const gr_sched *sched, int32_t *queued, int32_t *active, int32_t *done,
                          int64_t *steps);

/* ---- item-constrained top-K, stand-alone ---------------------------------- */

/* Selects the k best of n_rows*V candidate scores, cand device [n_rows][V]
 * float32, -inf marking invalid candidates: order score descending, then flat
 * index j*V+c ascending.  Writes out_flat device [k] int32 and out_score
 * device [k] float32 in rank order and n_out device [1] int32 = min(k, number
 * of candidates greater than -inf).  Enqueued on `stream`, does not wait.
 * Limits: n_rows*V <= 2**26, 1 <= k <= 1024.  The same selection runs inside
 * gr_beam_step. */
gr_status gr_topk_select(const float *cand, int32_t n_rows, int32_t V, int32_t k, int32_t *out_flat,
                         float *out_score, int32_t *n_out, void *stream);

/* ---- profiling ------------------------------------------------------------ */

/* Kernel kinds reported by gr_engine_profile_read. */
typedef enum {
  GR_PROF_CTX_ATTN = 0,   /* shared-context attention (per layer, or one launch for a group of layers) */
  GR_PROF_BEAM_MERGE = 1, /* BeamKV append + beam attention + merge, or the sum of hidden-vector partials */
  GR_PROF_LOGITS = 2,     /* codebook logits (one per step) */
  GR_PROF_TOPK = 3,       /* constrained log-softmax + top-K + BeamPath update (one per step) */
  GR_PROF_STEP = 4,       /* a whole gr_beam_step, first launch to last */
  GR_PROF_GEMM = 5,       /* layer chain: one projection launch (q/k/v, o, gate/up, down) */
  GR_PROF_NORM = 6        /* layer chain: input vectors, RMSNorms and the final norm */
} gr_prof_kind;

/* When enabled, gr_beam_step times each launch with HIP events carried by the
 * dispatch itself (hipExtLaunchKernel start/stop events: no marker packets are
 * inserted between kernels, so the timed stream runs as it does unprofiled).  The
 * events come from a bounded pool; a step waits for old events when it is full.
 * Buckets are keyed by kind and by the decode level of the step (0..n_levels-1;
 * steps whose requests are at different levels go to bucket n_levels). */
gr_status gr_engine_set_profiling(gr_engine *eng, int32_t enable);
/* As gr_engine_set_profiling, for the kinds whose bit (1u << GR_PROF_*) is set in `kinds` only (0:
 * off): a timed run can carry events on the launches it reports and none on the others. */
gr_status gr_engine_set_profiling_kinds(gr_engine *eng, uint32_t kinds);
/* In launch sequences of one launch per layer (the split-K steps' context attention and merge,
 * the layer chain's projections, norms, attention and finish), only the launches of layers l
 * with l % stride == 0 carry events while profiling is on; the buckets then average the timed
 * launches only.  stride >= 1 (1, the default, times every launch), else GR_E_INVALID_ARG.  A
 * timed run can so sample a kernel's duration with fewer events in its stream. */
gr_status gr_engine_set_profiling_stride(gr_engine *eng, int32_t stride);

/* Wave timeline of the context-attention kernel (measurement, not part of any decode).  Only the
 * separately built libgr_beam_timed.so records it; the product library returns
 * GR_E_UNSUPPORTED from gr_wave_times_read.  gr_wave_times_select(level, layer) picks the launch
 * to record (-1, -1: none, the default): from then on, every launch of that decode level and
 * layer overwrites the record.  gr_wave_times_read copies it to host memory the caller owns:
 * count must be 1024 x 8 x 8 = 65536 values, [workgroup][wave][field] with the fields entry,
 * token-loop start, token-loop end and partial stores done (100 MHz real-time stamps), then
 * over the token loop the shader-clock cycles spent in copy waits, in barriers and in the whole
 * loop, and the number of barriers; waves with no rows and workgroups past 1024 keep zeros.
 * Synchronous (the default stream).  Errors: GR_E_INVALID_ARG, GR_E_UNSUPPORTED, GR_E_DEVICE. */
gr_status gr_wave_times_select(int32_t level, int32_t layer);
gr_status gr_wave_times_read(int64_t *host, size_t count);

/* Waits for every recorded event, folds the elapsed times into the buckets and
 * returns one bucket: total milliseconds and number of launches, where a launch that
 * covers several layers counts once per layer (so total_ms / launches is the time per
 * layer).  level = -1 sums every level. */
gr_status gr_engine_profile_read(gr_engine *eng, int32_t kind, int32_t level, double *total_ms,
                                 int64_t *launches);

/* The same bucket's number of kernel dispatches (total_ms / dispatches is the time per
 * dispatch, comparable with a kernel trace). */
gr_status gr_engine_profile_dispatches(gr_engine *eng, int32_t kind, int32_t level, int64_t *dispatches);

/* Clears every bucket (pending events are folded first). */
gr_status gr_engine_profile_reset(gr_engine *eng);

/* Graph replay counters of a GR_ENGINE_GRAPH engine: steps that captured a new graph and steps
 * that replayed a kept one. */
gr_status gr_engine_graph_stats(const gr_engine *eng, int64_t *captures, int64_t *replays);

/* ---- inspection (tests and debugging; each synchronises `stream`) --------- */

/* Current beam set B_s of a request: *level = s, *n = n_s; parent host [cap]
 * (slot in B_{s-1}), codes host [cap][n_levels] (first s entries valid),
 * scores host [cap]. */
gr_status gr_debug_beam_state(gr_engine *eng, int64_t request_id, int32_t capacity, int32_t *parent,
                              int32_t *codes, float *scores, int32_t *n, int32_t *level,
                              void *stream);

/* BeamPath ancestry of B_s: anc host [cap][n_levels]; anc[j][t] is the BeamKV slot of
 * beam j's level-t token (t < s). */
gr_status gr_debug_beam_path(gr_engine *eng, int64_t request_id, int32_t capacity, int32_t *anc,
                             int32_t *n, void *stream);

/* Hidden vectors of the beams of the last completed step, host [cap][Hq*d]
 * float32, and the logits host [cap][V]; *n = number of beams of that step. */
gr_status gr_debug_hidden(gr_engine *eng, int64_t request_id, int32_t capacity, float *hidden,
                          float *logits, int32_t *n, void *stream);

/* Attention output of layer `layer` for the beams of the last completed
 * step, host [cap][Hq][d] float32.  Needs GR_ENGINE_DEBUG_ATTN. */
gr_status gr_debug_attn_out(gr_engine *eng, int64_t request_id, int32_t layer, int32_t capacity,
                            float *out, int32_t *n, void *stream);

/* Layer chain, engines created with GR_ENGINE_DEBUG_ATTN: the rows of the last completed step
 * that enter and leave each projection of layer `layer`, for the request's beams, as float32
 * host [cap][width]: which = GR_CHAIN_X_IN (the residual entering the layer, D), GR_CHAIN_XN_ATTN
 * (its norm, the q/k/v projection's input, D), GR_CHAIN_Q (Hq*d), GR_CHAIN_O (the attention
 * output, the output projection's input, Hq*d), GR_CHAIN_X_MID (the residual after it, D),
 * GR_CHAIN_XN_MLP (D), GR_CHAIN_ACT (the SwiGLU product, the down projection's input, I),
 * GR_CHAIN_X_OUT (the residual leaving the layer, D).  bf16 rows are widened exactly. */
enum { GR_CHAIN_X_IN = 0, GR_CHAIN_XN_ATTN = 1, GR_CHAIN_Q = 2, GR_CHAIN_O = 3, GR_CHAIN_X_MID = 4,
       GR_CHAIN_XN_MLP = 5, GR_CHAIN_ACT = 6, GR_CHAIN_X_OUT = 7 };
gr_status gr_debug_chain_rows(gr_engine *eng, int64_t request_id, int32_t layer, int32_t which, int32_t capacity,
                              float *out, int32_t *n, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GR_BEAM_H */
