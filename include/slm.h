/*
 * slm.h -- C ABI of libslm, the attention hot path of a bounded-generation
 * small-language-model engine, hand-written in HIP for AMD MI355X (gfx950).
 *
 * Source of the operations: the page "SLM 生成式高并发推理引擎：延迟约束下的
 * 有效吞吐优化" (abstract, §1.1 "两类在线执行形式", §1.2 "输入与状态边界").
 *   - Prefill-only requests run one prefill over a batch of variable-length
 *     samples, computing only the valid tokens of each sample (§1.2), and take
 *     their result at each sequence's last valid token (§1.1).
 *   - Beam-search requests run a prefill and then a fixed number of decode
 *     steps at a fixed width; every step merges per-beam candidates with the
 *     cumulative scores and keeps a fixed number, with parent indices (§1.1).
 *     All beams of one request share one prompt K/V and keep their own short
 *     suffix K/V (§1.2), and all state is planned at load time (§1.2, §02).
 *
 * Conventions for every call below:
 *   - Tensor arguments are DEVICE pointers, owned by the caller, contiguous,
 *     row-major in the layout stated, and 16-byte aligned.  bf16 tensors are
 *     passed as their 16-bit storage (uint16_t).
 *   - Calls are asynchronous and ordered on the context's stream.  The
 *     library never allocates or synchronises inside a call; the context owns
 *     one workspace allocated by slm_ctx_create and sized by slm_caps.
 *   - The return value reports host-side validation and launch failures.  No
 *     C++ exception crosses the ABI.  On an error nothing is launched, and
 *     slm_ctx_last_error() gives a human-readable detail.
 *   - Contents of device arguments (cu_seqlens, parent) cannot be validated
 *     on the host; kernels bound-check them and, on a violation, set the
 *     context's device error flag, which slm_ctx_check() reads
 *     (SLM_ERR_INVALID_ARG).  The affected outputs are then unspecified, but
 *     no kernel reads or writes out of bounds whatever those contents are.
 *   - A context is not thread-safe; calls that overlap on one stream are
 *     ordered, calls from several host threads on one context race.
 */
#ifndef SLM_H
#define SLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLM_ABI_VERSION 6   /* 3: slm_beam_attn_args gained prompt_cu, prompt_rows;
                               4: slm_beam_backtrack, slm_beam_search;
                               5: slm_packed_prefill_attn_noalloc;
                               6: slm_prefill_plan, slm_packed_prefill_attn_planned */

typedef enum {
    SLM_OK = 0,
    SLM_ERR_INVALID_ARG = 1,   /* a size, pointer or device-side index is wrong   */
    SLM_ERR_UNSUPPORTED = 2,   /* a legal shape this build has no kernel for      */
    SLM_ERR_CAPACITY = 3,      /* beyond the caps the context was created with    */
    SLM_ERR_ALIAS = 4,         /* an output overlaps an input                     */
    SLM_ERR_DEVICE = 5,        /* a HIP runtime call or launch failed             */
    SLM_ERR_OOM = 6            /* the workspace could not be allocated            */
} slm_status;

typedef enum { SLM_BF16 = 0, SLM_F32 = 1 } slm_dtype;

typedef struct slm_ctx slm_ctx;   /* opaque: device, stream, workspace, last error */

/* Load-time capacity plan (§1.2: input length, beam width and step count are
 * bounded before deployment, so state is preallocated).  Fields <= 0 are
 * replaced by the defaults in parentheses. */
typedef struct {
    int32_t max_requests;   /* requests per beam call                 (64)      */
    int32_t max_beams;      /* beam width and beams in                (512)     */
    int32_t max_vocab;      /* vocabulary size                        (262144)  */
    int32_t max_tokens;     /* packed prefill tokens per call         (1048576) */
    int32_t max_seqs;       /* packed prefill sequences per call      (8192)    */
    int32_t max_heads_q;    /* prefill query heads                    (64)      */
} slm_caps;

/* Create a context on HIP device `device`: sets that device current,
 * allocates the top-k workspace (about max_requests * max_beams^2 * 8 bytes)
 * and the prefill work-list workspace (about 16 * max_heads_q *
 * (max_tokens / 128 + max_seqs) bytes), and uses the null stream until
 * slm_ctx_set_stream.  *out is NULL on error.
 * device < 0 creates a dry-run context: every call performs its host-side
 * validation and returns its status without touching any device (usable on
 * machines without a GPU, e.g. to check argument handling). */
slm_status slm_ctx_create(int device, const slm_caps *caps, slm_ctx **out);
void slm_ctx_destroy(slm_ctx *ctx);
/* Order later calls on `hip_stream` (a hipStream_t; NULL = null stream). */
slm_status slm_ctx_set_stream(slm_ctx *ctx, void *hip_stream);
/* Synchronise the stream and read (then clear) the device error flag. */
slm_status slm_ctx_check(slm_ctx *ctx);
const char *slm_status_string(slm_status s);
const char *slm_ctx_last_error(const slm_ctx *ctx);
int slm_abi_version(void);

/*
 * Packed causal GQA prefill attention (abstract: Packed Prefill; §1.2: keep
 * each sequence's valid length, compute valid tokens only).
 *   q           [T, Hq, D]  bf16    queries, T = total_tokens packed tokens
 *   k, v        [T, Hkv, D] bf16    keys / values, after any position encoding
 *   cu_seqlens  [B+1] int32 DEVICE  sequence b is tokens cu[b] .. cu[b+1]-1;
 *               the caller guarantees cu[0] = 0, non-decreasing, cu[B] = T,
 *               every length <= max_seqlen (violations: device error flag)
 *   out         [T, Hq, D]  fp32 or bf16 (out_dtype)
 * For token i of sequence b and query head h:
 *   out = softmax_j(scale * q_i . k_j) v_j  over keys j = cu[b] .. i
 * (causal, diagonal included, no attention across sequences); query head h
 * reads KV head h / (Hq/Hkv).  Supported: head_dim 64 or 128, Hq % Hkv == 0.
 * Empty sequences are allowed and produce no rows.  out must not overlap
 * q, k, v or cu_seqlens.  total_tokens, num_seqs and n_heads_q must be within
 * the context caps (SLM_ERR_CAPACITY).
 */
slm_status slm_packed_prefill_attn(slm_ctx *ctx, const uint16_t *q, const uint16_t *k,
                                   const uint16_t *v, const int32_t *cu_seqlens,
                                   int32_t num_seqs, int32_t total_tokens,
                                   int32_t max_seqlen, int32_t n_heads_q,
                                   int32_t n_heads_kv, int32_t head_dim, float scale,
                                   void *out, slm_dtype out_dtype);

/*
 * The same attention with its work list built once per pack (abstract:
 * Packed Prefill; the layers of one forward pass all run over the same
 * packed batch, so the schedule of that batch is computed once).
 *
 * slm_prefill_plan builds, on the context's stream, the work list of the
 * pack described by cu_seqlens and the sizes (the arguments of
 * slm_packed_prefill_attn without the tensors) in the context's workspace,
 * and returns its id in *plan.  A context holds one plan: any later
 * slm_prefill_plan or slm_packed_prefill_attn call on it replaces the plan.
 * Small packs, which run without a work list, get a plan id too.
 *
 * slm_packed_prefill_attn_planned computes exactly what
 * slm_packed_prefill_attn computes for the same arguments, over the plan
 * `plan` instead of a newly built list.  cu_seqlens (the same pointer,
 * whose contents the caller keeps unchanged) and every size must be those
 * the plan was built for, and the plan must still be the context's current
 * one; otherwise SLM_ERR_INVALID_ARG and nothing is launched.  Runs over one
 * plan may follow each other without limit (each run leaves the list's
 * counters as the plan left them); they are ordered on the context's stream
 * like every call, so they may also be captured in a graph and replayed.
 */
slm_status slm_prefill_plan(slm_ctx *ctx, const int32_t *cu_seqlens, int32_t num_seqs,
                            int32_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                            int32_t n_heads_kv, int32_t head_dim, uint64_t *plan);
slm_status slm_packed_prefill_attn_planned(slm_ctx *ctx, uint64_t plan, const uint16_t *q,
                                           const uint16_t *k, const uint16_t *v,
                                           const int32_t *cu_seqlens, int32_t num_seqs,
                                           int32_t total_tokens, int32_t max_seqlen,
                                           int32_t n_heads_q, int32_t n_heads_kv,
                                           int32_t head_dim, float scale, void *out,
                                           slm_dtype out_dtype);

/*
 * Last-valid-token gather (§1.1: prefill-only outputs come from each
 * sequence's last valid token position).
 *   hidden [T, H] (dtype: 2 or 4 bytes per element), cu_seqlens as above,
 *   out [B, H]: out[b] = hidden[cu[b+1]-1], bit copy; an empty sequence
 *   gives a zero row.  out must not overlap hidden.
 */
slm_status slm_gather_last(slm_ctx *ctx, const void *hidden, const int32_t *cu_seqlens,
                           int32_t num_seqs, int32_t total_tokens, int32_t hidden_dim,
                           slm_dtype dtype, void *out);

/*
 * Beam decode attention over a shared prompt K/V and per-beam suffix K/V
 * (§1.2: beams of one request share one prompt K/V and keep short suffixes;
 * §1.1: parent indices carry beams across steps).  One call covers all
 * n_layers layers of one decode step.  Shapes (NL layers, R requests, W beams,
 * P prompt rows, S_cap suffix capacity):
 *   q            [NL, R, W, Hq, D]        bf16
 *   prefix_k/v   [NL, R, P, Hkv, D]       bf16  shared by the W beams
 *   suffix_k_in/v_in [NL, R, W, S_cap, Hkv, D] bf16  rows 0..hist_len-1, in
 *                the beam order BEFORE the last merge (may be NULL if hist_len = 0)
 *   k_new/v_new  [NL, R, W, Hkv, D]       bf16  this step's key/value row
 *   parent       [R, W] int32 DEVICE      last merge's parents, or NULL = identity
 *   suffix_k_out/v_out [NL, R, W, S_cap, Hkv, D]  rows 0..hist_len written:
 *                rows < hist_len = suffix_in[parent[j]] (bit copy), row
 *                hist_len = k_new/v_new; other rows untouched
 *   out          [NL, R, W, Hq, D]        fp32 or bf16
 * For beam j and query head h (KV head h / (Hq/Hkv)) the keys are the
 * request's prompt rows, the hist_len history rows of beam parent[j] and the
 * new row, all visible.  prompt_len is the prompt length, or with prompt_cu
 * (below) the longest prompt.  Needs hist_len + 1 <= S_cap, hist_len + 1 <= 8, head_dim 64
 * or 128, and the prompt K and V^T of one (layer, request, KV head) must fit
 * in one workgroup's LDS (P <= 576 at D = 64, P <= 256 at D = 128), else
 * SLM_ERR_UNSUPPORTED.  Outputs must not overlap any input or each other.
 * parent values outside [0, W) set the device error flag.
 */
typedef struct {
    int32_t n_layers, num_requests, width, prompt_len, hist_len, suffix_cap;
    int32_t n_heads_q, n_heads_kv, head_dim;
    float scale;
    const uint16_t *q, *prefix_k, *prefix_v, *suffix_k_in, *suffix_v_in, *k_new, *v_new;
    const int32_t *parent;
    uint16_t *suffix_k_out, *suffix_v_out;
    void *out;
    slm_dtype out_dtype;
    /* Prompts of different lengths (NULL = every request has prompt_len rows
     * in the [NL, R, P, Hkv, D] layout above): prompt_cu [R+1] int32 DEVICE
     * offsets, 0 = prompt_cu[0] <= ... <= prompt_cu[R] = prompt_rows, each
     * length at most prompt_len; prefix_k/v are then [NL, prompt_rows, Hkv, D]
     * with request r's prompt at rows prompt_cu[r] .. prompt_cu[r+1] -- the
     * layout a packed prefill of the R prompts writes.  Offsets that break
     * these rules set the device error flag (the request then sees no prompt). */
    const int32_t *prompt_cu;
    int32_t prompt_rows;
} slm_beam_attn_args;
slm_status slm_beam_decode_attn(slm_ctx *ctx, const slm_beam_attn_args *args);

/*
 * Prefill-only label head (§1.1, prefill-only models: after one prefill, the
 * next-token logits at each sequence's last valid token are read at the
 * target-label tokens only and turned into the business output by softmax,
 * top-K or a fixed mapping).
 *   hidden [T, H] bf16, cu_seqlens [B + 1] int32, lm_head [V, H] bf16 (only
 *   the label rows are read), labels [L] int32 token ids, label_map [L]
 *   int32 or NULL (device)
 *   logits, probs [B, L] fp32 (probs may be NULL); top_idx [B, K] int32,
 *   top_prob [B, K] fp32, top_class [B, K] int32 or NULL
 * For sequence b: h = hidden[cu[b+1] - 1] (a zero row if the sequence is
 * empty); logits[b, j] = h . lm_head[labels[j]] (bf16 products, fp32
 * accumulation, a fixed summation order); probs[b, :] = softmax over the L
 * label logits; top_idx[b, :] = the K labels with the largest logits,
 * largest first, the lower index first among equal logits; top_prob their
 * probabilities; top_class = label_map[top_idx] (= top_idx without a map).
 * Needs H % 16 == 0, 1 <= K <= L, L <= 4096, K <= 64; hidden and lm_head
 * 16-byte aligned.  Outputs must not overlap the inputs or each other.  A
 * label id outside [0, V) or an invalid cu_seqlens sets the device error
 * flag (SLM_ERR_INVALID_ARG at the next check); such a label reads row 0.
 */
slm_status slm_label_head(slm_ctx *ctx, const uint16_t *hidden, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t hidden_dim,
                          const uint16_t *lm_head, int32_t vocab, const int32_t *labels,
                          int32_t num_labels, int32_t k, const int32_t *label_map, float *logits,
                          float *probs, int32_t *top_idx, float *top_prob, int32_t *top_class);

/*
 * Beam top-k merge (§1.1: each step takes local candidates from every beam's
 * token distribution, merges them with the cumulative scores and keeps a
 * fixed number; the first step starts from the prefill's log-probs).
 *   logprobs [R, Win, V] fp32, cum [R, Win] fp32 (device)
 *   tokens, parent [R, W] int32; cum_out [R, W] fp32
 * For request r the candidates are (b, v) with score = cum[r,b] +
 * logprobs[r,b,v], one IEEE fp32 addition; they are ranked by score
 * descending, then by flat index f = b*V + v ascending (this total order makes
 * the result unique), and the first W are written in that order: token =
 * f mod V, parent = f div V, cum_out = score.  The first step passes Win = 1.
 * Needs 1 <= W <= Win*V, W <= 512, Win*V < 2^31, R <= caps.max_requests,
 * Win, W <= caps.max_beams, V <= caps.max_vocab.  NaN scores are a caller
 * error (their rank is unspecified).  Outputs must not overlap the inputs.
 */
slm_status slm_beam_topk_merge(slm_ctx *ctx, const float *logprobs, const float *cum,
                               int32_t num_requests, int32_t beams_in, int32_t vocab,
                               int32_t width, int32_t *tokens, int32_t *parent,
                               float *cum_out);

/*
 * Beam top-k merge on logits: the merge above with each beam row's
 * log-softmax folded in, so the log-probabilities are never written (§1.1:
 * the fixed beam-search node takes the model's output straight into the
 * merge).
 *   logits [R, Win, V] fp32 or bf16 (logits_dtype), cum [R, Win] fp32 (device)
 *   tokens, parent [R, W] int32; cum_out [R, W] fp32; lse_out [R, Win] fp32
 *   or NULL (each row's log-sum-exp, for inspection)
 * bf16 logits are widened exactly to fp32 and then treated as fp32 ones (half
 * the bytes read).
 * For row (r, b): lse = log sum_v exp(logits[r,b,v]), computed in fp32 from
 * the row's maximum (approximate: exp and log by the hardware's fp32
 * instructions, partial sums combined in a fixed order, so repeated calls
 * agree bitwise).  Candidate (b, v) scores cum[r,b] + (logits[r,b,v] - lse),
 * two fp32 operations; ranking, tie rule and outputs are those of
 * slm_beam_topk_merge on these scores.  Candidates whose exact scores are
 * closer than the lse's error may therefore rank in either order.
 * Logits must be finite or -inf, above -1e30, with a finite one in every
 * row.  Needs 1 <= W <= Win*V, W <= 512, Win <= 512, Win*V < 2^31, R <=
 * caps.max_requests, Win, W <= caps.max_beams, V <= caps.max_vocab.
 * Outputs must not overlap the inputs or each other.  The logits are read
 * once (one HBM pass); the call allocates nothing.
 */
slm_status slm_beam_topk_merge_logits(slm_ctx *ctx, const void *logits, slm_dtype logits_dtype,
                                      const float *cum, int32_t num_requests, int32_t beams_in,
                                      int32_t vocab, int32_t width, int32_t *tokens, int32_t *parent,
                                      float *cum_out, float *lse_out);

/*
 * Suffix K/V reorder after a merge (§1.1 parent index, §1.2 per-beam suffix):
 *   k_out[l,r,j,i] = k_in[l,r,parent[r,j],i] for rows i < rows, same for V;
 *   [NL, R, W, S_cap, Hkv, D] bf16 storage.  Rows >= rows are untouched.
 *   Needs n_heads_kv * head_dim % 8 == 0.  Outputs must not overlap inputs
 *   (no in-place gather).  parent values outside [0, W) set the device
 *   error flag; those rows are not written.
 */
slm_status slm_beam_reorder_suffix(slm_ctx *ctx, int32_t n_layers, int32_t num_requests,
                                   int32_t width, int32_t rows, int32_t suffix_cap,
                                   int32_t n_heads_kv, int32_t head_dim,
                                   const int32_t *parent, const uint16_t *k_in,
                                   const uint16_t *v_in, uint16_t *k_out, uint16_t *v_out);

/*
 * Final backtrack of a fixed-step beam search into its candidate sequences
 * (§1.1: a beam-search request returns a few candidate sequences; parent
 * indices carry the beams from merge to merge).
 *   tokens, parent [n_merges, R, W] int32 (device): the outputs of the
 *                n_merges merges in order; merge 0 took one beam in, so its
 *                parents are not read
 *   sequences    [R, W, n_merges] int32 (device): sequences[r][j][t] is the
 *                token that final beam j's ancestor took at merge t
 * Beam j after the last merge emitted tokens[n_merges-1][r][j]; its parent
 * there names the beam of the merge before, and so on back to merge 0.  The
 * beams keep the last merge's order (its cum_out holds their scores).  A
 * parent outside [0, W) at merges 1.. sets the device error flag and leaves
 * the earlier entries of that sequence at -1.  sequences must not overlap the
 * inputs.  One lane per final beam; the call reads n_merges * R * W * 8
 * bytes and writes R * W * n_merges * 4.
 */
slm_status slm_beam_backtrack(slm_ctx *ctx, const int32_t *tokens, const int32_t *parent, int32_t n_merges,
                              int32_t num_requests, int32_t width, int32_t *sequences);

/*
 * The whole fixed-step beam search of R requests in one call (§1.1: a
 * beam-search request runs a fixed number of decode steps at a fixed width;
 * abstract and §02: the fixed Beam Search is compiled into one node, with no
 * per-step control from the host).  The call enqueues, on the context's
 * stream and with no host synchronisation:
 *   merge 0   slm_beam_topk_merge(logprobs[0] [R,1,V], cum0 [R,1], W)
 *             -> tokens[0], parent[0], cum[0]
 *   for t = 1 .. n_steps:
 *     decode  slm_beam_decode_attn: hist_len = t-1, q[t-1], k_new[t-1],
 *             v_new[t-1], parents parent[t-1], suffix read from
 *             suffix_k/v[(t+1) % 2] (not at t = 1) and written to
 *             suffix_k/v[t % 2], attention into attn_out[t-1]
 *     merge t slm_beam_topk_merge(logprobs[t] [R,W,V], cum[t-1], W)
 *             -> tokens[t], parent[t], cum[t]
 *   reorder   slm_beam_reorder_suffix(parent[n_steps], rows n_steps) from
 *             suffix_k/v[n_steps % 2] into final_k/final_v (n_steps > 0)
 *   backtrack slm_beam_backtrack(tokens, parent) -> sequences (if not NULL)
 * Every launch's arguments are validated before the first is issued, so an
 * error leaves nothing enqueued.  The host pointer arrays (logprobs, q,
 * k_new, v_new, attn_out) are read during the call only; the call can be
 * captured into a graph.  Shapes and rules are those of the calls above;
 * tokens, parent and cum are [n_steps + 1, R, W], sequences [R, W,
 * n_steps + 1]; n_steps <= 8 and suffix_cap >= n_steps; the suffix and final
 * buffers must not overlap each other, nor attn_out the merge state.
 * attn_out entries may repeat (one buffer overwritten every step).
 */
typedef struct {
    int32_t n_layers, num_requests, width, prompt_len, n_steps, suffix_cap;
    int32_t n_heads_q, n_heads_kv, head_dim, vocab;
    float scale;
    const uint16_t *prefix_k, *prefix_v;   /* [NL, R, P, Hkv, D], or packed with prompt_cu */
    const int32_t *prompt_cu;              /* [R+1] or NULL, as in slm_beam_attn_args */
    int32_t prompt_rows;
    const float *cum0;                     /* [R] initial scores (zeros for fresh requests) */
    const float *const *logprobs;          /* n_steps + 1 device pointers: [R,1,V], then [R,W,V] */
    const uint16_t *const *q;              /* n_steps device pointers [NL, R, W, Hq, D] */
    const uint16_t *const *k_new;          /* n_steps device pointers [NL, R, W, Hkv, D] */
    const uint16_t *const *v_new;          /* n_steps device pointers [NL, R, W, Hkv, D] */
    uint16_t *suffix_k[2], *suffix_v[2];   /* [NL, R, W, S_cap, Hkv, D] each, used alternately */
    uint16_t *final_k, *final_v;           /* [NL, R, W, S_cap, Hkv, D]: rows < n_steps in the last order */
    void *const *attn_out;                 /* n_steps device pointers [NL, R, W, Hq, D] */
    slm_dtype out_dtype;
    int32_t *tokens, *parent;              /* [n_steps + 1, R, W] */
    float *cum;                            /* [n_steps + 1, R, W] */
    int32_t *sequences;                    /* [R, W, n_steps + 1] or NULL */
} slm_beam_search_args;
slm_status slm_beam_search(slm_ctx *ctx, const slm_beam_search_args *args);

/*
 * Packed prefill that allocates nothing, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It needs no context: it runs on the calling
 * thread's current device, on `hip_stream` (a hipStream_t of that device;
 * NULL = null stream), and computes exactly what slm_packed_prefill_attn
 * computes, with the same arguments, rules and statuses, through the same
 * kernels.
 *   - Its scratch memory (the persistent form's work list, its per-XCD
 *     counters and an error word) is one static array per device, 4 MiB +
 *     144 bytes, held until the process ends.  The work list bounds the pack:
 *     total_tokens * n_heads_q / 128 + num_seqs * n_heads_q must be at most
 *     262,144 (e.g. 1M tokens at 16 query heads with up to 8,192 sequences),
 *     else SLM_ERR_CAPACITY and nothing is launched.
 *   - Every call on a device shares that device's array, which keeps the
 *     last call's contents (each call rewrites what it reads).  Calls that
 *     overlap on one device -- on two streams, or from two processes' views
 *     of the same array -- race; serialise them.
 *   - err_flag: a device int32 the kernels set to a nonzero code when
 *     cu_seqlens breaks the caller guarantees (the caller zeroes it and reads
 *     it; the library never clears it); NULL: not reported.
 *   - No detail string: slm_ctx_last_error does not cover this call.
 * The first call on a device looks up the array's address there
 * (hipGetSymbolAddress); no call allocates or frees memory.
 */
slm_status slm_packed_prefill_attn_noalloc(void *hip_stream, const uint16_t *q, const uint16_t *k,
                                           const uint16_t *v, const int32_t *cu_seqlens, int32_t num_seqs,
                                           int32_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                                           int32_t n_heads_kv, int32_t head_dim, float scale, void *out,
                                           slm_dtype out_dtype, int32_t *err_flag);

#ifdef __cplusplus
}
#endif
#endif /* SLM_H */
