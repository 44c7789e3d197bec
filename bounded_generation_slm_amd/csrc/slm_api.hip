// C-ABI layer of libslm: context, load-time workspace, host-side validation
// and dispatch to the kernels.  The operations and their conventions are
// declared in include/slm.h.
//
// The context is the load-time plan of the page "SLM 生成式高并发推理引擎：
// 延迟约束下的有效吞吐优化" (§1.2 and §02): request count, beam width and
// vocabulary are bounded before serving, so the only workspace (the top-k
// stage-1 keys and a device error flag) is allocated once at create time and
// no call allocates or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/slm.h"
#include "kernels.h"

struct slm_ctx {
    int device = 0;
    bool dry_run = false;   // device < 0: validate arguments only, touch no device
    bool validating = false;   // slm_beam_search's first pass: validate every launch, issue none
    hipStream_t stream = nullptr;
    slm_caps caps{};
    uint64_t* topk_ws = nullptr;    // [R] 512-byte state lines (threshold, count, slots), then [R] key lists
    size_t topk_ws_bytes = 0;
    int64_t topk_lists = 0;         // stage-1 lists (of up to max_beams keys) per request
    int* err_flag = nullptr;
    int4* plan_items = nullptr;     // prefill work list: [plan_cap] entries, then 3 x 8 ints
    int plan_cap = 0;
    int num_cus = 256;
    size_t max_lds = 0;
    int topk_blocks_per_cu[2][slm::kTopkMaxWidth + 1] = {};   // stage-1 occupancy per [deep form][width] (0 = not queried)
    int topk_logits_blocks_per_cu[slm::kTopkMaxWidth + 1] = {0};   // the same, merge on logits
    slm::LaunchCache launch_cache;  // occupancy and LDS limits of the attention kernels on this device
    // the current prefill plan: the pack its work list was built for, and its id
    // (every call that rewrites the work list moves plan_gen on)
    struct PlanKey {
        const int32_t* cu;
        int32_t num_seqs, total_tokens, max_seqlen, n_heads_q, n_heads_kv, head_dim;
        bool operator==(const PlanKey& o) const {
            return cu == o.cu && num_seqs == o.num_seqs && total_tokens == o.total_tokens &&
                   max_seqlen == o.max_seqlen && n_heads_q == o.n_heads_q && n_heads_kv == o.n_heads_kv &&
                   head_dim == o.head_dim;
        }
    };
    uint64_t plan_gen = 0;
    bool plan_valid = false;
    PlanKey plan_key{};
    char last_error[512] = {0};
};

namespace {

slm_status fail(slm_ctx* ctx, slm_status s, const char* fmt, ...) {
    if (ctx) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(ctx->last_error, sizeof ctx->last_error, fmt, ap);
        va_end(ap);
    }
    return s;
}

slm_status ok(slm_ctx* ctx) {
    ctx->last_error[0] = 0;
    return SLM_OK;
}

// Validation passed: a dry-run context (or a validation pass) stops here,
// others launch.
#define SLM_LAUNCH(ctx, call, what) \
    (((ctx)->dry_run || (ctx)->validating) ? ok(ctx) : launched((ctx), (call), (what)))

slm_status launched(slm_ctx* ctx, hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ctx, SLM_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok(ctx);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

// Sets the context's device current for the launches that follow.
slm_status enter(slm_ctx* ctx) {
    if (!ctx) return SLM_ERR_INVALID_ARG;
    if (ctx->dry_run) return SLM_OK;
    if (hipSetDevice(ctx->device) != hipSuccess)
        return fail(ctx, SLM_ERR_DEVICE, "hipSetDevice(%d) failed", ctx->device);
    return SLM_OK;
}

}  // namespace

extern "C" {

int slm_abi_version(void) { return SLM_ABI_VERSION; }

const char* slm_status_string(slm_status s) {
    switch (s) {
        case SLM_OK: return "SLM_OK";
        case SLM_ERR_INVALID_ARG: return "SLM_ERR_INVALID_ARG";
        case SLM_ERR_UNSUPPORTED: return "SLM_ERR_UNSUPPORTED";
        case SLM_ERR_CAPACITY: return "SLM_ERR_CAPACITY";
        case SLM_ERR_ALIAS: return "SLM_ERR_ALIAS";
        case SLM_ERR_DEVICE: return "SLM_ERR_DEVICE";
        case SLM_ERR_OOM: return "SLM_ERR_OOM";
    }
    return "SLM_ERR_UNKNOWN";
}

const char* slm_ctx_last_error(const slm_ctx* ctx) { return ctx ? ctx->last_error : "null context"; }

slm_status slm_ctx_create(int device, const slm_caps* caps, slm_ctx** out) {
    if (!out) return SLM_ERR_INVALID_ARG;
    *out = nullptr;
    if (device < 0) {                       // dry run: host-side validation only
        slm_ctx* ctx = new (std::nothrow) slm_ctx;
        if (!ctx) return SLM_ERR_OOM;
        ctx->dry_run = true;
        ctx->device = -1;
        slm_caps c = caps ? *caps : slm_caps{};
        if (c.max_requests <= 0) c.max_requests = 64;
        if (c.max_beams <= 0) c.max_beams = slm::kTopkMaxWidth;
        if (c.max_vocab <= 0) c.max_vocab = 262144;
        if (c.max_tokens <= 0) c.max_tokens = 1 << 20;
        if (c.max_seqs <= 0) c.max_seqs = 8192;
        if (c.max_heads_q <= 0) c.max_heads_q = 64;
        ctx->caps = c;
        ctx->max_lds = 160 * 1024;          // gfx950 LDS per workgroup
        ctx->plan_cap = (int)std::min<int64_t>(slm::prefill_plan_entries(c.max_tokens, c.max_seqs, c.max_heads_q),
                                               INT32_MAX - 16);
        *out = ctx;
        return SLM_OK;
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return SLM_ERR_DEVICE;
    slm_ctx* ctx = new (std::nothrow) slm_ctx;
    if (!ctx) return SLM_ERR_OOM;
    ctx->device = device;
    slm_caps c = caps ? *caps : slm_caps{};
    if (c.max_requests <= 0) c.max_requests = 64;
    if (c.max_beams <= 0) c.max_beams = slm::kTopkMaxWidth;
    if (c.max_vocab <= 0) c.max_vocab = 262144;
    if (c.max_tokens <= 0) c.max_tokens = 1 << 20;
    if (c.max_seqs <= 0) c.max_seqs = 8192;
    if (c.max_heads_q <= 0) c.max_heads_q = 64;
    ctx->caps = c;
    if (hipSetDevice(device) != hipSuccess) {
        delete ctx;
        return SLM_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        delete ctx;
        return SLM_ERR_DEVICE;
    }
    ctx->max_lds = prop.sharedMemPerBlock;
    ctx->num_cus = prop.multiProcessorCount;
    const int64_t entries = slm::prefill_plan_entries(c.max_tokens, c.max_seqs, c.max_heads_q);
    if (entries > INT32_MAX - 16) {
        delete ctx;
        return SLM_ERR_INVALID_ARG;
    }
    ctx->plan_cap = (int)entries;
    ctx->topk_ws_bytes = slm::beam_topk_workspace_bytes(c.max_requests, c.max_beams);
    ctx->topk_lists = slm::beam_topk_lists(c.max_beams);
    if (hipMalloc((void**)&ctx->topk_ws, ctx->topk_ws_bytes) != hipSuccess ||
        hipMemset(ctx->topk_ws, 0, ctx->topk_ws_bytes) != hipSuccess ||
        hipMalloc((void**)&ctx->err_flag, sizeof(int)) != hipSuccess ||
        hipMemset(ctx->err_flag, 0, sizeof(int)) != hipSuccess ||
        hipMalloc((void**)&ctx->plan_items, sizeof(int4) * ((size_t)ctx->plan_cap + 8)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        if (ctx->topk_ws) (void)hipFree(ctx->topk_ws);
        if (ctx->err_flag) (void)hipFree(ctx->err_flag);
        if (ctx->plan_items) (void)hipFree(ctx->plan_items);
        delete ctx;
        return SLM_ERR_OOM;
    }
    *out = ctx;
    return SLM_OK;
}

void slm_ctx_destroy(slm_ctx* ctx) {
    if (!ctx) return;
    if (!ctx->dry_run && hipSetDevice(ctx->device) == hipSuccess) {
        (void)hipDeviceSynchronize();
        (void)hipFree(ctx->topk_ws);
        (void)hipFree(ctx->err_flag);
        (void)hipFree(ctx->plan_items);
    }
    delete ctx;
}

slm_status slm_ctx_set_stream(slm_ctx* ctx, void* hip_stream) {
    if (!ctx) return SLM_ERR_INVALID_ARG;
    ctx->stream = (hipStream_t)hip_stream;
    return ok(ctx);
}

slm_status slm_ctx_check(slm_ctx* ctx) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (ctx->dry_run) return ok(ctx);
    if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        return fail(ctx, SLM_ERR_DEVICE, "stream synchronisation failed: %s", hipGetErrorString(hipGetLastError()));
    int flag = 0;
    if (hipMemcpy(&flag, ctx->err_flag, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(ctx, SLM_ERR_DEVICE, "reading the device error flag failed");
    if (flag != 0) {
        (void)hipMemset(ctx->err_flag, 0, sizeof(int));
        if (flag == slm::kErrCuSeqlens)
            return fail(ctx, SLM_ERR_INVALID_ARG,
                        "cu_seqlens / prompt_cu: offsets not non-decreasing from 0 to the total, or a length above "
                        "the maximum");
        if (flag == slm::kErrLabel)
            return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: a label token id outside [0, vocab)");
        if (flag == slm::kErrSelect)
            return fail(ctx, SLM_ERR_DEVICE, "top-k: a selection pass limit was reached (equal keys)");
        return fail(ctx, SLM_ERR_INVALID_ARG, "parent index outside [0, width)");
    }
    return ok(ctx);
}

namespace {

enum PrefillMode { kPrefillFull, kPrefillPlanOnly, kPrefillRunOnly };

// Packed prefill in three forms: work list and attention (slm_packed_prefill_attn),
// the work list alone (slm_prefill_plan), the attention over the current plan
// (slm_packed_prefill_attn_planned).  The plan form takes no tensors.
slm_status prefill_call(slm_ctx* ctx, PrefillMode mode, uint64_t plan_id, uint64_t* plan_out, const uint16_t* q,
                        const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t total_tokens, int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                        int32_t head_dim, float scale, void* out, slm_dtype out_dtype) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    const bool tensors = mode != kPrefillPlanOnly;
    if (mode == kPrefillPlanOnly && !plan_out) return fail(ctx, SLM_ERR_INVALID_ARG, "prefill plan: plan is NULL");
    if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: negative size or non-positive head count / head_dim");
    if (n_heads_q % n_heads_kv != 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: n_heads_q %% n_heads_kv != 0");
    if (head_dim != 64 && head_dim != 128)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "prefill: head_dim %d (supported: 64, 128)", head_dim);
    if (tensors && out_dtype != SLM_F32 && out_dtype != SLM_BF16)
        return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: unknown out_dtype");
    if (tensors && (!(scale > 0.f) || !std::isfinite(scale)))
        return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: scale must be finite and positive");
    if (!cu_seqlens) return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: cu_seqlens is NULL");
    if (max_seqlen == 0 && total_tokens > 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: max_seqlen 0 with %d packed tokens", total_tokens);
    const slm_ctx::PlanKey key{cu_seqlens, num_seqs, total_tokens, max_seqlen, n_heads_q, n_heads_kv, head_dim};
    if (mode == kPrefillRunOnly && !(ctx->plan_valid && plan_id == ctx->plan_gen && key == ctx->plan_key))
        return fail(ctx, SLM_ERR_INVALID_ARG,
                    "prefill: plan %llu is not the context's current plan for this cu_seqlens and these sizes",
                    (unsigned long long)plan_id);
    const bool empty = total_tokens == 0 || num_seqs == 0;
    if (!empty) {
        if (tensors && (!q || !k || !v || !out)) return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: NULL tensor");
        if (tensors && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)))
            return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: tensors must be 16-byte aligned");
        if (max_seqlen > total_tokens)
            return fail(ctx, SLM_ERR_INVALID_ARG, "prefill: max_seqlen %d > total_tokens %d", max_seqlen,
                        total_tokens);
        if (total_tokens > ctx->caps.max_tokens || num_seqs > ctx->caps.max_seqs || n_heads_q > ctx->caps.max_heads_q)
            return fail(ctx, SLM_ERR_CAPACITY, "prefill: beyond the context caps (tokens %d, seqs %d, heads %d)",
                        ctx->caps.max_tokens, ctx->caps.max_seqs, ctx->caps.max_heads_q);
        if (slm::prefill_plan_entries(total_tokens, num_seqs, n_heads_q) > ctx->plan_cap)
            return fail(ctx, SLM_ERR_CAPACITY,
                        "prefill: the pack's work list (%lld entries) exceeds the workspace (%d)",
                        (long long)slm::prefill_plan_entries(total_tokens, num_seqs, n_heads_q), ctx->plan_cap);
        if (tensors) {
            const size_t T = (size_t)total_tokens, D = (size_t)head_dim;
            const size_t qb = T * n_heads_q * D * 2, kb = T * n_heads_kv * D * 2;
            const size_t ob = T * n_heads_q * D * (out_dtype == SLM_F32 ? 4 : 2);
            const size_t cb = ((size_t)num_seqs + 1) * 4;
            if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kb) || overlaps(out, ob, v, kb) ||
                overlaps(out, ob, cu_seqlens, cb))
                return fail(ctx, SLM_ERR_ALIAS, "prefill: out overlaps an input");
        }
    }
    slm::PrefillParams p{};
    p.q = q; p.k = k; p.v = v; p.cu = cu_seqlens; p.out = out; p.err = ctx->err_flag;
    p.num_seqs = num_seqs; p.total_tokens = total_tokens; p.max_seqlen = max_seqlen;
    p.n_heads_q = n_heads_q; p.n_heads_kv = n_heads_kv; p.group = n_heads_q / n_heads_kv;
    p.heads_per_block = (p.group % 2 == 0) ? 2 : 1;
    p.head_blocks = p.group / p.heads_per_block;
    const int qt_rows = 128 / p.heads_per_block;
    p.q_tiles = (max_seqlen + qt_rows - 1) / qt_rows;
    const int64_t units = (int64_t)num_seqs * n_heads_kv * p.head_blocks;
    if (units > INT32_MAX / 8) return fail(ctx, SLM_ERR_UNSUPPORTED, "prefill: too many sequences x heads");
    p.n_units = (int)units;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.plan_items = ctx->plan_items;
    p.plan_cap = ctx->plan_cap;
    p.plan_count = (int*)(ctx->plan_items + ctx->plan_cap);
    p.plan_off = p.plan_count + 8;
    p.plan_claim = p.plan_off + 8;
    p.plan_done = p.plan_claim + 8;
    if (mode != kPrefillRunOnly) {              // the work list is rewritten: earlier plans are void
        ++ctx->plan_gen;
        ctx->plan_valid = mode == kPrefillPlanOnly;
        ctx->plan_key = key;
        if (plan_out) *plan_out = ctx->plan_gen;
    }
    if (empty) return ok(ctx);
    // Large packs run as persistent workgroups over a device-built work list;
    // small ones launch one workgroup per work unit (no list to build).
    const int64_t est_units = ((int64_t)total_tokens * n_heads_q / 128) + 1;
    const bool persistent = est_units >= 8LL * ctx->num_cus && num_seqs <= slm::kPrefillPlanMaxSeqs;
    const int phases = mode == kPrefillFull ? slm::kPrefillPlan | slm::kPrefillRun
                                            : (mode == kPrefillPlanOnly ? slm::kPrefillPlan : slm::kPrefillRun);
    return SLM_LAUNCH(ctx, slm::launch_prefill_attn(p, head_dim, out_dtype == SLM_BF16, persistent, ctx->num_cus,
                                                    ctx->launch_cache, ctx->stream, phases), "prefill");
}

}  // namespace

slm_status slm_packed_prefill_attn(slm_ctx* ctx, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                   int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                                   int32_t head_dim, float scale, void* out, slm_dtype out_dtype) {
    return prefill_call(ctx, kPrefillFull, 0, nullptr, q, k, v, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                        n_heads_q, n_heads_kv, head_dim, scale, out, out_dtype);
}

slm_status slm_prefill_plan(slm_ctx* ctx, const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                            int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                            uint64_t* plan) {
    return prefill_call(ctx, kPrefillPlanOnly, 0, plan, nullptr, nullptr, nullptr, cu_seqlens, num_seqs,
                        total_tokens, max_seqlen, n_heads_q, n_heads_kv, head_dim, 1.f, nullptr, SLM_F32);
}

slm_status slm_packed_prefill_attn_planned(slm_ctx* ctx, uint64_t plan, const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const int32_t* cu_seqlens, int32_t num_seqs,
                                           int32_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                                           int32_t n_heads_kv, int32_t head_dim, float scale, void* out,
                                           slm_dtype out_dtype) {
    return prefill_call(ctx, kPrefillRunOnly, plan, nullptr, q, k, v, cu_seqlens, num_seqs, total_tokens,
                        max_seqlen, n_heads_q, n_heads_kv, head_dim, scale, out, out_dtype);
}

slm_status slm_gather_last(slm_ctx* ctx, const void* hidden, const int32_t* cu_seqlens, int32_t num_seqs,
                           int32_t total_tokens, int32_t hidden_dim, slm_dtype dtype, void* out) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (num_seqs < 0 || total_tokens < 0 || hidden_dim <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "gather: negative size or hidden_dim <= 0");
    if (dtype != SLM_F32 && dtype != SLM_BF16) return fail(ctx, SLM_ERR_INVALID_ARG, "gather: unknown dtype");
    if (num_seqs == 0) return ok(ctx);
    if (!cu_seqlens || !out || (!hidden && total_tokens > 0))
        return fail(ctx, SLM_ERR_INVALID_ARG, "gather: NULL pointer");
    const size_t row = (size_t)hidden_dim * (dtype == SLM_F32 ? 4 : 2);
    if (overlaps(out, row * num_seqs, hidden, row * total_tokens) ||
        overlaps(out, row * num_seqs, cu_seqlens, ((size_t)num_seqs + 1) * 4))
        return fail(ctx, SLM_ERR_ALIAS, "gather: out overlaps an input");
    slm::GatherParams p{};
    p.hidden = hidden; p.cu = cu_seqlens; p.out = out; p.err = ctx->err_flag;
    p.num_seqs = num_seqs; p.total_tokens = total_tokens; p.row_bytes = (int64_t)row;
    p.vec16 = (row % 16 == 0) && aligned16(hidden) && aligned16(out);
    if (((uintptr_t)hidden & 1) || ((uintptr_t)out & 1))
        return fail(ctx, SLM_ERR_INVALID_ARG, "gather: tensors must be 2-byte aligned");
    return SLM_LAUNCH(ctx, slm::launch_gather_last(p, ctx->stream), "gather");
}

slm_status slm_label_head(slm_ctx* ctx, const uint16_t* hidden, const int32_t* cu_seqlens, int32_t num_seqs,
                          int32_t total_tokens, int32_t hidden_dim, const uint16_t* lm_head, int32_t vocab,
                          const int32_t* labels, int32_t num_labels, int32_t k, const int32_t* label_map,
                          float* logits, float* probs, int32_t* top_idx, float* top_prob, int32_t* top_class) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (num_seqs < 0 || total_tokens < 0 || hidden_dim <= 0 || vocab <= 0 || num_labels <= 0 || k <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: a size is out of range");
    if (k > num_labels) return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: k %d > num_labels %d", k, num_labels);
    if (hidden_dim % 16 != 0) return fail(ctx, SLM_ERR_UNSUPPORTED, "label_head: hidden_dim must be a multiple of 16");
    if (num_labels > slm::kLabelMax || k > slm::kLabelTopMax)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "label_head: at most %d labels and k <= %d", slm::kLabelMax,
                    slm::kLabelTopMax);
    if (num_seqs == 0) return ok(ctx);
    if (!cu_seqlens || !lm_head || !labels || !logits || !top_idx || !top_prob || (!hidden && total_tokens > 0))
        return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: NULL pointer");
    if (!aligned16(hidden) || !aligned16(lm_head))
        return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: hidden and lm_head must be 16-byte aligned");
    const void* four[] = {cu_seqlens, labels, label_map, logits, probs, top_idx, top_prob, top_class};
    for (const void* q : four)
        if ((uintptr_t)q & 3) return fail(ctx, SLM_ERR_INVALID_ARG, "label_head: tensors must be 4-byte aligned");
    const size_t B = num_seqs, L = num_labels, K = k;
    const size_t hb = (size_t)total_tokens * hidden_dim * 2, wb = (size_t)vocab * hidden_dim * 2;
    struct Span { const void* p; size_t n; };
    const Span ins[] = {{hidden, hb}, {lm_head, wb}, {cu_seqlens, (B + 1) * 4}, {labels, L * 4}, {label_map, L * 4}};
    const Span outs[] = {{logits, B * L * 4}, {probs, B * L * 4}, {top_idx, B * K * 4}, {top_prob, B * K * 4},
                         {top_class, B * K * 4}};
    for (const Span& o : outs) {
        if (!o.p) continue;
        for (const Span& i : ins)
            if (i.p && overlaps(o.p, o.n, i.p, i.n)) return fail(ctx, SLM_ERR_ALIAS, "label_head: an output overlaps an input");
        for (const Span& o2 : outs)
            if (&o2 != &o && o2.p && overlaps(o.p, o.n, o2.p, o2.n))
                return fail(ctx, SLM_ERR_ALIAS, "label_head: outputs overlap each other");
    }
    slm::LabelHeadParams p{};
    p.hidden = hidden; p.cu = cu_seqlens; p.lm = lm_head; p.labels = labels; p.map = label_map;
    p.logits = logits; p.probs = probs; p.top_idx = top_idx; p.top_prob = top_prob; p.top_class = top_class;
    p.err = ctx->err_flag;
    p.num_seqs = num_seqs; p.total_tokens = total_tokens; p.hidden_dim = hidden_dim; p.vocab = vocab;
    p.num_labels = num_labels; p.k = k;
    return SLM_LAUNCH(ctx, slm::launch_label_head(p, ctx->stream), "label_head");
}

slm_status slm_beam_decode_attn(slm_ctx* ctx, const slm_beam_attn_args* a) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (!a) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: NULL args");
    if (a->n_layers <= 0 || a->num_requests <= 0 || a->width <= 0 || a->prompt_len < 0 || a->hist_len < 0 ||
        a->suffix_cap <= 0 || a->n_heads_q <= 0 || a->n_heads_kv <= 0 || a->head_dim <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "decode: a size is out of range");
    if (a->n_heads_q % a->n_heads_kv != 0) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: n_heads_q %% n_heads_kv != 0");
    if (a->hist_len + 1 > a->suffix_cap)
        return fail(ctx, SLM_ERR_INVALID_ARG, "decode: hist_len + 1 > suffix_cap");
    if (a->hist_len + 1 > slm::kDecodeMaxSuffix)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "decode: more than %d suffix rows", slm::kDecodeMaxSuffix);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "decode: head_dim %d (supported: 64, 128)", a->head_dim);
    if (a->out_dtype != SLM_F32 && a->out_dtype != SLM_BF16) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: unknown out_dtype");
    if (!(a->scale > 0.f) || !std::isfinite(a->scale)) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: bad scale");
    if (a->prompt_cu && (a->prompt_rows < 0 || (int64_t)a->prompt_rows > (int64_t)a->num_requests * a->prompt_len))
        return fail(ctx, SLM_ERR_INVALID_ARG, "decode: prompt_rows %d outside [0, num_requests * prompt_len]",
                    a->prompt_rows);
    if (a->prompt_cu && !aligned4(a->prompt_cu)) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: prompt_cu must be 4-byte aligned");
    if (!a->q || !a->k_new || !a->v_new || !a->out || !a->suffix_k_out || !a->suffix_v_out ||
        (a->prompt_len > 0 && (!a->prefix_k || !a->prefix_v)) ||
        (a->hist_len > 0 && (!a->suffix_k_in || !a->suffix_v_in)))
        return fail(ctx, SLM_ERR_INVALID_ARG, "decode: NULL tensor");
    const void* ptrs[] = {a->q, a->prefix_k, a->prefix_v, a->suffix_k_in, a->suffix_v_in, a->k_new, a->v_new,
                          a->suffix_k_out, a->suffix_v_out, a->out};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return fail(ctx, SLM_ERR_INVALID_ARG, "decode: tensors must be 16-byte aligned");
    const size_t lds = slm::beam_decode_lds_bytes(a->head_dim, a->prompt_len);
    if (lds > ctx->max_lds)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "decode: prompt_len %d x head_dim %d needs %zu B of LDS (> %zu)",
                    a->prompt_len, a->head_dim, lds, ctx->max_lds);
    const size_t NL = a->n_layers, R = a->num_requests, W = a->width, D = a->head_dim;
    const size_t Hq = a->n_heads_q, Hkv = a->n_heads_kv;
    if ((NL * R * W * Hq) > (size_t)INT32_MAX || NL * R * Hkv * 8 > (size_t)INT32_MAX ||
        W * Hq * D * 4 >= (size_t)INT32_MAX)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "decode: too many rows");
    const size_t qb = NL * R * W * Hq * D * 2, ob = NL * R * W * Hq * D * (a->out_dtype == SLM_F32 ? 4 : 2);
    const size_t prompt_rows = a->prompt_cu ? (size_t)a->prompt_rows : R * a->prompt_len;
    const size_t pb = NL * prompt_rows * Hkv * D * 2, sb = NL * R * W * a->suffix_cap * Hkv * D * 2;
    const size_t nb = NL * R * W * Hkv * D * 2, parb = R * W * 4;
    struct Buf { const void* p; size_t n; };
    const Buf ins[] = {{a->q, qb}, {a->prefix_k, pb}, {a->prefix_v, pb}, {a->suffix_k_in, sb}, {a->suffix_v_in, sb},
                       {a->k_new, nb}, {a->v_new, nb}, {a->parent, parb}, {a->prompt_cu, (R + 1) * 4}};
    const Buf outs[] = {{a->out, ob}, {a->suffix_k_out, sb}, {a->suffix_v_out, sb}};
    for (const Buf& o : outs)
        for (const Buf& i : ins)
            if (overlaps(o.p, o.n, i.p, i.n)) return fail(ctx, SLM_ERR_ALIAS, "decode: an output overlaps an input");
    if (overlaps(outs[0].p, outs[0].n, outs[1].p, outs[1].n) || overlaps(outs[0].p, outs[0].n, outs[2].p, outs[2].n) ||
        overlaps(outs[1].p, outs[1].n, outs[2].p, outs[2].n))
        return fail(ctx, SLM_ERR_ALIAS, "decode: outputs overlap each other");
    slm::DecodeParams p{};
    p.q = a->q; p.prefix_k = a->prefix_k; p.prefix_v = a->prefix_v;
    p.suffix_k_in = a->suffix_k_in; p.suffix_v_in = a->suffix_v_in; p.k_new = a->k_new; p.v_new = a->v_new;
    p.parent = a->parent; p.suffix_k_out = a->suffix_k_out; p.suffix_v_out = a->suffix_v_out; p.out = a->out;
    p.err = ctx->err_flag;
    p.n_layers = a->n_layers; p.num_requests = a->num_requests; p.width = a->width; p.prompt_len = a->prompt_len;
    p.hist_len = a->hist_len; p.suffix_cap = a->suffix_cap; p.n_heads_q = a->n_heads_q;
    p.n_heads_kv = a->n_heads_kv; p.group = a->n_heads_q / a->n_heads_kv;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.prompt_cu = a->prompt_cu;
    p.prompt_rows = (int)prompt_rows;
    return SLM_LAUNCH(ctx, slm::launch_beam_decode_attn(p, a->head_dim, a->out_dtype == SLM_BF16, ctx->num_cus,
                                                        ctx->launch_cache, ctx->stream),
                      "decode");
}

slm_status slm_beam_topk_merge(slm_ctx* ctx, const float* logprobs, const float* cum, int32_t num_requests,
                               int32_t beams_in, int32_t vocab, int32_t width, int32_t* tokens, int32_t* parent,
                               float* cum_out) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (num_requests < 0 || beams_in <= 0 || vocab <= 0 || width <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk: a size is out of range");
    if ((int64_t)width > (int64_t)beams_in * vocab)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk: width %d > beams_in * vocab", width);
    if ((int64_t)beams_in * vocab >= ((int64_t)1 << 31))
        return fail(ctx, SLM_ERR_UNSUPPORTED, "topk: beams_in * vocab must be below 2^31");
    if (width > slm::kTopkMaxWidth) return fail(ctx, SLM_ERR_UNSUPPORTED, "topk: width %d > %d", width, slm::kTopkMaxWidth);
    if (num_requests > ctx->caps.max_requests || beams_in > ctx->caps.max_beams || width > ctx->caps.max_beams ||
        vocab > ctx->caps.max_vocab)
        return fail(ctx, SLM_ERR_CAPACITY, "topk: beyond the context caps (requests %d, beams %d, vocab %d)",
                    ctx->caps.max_requests, ctx->caps.max_beams, ctx->caps.max_vocab);
    if (num_requests == 0) return ok(ctx);
    if (!logprobs || !cum || !tokens || !parent || !cum_out) return fail(ctx, SLM_ERR_INVALID_ARG, "topk: NULL tensor");
    if (((uintptr_t)logprobs & 3) || ((uintptr_t)cum & 3) || ((uintptr_t)tokens & 3) || ((uintptr_t)parent & 3) ||
        ((uintptr_t)cum_out & 3))
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk: tensors must be 4-byte aligned");
    const size_t R = num_requests;
    const size_t lpb = R * beams_in * (size_t)vocab * 4, cb = R * beams_in * 4, ob = R * width * 4;
    const void* outs[] = {tokens, parent, cum_out};
    for (const void* o : outs)
        if (overlaps(o, ob, logprobs, lpb) || overlaps(o, ob, cum, cb))
            return fail(ctx, SLM_ERR_ALIAS, "topk: an output overlaps an input");
    if (overlaps(tokens, ob, parent, ob) || overlaps(tokens, ob, cum_out, ob) || overlaps(parent, ob, cum_out, ob))
        return fail(ctx, SLM_ERR_ALIAS, "topk: outputs overlap each other");
    slm::TopkParams p{};
    p.logprobs = logprobs; p.cum = cum; p.tokens = tokens; p.parent = parent; p.cum_out = cum_out;
    p.err = ctx->err_flag;
    const int64_t R_cap = ctx->caps.max_requests;
    p.req_state = ctx->topk_ws;
    p.stage1 = ctx->topk_ws + slm::kTopkStateWords * R_cap;
    p.list_cap = ctx->topk_lists * ctx->caps.max_beams;
    p.num_requests = num_requests; p.beams_in = beams_in; p.vocab = vocab; p.width = width;
    // stage-1 waves take equal ranges of the flattened candidates, one per
    // resident wave (four waves per workgroup)
    p.deep = slm::beam_topk_deep(width, (int64_t)num_requests * beams_in * vocab);
    int bpc = ctx->topk_blocks_per_cu[p.deep][width];
    if (bpc == 0) {
        const bool query = !ctx->dry_run && !ctx->validating;
        bpc = query ? slm::beam_topk_blocks_per_cu(width, p.deep) : 1;
        if (query) ctx->topk_blocks_per_cu[p.deep][width] = bpc;
    }
    const int64_t resident = (int64_t)ctx->num_cus * bpc * 4;
    p.seg = slm::beam_topk_segment(num_requests, beams_in, vocab, resident, ctx->topk_lists);
    // sliced ranges where every slice still holds at least kTopkMinSegment
    // candidates and the request's waves fit its list (one flush each)
    {
        const int k = slm::kTopkSlices;
        const int64_t wpr = resident / num_requests / 4 * 4;
        if (k > 0 && wpr >= 4 && wpr < ctx->topk_lists &&
            (int64_t)beams_in * vocab / (wpr * k) >= slm::kTopkMinSegment) {
            p.wpr = (int)wpr;
            p.kslices = k;
        }
    }
    return SLM_LAUNCH(ctx, slm::launch_beam_topk_merge(p, ctx->stream), "topk");
}

slm_status slm_beam_topk_merge_logits(slm_ctx* ctx, const void* logits, slm_dtype logits_dtype, const float* cum,
                                      int32_t num_requests, int32_t beams_in, int32_t vocab, int32_t width,
                                      int32_t* tokens, int32_t* parent, float* cum_out, float* lse_out) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (num_requests < 0 || beams_in <= 0 || vocab <= 0 || width <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk_logits: a size is out of range");
    if ((int64_t)width > (int64_t)beams_in * vocab)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk_logits: width %d > beams_in * vocab", width);
    if ((int64_t)beams_in * vocab >= ((int64_t)1 << 31))
        return fail(ctx, SLM_ERR_UNSUPPORTED, "topk_logits: beams_in * vocab must be below 2^31");
    if (width > slm::kTopkMaxWidth || beams_in > slm::kTopkMaxWidth)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "topk_logits: width and beams_in must be at most %d", slm::kTopkMaxWidth);
    if (num_requests > ctx->caps.max_requests || beams_in > ctx->caps.max_beams || width > ctx->caps.max_beams ||
        vocab > ctx->caps.max_vocab)
        return fail(ctx, SLM_ERR_CAPACITY, "topk_logits: beyond the context caps (requests %d, beams %d, vocab %d)",
                    ctx->caps.max_requests, ctx->caps.max_beams, ctx->caps.max_vocab);
    if (logits_dtype != SLM_F32 && logits_dtype != SLM_BF16)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk_logits: logits must be fp32 or bf16");
    if (num_requests == 0) return ok(ctx);
    if (!logits || !cum || !tokens || !parent || !cum_out)
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk_logits: NULL tensor");
    const size_t xe = logits_dtype == SLM_BF16 ? 2 : 4;
    if (((uintptr_t)logits & (xe - 1)) || ((uintptr_t)cum & 3) || ((uintptr_t)tokens & 3) || ((uintptr_t)parent & 3) ||
        ((uintptr_t)cum_out & 3) || ((uintptr_t)lse_out & 3))
        return fail(ctx, SLM_ERR_INVALID_ARG, "topk_logits: misaligned tensor");
    const size_t R = num_requests;
    const size_t xb = R * beams_in * (size_t)vocab * xe, cb = R * beams_in * 4, ob = R * width * 4;
    const void* outs[] = {tokens, parent, cum_out};
    for (const void* o : outs)
        if (overlaps(o, ob, logits, xb) || overlaps(o, ob, cum, cb))
            return fail(ctx, SLM_ERR_ALIAS, "topk_logits: an output overlaps an input");
    if (overlaps(tokens, ob, parent, ob) || overlaps(tokens, ob, cum_out, ob) || overlaps(parent, ob, cum_out, ob))
        return fail(ctx, SLM_ERR_ALIAS, "topk_logits: outputs overlap each other");
    if (lse_out) {
        if (overlaps(lse_out, cb, logits, xb) || overlaps(lse_out, cb, cum, cb))
            return fail(ctx, SLM_ERR_ALIAS, "topk_logits: lse_out overlaps an input");
        for (const void* o : outs)
            if (overlaps(lse_out, cb, o, ob)) return fail(ctx, SLM_ERR_ALIAS, "topk_logits: lse_out overlaps an output");
    }
    slm::TopkParams p{};
    p.logprobs = (const float*)logits; p.cum = cum; p.tokens = tokens; p.parent = parent; p.cum_out = cum_out;
    p.lse_out = lse_out;
    p.logits_bf16 = logits_dtype == SLM_BF16;
    p.err = ctx->err_flag;
    const int64_t R_cap = ctx->caps.max_requests;
    p.req_state = ctx->topk_ws;
    p.stage1 = ctx->topk_ws + slm::kTopkStateWords * R_cap;
    p.list_cap = ctx->topk_lists * ctx->caps.max_beams;
    p.parts = (slm::TopkParams::Piece*)(p.stage1 + R_cap * p.list_cap);
    const int64_t parts_cap = slm::beam_topk_parts_cap(ctx->caps.max_requests, ctx->caps.max_beams);
    p.level2 = (uint64_t*)(p.parts + parts_cap);
    p.level2_w = ctx->caps.max_beams;
    p.level2_cnt = (int*)(p.level2 + R_cap * slm::kTopkLogitChunks * p.level2_w);
    p.num_requests = num_requests; p.beams_in = beams_in; p.vocab = vocab; p.width = width;
    int bpc = ctx->topk_logits_blocks_per_cu[width];
    if (bpc == 0) {
        const bool query = !ctx->dry_run && !ctx->validating;
        bpc = query ? slm::beam_topk_logits_blocks_per_cu(width) : 1;
        if (query) ctx->topk_logits_blocks_per_cu[width] = bpc;
    }
    const int64_t resident = (int64_t)ctx->num_cus * bpc * 4;
    p.seg = slm::beam_topk_logits_segment(num_requests, beams_in, vocab, resident, ctx->topk_lists, parts_cap, p.rpw,
                                          p.rows_per_chunk, p.chunks);
    if (p.chunks > slm::kTopkLogitChunks || p.rows_per_chunk > 256 ||
        (int64_t)p.rows_per_chunk * ((vocab - 1) / p.seg + 2) > slm::kTopkChunkPieces)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "topk_logits: no first-level chunking fits this shape");
    return SLM_LAUNCH(ctx, slm::launch_beam_topk_merge_logits(p, ctx->stream), "topk_logits");
}

slm_status slm_beam_reorder_suffix(slm_ctx* ctx, int32_t n_layers, int32_t num_requests, int32_t width,
                                   int32_t rows, int32_t suffix_cap, int32_t n_heads_kv, int32_t head_dim,
                                   const int32_t* parent, const uint16_t* k_in, const uint16_t* v_in,
                                   uint16_t* k_out, uint16_t* v_out) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (n_layers <= 0 || num_requests <= 0 || width <= 0 || rows < 0 || suffix_cap <= 0 || rows > suffix_cap ||
        n_heads_kv <= 0 || head_dim <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "reorder: a size is out of range");
    if ((n_heads_kv * head_dim) % 8 != 0)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "reorder: n_heads_kv * head_dim must be a multiple of 8");
    if (rows == 0) return ok(ctx);
    if (!parent || !k_in || !v_in || !k_out || !v_out) return fail(ctx, SLM_ERR_INVALID_ARG, "reorder: NULL tensor");
    if (!aligned16(k_in) || !aligned16(v_in) || !aligned16(k_out) || !aligned16(v_out))
        return fail(ctx, SLM_ERR_INVALID_ARG, "reorder: tensors must be 16-byte aligned");
    const size_t sb = (size_t)n_layers * num_requests * width * suffix_cap * n_heads_kv * head_dim * 2;
    const size_t pb = (size_t)num_requests * width * 4;
    const void* outs[] = {k_out, v_out};
    for (const void* o : outs)
        if (overlaps(o, sb, k_in, sb) || overlaps(o, sb, v_in, sb) || overlaps(o, sb, parent, pb))
            return fail(ctx, SLM_ERR_ALIAS, "reorder: an output overlaps an input");
    if (overlaps(k_out, sb, v_out, sb)) return fail(ctx, SLM_ERR_ALIAS, "reorder: outputs overlap each other");
    slm::ReorderParams p{};
    p.parent = parent; p.k_in = k_in; p.v_in = v_in; p.k_out = k_out; p.v_out = v_out; p.err = ctx->err_flag;
    p.n_layers = n_layers; p.num_requests = num_requests; p.width = width; p.rows = rows; p.suffix_cap = suffix_cap;
    p.row_elems = n_heads_kv * head_dim;
    return SLM_LAUNCH(ctx, slm::launch_reorder_suffix(p, ctx->stream), "reorder");
}

slm_status slm_beam_backtrack(slm_ctx* ctx, const int32_t* tokens, const int32_t* parent, int32_t n_merges,
                              int32_t num_requests, int32_t width, int32_t* sequences) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (n_merges <= 0 || num_requests < 0 || width <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "backtrack: a size is out of range");
    if ((int64_t)n_merges * num_requests * width > INT32_MAX)
        return fail(ctx, SLM_ERR_UNSUPPORTED, "backtrack: more than 2^31 - 1 entries");
    if (num_requests == 0) return ok(ctx);
    if (!tokens || !parent || !sequences) return fail(ctx, SLM_ERR_INVALID_ARG, "backtrack: NULL tensor");
    if (!aligned4(tokens) || !aligned4(parent) || !aligned4(sequences))
        return fail(ctx, SLM_ERR_INVALID_ARG, "backtrack: tensors must be 4-byte aligned");
    const size_t nb = (size_t)n_merges * num_requests * width * 4;
    if (overlaps(sequences, nb, tokens, nb) || overlaps(sequences, nb, parent, nb))
        return fail(ctx, SLM_ERR_ALIAS, "backtrack: sequences overlap an input");
    slm::BacktrackParams p{};
    p.tokens = tokens; p.parent = parent; p.seq = sequences; p.err = ctx->err_flag;
    p.n_merges = n_merges; p.num_requests = num_requests; p.width = width;
    return SLM_LAUNCH(ctx, slm::launch_backtrack(p, ctx->stream), "backtrack");
}

namespace {

// The launches of one fixed-step beam search, in order (see slm_beam_search).
// Stops at the first status other than SLM_OK.
slm_status beam_search_launches(slm_ctx* ctx, const slm_beam_search_args* a) {
    const int N = a->n_steps, R = a->num_requests, W = a->width;
    const size_t rw = (size_t)R * W;
    slm_status s = slm_beam_topk_merge(ctx, a->logprobs[0], a->cum0, R, 1, a->vocab, W, a->tokens, a->parent,
                                       a->cum);
    if (s != SLM_OK) return s;
    for (int t = 1; t <= N; ++t) {
        slm_beam_attn_args d{};
        d.n_layers = a->n_layers; d.num_requests = R; d.width = W; d.prompt_len = a->prompt_len;
        d.hist_len = t - 1; d.suffix_cap = a->suffix_cap; d.n_heads_q = a->n_heads_q; d.n_heads_kv = a->n_heads_kv;
        d.head_dim = a->head_dim; d.scale = a->scale;
        d.q = a->q[t - 1]; d.prefix_k = a->prefix_k; d.prefix_v = a->prefix_v;
        d.suffix_k_in = t > 1 ? a->suffix_k[(t + 1) % 2] : nullptr;
        d.suffix_v_in = t > 1 ? a->suffix_v[(t + 1) % 2] : nullptr;
        d.k_new = a->k_new[t - 1]; d.v_new = a->v_new[t - 1];
        d.parent = a->parent + (t - 1) * rw;
        d.suffix_k_out = a->suffix_k[t % 2]; d.suffix_v_out = a->suffix_v[t % 2];
        d.out = a->attn_out[t - 1]; d.out_dtype = a->out_dtype;
        d.prompt_cu = a->prompt_cu; d.prompt_rows = a->prompt_rows;
        s = slm_beam_decode_attn(ctx, &d);
        if (s != SLM_OK) return s;
        s = slm_beam_topk_merge(ctx, a->logprobs[t], a->cum + (t - 1) * rw, R, W, a->vocab, W, a->tokens + t * rw,
                                a->parent + t * rw, a->cum + t * rw);
        if (s != SLM_OK) return s;
    }
    if (N > 0) {
        s = slm_beam_reorder_suffix(ctx, a->n_layers, R, W, N, a->suffix_cap, a->n_heads_kv, a->head_dim,
                                    a->parent + N * rw, a->suffix_k[N % 2], a->suffix_v[N % 2], a->final_k,
                                    a->final_v);
        if (s != SLM_OK) return s;
    }
    if (a->sequences) s = slm_beam_backtrack(ctx, a->tokens, a->parent, N + 1, R, W, a->sequences);
    return s;
}

}  // namespace

slm_status slm_beam_search(slm_ctx* ctx, const slm_beam_search_args* a) {
    slm_status s = enter(ctx);
    if (s != SLM_OK) return s;
    if (!a) return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: NULL args");
    if (a->n_steps < 0 || a->n_steps > slm::kDecodeMaxSuffix || a->num_requests <= 0 || a->width <= 0 ||
        a->vocab <= 0)
        return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: n_steps %d outside [0, %d] or a size out of range",
                    a->n_steps, slm::kDecodeMaxSuffix);
    if (!a->logprobs || !a->cum0 || !a->tokens || !a->parent || !a->cum)
        return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: NULL pointer");
    if (a->n_steps > 0 && (!a->q || !a->k_new || !a->v_new || !a->attn_out || !a->final_k || !a->final_v))
        return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: NULL per-step pointer array or final suffix");
    if (a->n_steps > 0 && a->suffix_cap < a->n_steps)
        return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: suffix_cap %d < n_steps %d", a->suffix_cap, a->n_steps);
    const size_t rw = (size_t)a->num_requests * a->width, nb = ((size_t)a->n_steps + 1) * rw * 4;
    if (overlaps(a->tokens, nb, a->parent, nb) || overlaps(a->tokens, nb, a->cum, nb) ||
        overlaps(a->parent, nb, a->cum, nb))
        return fail(ctx, SLM_ERR_ALIAS, "beam_search: tokens, parent and cum overlap");
    if (a->n_steps > 0) {
        const size_t sb = (size_t)a->n_layers * rw * a->suffix_cap * a->n_heads_kv * a->head_dim * 2;
        const void* bufs[] = {a->suffix_k[0], a->suffix_k[1], a->suffix_v[0], a->suffix_v[1], a->final_k, a->final_v};
        for (int i = 0; i < 6; ++i) {
            if (!bufs[i]) return fail(ctx, SLM_ERR_INVALID_ARG, "beam_search: NULL suffix buffer");
            for (int j = 0; j < i; ++j)
                if (overlaps(bufs[i], sb, bufs[j], sb))
                    return fail(ctx, SLM_ERR_ALIAS, "beam_search: suffix buffers overlap each other");
        }
        const size_t ob = (size_t)a->n_layers * rw * a->n_heads_q * a->head_dim * (a->out_dtype == SLM_F32 ? 4 : 2);
        const void* state[] = {a->tokens, a->parent, a->cum};
        for (int t = 0; t < a->n_steps; ++t)
            for (const void* p : state)
                if (overlaps(a->attn_out[t], ob, p, nb))
                    return fail(ctx, SLM_ERR_ALIAS, "beam_search: attention output %d overlaps the merge state", t);
    }
    // every launch's own validation first, so that an invalid argument
    // anywhere in the sequence leaves nothing launched
    ctx->validating = true;
    s = beam_search_launches(ctx, a);
    ctx->validating = false;
    if (s != SLM_OK || ctx->dry_run) return s;
    return beam_search_launches(ctx, a);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Packed prefill without any allocation, for callers that cannot allocate
// device memory.  The persistent form's work list, its per-XCD counters and a
// device error word live in `scratch`, a fixed array of every device the
// library runs on; its address on a device is looked up once, with that
// device current, the first time the call runs there.
namespace {

constexpr int kNoAllocPlanEntries = 1 << 18;        // work-list entries (16 bytes each): 4 MiB
constexpr int kNoAllocDevices = 64;
// [kNoAllocPlanEntries] work list, [8] per-XCD counts / offsets / claims
// (written by the plan kernel of every call), [1] the error word used when the
// caller passes no flag of its own
static __device__ __align__(256) int4 scratch[kNoAllocPlanEntries + 9];

struct NoAllocDevice {
    std::mutex mu;            // host-side state of the device (not the device array)
    bool ready = false;
    slm_ctx ctx;              // no workspace of its own: plan_items is this device's scratch
};
NoAllocDevice g_noalloc[kNoAllocDevices];

slm_status noalloc_setup(NoAllocDevice& nd, int dev) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SLM_ERR_DEVICE;
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return SLM_ERR_DEVICE;
    slm_ctx& c = nd.ctx;
    c.device = dev;
    c.num_cus = cus;
    c.max_lds = (size_t)lds;
    c.caps = slm_caps{1, 1, 1, INT32_MAX, INT32_MAX, INT32_MAX};   // bounded by the work list below
    c.plan_items = (int4*)ptr;
    c.plan_cap = kNoAllocPlanEntries;
    c.err_flag = (int*)((int4*)ptr + kNoAllocPlanEntries + 8);
    nd.ready = true;
    return SLM_OK;
}

}  // namespace

extern "C" slm_status slm_packed_prefill_attn_noalloc(void* hip_stream, const uint16_t* q, const uint16_t* k,
                                                      const uint16_t* v, const int32_t* cu_seqlens, int32_t num_seqs,
                                                      int32_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                                                      int32_t n_heads_kv, int32_t head_dim, float scale, void* out,
                                                      slm_dtype out_dtype, int32_t* err_flag) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SLM_ERR_DEVICE;
    if (dev < 0 || dev >= kNoAllocDevices) return SLM_ERR_UNSUPPORTED;
    NoAllocDevice& nd = g_noalloc[dev];
    std::lock_guard<std::mutex> lock(nd.mu);
    if (!nd.ready) {
        const slm_status s = noalloc_setup(nd, dev);
        if (s != SLM_OK) return s;
    }
    slm_ctx& c = nd.ctx;
    int* const own_flag = c.err_flag;
    c.stream = (hipStream_t)hip_stream;
    if (err_flag) c.err_flag = err_flag;
    const slm_status s = slm_packed_prefill_attn(&c, q, k, v, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                                 n_heads_q, n_heads_kv, head_dim, scale, out, out_dtype);
    c.err_flag = own_flag;
    c.stream = nullptr;
    return s;
}
