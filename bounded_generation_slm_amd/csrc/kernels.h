// Internal launch interface between the C-ABI layer (slm_api.hip) and the
// kernels.  Host-side validation happens before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <utility>

namespace slm {

// Per-context launch state: the resident workgroups per CU of each kernel
// variant and the dynamic-LDS limits already raised, recorded the first time
// a variant or LDS size is seen, so later launches make no host query (and
// can be captured into a graph).  A context lives on one device, so nothing
// here is shared across devices.
struct LaunchCache {
    int prefill_per_cu[2][2][2] = {};                   // [head_dim 128][two heads per block][bf16 out]
    std::map<std::pair<int, size_t>, int> decode_occ;   // (variant, LDS bytes) -> workgroups per CU
    std::map<int, size_t> decode_lds_limit;             // variant -> dynamic-LDS limit already set
};

// Device error codes written to the context's flag word.
enum DeviceError : int {
    kErrNone = 0,
    kErrCuSeqlens = 1,     // cu_seqlens not monotone / out of [0,T] / length > max_seqlen
    kErrParent = 2,        // parent index outside [0, W)
    kErrSelect = 3,        // a top-k selection did not converge (equal keys: never for valid inputs)
    kErrLabel = 4,         // a label token id outside [0, vocab)
};


struct PrefillParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* cu;
    void* out;
    int* err;
    int num_seqs, total_tokens, max_seqlen;
    int n_heads_q, n_heads_kv, group;   // group = Hq / Hkv
    int heads_per_block;                // query heads of one KV group per workgroup
    int head_blocks;                    // group / heads_per_block
    int q_tiles;                        // query tiles per sequence (from max_seqlen)
    int n_units;                        // num_seqs * Hkv * head_blocks
    float scale_log2;                   // softmax scale * log2(e)
    // plan workspace (persistent form): work units per XCD
    int4* plan_items;                   // {s0, L, unit in sequence, query tile}
    int* plan_count;                    // [8] units per XCD
    int* plan_off;                      // [8] first unit of each XCD in plan_items
    int* plan_claim;                    // [8] per-XCD item counters
    int* plan_done;                     // [8] per-XCD finished-workgroup counters; the plan kernel zeroes
                                        // both, and the last workgroup of each run zeroes them again
    int plan_cap;                       // capacity of plan_items
};
// Prefill phases: the work list of a pack (persistent form only) and the
// attention over it; a plan serves any number of runs over the same pack.
constexpr int kPrefillPlan = 1, kPrefillRun = 2;
hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, bool out_bf16, bool persistent,
                               int num_cus, LaunchCache& cache, hipStream_t stream, int phases);
// the persistent form stages cu_seqlens in LDS: packs of fewer sequences only
constexpr int kPrefillPlanMaxSeqs = 15999;
// plan entries a pack can need: sum over sequences of ceil(L / qt_rows), per unit column
inline int64_t prefill_plan_entries(int64_t max_tokens, int64_t max_seqs, int64_t max_heads_q) {
    return max_tokens * max_heads_q / 128 + max_seqs * max_heads_q;
}

struct GatherParams {
    const void* hidden;
    const int32_t* cu;
    void* out;
    int* err;
    int num_seqs, total_tokens;
    int64_t row_bytes;
    bool vec16;                         // 16-byte copies (row and pointers aligned)
};
hipError_t launch_gather_last(const GatherParams& p, hipStream_t stream);

// Prefill-only label head: last-token hidden rows x label LM-head rows.
struct LabelHeadParams {
    const uint16_t* hidden;             // [T, H] bf16
    const int32_t* cu;                  // [B + 1]
    const uint16_t* lm;                 // [V, H] bf16 (only label rows read)
    const int32_t* labels;              // [L] token ids
    const int32_t* map;                 // [L] or null
    float* logits;                      // [B, L]
    float* probs;                       // [B, L] or null
    int32_t* top_idx;                   // [B, K]
    float* top_prob;                    // [B, K]
    int32_t* top_class;                 // [B, K] or null
    int* err;
    int num_seqs, total_tokens, hidden_dim, vocab, num_labels, k;
};
hipError_t launch_label_head(const LabelHeadParams& p, hipStream_t stream);
constexpr int kLabelMax = 4096;         // labels per call at most
constexpr int kLabelTopMax = 64;        // K at most

struct ReorderParams {
    const int32_t* parent;
    const uint16_t* k_in;
    const uint16_t* v_in;
    uint16_t* k_out;
    uint16_t* v_out;
    int* err;
    int n_layers, num_requests, width, rows, suffix_cap;
    int row_elems;                      // Hkv * D
};
hipError_t launch_reorder_suffix(const ReorderParams& p, hipStream_t stream);

struct BacktrackParams {
    const int32_t* tokens;              // [n_merges, R, W]
    const int32_t* parent;              // [n_merges, R, W]
    int32_t* seq;                       // [R, W, n_merges]
    int* err;
    int n_merges, num_requests, width;
};
hipError_t launch_backtrack(const BacktrackParams& p, hipStream_t stream);

struct DecodeParams {
    const uint16_t* q;
    const uint16_t* prefix_k;
    const uint16_t* prefix_v;
    const uint16_t* suffix_k_in;
    const uint16_t* suffix_v_in;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* parent;
    uint16_t* suffix_k_out;
    uint16_t* suffix_v_out;
    void* out;
    int* err;
    int n_layers, num_requests, width, prompt_len, hist_len, suffix_cap;
    int n_heads_q, n_heads_kv, group;
    float scale_log2;
    const int32_t* prompt_cu;   // [R+1] offsets of prompts packed per layer, or NULL (each prompt_len rows)
    int prompt_rows;            // rows per layer of the packed prompts (prompt_cu[R])
};
hipError_t launch_beam_decode_attn(const DecodeParams& p, int head_dim, bool out_bf16, int num_cus,
                                   LaunchCache& cache, hipStream_t stream);

struct TopkParams {
    const float* logprobs;
    const float* cum;
    int32_t* tokens;
    int32_t* parent;
    float* cum_out;
    uint64_t* stage1;                   // workspace: [R, list_cap] appended stage-1 keys
    uint64_t* req_state;                // workspace: [R] x kTopkStateWords (threshold, count), zero between calls
    int64_t list_cap;                   // keys per request list
    int64_t seg;                        // candidates per stage-1 wave (a multiple of 4)
    int wpr, kslices;                   // sliced ranges: waves per request, slices per wave (0: contiguous)
    bool deep;                          // stage 1 in the deep form (see beam_topk_deep)
    int num_requests, beams_in, vocab, width;
    // merge on logits only (logprobs then holds the logits):
    struct Piece {                      // one row's part of one stage-1 range
        float m, s;                     // max logit, sum of exp(x - m)
        int base, count;                // its kept keys in the request's list
    };
    Piece* parts;                       // workspace: per (stage-1 wave, row it touches)
    uint64_t* level2;                   // workspace: [R, kTopkLogitChunks, list W] first-level top W per chunk
    int* level2_cnt;                    // workspace: [R, kTopkLogitChunks] keys in each
    float* lse_out;                     // [R, Win] each row's log-sum-exp, or null
    int rpw;                            // part slots per stage-1 wave: rows one wave can touch
    int rows_per_chunk, chunks;         // first-level chunks of beam rows per request
    int level2_w;                       // key slots per chunk in level2 (max_beams)
    int* err;                           // device error flag
    bool logits_bf16;                   // merge on logits: bf16 logits (else fp32)
};
constexpr int kTopkLogitChunks = 64;    // first-level chunks per request at most
constexpr int kTopkChunkPieces = 512;   // pieces per first-level chunk at most
hipError_t launch_beam_topk_merge(const TopkParams& p, hipStream_t stream);
hipError_t launch_beam_topk_merge_logits(const TopkParams& p, hipStream_t stream);
size_t beam_topk_workspace_bytes(int max_requests, int max_beams);
int64_t beam_topk_lists(int max_beams);         // list slots (of up to max_beams keys) per request
int64_t beam_topk_parts_cap(int max_requests, int max_beams);
// candidates per stage-1 wave of the merge on logits: as beam_topk_segment, with
// every piece (one row's part of one range) taking a list slot, and the waves'
// part slots within parts_cap; sets rpw
int64_t beam_topk_logits_segment(int num_requests, int beams_in, int vocab, int64_t resident_waves, int64_t lists,
                                 int64_t parts_cap, int& rpw, int& rows_per_chunk, int& chunks);
int beam_topk_logits_blocks_per_cu(int width);
// candidates per stage-1 wave: the call split evenly over the resident waves,
// at least kTopkMinRange, and few enough ranges per request for its list
// (`lists` slots of W keys)
int64_t beam_topk_segment(int num_requests, int beams_in, int vocab, int64_t resident_waves, int64_t lists);
// Stage 1 runs in one of two forms: four rounds of loads in flight per wave
// at four workgroups per CU, or the deep form, eight rounds at three
// workgroups per CU with each wave's issue priority rotated.  The deep form
// serves widths above 256 (whose larger buffers need it) and calls of at
// least kTopkDeepMin candidates at any width: over the short-prompt search's
// merges (486M candidates, W = 100) it measured 4.6% faster, while calls of
// 78M candidates were even or up to 3.6% slower and the search's first
// merge (4.9M) 7% slower: the deeper pipeline pays on long streams, more
// waves on short ones.
constexpr int64_t kTopkDeepMin = (int64_t)1 << 27;
bool beam_topk_deep(int width, int64_t candidates);
int beam_topk_blocks_per_cu(int width, bool deep);   // resident stage-1 workgroups (4 waves) per CU
// Shortest stage-1 range of the merge on log-probs (first merges, one beam
// per request, measured best at 2,048: 1,024 tied at 8 x 400 beams and ran
// 4% slower at 32 x 100, 4,096 ran 10-35% slower)
constexpr int64_t kTopkMinRange = 2048;
// shortest sliced range, and shortest range of the merge on logits
constexpr int64_t kTopkMinSegment = 4096;
constexpr int kTopkStateWords = 64;     // 512-byte state line per request
constexpr int kTopkMaxChunks = 64;      // list slots per request at least
// stage-1 slices per wave when a request's candidates are sliced over its
// waves (each slice costs the stream pipeline one refill: 3 measured best
// against 2, 4 and 8 at 151,936-token vocabularies)
constexpr int kTopkSlices = 3;
size_t beam_decode_lds_bytes(int head_dim, int prompt_len);
constexpr int kTopkMaxWidth = 512;
constexpr int kDecodeMaxSuffix = 8;     // hist_len + 1 <= 8

}  // namespace slm
