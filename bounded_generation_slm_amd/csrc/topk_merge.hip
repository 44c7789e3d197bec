// Beam top-k merge for gfx950.
//
// Operation (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", §1.1):
// every step takes local candidates from each beam's token distribution,
// merges them with the cumulative scores and keeps a fixed number, recording
// each survivor's parent beam.  The candidate score is the fp32 sum
// cum[b] + logprob[b, v]; candidates rank by score descending, then by flat
// index f = b*V + v ascending.
//
// Keys: every candidate becomes one unique 64-bit key,
//   key = order(score) << 32 | (0xFFFFFFFF - f),
// where order() maps fp32 bits to an unsigned integer with the same order
// (-0 is canonicalised to +0 first, so the two compare equal as in IEEE).
// A larger key ranks first, and no two keys are equal, so "the top W" is a
// unique set and every selection below is exact.
//
// Two stages:
//   stage 1: each request's candidates are split among an equal share of
//            the resident waves, each wave taking kTopkSlices equal slices
//            spread over the request (one from each group of slices, in
//            alternating order, so a wave with an early, in a search
//            higher-ranked and costlier, slice also gets a late one); where
//            slices would be short, the flattened candidates of the call are
//            split into equal contiguous ranges instead.  A wave streams its
//            candidates once, keeping its top W keys of each request against
//            a threshold shared per request, and appends the keys not below
//            that shared bound (nor its own threshold) to the request's
//            list.  Exact: every
//            threshold is backed by W keys at or above it, so no final
//            winner is dropped.
//   stage 2: one workgroup per request reads its list, keeps the top W and
//            writes tokens, parents and scores in rank order.
// The streaming selector keeps candidates above a running threshold in an
// LDS buffer; when the buffer passes a soft capacity it radix-selects the
// W-th largest key (8-bit digits, wave64 scans), keeps the W keys at or above
// it and raises the threshold to it, so later candidates are rejected with
// one compare.  Insertion compacts each wave's survivors with ballots.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

constexpr int kTkThreads = 256;
constexpr int kPerThread = 16;                      // candidates per thread per round
constexpr int kRound = kTkThreads * kPerThread;     // 4096
constexpr int kSoftCap = 1024;                      // compact when above (>= max W)
constexpr int kPhysCap = kSoftCap + kRound;         // a full round always fits
constexpr int kMaxW = 512;

__device__ __forceinline__ uint32_t order_f32(float s) {
    uint32_t u = __builtin_bit_cast(uint32_t, s);
    u = (u == 0x80000000u) ? 0u : u;                // -0 ranks as +0
    return u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float unorder_f32(uint32_t o) {
    const uint32_t u = (o >> 31) ? (o ^ 0x80000000u) : ~o;
    return __builtin_bit_cast(float, u);
}
// Lowest score a key above thr can have: keys > thr need score >= this
// (equal scores are decided by the index half of the key).
__device__ __forceinline__ float thr_score(uint64_t thr) {
    const uint32_t hi = (uint32_t)(thr >> 32);
    return hi <= 0x007FFFFFu ? -INFINITY : unorder_f32(hi);   // at or below -inf's order
}
__device__ __forceinline__ uint64_t make_key(float score, uint32_t flat) {
    return ((uint64_t)order_f32(score) << 32) | (uint64_t)(0xFFFFFFFFu - flat);
}

constexpr int kBins = 2048;                         // radix-select bins per pass
constexpr int kBinBits = 11;
constexpr int kBinsPerThread = kBins / kTkThreads;

struct SelectorLds {
    uint64_t buf[kPhysCap];
    uint64_t surv[kMaxW];
    int hist[kBins];
    int wave_tot[kTkThreads / kWave];
    uint64_t wmin[kTkThreads / kWave], wmax[kTkThreads / kWave];
    uint64_t thr;          // keys > thr pass the filter
    int cnt;
    int spos;
    int digit, above, dcnt;
};

// Inclusive scan of one int per thread across the workgroup.
__device__ int block_inclusive_scan(int x, SelectorLds& s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s.wave_tot[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += s.wave_tot[w];
    __syncthreads();
    return x + add;
}

// Smallest and largest key of s.buf[0..cnt) inside [lo, hi]; all threads get them.
__device__ void block_minmax(SelectorLds& s, int cnt, uint64_t lo, uint64_t hi, uint64_t& mn, uint64_t& mx) {
    uint64_t a = ~0ull, b = 0ull;
    for (int i = threadIdx.x; i < cnt; i += kTkThreads) {
        const uint64_t key = s.buf[i];
        if (key >= lo && key <= hi) {
            a = key < a ? key : a;
            b = key > b ? key : b;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t x = __shfl_xor(a, off), y = __shfl_xor(b, off);
        a = x < a ? x : a;
        b = y > b ? y : b;
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s.wmin[wave] = a;
        s.wmax[wave] = b;
    }
    __syncthreads();
    mn = s.wmin[0];
    mx = s.wmax[0];
    for (int w = 1; w < kTkThreads / kWave; ++w) {
        mn = s.wmin[w] < mn ? s.wmin[w] : mn;
        mx = s.wmax[w] > mx ? s.wmax[w] : mx;
    }
    __syncthreads();
}

// k-th largest key (1-based) among s.buf[0..cnt).  All threads return it.
// Radix select whose 2048 bins always span the live [min, max] range of the
// keys still in play, so concentrated keys (log-probs share their sign and
// exponent bits) still spread over the bins instead of piling into one; one
// pass usually leaves a handful of keys.
// Each pass narrows [lo, hi] to one bin, at least 11 bits fewer, so distinct
// keys finish within 7 passes; kSelectPasses bounds the loop regardless.
constexpr int kSelectPasses = 16;
__device__ uint64_t select_kth(SelectorLds& s, int cnt, int k, int* err) {
    const int tid = threadIdx.x;
    uint64_t lo = 0ull, hi = ~0ull;
    int c = cnt;                                    // keys in [lo, hi]
    for (int pass = 0;; ++pass) {
        uint64_t mn, mx;
        block_minmax(s, cnt, lo, hi, mn, mx);
        if (k == 1) return mx;
        if (k == c) return mn;
        if (pass == kSelectPasses || mn == mx) {   // equal keys: not a valid input
            if (tid == 0) raise_error(err, kErrSelect);
            return mn;
        }
        lo = mn;
        hi = mx;                                    // c >= 2 distinct keys: mn < mx
        const int bits = 64 - __clzll(hi - lo);
        const int shift = bits > kBinBits ? bits - kBinBits : 0;
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) s.hist[tid + j * kTkThreads] = 0;
        __syncthreads();
        for (int i = tid; i < cnt; i += kTkThreads) {
            const uint64_t key = s.buf[i];
            if (key >= lo && key <= hi) atomicAdd(&s.hist[(key - lo) >> shift], 1);
        }
        __syncthreads();
        // thread t owns bins kBins-1-(t*8 .. t*8+7), scanning from the top
        int h[kBinsPerThread], sum = 0;
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) {
            h[j] = s.hist[kBins - 1 - (tid * kBinsPerThread + j)];
            sum += h[j];
        }
        const int incl = block_inclusive_scan(sum, s);
        int above = incl - sum;
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) {
            if (h[j] > 0 && above < k && k <= above + h[j]) {
                s.digit = kBins - 1 - (tid * kBinsPerThread + j);
                s.above = above;
                s.dcnt = h[j];
            }
            above += h[j];
        }
        __syncthreads();
        const uint64_t d = (uint64_t)s.digit;
        k -= s.above;
        c = s.dcnt;
        __syncthreads();
        const uint64_t nlo = lo + (d << shift);
        const uint64_t span = (shift == 0) ? 0ull : ((1ull << shift) - 1ull);
        hi = (hi - nlo > span) ? nlo + span : hi;
        lo = nlo;
    }
}

// Keep exactly the W largest keys in s.buf[0..W); raise the threshold.
__device__ void compact(SelectorLds& s, int width, int* err) {
    const int cnt = s.cnt;
    if (cnt <= width) return;                       // uniform: read after a barrier
    const uint64_t kth = select_kth(s, cnt, width, err);
    if (threadIdx.x == 0) s.spos = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kTkThreads) {
        const uint64_t key = s.buf[i];
        if (key >= kth) {
            const int pos = atomicAdd(&s.spos, 1);
            if (pos < width) s.surv[pos] = key;     // exactly width for distinct keys
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < width; i += kTkThreads) s.buf[i] = s.surv[i];
    if (threadIdx.x == 0) {
        s.cnt = width;
        s.thr = kth > s.thr ? kth : s.thr;
    }
    __syncthreads();
}

// Append every key > thr among this thread's candidates: one ballot per
// candidate slot gives each passing key its offset, and one LDS atomic per
// wave reserves the wave's slots.
__device__ __forceinline__ void insert(SelectorLds& s, const uint64_t (&keys)[kPerThread], uint64_t thr) {
    bool any = false;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) any |= keys[e] > thr;
    if (__ballot(any) == 0) return;                 // wave-uniform
    int off[kPerThread];
    int tot = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const uint64_t mask = __ballot(keys[e] > thr);
        off[e] = tot + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        tot += __popcll(mask);
    }
    int base = 0;
    if ((threadIdx.x & 63) == 0) base = atomicAdd(&s.cnt, tot);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
        if (keys[e] > thr) s.buf[base + off[e]] = keys[e];
}

// The W kept keys s.buf[0..n) in descending order, with no sort: keys are
// distinct, so a key's position is the number of kept keys above it.  Each
// thread ranks its keys j and j + 256 (W <= 512) in one pass over the kept
// keys, read two at a time (a zero after the last ranks below every key).
// out(pos, key) for every pos < W; positions n..W-1 (fewer than W keys) get
// key 0, which ranks below every key.  s.buf must be final (after a
// barrier); all threads call it.
template <class F>
__device__ __forceinline__ void write_ranked(SelectorLds& s, int n, int W, F&& out) {
    if (threadIdx.x == 0) s.buf[n] = 0ull;          // n <= W <= kMaxW: inside the buffer
    __syncthreads();
    const int j0 = threadIdx.x, j1 = threadIdx.x + kTkThreads;
    const uint64_t k0 = j0 < n ? s.buf[j0] : ~0ull, k1 = j1 < n ? s.buf[j1] : ~0ull;
    int p0 = 0, p1 = 0;
#pragma unroll 4
    for (int i = 0; i < n; i += 2) {
        const uint64_t a = s.buf[i], b = s.buf[i + 1];
        p0 += (a > k0 ? 1 : 0) + (b > k0 ? 1 : 0);
        p1 += (a > k1 ? 1 : 0) + (b > k1 ? 1 : 0);
    }
    if (j0 < W) out(j0 < n ? p0 : j0, j0 < n ? k0 : 0ull);
    if (j1 < W) out(j1 < n ? p1 : j1, j1 < n ? k1 : 0ull);
}

__device__ __forceinline__ uint64_t load_relaxed(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Request r's shared state, one 512-byte line of its own (the requests'
// counters and thresholds land on different memory channels): word 0 the
// shared threshold, word 1 the appended key count.
__device__ __forceinline__ uint64_t* req_thr(const TopkParams& p, int r) {
    return p.req_state + (int64_t)r * kTopkStateWords;
}
__device__ __forceinline__ int* req_cnt(const TopkParams& p, int r) {
    return (int*)(p.req_state + (int64_t)r * kTopkStateWords + 1);
}
// Words 32..63: with m = slots(W) slots and q = ceil(W / m), slot s holds
// the best q-th key that any wave w with w % m == s has held.  m waves with
// disjoint candidates, each holding q keys at or above its slot's value,
// together hold m * q >= W keys at or above the smallest slot: that minimum
// bounds the request's final W-th key from below, and since each slot sees
// the best of many waves it tracks the W-th key of everything the request's
// waves have seen so far, far above any one wave's own W-th key.
constexpr int kSlot0 = 32, kMaxSlots = 32;
__host__ __device__ inline int topk_slots(int W) { return min(kMaxSlots, max(1, (W + 7) / 8)); }
__device__ __forceinline__ uint64_t* req_slot(const TopkParams& p, int r, int s) {
    return p.req_state + (int64_t)r * kTopkStateWords + kSlot0 + s;
}

// ---- stage 1: one wave per equal range of the flattened candidates ----
//
// Each wave owns a private LDS region (candidate buffer and 256 radix bins);
// its candidate count and threshold live in wave-uniform registers, so the
// streaming loop has no workgroup barrier and no LDS atomic.  Loads are
// unconditional (addresses clamped into the chunk, values masked afterwards)
// and rotate through four register buffers, four rounds in flight.  A
// candidate is first screened on its fp32 score alone; the 64-bit key is
// built only in the rare rounds where a lane passes.
constexpr int kWLanes = 64;
constexpr int kWPerLane = 8;                        // candidates per lane per round
constexpr int kWRound = kWLanes * kWPerLane;        // 512
// Rounds in flight per wave: 4 where four workgroups share a CU, 8 in the
// deep form at three (its registers allow it, and fewer waves each need more
// bytes in flight); the deep form serves W > 256, whose wider buffers leave
// room for three workgroups only, and long calls (beam_topk_deep).
__host__ __device__ constexpr int stream_depth(bool deep) { return deep ? 8 : 4; }
__host__ __device__ inline bool wide_width(int W) { return W > kWRound / 2; }
constexpr int kWDepth = 4;                          // the merge on logits: rounds in flight
constexpr int kWBins = 256;

// LDS layout of one wave, in 8-byte words: buf[soft + kWRound], hist[kWBins]
// ints.  Above W = 256 a round's own W-th key is a loose bound (W of its 512
// candidates are above it) and such a wave would compact every round or two
// while its threshold is still loose, so its buffer keeps a round's worth of
// slots (512) free after a compaction; narrower ones compact at 512 keys,
// which raises their threshold sooner.  Four workgroups fit a CU up to
// W = 256, three up to W = 512.
__host__ __device__ inline int wave_soft_cap(int W) { return wide_width(W) ? W + kWRound : kWRound; }
__host__ __device__ inline int wave_lds_words(int W) {
    return wave_soft_cap(W) + kWRound + kWBins / 2;
}

__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_wave_barrier(); }

// Broadcast lane 0's 64-bit value (readfirstlane works on 32-bit ints).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_umin64(uint64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t y = __shfl_xor(x, off);
        x = y < x ? y : x;
    }
    return x;
}
__device__ __forceinline__ uint64_t wave_umax64(uint64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t y = __shfl_xor(x, off);
        x = y > x ? y : x;
    }
    return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// k-th largest (1-based) of buf[0..cnt), wave-level radix select over the
// live [min, max] range (see select_kth).  With k2 > 0, *b2 also receives,
// from the first pass's histogram, a value below which at most cnt - k2 keys
// lie (the lower edge of the bin holding the k2-th largest, minus one): at
// least k2 keys are above it.
__device__ uint64_t wave_select_kth(const uint64_t* buf, int* hist, int cnt, int k, int lane, int* err, int k2 = 0,
                                    uint64_t* b2 = nullptr) {
    uint64_t lo = 0ull, hi = ~0ull;
    int c = cnt;
    for (int pass = 0;; ++pass) {
        uint64_t a = ~0ull, b = 0ull;
        for (int i = lane; i < cnt; i += kWLanes) {
            const uint64_t key = buf[i];
            if (key >= lo && key <= hi) {
                a = key < a ? key : a;
                b = key > b ? key : b;
            }
        }
        const uint64_t mn = wave_umin64(a), mx = wave_umax64(b);
        if (k == 1) return mx;
        if (k == c) return mn;
        if (pass == kSelectPasses || mn == mx) {   // equal keys: not a valid input (8 bits a pass: 8 passes)
            if (lane == 0) raise_error(err, kErrSelect);
            return mn;
        }
        lo = mn;
        hi = mx;
        const int bits = 64 - __clzll(hi - lo);
        const int shift = bits > 8 ? bits - 8 : 0;
#pragma unroll
        for (int j = 0; j < kWBins / kWLanes; ++j) hist[lane + j * kWLanes] = 0;
        wave_fence();
        for (int i = lane; i < cnt; i += kWLanes) {
            const uint64_t key = buf[i];
            if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1);
        }
        wave_fence();
        int h[kWBins / kWLanes], sum = 0;           // lane l owns bins 255-4l .. 252-4l
#pragma unroll
        for (int j = 0; j < kWBins / kWLanes; ++j) {
            h[j] = hist[kWBins - 1 - (lane * (kWBins / kWLanes) + j)];
            sum += h[j];
        }
        wave_fence();
        const int incl = wave_incl_scan(sum, lane);
        int above = incl - sum, digit = -1, dabove = 0, dcnt = 0, digit2 = -1;
#pragma unroll
        for (int j = 0; j < kWBins / kWLanes; ++j) {
            if (h[j] > 0 && above < k && k <= above + h[j]) {
                digit = kWBins - 1 - (lane * (kWBins / kWLanes) + j);
                dabove = above;
                dcnt = h[j];
            }
            if (h[j] > 0 && above < k2 && k2 <= above + h[j]) digit2 = kWBins - 1 - (lane * (kWBins / kWLanes) + j);
            above += h[j];
        }
        if (pass == 0 && k2 > 0) {                  // the first pass's histogram covers every key
            const uint64_t w2 = __ballot(digit2 >= 0);
            if (w2) {
                const uint64_t e2 = lo + ((uint64_t)__shfl(digit2, __builtin_ctzll(w2)) << shift);
                *b2 = e2 > 0 ? e2 - 1ull : 0ull;
            }
        }
        const uint64_t who = __ballot(digit >= 0);  // exactly one lane
        const int src = __builtin_ctzll(who);
        digit = __shfl(digit, src);
        k -= __shfl(dabove, src);
        c = __shfl(dcnt, src);
        const uint64_t nlo = lo + ((uint64_t)digit << shift);
        const uint64_t span = (shift == 0) ? 0ull : ((1ull << shift) - 1ull);
        hi = (hi - nlo > span) ? nlo + span : hi;
        lo = nlo;
    }
}

// Keep exactly the W largest keys of buf[0..cnt) in buf[0..W).  Returns the
// W-th key (the new threshold); cnt becomes W.  In place: a kept key moves
// to pos + (kept lanes below it) <= its own index, and each group of 64 is
// read before any of its writes, so no key is overwritten before it is read.
__device__ uint64_t wave_compact(uint64_t* buf, int* hist, int& cnt, int W, int lane, int* err, int k2 = 0,
                             uint64_t* b2 = nullptr) {
    const uint64_t kth = wave_select_kth(buf, hist, cnt, W, lane, err, k2, b2);
    int pos = 0;
    for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
        const int i = i0 + lane;
        const uint64_t key = i < cnt ? buf[i] : 0ull;
        const bool keep = i < cnt && key >= kth;
        const uint64_t m = __ballot(keep);
        if (keep && pos + lanes_below(m) < W) buf[pos + lanes_below(m)] = key;   // exactly W for distinct keys
        pos += __popcll(m);
    }
    wave_fence();
    cnt = W;
    return kth;
}

// Shared lower bound of request r's W-th key: lane l < m reads slot l, the
// other lanes word 0 (the best single-wave W-th key).
__device__ __forceinline__ const uint64_t* bound_addr(const TopkParams& p, int r, int lane, int m) {
    return p.req_state + (int64_t)r * kTopkStateWords + (lane < m ? kSlot0 + lane : 0);
}
__device__ __forceinline__ uint64_t bound_issue(const TopkParams& p, int r, int lane, int m) {
    return load_relaxed(bound_addr(p, r, lane, m));
}
__device__ __forceinline__ uint64_t bound_take(uint64_t v, int lane, int m) {
    uint64_t s = lane < m ? v : ~0ull;
#pragma unroll
    for (int off = 1; off < kMaxSlots; off <<= 1) {                 // lanes 0..31 hold every slot
        const uint64_t y = __shfl_xor(s, off);
        s = y < s ? y : s;
    }
    const uint64_t slots = uniform_u64(s);                          // lane 0: min over the slots
    const uint64_t w0 = ((uint64_t)__builtin_amdgcn_readlane((int)(v >> 32), 63) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);   // lane 63 >= m
    return slots > w0 ? slots : w0;
}

// A key threshold from one round: the W-th largest of its valid candidates'
// order-preserving score bits, truncated to the top 16 (sign, exponent, 7
// mantissa bits).  At least W of the round's candidates have a key above it,
// so it bounds the request's final W-th key from below.  0 (no bound) when
// fewer than W are valid.  A bitwise search counted with ballots: no LDS,
// one pass over the registers per bit.
__device__ __forceinline__ uint64_t round_bound(const float (&sc)[kWPerLane], const bool (&valid)[kWPerLane],
                                                int W) {
    uint32_t o[kWPerLane];
    int nvalid = 0;
#pragma unroll
    for (int k = 0; k < kWPerLane; ++k) {
        o[k] = valid[k] ? order_f32(sc[k]) : 0u;
        nvalid += __popcll(__ballot(valid[k]));
    }
    if (nvalid < W) return 0ull;
    uint32_t tv = 0;
    for (int b = 31; b >= 16; --b) {
        const uint32_t cand = tv | (1u << b);
        int n = 0;
#pragma unroll
        for (int k = 0; k < kWPerLane; ++k) n += __popcll(__ballot(o[k] >= cand));
        if (n >= W) tv = cand;
    }
    // tv: the W-th largest of the scores' top 16 order bits, so at least W
    // candidates have order >= tv; it is nonzero (order(-inf) > 2^16)
    return ((uint64_t)tv << 32) - 1ull;
}

// The log-probs (logits) are read once: the stream's loads carry the
// non-temporal policy (measured faster than cached loads on this path).  All
// loads are ordinary compiler-visible loads, so the compiler tracks their
// destination registers and places the waits.
// f(integral_constant<int, 0>), f(..1), ... f(..N-1) in order while each
// returns true; true if all did.
template <class F, int... J>
__device__ __forceinline__ bool for_each_step_impl(F&& f, std::integer_sequence<int, J...>) {
    return (f(std::integral_constant<int, J>{}) && ...);
}
template <int N, class F>
__device__ __forceinline__ bool for_each_step(F&& f) {
    return for_each_step_impl(f, std::make_integer_sequence<int, N>{});
}

// Issue priority of the calling wave (s_setprio takes an immediate; k is
// wave-uniform).
__device__ __forceinline__ void set_wave_prio(int k) {
    if (k == 0)
        __builtin_amdgcn_s_setprio(0);
    else if (k == 1)
        __builtin_amdgcn_s_setprio(1);
    else if (k == 2)
        __builtin_amdgcn_s_setprio(2);
    else
        __builtin_amdgcn_s_setprio(3);
}
__device__ __forceinline__ f32x4 stream_load16(const float* p) {
    return __builtin_nontemporal_load((const f32x4*)p);
}
__device__ __forceinline__ float stream_load4(const float* p) { return __builtin_nontemporal_load(p); }

template <bool VEC, int DEPTH>
__global__ __launch_bounds__(kTkThreads, (DEPTH == stream_depth(false) ? 4 : 3)) void topk_stage1_kernel(
    const TopkParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t wave_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wid = (int64_t)blockIdx.x * (kTkThreads / kWLanes) + wave;
    const int V = p.vocab, W = p.width;
    const int64_t req_len = (int64_t)p.beams_in * V;           // candidates of one request
    const int64_t total = (int64_t)p.num_requests * req_len;
    // This wave's candidates: one contiguous range of p.seg, or (sliced) k of
    // the wpr * k equal slices of request w / wpr, one from each group of wpr
    // consecutive slices (l = w % wpr picks which), so every wave streams the
    // same amount and each stretch of rows is spread over many waves.  Slice
    // bounds are multiples of 4 (whole 16-byte loads), the last one the
    // request's end.
    const bool sliced = p.kslices > 0;
    const int64_t den = sliced ? (int64_t)p.wpr * p.kslices : 1;
    const int64_t wl = sliced ? wid % p.wpr : 0;
    const int64_t rbase = sliced ? wid / p.wpr * req_len : 0;
    auto slice_at = [&](int64_t j) {
        return rbase + (j == den ? req_len : (j * req_len / den) & ~(int64_t)3);
    };
    // pass si takes slice si * wpr + l on even passes and the mirrored
    // (si + 1) * wpr - 1 - l on odd ones, so a wave with an early (in a
    // search: higher-ranked, heavier) slice also gets a late one
    auto slice_of = [&](int si) {
        return (si & 1) ? (int64_t)(si + 1) * p.wpr - 1 - wl : (int64_t)si * p.wpr + wl;
    };
    int64_t a = sliced ? slice_at(slice_of(0)) : wid * p.seg;   // this wave's range [a, end)
    if (a >= total) return;                                     // no barriers below: waves are independent
    int64_t end = sliced ? slice_at(slice_of(0) + 1) : min(total, a + p.seg);
    uint64_t* buf = wave_lds + (size_t)wave * wave_lds_words(W);
    const int soft = wave_soft_cap(W);
    int* hist = (int*)(buf + soft + kWRound);

    int r = (int)(a / req_len);
    const int m_slots = topk_slots(W);
    uint64_t thr = bound_take(bound_issue(p, r, lane, m_slots), lane, m_slots);  // keys > thr pass
    uint64_t pub = 0, pubq = 0;                                 // last W-th / q-th keys published for r
    const int q = (W + m_slots - 1) / m_slots;
    const int slot = (int)(wid % m_slots);
    int cnt = 0;

    // Publish a W-th-key bound to word 0 and a q-th-key bound to this wave's
    // slot (each backed by that many of this wave's candidates at or above
    // it).  The atomics return nothing.
    auto publish = [&](uint64_t own, uint64_t oq) {
        if (own > pub && lane == 0) atomicMax((unsigned long long*)req_thr(p, r), (unsigned long long)own);
        if (oq > pubq && lane == 0) atomicMax((unsigned long long*)req_slot(p, r, slot), (unsigned long long)oq);
        pub = own > pub ? own : pub;
        pubq = oq > pubq ? oq : pubq;
    };
    // Keep the W largest keys, raise the threshold to the W-th and publish it
    // and the q-th of them.
    auto shrink = [&]() {
        wave_fence();
        uint64_t oq = 0;                                        // q keys above it: from the same select
        const uint64_t own = wave_compact(buf, hist, cnt, W, lane, p.err, q < W ? q : 0, &oq);
        thr = own > thr ? own : thr;
        if (q >= W) oq = own;
        wave_fence();
        publish(own, oq);
    };
    // Append the keys not below request r's shared threshold, nor below this
    // wave's own threshold (also a bound of r's W-th key), to r's list.
    auto count_keep = [&](uint64_t gu) {
        int k = 0;
        for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
            const int i = i0 + lane;
            k += __popcll(__ballot(i < cnt && buf[i] >= gu));
        }
        return k;
    };
    auto flush = [&]() {
        wave_fence();
        uint64_t gu = bound_take(bound_issue(p, r, lane, m_slots), lane, m_slots);
        gu = thr > gu ? thr : gu;
        int n_keep = count_keep(gu);
        if (n_keep > W) {                                       // at most W keys per flush (list capacity)
            shrink();
            gu = thr > gu ? thr : gu;
            n_keep = count_keep(gu);
        }
        int base = 0;
        if (lane == 0 && n_keep > 0) base = atomicAdd(req_cnt(p, r), n_keep);
        base = __shfl(base, 0);
        uint64_t* list = p.stage1 + (int64_t)r * p.list_cap;
        for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
            const int i = i0 + lane;
            const bool keep = i < cnt && buf[i] >= gu;
            const uint64_t m = __ballot(keep);
            if (keep) list[base + lanes_below(m)] = buf[i];
            base += __popcll(m);
        }
        wave_fence();
        cnt = 0;
    };

    constexpr int NV = kWPerLane / 4;
    // The deep form runs three workgroups per CU, and under oldest-first issue
    // arbitration the workgroups dispatched later to a CU streamed ~15% slower,
    // so the call ended with them.  There each wave steps its issue priority
    // through the four levels, one per group of DEPTH rounds, starting from its
    // index mod 4, so no wave stays behind the others for long.  (At four
    // workgroups per CU the rotation measured slightly slower; that form keeps
    // the default priority.)
    constexpr bool rotate = DEPTH > stream_depth(false);
    int prio = (int)(wid & 3);
    for (int si = 0;;) {
        while (a < end) {
            const int64_t row = a / V;                              // r * Win + b
            const int rr = (int)(row / p.beams_in);
            if (rr != r) {                                          // the range enters the next request
                flush();
                r = rr;
                thr = bound_take(bound_issue(p, r, lane, m_slots), lane, m_slots);
                pub = 0;
                pubq = 0;
            }
            const int64_t pe = min(end, (row + 1) * V);             // this piece: [a, pe) inside one row
            const int n = (int)(pe - a);
            const float* lp = p.logprobs + a;
            const float c = p.cum[row];
            const uint32_t f0 = (uint32_t)(a - (int64_t)r * req_len);   // flat index b*V + v of lp[0]
            const uint64_t* baddr = bound_addr(p, r, lane, m_slots);
            const int rounds = (n + kWRound - 1) / kWRound;
            f32x4 B[DEPTH][NV];
            // loads of round rd (clamped into the piece: rounds past its end
            // re-read valid addresses, and their values are never used)
            auto fetch = [&](int rd, f32x4 (&dst)[NV]) __attribute__((always_inline)) {
    #pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const int i0 = rd * kWRound + (j * kWLanes + lane) * 4;
                    if (VEC) {
                        dst[j] = stream_load16(lp + min(i0, n - 4));
                    } else {
    #pragma unroll
                        for (int e = 0; e < 4; ++e) dst[j][e] = stream_load4(lp + min(i0 + e, n - 1));
                    }
                }
            };
            auto round = [&](int rd, f32x4 (&src)[NV]) __attribute__((always_inline)) {
                float sc[kWPerLane];
    #pragma unroll
                for (int j = 0; j < NV; ++j)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) sc[j * 4 + e] = c + src[j][e];   // the candidate score: one fp32 add
                if (rd == 0) {                                      // a piece's first round: bound it at once
                    bool valid[kWPerLane];
    #pragma unroll
                    for (int j = 0; j < NV; ++j)
    #pragma unroll
                        for (int e = 0; e < 4; ++e) valid[j * 4 + e] = (j * kWLanes + lane) * 4 + e < n;
                    const uint64_t rb = round_bound(sc, valid, W);
                    const uint64_t rq = q < W ? round_bound(sc, valid, q) : rb;
                    thr = rb > thr ? rb : thr;
                    publish(rb, rq);
                }
                const float ts = thr_score(thr);
                bool maybe = false;
    #pragma unroll
                for (int k = 0; k < kWPerLane; ++k) maybe |= sc[k] >= ts;
                if (__ballot(maybe) == 0) return;                   // the common case once a threshold is set
    #pragma unroll
                for (int j = 0; j < NV; ++j)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = sc[j * 4 + e] >= ts;
                        if (__ballot(ok) == 0) continue;            // uniform: no lane has a candidate here
                        const int i = rd * kWRound + (j * kWLanes + lane) * 4 + e;
                        const uint64_t key = (ok && i < n) ? make_key(sc[j * 4 + e], f0 + (uint32_t)i) : 0ull;
                        const bool pass = key > thr;
                        const uint64_t m = __ballot(pass);
                        if (pass) buf[cnt + lanes_below(m)] = key;
                        cnt += __popcll(m);
                    }
                if (cnt > soft) shrink();
            };
            // DEPTH rounds of loads stay in flight: before round rd + j the loads
            // of round rd + j + DEPTH - 1 go out into the buffer round rd + j - 1
            // freed.  The shared bound is read once per group of DEPTH rounds,
            // issued with the group's first loads and taken up at its last round;
            // in a piece's first group it is also read right after round 0 (whose
            // W-th and q-th bounds every wave publishes at about the same time)
            // and taken at rounds 1 and 3, so the waves start filtering on each
            // other's first rounds instead of their own loose thresholds.
            // (Each step is its own instantiation, so every buffer index is a
            // constant and the buffers stay in registers.)
            uint64_t sh = 0;
            int rd = 0;
            auto step = [&](auto jc) __attribute__((always_inline)) {   // false once the piece is done
                constexpr int j = decltype(jc)::value;
                if constexpr (j == 0) {
                    fetch(rd + DEPTH - 1, B[DEPTH - 1]);
                    if (rd != 0) sh = load_relaxed(baddr);
                } else {
                    fetch(rd + DEPTH - 1 + j, B[j - 1]);
                }
                if constexpr (j == 1 || (j == 3 && DEPTH > 4)) {
                    if (rd == 0) {                                  // a piece's first group: take the bound early
                        const uint64_t u = bound_take(sh, lane, m_slots);
                        thr = u > thr ? u : thr;
                        sh = load_relaxed(baddr);
                    }
                }
                if constexpr (j == DEPTH - 1) {
                    const uint64_t u = bound_take(sh, lane, m_slots);
                    thr = u > thr ? u : thr;
                }
                round(rd + j, B[j]);
                if constexpr (j == 0)
                    if (rd == 0) sh = load_relaxed(baddr);          // after this round's own bounds went out
                return rd + j + 1 < rounds;                         // wave-uniform
            };
            for_each_step<DEPTH - 1>([&](auto jc) __attribute__((always_inline)) {
                fetch(decltype(jc)::value, B[decltype(jc)::value]);
                return true;
            });
            for (; rd < rounds; rd += DEPTH) {
                if constexpr (rotate) set_wave_prio(prio++ & 3);
                if (!for_each_step<DEPTH>(step)) break;
            }
            a = pe;
        }
        if (!sliced || ++si == p.kslices) break;
        const int64_t j = slice_of(si);
        a = slice_at(j);
        end = slice_at(j + 1);
    }
    flush();
}

// Stage 2: per request, over the keys the chunks appended to its list.
__global__ __launch_bounds__(kTkThreads) void topk_stage2_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    const int r = blockIdx.x;
    const int W = p.width, V = p.vocab;
    const int n = *req_cnt(p, r);
    const uint64_t* in = p.stage1 + (int64_t)r * p.list_cap;
    if (threadIdx.x == 0) {
        s.cnt = 0;
        s.thr = 0;
    }
    __syncthreads();
    const int rounds = (n + kRound - 1) / kRound;
    auto fetch = [&](int rd, uint64_t (&keys)[kPerThread]) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = rd * kRound + j * kTkThreads + threadIdx.x;
            keys[j] = i < n ? in[i] : 0ull;
        }
    };
    uint64_t cur[kPerThread], nxt[kPerThread];      // the next round's keys load during this round
    fetch(0, cur);
    for (int rd = 0; rd < rounds; ++rd) {
        if (rd + 1 < rounds) fetch(rd + 1, nxt);
        insert(s, cur, s.thr);
        __syncthreads();
        if (s.cnt > kSoftCap) compact(s, W, p.err);
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) cur[j] = nxt[j];
    }
    compact(s, W, p.err);
    write_ranked(s, min(s.cnt, W), W, [&](int j, uint64_t key) {
        const uint32_t f = 0xFFFFFFFFu - (uint32_t)key;
        p.tokens[(int64_t)r * W + j] = (int32_t)(f % (uint32_t)V);
        p.parent[(int64_t)r * W + j] = (int32_t)(f / (uint32_t)V);
        p.cum_out[(int64_t)r * W + j] = unorder_f32((uint32_t)(key >> 32));
    });
    // leave the request's shared state cleared for the next call
    if (threadIdx.x < kSlot0 + kMaxSlots)       // words 0..63: threshold, count, slots
        __hip_atomic_store(p.req_state + (int64_t)r * kTopkStateWords + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}


// ---- the merge on logits: each beam row's log-softmax folded in ----
//
// The score of (b, v) is cum[b] + (x[b, v] - lse[b]) with lse[b] the
// log-sum-exp of row b's logits, so within one row candidates rank by the
// logit alone: a request's top W lie among the top W logits of each row,
// and the top W of each piece (one row's part of one wave's range) contain
// those.  Stage 1 streams the logits once, keeping per piece its W largest
// logit keys (key = order(x) << 32 | ~f) and the piece's (max, sum of
// exp(x - max)); stage 2 combines each row's pieces into its lse, re-keys
// every kept candidate by its fp32 score fl(cum + fl(x - lse)) and selects
// as the merge on log-probs does.  No bound is shared across rows: a
// candidate's score needs its row's lse, known only once the row is done.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLogitFloor = -1e30f;              // running max before any finite logit

__device__ __forceinline__ int64_t part_slot(int64_t wid, int64_t row, int64_t seg, int V, int rpw) {
    return wid * rpw + (row - wid * seg / V);
}

// BF16: the logits are bf16 (8 per 16-byte load; lane l of a round holds
// elements 8l .. 8l + 7), else fp32 (two 16-byte loads of 4, at 4l and 256 + 4l).
template <bool VEC, bool BF16>
__global__ __launch_bounds__(kTkThreads) void topk_logits_stage1_kernel(const TopkParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t wave_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wid = (int64_t)blockIdx.x * (kTkThreads / kWLanes) + wave;
    const int V = p.vocab, W = p.width;
    const int64_t req_len = (int64_t)p.beams_in * V;
    const int64_t total = (int64_t)p.num_requests * req_len;
    int64_t a = wid * p.seg;                                    // this wave's range [a, end)
    if (a >= total) return;                                     // no barriers below: waves are independent
    const int64_t end = min(total, a + p.seg);
    uint64_t* buf = wave_lds + (size_t)wave * wave_lds_words(W);
    const int soft = wave_soft_cap(W);
    int* hist = (int*)(buf + soft + kWRound);

    constexpr int NV = BF16 ? 1 : kWPerLane / 4;               // 16-byte registers per round
    // issue priority stepped through the four levels per group of rounds, as
    // in the merge on log-probs (here it measured faster at every width)
    int prio = (int)(wid & 3);
    // element k (0..7) of this lane in round rd
    auto elem = [&](int rd, int k) {
        return BF16 ? rd * kWRound + lane * 8 + k : rd * kWRound + ((k >> 2) * kWLanes + lane) * 4 + (k & 3);
    };
    while (a < end) {
        const int64_t row = a / V;                              // r * Win + b
        const int r = (int)(row / p.beams_in);
        const int64_t pe = min(end, (row + 1) * V);             // this piece: [a, pe) inside one row
        const int n = (int)(pe - a);
        const float* xp = p.logprobs + a;
        const uint16_t* xh = (const uint16_t*)p.logprobs + a;    // BF16
        const uint32_t f0 = (uint32_t)(a - (int64_t)r * req_len);   // flat index b*V + v of xp[0]
        const int rounds = (n + kWRound - 1) / kWRound;
        uint64_t thr = 0;                                       // keys > thr pass (this piece only)
        int cnt = 0;
        float lm = kLogitFloor, ls = 0.f;                       // lane's running max, sum of exp(x - lm)
        auto shrink = [&]() {
            wave_fence();
            const uint64_t own = wave_compact(buf, hist, cnt, W, lane, p.err);
            thr = own > thr ? own : thr;
            wave_fence();
        };
        using Buf = std::conditional_t<BF16, u32x4, f32x4>;     // one round: 8 bf16 bit pairs, or 2 x 4 fp32
        Buf B0[NV], B1[NV], B2[NV], B3[NV];
        auto fetch = [&](int rd, Buf (&dst)[NV]) {
            if constexpr (BF16) {
                const int i0 = elem(rd, 0);
                if (VEC) {
                    dst[0] = __builtin_nontemporal_load((const u32x4*)(xh + min(i0, n - 8)));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[0][e] = (uint32_t)__builtin_nontemporal_load(xh + min(i0 + 2 * e, n - 1)) |
                                    ((uint32_t)__builtin_nontemporal_load(xh + min(i0 + 2 * e + 1, n - 1)) << 16);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const int i0 = elem(rd, 4 * j);
                    if (VEC) {
                        dst[j] = stream_load16(xp + min(i0, n - 4));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) dst[j][e] = stream_load4(xp + min(i0 + e, n - 1));
                    }
                }
            }
        };
        auto round = [&](int rd, Buf (&src)[NV]) {
            float x[kWPerLane];
            bool valid[kWPerLane];
#pragma unroll
            for (int k = 0; k < kWPerLane; ++k) {
                if constexpr (BF16) {
                    const uint32_t w2 = src[0][k >> 1];
                    x[k] = bf16_bits_to_f32((k & 1) ? (w2 >> 16) : (w2 & 0xFFFFu));
                } else {
                    x[k] = src[k >> 2][k & 3];
                }
                valid[k] = elem(rd, k) < n;
            }
            // the row's normaliser: clamped re-reads are logits of this piece
            // too, so they may join the max but not the sum
            float rmax = x[0];
#pragma unroll
            for (int k = 1; k < kWPerLane; ++k) rmax = fmaxf(rmax, x[k]);
            if (rmax > lm) {
                ls *= fast_exp2((lm - rmax) * kLog2e);
                lm = rmax;
            }
            const float ml = lm * kLog2e;
#pragma unroll
            for (int k = 0; k < kWPerLane; ++k) {
                const float e = fast_exp2(fmaf(x[k], kLog2e, -ml));
                ls += valid[k] ? e : 0.f;
            }
            // candidates: the piece's W largest logits
            if (rd == 0 && W <= kWRound / 2) {                  // a piece's first round: bound it at once
                const uint64_t rb = round_bound(x, valid, W);
                thr = rb > thr ? rb : thr;
            }
            const float ts = thr_score(thr);
            bool maybe = false;
#pragma unroll
            for (int k = 0; k < kWPerLane; ++k) maybe |= x[k] >= ts;
            if (__ballot(maybe) == 0) return;
#pragma unroll
            for (int k = 0; k < kWPerLane; ++k) {
                    const bool ok = x[k] >= ts;
                    if (__ballot(ok) == 0) continue;
                    const int i = elem(rd, k);
                    const uint64_t key = (ok && i < n) ? make_key(x[k], f0 + (uint32_t)i) : 0ull;
                    const bool pass = key > thr;
                    const uint64_t m = __ballot(pass);
                    if (pass) buf[cnt + lanes_below(m)] = key;
                    cnt += __popcll(m);
                }
            if (cnt > soft) shrink();
        };
        fetch(0, B0);
        fetch(1, B1);
        fetch(2, B2);
        for (int rd = 0; rd < rounds; rd += kWDepth) {
            set_wave_prio(prio++ & 3);
            fetch(rd + 3, B3);
            round(rd, B0);
            if (rd + 1 >= rounds) break;
            fetch(rd + 4, B0);
            round(rd + 1, B1);
            if (rd + 2 >= rounds) break;
            fetch(rd + 5, B1);
            round(rd + 2, B2);
            if (rd + 3 >= rounds) break;
            fetch(rd + 6, B2);
            round(rd + 3, B3);
        }
        // the piece's (max, sum of exp(x - max)) over its lanes
        float M = lm;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        float S = ls * fast_exp2((lm - M) * kLog2e);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off);
        // the piece's W largest keys go to request r's list
        wave_fence();
        if (cnt > W) shrink();
        int base = 0;
        if (lane == 0 && cnt > 0) base = atomicAdd(req_cnt(p, r), cnt);
        base = __shfl(base, 0);
        uint64_t* list = p.stage1 + (int64_t)r * p.list_cap;
        for (int i = lane; i < cnt; i += kWLanes) list[base + i] = buf[i];
        if (lane == 0) p.parts[part_slot(wid, row, p.seg, V, p.rpw)] = TopkParams::Piece{M, S, base, cnt};
        wave_fence();
        a = pe;
    }
}

// Stage 2 of the merge on logits, first level: one workgroup per (chunk of
// beam rows, request).  Each row's lse from its pieces (in piece order), then
// the rows' kept candidates re-keyed by score and reduced to the chunk's top
// W, written unsorted to the chunk's level-2 slot.
__global__ __launch_bounds__(kTkThreads) void topk_logits_chunk_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    __shared__ float lse_s[kTkThreads];
    __shared__ int first_s[kTkThreads + 1];                 // first piece of each row (prefix over rows)
    __shared__ int pbase[kTopkChunkPieces];
    __shared__ int pfx[kTopkChunkPieces + 1];               // prefix of the pieces' key counts
    const int c = blockIdx.x, r = blockIdx.y;
    const int W = p.width, V = p.vocab, Win = p.beams_in;
    const int b0 = c * p.rows_per_chunk, b1 = min(Win, b0 + p.rows_per_chunk);
    const int tid = threadIdx.x;
    // rows: lse and piece counts (rows_per_chunk <= kTkThreads: one row per thread)
    int npieces = 0;
    int64_t w0 = 0;
    const int b = b0 + tid;
    if (b < b1) {
        const int64_t row = (int64_t)r * Win + b;
        w0 = row * V / p.seg;
        const int64_t w1 = (row * V + V - 1) / p.seg;
        npieces = (int)(w1 - w0 + 1);
        float M = kLogitFloor;
        for (int64_t w = w0; w <= w1; ++w) M = fmaxf(M, p.parts[part_slot(w, row, p.seg, V, p.rpw)].m);
        float S = 0.f;
        for (int64_t w = w0; w <= w1; ++w) {
            const TopkParams::Piece q = p.parts[part_slot(w, row, p.seg, V, p.rpw)];
            S += q.s * fast_exp2((q.m - M) * kLog2e);
        }
        const float lse = M + __builtin_amdgcn_logf(S) * kLn2;
        lse_s[tid] = lse;
        if (p.lse_out) p.lse_out[row] = lse;
    }
    const int incl = block_inclusive_scan(npieces, s);
    first_s[tid + 1] = incl;
    if (tid == 0) first_s[0] = 0;
    __syncthreads();
    const int total_pieces = first_s[kTkThreads];           // <= kTopkChunkPieces (host sizing)
    if (b < b1) {
        const int64_t row = (int64_t)r * Win + b;
        for (int j = 0; j < npieces; ++j) {
            const TopkParams::Piece q = p.parts[part_slot(w0 + j, row, p.seg, V, p.rpw)];
            pbase[first_s[tid] + j] = q.base;
            pfx[first_s[tid] + j + 1] = q.count;
        }
    }
    if (tid == 0) {
        pfx[0] = 0;
        s.cnt = 0;
        s.thr = 0;
    }
    __syncthreads();
    // prefix of the counts (two entries per thread)
    {
        const int i0 = 1 + 2 * tid, i1 = i0 + 1;
        const int v0 = i0 <= total_pieces ? pfx[i0] : 0, v1 = i1 <= total_pieces ? pfx[i1] : 0;
        const int inc = block_inclusive_scan(v0 + v1, s);
        if (i0 <= total_pieces) pfx[i0] = inc - v1;
        if (i1 <= total_pieces) pfx[i1] = inc;
    }
    __syncthreads();
    const int n = pfx[total_pieces];
    const uint64_t* in = p.stage1 + (int64_t)r * p.list_cap;
    const float* cum = p.cum + (int64_t)r * Win;
    const int rounds = (n + kRound - 1) / kRound;
    for (int rd = 0; rd < rounds; ++rd) {
        const uint64_t thr = s.thr;
        uint64_t keys[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = rd * kRound + j * kTkThreads + tid;
            keys[j] = 0ull;
            if (i < n) {
                int lo = 0, hi = total_pieces - 1;              // the piece holding key i: pfx[k] <= i < pfx[k+1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (pfx[mid] <= i) lo = mid; else hi = mid - 1;
                }
                const uint64_t k = in[pbase[lo] + (i - pfx[lo])];
                const uint32_t f = 0xFFFFFFFFu - (uint32_t)k;
                const int bb = (int)(f / (uint32_t)V);
                const float x = unorder_f32((uint32_t)(k >> 32));
                keys[j] = make_key(cum[bb] + (x - lse_s[bb - b0]), f);
            }
        }
        insert(s, keys, thr);
        __syncthreads();
        if (s.cnt > kSoftCap) compact(s, W, p.err);
    }
    compact(s, W, p.err);
    const int kept = min(s.cnt, W);
    uint64_t* out = p.level2 + ((int64_t)r * kTopkLogitChunks + c) * p.level2_w;
    for (int j = tid; j < kept; j += kTkThreads) out[j] = s.buf[j];
    if (tid == 0) p.level2_cnt[r * kTopkLogitChunks + c] = kept;
}

// Second level: per request, the chunks' keys -> the final W, sorted.
__global__ __launch_bounds__(kTkThreads) void topk_logits_final_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    const int r = blockIdx.x;
    const int W = p.width, V = p.vocab;
    const int n = p.chunks * W;                             // chunk c's keys at [c*W, c*W + cnt_c)
    if (threadIdx.x == 0) {
        s.cnt = 0;
        s.thr = 0;
    }
    __syncthreads();
    const int rounds = (n + kRound - 1) / kRound;
    for (int rd = 0; rd < rounds; ++rd) {
        const uint64_t thr = s.thr;
        uint64_t keys[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int i = rd * kRound + j * kTkThreads + threadIdx.x;
            keys[j] = 0ull;
            if (i < n) {
                const int c = i / W, e = i - c * W;
                if (e < p.level2_cnt[r * kTopkLogitChunks + c])
                    keys[j] = p.level2[((int64_t)r * kTopkLogitChunks + c) * p.level2_w + e];
            }
        }
        insert(s, keys, thr);
        __syncthreads();
        if (s.cnt > kSoftCap) compact(s, W, p.err);
    }
    compact(s, W, p.err);
    write_ranked(s, min(s.cnt, W), W, [&](int j, uint64_t key) {
        const uint32_t f = 0xFFFFFFFFu - (uint32_t)key;
        p.tokens[(int64_t)r * W + j] = (int32_t)(f % (uint32_t)V);
        p.parent[(int64_t)r * W + j] = (int32_t)(f / (uint32_t)V);
        p.cum_out[(int64_t)r * W + j] = unorder_f32((uint32_t)(key >> 32));
    });
    if (threadIdx.x < kSlot0 + kMaxSlots)       // leave the request's state line cleared
        __hip_atomic_store(p.req_state + (int64_t)r * kTopkStateWords + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int64_t beam_topk_lists(int max_beams) {
    // the merge on log-probs needs about max(max_beams, kTopkMaxChunks) slots;
    // the merge on logits one more per beam row (every row boundary inside a
    // range starts a piece of its own)
    return std::max<int64_t>(max_beams, kTopkMaxChunks) + max_beams + 1;
}

int64_t beam_topk_parts_cap(int max_requests, int max_beams) {
    // about one part per row plus two per stage-1 wave (16384 resident waves)
    return (int64_t)max_requests * max_beams + 2 * 16384 + 64;
}

size_t beam_topk_workspace_bytes(int max_requests, int max_beams) {
    // per request: a 512-byte state line (threshold, append count, slots) and
    // a list of beam_topk_lists(max_beams) * max_beams keys; then, for the
    // merge on logits, the pieces, the level-2 keys and their counts
    return (size_t)max_requests * (kTopkStateWords + (size_t)beam_topk_lists(max_beams) * max_beams) *
               sizeof(uint64_t) +
           (size_t)beam_topk_parts_cap(max_requests, max_beams) * sizeof(TopkParams::Piece) +
           (size_t)max_requests * kTopkLogitChunks * max_beams * sizeof(uint64_t) +
           (size_t)max_requests * kTopkLogitChunks * sizeof(int);
}

size_t beam_topk_stage1_lds(int width) {
    return (size_t)wave_lds_words(width) * sizeof(uint64_t) * (kTkThreads / kWLanes);
}

int64_t beam_topk_segment(int num_requests, int beams_in, int vocab, int64_t resident_waves, int64_t lists) {
    const int64_t total = (int64_t)num_requests * beams_in * vocab;
    const int64_t req_len = (int64_t)beams_in * vocab;
    int64_t seg = (total + resident_waves - 1) / std::max<int64_t>(1, resident_waves);   // one range per resident wave
    seg = std::max<int64_t>(seg, kTopkMinRange);
    // a request's list takes at most W keys from each range that overlaps it:
    // ceil(req_len / seg) + 1 ranges must fit its `lists` W-key slots
    seg = std::max<int64_t>(seg, (req_len + lists - 2) / std::max<int64_t>(1, lists - 1));
    return (seg + 3) & ~(int64_t)3;                             // whole float4s
}

hipError_t launch_beam_topk_merge(const TopkParams& p, hipStream_t stream) {
    if (p.num_requests == 0) return hipSuccess;
    const bool vec = (p.vocab % 4 == 0) && (((uintptr_t)p.logprobs & 15) == 0);
    // stage 2 resets the shared state it consumed; nothing else touches it
    const int64_t total = (int64_t)p.num_requests * p.beams_in * p.vocab;
    const int64_t waves = p.kslices > 0 ? (int64_t)p.num_requests * p.wpr : (total + p.seg - 1) / p.seg;
    const int64_t blocks = (waves + kTkThreads / kWLanes - 1) / (kTkThreads / kWLanes);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const size_t lds = beam_topk_stage1_lds(p.width);
    constexpr int D4 = stream_depth(false), D8 = stream_depth(true);
    auto kern = vec ? (p.deep ? topk_stage1_kernel<true, D8> : topk_stage1_kernel<true, D4>)
                    : (p.deep ? topk_stage1_kernel<false, D8> : topk_stage1_kernel<false, D4>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kTkThreads), lds, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stage2_kernel, dim3(p.num_requests), dim3(kTkThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) {
        // stage 2 clears the shared state; without it it must not leak into the next call
        (void)hipStreamSynchronize(stream);
        (void)hipMemset(p.req_state, 0, sizeof(uint64_t) * kTopkStateWords * (size_t)p.num_requests);
    }
    return e;
}

int64_t beam_topk_logits_segment(int num_requests, int beams_in, int vocab, int64_t resident_waves, int64_t lists,
                                 int64_t parts_cap, int& rpw, int& rows_per_chunk, int& chunks) {
    const int64_t total = (int64_t)num_requests * beams_in * vocab;
    const int64_t req_len = (int64_t)beams_in * vocab;
    int64_t seg = (total + resident_waves - 1) / std::max<int64_t>(1, resident_waves);
    seg = std::max<int64_t>(seg, kTopkMinSegment);
    // the pieces of one request: at most ceil(req_len / seg) + 1 ranges overlap
    // it, and each of its beams_in - 1 inner row boundaries splits one more
    const int64_t free_slots = std::max<int64_t>(1, lists - beams_in - 1);
    seg = std::max<int64_t>(seg, (req_len + free_slots - 1) / free_slots);
    seg = (seg + 7) & ~(int64_t)7;                              // whole 16-byte loads of fp32 or bf16
    for (;;) {
        const int64_t waves = (total + seg - 1) / seg;
        const int64_t per = (seg - 1) / vocab + 2;              // rows one range can touch
        // first-level chunks: about 256 workgroups over the call, at most
        // kTkThreads rows and kTopkChunkPieces pieces each, kTopkLogitChunks
        // per request
        const int64_t ppr = (vocab - 1) / seg + 2;              // pieces one row can have
        int64_t rpc = ((int64_t)num_requests * beams_in + 255) / 256;
        rpc = std::min<int64_t>(std::max<int64_t>(rpc, 1), 256);
        rpc = std::min<int64_t>(rpc, std::max<int64_t>(1, kTopkChunkPieces / ppr));
        rpc = std::max<int64_t>(rpc, (beams_in + kTopkLogitChunks - 1) / kTopkLogitChunks);
        const bool chunks_fit = rpc <= 256 && rpc * ppr <= kTopkChunkPieces;
        if ((waves * per <= parts_cap && chunks_fit) || seg >= total) {
            rpw = (int)per;
            rows_per_chunk = (int)rpc;
            chunks = (int)((beams_in + rpc - 1) / rpc);
            return seg;
        }
        seg = (2 * seg + 7) & ~(int64_t)7;
    }
}

hipError_t launch_beam_topk_merge_logits(const TopkParams& p, hipStream_t stream) {
    if (p.num_requests == 0) return hipSuccess;
    const bool vec = (p.vocab % (p.logits_bf16 ? 8 : 4) == 0) && (p.seg % 8 == 0) && (((uintptr_t)p.logprobs & 15) == 0);
    const int64_t total = (int64_t)p.num_requests * p.beams_in * p.vocab;
    const int64_t waves = (total + p.seg - 1) / p.seg;
    const int64_t blocks = (waves + kTkThreads / kWLanes - 1) / (kTkThreads / kWLanes);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const size_t lds = beam_topk_stage1_lds(p.width);
    if (p.logits_bf16) {
        if (vec)
            hipLaunchKernelGGL((topk_logits_stage1_kernel<true, true>), dim3((unsigned)blocks), dim3(kTkThreads), lds,
                               stream, p);
        else
            hipLaunchKernelGGL((topk_logits_stage1_kernel<false, true>), dim3((unsigned)blocks), dim3(kTkThreads), lds,
                               stream, p);
    } else if (vec) {
        hipLaunchKernelGGL((topk_logits_stage1_kernel<true, false>), dim3((unsigned)blocks), dim3(kTkThreads), lds,
                           stream, p);
    } else {
        hipLaunchKernelGGL((topk_logits_stage1_kernel<false, false>), dim3((unsigned)blocks), dim3(kTkThreads), lds,
                           stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_logits_chunk_kernel, dim3(p.chunks, p.num_requests), dim3(kTkThreads), 0, stream, p);
    e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(topk_logits_final_kernel, dim3(p.num_requests), dim3(kTkThreads), 0, stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(stream);
        (void)hipMemset(p.req_state, 0, sizeof(uint64_t) * kTopkStateWords * (size_t)p.num_requests);
    }
    return e;
}

int beam_topk_logits_blocks_per_cu(int width) {
    int n = 0;
    const size_t lds = beam_topk_stage1_lds(width);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)topk_logits_stage1_kernel<true, false>, kTkThreads,
                                                     lds) != hipSuccess ||
        n <= 0)
        n = 1;
    return n;
}

bool beam_topk_deep(int width, int64_t candidates) { return wide_width(width) || candidates >= kTopkDeepMin; }

int beam_topk_blocks_per_cu(int width, bool deep) {
    int n = 0;
    const size_t lds = beam_topk_stage1_lds(width);
    const void* kern = deep ? (const void*)topk_stage1_kernel<true, stream_depth(true)>
                            : (const void*)topk_stage1_kernel<true, stream_depth(false)>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kTkThreads, lds) !=
            hipSuccess || n <= 0)
        n = 1;
    return n;
}

}  // namespace slm
