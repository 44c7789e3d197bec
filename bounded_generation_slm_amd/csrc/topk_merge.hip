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
// Two stages (both HBM-bound streaming, one pass over their input):
//   stage 1: one workgroup per (request, beam row, vocabulary chunk) streams
//            its log-probs, keeping the chunk's top W keys.  Exact: a global
//            winner has fewer than W candidates of its own chunk above it.
//            Short calls (the first merge has one row per request) split
//            rows into chunks so that enough workgroups fill the GPU.
//   stage 2: one workgroup per request streams the Win*W stage-1 keys, keeps
//            the top W, sorts them and writes tokens, parents and scores.
// The streaming selector keeps candidates above a running threshold in an
// LDS buffer; when the buffer passes a soft capacity it radix-selects the
// W-th largest key (8-bit digits, wave64 scans), keeps the W keys at or above
// it and raises the threshold to it, so later candidates are rejected with
// one compare.  Insertion compacts each wave's survivors with ballots.
#include <algorithm>

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
__device__ uint64_t select_kth(SelectorLds& s, int cnt, int k) {
    const int tid = threadIdx.x;
    uint64_t lo = 0ull, hi = ~0ull;
    int c = cnt;                                    // keys in [lo, hi]
    for (;;) {
        uint64_t mn, mx;
        block_minmax(s, cnt, lo, hi, mn, mx);
        if (k == 1) return mx;
        if (k == c) return mn;
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
__device__ void compact(SelectorLds& s, int width) {
    const int cnt = s.cnt;
    if (cnt <= width) return;                       // uniform: read after a barrier
    const uint64_t kth = select_kth(s, cnt, width);
    if (threadIdx.x == 0) s.spos = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kTkThreads) {
        const uint64_t key = s.buf[i];
        if (key >= kth) s.surv[atomicAdd(&s.spos, 1)] = key;
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

// Bitonic sort of s.buf[0..512) descending (entries >= n padded with 0).
__device__ void sort_desc_512(SelectorLds& s, int n) {
    for (int i = threadIdx.x + n; i < kMaxW; i += kTkThreads) s.buf[i] = 0;
    __syncthreads();
    for (int size = 2; size <= kMaxW; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int t = threadIdx.x;              // 256 threads, one pair each
            const int i = 2 * t - (t & (stride - 1));
            const int j = i + stride;
            const bool desc = (i & size) == 0;
            const uint64_t a = s.buf[i], b = s.buf[j];
            if ((a < b) == desc) {
                s.buf[i] = b;
                s.buf[j] = a;
            }
            __syncthreads();
        }
}

__device__ __forceinline__ uint64_t load_relaxed(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- stage 1: one wave per (request, beam row, vocabulary chunk) ----
//
// Each wave owns a private LDS region (candidate buffer, survivor area, 256
// radix bins); its candidate count and threshold live in wave-uniform
// registers, so the streaming loop has no workgroup barrier and no LDS
// atomic.  Loads are unconditional (addresses clamped into the chunk, values
// masked afterwards) and rotate through four register buffers, four rounds in
// flight.  A candidate is first screened on its fp32 score alone; the 64-bit
// key is built only in the rare rounds where a lane passes.
constexpr int kWLanes = 64;
constexpr int kWPerLane = 8;                        // candidates per lane per round
constexpr int kWRound = kWLanes * kWPerLane;        // 512
constexpr int kWDepth = 4;                          // rounds in flight
constexpr int kWBins = 256;

// LDS layout of one wave, in 8-byte words: buf[soft + kWRound], surv[even(W)],
// hist[kWBins] ints.
__host__ __device__ inline int wave_soft_cap(int W) { return W > 256 ? 512 : 256; }
__host__ __device__ inline int wave_lds_words(int W) {
    return wave_soft_cap(W) + kWRound + ((W + 1) & ~1) + kWBins / 2;
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
// live [min, max] range (see select_kth).
__device__ uint64_t wave_select_kth(const uint64_t* buf, int* hist, int cnt, int k, int lane) {
    uint64_t lo = 0ull, hi = ~0ull;
    int c = cnt;
    for (;;) {
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
        int above = incl - sum, digit = -1, dabove = 0, dcnt = 0;
#pragma unroll
        for (int j = 0; j < kWBins / kWLanes; ++j) {
            if (h[j] > 0 && above < k && k <= above + h[j]) {
                digit = kWBins - 1 - (lane * (kWBins / kWLanes) + j);
                dabove = above;
                dcnt = h[j];
            }
            above += h[j];
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
// W-th key (the new threshold); cnt becomes W.
__device__ uint64_t wave_compact(uint64_t* buf, uint64_t* surv, int* hist, int& cnt, int W, int lane) {
    const uint64_t kth = wave_select_kth(buf, hist, cnt, W, lane);
    int pos = 0;
    for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
        const int i = i0 + lane;
        const uint64_t key = i < cnt ? buf[i] : 0ull;
        const bool keep = i < cnt && key >= kth;
        const uint64_t m = __ballot(keep);
        if (keep) surv[pos + lanes_below(m)] = key;
        pos += __popcll(m);
    }
    wave_fence();
    for (int i = lane; i < W; i += kWLanes) buf[i] = surv[i];
    wave_fence();
    cnt = W;
    return kth;
}

template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void topk_stage1_kernel(const TopkParams p) {
    extern __shared__ __attribute__((aligned(16))) uint64_t wave_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * (kTkThreads / kWLanes) + wave;
    const int64_t items = (int64_t)p.num_requests * p.beams_in * p.chunks;
    if (item >= items) return;                      // no barriers below: waves are independent
    const int W = p.width;
    uint64_t* buf = wave_lds + (size_t)wave * wave_lds_words(W);
    const int soft = wave_soft_cap(W);
    uint64_t* surv = buf + soft + kWRound;
    int* hist = (int*)(surv + ((W + 1) & ~1));

    const int chunk = (int)(item % p.chunks);
    const int64_t row = item / p.chunks;            // r * Win + b
    const int r = (int)(row / p.beams_in), b = (int)(row % p.beams_in);
    const int V = p.vocab;
    const int v_begin = chunk * p.chunk_len;
    const int v_end = min(V, v_begin + p.chunk_len);
    const float* lp = p.logprobs + row * V;
    const float c = p.cum[row];
    const uint32_t fbase = (uint32_t)b * (uint32_t)V;
    // start from the request's shared threshold: the best W-th key any
    // finished chunk of this request has published (a lower bound of the
    // request's final W-th key, so filtering with it is exact)
    uint64_t thr = uniform_u64(__hip_atomic_load(p.req_thr + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    int cnt = 0;

    const int n = v_end - v_begin;
    const int rounds = (n + kWRound - 1) / kWRound;
    constexpr int NV = kWPerLane / 4;
    f32x4 B0[NV], B1[NV], B2[NV], B3[NV];
    auto fetch = [&](int rd, f32x4 (&dst)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int v0 = v_begin + rd * kWRound + (j * kWLanes + lane) * 4;
            if (VEC) {
                dst[j] = *(const f32x4*)(lp + min(v0, v_end - 4));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[j][e] = lp[min(v0 + e, v_end - 1)];
            }
        }
    };
    auto round = [&](int rd, const f32x4 (&src)[NV]) {
        const float ts = thr_score(thr);
        float sc[kWPerLane];
        bool maybe = false;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[j * 4 + e] = c + src[j][e];      // the candidate score: one fp32 add
                maybe |= sc[j * 4 + e] >= ts;
            }
        if (__ballot(maybe) == 0) return;           // the common case once a threshold is set
        int tot = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = v_begin + rd * kWRound + (j * kWLanes + lane) * 4 + e;
                const uint64_t key = v < v_end ? make_key(sc[j * 4 + e], fbase + (uint32_t)v) : 0ull;
                const bool pass = key > thr;
                const uint64_t m = __ballot(pass);
                if (pass) buf[cnt + tot + lanes_below(m)] = key;
                tot += __popcll(m);
            }
        cnt += tot;
        if (cnt > soft) {
            wave_fence();
            thr = wave_compact(buf, surv, hist, cnt, W, lane);
        }
    };
    fetch(0, B0);
    fetch(1, B1);
    fetch(2, B2);
    for (int rd = 0; rd < rounds; rd += kWDepth) {
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
    wave_fence();
    if (cnt > W) thr = wave_compact(buf, surv, hist, cnt, W, lane);
    // publish this chunk's W-th key when it alone holds W candidates
    if (cnt >= W && lane == 0) atomicMax((unsigned long long*)p.req_thr + r, (unsigned long long)thr);
    const uint64_t gu = uniform_u64(__hip_atomic_load(p.req_thr + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    // append the keys not below the shared threshold to the request's list
    int total = 0;
    for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
        const int i = i0 + lane;
        total += __popcll(__ballot(i < cnt && buf[i] >= gu));
    }
    int base = 0;
    if (lane == 0 && total > 0) base = atomicAdd(p.req_cnt + r, total);
    base = __shfl(base, 0);
    uint64_t* list = p.stage1 + (int64_t)r * p.list_cap;
    for (int i0 = 0; i0 < cnt; i0 += kWLanes) {
        const int i = i0 + lane;
        const bool keep = i < cnt && buf[i] >= gu;
        const uint64_t m = __ballot(keep);
        if (keep) list[base + lanes_below(m)] = buf[i];
        base += __popcll(m);
    }
}

// Stage 2: per request, over the keys the chunks appended to its list.
__global__ __launch_bounds__(kTkThreads) void topk_stage2_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    const int r = blockIdx.x;
    const int W = p.width, V = p.vocab;
    const int n = p.req_cnt[r];
    const uint64_t* in = p.stage1 + (int64_t)r * p.list_cap;
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
            keys[j] = i < n ? in[i] : 0ull;
        }
        insert(s, keys, thr);
        __syncthreads();
        if (s.cnt > kSoftCap) compact(s, W);
    }
    compact(s, W);
    sort_desc_512(s, min(s.cnt, W));
    for (int j = threadIdx.x; j < W; j += kTkThreads) {
        const uint64_t key = s.buf[j];
        const uint32_t f = 0xFFFFFFFFu - (uint32_t)key;
        p.tokens[(int64_t)r * W + j] = (int32_t)(f % (uint32_t)V);
        p.parent[(int64_t)r * W + j] = (int32_t)(f / (uint32_t)V);
        p.cum_out[(int64_t)r * W + j] = unorder_f32((uint32_t)(key >> 32));
    }
    // leave the request's shared state cleared for the next call
    if (threadIdx.x == 0) {
        __hip_atomic_store(p.req_thr + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.req_cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

size_t beam_topk_workspace_bytes(int max_requests, int max_beams) {
    // per request: a shared threshold (8 B), an append count (4 B, padded to
    // 8) and a list of up to max(max_beams, kTopkMaxChunks) * max_beams keys
    const size_t per_req_lists = std::max<size_t>((size_t)max_beams, kTopkMaxChunks);
    return (size_t)max_requests * (2 + per_req_lists * max_beams) * sizeof(uint64_t);
}

int beam_topk_chunks(int num_requests, int beams_in, int vocab, int max_chunks) {
    const int64_t rows = (int64_t)num_requests * beams_in;
    int64_t c = (kTopkMinItems + rows - 1) / rows;           // enough waves to fill the GPU
    c = std::min<int64_t>(c, std::max<int64_t>(1, vocab / (8 * kWRound)));  // chunks of 8+ wave rounds
    c = std::min<int64_t>(c, std::min(max_chunks, kTopkMaxChunks));  // the request's list must hold them
    return (int)std::max<int64_t>(1, c);
}

hipError_t launch_beam_topk_merge(const TopkParams& p, hipStream_t stream) {
    if (p.num_requests == 0) return hipSuccess;
    const bool vec = (p.vocab % 4 == 0) && (((uintptr_t)p.logprobs & 15) == 0) && (p.chunk_len % 4 == 0);
    // stage 2 resets the shared state it consumed; nothing else touches it
    const int64_t items = (int64_t)p.num_requests * p.beams_in * p.chunks;
    const int64_t blocks = (items + kTkThreads / kWLanes - 1) / (kTkThreads / kWLanes);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)wave_lds_words(p.width) * sizeof(uint64_t) * (kTkThreads / kWLanes);
    if (vec)
        hipLaunchKernelGGL(topk_stage1_kernel<true>, dim3((unsigned)blocks), dim3(kTkThreads), lds, stream, p);
    else
        hipLaunchKernelGGL(topk_stage1_kernel<false>, dim3((unsigned)blocks), dim3(kTkThreads), lds, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stage2_kernel, dim3(p.num_requests), dim3(kTkThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) {
        // stage 2 clears the shared state; without it it must not leak into the next call
        (void)hipStreamSynchronize(stream);
        (void)hipMemset(p.req_thr, 0, sizeof(uint64_t) * (size_t)p.num_requests);
        (void)hipMemset(p.req_cnt, 0, sizeof(int) * (size_t)p.num_requests);
    }
    return e;
}

}  // namespace slm
