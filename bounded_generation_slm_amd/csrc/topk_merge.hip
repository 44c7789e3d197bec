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
//   stage 1: one workgroup per (request, beam) row streams the V log-probs,
//            keeping the row's top W keys.  Exact: a global winner from row b
//            has fewer than W candidates of row b ranked above it.
//   stage 2: one workgroup per request streams the Win*W stage-1 keys, keeps
//            the top W, sorts them and writes tokens, parents and scores.
// The streaming selector keeps candidates above a running threshold in an
// LDS buffer; when the buffer passes a soft capacity it radix-selects the
// W-th largest key (8-bit digits, wave64 scans), keeps the W keys at or above
// it and raises the threshold to it, so later candidates are rejected with
// one compare.  Insertion compacts each wave's survivors with ballots.
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

constexpr int kTkThreads = 256;
constexpr int kPerThread = 16;                      // candidates per thread per round
constexpr int kRound = kTkThreads * kPerThread;     // 4096
constexpr int kSoftCap = 2048;                      // compact when above (>= max W)
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
__device__ __forceinline__ uint64_t make_key(float score, uint32_t flat) {
    return ((uint64_t)order_f32(score) << 32) | (uint64_t)(0xFFFFFFFFu - flat);
}

struct SelectorLds {
    uint64_t buf[kPhysCap];
    uint64_t surv[kMaxW];
    int hist[256];
    int wave_tot[kTkThreads / kWave];
    uint64_t thr;          // keys > thr pass the filter
    uint64_t kth;
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

// k-th largest key (1-based) among s.buf[0..cnt).  All threads return it.
__device__ uint64_t select_kth(SelectorLds& s, int cnt, int k) {
    const int tid = threadIdx.x;
    uint64_t prefix = 0, pmask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
        s.hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < cnt; i += kTkThreads) {
            const uint64_t key = s.buf[i];
            if ((key & pmask) == prefix) atomicAdd(&s.hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        const int c = s.hist[255 - tid];            // thread t scans bins from the top
        const int incl = block_inclusive_scan(c, s);
        const int excl = incl - c;
        if (c > 0 && excl < k && k <= incl) {
            s.digit = 255 - tid;
            s.above = excl;
            s.dcnt = c;
        }
        __syncthreads();
        prefix |= (uint64_t)s.digit << shift;
        pmask |= (uint64_t)0xFF << shift;
        k -= s.above;
        const int dcnt = s.dcnt;
        __syncthreads();
        if (dcnt == 1) {                            // the prefix now names one key
            for (int i = tid; i < cnt; i += kTkThreads) {
                const uint64_t key = s.buf[i];
                if ((key & pmask) == prefix) s.kth = key;
            }
            __syncthreads();
            return s.kth;
        }
    }
    return prefix;                                  // all 64 bits fixed
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
        s.thr = kth;
    }
    __syncthreads();
}

// Append every key > thr among this thread's candidates (wave ballots).
__device__ __forceinline__ void insert(SelectorLds& s, const uint64_t (&keys)[kPerThread], uint64_t thr) {
    bool any = false;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) any |= keys[e] > thr;
    if (__ballot(any) == 0) return;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const bool pass = keys[e] > thr;
        const uint64_t mask = __ballot(pass);
        if (mask == 0) continue;
        int base = 0;
        if (lane == 0) base = atomicAdd(&s.cnt, __popcll(mask));
        base = __shfl(base, 0);
        if (pass) s.buf[base + __popcll(mask & ((1ull << lane) - 1))] = keys[e];
    }
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

// Stage 1: per (request, beam) row.  VEC: 16-byte aligned rows (V % 4 == 0).
template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void topk_stage1_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    const int row = blockIdx.x;                     // r * Win + b
    const int b = row % p.beams_in;
    const int V = p.vocab, W = p.width;
    const float* lp = p.logprobs + (int64_t)row * V;
    const float c = p.cum[row];
    const uint32_t fbase = (uint32_t)b * (uint32_t)V;
    if (threadIdx.x == 0) {
        s.cnt = 0;
        s.thr = 0;
    }
    __syncthreads();
    const int rounds = (V + kRound - 1) / kRound;
    f32x4 cur[kPerThread / 4], nxt[kPerThread / 4];
    auto fetch = [&](int rd, f32x4 (&dst)[kPerThread / 4]) {
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j) {
            const int v0 = rd * kRound + (j * kTkThreads + threadIdx.x) * 4;
            if (VEC) {
                dst[j] = v0 < V ? *(const f32x4*)(lp + v0) : f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[j][e] = v0 + e < V ? lp[v0 + e] : 0.f;
            }
        }
    };
    fetch(0, cur);
    for (int rd = 0; rd < rounds; ++rd) {
        if (rd + 1 < rounds) fetch(rd + 1, nxt);
        const uint64_t thr = s.thr;
        uint64_t keys[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = rd * kRound + (j * kTkThreads + threadIdx.x) * 4 + e;
                keys[j * 4 + e] = v < V ? make_key(c + cur[j][e], fbase + (uint32_t)v) : 0ull;
            }
        insert(s, keys, thr);
        __syncthreads();
        if (s.cnt > kSoftCap) compact(s, W);
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j) cur[j] = nxt[j];
    }
    compact(s, W);
    const int n = min(s.cnt, W);
    const int wp = (W + 1) & ~1;                    // even row stride: 16-byte aligned pairs
    uint64_t* out = p.stage1 + (int64_t)row * wp;
    for (int i = threadIdx.x; i < wp; i += kTkThreads) out[i] = i < n ? s.buf[i] : 0ull;
}

// Stage 2: per request, over the Win rows of stage-1 keys (0 = empty slot;
// rows are padded to an even length so pairs load as 16 bytes).
__global__ __launch_bounds__(kTkThreads) void topk_stage2_kernel(const TopkParams p) {
    __shared__ SelectorLds s;
    const int r = blockIdx.x;
    const int W = p.width, V = p.vocab;
    const int64_t n = (int64_t)p.beams_in * ((W + 1) & ~1);
    const uint64_t* in = p.stage1 + (int64_t)r * n;
    if (threadIdx.x == 0) {
        s.cnt = 0;
        s.thr = 0;
    }
    __syncthreads();
    const int64_t rounds = (n + kRound - 1) / kRound;
    for (int64_t rd = 0; rd < rounds; ++rd) {
        const uint64_t thr = s.thr;
        uint64_t keys[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread / 2; ++j) {
            const int64_t i0 = rd * kRound + (int64_t)(j * kTkThreads + threadIdx.x) * 2;
            if (i0 + 1 < n) {
                const u32x4 x = *(const u32x4*)(in + i0);
                keys[2 * j] = ((uint64_t)x[1] << 32) | x[0];
                keys[2 * j + 1] = ((uint64_t)x[3] << 32) | x[2];
            } else {
                keys[2 * j] = i0 < n ? in[i0] : 0ull;
                keys[2 * j + 1] = 0ull;
            }
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
}

}  // namespace

size_t beam_topk_workspace_bytes(int max_requests, int max_beams) {
    return (size_t)max_requests * max_beams * ((max_beams + 1) & ~1) * sizeof(uint64_t);
}

hipError_t launch_beam_topk_merge(const TopkParams& p, hipStream_t stream) {
    if (p.num_requests == 0) return hipSuccess;
    const bool vec = (p.vocab % 4 == 0) && (((uintptr_t)p.logprobs & 15) == 0);
    const unsigned rows = (unsigned)((int64_t)p.num_requests * p.beams_in);
    if (vec)
        hipLaunchKernelGGL(topk_stage1_kernel<true>, dim3(rows), dim3(kTkThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(topk_stage1_kernel<false>, dim3(rows), dim3(kTkThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stage2_kernel, dim3(p.num_requests), dim3(kTkThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace slm
