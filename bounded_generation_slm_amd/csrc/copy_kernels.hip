// Pure data movement on the hot path: last-valid-token gather, the
// parent-indexed suffix K/V reorder and the final backtrack of the parents
// into token sequences.  All are bit copies.
//
// Gather (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", §1.1): a
// prefill-only request reads its result at each sequence's last valid token,
// so only B rows, not T, reach the head that follows.
// Reorder (same page, §1.1 parent index, §1.2 per-beam suffix K/V): after a
// merge every beam takes its parent's suffix rows.
// Backtrack (same page, §1.1: a beam-search request returns a few candidate
// sequences): after the last merge every beam follows its parents back to
// the first merge, one token per merge.
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

// One workgroup per sequence; 16-byte copies when the row allows, else 2-byte.
__global__ __launch_bounds__(256) void gather_last_kernel(const GatherParams p) {
    const int b = blockIdx.x;
    const int s0 = p.cu[b], s1 = p.cu[b + 1];
    const bool bad = s0 < 0 || s1 < s0 || s1 > p.total_tokens;
    if (bad && threadIdx.x == 0) raise_error(p.err, kErrCuSeqlens);
    char* dst = (char*)p.out + (int64_t)b * p.row_bytes;
    const bool empty = bad || s1 == s0;
    const char* src = (const char*)p.hidden + (int64_t)(empty ? 0 : s1 - 1) * p.row_bytes;
    if (p.vec16) {
        for (int64_t i = threadIdx.x; i < p.row_bytes / 16; i += blockDim.x)
            ((u32x4*)dst)[i] = empty ? u32x4{0u, 0u, 0u, 0u} : ((const u32x4*)src)[i];
    } else {
        for (int64_t i = threadIdx.x; i < p.row_bytes / 2; i += blockDim.x)
            ((uint16_t*)dst)[i] = empty ? (uint16_t)0 : ((const uint16_t*)src)[i];
    }
}

// Flat grid over 16-byte chunks (row_elems % 8 == 0) of all copied rows.
__global__ __launch_bounds__(256) void reorder_suffix_kernel(const ReorderParams p, int64_t n_chunks) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n_chunks) return;
    const int cpr = p.row_elems / 8;                  // chunks per row
    const int64_t row = c / cpr;
    const int part = (int)(c % cpr);
    const int i = (int)(row % p.rows);                // suffix row
    const int64_t beam = row / p.rows;                // (l, r, j) flattened
    const int j = (int)(beam % p.width);
    const int64_t lr = beam / p.width;
    const int r = (int)(lr % p.num_requests);
    const int src = p.parent[r * p.width + j];
    if (src < 0 || src >= p.width) {
        raise_error(p.err, kErrParent);
        return;
    }
    const int64_t dst_off = ((beam * p.suffix_cap + i) * p.row_elems) + part * 8;
    const int64_t src_off = (((lr * p.width + src) * p.suffix_cap + i) * p.row_elems) + part * 8;
    *(u32x4*)(p.k_out + dst_off) = *(const u32x4*)(p.k_in + src_off);
    *(u32x4*)(p.v_out + dst_off) = *(const u32x4*)(p.v_in + src_off);
}

// One lane per final beam (r, j): its sequence is written from the last
// merge back to the first.  The [n, R, W] inputs are read a step at a time,
// each step by the W lanes of a request at once; the [R, W, n] output row of a
// beam is contiguous.  A parent outside [0, W) flags the error and leaves the
// earlier entries of that sequence at -1.
__global__ __launch_bounds__(256) void backtrack_kernel(const BacktrackParams p) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (int64_t)p.num_requests * p.width) return;
    const int r = (int)(id / p.width);
    int b = (int)(id % p.width);
    int32_t* out = p.seq + id * p.n_merges;
    for (int t = p.n_merges - 1; t >= 0; --t) {
        const int64_t at = ((int64_t)t * p.num_requests + r) * p.width + b;
        out[t] = p.tokens[at];
        const int nb = p.parent[at];
        if (t > 0 && (nb < 0 || nb >= p.width)) {
            raise_error(p.err, kErrParent);
            for (int u = t - 1; u >= 0; --u) out[u] = -1;
            return;
        }
        b = nb;
    }
}

}  // namespace

hipError_t launch_backtrack(const BacktrackParams& p, hipStream_t stream) {
    const int64_t n = (int64_t)p.num_requests * p.width;
    if (n == 0 || p.n_merges == 0) return hipSuccess;
    hipLaunchKernelGGL(backtrack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gather_last(const GatherParams& p, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_last_kernel, dim3(p.num_seqs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_reorder_suffix(const ReorderParams& p, hipStream_t stream) {
    const int64_t n_chunks = (int64_t)p.n_layers * p.num_requests * p.width * p.rows * (p.row_elems / 8);
    if (n_chunks == 0) return hipSuccess;
    const int64_t blocks = (n_chunks + 255) / 256;
    hipLaunchKernelGGL(reorder_suffix_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n_chunks);
    return hipGetLastError();
}

}  // namespace slm
