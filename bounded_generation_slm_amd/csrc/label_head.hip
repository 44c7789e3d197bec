// Prefill-only label head for gfx950.
//
// Operation (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", §1.1,
// prefill-only models): one prefill, then the next-token logits at each
// sequence's last valid token, of the target-label tokens only, turned into
// the business output by softmax, top-K or a fixed mapping.  Only the L
// label rows of the LM head are read, so the head is a B x L x H product
// instead of B x V x H.
//
// Two kernels:
//   logits: one workgroup (4 waves) per 32 sequences x 32 labels; each wave
//           accumulates a quarter of the hidden dimension with
//           v_mfma_f32_32x32x16_bf16 (label rows as the A operand, last-token
//           rows as B, both straight from global memory: every operand byte
//           is used once per tile), and the four partial tiles are summed in
//           LDS in a fixed order (repeated calls agree bitwise);
//   select: one wave per sequence: max, softmax over the labels, then the
//           top K by K rounds of a wave argmax (largest logit, lower label
//           index among equals), with the fixed mapping applied.
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

constexpr int kLhWaves = 4;
constexpr float kLog2eLh = 1.4426950408889634f;

__global__ __launch_bounds__(kLhWaves * kWave) void label_logits_kernel(const LabelHeadParams p) {
    __shared__ float part[kLhWaves][16][64];            // per wave: its f32x16 accumulator, by lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int b0 = blockIdx.x * 32, l0 = blockIdx.y * 32;
    const int H = p.hidden_dim;
    // this lane's rows: label row (A operand) and last-token row (B operand)
    const int lj = l0 + n;
    int lid = lj < p.num_labels ? p.labels[lj] : 0;
    if (lid < 0 || lid >= p.vocab) {
        if (lj < p.num_labels) raise_error(p.err, kErrLabel);
        lid = 0;
    }
    const int b = b0 + n;
    int64_t last = -1;
    if (b < p.num_seqs) {
        const int s0 = p.cu[b], s1 = p.cu[b + 1];
        if (s0 < 0 || s1 < s0 || s1 > p.total_tokens) raise_error(p.err, kErrCuSeqlens);
        else if (s1 > s0) last = s1 - 1;
    }
    const uint16_t* arow = p.lm + (int64_t)lid * H + hf * 8;
    const uint16_t* brow = p.hidden + (last < 0 ? 0 : last) * H + hf * 8;
    const bool bz = last < 0;                           // empty sequence (or past B): a zero row
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const int nks = H / 16, per = (nks + kLhWaves - 1) / kLhWaves;
    const int ks0 = wave * per, ks1 = min(nks, ks0 + per);
    for (int ks = ks0; ks < ks1; ++ks) {
        const u32x4 a = *(const u32x4*)(arow + ks * 16);
        const u32x4 bb = bz ? u32x4{0u, 0u, 0u, 0u} : *(const u32x4*)(brow + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bb), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave != 0) return;
    // element i of lane (n, hf): label l0 + 8 (i / 4) + 4 hf + i % 4, sequence b0 + n
    if (b >= p.num_seqs) return;
    float* zrow = p.logits + (int64_t)b * p.num_labels;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float z = ((part[0][i][lane] + part[1][i][lane]) + part[2][i][lane]) + part[3][i][lane];
        const int l = l0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (l < p.num_labels) zrow[l] = z;
    }
}

constexpr int kLhPerLane = kLabelMax / kWave;           // logits one lane holds at most

// PER: logits per lane, at least ceil(L / 64).  Every loop below is unrolled
// over PER, so a variant sized for 4,096 labels spent ~20 us on 64.
template <int PER>
__global__ __launch_bounds__(kLhWaves * kWave) void label_select_kernel(const LabelHeadParams p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kLhWaves + (threadIdx.x >> 6);
    if (b >= p.num_seqs) return;                        // whole waves: no barriers below
    const int L = p.num_labels;
    const float* zrow = p.logits + (int64_t)b * L;
    float z[PER];                                       // label lane + 64 t
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
        const int j = lane + 64 * t;
        z[t] = j < L ? zrow[j] : -INFINITY;
        m = fmaxf(m, z[t]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float mc = m * kLog2eLh;
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < PER; ++t)
        if (lane + 64 * t < L) s += fast_exp2(fmaf(z[t], kLog2eLh, -mc));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    const float inv = 1.f / s;
    if (p.probs) {
        float* prow = p.probs + (int64_t)b * L;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int j = lane + 64 * t;
            if (j < L) prow[j] = fast_exp2(fmaf(z[t], kLog2eLh, -mc)) * inv;
        }
    }
    // top K: each round takes the largest logit not yet taken, lower index first
    uint64_t taken = 0;                                 // bit t: label lane + 64 t is taken
    for (int k = 0; k < p.k; ++k) {
        float best = -INFINITY;
        int bj = INT32_MAX;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int j = lane + 64 * t;
            if (j < L && !((taken >> t) & 1ull) && (z[t] > best || bj == INT32_MAX)) {
                best = z[t];
                bj = j;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ob = __shfl_xor(best, off);
            const int oj = __shfl_xor(bj, off);
            if (ob > best || (ob == best && oj < bj)) {
                best = ob;
                bj = oj;
            }
        }
        if ((bj & 63) == lane) taken |= 1ull << (bj >> 6);
        if (lane == 0) {
            const int64_t o = (int64_t)b * p.k + k;
            p.top_idx[o] = bj;
            p.top_prob[o] = fast_exp2(fmaf(best, kLog2eLh, -mc)) * inv;
            if (p.top_class) p.top_class[o] = p.map ? p.map[bj] : bj;
        }
    }
}

}  // namespace

hipError_t launch_label_head(const LabelHeadParams& p, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    const dim3 g1((p.num_seqs + 31) / 32, (p.num_labels + 31) / 32);
    hipLaunchKernelGGL(label_logits_kernel, g1, dim3(kLhWaves * kWave), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((p.num_seqs + kLhWaves - 1) / kLhWaves), b2(kLhWaves * kWave);
    const int per = (p.num_labels + kWave - 1) / kWave;     // num_labels <= kLabelMax
    if (per <= 1)
        hipLaunchKernelGGL(label_select_kernel<1>, g2, b2, 0, stream, p);
    else if (per <= 4)
        hipLaunchKernelGGL(label_select_kernel<4>, g2, b2, 0, stream, p);
    else if (per <= 16)
        hipLaunchKernelGGL(label_select_kernel<16>, g2, b2, 0, stream, p);
    else
        hipLaunchKernelGGL(label_select_kernel<kLhPerLane>, g2, b2, 0, stream, p);
    return hipGetLastError();
}

}  // namespace slm
