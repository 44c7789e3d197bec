// Packed causal GQA prefill attention for gfx950.
//
// Operation (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", abstract
// "Packed Prefill" and §1.2): sequences are packed back to back with no
// padding; each query attends causally to the keys of its own sequence only.
//
// Work decomposition: a workgroup (4 waves) owns one (sequence, KV head, block
// of query heads of that group, query tile).  The query heads of one GQA group
// share every K/V tile staged in LDS.  Each wave owns 32 query rows of one
// head and runs the online softmax in registers:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, K tile from LDS, Q^T in VGPRs)
//   O^T += V^T P^T
// Computing S transposed puts each lane on one query column, so the row max
// and row sum are in-lane plus one cross-half exchange, and the accumulator
// layout of S^T is exactly the B-operand layout P^T needs: no shuffle of P.
// V is written to LDS transposed ([d][key]) with its keys pre-permuted so
// that every V^T operand is a single 16-byte LDS read.
//
// Grid mapping is XCD-aware: the query tiles of one (sequence, head block)
// are consecutive on one XCD (blockIdx % 8), so the K/V rows they share are
// fetched from HBM once and re-read from that XCD's L2.  Heavier tiles (later
// query tiles, which see more keys) are dispatched first within a unit.
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

constexpr int kKT = 64;                 // keys per K/V tile

template <int D, int NH, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(const PrefillParams p) {
    constexpr int QT = 128 / NH;        // query rows per workgroup
    constexpr int WPH = 4 / NH;         // waves per query head
    constexpr int KROW = D + 8;         // K tile row stride (bf16), +16 B against bank conflicts
    constexpr int VROW = kKT + 8;       // V^T tile row stride (bf16)
    constexpr int NKS = D / 16;         // k-steps of S^T over the head dim
    constexpr int NDB = D / 32;         // 32-row blocks of O^T
    constexpr int NVU = 8 * (D / 8);    // V transpose units: (16-key chunk, half) x d-group
    constexpr int NKC = kKT * D / 8;    // 16-byte chunks of one K tile
    constexpr int KCT = NKC / 256;      // K chunks per thread

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKT * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VROW];

    const int idx = blockIdx.x;
    const int xcd = idx % kNumXcd, slot = idx / kNumXcd;
    const int unit = (slot / p.q_tiles) * kNumXcd + xcd;
    const int qt = p.q_tiles - 1 - slot % p.q_tiles;
    if (unit >= p.n_units) return;
    const int per_seq = p.n_heads_kv * p.head_blocks;
    const int b = unit / per_seq;
    const int g = (unit % per_seq) / p.head_blocks;
    const int hb = unit % p.head_blocks;

    const int s0 = p.cu[b], s1 = p.cu[b + 1];
    if (s0 < 0 || s1 < s0 || s1 > p.total_tokens || s1 - s0 > p.max_seqlen) {
        if (threadIdx.x == 0) raise_error(p.err, kErrCuSeqlens);
        return;
    }
    const int L = s1 - s0;
    const int q0 = qt * QT;
    if (q0 >= L) return;
    const int ntiles = (min(q0 + QT, L) + kKT - 1) / kKT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int h = g * p.group + hb * NH + wave / WPH;
    const int wrow0 = q0 + (wave % WPH) * 32;   // first query row of this wave
    const int qrow = wrow0 + n;                 // this lane's query row (in-sequence)
    const bool qvalid = qrow < L;

    // Q^T operand: lane (n, hf) holds d = ks*16 + hf*8 .. +7 of query row n
    u32x4 qreg[NKS];
    {
        const uint16_t* qp = p.q + ((int64_t)(s0 + qrow) * p.n_heads_q + h) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qreg[ks] = qvalid ? *(const u32x4*)(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    // ---- tile staging: global -> registers (prefetch) -> LDS ----
    // V unit u < NVU: 16-key chunk c = (u&7)>>1, half vh = u&1, d-group dg = u>>3;
    // it loads keys 16c + 8(e/4) + 4vh + e%4 (e = 0..7) at d = 8dg..8dg+7.
    const bool v_thread = tid < NVU;
    const int vc = (tid & 7) >> 1, vh = tid & 1, vdg = tid >> 3;
    u32x4 vbuf[8];
    u32x4 kbuf[KCT];
    const int64_t kv_stride = (int64_t)p.n_heads_kv * D;
    const uint16_t* kbase = p.k + (int64_t)s0 * kv_stride + (int64_t)g * D;
    const uint16_t* vbase = p.v + (int64_t)s0 * kv_stride + (int64_t)g * D;

    auto load_tile = [&](int k0) {
        if (v_thread) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = k0 + 16 * vc + 8 * (e >> 2) + 4 * vh + (e & 3);
                vbuf[e] = key < L ? *(const u32x4*)(vbase + key * kv_stride + vdg * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < KCT; ++i) {
            const int cid = tid + 256 * i;
            const int key = k0 + cid / (D / 8), dg = cid % (D / 8);
            kbuf[i] = key < L ? *(const u32x4*)(kbase + key * kv_stride + dg * 8)
                              : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&]() {
        if (v_thread) {
            // 8x8 transpose of 16-bit values: row e = key, column dd = d
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                u32x4 t;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t a = vbuf[2 * w][dd >> 1], c = vbuf[2 * w + 1][dd >> 1];
                    t[w] = (dd & 1) ? ((a >> 16) | (c & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c << 16));
                }
                *(u32x4*)(vt_lds + (vdg * 8 + dd) * VROW + 16 * vc + 8 * vh) = t;
            }
        }
#pragma unroll
        for (int i = 0; i < KCT; ++i) {
            const int cid = tid + 256 * i;
            *(u32x4*)(k_lds + (cid / (D / 8)) * KROW + (cid % (D / 8)) * 8) = kbuf[i];
        }
    };

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kKT;
        __syncthreads();                       // previous tile fully consumed
        store_tile();
        __syncthreads();                       // tile t visible
        if (t + 1 < ntiles) load_tile(k0 + kKT);
        if (k0 > wrow0 + 31) continue;         // whole tile above this wave's diagonal

        // S^T = K Q^T for 64 keys x 32 queries
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 a = *(const u32x4*)(k_lds + (kb * 32 + n) * KROW + ks * 16 + hf * 8);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[ks]),
                                                                   sacc[kb], 0, 0, 0);
            }
        }
        // scale, causal mask (keys beyond L are above every valid row's diagonal)
        const bool need_mask = k0 + kKT - 1 > wrow0;
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = sacc[kb][i] * p.scale_log2;
                if (need_mask) {
                    const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (key > qrow) x = -INFINITY;
                }
                sacc[kb][i] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m, tmax);     // finite: key 0 is in tile 0 for every row
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        float psum = 0.f;
        uint32_t pk[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = fast_exp2(sacc[kb][i] - mnew);
                const float p1 = fast_exp2(sacc[kb][i + 1] - mnew);
                psum += p0 + p1;
                pk[kb][i >> 1] = pack_bf16x2(p0, p1);
            }
        lsum = lsum * alpha + psum;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        // O^T += V^T P^T, 16 keys per k-step
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4 pb = {pk[kb][4 * j], pk[kb][4 * j + 1], pk[kb][4 * j + 2], pk[kb][4 * j + 3]};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x4 a = *(const u32x4*)(vt_lds + (db * 32 + n) * VROW + 16 * (2 * kb + j) + 8 * hf);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), o[db], 0, 0, 0);
                }
            }
    }

    lsum += __shfl_xor(lsum, 32);
    if (!qvalid) return;
    const float inv = 1.f / lsum;
    const int64_t obase = ((int64_t)(s0 + qrow) * p.n_heads_q + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = db * 32 + 8 * i4 + 4 * hf;
            const float r0 = o[db][4 * i4] * inv, r1 = o[db][4 * i4 + 1] * inv;
            const float r2 = o[db][4 * i4 + 2] * inv, r3 = o[db][4 * i4 + 3] * inv;
            if constexpr (OUT_BF16) {
                *(u32x2*)((uint16_t*)p.out + obase + d) = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
            } else {
                *(f32x4*)((float*)p.out + obase + d) = f32x4{r0, r1, r2, r3};
            }
        }
}

template <int D, int NH, bool OUT_BF16>
hipError_t launch_variant(const PrefillParams& p, hipStream_t stream) {
    const int64_t units_padded = ((int64_t)p.n_units + kNumXcd - 1) / kNumXcd * kNumXcd;
    const int64_t blocks = units_padded * p.q_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_attn_kernel<D, NH, OUT_BF16>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, bool out_bf16,
                               hipStream_t stream) {
    const int nh = p.heads_per_block;
    if (head_dim == 128) {
        if (nh == 2) return out_bf16 ? launch_variant<128, 2, true>(p, stream) : launch_variant<128, 2, false>(p, stream);
        return out_bf16 ? launch_variant<128, 1, true>(p, stream) : launch_variant<128, 1, false>(p, stream);
    }
    if (nh == 2) return out_bf16 ? launch_variant<64, 2, true>(p, stream) : launch_variant<64, 2, false>(p, stream);
    return out_bf16 ? launch_variant<64, 1, true>(p, stream) : launch_variant<64, 1, false>(p, stream);
}

}  // namespace slm
