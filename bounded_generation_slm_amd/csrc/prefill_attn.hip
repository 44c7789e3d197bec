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
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, K from LDS, Q^T in VGPRs)
//   O^T += V^T P^T
// Computing S transposed puts each lane on one query column, so the row max
// and row sum are in-lane plus one cross-half exchange, and the accumulator
// layout of S^T is exactly the B-operand layout P^T needs: no shuffle of P.
//
// K/V staging: 32-key tiles go from HBM straight into a 3-stage LDS ring with
// global_load_lds_dwordx4 (no register staging), two tiles ahead of the
// compute, one workgroup barrier per tile.  K rows are stored with their
// 16-byte chunks XOR-swizzled by row so the K operand reads are conflict-free.
// V stays row-major; its V^T operand comes from ds_read_b64_tr_b16, whose
// 16-lane transpose hands each lane one d column of four keys.
//
// Grid mapping is XCD-aware: the query tiles of one (sequence, head block)
// are consecutive on one XCD (blockIdx % 8), so the K/V rows they share are
// fetched from HBM once and re-read from that XCD's L2.  Heavier tiles (later
// query tiles, which see more keys) are dispatched first within a unit.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kKT = 32;                 // keys per K/V tile
constexpr int kStages = 3;              // LDS ring depth (two tiles in flight)

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at "no wait")
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

// ds_read_b64_tr_b16 issued directly, with a compile-time byte offset: the
// compiler neither tracks nor waits for it, so the caller waits with
// wait_lgkm0() before using the result.  (Through the builtin, the compiler
// would also wait for every in-flight direct-to-LDS load of later tiles.)
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}

template <int D, int NH, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(const PrefillParams p) {
    constexpr int QT = 128 / NH;        // query rows per workgroup
    constexpr int WPH = 4 / NH;         // waves per query head
    constexpr int NKS = D / 16;         // k-steps of S^T over the head dim
    constexpr int NDB = D / 32;         // 32-row blocks of O^T
    constexpr int ROWB = D * 2;         // bytes of one K/V row in LDS
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int TILEB = kKT * ROWB;   // bytes of one K (or V) tile
    constexpr int STAGEB = 2 * TILEB;   // K tile then V tile
    constexpr int LPW = TILEB / 1024 / 4;   // direct loads per wave per K (or V) tile
    static_assert(LPW >= 1, "tile too small for 4 waves");

    __shared__ __attribute__((aligned(1024))) char lds[kStages * STAGEB];

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
    const int last_tile = min(wrow0 + 31, L - 1) / kKT;   // last tile with a visible key
    const float c = p.scale_log2;

    // Q^T operand: lane (n, hf) holds d = ks*16 + hf*8 .. +7 of query row n
    u32x4 qreg[NKS];
    {
        const uint16_t* qp = p.q + ((int64_t)(s0 + min(qrow, L - 1)) * p.n_heads_q + h) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qreg[ks] = *(const u32x4*)(qp + ks * 16);
    }

    // Per-lane LDS byte offsets inside one stage.  K row r keeps its 16-byte
    // chunk c at position c ^ (r % CPR); V row r keeps chunk c at position
    // c ^ (2 * (r % 4)), so transpose reads of four consecutive rows hit
    // distinct banks.
    int koff[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = n * ROWB + (((2 * ks + hf) ^ (n % CPR)) * 16);
    // V^T operand of k-step j, d-block db: in each 16-lane group, lane r
    // points at 4 d's of key ka (first read) or ka + 8 (second read) and
    // receives its own d column of four keys.  Those keys are 16j + 8(e/4) +
    // 4hf + e%4, the keys the P^T operand of the same k-step holds.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    uint32_t voff[2][NDB][2];
    {
        const int grp = lane >> 4, r = lane & 15;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int dcol = db * 32 + 16 * (grp & 1) + 4 * (r & 3);
                const int chunk = dcol / 8, within = (dcol % 8) * 2;
                const int ka = 16 * j + 4 * (grp >> 1) + (r >> 2), kb2 = ka + 8;
                voff[j][db][0] = lds_base + TILEB + ka * ROWB + ((chunk ^ (2 * (ka & 3))) * 16) + within;
                voff[j][db][1] = lds_base + TILEB + kb2 * ROWB + ((chunk ^ (2 * (kb2 & 3))) * 16) + within;
            }
    }
    // Direct loads of one tile: each wave writes LPW contiguous KiB of K and of
    // V.  Rows past the sequence re-read its last row (finite values; every
    // such key is masked).
    const int64_t kv_stride = (int64_t)p.n_heads_kv * D;
    const uint16_t* kbase = p.k + (int64_t)s0 * kv_stride + (int64_t)g * D;
    const uint16_t* vbase = p.v + (int64_t)s0 * kv_stride + (int64_t)g * D;
    int dma_r[LPW], dma_ck[LPW], dma_cv[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int byte = (wave * LPW + i) * 1024 + lane * 16;
        dma_r[i] = byte / ROWB;
        const int pos = (byte % ROWB) / 16;
        dma_ck[i] = (pos ^ (dma_r[i] % CPR)) * 8;
        dma_cv[i] = (pos ^ (2 * (dma_r[i] & 3))) * 8;
    }
    auto issue_tile = [&](int t, auto stage_c) {
        constexpr int stage = decltype(stage_c)::value;
        const int k0 = t * kKT;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int64_t row = (int64_t)min(k0 + dma_r[i], L - 1) * kv_stride;
            char* kdst = lds + stage * STAGEB + (wave * LPW + i) * 1024;
            __builtin_amdgcn_global_load_lds((glb_void*)(kbase + row + dma_ck[i]), (lds_void*)kdst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glb_void*)(vbase + row + dma_cv[i]), (lds_void*)(kdst + TILEB), 16, 0, 0);
        }
    };

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m = -INFINITY, lsum = 0.f;            // running max in raw (unscaled) score units

    // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
    auto compute = [&](int k0, auto stage_c, auto mask_c) {
        constexpr int stage = decltype(stage_c)::value;
        constexpr bool MASK = decltype(mask_c)::value;
        const char* kt = lds + stage * STAGEB;
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const u32x4 a = *(const u32x4*)(kt + koff[ks]);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[ks]), sacc, 0, 0, 0);
        }
        u32x2 vop[2][NDB][2];                   // V^T operands, read while the softmax runs
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                vop[j][db][0] = lds_read_tr16<stage * STAGEB>(voff[j][db][0]);
                vop[j][db][1] = lds_read_tr16<stage * STAGEB>(voff[j][db][1]);
            }
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (MASK && k0 + 8 * (i >> 2) + 4 * hf + (i & 3) > qrow) sacc[i] = -INFINITY;
            tmax = fmaxf(tmax, sacc[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m, tmax);      // finite: key 0 is in tile 0 for every row
        if (__ballot(mnew > m) != 0) {          // rescale only when some running max moved
            const float alpha = fast_exp2((m - mnew) * c);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            m = mnew;
        }
        const float mc = m * c;
        float psum = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = fast_exp2(fmaf(sacc[i], c, -mc)), p1 = fast_exp2(fmaf(sacc[i + 1], c, -mc));
            psum += p0 + p1;
            pk[i >> 1] = pack_bf16x2(p0, p1);
        }
        lsum += psum;
        wait_lgkm0();                           // the transpose reads have landed
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 pb = {pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x4 a = {vop[j][db][0][0], vop[j][db][0][1], vop[j][db][1][0], vop[j][db][1][1]};
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), o[db], 0, 0, 0);
            }
        }
    };
    auto tile = [&](int t, auto stage_c) {
        constexpr int stage = decltype(stage_c)::value;
        wait_vmcnt<2 * LPW>();                  // this wave's loads of tile t have landed
        __builtin_amdgcn_s_barrier();           // ... and every wave's; tile t-1 is consumed
        issue_tile(t + 2, std::integral_constant<int, (stage + 2) % kStages>{});
        if (t > last_tile) return;              // whole tile above this wave's diagonal
        const int k0 = t * kKT;
        if (k0 + kKT - 1 > wrow0)
            compute(k0, stage_c, std::true_type{});
        else
            compute(k0, stage_c, std::false_type{});
    };

    issue_tile(0, std::integral_constant<int, 0>{});
    issue_tile(1, std::integral_constant<int, 1>{});   // past the last tile it re-reads valid rows
    for (int t = 0; t < ntiles; t += kStages) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 >= ntiles) break;
        tile(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 >= ntiles) break;
        tile(t + 2, std::integral_constant<int, 2>{});
    }

    wait_vmcnt<0>();                            // the tiles issued past the end must land
    lsum += __shfl_xor(lsum, 32);
    const float inv = 1.f / lsum;

    // Epilogue through LDS: each wave writes its 32 x D block (row-major,
    // rows padded by 16 bytes) into the freed ring, then reads it back so
    // that every store instruction writes whole contiguous row segments.
    // Done in passes of 64 columns so the four waves fit the ring.
    constexpr int OB = OUT_BF16 ? 2 : 4;        // output bytes per element
    constexpr int PCOLS = D == 64 ? 32 : 64;    // columns per pass
    constexpr int PROWB = PCOLS * OB + 16;      // padded LDS row bytes
    constexpr int WAVEB = 32 * PROWB;           // LDS bytes per wave per pass
    static_assert(4 * WAVEB <= kStages * STAGEB, "epilogue staging must fit the ring");
    constexpr int CH = PCOLS * OB / 16;         // 16-byte chunks per row segment
    __builtin_amdgcn_s_barrier();               // every wave is done with the ring
    char* wbuf = lds + wave * WAVEB;
    const int64_t orow0 = (int64_t)(s0 + wrow0) * p.n_heads_q + h;   // output row of this wave's row 0
#pragma unroll
    for (int pass = 0; pass < D / PCOLS; ++pass) {
#pragma unroll
        for (int dbp = 0; dbp < PCOLS / 32; ++dbp) {
            const int db = pass * (PCOLS / 32) + dbp;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int col = dbp * 32 + 8 * i4 + 4 * hf;
                const float r0 = o[db][4 * i4] * inv, r1 = o[db][4 * i4 + 1] * inv;
                const float r2 = o[db][4 * i4 + 2] * inv, r3 = o[db][4 * i4 + 3] * inv;
                if constexpr (OUT_BF16)
                    *(u32x2*)(wbuf + n * PROWB + col * OB) = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
                else
                    *(f32x4*)(wbuf + n * PROWB + col * OB) = f32x4{r0, r1, r2, r3};
            }
        }
        __builtin_amdgcn_wave_barrier();        // the wave reads back what its lanes wrote
#pragma unroll
        for (int k = 0; k < 32 * CH / 64; ++k) {
            const int chunk = k * 64 + lane;
            const int row = chunk / CH, c16 = chunk % CH;
            const u32x4 v = *(const u32x4*)(wbuf + row * PROWB + c16 * 16);
            if (wrow0 + row < L)
                *(u32x4*)((char*)p.out + ((orow0 + (int64_t)row * p.n_heads_q) * D + pass * PCOLS) * OB + c16 * 16) = v;
        }
        __builtin_amdgcn_wave_barrier();        // before the next pass overwrites the buffer
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
