// Fixed-step beam-search decode attention for gfx950: one shared prompt K/V
// per request, one short suffix K/V per beam.
//
// Operation (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", §1.2: the
// beams of one request share one prompt K/V and each keeps a short suffix
// K/V; §1.1: beams carry parent indices across steps).  For beam j and query
// head h the keys are the P prompt rows of its request, the history rows of
// its parent beam and its own new row, all visible.
//
// Work decomposition: a workgroup (8 waves; 16 when the prompt's LDS copy is
// too large for two workgroups per CU) owns one (layer, request, KV head,
// chunk of query rows).  The query rows of a (layer, request, KV head)
// are the W beams x G query heads of the group, stacked in the MFMA M
// dimension (row m = beam * G + head-in-group).  The prompt K and V^T of the
// unit are staged in LDS once per workgroup and reused by every 32-row block,
// so prompt K/V bytes come from HBM once per request instead of once per beam.
// Each wave runs S^T = K Q^T and O^T += V^T P^T on the prompt (as in packed
// prefill, online softmax in registers), then folds in the beam's own suffix
// keys with vector dot products.  The workgroup also writes the suffix in the
// current beam order (parent's history rows + the new row), so the reorder
// after the previous merge costs no separate pass.
#include <map>
#include <type_traits>

#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// c + a.lo * b.lo + a.hi * b.hi over packed bf16 pairs, fp32 accumulation (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

constexpr size_t kDecSmallLds = 80 * 1024;     // two workgroups per CU fit
// fp32 output staged per wave through LDS, one 32-column half of the 32-row
// block at a time (row pitch 36 floats: the 16-byte writes of 16 lanes and
// the 16-byte reads of 16 lanes each cover all 64 banks once)
constexpr int kStageRow = 36;
constexpr size_t kStageWaveBytes = 32 * kStageRow * sizeof(float);

template <int D>
struct DecodeLds {
    static constexpr int KROW = D + 8;
    static __host__ __device__ int p_pad(int P) { return (P + 63) / 64 * 64; }
    static __host__ __device__ int vrow(int P) { return p_pad(P) + 8; }
    static __host__ __device__ size_t bytes(int P) {
        return ((size_t)p_pad(P) * KROW + (size_t)D * vrow(P)) * sizeof(uint16_t);
    }
};

// STAGE: the fp32 output leaves through a per-wave LDS tile, so each store
// instruction writes whole 128-byte row halves (eight rows) instead of 32-byte
// pieces of 32 rows.
// Occupancy: four waves per SIMD at head_dim 64 (two 8-wave workgroups, or
// one of 16 waves, per CU), two at 128.
template <int D, bool OUT_BF16, int NTHR, bool STAGE>
__global__ __launch_bounds__(NTHR, (D == 64 ? 4 : 2)) void beam_decode_attn_kernel(const DecodeParams p,
                                                                          int chunks, int chunk_rows) {
    constexpr int NKS = D / 16, NDB = D / 32, KROW = D + 8;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    static_assert(!STAGE || !OUT_BF16, "the staged epilogue writes fp32");

    const int R = p.num_requests, W = p.width, G = p.group, Hkv = p.n_heads_kv;
    const int n_units = p.n_layers * R * Hkv;
    const int idx = blockIdx.x;
    const int xcd = idx % kNumXcd, slot = idx / kNumXcd;
    const int unit = (slot / chunks) * kNumXcd + xcd;
    const int chunk = slot % chunks;
    if (unit >= n_units) return;
    const int g = unit % Hkv;
    const int lr = unit / Hkv;                    // l * R + r
    const int r = lr % R;
    const int M = W * G;
    const int row0 = chunk * chunk_rows;
    if (row0 >= M) return;
    const int row1 = min(M, row0 + chunk_rows);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int64_t kv_row = (int64_t)Hkv * D;      // elements between consecutive rows

    // This request's prompt: P rows from row prow0 of its layer's prompt block
    // (layer_rows rows per layer).  Packed prompts of different lengths come
    // with offsets; offsets that break their rules flag the error and leave
    // the request without a prompt.
    int Pr = p.prompt_len;
    int64_t prow0 = (int64_t)r * Pr, layer_rows = (int64_t)R * Pr;
    if (p.prompt_cu) {
        const int a = p.prompt_cu[r], b = p.prompt_cu[r + 1];
        layer_rows = p.prompt_rows;
        const bool ok = a >= 0 && b >= a && b <= p.prompt_rows && b - a <= p.prompt_len && (r > 0 || a == 0) &&
                        (r < R - 1 || b == p.prompt_rows);
        if (!ok && tid == 0) raise_error(p.err, kErrCuSeqlens);
        Pr = ok ? b - a : 0;
        prow0 = ok ? a : 0;
    }
    const int P = Pr;
    const int PP = DecodeLds<D>::p_pad(P);        // within the launch's LDS: P <= prompt_len
    const int VROW = DecodeLds<D>::vrow(P);
    uint16_t* k_lds = lds;                        // [PP][KROW]
    uint16_t* vt_lds = lds + (size_t)PP * KROW;   // [D][VROW], keys permuted per 16

    // ---- stage prompt K and V^T of (l, r, g) into LDS ----
    {
        const int64_t base = ((int64_t)(lr / R) * layer_rows + prow0) * kv_row + (int64_t)g * D;
        const uint16_t* pk = p.prefix_k + base;
        const uint16_t* pv = p.prefix_v + base;
        // K rows in batches of KU chunks per thread: a batch's loads all go out
        // before its LDS writes, so a batch costs one memory round trip
        constexpr int KU = 4;
        const int kchunks = PP * (D / 8);
        for (int c0 = tid; c0 < kchunks; c0 += NTHR * KU) {
            u32x4 x[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int c = c0 + u * NTHR, key = c / (D / 8), dg = c % (D / 8);
                x[u] = c < kchunks && key < P ? *(const u32x4*)(pk + key * kv_row + dg * 8) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int c = c0 + u * NTHR, key = c / (D / 8), dg = c % (D / 8);
                if (c < kchunks) *(u32x4*)(k_lds + key * KROW + dg * 8) = x[u];
            }
        }
        // V^T: unit = (16-key chunk c16, half vh, d-group dg); keys 16c16 + 8(e/4) + 4vh + e%4
        const int vunits = (PP / 16) * 2 * (D / 8);
        for (int u = tid; u < vunits; u += NTHR) {
            const int c8 = u % ((PP / 16) * 2), dg = u / ((PP / 16) * 2);
            const int c16 = c8 >> 1, vh = c8 & 1;
            u32x4 vb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = 16 * c16 + 8 * (e >> 2) + 4 * vh + (e & 3);
                vb[e] = key < P ? *(const u32x4*)(pv + key * kv_row + dg * 8) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                u32x4 t;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t a = vb[2 * w][dd >> 1], c = vb[2 * w + 1][dd >> 1];
                    t[w] = (dd & 1) ? ((a >> 16) | (c & 0xFFFF0000u)) : ((a & 0xFFFFu) | (c << 16));
                }
                *(u32x4*)(vt_lds + (dg * 8 + dd) * VROW + 16 * c16 + 8 * vh) = t;
            }
        }
    }

    // ---- suffix in the current order for the beams whose first row is here ----
    {
        const int wb0 = (row0 + G - 1) / G, wb1 = (row1 + G - 1) / G;   // beams with w*G in [row0,row1)
        const int rows_out = p.hist_len + 1;
        const int cpr = D / 8;                                          // 16-byte chunks per row
        const int total = (wb1 - wb0) * rows_out * cpr;
        // in batches of CU chunks per thread: parent indices, then the rows,
        // then the stores (two memory round trips per batch)
        constexpr int CU = 4;
        for (int c0 = tid; c0 < total; c0 += NTHR * CU) {
            int src[CU];
#pragma unroll
            for (int u = 0; u < CU; ++u) {
                const int c = c0 + u * NTHR;
                const int i = (c / cpr) % rows_out, w = wb0 + c / (cpr * rows_out);
                src[u] = c < total && i < p.hist_len && p.parent ? p.parent[r * W + w] : w;
            }
            u32x4 kx[CU], vx[CU];
#pragma unroll
            for (int u = 0; u < CU; ++u) {
                const int c = c0 + u * NTHR;
                const int part = c % cpr, i = (c / cpr) % rows_out, w = wb0 + c / (cpr * rows_out);
                kx[u] = vx[u] = u32x4{0u, 0u, 0u, 0u};
                if (c < total) {
                    const uint16_t *ks, *vs;
                    if (i < p.hist_len) {
                        if (src[u] < 0 || src[u] >= W) {
                            raise_error(p.err, kErrParent);
                            src[u] = w;
                        }
                        const int64_t so = ((((int64_t)lr * W + src[u]) * p.suffix_cap + i) * Hkv + g) * D + part * 8;
                        ks = p.suffix_k_in + so;
                        vs = p.suffix_v_in + so;
                    } else {
                        const int64_t so = (((int64_t)lr * W + w) * Hkv + g) * D + part * 8;
                        ks = p.k_new + so;
                        vs = p.v_new + so;
                    }
                    kx[u] = *(const u32x4*)ks;
                    vx[u] = *(const u32x4*)vs;
                }
            }
#pragma unroll
            for (int u = 0; u < CU; ++u) {
                const int c = c0 + u * NTHR;
                const int part = c % cpr, i = (c / cpr) % rows_out, w = wb0 + c / (cpr * rows_out);
                if (c < total) {
                    const int64_t dst = ((((int64_t)lr * W + w) * p.suffix_cap + i) * Hkv + g) * D + part * 8;
                    *(u32x4*)(p.suffix_k_out + dst) = kx[u];
                    *(u32x4*)(p.suffix_v_out + dst) = vx[u];
                }
            }
        }
    }
    __syncthreads();

    const float c = p.scale_log2;
    for (int blk = row0 + wave * 32; blk < row1; blk += 32 * (NTHR / kWave)) {
        const int m = blk + n;                    // this lane's query row
        const bool valid = m < row1;
        const int w = valid ? m / G : 0;
        const int hh = valid ? m % G : 0;
        const int h = g * G + hh;
        const int64_t qoff = (((int64_t)lr * W + w) * p.n_heads_q + h) * D;

        u32x4 qreg[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qreg[ks] = valid ? *(const u32x4*)(p.q + qoff + ks * 16 + hf * 8) : u32x4{0u, 0u, 0u, 0u};
        // the beam's history rows are its parent's (read now, used after the prompt)
        int src = w;
        if (p.parent && p.hist_len > 0) src = p.parent[r * W + w];

        f32x16 o[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        float mrun = -INFINITY, lsum = 0.f;

        // ---- prompt keys, 64 at a time ----
        // Running max in raw score units with the scale folded into exp2; the
        // reference max may trail the true one by up to kMaxLag (log2 units),
        // so O and the row sum are rescaled only when some row's max moves
        // further (after the first chunk almost never).  Only the last chunk
        // of a prompt whose length is not a multiple of 64 masks keys >= P.
        auto chunk = [&](int k0, auto masked) {
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const u32x4 a = *(const u32x4*)(k_lds + (k0 + kb * 32 + n) * KROW + ks * 16 + hf * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[ks]),
                                                                       sacc[kb], 0, 0, 0);
                }
            }
            if constexpr (decltype(masked)::value) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (k0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3) >= P) sacc[kb][i] = -INFINITY;
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
            tmax = max_halves(tmax);
            const float mnew = fmaxf(mrun, tmax);  // finite: every chunk holds a prompt key
            if (__ballot((mnew - mrun) * c > kMaxLag) != 0) {   // mrun = -inf on the first chunk: taken
                const float alpha = fast_exp2((mrun - mnew) * c);
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                mrun = mnew;
            }
            const float mc = mrun * c;
            float psum = 0.f;
            uint32_t pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = fast_exp2(fmaf(sacc[kb][i], c, -mc));
                    const float p1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -mc));
                    psum += p0 + p1;
                    pk[kb][i >> 1] = pack_bf16x2(p0, p1);
                }
            lsum += psum;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4 pb = {pk[kb][4 * j], pk[kb][4 * j + 1], pk[kb][4 * j + 2], pk[kb][4 * j + 3]};
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const u32x4 a = *(const u32x4*)(vt_lds + (db * 32 + n) * VROW + k0 + 16 * (2 * kb + j) + 8 * hf);
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), o[db], 0, 0, 0);
                    }
                }
        };
        const int nfull = P / 64;
        for (int kc = 0; kc < nfull; ++kc) chunk(kc * 64, std::false_type{});
        if (P % 64 != 0) chunk(nfull * 64, std::true_type{});
        mrun *= c;                                // scaled (log2) units from here on

        // ---- the beam's own suffix: parent's history rows, then the new row ----
        if (src < 0 || src >= W) src = w;         // flagged by the suffix copy above
        const int ns = p.hist_len + 1;
        // One row at a time with the online update; a row's K and V halves
        // are loaded together, so each row costs one memory round trip,
        // and the dot products take the bf16 pairs as they are (v_dot2).
#pragma unroll 1
        for (int i = 0; i < ns; ++i) {
            const bool hist = i < p.hist_len;
            const int64_t ro = hist ? ((((int64_t)lr * W + src) * p.suffix_cap + i) * Hkv + g) * D
                                    : (((int64_t)lr * W + w) * Hkv + g) * D;
            const uint16_t* kr = (hist ? p.suffix_k_in : p.k_new) + ro;
            const uint16_t* vr = (hist ? p.suffix_v_in : p.v_new) + ro;
            u32x4 kv[NKS];
            u32x2 vv[NDB * 4];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) kv[ks] = *(const u32x4*)(kr + ks * 16 + hf * 8);
#pragma unroll
            for (int j = 0; j < NDB * 4; ++j) vv[j] = *(const u32x2*)(vr + (j >> 2) * 32 + 8 * (j & 3) + 4 * hf);
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) part = dot2_bf16(qreg[ks][e], kv[ks][e], part);
            part = sum_halves(part);
            const float s = part * p.scale_log2;
            // as in the prompt pass: the reference max may trail by up to
            // kMaxLag, so O and the row sum are rescaled only when a row's
            // score moves further (weights stay below 2^kMaxLag)
            if (__ballot(s - mrun > kMaxLag) != 0) {
                const float mnew = fmaxf(mrun, s);  // finite: s is
                const float alpha = fast_exp2(mrun - mnew);
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                mrun = mnew;
            }
            const float pi = fast_exp2(s - mrun);
            lsum += hf == 0 ? pi : 0.f;             // both halves hold the same score
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const u32x2 x = vv[db * 4 + i4];
                    o[db][4 * i4 + 0] = fmaf(pi, bf16_bits_to_f32(x[0] & 0xFFFFu), o[db][4 * i4 + 0]);
                    o[db][4 * i4 + 1] = fmaf(pi, bf16_bits_to_f32(x[0] >> 16), o[db][4 * i4 + 1]);
                    o[db][4 * i4 + 2] = fmaf(pi, bf16_bits_to_f32(x[1] & 0xFFFFu), o[db][4 * i4 + 2]);
                    o[db][4 * i4 + 3] = fmaf(pi, bf16_bits_to_f32(x[1] >> 16), o[db][4 * i4 + 3]);
                }
        }

        lsum = sum_halves(lsum);
        if constexpr (STAGE) {
            // tile [32 rows][kStageRow] floats behind the prompt copy, one per wave
            float* st = (float*)(vt_lds + (size_t)D * VROW) + (size_t)wave * 32 * kStageRow;
            const float inv = valid ? 1.f / lsum : 0.f;
            const int c = lane >> 3, rr = lane & 7;   // read side: 16-byte chunk c of row 8k + rr
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    *(f32x4*)(st + n * kStageRow + 8 * i4 + 4 * hf) =
                        f32x4{o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv, o[db][4 * i4 + 2] * inv,
                              o[db][4 * i4 + 3] * inv};
                __builtin_amdgcn_wave_barrier();      // LDS is in order within a wave
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int row = 8 * k + rr, m2 = blk + row;
                    const f32x4 x = *(const f32x4*)(st + row * kStageRow + 4 * c);
                    if (m2 < row1) {
                        const int64_t qo2 = (((int64_t)lr * W + m2 / G) * p.n_heads_q + g * G + m2 % G) * D;
                        __builtin_nontemporal_store(x, (f32x4*)((float*)p.out + qo2 + db * 32 + 4 * c));
                    }
                }
                __builtin_amdgcn_wave_barrier();      // reads of this half before the next half's writes
            }
        } else if (valid) {
            const float inv = 1.f / lsum;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int d = db * 32 + 8 * i4 + 4 * hf;
                    const float r0 = o[db][4 * i4] * inv, r1 = o[db][4 * i4 + 1] * inv;
                    const float r2 = o[db][4 * i4 + 2] * inv, r3 = o[db][4 * i4 + 3] * inv;
                    if constexpr (OUT_BF16) {
                        *(u32x2*)((uint16_t*)p.out + qoff + d) = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
                    } else {
                        // ordinary stores: these 32-byte pieces of 32 rows
                        // with the non-temporal hint took the 8-wave form from
                        // ~130 to ~310 us at prompts of 136-256 rows (the
                        // 16-wave form measured the same either way)
                        *(f32x4*)((float*)p.out + qoff + d) = f32x4{r0, r1, r2, r3};
                    }
                }
        }
    }
}

// Rows of a (layer, request, KV head) unit are split over `chunks`
// workgroups of whole 32-row blocks.  Cost model: the launch runs in
// ceil(workgroups / resident) rounds, and a round lasts as long as its
// busiest wave's blocks plus the prompt staging (taken as half a block);
// the split with the least cost wins, the fewest chunks on ties.
int decode_chunks(int64_t units, int blocks32, int waves, int64_t resident) {
    int best = 1;
    int64_t best_cost = INT64_MAX;
    for (int c = 1; c <= blocks32; ++c) {
        const int per_wg = (blocks32 + c - 1) / c;
        const int per_wave = (per_wg + waves - 1) / waves;
        const int64_t rounds = (units * c + resident - 1) / resident;
        const int64_t cost = rounds * (2 * per_wave + 1);
        if (cost < best_cost) {
            best = c;
            best_cost = cost;
        }
        if (per_wave == 1) break;                 // more chunks only add staging
    }
    return best;
}

template <int D, bool OUT_BF16, int NTHR, bool STAGE>
hipError_t launch_variant(const DecodeParams& p, int num_cus, LaunchCache& cache, hipStream_t stream) {
    const int n_units = p.n_layers * p.num_requests * p.n_heads_kv;
    const int M = p.width * p.group;
    const int blocks32 = (M + 31) / 32;
    const int64_t units_padded = ((int64_t)n_units + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (units_padded == 0 || blocks32 == 0) return hipSuccess;
    const size_t lds = DecodeLds<D>::bytes(p.prompt_len) + (STAGE ? (NTHR / kWave) * kStageWaveBytes : 0);
    auto kern = beam_decode_attn_kernel<D, OUT_BF16, NTHR, STAGE>;
    // raise the kernel's dynamic-LDS limit only when a call needs more than
    // before, and query the workgroups per CU once per LDS size (no host call
    // per launch, so launches can be graph-captured); the context's cache
    // records both for its device
    const int variant = (D == 128) * 8 + OUT_BF16 * 4 + (NTHR == 1024) * 2 + STAGE;
    size_t& lds_limit = cache.decode_lds_limit[variant];
    if (lds > lds_limit) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_limit = lds;
    }
    auto it = cache.decode_occ.find({variant, lds});
    if (it == cache.decode_occ.end()) {
        int n = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)kern, NTHR, lds);
        if (e != hipSuccess) return e;
        it = cache.decode_occ.emplace(std::make_pair(variant, lds), max(1, n)).first;
    }
    const int per_cu = it->second;
    int chunks = decode_chunks(units_padded, blocks32, NTHR / kWave, (int64_t)num_cus * per_cu);
    const int chunk_rows = (blocks32 + chunks - 1) / chunks * 32;
    chunks = (M + chunk_rows - 1) / chunk_rows;
    const int64_t blocks = units_padded * chunks;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NTHR), lds, stream, p, chunks, chunk_rows);
    return hipGetLastError();
}

}  // namespace

size_t beam_decode_lds_bytes(int head_dim, int prompt_len) {
    return head_dim == 128 ? DecodeLds<128>::bytes(prompt_len) : DecodeLds<64>::bytes(prompt_len);
}

hipError_t launch_beam_decode_attn(const DecodeParams& p, int head_dim, bool out_bf16, int num_cus,
                                   LaunchCache& cache, hipStream_t stream) {
    // A prompt copy too large for two workgroups per CU is shared by 16 waves
    // (head_dim 64; at 128 the registers of 16 waves would not hold a lane's state).
    // The fp32 output is staged through LDS where the tiles still leave room
    // for two workgroups per CU.
    const size_t prompt_lds = beam_decode_lds_bytes(head_dim, p.prompt_len);
    const bool wide = head_dim == 64 && prompt_lds > kDecSmallLds;
    const bool stage = head_dim == 64 && !out_bf16 && prompt_lds + 8 * kStageWaveBytes <= kDecSmallLds;
    if (head_dim == 128)
        return out_bf16 ? launch_variant<128, true, 512, false>(p, num_cus, cache, stream)
                        : launch_variant<128, false, 512, false>(p, num_cus, cache, stream);
    if (out_bf16)
        return wide ? launch_variant<64, true, 1024, false>(p, num_cus, cache, stream)
                    : launch_variant<64, true, 512, false>(p, num_cus, cache, stream);
    if (stage) return launch_variant<64, false, 512, true>(p, num_cus, cache, stream);
    return wide ? launch_variant<64, false, 1024, false>(p, num_cus, cache, stream)
                : launch_variant<64, false, 512, false>(p, num_cus, cache, stream);
}

}  // namespace slm
