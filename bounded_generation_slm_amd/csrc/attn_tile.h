// 32-key attention tiles for gfx950, shared by packed prefill and beam decode.
//
// A tile holds 32 keys of K and V in LDS (K rows with their 16-byte chunks
// XOR-swizzled by row, V rows swizzled for transposed reads).  A wave owns 32
// query rows and computes, per tile,
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, K from LDS, Q^T in VGPRs)
//   O^T += V^T P^T
// with the online softmax in registers.  Computing S transposed puts each
// lane on one query column, so the row max and sum are in-lane plus one
// cross-half exchange, and the accumulator layout of S^T is exactly the
// B-operand layout P^T needs.  V^T comes from ds_read_b64_tr_b16.
#pragma once
#include "common.h"

namespace slm {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kKT = 32;                 // keys per K/V tile
constexpr int kStages = 3;              // LDS ring depth (two tiles in flight)
constexpr float kMaxLag = 8.f;          // how far (log2 units) the softmax reference max may trail

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at "no wait")
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// s_waitcnt with only an lgkmcnt limit
template <int N>
__device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (N << 8) | (0x3 << 14));
}
__device__ __forceinline__ void wait_lgkm0() { wait_lgkm<0>(); }
// Registers filled by the inline-asm loads below are invisible to the
// compiler's dependency tracking: it may move their (side-effect free)
// consumers such as MFMAs above the wait that guards them.  Passing each such
// register through an empty volatile asm after the wait pins the order.
template <class T>
__device__ __forceinline__ void pin_after_wait(T& x) {
    asm volatile("" : "+v"(x));
}

// Memory operations issued directly: the compiler neither tracks nor waits
// for them, so every use is preceded by an explicit wait.  (The compiler would
// otherwise wait for all in-flight direct-to-LDS loads before each LDS access
// it cannot disambiguate, draining the tile pipeline.)
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}
__device__ __forceinline__ void lds_write16(uint32_t addr, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}
__device__ __forceinline__ u32x4 global_load16(const void* p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

template <int D>
struct Geo {
    static constexpr int NKS = D / 16;          // k-steps of S^T over the head dim
    static constexpr int NDB = D / 32;          // 32-row blocks of O^T
    static constexpr int ROWB = D * 2;          // bytes of one K/V row in LDS
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int TILEB = kKT * ROWB;    // bytes of one K (or V) tile
    static constexpr int STAGEB = 2 * TILEB;    // K tile then V tile
    static constexpr int LPW = TILEB / 1024 / 4;    // direct loads per wave per K (or V) tile
    static_assert(LPW >= 1, "tile too small for 4 waves");
};

// Per-lane offsets that do not depend on the work unit.
template <int D>
struct LaneConst {
    int koff[Geo<D>::NKS];                      // K operand, per k-step
    uint32_t voff[Geo<D>::NDB];                 // V^T transpose reads (k-step 0, first read)
    int dma_r[Geo<D>::LPW], dma_ck[Geo<D>::LPW], dma_cv[Geo<D>::LPW];
};

// K row r keeps its 16-byte chunk c at position c ^ (r % CPR); V row r keeps
// chunk c at position c ^ (2 * (r % 4)), so transpose reads of four
// consecutive rows hit distinct banks.
template <int D>
__device__ __forceinline__ void make_lane_const(LaneConst<D>& lc, int lane, int wave, uint32_t ring_base) {
    using G = Geo<D>;
    const int n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) lc.koff[ks] = ring_base + n * G::ROWB + (((2 * ks + hf) ^ (n % G::CPR)) * 16);
    // V^T operand of k-step j, d-block db: in each 16-lane group, lane r
    // points at 4 d's of key ka (first read) or ka + 8 (second read) and
    // receives its own d column of four keys.  Those keys are 16j + 8(e/4) +
    // 4hf + e%4, the keys the P^T operand of the same k-step holds.  The
    // swizzle term depends on ka % 4 only, which neither j (16 keys) nor the
    // second read (8 keys) changes, so those steps are constant offsets.
    const int grp = lane >> 4, r = lane & 15;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        const int dcol = db * 32 + 16 * (grp & 1) + 4 * (r & 3);
        const int chunk = dcol / 8, within = (dcol % 8) * 2;
        const int ka = 4 * (grp >> 1) + (r >> 2);
        lc.voff[db] = ring_base + G::TILEB + ka * G::ROWB + ((chunk ^ (2 * (ka & 3))) * 16) + within;
    }
#pragma unroll
    for (int i = 0; i < G::LPW; ++i) {
        const int byte = (wave * G::LPW + i) * 1024 + lane * 16;
        lc.dma_r[i] = byte / G::ROWB;
        const int pos = (byte % G::ROWB) / 16;
        lc.dma_ck[i] = (pos ^ (lc.dma_r[i] % G::CPR)) * 8;
        lc.dma_cv[i] = (pos ^ (2 * (lc.dma_r[i] & 3))) * 8;
    }
}

// Direct loads of one tile into stage STAGE: each wave writes LPW contiguous
// KiB of K and of V (2 * LPW vector-memory instructions).  Rows past the
// sequence re-read its last row (finite values; every such key is masked).
template <int D, int STAGE>
__device__ __forceinline__ void issue_tile(char* ring, const LaneConst<D>& lc, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t kv_stride, int k0, int L, int wave) {
    using G = Geo<D>;
#pragma unroll
    for (int i = 0; i < G::LPW; ++i) {
        const int64_t row = (int64_t)min(k0 + lc.dma_r[i], L - 1) * kv_stride;
        char* kdst = ring + STAGE * G::STAGEB + (wave * G::LPW + i) * 1024;
        __builtin_amdgcn_global_load_lds((glb_void*)(kbase + row + lc.dma_ck[i]), (lds_void*)kdst, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(vbase + row + lc.dma_cv[i]), (lds_void*)(kdst + G::TILEB), 16, 0, 0);
    }
}

// One 32-key tile: S^T = K Q^T, online softmax (running max m in raw score
// units, scale folded into exp2), O^T += V^T P^T.  The tile sits at LDS
// address tbase + STAGE * STAGEB (relative to the lane constants' base).  When
// MASK and apply, key kk of the tile (0..31) is left out where kk > lim (the
// causal limit of the lane's query row, relative to the tile's first key).
// The first tile a row sees must hold one of its keys (its running max then
// becomes finite).
template <int D, int STAGE, bool MASK>
__device__ __forceinline__ void attend_tile(const LaneConst<D>& lc, uint32_t tbase,
                                            const u32x4 (&qreg)[Geo<D>::NKS], int hf, float c, float& m,
                                            float& lsum, f32x16 (&o)[Geo<D>::NDB], bool apply, int lim) {
    using G = Geo<D>;
    constexpr int H = G::NKS / 2;
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    u32x4 ka[G::NKS];                           // K operand rows, read in two halves
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) ka[ks] = lds_read16_at<STAGE * G::STAGEB>(lc.koff[ks] + tbase);
    wait_lgkm<H>();
#pragma unroll
    for (int ks = 0; ks < H; ++ks) {
        pin_after_wait(ka[ks]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks]), as_bf16x8(qreg[ks]), sacc, 0, 0, 0);
    }
    wait_lgkm0();
#pragma unroll
    for (int ks = H; ks < G::NKS; ++ks) {
        pin_after_wait(ka[ks]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks]), as_bf16x8(qreg[ks]), sacc, 0, 0, 0);
    }
    u32x2 vop[G::NDB][2];                       // V^T operands of k-step 0, read while the softmax runs
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        vop[db][0] = lds_read_tr16<STAGE * G::STAGEB>(lc.voff[db] + tbase);
        vop[db][1] = lds_read_tr16<STAGE * G::STAGEB + 8 * G::ROWB>(lc.voff[db] + tbase);
    }
    if (MASK && apply) {                        // element i holds key 8 (i / 4) + 4 hf + i % 4
        const int lh = lim - 4 * hf;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + (i & 3) > lh) sacc[i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[i]);
    tmax = max_halves(tmax);
    // The reference max m may trail the true running max by up to kMaxLag in
    // exponent units: every weight exp2((s - m) c) then stays below 2^kMaxLag,
    // and O and the row sum carry one common factor that the final division
    // removes.  So O is rescaled only when some row's max moved further than
    // that, which after the first tile is rare.
    const float mnew = fmaxf(m, tmax);          // finite: key 0 is in tile 0 for every row
    if (__ballot((mnew - m) * c > kMaxLag) != 0) {   // m = -inf on the first tile: always taken
        const float alpha = fast_exp2((m - mnew) * c);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
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
    wait_lgkm0();                               // the transpose reads have landed
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        pin_after_wait(vop[db][0]);
        pin_after_wait(vop[db][1]);
    }
    {
        const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            const u32x4 a = {vop[db][0][0], vop[db][0][1], vop[db][1][0], vop[db][1][1]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), o[db], 0, 0, 0);
            vop[db][0] = lds_read_tr16<STAGE * G::STAGEB + 16 * G::ROWB>(lc.voff[db] + tbase);   // k-step 1
            vop[db][1] = lds_read_tr16<STAGE * G::STAGEB + 24 * G::ROWB>(lc.voff[db] + tbase);
        }
    }
    wait_lgkm0();
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        pin_after_wait(vop[db][0]);
        pin_after_wait(vop[db][1]);
    }
    {
        const u32x4 pb = {pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            const u32x4 a = {vop[db][0][0], vop[db][0][1], vop[db][1][0], vop[db][1][1]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), o[db], 0, 0, 0);
        }
    }
}

}  // namespace slm
