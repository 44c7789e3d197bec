// Packed causal GQA prefill attention for gfx950.
//
// Operation (page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化", abstract
// "Packed Prefill" and §1.2): sequences are packed back to back with no
// padding; each query attends causally to the keys of its own sequence only.
//
// Work unit: one (sequence, KV head, block of query heads of that group,
// query tile), processed by a workgroup of 4 waves.  The query heads of one
// GQA group share every K/V tile staged in LDS.  Each wave owns 32 query rows
// of one head and runs the online softmax in registers:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, K from LDS, Q^T in VGPRs)
//   O^T += V^T P^T
// Computing S transposed puts each lane on one query column, so the row max
// and row sum are in-lane plus one cross-half exchange, and the accumulator
// layout of S^T is exactly the B-operand layout P^T needs: no shuffle of P.
//
// K/V staging: 32-key tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging).  K rows are stored with
// their 16-byte chunks XOR-swizzled by row so the K operand reads are
// conflict-free.  V stays row-major; its V^T operand comes from
// ds_read_b64_tr_b16, whose 16-lane transpose hands each lane one d column of
// four keys.
//
// Two launch forms share the per-tile code:
//   * one workgroup per work unit (small packs), XCD-aware block order with
//     the heaviest query tiles of all units first, a 3-stage ring two tiles
//     ahead of the compute, one barrier per tile;
//   * for large packs, a plan kernel lists the non-empty work units per XCD
//     (the units of one (sequence, head block) on one XCD so they share its
//     L2, heavier query tiles first), and persistent workgroups walk their
//     XCD's list as one continuous K/V stream of 64-key steps (two tiles per
//     barrier, a four-tile ring used as two halves): the next unit's first
//     tiles are in flight while the current unit finishes, and each unit's
//     output leaves through unconditional buffer stores.  The list depends
//     only on cu_seqlens and the sizes, so it can be built once per pack and
//     run by every layer (the plan and run phases); each run's last
//     workgroup per XCD leaves the list's counters as the plan left them.
#include <type_traits>

#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace slm {
namespace {

// A wave-uniform 16-byte entry through the scalar cache, waited for at once.
__device__ __forceinline__ int4 scalar_load16(const int4* p) {
    int4 r;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
    return r;
}
__device__ __forceinline__ int scalar_load4(const int* p) {
    int r;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
    return r;
}
// Epilogue geometry: each wave stages its 32 x D block through LDS in passes
// of PCOLS columns (rows padded by 16 bytes), then stores whole contiguous
// row segments, of 128 bytes (one cache line: 32 fp32 or 64 bf16 columns)
// except for bf16 at D = 64, whose 64-column staging would no longer fit the
// persistent ring's free half.  (bf16 staged 32 columns at a time at D = 128
// left half lines, which the non-temporal stores wrote 5% slower.)
template <int D, bool OUT_BF16>
struct Epi {
    static constexpr int OB = OUT_BF16 ? 2 : 4;             // output bytes per element
    static constexpr int PCOLS = (OUT_BF16 && D == 64) ? 32 : 128 / OB;   // columns per pass
    static constexpr int PROWB = PCOLS * OB + 16;           // padded LDS row bytes
    static constexpr int WAVEB = 32 * PROWB;                // LDS bytes per wave
    static constexpr int CH = PCOLS * OB / 16;              // 16-byte chunks per row segment
    static constexpr int NPASS = D / PCOLS;
    static constexpr int SPP = 32 * CH / 64;                // stores per lane per pass
    static constexpr int NST = NPASS * SPP;                 // stores per lane per unit
};

// Normalised rows of one wave into its LDS staging block (pass `pass`).
template <int D, bool OUT_BF16>
__device__ __forceinline__ void epi_stage(uint32_t wbuf, const f32x16 (&o)[Geo<D>::NDB], float inv, int pass,
                                          int n, int hf) {
    using E = Epi<D, OUT_BF16>;
#pragma unroll
    for (int dbp = 0; dbp < E::PCOLS / 32; ++dbp) {
        const int db = pass * (E::PCOLS / 32) + dbp;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int col = dbp * 32 + 8 * i4 + 4 * hf;
            const float r0 = o[db][4 * i4] * inv, r1 = o[db][4 * i4 + 1] * inv;
            const float r2 = o[db][4 * i4 + 2] * inv, r3 = o[db][4 * i4 + 3] * inv;
            const uint32_t a = wbuf + n * E::PROWB + col * E::OB;
            if constexpr (OUT_BF16) {
                const u32x2 v = {pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
                asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
            } else {
                lds_write16(a, u32x4{__builtin_bit_cast(uint32_t, r0), __builtin_bit_cast(uint32_t, r1),
                                     __builtin_bit_cast(uint32_t, r2), __builtin_bit_cast(uint32_t, r3)});
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One workgroup per work unit.
template <int D, int NH, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(const PrefillParams p) {
    using G = Geo<D>;
    using E = Epi<D, OUT_BF16>;
    constexpr int QT = 128 / NH;        // query rows per workgroup
    constexpr int WPH = 4 / NH;         // waves per query head
    static_assert(4 * E::WAVEB <= kStages * G::STAGEB, "epilogue staging must fit the ring");

    __shared__ __attribute__((aligned(1024))) char ring[kStages * G::STAGEB];

    // Block order: every unit's last (heaviest) query tile first, then every
    // unit's next one, and so on, so the long chains of key tiles start first
    // and the light tiles fill in behind them (unit-major order started the
    // last units' heavy tiles late: a 15-sequence pack took 30 us instead of
    // 25); unit u stays on XCD u % 8, whose L2 its query tiles share.
    const int idx = blockIdx.x;
    const int xcd = idx % kNumXcd, slot = idx / kNumXcd;
    const int upx = (p.n_units + kNumXcd - 1) / kNumXcd;   // units per XCD
    const int unit = (slot % upx) * kNumXcd + xcd;
    const int qt = p.q_tiles - 1 - slot / upx;
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
    const int last_tile = wrow0 < L ? min(wrow0 + 31, L - 1) / kKT : -1;   // last tile it needs
    const float c = p.scale_log2;

    u32x4 qreg[G::NKS];                         // Q^T: lane (n, hf) holds d = ks*16 + hf*8 .. +7
    {
        const uint16_t* qp = p.q + ((int64_t)(s0 + min(qrow, L - 1)) * p.n_heads_q + h) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks) qreg[ks] = *(const u32x4*)(qp + ks * 16);
    }
    LaneConst<D> lc;
    make_lane_const<D>(lc, lane, wave, lds_addr(ring));
    const int64_t kv_stride = (int64_t)p.n_heads_kv * D;
    const uint16_t* kbase = p.k + (int64_t)s0 * kv_stride + (int64_t)g * D;
    const uint16_t* vbase = p.v + (int64_t)s0 * kv_stride + (int64_t)g * D;

    f32x16 o[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    auto tile = [&](int t, auto stage_c) {
        constexpr int stage = decltype(stage_c)::value;
        wait_vmcnt<2 * G::LPW>();               // this wave's loads of tile t have landed
        __builtin_amdgcn_s_barrier();           // ... and every wave's; tile t-1 is consumed
        issue_tile<D, (stage + 2) % kStages>(ring, lc, kbase, vbase, kv_stride, (t + 2) * kKT, L, wave);
        if (t > last_tile) return;              // whole tile above this wave's diagonal
        const int k0 = t * kKT;
        if (k0 + kKT - 1 > wrow0)
            attend_tile<D, stage, true>(lc, 0u, qreg, hf, c, m, lsum, o, true, qrow - k0);
        else
            attend_tile<D, stage, false>(lc, 0u, qreg, hf, c, m, lsum, o, false, 0);
    };
    issue_tile<D, 0>(ring, lc, kbase, vbase, kv_stride, 0, L, wave);
    issue_tile<D, 1>(ring, lc, kbase, vbase, kv_stride, kKT, L, wave);   // past the end it re-reads valid rows
    for (int t = 0; t < ntiles; t += kStages) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 >= ntiles) break;
        tile(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 >= ntiles) break;
        tile(t + 2, std::integral_constant<int, 2>{});
    }
    wait_vmcnt<0>();                            // the tiles issued past the end must land
    lsum = sum_halves(lsum);
    const float inv = 1.f / lsum;

    __builtin_amdgcn_s_barrier();               // every wave is done with the ring
    const uint32_t wbuf = lds_addr(ring) + wave * E::WAVEB;
    const int64_t orow0 = (int64_t)(s0 + wrow0) * p.n_heads_q + h;   // output row of this wave's row 0
#pragma unroll
    for (int pass = 0; pass < E::NPASS; ++pass) {
        epi_stage<D, OUT_BF16>(wbuf, o, inv, pass, n, hf);
        wait_lgkm0();
#pragma unroll
        for (int k = 0; k < E::SPP; ++k) {
            const int chunk = k * 64 + lane;
            const int row = chunk / E::CH, c16 = chunk % E::CH;
            const u32x4 v = lds_read16(wbuf + row * E::PROWB + c16 * 16);
            wait_lgkm0();
            if (wrow0 + row < L)
                *(u32x4*)((char*)p.out + ((orow0 + (int64_t)row * p.n_heads_q) * D + pass * E::PCOLS) * E::OB +
                          c16 * 16) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Plan: the non-empty work items of the pack, per XCD.  Unit u (sequence b =
// u / per_seq, head block u % per_seq) belongs to XCD u % 8; an item is one
// query tile of a unit.  Each XCD's list holds its units in order, each unit's
// query tiles heaviest first, so that consecutive items share K/V.  Workgroup
// x builds XCD x's list: it stages cu_seqlens in LDS, counts the tiles of
// every XCD's list (for the list offsets), then scans and writes its own units.
constexpr int kPlanThreads = 256;

__device__ __forceinline__ int plan_unit_tiles(const PrefillParams& p, const int* cu, int u, int per_seq,
                                               int qt_rows, int& s0, int& L) {
    s0 = 0;
    L = 0;
    if (u >= p.n_units) return 0;
    const int b = u / per_seq;
    const int a = cu[b], e = cu[b + 1];
    if (a < 0 || e < a || e > p.total_tokens || e - a > p.max_seqlen) {
        raise_error(p.err, kErrCuSeqlens);
        return 0;
    }
    s0 = a;
    L = e - a;
    return (L + qt_rows - 1) / qt_rows;
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(const PrefillParams p) {
    extern __shared__ int cu_lds[];             // cu_seqlens, num_seqs + 1 entries
    __shared__ int tot[kNumXcd];
    __shared__ int wsum[kPlanThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, x = blockIdx.x;
    for (int i = tid; i <= p.num_seqs; i += kPlanThreads) cu_lds[i] = p.cu[i];
    if (tid < kNumXcd) tot[tid] = 0;
    __syncthreads();
    const int per_seq = p.n_heads_kv * p.head_blocks;
    const int qt_rows = 128 / p.heads_per_block;
    // Sequence b's per_seq units u = b * per_seq + j have one tile count; unit
    // j of it lands on XCD (b * per_seq + j) % 8.
    int mine[kNumXcd];
#pragma unroll
    for (int y = 0; y < kNumXcd; ++y) mine[y] = 0;
    for (int b = tid; b < p.num_seqs; b += kPlanThreads) {
        int s0, L;
        const int nq = plan_unit_tiles(p, cu_lds, b * per_seq, per_seq, qt_rows, s0, L);
        const int first = (b * per_seq) % kNumXcd;
#pragma unroll
        for (int y = 0; y < kNumXcd; ++y) {
            const int j0 = (y - first + kNumXcd) % kNumXcd;      // first j of this sequence on XCD y
            mine[y] += j0 < per_seq ? nq * ((per_seq - j0 + kNumXcd - 1) / kNumXcd) : 0;
        }
    }
#pragma unroll
    for (int y = 0; y < kNumXcd; ++y) {
        int v = mine[y];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0 && v) atomicAdd(&tot[y], v);
    }
    __syncthreads();
    int pos0 = 0;
    for (int y = 0; y < x; ++y) pos0 += tot[y];
    if (tid == 0) {
        p.plan_count[x] = tot[x];
        p.plan_off[x] = pos0;
        p.plan_claim[x] = 0;
        p.plan_done[x] = 0;
    }
    const int n_mine = (p.n_units - x + kNumXcd - 1) / kNumXcd;   // units x, x + 8, ...
    for (int base = 0; base < n_mine; base += kPlanThreads) {
        const int i = base + tid;
        int s0 = 0, L = 0;
        const int nq = i < n_mine ? plan_unit_tiles(p, cu_lds, i * kNumXcd + x, per_seq, qt_rows, s0, L) : 0;
        int incl = nq;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < kPlanThreads / kWave; ++w) {
            before += w < wave ? wsum[w] : 0;
            all += wsum[w];
        }
        int pos = pos0 + before + incl - nq;
        const int unit_in_seq = (i * kNumXcd + x) % per_seq;
        for (int j = 0; j < nq; ++j, ++pos) {
            if (pos >= p.plan_cap) {
                raise_error(p.err, kErrCuSeqlens);
                break;
            }
            p.plan_items[pos] = int4{s0, L, unit_in_seq, nq - 1 - j};
        }
        pos0 += all;
        __syncthreads();                        // wsum is rewritten by the next chunk
    }
}

// ---------------------------------------------------------------------------
// Persistent workgroups over the plan.  The resident workgroups of an XCD take
// that XCD's items in list order: workgroup l starts with item l, and each
// later item comes from the XCD's counter (item index = workgroups per XCD +
// ticket).  Claiming in order, each item shortly before it is needed, keeps
// the items in flight a compact window of the list, so a unit's query tiles
// run side by side and its K/V is read from HBM about once and from the XCD's
// L2 after that.
//
// A step covers 64 keys: two 32-key tiles, staged together in one half of a
// four-tile LDS ring while the next step's two tiles load into the other
// half, so each workgroup barrier, wait and issue serves 64 keys.
//
// Vector-memory instructions are counted so that each step's wait covers its
// two tiles and nothing newer: per step 4*LPW direct loads, then, at the end
// of an item, NST unconditional buffer stores and NKS Q loads for the next
// item (inline asm).  Wave 0 also issues one counter atomic per item; it is
// left out of the counts, which can only make a wait cover one more operation.
//
// A ticket reaches the other waves through LDS.  The ticket for the next item
// is claimed with the loads of an item's last step, just before them; the
// next step's wait has covered it, and wave 0 writes it to LDS before that
// step's barrier.  The issue side needs it at its next call, one step later,
// so it has always been published; a defensive path still waits for it
// explicitly should it not have been.  Claiming late keeps the items of a
// sequence (claimed in list order) running side by side: an item claimed at
// the start of a long predecessor would start many steps after its list
// neighbours, and the K/V they share would have left L2 by then (claiming at
// an item's first step read about 11% more from HBM).
// One counter increment by lane `sel` (0 or 1) of the wave; the old value
// lands in that lane of tk, written in place (tk is an in/out operand, so the
// register is never copied while the atomic is in flight).
__device__ __forceinline__ void claim_ticket(uint32_t& tk, int sel, int* counter) {
    uint64_t saved;
    const uint64_t lane_mask = 1ull << sel;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_and_b64 exec, exec, %4\n\t"
        "global_atomic_add %0, %2, %3, %5 sc0\n\t"
        "s_mov_b64 exec, %1"
        : "+v"(tk), "=&s"(saved)
        : "v"(0u), "v"(1u), "s"(lane_mask), "s"(counter)
        : "memory");
}
// Lane `sel` of v (uniform result).
__device__ __forceinline__ uint32_t read_lane(uint32_t v, int sel) {
    uint32_t r;
    asm volatile("v_readlane_b32 %0, %1, %2" : "=s"(r) : "v"(v), "s"(sel));
    return r;
}
// A uniform value the optimiser cannot see through: selects between such
// values stay selects of values (a select between two loads of one object
// is otherwise folded into one load at a computed offset, which keeps that
// object in private memory).
__device__ __forceinline__ int opaque_uniform(int v) {
    asm volatile("" : "+s"(v));
    return v;
}
__device__ __forceinline__ uint32_t read_lane0(uint32_t v) {
    uint32_t r;
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ void lds_write4_wait(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_read4_uniform(uint32_t addr) {
    uint32_t r;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr) : "memory");
    return (int)read_lane0(r);
}

// Work item as read from the plan.
struct PItem {
    int s0, L, q0, ntiles, g, h0;               // h0: first query head of the item
};

// State of one persistent workgroup.  Everything lives in this one object,
// reached only through its members, so that after inlining every field is
// promoted to a register (state shared by nested closures can stay in
// private memory).
template <int D, int NH, bool OUT_BF16>
struct PersistentTask {
    using G = Geo<D>;
    using E = Epi<D, OUT_BF16>;
    static constexpr int QT = 128 / NH;
    static constexpr int WPH = 4 / NH;
    static constexpr int KS = 2 * kKT;          // keys per step
    static constexpr int DMA = 4 * G::LPW;      // vector-memory ops per step's tile issue
    static constexpr int QL = G::NKS;           // Q loads per item
    static constexpr int ST = E::NST;           // output stores per item
    // the epilogue stages its rows in the half of the ring the finished step
    // read (after a barrier), where it fits; else in an area of its own
    static constexpr bool EPI_IN_RING = 4 * E::WAVEB <= 2 * G::STAGEB;
    static constexpr int LDS_BYTES = 4 * G::STAGEB + (EPI_IN_RING ? 0 : 4 * E::WAVEB);

    // fixed
    const PrefillParams* pp;
    char* ring;
    const int4* list;
    int* counter;
    int cnt, wx, lane, wave, n, hf;
    float c;
    int64_t kv_stride, out_bytes;
    uint32_t ring_addr, slot_addr;
    LaneConst<D> lc;
    // ticket of the next item (lane 0 of wave 0) and the LDS slot it is published in
    uint32_t tk;
    int slot_item, slot_pub;                    // item the slot holds, step whose barrier published it
    bool pend;                                  // a claimed ticket is not yet published
    int pend_item, pend_ps;                     // its item and the step from which it has landed
    // issue side: one step ahead of the compute side
    PItem iu;
    int ki, ti;                                 // item number and next step within it
    bool claimed;                               // the ticket of item ki + 1 is claimed
    bool need_next;                             // iu is fully issued: start item ki + 1 at the next call
    bool idone;                                 // no item after iu
    int ih0, ih1;                               // list index of items ki, ki - 1
    PItem iu1;                                  // item ki - 1 (valid when ih1 indexes the list)
    // compute side
    PItem cu;
    int jc, tc, h, wrow0, qrow, last_tile;
    u32x4 qreg[G::NKS];
    f32x16 o[G::NDB];
    float m, lsum;
    int end1;                                   // what the previous step issued at its end: 0 nothing,
                                                // 1 a store burst (ST ops), 2 stores then Q loads (ST + QL ops)
    bool fresh, done;
    int step_no;

    __device__ __forceinline__ PItem decode(int idx) const {
        const int4 e = scalar_load16(list + idx);
        PItem u;
        u.s0 = e.x;
        u.L = e.y;
        u.g = e.z / pp->head_blocks;
        u.h0 = u.g * pp->group + (e.z % pp->head_blocks) * NH;
        u.q0 = e.w * QT;
        u.ntiles = (min(u.q0 + QT, u.L) + KS - 1) / KS;     // steps of 64 keys
        return u;
    }

    __device__ __forceinline__ void publish(int step) {
        if (wave == 0) lds_write4_wait(slot_addr, (uint32_t)wx + read_lane(tk, 0));
        slot_item = pend_item;
        slot_pub = step;
        pend = false;
    }

    // The two tiles of the issue side's next step into ring half HALF.
    template <int HALF>
    __device__ __forceinline__ void issue_next(int step) {
        if (need_next) {                        // start item ki + 1
            need_next = false;
            const int want = ki + 1;
            const bool ready = opaque_uniform(slot_item) == want && opaque_uniform(slot_pub) <= step;
            if (!ready) {                       // not expected: wait for the ticket explicitly
                if (wave == 0) wait_vmcnt<0>();
                if (pend) publish(step);
                __builtin_amdgcn_s_barrier();
            }
            const int idx = lds_read4_uniform(slot_addr);
            ki = want;
            ih1 = ih0;
            ih0 = idx;
            iu1 = iu;                           // item ki - 1, decoded when it started
            if (idx < cnt) {
                iu = decode(idx);
                ti = 0;
                claimed = false;
            } else {
                idone = true;
            }
        }
        if (!idone && !claimed && iu.ntiles - ti <= 1) {   // ticket of item ki + 1, before its last step's loads
            if (wave == 0) claim_ticket(tk, 0, counter);
            claimed = true;
            pend = true;
            pend_item = ki + 1;
            pend_ps = step + 1;
        }
        const uint16_t* kb = pp->k + (int64_t)iu.s0 * kv_stride + (int64_t)iu.g * D;
        const uint16_t* vb = pp->v + (int64_t)iu.s0 * kv_stride + (int64_t)iu.g * D;
        const int t = idone ? iu.ntiles - 1 : ti;   // past the last item: re-read its last step's tiles
        issue_tile<D, 2 * HALF>(ring, lc, kb, vb, kv_stride, t * KS, iu.L, wave);
        issue_tile<D, 2 * HALF + 1>(ring, lc, kb, vb, kv_stride, t * KS + kKT, iu.L, wave);
        if (!idone && ++ti == iu.ntiles) need_next = true;
    }

    __device__ __forceinline__ void bind() {
        h = cu.h0 + wave / WPH;
        wrow0 = cu.q0 + (wave % WPH) * 32;
        qrow = wrow0 + n;
        last_tile = wrow0 < cu.L ? min(wrow0 + 31, cu.L - 1) / kKT : -1;
    }
    __device__ __forceinline__ void load_q() {
        const uint16_t* qp = pp->q + ((int64_t)(cu.s0 + min(qrow, cu.L - 1)) * pp->n_heads_q + h) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks) qreg[ks] = global_load16(qp + ks * 16);
    }
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        m = -INFINITY;
        lsum = 0.f;
    }

    // The finished item's output: rows u.s0 + u.q0 .. +QT of heads u.h0 ..
    // +NH, staged per wave at LDS address wbuf and stored with buffer stores
    // (offsets of rows outside the sequence are out of range, so those stores
    // are dropped and the count is fixed).
    __device__ __forceinline__ void epilogue(const PItem& u, int u_wrow0, int u_h, uint32_t wbuf) {
        const float inv = 1.f / sum_halves(lsum);
        const int64_t base = ((int64_t)(u.s0 + u.q0) * pp->n_heads_q) * D * E::OB;
        const int64_t span = min((int64_t)QT * pp->n_heads_q * D * E::OB, out_bytes - base);
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((char*)pp->out + base, 0, (int)span, 0x00020000);
#pragma unroll
        for (int pass = 0; pass < E::NPASS; ++pass) {
            epi_stage<D, OUT_BF16>(wbuf, o, inv, pass, n, hf);
            wait_lgkm0();
#pragma unroll
            for (int k = 0; k < E::SPP; ++k) {
                const int chunk = k * 64 + lane;
                const int row = chunk / E::CH, c16 = chunk % E::CH;
                const u32x4 v = lds_read16(wbuf + row * E::PROWB + c16 * 16);
                const int r = u_wrow0 - u.q0 + row;
                const int off = u_wrow0 + row < u.L
                                    ? (int)(((int64_t)r * pp->n_heads_q + u_h) * D * E::OB +
                                            pass * E::PCOLS * E::OB + c16 * 16)
                                    : 0x7FFFFFF0;
                wait_lgkm0();
                __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 2);   // nt: never re-read
            }
        }
    }

    // One step of the compute side on ring half HALF: its two tiles landed
    // (waited here), the next step's tiles go out into the other half.
    template <int HALF>
    __device__ __forceinline__ void step() {
        // wait for this step's tile loads: what the previous step issued after them may stay in flight
        if (end1 == 0)
            wait_vmcnt<0>();
        else if (end1 == 1)
            wait_vmcnt<ST>();
        else
            wait_vmcnt<ST + QL>();
        if (pend && pend_ps <= step_no) publish(step_no);   // the ticket has landed
        __builtin_amdgcn_s_barrier();           // every wave's loads landed; the other half is consumed
        issue_next<1 - HALF>(step_no);
        if (fresh) wait_vmcnt<DMA>();           // this item's Q rows (issued just before this step's tile loads)
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks) pin_after_wait(qreg[ks]);
        const int u0 = 2 * tc;                  // this step's first 32-key tile within the item
        if (u0 <= last_tile)
            attend_tile<D, 2 * HALF, true>(lc, 0u, qreg, hf, c, m, lsum, o, u0 * kKT + kKT - 1 > wrow0,
                                           qrow - u0 * kKT);
        if (u0 + 1 <= last_tile)
            attend_tile<D, 2 * HALF + 1, true>(lc, 0u, qreg, hf, c, m, lsum, o, (u0 + 1) * kKT + kKT - 1 > wrow0,
                                               qrow - (u0 + 1) * kKT);
        end1 = 0;
        fresh = false;
        ++step_no;
        if (++tc == cu.ntiles) {
            // the issue side has started item jc + 1 and at most one more;
            // take the item as the issue side decoded it
            const bool sel0 = ki == jc + 1;
            const int a0 = opaque_uniform(ih0), a1 = opaque_uniform(ih1);
            const int nidx = sel0 ? a0 : a1;
            const bool more = nidx >= 0 && nidx < cnt;
            const PItem fin = cu;
            const int fin_wrow0 = wrow0, fin_h = h;
            if (more) {
                const PItem& nu = sel0 ? iu : iu1;
                cu.s0 = __builtin_amdgcn_readfirstlane(nu.s0);   // uniform by construction
                cu.L = __builtin_amdgcn_readfirstlane(nu.L);
                cu.q0 = __builtin_amdgcn_readfirstlane(nu.q0);
                cu.ntiles = __builtin_amdgcn_readfirstlane(nu.ntiles);
                cu.g = __builtin_amdgcn_readfirstlane(nu.g);
                cu.h0 = __builtin_amdgcn_readfirstlane(nu.h0);
                bind();
            }
            uint32_t wbuf;
            if constexpr (EPI_IN_RING) {
                __builtin_amdgcn_s_barrier();   // every wave is done reading this half
                wbuf = ring_addr + 2 * HALF * G::STAGEB + wave * E::WAVEB;
            } else {
                wbuf = ring_addr + 4 * G::STAGEB + wave * E::WAVEB;
            }
            epilogue(fin, fin_wrow0, fin_h, wbuf);   // ST ops; its LDS reads have landed before it returns
            if (more) load_q();                 // QL ops, after the stores: qreg is free during the epilogue
            end1 = more ? 2 : 1;
            reset();
            ++jc;
            tc = 0;
            fresh = more;
            done = !more;
        }
    }
};

template <int D, int NH, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void prefill_persistent_kernel(const PrefillParams p) {
    using E = Epi<D, OUT_BF16>;
    using Task = PersistentTask<D, NH, OUT_BF16>;
    __shared__ __attribute__((aligned(1024))) char ring[Task::LDS_BYTES];
    __shared__ int slot[1];                     // list index of the next item

    const int x = blockIdx.x % kNumXcd, l = blockIdx.x / kNumXcd;
    const int cnt = scalar_load4(p.plan_count + x);
    if (l >= cnt) return;

    Task T;
    T.pp = &p;
    T.ring = ring;
    T.list = p.plan_items + scalar_load4(p.plan_off + x);
    T.counter = p.plan_claim + x;
    T.cnt = cnt;
    T.wx = gridDim.x / kNumXcd;
    T.lane = threadIdx.x & 63;
    T.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: wave-0 work is a scalar branch
    T.n = T.lane & 31;
    T.hf = T.lane >> 5;
    T.c = p.scale_log2;
    T.kv_stride = (int64_t)p.n_heads_kv * D;
    T.out_bytes = (int64_t)p.total_tokens * p.n_heads_q * D * E::OB;
    T.ring_addr = lds_addr(ring);
    T.slot_addr = lds_addr(slot);
    make_lane_const<D>(T.lc, T.lane, T.wave, lds_addr(ring));

    // ticket of item 1, claimed up front
    T.tk = 0;
    if (T.wave == 0) {
        claim_ticket(T.tk, 0, T.counter);
        wait_vmcnt<0>();
        lds_write4_wait(T.slot_addr, (uint32_t)T.wx + read_lane(T.tk, 0));
    }
    __builtin_amdgcn_s_barrier();
    T.slot_item = 1;
    T.slot_pub = -1000;
    T.pend = false;
    T.pend_item = 0;
    T.pend_ps = 0;

    T.iu = T.decode(l);
    T.ki = 0;
    T.ti = 0;
    T.claimed = true;
    T.need_next = false;
    T.idone = false;
    T.ih0 = l;
    T.ih1 = -1;
    T.iu1 = T.iu;
    T.cu = T.iu;
    T.jc = 0;
    T.tc = 0;
    T.bind();
    T.reset();
    T.end1 = 0;
    T.fresh = false;
    T.done = false;
    T.step_no = 0;

    T.load_q();
    T.template issue_next<0>(-1);               // the first step's wait (vmcnt 0) also covers the Q rows
    for (;;) {
        T.template step<0>();
        if (T.done) break;
        T.template step<1>();
        if (T.done) break;
    }
    wait_vmcnt<0>();                            // loads and tickets issued past the end land before the LDS is released
    // The XCD's counters start the next run over the same plan at zero: every
    // active workgroup counts itself out once its last ticket has returned
    // (waited just above), and the last one clears both counters.  Exactly
    // min(workgroups per XCD, items) workgroups take part.
    if (threadIdx.x == 0 && atomicAdd(p.plan_done + x, 1) == min(T.wx, cnt) - 1) {
        p.plan_claim[x] = 0;
        p.plan_done[x] = 0;
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

template <int D, int NH, bool OUT_BF16>
hipError_t launch_persistent(const PrefillParams& p, int num_cus, LaunchCache& cache, hipStream_t stream,
                             int phases) {
    int& per_cu = cache.prefill_per_cu[D == 128][NH == 2][OUT_BF16];   // resident workgroups per CU
    if (per_cu == 0) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, (const void*)prefill_persistent_kernel<D, NH, OUT_BF16>, 256, 0);
        if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    }
    const int grid = max(kNumXcd, per_cu * num_cus / kNumXcd * kNumXcd);
    if (phases & kPrefillPlan) {
        const size_t plan_lds = sizeof(int) * ((size_t)p.num_seqs + 1);   // num_seqs < kPrefillPlanMaxSeqs
        hipLaunchKernelGGL(prefill_plan_kernel, dim3(kNumXcd), dim3(kPlanThreads), plan_lds, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phases & kPrefillRun) {
        hipLaunchKernelGGL((prefill_persistent_kernel<D, NH, OUT_BF16>), dim3(grid), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int D, int NH, bool OUT_BF16>
hipError_t dispatch(const PrefillParams& p, bool persistent, int num_cus, LaunchCache& cache, hipStream_t stream,
                    int phases) {
    if (persistent) return launch_persistent<D, NH, OUT_BF16>(p, num_cus, cache, stream, phases);
    return (phases & kPrefillRun) ? launch_variant<D, NH, OUT_BF16>(p, stream) : hipSuccess;   // no plan to build
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, bool out_bf16, bool persistent, int num_cus,
                               LaunchCache& cache, hipStream_t stream, int phases) {
    const int nh = p.heads_per_block;
    if (head_dim == 128) {
        if (nh == 2)
            return out_bf16 ? dispatch<128, 2, true>(p, persistent, num_cus, cache, stream, phases)
                            : dispatch<128, 2, false>(p, persistent, num_cus, cache, stream, phases);
        return out_bf16 ? dispatch<128, 1, true>(p, persistent, num_cus, cache, stream, phases)
                        : dispatch<128, 1, false>(p, persistent, num_cus, cache, stream, phases);
    }
    if (nh == 2)
        return out_bf16 ? dispatch<64, 2, true>(p, persistent, num_cus, cache, stream, phases)
                        : dispatch<64, 2, false>(p, persistent, num_cus, cache, stream, phases);
    return out_bf16 ? dispatch<64, 1, true>(p, persistent, num_cus, cache, stream, phases)
                    : dispatch<64, 1, false>(p, persistent, num_cus, cache, stream, phases);
}

}  // namespace slm
