// smla_attn128.hip -- sparse MLA attention over the bf16 cache with all 128
// heads of a token in one workgroup (h_q = 128).
//
// What is computed follows the vLLM page "vllm/v1/attention/backends/mla/
// flashmla_sparse.py" (FLASHMLA_SPARSE backend): the index conversion of
// triton_convert_req_index_to_global_index, the fp8_ds_mla row format of the
// module note, and the multi-query attention with 576-wide keys and 512-wide
// values that FlashMLASparseImpl.forward runs (_bf16_flash_mla_kernel for the
// bf16 cache). How it is computed is this library's own design for gfx950:
//
//  * Workgroup = one query token x all 128 heads x one part of its top-k list.
//    Every gathered tile of 32 cache rows is shared by the 128 heads: it is
//    copied into LDS once and read by four waves, one per SIMD.
//  * Wave w computes S^T = K q^T and the online softmax for heads 32 w .. 32 w
//    + 31, with 32x32 MFMAs: one MFMA covers 32 rows x 32 heads, so a K fragment
//    read from LDS feeds all 32 heads of the wave. The S^T accumulator gives
//    lane l head l mod 32 and 16 of the tile's rows (the other 16 are in lane l
//    xor 32), so the head's max and sum need one cross-lane step, and the
//    weights are already in the B-operand layout of the PV MFMA (its 16 k-rows
//    per step are taken in the accumulator's row order; the transposed V^T
//    reads gather the same rows in that order).
//  * PV is split by output dims: each wave publishes its head block's weights
//    in LDS, and after a second barrier adds O^T += V^T P^T for output dims
//    128 w .. 128 w + 127 of all 128 heads, so each V^T fragment is read by one
//    wave instead of four.
//  * O^T of the wave's dims (128 dims x 128 heads, fp32) lives in the 256
//    accumulation registers (AGPRs); q (bf16, 144 registers per lane) lives in
//    ordinary registers for the whole kernel.
//  * The fp8_ds_mla cache keeps the 64-head kernel at h_q = 128 (two
//    workgroups per token): there its QK^T and PV waves overlap on each SIMD,
//    while one wave per SIMD here leaves the fp8 tile's dependency chain
//    (dequantisation scales, hi + lo q terms) exposed.
//  * Prologue, gather, compaction and the explicit-wait discipline are those
//    of the 64-head kernel: the indices and the block-table row come into LDS
//    in one round trip, valid slots are compacted in list order, each row is
//    copied as stored by one or two global_load_lds_dwordx4 instructions, and
//    the compiler sees no vector-memory load it would wait for inside the loop.
//  * Output: one part writes bf16 rows of o (staged in LDS, stored coalesced)
//    and lse; a top-k part writes its fp32 O / l and lse for merge_kernel.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float f32x16 __attribute__((__vector_size__(64)));

// bf16 rows: 1152 bytes, stored at a 1168-byte stride (16 consecutive rows fall
// on distinct banks for the 16-byte K reads and the transposed V reads). The
// tile loop cycles through two ring buffers (tile r and the copy of tile r + 1):
// deeper rings measured slower (three 4 %, four 7 %). The LDS before the slot
// list holds four buffers' worth, which the bf16 output staging of 128 heads
// needs at the end.
struct Cfg128 {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kHeads = 128;
    static constexpr int kRowBytes = RowFmt<kCacheBf16>::kBytes;
    static constexpr int kChunksPerRow = kRowBytes / 16;
    static constexpr int kRowStride = kBf16RowBytes + 16;
    static constexpr int kRowBlockBytes = 16 * kRowStride;
    static constexpr int kInstrPerRow = (kChunksPerRow + 63) / 64;
    static constexpr int kRowsPerWave = kTile / kWaves;
    static constexpr int kDmaPerWave = kRowsPerWave * kInstrPerRow;  // copy instructions per wave and tile
    static constexpr int kBufBytes = (kRB * kRowBlockBytes + 255) / 256 * 256;
    static constexpr int kNBuf = 2;                                  // ring buffers of the tile loop
    static constexpr int kOffSlots = 4 * kBufBytes;                  // the ring, or the output staging
    // top-k positions compacted into LDS per round (512 and 1024 measured alike)
    static constexpr int kChunk = 512;
    static constexpr int kOffMisc = kOffSlots + kChunk * 4;
    // P^T operands of the four head blocks, hi and lo terms ([pass][head block]
    // [k-step][lane], 16 KB), in ring space the two-buffer loop leaves free
    static constexpr int kOffP = 2 * kBufBytes;
    static constexpr int kOffHeadF = kOffMisc + 512;                   // 1 / l of the 128 heads
    static constexpr int kLdsBytes = kOffHeadF + 512;
    static constexpr int kStageRow = kDv * 2 + 16;                     // bf16 output staging row
    static constexpr int kBtLdsMax = 2 * kBufBytes / 4;                // table entries in buffers 0, 1
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one gfx950 workgroup");
    static_assert(kOffP + 2 * 4 * 2 * 1024 <= kOffSlots, "P^T fits the ring space past the loop's buffers");
    static_assert(kHeads * kStageRow <= kOffMisc, "output staging fits the ring and the slot list");
    static_assert(kTile % kWaves == 0, "whole rows per wave");
    static_assert(kDmaPerWave * (kNBuf - 2) <= 63, "copies in flight within the vmcnt range");
    static_assert(16 + (kChunk / kThreads) * kWaves <= 128, "compaction counts fit");
};

// O^T += A B with O held in accumulation registers (AGPRs). O of a wave's 32
// heads takes all 256 of them, so the file is compiled with MFMA results in
// ordinary registers (the S^T accumulator among them) and this one product is
// written out: the compiler sees a plain AGPR operand and places no wait for
// the matrix pipe around it, nor for the VALU results the MFMA reads. Four wait
// states therefore precede it (operands just written by VALU instructions);
// code that reads O itself goes through o_settle() first.
__device__ __forceinline__ void mfma_o(f32x16 &o, const bf16x8 &a, const bf16x8 &b)
{
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// Enough wait states for the last 32x32x16 MFMA's result (16 passes) before a
// VALU or v_accvgpr access of O. Every block of O is an operand, so no read of
// O can be scheduled above the wait.
__device__ __forceinline__ void o_settle(f32x16 (&o)[16])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]),
                   "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                   "+a"(o[14]), "+a"(o[15])
                 :
                 : "memory");
}

// O^T := 0 by an MFMA of zero operands (no v_accvgpr writes of the compiler);
// the zero registers may just have been written, hence the wait states.
__device__ __forceinline__ void o_zero(f32x16 &o)
{
    const bf16x8 z = {};
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(o) : "v"(z));
}

// How far (log2 units) a head's logits may rise above the reference its first
// tile set before the weights exp2(s - reference) risk overflow: 2^64 leaves
// fp32 and bf16 (same exponent range) far from their limit even summed over
// 2^20 rows. Past it, the workgroup redoes the list in two passes.
constexpr float kRefHeadroom = 64.0f;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn128_kernel(const KParams p)
{
    using C = Cfg128;
    constexpr int kPer = C::kChunk / C::kThreads;   // top-k positions per thread per round

    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
    uint8_t *ring = smem;
    int32_t *lds_slots = (int32_t *)(smem + C::kOffSlots);
    int32_t *lds_misc = (int32_t *)(smem + C::kOffMisc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5;          // lane half: rows 4 hh + 8 j + i of the accumulator
    const int n32 = lane & 31;         // accumulator column: head 32 wave + n32; K / V row for operands

    // Workgroup id -> (token, part); all parts of one token get the same id
    // mod 8, the XCD the hardware dispatches them to.
    int bid = blockIdx.x;
    const int xcd = bid & 7;
    bid >>= 3;
    const int s = bid % p.S;
    const int t = (bid / p.S) * 8 + xcd;
    if (t >= p.T)
        return;
    const int head = 32 * wave + n32;
    const float c2 = p.log2e_scale;
    const int32_t *topk_row = p.topk + (size_t)t * p.K;
    const int req = p.slot_in ? 0 : p.req_id[t];
    const int pos_begin = s * p.split_len;
    const int pos_end = min(p.K, pos_begin + p.split_len);

    // ---- q of this lane's head, requested first (plain loads; their wait is
    //      placed where the prologue has already waited for everything):
    //      k-step ks (16 columns) holds columns 16 ks + 8 hh .. + 7.
    const uint4 *qrow = (const uint4 *)(p.q + ((size_t)t * p.H + head) * kDqk);
    constexpr int kQ = 36;             // 16-byte pieces of q per lane
    u32x4 qraw[kQ];
#pragma unroll
    for (int k = 0; k < kQ; ++k) {
        qraw[k] = __builtin_bit_cast(u32x4, qrow[2 * k + hh]);
    }

    // ---- one round of the list: indices and the block-table row into LDS in
    //      one round trip, slots computed from LDS (as in the 64-head kernel)
    const int32_t *bt_lds = (const int32_t *)smem;
    const int32_t *idx_lds = lds_slots;
    const bool bt_in_lds = !p.slot_in && (unsigned)req < (unsigned)p.R && p.MB <= C::kBtLdsMax;
    // Both read the lane id through late(): the per-lane addresses they form are
    // rebuilt every round instead of being held across the tile loop.
    auto fetch_round = [&](int chunk0, int (&slotv)[kPer]) __attribute__((always_inline)) {
        const int lane = late(tid & 63), tid = 64 * wave + lane;
        const int n = min(pos_end, chunk0 + C::kChunk) - chunk0;
        const uint32_t idx_base = (uint32_t)(uintptr_t)LDS_PTR(int32_t, lds_slots);
        for (int e0 = 64 * wave; e0 < n; e0 += C::kThreads) {
            if (e0 + lane < n)
                dma4(topk_row + chunk0 + e0 + lane, __builtin_amdgcn_readfirstlane(idx_base + 4u * (uint32_t)e0));
        }
        if (bt_in_lds) {
            const int32_t *bt_row = p.bt + (size_t)req * p.MB;
            const uint32_t bt_base = (uint32_t)(uintptr_t)LDS_PTR(uint8_t, smem);
            for (int e0 = 64 * wave; e0 < p.MB; e0 += C::kThreads) {
                if (e0 + lane < p.MB)
                    dma4(bt_row + e0 + lane, __builtin_amdgcn_readfirstlane(bt_base + 4u * (uint32_t)e0));
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int idxv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + C::kThreads * j;
            idxv[j] = i < n ? idx_lds[i] : -1;
        }
        if (p.slot_in) {
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                slotv[j] = given_slot(idxv[j], p.NB);
        } else if (bt_in_lds) {
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                slotv[j] = finish_slot(bt_lds[slot_position_ok(req, idxv[j], p.R, p.MB) ? (idxv[j] >> 6) : 0], req,
                                       idxv[j], p.R, p.MB, p.NB);
        } else {
            // a table row too long for the ring: each thread's entries copied
            // from the table into words of ring buffer 0, then read back
            const uint32_t own_base = (uint32_t)(uintptr_t)LDS_PTR(int32_t, (int32_t *)smem) +
                                      4u * 64u * (uint32_t)(kPer * wave);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const bool ok = slot_position_ok(req, idxv[j], p.R, p.MB);
                dma4(p.bt + (ok ? (size_t)req * p.MB + (idxv[j] >> 6) : 0),
                     __builtin_amdgcn_readfirstlane(own_base + 4u * 64u * (uint32_t)j));
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                slotv[j] = finish_slot(((const int32_t *)smem)[64 * (kPer * wave + j) + lane], req, idxv[j], p.R,
                                       p.MB, p.NB);
        }
    };

    // valid slots of the round into LDS in list order (two barriers)
    auto compact = [&](int chunk0, int (&slotv)[kPer]) __attribute__((always_inline)) {
        const int lane = late(tid & 63), tid = 64 * wave + lane;
        const int chunk_n = min(C::kChunk, pos_end - chunk0);
        if (p.phys_out != nullptr) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = tid + C::kThreads * j;
                if (i < chunk_n)
                    p.phys_out[(size_t)t * p.K + chunk0 + i] = slotv[j];
            }
        }
        uint64_t masks[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            masks[j] = __ballot(slotv[j] >= 0);
            if (lane == 0)
                lds_misc[16 + j * C::kWaves + wave] = __popcll(masks[j]);
        }
        __syncthreads();
        const int my_count = lds_misc[16 + (lane & 31)];
        int base[kPer];
        const int n_valid = compaction_bases<kPer, C::kWaves>(my_count, wave, base);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (slotv[j] >= 0)
                lds_slots[base[j] + lanes_below(masks[j])] = slotv[j];
        __syncthreads();
        return n_valid;
    };

    int slotv[kPer];
    fetch_round(pos_begin, slotv);

    // q is complete here (the round's wait covered its loads). Each register
    // passes through an empty asm, so the compiler's wait for the loads is
    // placed here and never inside the tile loop.
#pragma unroll
    for (int k = 0; k < kQ; ++k)
        asm volatile("" : "+v"(qraw[k]));

    // q as the B operand of the QK^T MFMAs, k-steps 0..35
    bf16x8 qb[kQ];
#pragma unroll
    for (int k = 0; k < kQ; ++k)
        qb[k] = __builtin_bit_cast(bf16x8, qraw[k]);

    // ---- per-lane LDS offsets inside a tile buffer, derived from the lane id in
    //      every tile (from late(lane): held across the tile loop instead, they and
    //      the row numbers below would take registers that q and O need)
    struct Offs {
        int k;          // K rows for the A operand: row n32, half hh
        int v[2][2];    // V^T transposed reads: [k-step][row quad]
        int lim_off;    // 4 hh: accumulator rows are 8 j + i + 4 hh
    };
    auto offsets = [&]() __attribute__((always_inline)) {
        const int ln = late(lane);
        const int h2 = ln >> 5, c32 = ln & 31;
        Offs f;
        f.k = lds_row<C>(c32) + 16 * h2;
        const int vg = ln >> 4, vj = ln & 15;   // 16-lane group g, lane j in it
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) {
                // lane j of a 16-lane group supplies row j / 4 of the 4-row read
                const int row = 16 * ks + 8 * qd + 4 * (vg >> 1) + (vj >> 2);
                f.v[ks][qd] = lds_row<C>(row) + 2 * (16 * (vg & 1) + 4 * (vj & 3));
            }
        }
        f.lim_off = 4 * h2;
        return f;
    };

    f32x16 o[16];
#pragma unroll
    for (int db = 0; db < 16; ++db)
        o_zero(o[db]);
    // The online softmax keeps a fixed reference per head (log2 units): the max
    // of the head's first tile. O is never rescaled (it lives in AGPRs, where
    // VALU cannot reach it); later weights exp2(s - m_ref) may exceed 1. If a
    // tile's max rises more than kRefHeadroom above the reference, the list is
    // redone: a pass that finds each head's exact max (QK^T only), then the
    // full pass with that max as the reference.
    float m_ref = -INFINITY, l_part = 0.f;
    bool ref_set = false;                      // wave-uniform
    // Restart flags, one per tile parity: tile r may set flag[r & 1]; the waves
    // read flag[(r - 1) & 1] after the barrier that opens tile r, which every
    // write made during tile r - 1 precedes, and no wave can be writing it
    // then (a wave in tile r writes the other one), so all four waves decide
    // alike. They act on it after tile r, so the read's latency is hidden; the
    // restart discards that tile's work with the rest of the pass.
    int *restart_flag = lds_misc + 2;
    if (tid == 0) {
        restart_flag[0] = 0;                   // published by the compaction's barriers
        restart_flag[1] = 0;
    }

    // One tile. kMode 0: reference from the first tile, headroom check; 1: max
    // only (no PV); 2: fixed reference. exact: P as hi + lo bf16 (two PV sweeps).
    // The LDS fragments are software-pipelined by hand: each stage reads the
    // next group's fragments while its own MFMAs run. In QK^T a scheduling
    // barrier closes every stage, so no more than two groups of K fragments are
    // ever live beside q (144 registers) and the 256 accumulators of O; the PV
    // stages are left to the compiler's schedule (measured faster).
    auto tile = [&](const uint8_t *buf, int n_tile, bool exact, auto mode_c, int *flag, auto &&copy)
                    __attribute__((always_inline)) {
        constexpr int kMode = decltype(mode_c)::value;
        const Offs f = offsets();
        const int off_k = f.k;
        f32x16 acc = {};
        {
            constexpr int KG = 6;      // k-steps per stage
            bf16x8 cur[KG], nxt[KG];
#pragma unroll
            for (int j = 0; j < KG; ++j)
                cur[j] = *(const bf16x8 *)(buf + off_k + 32 * j);
#pragma unroll
            for (int g0 = 0; g0 < 36; g0 += KG) {
                if (g0 + KG < 36) {
#pragma unroll
                    for (int j = 0; j < KG; ++j)
                        nxt[j] = *(const bf16x8 *)(buf + off_k + 32 * (g0 + KG + j));
                }
#pragma unroll
                for (int j = 0; j < KG; ++j)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[j], qb[g0 + j], acc, 0, 0, 0);
                // this stage's share of the refill copies, issued while its MFMAs run
#pragma unroll
                for (int k = 3 * (g0 / KG); k < 3 * (g0 / KG) + 3; ++k)
                    copy(k);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < KG; ++j)
                    cur[j] = nxt[j];
            }
        }

        // softmax in log2 units (scale c2 > 0 applied to the max and in the exp2
        // argument); rows past the tile's valid count are -inf
        float lmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (n_tile < kTile)
                acc[e] = 8 * (e >> 2) + (e & 3) < n_tile - f.lim_off ? acc[e] : -INFINITY;
            lmax = fmaxf(lmax, acc[e]);
        }
        lmax = xor32_max(lmax) * c2;
        if constexpr (kMode == 1) {
            m_ref = fmaxf(m_ref, lmax);
            return;
        }
        if constexpr (kMode == 0) {
            if (!ref_set) {
                m_ref = lmax;
                ref_set = true;
            } else if (__ballot(lmax > m_ref + kRefHeadroom) != 0 && lane == 0) {
                *flag = 1;
            }
        }
        float pw[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            pw[e] = __builtin_amdgcn_exp2f(fmaf(acc[e], c2, -m_ref));
            l_part += pw[e];
        }

        // ---- O^T += V^T P^T; k-step ks takes accumulator elements 8 ks .. 8 ks + 7.
        auto load_v = [&](int db, int ks) __attribute__((always_inline)) -> uint4 {
            const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(i16x4, buf + f.v[ks][0] + 64 * db)));
            const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(i16x4, buf + f.v[ks][1] + 64 * db)));
            return make_uint4(w0.x, w0.y, w1.x, w1.y);
        };
        // weights w as bf16 B operands: hi terms, or (lo) what hi misses
        auto pack = [&](const float (&w)[16], bool lo, bf16x8 (&pp)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 p0 = {w[8 * ks], w[8 * ks + 1], w[8 * ks + 2], w[8 * ks + 3]};
                const f32x4 p1 = {w[8 * ks + 4], w[8 * ks + 5], w[8 * ks + 6], w[8 * ks + 7]};
                pp[ks] = pack_p(p0, p1);
                if (lo)
                    pp[ks] = pack_p_residual(p0, p1, pp[ks]);
            }
        };
        // publish this wave's P^T operands (head block `wave`), then PV over this
        // wave's output dims 128 wave .. 128 wave + 127 for all four head blocks:
        // each V^T fragment is read by one wave instead of four
        bf16x8 *p_x = (bf16x8 *)(smem + C::kOffP);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (pass == 1 && !exact)
                break;
            bf16x8 pp[2];
            pack(pw, pass == 1, pp);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                p_x[((pass * 4 + wave) * 2 + ks) * 64 + lane] = pp[ks];
        }
        // the first dim block's V^T fragments before the barrier: tile r landed
        // at the previous one, and nothing writes it during the tile
        uint4 v_pre[1][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            v_pre[0][ks] = load_v(4 * wave, ks);
        __syncthreads();     // every head block's P^T is published
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (pass == 1 && !exact)
                break;
            bf16x8 pv[4][2];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    pv[hb][ks] = p_x[((pass * 4 + hb) * 2 + ks) * 64 + lane];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 v0 = d < 1 ? v_pre[0][0] : load_v(4 * wave + d, 0);
                const uint4 v1 = d < 1 ? v_pre[0][1] : load_v(4 * wave + d, 1);
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    mfma_o(o[4 * hb + d], __builtin_bit_cast(bf16x8, v0), pv[hb][0]);
                    mfma_o(o[4 * hb + d], __builtin_bit_cast(bf16x8, v1), pv[hb][1]);
                }
            }
        }
    };

    // ---- the list, one round of up to kChunk positions at a time. Returns
    //      true when mode 0 found a head past its headroom (the tile loop stops
    //      at the next barrier, with every copy landed).
    auto run = [&](auto mode_c, bool first_fetched) __attribute__((always_inline)) -> bool {
        constexpr int kMode = decltype(mode_c)::value;
        // every path into the compaction has just fetched its round: slotv is
        // dead while the tiles run
        if (!first_fetched && pos_begin < pos_end)
            fetch_round(pos_begin, slotv);
        for (int chunk0 = pos_begin; chunk0 < pos_end;) {
            const int n_valid = compact(chunk0, slotv);
            const bool exact_p = n_valid <= kExactPRows;
            const int n_tiles = (n_valid + kTile - 1) / kTile;
            // tiles 0 .. kNBuf - 2 now; iteration r refills the buffer tile r - 1 freed
            int issued = min(n_tiles, C::kNBuf - 1);
#pragma unroll
            for (int i = 0; i < C::kNBuf - 1; ++i) {
                if (i < issued)
                    issue_tile<C>(p.cache, lds_slots + i * kTile, min(kTile, n_valid - i * kTile),
                                  ring + i * C::kBufBytes, wave, lane);
            }
            bool stop = false;
            // Iteration r: tile r, and (copy_c) the refill of the buffer tile r - 1
            // freed with tile r + kNBuf - 1, whose 16 copy instructions of this wave
            // go out between the QK^T stages (tile() calls copy(k)). The
            // iterations with and without a refill run as two loops, so no branch
            // on it sits in the run of MFMAs.
            auto iteration = [&](int r, auto copy_c) __attribute__((always_inline)) -> bool {
                constexpr bool kCopy = decltype(copy_c)::value;
                // this wave's rows of tile r have landed ...
                wait_vmcnt(C::kDmaPerWave * (issued - r - 1));
                // ... and every wave's; every wave is done with tile r - 1
                __syncthreads();
                // the restart flag of tile r - 1 is read now and acted on after tile r
                // (no wait for the read before the tile's work; a restart discards
                // that work anyway)
                int flag_seen = 0;
                if (kMode == 0)
                    flag_seen = restart_flag[(r + 1) & 1];
                int rf_slot = 0;
                uint32_t rf_base = 0;
                if constexpr (kCopy) {
                    const int ln = late(lane);
                    const int ri = C::kRowsPerWave * wave + ln % C::kRowsPerWave;
                    rf_slot = lds_slots[issued * kTile + (ri < min(kTile, n_valid - issued * kTile) ? ri : 0)];
                    rf_base = __builtin_amdgcn_readfirstlane(
                        (uint32_t)(uintptr_t)LDS_PTR(uint8_t, ring + (issued % C::kNBuf) * C::kBufBytes) +
                        (uint32_t)lds_row<C>(C::kRowsPerWave * wave));
                }
                // copy k: row k / 2 of this wave's rows, chunks 0..63 (k even) or 64..71
                auto copy = [&](int k) __attribute__((always_inline)) {
                    if constexpr (kCopy) {
                        if (k >= C::kDmaPerWave)
                            return;
                        const int i = k >> 1, part = k & 1;
                        const int ln = late(lane);
                        const int slot = __builtin_amdgcn_readlane(rf_slot, i);
                        const uint8_t *src = p.cache + (size_t)(uint32_t)slot * C::kRowBytes + 16 * (64 * part + ln);
                        const uint32_t dst = __builtin_amdgcn_readfirstlane(
                            rf_base + (uint32_t)(lds_row<C>(C::kRowsPerWave * wave + i) -
                                                 lds_row<C>(C::kRowsPerWave * wave)) + 1024u * (uint32_t)part);
                        if (part == 0)
                            dma16(src, dst);
                        else
                            dma16_lanes(src, dst, (1ull << (C::kChunksPerRow - 64)) - 1ull);
                    }
                };
                tile(ring + (r % C::kNBuf) * C::kBufBytes, min(kTile, n_valid - r * kTile), exact_p, mode_c,
                     restart_flag + (r & 1), copy);
                if constexpr (kCopy)
                    ++issued;
                return kMode == 0 && flag_seen != 0;
            };
            const int r_copy = max(0, n_tiles - (C::kNBuf - 1));   // iterations with a refill
            int r = 0;
            for (; r < r_copy && !stop; ++r)
                stop = iteration(r, std::true_type{});
            for (; r < n_tiles && !stop; ++r)
                stop = iteration(r, std::false_type{});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies of tiles a stop left unread
            __syncthreads();     // ring and slot list are free for the next round
            if (kMode == 0 && (stop || (restart_flag[0] | restart_flag[1]) != 0))
                return true;
            chunk0 += C::kChunk;
            if (chunk0 < pos_end)
                fetch_round(chunk0, slotv);
        }
        return false;
    };
    if (run(std::integral_constant<int, 0>{}, true)) {
        // a head's logits rose past the headroom: exact maxima, then the full pass
        // (O's registers may serve the max-only pass once its last MFMA is done)
        o_settle(o);
        m_ref = -INFINITY;
        run(std::integral_constant<int, 1>{}, false);
        l_part = 0.f;
#pragma unroll
        for (int db = 0; db < 16; ++db)
            o_zero(o[db]);
        run(std::integral_constant<int, 2>{}, false);
    }

    // ---- epilogue: the head's row sum (this lane's rows and the other half's);
    //      o[4 hb + d] holds dims 128 wave + 32 d + 8 j + 4 hh + i of head
    //      32 hb + n32, so every wave needs 1 / l of all 128 heads
    o_settle(o);
    const float l = xor32_sum(l_part);
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    // natural-log lse (v_log_f32 is log2; l >= 1 here: the row that set the max adds >= 1)
    const float lse_v = l > 0.f ? (m_ref + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
    float *head_f = (float *)(smem + C::kOffHeadF);
    if (hh == 0)
        head_f[head] = inv_l;
    __syncthreads();        // every head's factor is published; the ring and P^T are free
    float inv_hb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
        inv_hb[hb] = head_f[32 * hb + n32];
    if (!p.partials) {
        // bf16 rows staged in LDS, then written out coalesced
        uint8_t *stage = smem;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x16 &ob = o[4 * hb + d];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = ob[4 * j] * inv_hb[hb], v1 = ob[4 * j + 1] * inv_hb[hb];
                    const float v2 = ob[4 * j + 2] * inv_hb[hb], v3 = ob[4 * j + 3] * inv_hb[hb];
                    *(uint2 *)(stage + (32 * hb + n32) * C::kStageRow + 2 * (128 * wave + 32 * d + 8 * j + 4 * hh)) =
                        make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
                }
            }
        }
        if (hh == 0 && p.lse != nullptr)
            p.lse[(size_t)t * p.H + head] = lse_v;
        __syncthreads();
        uint16_t *dst = p.out + (size_t)t * p.H * kDv;
        for (int u = tid; u < C::kHeads * kDv / 8; u += C::kThreads) {
            const int row = u / (kDv / 8), c8 = u % (kDv / 8);
            *(uint4 *)(dst + 8 * u) = *(const uint4 *)(stage + row * C::kStageRow + 16 * c8);
        }
    } else {
        // fp32 O / l of this part and its lse, for merge_kernel
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            float *po = p.part_o + (((size_t)t * p.S + s) * p.H + 32 * hb + n32) * kDv + 128 * wave;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(f32x4 *)(po + 32 * d + 8 * j + 4 * hh) =
                        f32x4{o[4 * hb + d][4 * j] * inv_hb[hb], o[4 * hb + d][4 * j + 1] * inv_hb[hb],
                              o[4 * hb + d][4 * j + 2] * inv_hb[hb], o[4 * hb + d][4 * j + 3] * inv_hb[hb]};
            }
        }
        if (hh == 0)
            p.part_lse[((size_t)t * p.S + s) * p.H + head] = lse_v;
    }
}

}  // namespace

hipError_t launch_attn128(const KParams &p, hipStream_t stream)
{
    const int64_t tq = (p.T + 7) / 8;
    const dim3 grid((unsigned)(tq * 8 * p.S));
    hipLaunchKernelGGL(attn128_kernel, grid, dim3(Cfg128::kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace smla
