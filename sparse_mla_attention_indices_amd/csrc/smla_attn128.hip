// smla_attn128.hip -- sparse MLA attention with all 128 heads of a token in one
// workgroup (h_q = 128), for both cache formats.
//
// What is computed follows the vLLM page "vllm/v1/attention/backends/mla/
// flashmla_sparse.py" (FLASHMLA_SPARSE backend): the index conversion of
// triton_convert_req_index_to_global_index, the fp8_ds_mla row format of the
// module note, and the multi-query attention with 576-wide keys and 512-wide
// values that FlashMLASparseImpl.forward runs (_bf16_flash_mla_kernel for the
// bf16 cache, _fp8_flash_mla_kernel for fp8_ds_mla). How it is computed is this
// library's own design for gfx950:
//
//  * Workgroup = one query token x all 128 heads x one part of its top-k list.
//    Every gathered tile of 32 cache rows is shared by the 128 heads: it is
//    copied into LDS once and read by four waves, one per SIMD.
//  * Wave w owns heads 32 w .. 32 w + 31 whole: S^T = K q^T, the online softmax
//    and O^T += V^T P^T, with 32x32 MFMAs. One MFMA covers 32 rows x 32 heads,
//    so a K fragment read from LDS feeds all 32 heads of the wave. The S^T
//    accumulator gives lane l head l mod 32 and 16 of the tile's rows (the other
//    16 are in lane l xor 32), so the head's max and sum need one cross-lane
//    step, and the weights are already the B operand of the PV MFMA (its 16
//    k-rows per step are taken in the accumulator's row order; the transposed
//    V^T reads gather the same rows in that order). No weight goes through LDS.
//  * O^T of the wave's 32 heads (32 x 512 fp32) lives in the 256 accumulation
//    registers (AGPRs); q lives in ordinary registers for the whole kernel:
//    bf16 columns for the bf16 cache; for fp8, the 512 latent columns as hi + lo
//    e4m3 terms with a power-of-two scale per head and 128-column group (the
//    scaled MFMA applies it), and the 64 RoPE columns as bf16 in LDS.
//  * fp8: the raw e4m3 K bytes feed v_mfma_scale_f32_32x32x64_f8f6f4; each
//    128-column group's partial S is multiplied by its rows' scales; V^T is
//    converted to bf16 exactly and the weights of each 128-dim output group
//    carry that group's row scales, so dequantisation adds no rounding.
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

#include <type_traits>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float f32x16 __attribute__((__vector_size__(64)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

template <int FMT> struct Ring128;
// bf16 rows: 1152 bytes, stored at a 1168-byte stride (16 consecutive rows fall
// on distinct banks for the 16-byte K reads and the transposed V reads); four
// ring buffers.
template <> struct Ring128<kCacheBf16> {
    static constexpr int kRowStride = kBf16RowBytes + 16;
    static constexpr int kBlockGap = 0;
    static constexpr int kNBuf = 4;
};
// fp8_ds_mla rows: 656 bytes at their own stride, rows 16..31 of a tile 16
// bytes later (the transposed V reads touch rows r and r + 8); six buffers
// (the RoPE part of q takes the room of a seventh).
template <> struct Ring128<kCacheFp8> {
    static constexpr int kRowStride = kFp8RowBytes;
    static constexpr int kBlockGap = 16;
    static constexpr int kNBuf = 6;
};

template <int FMT>
struct Cfg128 {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kHeads = 128;
    static constexpr int kRowBytes = RowFmt<FMT>::kBytes;
    static constexpr int kChunksPerRow = kRowBytes / 16;
    static constexpr int kRowStride = Ring128<FMT>::kRowStride;
    static constexpr int kRowBlockBytes = 16 * kRowStride + Ring128<FMT>::kBlockGap;
    static constexpr int kInstrPerRow = (kChunksPerRow + 63) / 64;
    static constexpr int kRowsPerWave = kTile / kWaves;
    static constexpr int kDmaPerWave = kRowsPerWave * kInstrPerRow;  // copy instructions per wave and tile
    static constexpr int kBufBytes = (kRB * kRowBlockBytes + 255) / 256 * 256;
    static constexpr int kNBuf = Ring128<FMT>::kNBuf;
    static constexpr int kOffSlots = kNBuf * kBufBytes;
    // fp8: the RoPE columns of q (bf16), 16 bytes per lane and k-step, lane-major
    static constexpr int kOffQRope = kOffSlots + kMaxChunk * 4;
    static constexpr int kQRopeBytes = FMT == kCacheFp8 ? kWaves * 4 * 64 * 16 : 0;
    static constexpr int kOffMisc = kOffQRope + kQRopeBytes;
    static constexpr int kLdsBytes = kOffMisc + 512;
    static constexpr int kStageRow = kDv * 2 + 16;                     // bf16 output staging row
    static constexpr int kBtLdsMax = 2 * kBufBytes / 4;                // table entries in buffers 0, 1
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one gfx950 workgroup");
    static_assert(kHeads * kStageRow <= kOffQRope, "output staging fits the ring and the slot list");
    static_assert(kTile % kWaves == 0, "whole rows per wave");
    static_assert(kDmaPerWave * (kNBuf - 2) <= 63, "copies in flight within the vmcnt range");
    static_assert(16 + (kMaxChunk / kThreads) * kWaves <= 128, "compaction counts fit");
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

template <int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn128_kernel(const KParams p)
{
    using C = Cfg128<FMT>;
    constexpr bool kFp8 = FMT == kCacheFp8;
    constexpr int kPer = kMaxChunk / C::kThreads;   // top-k positions per thread per round

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
    //      placed where the prologue has already waited for everything)
    //      bf16: k-step ks (16 columns) holds columns 16 ks + 8 hh .. + 7.
    //      fp8:  latent k-instruction i (64 columns) holds columns
    //            64 i + 16 hh + 0..15 and 64 i + 32 + 16 hh + 0..15 (the
    //            scaled MFMA's operand order); RoPE k-step ks as bf16.
    const uint4 *qrow = (const uint4 *)(p.q + ((size_t)t * p.H + head) * kDqk);
    constexpr int kQ = 36;             // 16-byte pieces of q per lane
    u32x4 qraw[kQ];
#pragma unroll
    for (int k = 0; k < kQ; ++k) {
        uint4 w;
        if constexpr (kFp8)
            w = k < 32 ? qrow[(k >> 2) * 8 + (k & 2) * 2 + 2 * hh + (k & 1)] : qrow[64 + 2 * (k - 32) + hh];
        else
            w = qrow[2 * k + hh];
        qraw[k] = __builtin_bit_cast(u32x4, w);
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
        const int n = min(pos_end, chunk0 + kMaxChunk) - chunk0;
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
        const int chunk_n = min(kMaxChunk, pos_end - chunk0);
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
        int n_valid = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
#pragma unroll
            for (int w = 0; w < C::kWaves; ++w) {
                const int cw = __builtin_amdgcn_readlane(my_count, j * C::kWaves + w);
                if (w == wave && slotv[j] >= 0)
                    lds_slots[n_valid + __builtin_amdgcn_mbcnt_hi((uint32_t)(masks[j] >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)masks[j], 0u))] =
                        slotv[j];
                n_valid += cw;
            }
        }
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

    // q operands
    bf16x8 qb[kFp8 ? 1 : 36];          // bf16 cache: k-steps 0..35
    i32x8 qh[kFp8 ? 8 : 1], ql[kFp8 ? 8 : 1];
    int qsc[kFp8 ? 4 : 1];             // fp8: e8m0 scale of q per 128-column group (the lo term's extra
                                       // 2^-4 is the K operand's scale in its MFMA)
    // fp8: RoPE k-step ks of this lane in LDS (each lane reads back only what it wrote)
    uint8_t *const qrope = smem + C::kOffQRope + 4096 * wave + 16 * lane;
    if constexpr (!kFp8) {
#pragma unroll
        for (int k = 0; k < 36; ++k)
            qb[k] = __builtin_bit_cast(bf16x8, qraw[k]);
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            *(u32x4 *)(qrope + 1024 * ks) = qraw[32 + ks];
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            // the group's 64 values of this lane are qraw[8 G .. 8 G + 7]; the
            // largest magnitude compared on the bf16 bits (same order as the values)
            uint32_t mbits = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = qraw[8 * G + c][e];
                    mbits = max(mbits, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
                }
            }
            mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 32));   // the head's other half of the group
            // block exponent: the largest |q| of the group maps into [128, 256)
            const int ex = max((int)((mbits >> 7) & 0xFF) - 127 - 7, -120);
            const float down = __uint_as_float((uint32_t)(127 - ex) << 23);     // 2^-ex, exact
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                uint32_t hw[8], lw[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // values 32 ii + 4 j .. + 3: two words of qraw[8 G + 4 ii + j / 2]
                    const u32x4 src = qraw[8 * G + 4 * ii + (j >> 1)];
                    const uint32_t w0 = src[2 * (j & 1)], w1 = src[2 * (j & 1) + 1];
                    const float x[4] = {bf16_lo(w0) * down, bf16_hi(w0) * down, bf16_lo(w1) * down,
                                        bf16_hi(w1) * down};
                    s16x2 h = {0, 0};
                    h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[0], x[1], 1.0f, false);
                    h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[2], x[3], 1.0f, true);
                    hw[j] = __builtin_bit_cast(uint32_t, h);
                    // what the hi term misses, times 16 (the lo term's scale is 2^(ex - 4))
                    const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], 1.0f, false);
                    const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], 1.0f, true);
                    s16x2 l = {0, 0};
                    l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, (x[0] - b0[0]) * 16.f, (x[1] - b0[1]) * 16.f, 1.0f, false);
                    l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, (x[2] - b1[0]) * 16.f, (x[3] - b1[1]) * 16.f, 1.0f, true);
                    lw[j] = __builtin_bit_cast(uint32_t, l);
                }
                qh[2 * G + ii] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
                ql[2 * G + ii] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
            }
            qsc[G] = 127 + ex;
        }
    }

    // ---- per-lane LDS offsets inside a tile buffer, derived from the lane id in
    //      every tile (from late(lane): held across the tile loop instead, they and
    //      the row numbers below would take registers that q and O need)
    struct Offs {
        int k;          // K / RoPE rows for the A operand: row n32, half hh
        int v[2][2];    // V^T transposed reads: bf16 [k-step][row quad]; fp8 [k-step][0]
        int sc;         // fp8: scale of accumulator row e, group G at sc + sc_const(e) + 4 G
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
            if constexpr (kFp8) {
                // lanes 2k, 2k+1 supply row number k of the operand's 8 rows
                const int k = vj >> 1;
                const int row = 16 * ks + 8 * (k >> 2) + 4 * (vg >> 1) + (k & 3);
                f.v[ks][0] = lds_row<C>(row) + 16 * (vg & 1) + 8 * (vj & 1);
                f.v[ks][1] = 0;
            } else {
#pragma unroll
                for (int qd = 0; qd < 2; ++qd) {
                    const int row = 16 * ks + 8 * qd + 4 * (vg >> 1) + (vj >> 2);
                    f.v[ks][qd] = lds_row<C>(row) + 2 * (16 * (vg & 1) + 4 * (vj & 3));
                }
            }
        }
        // accumulator rows 8 j + i (+ 4 hh) stay inside their 16-row block, so
        // only the half's offset varies per lane
        f.sc = 4 * C::kRowStride * h2 + 512;
        f.lim_off = 4 * h2;
        return f;
    };
    auto sc_const = [](int e) { return lds_row<C>(8 * (e >> 2) + (e & 3)); };

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
    // then (a wave in tile r writes the other one), so all four waves decide alike.
    int *restart_flag = lds_misc + 2;
    if (tid == 0) {
        restart_flag[0] = 0;                   // published by the compaction's barriers
        restart_flag[1] = 0;
    }

    // One tile. kMode 0: reference from the first tile, headroom check; 1: max
    // only (no PV); 2: fixed reference. exact: P as hi + lo bf16 (two PV sweeps).
    // The LDS fragments are software-pipelined by hand: each stage reads the
    // next group's fragments while its own MFMAs run, and a scheduling barrier
    // closes every stage, so no more than two groups of fragments are ever
    // live beside q (144 registers) and the 256 accumulators of O.
    auto tile = [&](const uint8_t *buf, int n_tile, bool exact, auto mode_c, int *flag) __attribute__((always_inline)) {
        constexpr int kMode = decltype(mode_c)::value;
        const Offs f = offsets();
        const int off_k = f.k, off_sc = f.sc;
        f32x16 acc = {};
        if constexpr (!kFp8) {
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
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < KG; ++j)
                    cur[j] = nxt[j];
            }
        } else {
            // stage i (k-instruction i, 64 columns of group i / 2): its K fragment
            // was read one stage ahead; the group's 16 row scales are read at the
            // start of its second stage and applied after that stage's MFMAs
            auto load_k = [&](int i) __attribute__((always_inline)) -> i32x8 {
                const uint4 a0 = *(const uint4 *)(buf + off_k + 64 * i);
                const uint4 a1 = *(const uint4 *)(buf + off_k + 64 * i + 32);
                return i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            };
            i32x8 kc = load_k(0), kn;
            f32x16 part = {};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int G = i >> 1;
                if (i < 7)
                    kn = load_k(i + 1);
                float scc[16];
                if (i & 1) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        scc[e] = *(const float *)(buf + off_sc + sc_const(e) + 4 * G);
                }
                part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kc, qh[i], (i & 1) ? part : f32x16{}, 0, 0, 0,
                                                                       127, 0, qsc[G]);
                part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kc, ql[i], part, 0, 0, 0, 123, 0, qsc[G]);
                if (i & 1) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[e] = fmaf(scc[e], part[e], acc[e]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (i < 7)
                    kc = kn;
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = *(const bf16x8 *)(buf + off_k + RowFmt<kCacheFp8>::kRope + 32 * ks);
                const bf16x8 b = *(const bf16x8 *)(smem + C::kOffQRope + 4096 * wave + 16 * late(lane) + 1024 * ks);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
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
        lmax = fmaxf(lmax, __shfl_xor(lmax, 32)) * c2;
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
        //      Stages of four (dim block, k-step) pairs, the next stage's V^T
        //      fragments read while the current MFMAs run.
        using VFrag = std::conditional_t<kFp8, uint2, uint4>;
        auto load_v = [&](int db, int ks) __attribute__((always_inline)) -> VFrag {
            if constexpr (kFp8) {
                const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, buf + f.v[ks][0] + 32 * db));
                return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
            } else {
                const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(i16x4, buf + f.v[ks][0] + 64 * db)));
                const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(i16x4, buf + f.v[ks][1] + 64 * db)));
                return make_uint4(w0.x, w0.y, w1.x, w1.y);
            }
        };
        // dim blocks db0 .. db0 + 3, both k-steps: 8 MFMAs with the weights p
        auto pv_group = [&](int db0, const bf16x8 (&pp)[2]) __attribute__((always_inline)) {
            VFrag vc[4], vn[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vc[j] = load_v(db0 + (j >> 1), j & 1);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                if (h2 == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        vn[j] = load_v(db0 + 2 + (j >> 1), j & 1);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int db = db0 + 2 * h2 + (j >> 1), ks = j & 1;
                    bf16x8 a;
                    if constexpr (kFp8)
                        a = e4m3x8_to_bf16x8(vc[j]);
                    else
                        a = __builtin_bit_cast(bf16x8, vc[j]);
                    mfma_o(o[db], a, pp[ks]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (h2 == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        vc[j] = vn[j];
                }
            }
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
        bf16x8 pp[2];
        if constexpr (!kFp8) {
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                if (pass == 1 && !exact)
                    break;
                pack(pw, pass == 1, pp);
#pragma unroll
                for (int db0 = 0; db0 < 16; db0 += 4)
                    pv_group(db0, pp);
            }
        } else {
            // output group G (dims 128 G ..): the weights carry the rows' group-G scales
#pragma unroll
            for (int G = 0; G < 4; ++G) {
                float ws[16];
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    ws[e] = pw[e] * *(const float *)(buf + off_sc + sc_const(e) + 4 * G);
#pragma unroll
                for (int pass = 0; pass < 2; ++pass) {
                    if (pass == 1 && !exact)
                        break;
                    pack(ws, pass == 1, pp);
                    pv_group(4 * G, pp);
                }
            }
        }
    };

    // ---- the list, one round of up to kMaxChunk positions at a time. Returns
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
            for (int r = 0; r < n_tiles; ++r) {
                // this wave's rows of tile r have landed ...
                wait_vmcnt(C::kDmaPerWave * (issued - r - 1));
                // ... and every wave's; every wave is done with tile r - 1
                __syncthreads();
                if (kMode == 0 && restart_flag[(r + 1) & 1] != 0) {
                    stop = true;
                    break;
                }
                if (issued < n_tiles) {
                    issue_tile<C>(p.cache, lds_slots + issued * kTile, min(kTile, n_valid - issued * kTile),
                                  ring + (issued % C::kNBuf) * C::kBufBytes, wave, lane);
                    ++issued;
                }
                tile(ring + (r % C::kNBuf) * C::kBufBytes, min(kTile, n_valid - r * kTile), exact_p, mode_c,
                     restart_flag + (r & 1));
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies of tiles a stop left unread
            __syncthreads();     // ring and slot list are free for the next round
            if (kMode == 0 && (stop || (restart_flag[0] | restart_flag[1]) != 0))
                return true;
            chunk0 += kMaxChunk;
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

    // ---- epilogue: the head's row sum (this lane's rows and the other half's)
    o_settle(o);
    const float l = l_part + __shfl_xor(l_part, 32);
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    // natural-log lse (v_log_f32 is log2; l >= 1 here: the row that set the max adds >= 1)
    const float lse_v = l > 0.f ? (m_ref + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
    if (!p.partials) {
        // bf16 rows staged in LDS (ring free), then written out coalesced
        uint8_t *stage = smem;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v0 = o[db][4 * j] * inv_l, v1 = o[db][4 * j + 1] * inv_l;
                const float v2 = o[db][4 * j + 2] * inv_l, v3 = o[db][4 * j + 3] * inv_l;
                *(uint2 *)(stage + head * C::kStageRow + 2 * (32 * db + 8 * j + 4 * hh)) =
                    make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
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
        float *po = p.part_o + (((size_t)t * p.S + s) * p.H + head) * kDv;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *(f32x4 *)(po + 32 * db + 8 * j + 4 * hh) =
                    f32x4{o[db][4 * j] * inv_l, o[db][4 * j + 1] * inv_l, o[db][4 * j + 2] * inv_l,
                          o[db][4 * j + 3] * inv_l};
        }
        if (hh == 0)
            p.part_lse[((size_t)t * p.S + s) * p.H + head] = lse_v;
    }
}

}  // namespace

hipError_t launch_attn128(CacheFormat fmt, const KParams &p, hipStream_t stream)
{
    const int64_t tq = (p.T + 7) / 8;
    const dim3 grid((unsigned)(tq * 8 * p.S));
    if (fmt == kCacheFp8)
        hipLaunchKernelGGL(attn128_kernel<kCacheFp8>, grid, dim3(Cfg128<kCacheFp8>::kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(attn128_kernel<kCacheBf16>, grid, dim3(Cfg128<kCacheBf16>::kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace smla
