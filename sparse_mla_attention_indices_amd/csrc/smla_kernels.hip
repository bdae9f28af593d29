// smla_kernels.hip -- CDNA4 (gfx950) kernels for sparse MLA forward over top-k
// indices: index conversion, the fused gather -> QK^T -> online softmax -> PV
// attention kernel, and the log-sum-exp merge of top-k splits.
//
// What is computed follows the vLLM page "vllm/v1/attention/backends/mla/
// flashmla_sparse.py" (FLASHMLA_SPARSE backend): the index conversion of
// triton_convert_req_index_to_global_index (docstring and kernel), the
// fp8_ds_mla row format of the module note, and the multi-query attention with
// 576-wide keys and 512-wide values that FlashMLASparseImpl.forward runs for
// both cache formats. How it is computed here is this library's own design for
// 64-wide wavefronts, MFMA and the 160 KB LDS of a gfx950 compute unit.
//
// attn_pc_kernel (fp8 cache, 64 heads per workgroup, the decode batches) gives
// each SIMD one QK^T wave (16 heads over all 576 columns: S^T, online softmax,
// P^T into LDS) and one PV wave (128 output dims of all 64 heads), PV one tile
// behind QK^T; it is described where it is defined. attn_kernel covers the
// bf16 cache and 16- or 32-head fp8 workgroups:
//
//  * Workgroup = one query token x 16, 32 or 64 heads x one part ("split") of
//    the token's top-k list. Every wave owns 16 heads and one half of the 576
//    columns ("dh"), so a 64-head workgroup has eight waves, two per SIMD, and
//    each wave stays within 256 registers.
//  * Prologue: the indices and q are requested together, the block-table
//    lookups as soon as the indices arrive, and q is prepared while those are in
//    flight. The valid slots are compacted into LDS: runs of -1 cost nothing,
//    only the last tile is ragged.
//  * Gather: global_load_lds_dwordx4 copies the cache rows of a 32-row tile,
//    as stored (fp8_ds_mla 656 B or bf16 1152 B), one row per wave instruction,
//    straight into one of a ring of LDS buffers; the next tiles are in flight
//    while one is used.
//  * QK^T runs transposed, S^T = K q^T, with q in registers. fp8: the raw e4m3
//    K bytes feed v_mfma_scale_f32_16x16x128_f8f6f4 against q written as hi + lo
//    e4m3 terms (exact for elements within 2^13 of their group's largest, an
//    absolute error below 2^-21 of it otherwise); each 128-column group's partial
//    sum is multiplied by
//    that group's row scales in fp32. bf16: v_mfma_f32_16x16x32_bf16. The two
//    column halves add their partial S^T through LDS.
//  * Softmax: the S^T accumulator layout gives a lane one head and four rows
//    per block, and the weights are already in the B-operand layout of
//    O^T += V^T P^T. The running max moves (and O is rescaled) only when a tile
//    exceeds it by 2^8; the test uses each lane's own rows, so the common case
//    needs no cross-lane step. Row sums stay per lane until the end.
//  * PV reads V straight from the row-major raw tile with the gfx950 LDS
//    transpose loads (ds_read_b64_tr_b8 for fp8, ds_read_b64_tr_b16 for bf16).
//    For fp8 the weights of each 128-wide output group carry that group's row
//    scales, so dequantisation adds no rounding anywhere. A short list (few
//    valid rows, so large weights) feeds P as two bf16 terms, hi + lo. With
//    fp8 and several head blocks, PV of one tile runs in the same phase as QK^T
//    of the next.
//  * Output: one split writes the bf16 rows and lse; a top-k split writes its
//    fp32 partial (O / l) and lse, and merge_kernel, launched after it on the
//    same stream, combines the parts in index order.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {


// Compile-time shape of one instantiation: NHH groups of 16 heads, two waves
// (column halves) per group.
//
// A tile's rows sit in LDS as stored in HBM, but with a row stride and a gap
// after every 16 rows chosen so that the LDS reads of one instruction spread
// over distinct banks: fp8 rows keep their 656-byte stride (16 consecutive rows
// fall on distinct banks) and rows 16..31 start 16 bytes later than a plain
// stride would put them (the transposed V reads touch rows r and r + 16
// together); bf16 rows get a 1168-byte stride (1152 + 16). nvfp4 rows keep
// their 352-byte stride in the ring; their latent values, dequantised to bf16
// as QK^T reads them, are stored in a tile laid out as the bf16 cache's
// (kOffConv), which PV reads V^T from.
template <int FMT, int NHH>
struct Cfg {
    static constexpr int kWaves = 2 * NHH;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kHeads = 16 * NHH;                          // heads per workgroup
    static constexpr int kRowBytes = RowFmt<FMT>::kBytes;            // bytes of a row in HBM
    static constexpr int kChunksPerRow = kRowBytes / 16;             // 16-byte pieces per row
    static constexpr int kRowStride = FMT == kCacheBf16 ? kRowBytes + 16 : kRowBytes;  // in LDS
    static constexpr int kBlockGap = FMT == kCacheFp8 ? 16 : 0;
    static constexpr int kRowBlockBytes = 16 * kRowStride + kBlockGap;                 // 16 rows
    // Tile copies: one wave instruction moves 64 16-byte pieces of one row, so
    // a row takes kInstrPerRow of them; each wave copies kRowsPerWave rows.
    static constexpr int kInstrPerRow = (kChunksPerRow + 63) / 64;
    static constexpr int kRowsPerWave = kTile / kWaves;
    static constexpr int kDmaPerWave = kRowsPerWave * kInstrPerRow;  // wave instructions per tile
    static constexpr int kBufBytes = (kRB * kRowBlockBytes + 1023) / 1024 * 1024;   // ring buffer stride
    // 64 heads: one workgroup per CU; fewer heads: two workgroups per CU
    // share the LDS (fp8).
    static constexpr int kNBuf = NHH == 4 ? (FMT == kCacheFp8 ? 4 : 2) : 2;
    // nvfp4: the bf16 tile the latent values are stored into for PV
    static constexpr int kConvBytes = FMT == kCacheNvfp4 ? Cfg<kCacheBf16, NHH>::kBufBytes : 0;
    // PV is split by output dims: wave w owns dims [w * kDimsPerWave, ...) of
    // every head of the workgroup, kDimBlocks blocks of 16 dims.
    static constexpr int kDimsPerWave = kDv / kWaves;
    static constexpr int kDimBlocks = kDimsPerWave / 16;
    static_assert(NHH * kDimBlocks == 16, "sixteen 16x16 output blocks per wave");
    static constexpr int kXchgBytes = kWaves * kRB * 1024;           // partial S^T exchange
    // P^T operands per (scale group, head block): hi and lo terms, 1 KB each
    static constexpr int kPBytes = NHH > 1 ? 2 * 4 * NHH * 1024 : 0;
    // top-k positions compacted into LDS per round (1024: halving it cost the
    // 16-head decode 4-5 % at top-k 2048, whose parts then take two rounds)
    static constexpr int kChunk = 1024;
    static constexpr int kSlotsBytes = kChunk * 4;
    static constexpr int kOffConv = kNBuf * kBufBytes;
    static constexpr int kOffXchg = kOffConv + kConvBytes;
    static constexpr int kOffP = kOffXchg + kXchgBytes;
    static constexpr int kOffSlots = kOffP + kPBytes;
    static constexpr int kOffMisc = kOffSlots + kSlotsBytes;         // compaction counts
    static constexpr int kOffHead = kOffMisc + 512;                  // per-head factors, rescale flags
    // (64 heads: the fp32 output staging needs more than the loop's regions)
    static constexpr int kLdsBytes = kOffHead + 1024 > kHeads * (kDv + 4) * 4 ? kOffHead + 1024 : kHeads * (kDv + 4) * 4;
    static_assert(kRowBlockBytes % 16 == 0, "row blocks are whole 16-byte slots");
    static_assert(kRB * kRowBlockBytes <= kBufBytes, "a tile fits its ring buffer");
    static_assert(kTile % kWaves == 0 && kRowsPerWave <= 64, "whole rows per wave");
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one gfx950 workgroup");
    static_assert(kHeads * kDv * 2 <= kLdsBytes, "bf16 output staging fits");
    static_assert(kHeads * (kDv + 4) * 4 <= kLdsBytes, "fp32 partial staging fits");
    static_assert(16 + (kChunk / kThreads) * kWaves <= 128, "compaction counts fit");
};


// ------------------------------------------------------------- attention

template <int FMT, int NHH>
__global__ __launch_bounds__(128 * NHH) __attribute__((amdgpu_waves_per_eu(NHH == 1 ? 1 : 2)))
void attn_kernel(const KParams p)
{
    using C = Cfg<FMT, NHH>;
    // the layout the MFMA operands are read in: nvfp4 latent values are
    // dequantised to bf16 as QK^T reads them and stored in that layout for PV
    constexpr int TF = FMT == kCacheNvfp4 ? kCacheBf16 : FMT;
    using CT = Cfg<TF, NHH>;
    constexpr int RB = kRB;
    constexpr int RS = CT::kRowStride;
    constexpr int RBB = CT::kRowBlockBytes;
    constexpr int kPer = C::kChunk / C::kThreads;    // top-k positions per thread per round
    static_assert(FMT != kCacheNvfp4 || NHH == 1, "nvfp4 runs 16-head workgroups");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
    uint8_t *ring = smem;
    f32x4 *xchg = (f32x4 *)(smem + C::kOffXchg);
    int32_t *lds_slots = (int32_t *)(smem + C::kOffSlots);
    int32_t *lds_misc = (int32_t *)(smem + C::kOffMisc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, n16 = lane & 15;
    const int dh = wave & 1, hh = wave >> 1;

    // Workgroup id -> (token, split, head block); all workgroups of one token
    // get the same id mod 8, the XCD the hardware dispatches them to.
    int bid = blockIdx.x;
    const int xcd = bid & 7;
    bid >>= 3;
    const int hb_wg = bid % p.HB;
    bid /= p.HB;
    const int s = bid % p.S;
    const int t = (bid / p.S) * 8 + xcd;
    if (t >= p.T)
        return;

    const int wg_head0 = hb_wg * C::kHeads;
    const int head = wg_head0 + 16 * hh + n16;      // this lane's head
    const float c2 = p.log2e_scale;
    const int32_t *topk_row = p.topk + (size_t)t * p.K;
    const int req = p.slot_in ? 0 : p.req_id[t];

    // q^T B operands. bf16 cache: lane (head, group g) holds 8 columns per
    // k-step of v_mfma_f32_16x16x32_bf16: latent 256*dh + 32k + 8g (k < 8), RoPE
    // 512 + 32*dh + 8g (k = 8). fp8 cache: the RoPE step is the same (qb[8]); the
    // latent goes through v_mfma_scale_f32_16x16x128_f8f6f4 on the raw e4m3 K
    // bytes, so q is written as hi + lo e4m3 terms with a power-of-two scale per
    // head and 128-column group (exact for elements within 2^13 of the group's
    // largest; below that hi and lo fall into e4m3's subnormal steps and the
    // absolute error stays below 2^-21 of the largest): lane (head, g) holds
    // columns 128*(2*dh + gi) + 32g .. +31.
    bf16x8 qb[9];
    i32x8 qh[2], ql[2];         // fp8: hi and lo e4m3 terms of the 32 columns
    int qsh[2], qsl[2];         // fp8: their e8m0 block scales (2^(e - 127))

    const int pos_begin = s * p.split_len;
    const int pos_end = min(p.K, pos_begin + p.split_len);

    constexpr int DB = C::kDimBlocks;
    // O^T, 16 blocks: o[hb * DB + db] holds dims dim0 + 16*db + 4g + i of head
    // 16*hb + n16 of the workgroup, dim0 = wave * kDimsPerWave
    f32x4 o[16];
    const int dim0 = wave * C::kDimsPerWave;
    float m_run, l_part;    // head block hh: log2-domain running max (same in a head's 4 lanes), lane's row sum
    float *head_f = (float *)(smem + C::kOffHead);           // [4][16] per-head factors
    int *resc_flag = (int *)(smem + C::kOffHead + 256);      // [4] head block moved its max this tile
    float *alpha_lds = (float *)(smem + C::kOffHead + 512);  // [4][16] rescale factors

    // fp8 with several head blocks runs software-pipelined: one phase of the
    // tile loop does PV of tile i - 1 (its V^T fragments were read into
    // registers before the previous exchange, its P^T waits in LDS) together
    // with QK^T of tile i, so two independent MFMA chains interleave and a
    // tile needs two barriers instead of three.
    constexpr bool kPipe = FMT == kCacheFp8 && NHH > 1;
    bf16x8 *p_lds = (bf16x8 *)(smem + C::kOffP);          // [lo][group][head block][lane]
    uint2 vf8_pend[DB];         // pipelined fp8: V^T fragments of the tile whose PV is pending

    // PV, part 1 (after the barrier that publishes P^T): rescale O for head
    // blocks whose max moved, and in exact mode add the lo terms of P.
    // flags / al: resc_flag and alpha_lds of the pending tile, read right after
    // the barrier so their latency overlaps the copy issue.
    auto pv_pre = [&](const uint2 *vf, bool exact, const int *flags, const float *al_in) __attribute__((always_inline)) {
        const int G = dim0 >> 7;                                // scale group of this wave's dims
#pragma unroll
        for (int hb = 0; hb < NHH; ++hb) {
            if (flags[hb]) {
                const float al = al_in[hb];
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[hb * DB + db] *= al;
            }
        }
        if (exact) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 a = e4m3x8_to_bf16x8(vf[db]);
#pragma unroll
                for (int hb = 0; hb < NHH; ++hb)
                    o[hb * DB + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, p_lds[((4 + G) * NHH + hb) * 64 + lane], o[hb * DB + db], 0, 0, 0);
            }
        }
    };
    // PV, part 2: O^T += V^T P^T (hi terms) over dim blocks [db0, db1) of this
    // wave's dims, branch-free; pv: the P^T operands (pv_load).
    auto pv_load = [&](bf16x8 *pv) __attribute__((always_inline)) {
        const int G = dim0 >> 7;
#pragma unroll
        for (int hb = 0; hb < NHH; ++hb)
            pv[hb] = p_lds[(G * NHH + hb) * 64 + lane];
    };
    auto pv_part = [&](const uint2 *vf, const bf16x8 *pv, int db0, int db1) __attribute__((always_inline)) {
#pragma unroll
        for (int db = db0; db < db1; ++db) {
            const bf16x8 a = e4m3x8_to_bf16x8(vf[db]);
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb)
                o[hb * DB + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pv[hb], o[hb * DB + db], 0, 0, 0);
        }
    };

    // One tile: S^T = K q^T, online softmax, O^T += V^T P^T. exact: P enters PV
    // as hi + lo bf16 terms (wave-uniform). Pipelined: the tile stops after
    // publishing P^T; its PV runs in the next phase. mid(gi) runs right after
    // the QK^T MFMAs of column group gi are issued (fp8), so independent work
    // (the pending PV) can fill the wait for their results.
    auto tile = [&](const uint8_t *buf, int n_tile, bool exact, auto &&mid) __attribute__((always_inline)) {
        // V^T is read from the tile itself, or for nvfp4 from the bf16 values
        // this wave stored while converting its K fragments (same layout)
        const uint8_t *vbuf = FMT == kCacheNvfp4 ? smem + C::kOffConv : buf;
        // per-lane LDS offsets inside the tile buffer
        const int off_k = n16 * RS;                      // K rows 16*rb + n16 (+ rb * RBB)
        const int off_sc = (4 * g) * RS;                 // accumulator rows 16*rb + 4g + i
        // fp8 V^T (ds_read_b64_tr_b8): source lane n16 = 2k + h reads row k of
        // {4g..4g+3, 16+4g..16+4g+3}, bytes 8h..8h+7 of a 16-byte column block
        const int vk = n16 >> 1;
        const int off_v8 = (vk >> 2) * RBB + (4 * g + (vk & 3)) * RS + 8 * (n16 & 1);
        // bf16 V^T (ds_read_b64_tr_b16): source lane n16 = 4k + a reads row 4g + k
        // (and 16 + 4g + k), dims 4a..4a+3 of a 16-dim block
        const int off_v16 = (4 * g + (n16 >> 2)) * RS + 8 * (n16 & 3);

        // ---- S^T over this wave's column half for head block hh (K rows
        //      16*rb + n16; accumulator rows 16*rb + 4g + i)
        f32x4 acc[RB];
        f32x4 sc[2][RB];        // fp8: scales of rows 16*rb + 4g + i, groups 2*dh + gi
        uint2 vf8[DB];          // fp8: V^T fragments of this wave's dims, read before the exchange
        if constexpr (FMT == kCacheFp8) {
            bf16x8 rf[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                rf[rb] = *(const bf16x8 *)(buf + rb * RBB + off_k + RowFmt<TF>::kRope + 64 * dh + 16 * g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float2 v = *(const float2 *)(buf + rb * RBB + off_sc + i * RS + 512 + 8 * dh);
                    sc[0][rb][i] = v.x;
                    sc[1][rb][i] = v.y;
                }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                // raw e4m3 K bytes of column group 2*dh + gi: row 16*rb + n16,
                // columns 32g .. 32g + 31 of the group
                i32x8 kf[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint4 *src = (const uint4 *)(buf + rb * RBB + off_k + 128 * (2 * dh + gi) + 32 * g);
                    const uint4 a0 = src[0], a1 = src[1];
                    kf[rb] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                }
                f32x4 part[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    part[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        kf[rb], qh[gi], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, qsh[gi]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    part[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        kf[rb], ql[gi], part[rb], 0, 0, 0, 127, 0, qsl[gi]);
                mid(gi);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb] += sc[gi][rb] * part[rb];
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf[rb], qb[8], acc[rb], 0, 0, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    LDS_PTR(i32x2, buf + off_v8 + dim0 + 16 * db));
                vf8[db] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
            }
        } else if constexpr (FMT == kCacheNvfp4) {
            // raw rows (ring layout C). Lane (n16, g) turns the 8 latent codes of
            // row 16*rb + n16, columns 256*dh + 32*k + 8*g .. + 7, into bf16: each
            // code to fp32, times its 16-value block's E4M3 scale, to bf16 (exact at
            // every step: E2M1 x E4M3 has at most 6 significant bits; the scaled
            // conversions would apply only the scale's exponent). The fragment
            // feeds the MFMA and is stored where the bf16 layout puts it, so this
            // wave's PV reads V^T of its own dims from there: no other wave
            // touches those columns, and the next tile's stores follow this
            // tile's reads in the wave's program order.
            using F = RowFmt<kCacheNvfp4>;
            const uint8_t *row_b[RB];
            uint4 scw[RB];          // the row's scales 16*dh .. 16*dh + 15 (this half's blocks)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                row_b[rb] = buf + lds_row<C>(16 * rb + n16);
                scw[rb] = *(const uint4 *)(row_b[rb] + F::kScales + 16 * dh);
                acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const bool odd_blk = (g >> 1) != 0;     // columns 8g.. of a 32-column step: block 2k + (g >> 1)
            // every code word and the RoPE bytes first: the stores below go to
            // another LDS region, which the compiler cannot tell, so a read
            // after a store would wait for it
            uint32_t code_w[8][RB];
            uint2 rope_w[RB];
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    code_w[k][rb] = *(const uint32_t *)(row_b[rb] + 128 * dh + 16 * k + 4 * g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                rope_w[rb] = *(const uint2 *)(row_b[rb] + F::kRope + 32 * dh + 8 * g);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint32_t codes = code_w[k][rb];
                    const uint32_t sw = k < 2 ? scw[rb].x : k < 4 ? scw[rb].y : k < 6 ? scw[rb].z : scw[rb].w;
                    const f32x2 s2 = (k & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, true)
                                             : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
                    const float scl = odd_blk ? s2[1] : s2[0];
                    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
                    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
                    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
                    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
                    const uint4 w = make_uint4(pack_bf16(f0[0] * scl, f0[1] * scl), pack_bf16(f1[0] * scl, f1[1] * scl),
                                               pack_bf16(f2[0] * scl, f2[1] * scl), pack_bf16(f3[0] * scl, f3[1] * scl));
                    *(uint4 *)(smem + C::kOffConv + rb * RBB + off_k + 2 * (256 * dh + 32 * k + 8 * g)) = w;
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), qb[k],
                                                                      acc[rb], 0, 0, 0);
                }
            }
            // RoPE: 8 E4M3 bytes per lane, exact in bf16
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(rope_w[rb]), qb[8], acc[rb], 0, 0, 0);
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const int col = k < 8 ? 2 * (256 * dh + 32 * k + 8 * g) : RowFmt<TF>::kRope + 64 * dh + 16 * g;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const bf16x8 a = *(const bf16x8 *)(buf + rb * RBB + off_k + col);
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[k], acc[rb], 0, 0, 0);
                }
            }
        }

        // ---- add the other column half's partial S^T (same lane slots)
        if constexpr (kPipe)
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            xchg[(wave * RB + rb) * 64 + lane] = acc[rb];
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            acc[rb] += xchg[((wave ^ 1) * RB + rb) * 64 + lane];

        // ---- online softmax of head block hh in log2 units. The running max
        //      moves only when some row exceeds it by 2^8 (tested on each lane's
        //      own rows, moved to the whole head's max).
        // (the scale c2 > 0 is applied to the maximum here and inside the exp2
        // argument below: max(c2 * a) = c2 * max(a) exactly)
        float lmax = -INFINITY;
        if (n_tile == kTile) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lmax = fmaxf(lmax, acc[rb][i]);
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[rb][i] = 16 * rb + 4 * g + i < n_tile ? acc[rb][i] : -INFINITY;
                    lmax = fmaxf(lmax, acc[rb][i]);
                }
        }
        lmax *= c2;
        bool moved = false;
        float alpha = 1.f;
        if (__ballot(lmax > m_run + kLazyRescale) != 0) {
            const float mx = xor32_max(xor16_max(lmax));
            if (mx > m_run + kLazyRescale) {
                alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
                l_part *= alpha;
                m_run = mx;
            }
            moved = true;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[rb][i] = __builtin_amdgcn_exp2f(fmaf(acc[rb][i], c2, -m_run));
                l_part += acc[rb][i];
            }

        // ---- P^T operands. fp8: the weights for output group G carry that
        //      group's row scales; this wave has the scales of groups 2*dh, 2*dh+1.
        bf16x8 pbh[2], pbl[2];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            f32x4 p0 = acc[0], p1 = acc[1];
            if constexpr (FMT == kCacheFp8) {
                p0 *= sc[gi][0];
                p1 *= sc[gi][1];
            }
            pbh[gi] = pack_p(p0, p1);
            if (exact)
                pbl[gi] = pack_p_residual(p0, p1, pbh[gi]);
        }

        if constexpr (NHH == 1) {
            // one head block: this wave's dims are groups 2*dh, 2*dh + 1 and it
            // holds their operands itself
            if (moved) {
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    o[k] *= alpha;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int gi = db >> 3;
                bf16x8 a;
                if constexpr (FMT == kCacheFp8) {
                    a = e4m3x8_to_bf16x8(vf8[db]);
                } else {
                    const int colb = 2 * (dim0 + 16 * db);
                    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, vbuf + off_v16 + colb)));
                    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, vbuf + RBB + off_v16 + colb)));
                    a = __builtin_bit_cast(bf16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
                }
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pbh[gi], o[db], 0, 0, 0);
                if (exact)
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pbl[gi], o[db], 0, 0, 0);
            }
        } else {
            // ---- hand P^T of head block hh for groups 2*dh, 2*dh + 1 (and the
            //      rescale factor when the max moved) to the waves owning those dims
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                p_lds[((2 * dh + gi) * NHH + hh) * 64 + lane] = pbh[gi];
                if (exact)
                    p_lds[((4 + 2 * dh + gi) * NHH + hh) * 64 + lane] = pbl[gi];
            }
            if (dh == 0) {
                if (lane == 0)
                    resc_flag[hh] = moved ? 1 : 0;
                if (moved && g == 0)
                    alpha_lds[hh * 16 + n16] = alpha;
            }
            if constexpr (kPipe) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    vf8_pend[db] = vf8[db];
                return;
            }
            __syncthreads();
            // ---- O^T += V^T P^T over this wave's dims for every head block
            const int G = dim0 >> 7;                                // scale group of this wave's dims
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb) {
                if (resc_flag[hb]) {
                    const float al = alpha_lds[hb * 16 + n16];
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        o[hb * DB + db] *= al;
                }
            }
            bf16x8 pv[NHH];
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb)
                pv[hb] = p_lds[(G * NHH + hb) * 64 + lane];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x8 a;
                if constexpr (FMT == kCacheFp8) {
                    a = e4m3x8_to_bf16x8(vf8[db]);
                } else {
                    const int colb = 2 * (dim0 + 16 * db);
                    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, vbuf + off_v16 + colb)));
                    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, vbuf + RBB + off_v16 + colb)));
                    a = __builtin_bit_cast(bf16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
                }
#pragma unroll
                for (int hb = 0; hb < NHH; ++hb)
                    o[hb * DB + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pv[hb], o[hb * DB + db], 0, 0, 0);
                if (exact) {
#pragma unroll
                    for (int hb = 0; hb < NHH; ++hb)
                        o[hb * DB + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a, p_lds[((4 + G) * NHH + hb) * 64 + lane], o[hb * DB + db], 0, 0, 0);
                }
            }
        }
    };

    float inv_l_hb[NHH];        // per head block: 1 / l of head 16*hb + n16
    float lse_hb[NHH];          // and its natural-log lse
    {
        // the first round's indices first: their round trip overlaps q's
        int idxv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = pos_begin + tid + C::kThreads * j;
            idxv[j] = i < min(pos_end, pos_begin + C::kChunk) ? topk_row[i] : -1;
        }
        // q's raw bytes are loaded now and worked on once the first round's
        // block-table lookups are in flight.
        const uint16_t *qrow = p.q + ((size_t)t * p.H + head) * kDqk;
        uint4 qraw[9];      // fp8: [4 * gi + c] latent, [8] RoPE; bf16: k-steps 0..8
        if constexpr (FMT == kCacheFp8) {
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    qraw[4 * gi + c] = ((const uint4 *)(qrow + 128 * (2 * dh + gi) + 32 * g))[c];
            qraw[8] = *(const uint4 *)(qrow + 512 + 32 * dh + 8 * g);
        } else {
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                const int col = k < 8 ? 256 * dh + 32 * k + 8 * g : 512 + 32 * dh + 8 * g;
                qraw[k] = *(const uint4 *)(qrow + col);
            }
        }
        int slotv[kPer];    // block-table entries until q is done, then slots
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            slotv[j] = p.slot_in ? 0 : lookup_block(req, idxv[j], p.bt, p.R, p.MB);
        {
            // each q value is used here, so the compiler waits for these loads
            // before the tile loop rather than inside it (it cannot see the
            // explicit waits that order the tile copies)
#pragma unroll
            for (int k = 0; k < 9; ++k)
                asm volatile("" : "+v"(qraw[k].x), "+v"(qraw[k].y), "+v"(qraw[k].z), "+v"(qraw[k].w));
            if constexpr (FMT == kCacheFp8) {
                qb[8] = __builtin_bit_cast(bf16x8, qraw[8]);
#pragma unroll
                for (int gi = 0; gi < 2; ++gi) {
                    float v[32];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 w = qraw[4 * gi + c];
                        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[8 * c + 2 * e] = bf16_lo(ww[e]);
                            v[8 * c + 2 * e + 1] = bf16_hi(ww[e]);
                        }
                    }
                    float amax = 0.f;
#pragma unroll
                    for (int i = 0; i < 32; ++i)
                        amax = fmaxf(amax, fabsf(v[i]));
                    // the MFMA applies one B scale per column (head) to all 128 k of the
                    // group, so the exponent is shared by the head's four lanes
                    amax = xor32_max(xor16_max(amax));
                    // block exponent: the largest |q| maps into [128, 256), within e4m3's range
                    const int ex = max((int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 7, -120);
                    // the conversions apply the powers of two themselves (fp8 = x / scale
                    // rounded, f32 = fp8 x scale; both exact): hi in units of 2^ex, and
                    // what it misses, exactly, in units of 2^(ex - 4)
                    const float up_hi = __uint_as_float((uint32_t)(127 + ex) << 23);      // 2^ex
                    const float up_lo = __uint_as_float((uint32_t)(127 + ex - 4) << 23);  // 2^(ex - 4)
                    uint32_t hw[8], lw[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float *x = v + 4 * j;
                        s16x2 h = {0, 0};
                        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[0], x[1], up_hi, false);
                        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[2], x[3], up_hi, true);
                        hw[j] = __builtin_bit_cast(uint32_t, h);
                        const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], up_hi, false);
                        const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], up_hi, true);
                        s16x2 l = {0, 0};
                        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x[0] - b0[0], x[1] - b0[1], up_lo, false);
                        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x[2] - b1[0], x[3] - b1[1], up_lo, true);
                        lw[j] = __builtin_bit_cast(uint32_t, l);
                    }
                    qh[gi] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
                    ql[gi] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
                    qsh[gi] = 127 + ex;
                    qsl[gi] = 127 + ex - 4;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 9; ++k)
                    qb[k] = __builtin_bit_cast(bf16x8, qraw[k]);
            }
        }
        // finish the lookups only now: tied to the last q operand, the wait for
        // the block-table loads is not scheduled into the q arithmetic above
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if constexpr (FMT == kCacheFp8)
                asm volatile("" : "+v"(slotv[j]) : "v"(ql[0]), "v"(ql[1]));
            slotv[j] = p.slot_in ? given_slot(idxv[j], p.NB) : finish_slot(slotv[j], req, idxv[j], p.R, p.MB, p.NB);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k)
            o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_part = 0.f;
        // the workgroups of head block 0 write the converted slots
        const bool write_phys = p.phys_out != nullptr && hb_wg == 0;


        for (int chunk0 = pos_begin; chunk0 < pos_end; chunk0 += C::kChunk) {
            const int chunk_n = min(C::kChunk, pos_end - chunk0);

            // ---- convert (all lookups in flight together), then compact the valid
            //      slots in list order with one exchange of per-wave counts
            if (chunk0 != pos_begin) {
                // a later round of a long list: its indices, then their slots (loaded
                // here, so no load is left in flight across the tile loop)
#pragma unroll
                for (int j = 0; j < kPer; ++j) {
                    const int i = chunk0 + tid + C::kThreads * j;
                    idxv[j] = i < pos_end ? topk_row[i] : -1;
                }
#pragma unroll
                for (int j = 0; j < kPer; ++j)
                    slotv[j] = p.slot_in ? given_slot(idxv[j], p.NB)
                                         : finish_slot(lookup_block(req, idxv[j], p.bt, p.R, p.MB), req,
                                                       idxv[j], p.R, p.MB, p.NB);
            }
            if (write_phys) {
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
            // all counts in one read (lane i holds count i), then taken as scalars:
            // no chain of dependent LDS round trips
            const int my_count = lds_misc[16 + (lane & 31)];
            int base[kPer];
            const int n_valid = compaction_bases<kPer, C::kWaves>(my_count, wave, base);
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (slotv[j] >= 0)
                    lds_slots[base[j] + lanes_below(masks[j])] = slotv[j];
            __syncthreads();
            const bool exact_p = n_valid <= kExactPRows;
            const int n_tiles = (n_valid + kTile - 1) / kTile;
            // from here on the only vector-memory instructions in flight are tile copies
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // this wave's copy instructions per tile
            constexpr int dma_w = C::kDmaPerWave;

            for (int i = 0; i < min(C::kNBuf - 1, n_tiles); ++i)
                issue_tile<C>(p.cache, lds_slots + i * kTile, min(kTile, n_valid - i * kTile),
                              ring + i * C::kBufBytes, wave, lane);

            if constexpr (kPipe) {
                // the PV pending before the first tile adds nothing: zero weights,
                // zero fragments, no rescale (ordered before any read by the first
                // barrier below)
#pragma unroll
                for (int k = wave; k < 2 * 4 * NHH; k += C::kWaves)
                    p_lds[k * 64 + lane] = bf16x8{};
                if (tid < NHH)
                    resc_flag[tid] = 0;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    vf8_pend[db] = make_uint2(0u, 0u);
            }
            for (int it = 0; it < n_tiles; ++it) {
                wait_vmcnt(dma_w * min(C::kNBuf - 2, n_tiles - 1 - it));
                // every wave's pieces of tile `it` landed; tile it-1 is done (its PV
                // only needs registers and the published P^T)
                __syncthreads();
                // The copy issue, the pending PV and QK^T run at raised wave
                // priority: the SIMD's other wave (another workgroup, usually in
                // its softmax phase) fills the gaps of this MFMA stream instead of
                // competing with it.
                if constexpr (kPipe)
                    __builtin_amdgcn_s_setprio(1);
                int rflag[NHH];
                float ralpha[NHH];
                if constexpr (kPipe) {
#pragma unroll
                    for (int hb = 0; hb < NHH; ++hb) {
                        rflag[hb] = resc_flag[hb];
                        ralpha[hb] = alpha_lds[hb * 16 + n16];
                    }
                }
                if (it + C::kNBuf - 1 < n_tiles) {
                    const int nt = it + C::kNBuf - 1;
                    issue_tile<C>(p.cache, lds_slots + nt * kTile, min(kTile, n_valid - nt * kTile),
                                  ring + (nt % C::kNBuf) * C::kBufBytes, wave, lane);
                }
                if constexpr (kPipe) {
                    // PV of the previous tile, half of its dims after each
                    // column group's QK^T MFMAs
                    pv_pre(vf8_pend, exact_p, rflag, ralpha);
                    bf16x8 pvp[NHH];
                    pv_load(pvp);
                    tile(ring + (it % C::kNBuf) * C::kBufBytes, min(kTile, n_valid - it * kTile), exact_p,
                         [&](int gi) __attribute__((always_inline)) {
                             pv_part(vf8_pend, pvp, gi * (DB / 2), (gi + 1) * (DB / 2));
                         });
                } else {
                    tile(ring + (it % C::kNBuf) * C::kBufBytes, min(kTile, n_valid - it * kTile), exact_p,
                         [](int) {});
                }
            }
            if constexpr (kPipe) {
                __syncthreads();     // P^T of the last tile is visible
                int rflag[NHH];
                float ralpha[NHH];
#pragma unroll
                for (int hb = 0; hb < NHH; ++hb) {
                    rflag[hb] = resc_flag[hb];
                    ralpha[hb] = alpha_lds[hb * 16 + n16];
                }
                pv_pre(vf8_pend, exact_p, rflag, ralpha);
                bf16x8 pvp[NHH];
                pv_load(pvp);
                pv_part(vf8_pend, pvp, 0, DB);
            }
            __syncthreads();     // ring, exchanges and slot list are free for the next round
        }

        // ---- per-head results of head block hh (m_run and the row sums are the
        //      same in both column halves), handed to every wave through LDS
        {
            float l = l_part;
            l = xor32_sum(xor16_sum(l));
            // natural-log LSE; v_log_f32 is log2 (l >= 1 here: the row that set m_run adds >= 1)
            const float inv_l = l > 0.f ? 1.f / l : 0.f;
            const float lse_v = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
            if (dh == 0 && g == 0) {
                head_f[hh * 16 + n16] = inv_l;
                head_f[64 + hh * 16 + n16] = lse_v;
            }
            __syncthreads();
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb) {
                inv_l_hb[hb] = head_f[hb * 16 + n16];
                lse_hb[hb] = head_f[64 + hb * 16 + n16];
            }
        }

    }

    // ---- output rows of this workgroup's heads, staged in LDS and written out
    //      coalesced. One split: the bf16 rows of the result. A top-k split: the
    //      fp32 partial O / l and its lse, head-major, for merge_kernel.
    __syncthreads();        // every wave is done with the exchange areas
    const int n16_late = late(n16);
    if (!p.partials) {
        uint16_t *stage = (uint16_t *)smem;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int hb = k / DB, db = k % DB;
            const f32x4 v = o[k] * inv_l_hb[hb];
            *(uint2 *)(stage + (16 * hb + n16_late) * kDv + dim0 + 16 * db + 4 * g) =
                make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
        }
        if (wave == 0 && g == 0 && p.lse != nullptr) {
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb)
                p.lse[(size_t)t * p.H + wg_head0 + 16 * hb + n16] = lse_hb[hb];
        }
        __syncthreads();
        uint16_t *dst = p.out + ((size_t)t * p.H + wg_head0) * kDv;
        for (int u = tid; u < C::kHeads * kDv / 8; u += C::kThreads)
            *(uint4 *)(dst + 8 * u) = *(const uint4 *)(stage + 8 * u);
    } else {
        // rows padded by 16 bytes: the 16 heads of one store fall on distinct banks
        constexpr int kRow = kDv + 4;
        float *stage = (float *)smem;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int hb = k / DB, db = k % DB;
            *(f32x4 *)(stage + (16 * hb + n16_late) * kRow + dim0 + 16 * db + 4 * g) = o[k] * inv_l_hb[hb];
        }
        if (wave == 0 && g == 0) {
#pragma unroll
            for (int hb = 0; hb < NHH; ++hb)
                p.part_lse[((size_t)t * p.S + s) * p.H + wg_head0 + 16 * hb + n16] = lse_hb[hb];
        }
        __syncthreads();
        float *dst = p.part_o + (((size_t)t * p.S + s) * p.H + wg_head0) * kDv;
        for (int u = tid; u < C::kHeads * kDv / 4; u += C::kThreads) {
            const int row = u / (kDv / 4), c4 = u % (kDv / 4);
            *(f32x4 *)(dst + 4 * u) = *(const f32x4 *)(stage + row * kRow + 4 * c4);
        }
    }
}

// ------------------------------------------------- attention, QK^T waves and PV waves (fp8)

// Shape of an attn_pc_kernel workgroup: 64 heads of one token and one part of
// its top-k list, eight waves in two roles, one of each per SIMD:
//  * QK^T wave w (w < 4): head block w (16 heads) over all 576 columns --
//    S^T = K q^T, the online softmax, and the P^T operands of all four scale
//    groups, published through LDS;
//  * PV wave 4 + w: output dims 128 w .. 128 w + 127 (scale group w) of all
//    four head blocks -- each V^T fragment is read and converted once and
//    feeds four MFMAs -- and a quarter of every tile's copy instructions.
// PV runs one tile behind QK^T, so the SIMD interleaves one wave's MFMAs with
// the other's VALU and LDS work. P^T, the rescale flags and factors are double
// buffered by tile parity; one barrier per tile orders everything.
struct CfgPC {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 512;
    static constexpr int kHeads = 64;
    static constexpr int kRowBytes = kFp8RowBytes;
    static constexpr int kChunksPerRow = kRowBytes / 16;
    static constexpr int kRowStride = kRowBytes;
    static constexpr int kRowBlockBytes = 16 * kRowStride + 16;
    static constexpr int kInstrPerRow = 1;
    static constexpr int kRowsPerWave = kTile / 4;                   // first tiles: the four PV waves
    static constexpr int kDmaPerWave = kRowsPerWave;
    static constexpr int kBufBytes = (kRB * kRowBlockBytes + 1023) / 1024 * 1024;
    // ring buffers of a long list: four measured faster than five (c2 43.0 ->
    // 42.0 us, config 5 2.93 -> 2.86 ms) and three slower (c2 50 us)
    static constexpr int kNBuf = 4;
    static constexpr int kNBufExact = 3;                             // ring buffers of a short list
    // ring space: five buffers, so a short list's P^T lo terms fit past its three
    static constexpr int kRingBytes = 5 * kBufBytes;
    static constexpr int kPBytes = 2 * 4 * 4 * 1024;                 // [parity][head block][group] P^T hi
    // top-k positions compacted into LDS per round: one per thread (512
    // measured faster than 1024: c2 by 1 %, config 5 by 3 %)
    static constexpr int kChunk = 512;
    static constexpr int kSlotsBytes = kChunk * 4;
    static constexpr int kOffP = kRingBytes;
    static constexpr int kOffPLo = kNBufExact * kBufBytes;           // short lists: P^T lo terms
    static constexpr int kOffHead = kOffP + kPBytes;                 // flags, factors, max and sums
    // q of the four QK^T waves' head blocks (16 rows of 1152 bytes each), held
    // from the kernel start to the first barrier of the tile loop in space the
    // loop fills only after it: ring buffers 2.. and P^T
    static constexpr int kQBlockBytes = 16 * kDqk * 2;
    static constexpr int kOffQ = 2 * kBufBytes;
    // the request's block-table row, copied into ring buffers 0 and 1 (free until
    // the first tile copies, which start after the first round's compaction), so
    // its load runs beside the indices' instead of after them
    static constexpr int kBtLdsMax = kOffQ / 4;                       // entries
    static constexpr int kOffSlots = kOffHead + 1024;
    static constexpr int kOffMisc = kOffSlots + kSlotsBytes;         // compaction counts
    static constexpr int kLdsBytes = kOffMisc + 512;
    static constexpr int kStageBf16 = kDv + 8;                       // padded staging rows
    static constexpr int kStageF32 = kDv + 4;
    static_assert(kChunksPerRow <= 64, "one copy instruction per row");
    static_assert(kOffPLo + kPBytes <= kOffP, "lo terms fit the ring buffers a short list leaves free");
    static_assert(kNBuf * kBufBytes <= kRingBytes, "a long list's ring fits the ring space");
    static_assert(kNBufExact >= 3, "the ring holds tiles r - 1, r and the copy of r + 1");
    static_assert(kOffQ + 4 * kQBlockBytes <= kOffHead, "q staging stays clear of tiles 0, 1 and the flags");
    static_assert(kQBlockBytes % 1024 == 0, "q staging in whole-wave copies");
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one gfx950 workgroup");
    static_assert(kHeads * kStageF32 * 4 <= kOffHead, "staging fits the ring and P^T");
    static_assert(16 + (kChunk / kThreads) * kWaves <= 128, "compaction counts fit");
};

// Refills (tiles kNBuf and later) are copied by all eight waves, four rows each.
struct CfgPCRefill : CfgPC {
    static constexpr int kRowsPerWave = kTile / kWaves;
    static constexpr int kDmaPerWave = kRowsPerWave;
};

// The fp8_ds_mla path (a1-a6 and the per-split part of a7). Iteration r of the
// tile loop, after the barrier (tile r has landed; P^T of tile r - 1 is
// published; tile r - 2 is done): the QK^T waves process tile r into P^T
// parity r & 1; the PV waves add V^T P^T of tile r - 1 to their slices of O.
// At the end of its iteration every wave copies its four rows of the tiles
// whose buffers the barrier freed (tile r - 2's buffer takes tile
// r - 2 + nbuf): with eight waves issuing, the copies run at about twice the
// rate of four, and a wave stalled on one waits where it would otherwise wait
// at the next barrier.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_pc_kernel(const KParams p)
{
    using C = CfgPC;
    constexpr int RB = kRB;
    constexpr int RS = C::kRowStride;
    constexpr int RBB = C::kRowBlockBytes;
    constexpr int kPer = C::kChunk / C::kThreads;    // top-k positions per thread per round
    constexpr int kRope = RowFmt<kCacheFp8>::kRope;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
    uint8_t *ring = smem;
    bf16x8 *p_hi = (bf16x8 *)(smem + C::kOffP);              // [parity][hb][group][lane]
    bf16x8 *p_lo = (bf16x8 *)(smem + C::kOffPLo);
    int *resc_flag = (int *)(smem + C::kOffHead);            // [parity][hb] the block's max moved
    float *alpha_lds = (float *)(smem + C::kOffHead + 64);   // [parity][hb][16] its rescale factors
    float *m_lds = (float *)(smem + C::kOffHead + 576);      // [hb][16] final max
    float *l_lds = (float *)(smem + C::kOffHead + 832);      // [hb][16] final row sum
    int32_t *lds_slots = (int32_t *)(smem + C::kOffSlots);
    int32_t *lds_misc = (int32_t *)(smem + C::kOffMisc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, n16 = lane & 15;
    const bool qk_role = wave < 4;
    const int rw = wave & 3;       // head block (QK^T wave) or dim group (PV wave)

    // Workgroup id -> (token, split, head group); all workgroups of one token
    // get the same id mod 8, the XCD the hardware dispatches them to.
    int bid = blockIdx.x;
    const int xcd = bid & 7;
    bid >>= 3;
    const int hg = bid % p.HB;
    bid /= p.HB;
    const int s = bid % p.S;
    const int t = (bid / p.S) * 8 + xcd;
    if (t >= p.T)
        return;

    const int wg_head0 = hg * C::kHeads;
    const float c2 = p.log2e_scale;
    const int32_t *topk_row = p.topk + (size_t)t * p.K;
    const int req = p.slot_in ? 0 : p.req_id[t];
    const int pos_begin = s * p.split_len;
    const int pos_end = min(p.K, pos_begin + p.split_len);

    // QK^T waves hold q^T as the B operands: the latent goes through
    // v_mfma_scale_f32_16x16x128_f8f6f4 on the raw e4m3 K bytes, so q is written
    // as hi + lo e4m3 terms with a power-of-two scale per head and 128-column
    // group G (exact within 2^13 of the group's largest magnitude, absolute error
    // below 2^-21 of it further down): lane (head, g) holds columns 128 G + 32 g .. + 31
    // (qh, ql, scales qsh, qsl). RoPE: bf16 (qr), k-step ks holds columns
    // 512 + 32 ks + 8 g .. + 7.
    // QK^T and online softmax of head block rw on one tile; publishes the P^T
    // operands of all four scale groups into parity par (and the rescale
    // factors when the running max moved).
    auto qk_tile = [&](const uint8_t *buf, int n_tile, int par, auto exact_c, const i32x8 (&qh)[4],
                       const i32x8 (&ql)[4], const int (&qsh)[4], const int (&qsl)[4], const bf16x8 (&qr)[2],
                       float &m_run, float &l_part) __attribute__((always_inline)) {
        constexpr bool exact = decltype(exact_c)::value;
        const int off_k = n16 * RS;                      // K rows 16 rb + n16
        const int off_sc = (4 * g) * RS;                 // accumulator rows 16 rb + 4 g + i
        f32x4 sc[RB][4];        // four group scales of accumulator row 16 rb + 4 g + i
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[rb][i] = *(const f32x4 *)(buf + rb * RBB + off_sc + i * RS + 512);
        f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            i32x8 kf[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint4 *src = (const uint4 *)(buf + rb * RBB + off_k + 128 * G + 32 * g);
                const uint4 a0 = src[0], a1 = src[1];
                kf[rb] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            }
            f32x4 part[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                part[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    kf[rb], qh[G], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, qsh[G]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                part[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    kf[rb], ql[G], part[rb], 0, 0, 0, 127, 0, qsl[G]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rb][i] = fmaf(sc[rb][i][G], part[rb][i], acc[rb][i]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bf16x8 rf = *(const bf16x8 *)(buf + rb * RBB + off_k + kRope + 64 * ks + 16 * g);
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf, qr[ks], acc[rb], 0, 0, 0);
            }

        // online softmax in log2 units. The running max moves only when some
        // row exceeds it by 2^8 (tested on each lane's own rows, moved to the
        // whole head's max). The scale c2 > 0 is applied to the maximum and
        // inside the exp2 argument: max(c2 * a) = c2 * max(a).
        float lmax = -INFINITY;
        if (n_tile == kTile) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lmax = fmaxf(lmax, acc[rb][i]);
        } else {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[rb][i] = 16 * rb + 4 * g + i < n_tile ? acc[rb][i] : -INFINITY;
                    lmax = fmaxf(lmax, acc[rb][i]);
                }
        }
        lmax *= c2;
        bool moved = false;
        float alpha = 1.f;
        if (__ballot(lmax > m_run + kLazyRescale) != 0) {
            const float mx = xor32_max(xor16_max(lmax));
            if (mx > m_run + kLazyRescale) {
                alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
                l_part *= alpha;
                m_run = mx;
            }
            moved = true;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[rb][i] = __builtin_amdgcn_exp2f(fmaf(acc[rb][i], c2, -m_run));
                l_part += acc[rb][i];
            }
        // P^T operands: the weights for output group G carry that group's row
        // scales, so the dequantisation adds no rounding
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            f32x4 p0, p1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = acc[0][i] * sc[0][i][G];
                p1[i] = acc[1][i] * sc[1][i][G];
            }
            const bf16x8 hi = pack_p(p0, p1);
            p_hi[((par * 4 + rw) * 4 + G) * 64 + lane] = hi;
            if constexpr (exact)
                p_lo[((par * 4 + rw) * 4 + G) * 64 + lane] = pack_p_residual(p0, p1, hi);
        }
        if (lane == 0)
            resc_flag[par * 4 + rw] = moved ? 1 : 0;
        if (moved && g == 0)
            alpha_lds[(par * 4 + rw) * 16 + n16] = alpha;
    };

    // ---- compaction of one round of the list (up to kChunk positions):
    //      converted slots of valid positions into LDS in list order with one
    //      exchange of per-wave counts; every wave takes part (two barriers)
    const bool write_phys = p.phys_out != nullptr && hg == 0;   // head group 0 writes the slots
    auto compact = [&](int chunk0, int (&slotv)[kPer]) __attribute__((always_inline)) {
        const int chunk_n = min(C::kChunk, pos_end - chunk0);
        if (write_phys) {
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
    // Slots of one round of the list (up to kChunk positions from chunk0),
    // one round trip: the round's indices (into the slot-list area, which the
    // compaction fills only after every index has been read) and, beside them,
    // the request's whole block-table row (into ring buffers 0 and 1, free until
    // the round's first tile copies) are copied straight into LDS. In the first
    // round the QK^T waves then copy q of their 16 heads (contiguous rows),
    // needed only once the first tile has landed. Every load of the kernel is
    // such an explicit copy with an explicit wait: the compiler sees no vector
    // memory load, so it places no wait of its own (one would also cover the
    // copies in flight, in the tile loop too).
    const int32_t *bt_lds = (const int32_t *)smem;
    const int32_t *idx_lds = lds_slots;
    const bool bt_in_lds = !p.slot_in && (unsigned)req < (unsigned)p.R && p.MB <= C::kBtLdsMax;
    auto fetch_round = [&](int chunk0, int (&slotv)[kPer]) __attribute__((always_inline)) {
        const int n = min(pos_end, chunk0 + C::kChunk) - chunk0;
        // wave w copies entries 64 (8 k + w) .. + 63 of each list; lanes past its
        // end are inactive
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
        const bool q_now = qk_role && chunk0 == pos_begin;
        if (q_now) {
            const uint8_t *qsrc = (const uint8_t *)(p.q + ((size_t)t * p.H + wg_head0 + 16 * rw) * kDqk);
            const uint32_t qdst = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)LDS_PTR(uint8_t, smem + C::kOffQ + rw * C::kQBlockBytes));
#pragma unroll
            for (int k = 0; k < C::kQBlockBytes / 1024; ++k)
                dma16(qsrc + 1024 * k + 16 * lane, qdst + 1024u * k);
        }
        // every wave's index and table copies have landed (q's copies, issued
        // after them, may still be in flight: loads complete in order)
        wait_vmcnt(q_now ? C::kQBlockBytes / 1024 : 0);
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
            // a table row too long for the ring buffers: each thread's entries are
            // copied from the table itself into words of ring buffer 0 (lane l of
            // wave w, position j: word 64 (kPer w + j) + l), then read back
            const uint32_t own_base = (uint32_t)(uintptr_t)LDS_PTR(int32_t, (int32_t *)smem) +
                                      4u * 64u * (uint32_t)(kPer * wave);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const bool ok = slot_position_ok(req, idxv[j], p.R, p.MB);
                dma4(p.bt + (ok ? (size_t)req * p.MB + (idxv[j] >> 6) : 0),
                     __builtin_amdgcn_readfirstlane(own_base + 4u * 64u * (uint32_t)j));
            }
            wait_vmcnt(0);
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                slotv[j] = finish_slot(((const int32_t *)smem)[64 * (kPer * wave + j) + lane], req, idxv[j], p.R,
                                       p.MB, p.NB);
        }
    };
    int slotv[kPer];
    fetch_round(pos_begin, slotv);

    // split partials in bf16 (hi rows only, unless the split is short enough
    // for the exact path: then fp32 staging, written out as hi + lo rows)
    int valid_total = 0;
    if (qk_role) {
        // ================= QK^T waves: head block rw =================
        i32x8 qh[4], ql[4];
        int qsh[4], qsl[4];
        bf16x8 qr[2];
        float m_run = -INFINITY, l_part = 0.f;   // log2-domain running max (same in a head's 4 lanes), row sum
        for (int chunk0 = pos_begin; chunk0 < pos_end; chunk0 += C::kChunk) {
            if (chunk0 != pos_begin)
                fetch_round(chunk0, slotv);
            const int n_valid = compact(chunk0, slotv);
            valid_total += n_valid;
            const bool exact_p = n_valid <= kExactPRows;
            const int nbuf = exact_p ? C::kNBufExact : C::kNBuf;
            const int n_tiles = (n_valid + kTile - 1) / kTile;
            if (chunk0 == pos_begin) {
                // q, loaded and written as hi + lo e4m3 terms while the
                // PV waves' first copies are in flight
                uint4 qraw[18];     // [4 * G + c] latent of group G, [16 + ks] RoPE k-step ks
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // this wave's q copies
                const uint16_t *qrow = (const uint16_t *)(smem + C::kOffQ + rw * C::kQBlockBytes) + n16 * kDqk;
#pragma unroll
                for (int G = 0; G < 4; ++G)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        qraw[4 * G + c] = ((const uint4 *)(qrow + 128 * G + 32 * g))[c];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    qraw[16 + ks] = *(const uint4 *)(qrow + kDv + 32 * ks + 8 * g);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    qr[ks] = __builtin_bit_cast(bf16x8, qraw[16 + ks]);
#pragma unroll
                for (int G = 0; G < 4; ++G) {
                    float v[32];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 w = qraw[4 * G + c];
                        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[8 * c + 2 * e] = bf16_lo(ww[e]);
                            v[8 * c + 2 * e + 1] = bf16_hi(ww[e]);
                        }
                    }
                    float amax = 0.f;
#pragma unroll
                    for (int i = 0; i < 32; ++i)
                        amax = fmaxf(amax, fabsf(v[i]));
                    // the MFMA applies one B scale per column (head) to all 128 k of
                    // the group, so the exponent is shared by the head's four lanes
                    amax = xor32_max(xor16_max(amax));
                    // block exponent: the largest |q| maps into [128, 256), within e4m3's range
                    const int ex = max((int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 7, -120);
                    // the conversions apply the powers of two themselves (fp8 = x / scale
                    // rounded, f32 = fp8 x scale; both exact): hi in units of 2^ex, and
                    // what it misses, exactly, in units of 2^(ex - 4)
                    const float up_hi = __uint_as_float((uint32_t)(127 + ex) << 23);      // 2^ex
                    const float up_lo = __uint_as_float((uint32_t)(127 + ex - 4) << 23);  // 2^(ex - 4)
                    uint32_t hw[8], lw[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float *x = v + 4 * j;
                        s16x2 h = {0, 0};
                        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[0], x[1], up_hi, false);
                        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x[2], x[3], up_hi, true);
                        hw[j] = __builtin_bit_cast(uint32_t, h);
                        const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], up_hi, false);
                        const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[j], up_hi, true);
                        s16x2 l = {0, 0};
                        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x[0] - b0[0], x[1] - b0[1], up_lo, false);
                        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, x[2] - b1[0], x[3] - b1[1], up_lo, true);
                        lw[j] = __builtin_bit_cast(uint32_t, l);
                    }
                    qh[G] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
                    ql[G] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
                    qsh[G] = 127 + ex;
                    qsl[G] = 127 + ex - 4;
                }
            }
            int issued = min(n_tiles, nbuf);     // tiles whose copies have been issued
            auto tiles = [&](auto exact_c) __attribute__((always_inline)) {
                for (int r = 0; r <= n_tiles; ++r) {
                    // this wave's rows of tile r have landed (it copies refills only) ...
                    if (r < n_tiles)
                        wait_vmcnt(CfgPCRefill::kDmaPerWave * max(0, issued - max(nbuf, r + 1)));
                    // ... and every wave's; tile r - 2 is done with its buffer and P^T parity
                    __syncthreads();
                    if (r < n_tiles)
                        qk_tile(ring + (r % nbuf) * C::kBufBytes, min(kTile, n_valid - r * kTile), r & 1, exact_c,
                                qh, ql, qsh, qsl, qr, m_run, l_part);
                    const int hi = min(n_tiles, r - 1 + nbuf);
                    for (int nt = max(issued, nbuf); nt < hi; ++nt)
                        issue_tile<CfgPCRefill>(p.cache, lds_slots + nt * kTile, min(kTile, n_valid - nt * kTile),
                                                ring + (nt % nbuf) * C::kBufBytes, wave, lane);
                    issued = max(issued, hi);
                }
            };
            if (exact_p)
                tiles(std::true_type{});
            else
                tiles(std::false_type{});
            __syncthreads();     // ring, P^T and slot list are free for the next round
        }
        // (max, row sum) of each head to the PV waves
        float l = l_part;
        l = xor32_sum(xor16_sum(l));
        if (g == 0) {
            m_lds[rw * 16 + n16] = m_run;
            l_lds[rw * 16 + n16] = l;
        }
        __syncthreads();
        // lse of this head block (natural log; v_log_f32 is log2, and l >= 1
        // here: the row that set the max adds >= 1)
        if (g == 0) {
            const float lse_v = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
            if (!p.partials) {
                if (p.lse != nullptr)
                    p.lse[(size_t)t * p.H + wg_head0 + 16 * rw + n16] = lse_v;
            } else {
                p.part_lse[((size_t)t * p.S + s) * p.H + wg_head0 + 16 * rw + n16] = lse_v;
            }
        }
        __syncthreads();    // the PV waves have staged the output
    } else {
        // ================= PV waves: output dims 128 rw .. 128 rw + 127 =================
        // o[8 * hb + db] holds dims 128 rw + 16 db + 4 g + i of head 16 hb + n16
        f32x4 o[32];
#pragma unroll
        for (int k = 0; k < 32; ++k)
            o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        // V^T (ds_read_b64_tr_b8): source lane n16 = 2k + h reads row k of
        // {4g..4g+3, 16+4g..16+4g+3}, bytes 8h..8h+7 of a 16-byte column block;
        // this wave's dims start at byte 128 * rw of the row
        const int vk = n16 >> 1;
        const int off_v8 = (vk >> 2) * RBB + (4 * g + (vk & 3)) * RS + 8 * (n16 & 1) + 128 * rw;
        constexpr int dma_w = C::kDmaPerWave;
        for (int chunk0 = pos_begin; chunk0 < pos_end; chunk0 += C::kChunk) {
            if (chunk0 != pos_begin)
                fetch_round(chunk0, slotv);
            const int n_valid = compact(chunk0, slotv);
            valid_total += n_valid;
            const bool exact_p = n_valid <= kExactPRows;
            const int nbuf = exact_p ? C::kNBufExact : C::kNBuf;
            const int n_tiles = (n_valid + kTile - 1) / kTile;
            // the first tiles' copies (every buffer starts free); from here on the
            // only vector-memory instructions in flight are tile copies
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // the first two tiles now; the rest of the ring during iteration 0,
            // while the QK^T waves already work on tile 0 (copies of a cold
            // start queue behind the whole chip's, and a wave issuing them
            // stalls)
            int issued = min(n_tiles, 2);
            for (int i = 0; i < issued; ++i)
                issue_tile<C>(p.cache, lds_slots + i * kTile, min(kTile, n_valid - i * kTile),
                              ring + i * C::kBufBytes, rw, lane);
            const bool exact_s = __builtin_amdgcn_readfirstlane(exact_p ? 1 : 0) != 0;
            uint2 vf_next[8];     // V^T (e4m3) of the tile the next iteration's PV takes
#pragma unroll
            for (int db = 0; db < 8; ++db)
                vf_next[db] = make_uint2(0u, 0u);
            {
                for (int r = 0; r <= n_tiles; ++r) {
                    // this wave's rows of tile r have landed (eight per first
                    // tile, four per refill) ...
                    if (r < n_tiles)
                        wait_vmcnt(dma_w * max(0, min(issued, nbuf) - (r + 1)) +
                                   CfgPCRefill::kDmaPerWave * max(0, issued - max(nbuf, r + 1)));
                    // ... and every wave's; P^T of tile r - 1 is published; tile
                    // r - 2 is done with its buffer
                    __syncthreads();
                    if (r == 0) {
                        // the rest of the first tiles, while the QK^T waves work on tile 0
                        const int hi0 = min(n_tiles, nbuf);
                        for (int nt = issued; nt < hi0; ++nt)
                            issue_tile<C>(p.cache, lds_slots + nt * kTile, min(kTile, n_valid - nt * kTile),
                                          ring + nt * C::kBufBytes, rw, lane);
                        issued = max(issued, hi0);
                    }
                    if (r >= 1) {
                        // ---- O^T += V^T P^T of tile r - 1 over this wave's dims
                        const int par = (r - 1) & 1;
                        // the LDS reads after the barrier, issued before the first
                        // wait: the four head blocks' rescale flags (one 16-byte read)
                        // and their P^T hi operands (V^T was read before the barrier)
                        uint2 vf[8];     // read at the end of the last iteration
#pragma unroll
                        for (int db = 0; db < 8; ++db)
                            vf[db] = vf_next[db];
                        const int4 fl = *(const int4 *)(resc_flag + par * 4);
                        bf16x8 ph[4];
#pragma unroll
                        for (int hb = 0; hb < 4; ++hb)
                            ph[hb] = p_hi[((par * 4 + hb) * 4 + rw) * 64 + lane];
                        // scalar branches: O is rescaled in place (a lane-divergent one
                        // would keep a second copy of the accumulators)
                        if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
                            const int fls[4] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
                            for (int hb = 0; hb < 4; ++hb) {
                                if (__builtin_amdgcn_readfirstlane(fls[hb])) {
                                    const float al = alpha_lds[(par * 4 + hb) * 16 + n16];
#pragma unroll
                                    for (int db = 0; db < 8; ++db)
                                        o[hb * 8 + db] *= al;
                                }
                            }
                        }
                        // V^T converted four blocks at a time, each block feeding the
                        // four head blocks
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            bf16x8 va[4];
#pragma unroll
                            for (int d = 0; d < 4; ++d)
                                va[d] = e4m3x8_to_bf16x8(vf[4 * half + d]);
#pragma unroll
                            for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
                                for (int d = 0; d < 4; ++d)
                                    o[hb * 8 + 4 * half + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        va[d], ph[hb], o[hb * 8 + 4 * half + d], 0, 0, 0);
                                if (exact_s) {
                                    const bf16x8 pl = p_lo[((par * 4 + hb) * 4 + rw) * 64 + lane];
#pragma unroll
                                    for (int d = 0; d < 4; ++d)
                                        o[hb * 8 + 4 * half + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                            va[d], pl, o[hb * 8 + 4 * half + d], 0, 0, 0);
                                }
                            }
                        }
                    }
                    // refills whose buffers the barrier freed: rows 4 wave .. 4 wave + 3
                    const int hi = min(n_tiles, r - 1 + nbuf);
                    for (int nt = max(issued, nbuf); nt < hi; ++nt)
                        issue_tile<CfgPCRefill>(p.cache, lds_slots + nt * kTile, min(kTile, n_valid - nt * kTile),
                                                ring + (nt % nbuf) * C::kBufBytes, wave, lane);
                    issued = max(issued, hi);
                    // V^T of tile r for the next iteration, read while this wave
                    // would otherwise wait at the barrier (tile r has landed; its
                    // buffer is refilled only after the next iteration's PV)
                    if (r < n_tiles) {
                        const uint8_t *nbufp = ring + (r % nbuf) * C::kBufBytes;
#pragma unroll
                        for (int db = 0; db < 8; ++db) {
                            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                LDS_PTR(i32x2, nbufp + off_v8 + 16 * db));
                            vf_next[db] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
                        }
                    }
                }
            }
            __syncthreads();     // ring, P^T and slot list are free for the next round
        }
        __syncthreads();        // (max, row sum) of every head are in LDS
        // ---- this wave's slice of the output rows, normalised, staged in LDS
        //      (rows padded so the 16 heads of one store fall on distinct banks)
        const int n16_late = late(n16);
        const int dim0 = 128 * rw;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            const float l0 = l_lds[hb * 16 + n16];
            const float inv_l = l0 > 0.f ? 1.f / l0 : 0.f;
            if (!p.partials || (p.part_exact != nullptr && valid_total > kExactPRows)) {
                uint16_t *stage = (uint16_t *)smem;
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const f32x4 v = o[hb * 8 + db] * inv_l;
                    *(uint2 *)(stage + (16 * hb + n16_late) * C::kStageBf16 + dim0 + 16 * db + 4 * g) =
                        make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
                }
            } else {
                float *stage = (float *)smem;
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    *(f32x4 *)(stage + (16 * hb + n16_late) * C::kStageF32 + dim0 + 16 * db + 4 * g) =
                        o[hb * 8 + db] * inv_l;
            }
        }
        __syncthreads();
    }

    // ---- the staged rows written out coalesced. One split: the bf16 rows of
    //      the result. A top-k split: the fp32 partial O / l, head-major, for
    //      merge_kernel.
    const bool bf16_parts = p.partials && p.part_exact != nullptr;
    if (bf16_parts && tid == 0 && hg == 0)
        p.part_exact[(size_t)t * p.S + s] = valid_total <= kExactPRows ? 1 : 0;
    if (!p.partials || (bf16_parts && valid_total > kExactPRows)) {
        const uint16_t *stage = (const uint16_t *)smem;
        uint16_t *dst = !p.partials ? p.out + ((size_t)t * p.H + wg_head0) * kDv
                                    : (uint16_t *)p.part_o + (((size_t)t * p.S + s) * 2 * p.H + wg_head0) * kDv;
        for (int u = tid; u < C::kHeads * kDv / 8; u += C::kThreads) {
            const int row = u / (kDv / 8), c8 = u % (kDv / 8);
            // streamed past the caches: read once by the merge, or not at all
            // here (the result); the kernel's end then writes back less
            const uint4 val = *(const uint4 *)(stage + row * C::kStageBf16 + 8 * c8);
            __builtin_nontemporal_store(u32x4{val.x, val.y, val.z, val.w}, (u32x4 *)(dst + 8 * u));
        }
    } else if (bf16_parts) {
        // a short split: hi rows in the slot's first half, residual rows in its second
        const float *stage = (const float *)smem;
        uint16_t *dst = (uint16_t *)p.part_o + (((size_t)t * p.S + s) * 2 * p.H + wg_head0) * kDv;
        const size_t lo_off = (size_t)p.H * kDv;
        for (int u = tid; u < C::kHeads * kDv / 4; u += C::kThreads) {
            const int row = u / (kDv / 4), c4 = u % (kDv / 4);
            const f32x4 v = *(const f32x4 *)(stage + row * C::kStageF32 + 4 * c4);
            const uint32_t h01 = pack_bf16(v[0], v[1]), h23 = pack_bf16(v[2], v[3]);
            *(uint2 *)(dst + 4 * u) = make_uint2(h01, h23);
            *(uint2 *)(dst + lo_off + 4 * u) =
                make_uint2(pack_bf16(v[0] - bf16_lo(h01), v[1] - bf16_hi(h01)),
                           pack_bf16(v[2] - bf16_lo(h23), v[3] - bf16_hi(h23)));
        }
    } else {
        const float *stage = (const float *)smem;
        float *dst = p.part_o + (((size_t)t * p.S + s) * p.H + wg_head0) * kDv;
        for (int u = tid; u < C::kHeads * kDv / 4; u += C::kThreads) {
            const int row = u / (kDv / 4), c4 = u % (kDv / 4);
            *(f32x4 *)(dst + 4 * u) = *(const f32x4 *)(stage + row * C::kStageF32 + 4 * c4);
        }
    }
}

// Log-sum-exp merge of a token's top-k splits: thread (t, h, c) combines
// kDpt consecutive dims (group c) of head h over the splits in index order
// (weights exp(lse_s - max lse), normalised by their sum) and writes the bf16
// output and, once per head, the merged natural-log lse. A split with
// lse = -inf (no valid position) has weight 0; a head with none at all gets 0
// and -inf. KS > 0: exactly KS splits, every load issued before the first is
// used; KS = 0: any count, in batches of 8. BF: the partials are bf16 hi rows
// (the first half of each split's fp32 slot), plus residual rows (the second
// half) for the splits part_exact flags, which are loaded only after the
// flags; a thread then takes 8 dims, one 16-byte load per row. fp32 partials:
// 4 dims, also one 16-byte load per row.
template <bool BF> struct MergeVec;
template <> struct MergeVec<false> { typedef float type __attribute__((__vector_size__(16))); };
template <> struct MergeVec<true> { typedef float type __attribute__((__vector_size__(32))); };

template <int KS, bool BF>
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ part_o,
                                                    const float *__restrict__ part_lse,
                                                    const int32_t *__restrict__ part_exact,
                                                    uint16_t *__restrict__ out, float *__restrict__ lse,
                                                    int T, int H, int S)
{
    constexpr int kDpt = BF ? 8 : 4;                  // dims per thread
    constexpr int kGroups = kDv / kDpt;               // threads per (token, head)
    typedef typename MergeVec<BF>::type vec;
    // Workgroup id -> (token, run of heads): the workgroups of token t get id
    // mod 8 = t mod 8, the XCD whose L2 the attention kernel wrote t's
    // partials through.
    const int wpt = H * kGroups / 256;                // workgroups per token
    const int bid = blockIdx.x;
    const int tt = (bid >> 3) / wpt * 8 + (bid & 7);
    if (tt >= T)
        return;
    const int64_t gid = ((int64_t)tt * wpt + (bid >> 3) % wpt) * 256 + threadIdx.x;
    const int c = (int)(gid % kGroups);
    const int64_t th = gid / kGroups;                 // t * H + h
    const int t = (int)(th / H), h = (int)(th - (int64_t)t * H);
    if constexpr (KS > 0)
        S = KS;
    const float *pl = part_lse + (size_t)t * S * H + h;
    // one split's rows of all heads, in 16-byte units: fp32 rows (fp32), or
    // the hi rows, with the residual rows right after them (BF)
    const size_t ostride = (size_t)H * kGroups;
    const f32x4 *po = (const f32x4 *)part_o + ((size_t)t * S * H + h) * kGroups + c;
    const uint4 *pb = (const uint4 *)part_o + ((size_t)t * S * 2 * H + h) * kGroups + c;
    const int32_t *pe = BF ? part_exact + (size_t)t * S : nullptr;
    // 8 bf16 values to fp32 (used only with BF)
    auto unpack = [](uint4 u) __attribute__((always_inline)) -> vec {
        vec v = {};
        if constexpr (BF) {
            v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
            v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
        }
        return v;
    };
    auto load = [&](int s2) __attribute__((always_inline)) -> vec {
        if constexpr (BF)
            return unpack(pb[(size_t)s2 * 2 * ostride]);
        else
            return po[(size_t)s2 * ostride];
    };
    auto residual = [&](int s2) __attribute__((always_inline)) -> vec {
        return unpack(pb[(size_t)s2 * 2 * ostride + ostride]);
    };
    float M = -INFINITY, W = 0.f;
    vec acc = {};
    if constexpr (KS > 0) {
        float l[KS];
        vec v[KS];
        int ex[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            l[s2] = pl[(size_t)s2 * H];
            v[s2] = load(s2);
            ex[s2] = BF ? pe[s2] : 0;
        }
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                if (ex[s2])
                    v[s2] += residual(s2);
        }
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
            M = fmaxf(M, l[s2]);
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const float w = M == -INFINITY ? 0.f : __expf(l[s2] - M);
            acc += w * v[s2];
            W += w;
        }
    } else {
        for (int s2 = 0; s2 < S; ++s2)
            M = fmaxf(M, pl[(size_t)s2 * H]);
        for (int s0 = 0; s0 < S; s0 += 8) {
            vec v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (s0 + k < S)
                    v[k] = load(s0 + k);
            if constexpr (BF) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (s0 + k < S && pe[s0 + k])
                        v[k] += residual(s0 + k);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (s0 + k < S) {
                    const float w = M == -INFINITY ? 0.f : __expf(pl[(size_t)(s0 + k) * H] - M);
                    acc += w * v[k];
                    W += w;
                }
        }
    }
    const vec o = acc * (W > 0.f ? 1.f / W : 0.f);
    if constexpr (BF)
        *(uint4 *)(out + th * kDv + kDpt * c) = make_uint4(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                                                           pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7]));
    else
        *(uint2 *)(out + th * kDv + kDpt * c) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
    if (c == 0 && lse != nullptr)
        lse[th] = W > 0.f ? M + logf(W) : -INFINITY;
}

// Cache writer [flashmla_sparse.py page, FlashMLASparseImpl.forward: the
// concat_and_cache_mla call; cache format note]: one wave per token writes its
// 512 latent and 64 RoPE values into the row at slot_mapping[t]. fp8_ds_mla:
// lane l holds latent values 8l .. 8l + 7, so each 128-value group is one row of
// 16 lanes; the group's scale is amax / 448 in float32 (1.0 for an all-zero
// group) and each byte is x / scale (float32 division) rounded to the nearest
// e4m3 value, ties to even. nvfp4_ds_mla: lane l holds latent values 8l ..
// 8l + 7, so each 16-value block is a lane pair; the block's scale is the e4m3
// value nearest to amax / 6 and each code the E2M1 value nearest to x / scale
// (both float32 divisions, ties to even, saturating); RoPE values are rounded
// to e4m3. bf16: the row is copied. Slots outside [0, num_slots) write
// nothing. Four tokens per 256-thread block.
template <int FMT>
__global__ __launch_bounds__(256) void cache_write_kernel(const uint16_t *__restrict__ k_c,
                                                          const uint16_t *__restrict__ k_pe,
                                                          const int64_t *__restrict__ slot_mapping,
                                                          uint8_t *__restrict__ cache, int64_t num_tokens,
                                                          int64_t num_slots)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= num_tokens)
        return;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots)
        return;
    const uint4 lat = ((const uint4 *)(k_c + t * kDv))[lane];
    uint4 rope = make_uint4(0u, 0u, 0u, 0u);
    if (lane < 8)
        rope = ((const uint4 *)(k_pe + t * (kDqk - kDv)))[lane];
    if constexpr (FMT == kCacheBf16) {
        uint8_t *row = cache + slot * kBf16RowBytes;
        ((uint4 *)row)[lane] = lat;
        if (lane < 8)
            ((uint4 *)(row + 2 * kDv))[lane] = rope;
    } else if constexpr (FMT == kCacheNvfp4) {
        // lane l: latent 8l .. 8l + 7, half of 16-value block l / 2
        uint8_t *row = cache + slot * kNvfp4RowBytes;
        const uint32_t w[4] = {lat.x, lat.y, lat.z, lat.w};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_lo(w[e]);
            v[2 * e + 1] = bf16_hi(w[e]);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        // the block scale: the e4m3 value nearest to amax / 6 (ties to even,
        // at most 448); a scale that rounds to zero stores zero codes
        const float want = fminf(amax / 6.f, 448.f);
        const uint32_t sc_code =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, want, want, 1.0f, false)) &
            0xFFu;
        const float scale = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc_code, 1.0f, false)[0];
        uint32_t codes = 0;
        if (scale > 0.f) {
            // each code: the E2M1 value nearest to x / scale (ties to even), at most 6
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                x[i] = fminf(fmaxf(v[i] / scale, -6.f), 6.f);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, x[0], x[1], 1.0f, 0);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, x[2], x[3], 1.0f, 1);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, x[4], x[5], 1.0f, 2);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, x[6], x[7], 1.0f, 3);
        }
        ((uint32_t *)row)[lane] = codes;
        if ((lane & 1) == 0)
            row[RowFmt<kCacheNvfp4>::kScales + (lane >> 1)] = (uint8_t)sc_code;
        if (lane < 8) {
            // RoPE: the nearest e4m3 bytes, saturating at 448
            const uint32_t rw[4] = {rope.x, rope.y, rope.z, rope.w};
            uint32_t rc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float a0 = fminf(fmaxf(bf16_lo(rw[2 * j]), -448.f), 448.f);
                const float a1 = fminf(fmaxf(bf16_hi(rw[2 * j]), -448.f), 448.f);
                const float a2 = fminf(fmaxf(bf16_lo(rw[2 * j + 1]), -448.f), 448.f);
                const float a3 = fminf(fmaxf(bf16_hi(rw[2 * j + 1]), -448.f), 448.f);
                s16x2 c = {0, 0};
                c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, a0, a1, 1.0f, false);
                c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, a2, a3, 1.0f, true);
                rc[j] = __builtin_bit_cast(uint32_t, c);
            }
            ((uint2 *)(row + RowFmt<kCacheNvfp4>::kRope))[lane] = make_uint2(rc[0], rc[1]);
        }
    } else {
        uint8_t *row = cache + slot * kFp8RowBytes;
        const uint32_t w[4] = {lat.x, lat.y, lat.z, lat.w};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_lo(w[e]);
            v[2 * e + 1] = bf16_hi(w[e]);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, d));
        const float scale = amax > 0.f ? amax / 448.f : 1.f;
        uint32_t code[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            s16x2 c = {0, 0};
            c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, v[4 * j] / scale, v[4 * j + 1] / scale, 1.0f, false);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, v[4 * j + 2] / scale, v[4 * j + 3] / scale, 1.0f, true);
            code[j] = __builtin_bit_cast(uint32_t, c);
        }
        ((uint2 *)row)[lane] = make_uint2(code[0], code[1]);
        if ((lane & 15) == 0)
            ((float *)(row + kDv))[lane >> 4] = scale;
        if (lane < 8)
            ((uint4 *)(row + kDv + 16))[lane] = rope;
    }
}

__global__ __launch_bounds__(256) void convert_kernel(const int32_t *__restrict__ req_id,
                                                      const int32_t *__restrict__ bt,
                                                      const int32_t *__restrict__ topk,
                                                      int32_t *__restrict__ out, int64_t total,
                                                      int topk_len, int num_reqs, int max_blocks,
                                                      int64_t num_blocks)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int t = (int)(i / topk_len);
        out[i] = convert_slot(req_id[t], topk[i], bt, num_reqs, max_blocks, num_blocks);
    }
}

// Index conversion with a prefill workspace [flashmla_sparse.py page,
// _convert_req_index_to_global_index_kernel, HAS_PREFILL branch]: a token with
// a prefill request id r >= 0 maps a valid index to workspace_starts[r] + index
// (no block-table read); other tokens convert as convert_kernel.
__global__ __launch_bounds__(256) void convert_ws_kernel(const int32_t *__restrict__ req_id,
                                                         const int32_t *__restrict__ bt,
                                                         const int32_t *__restrict__ topk,
                                                         const int32_t *__restrict__ prefill_rid,
                                                         const int32_t *__restrict__ ws_starts,
                                                         int32_t *__restrict__ out, int64_t total, int topk_len,
                                                         int num_reqs, int max_blocks, int64_t num_blocks,
                                                         int num_prefills)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int t = (int)(i / topk_len);
        const int r = prefill_rid[t];
        const int idx = topk[i];
        if (r < 0)
            out[i] = convert_slot(req_id[t], idx, bt, num_reqs, max_blocks, num_blocks);
        else
            out[i] = r < num_prefills && idx >= 0 && (idx >> 6) < max_blocks ? ws_starts[r] + idx : -1;
    }
}

// e4m3 x scale rounded once to the nearest bf16, ties to even. The float32
// product p and its exact residual e = fma(x, s, -p) (x has 4 significant
// bits, so x * s is p + e exactly while p is a normal float) decide the one
// case where rounding p alone could differ: p exactly halfway between two bf16
// values, where the residual's sign says which side the true product is on.
__device__ __forceinline__ uint32_t bf16_of_product(float x, float sc)
{
    const float pr = x * sc;
    const float e = fmaf(x, sc, -pr);
    const uint32_t u = __float_as_uint(pr);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;        // nearest, ties to even
    if ((u & 0xFFFFu) == 0x8000u && e != 0.f)                   // p is a tie; the product is not
        r = ((e > 0.f) == (pr > 0.f)) ? (u >> 16) + 1u : (u >> 16);
    return r;
}

// Upconvert [flashmla_sparse.py page, _forward_fp8_kv_separate_prefill_decode:
// cp_gather_and_upconvert_fp8_kv_cache]. One wave per R consecutive positions of
// one request: R divides the cache block size, so the R rows share one
// block-table entry and lie back to back both in their cache block and in the
// workspace. The wave reads its three index words once, issues every row load
// before the first conversion, then lane l turns latent bytes 8l .. 8l + 7
// (scale group l / 16) of each row into 16 bytes of bf16. The 4R per-128
// scales come in with one dword load (lane 4r + g holds row r's scale g) and
// reach their lanes through a cross-lane read; the RoPE bytes are copied as
// R * 8 16-byte pieces. A position past the table, or a table entry outside
// the cache, writes zeros; rows outside the workspace are not written.
constexpr int kUpRows = 4;

template <int R>
__global__ __launch_bounds__(256) void upconvert_kernel(const uint8_t *__restrict__ cache, int64_t num_blocks,
                                                        const int32_t *__restrict__ bt, int max_blocks,
                                                        const int32_t *__restrict__ seq_lens,
                                                        const int32_t *__restrict__ ws_starts,
                                                        uint16_t *__restrict__ ws, int64_t ws_rows)
{
    static_assert(kBlock % R == 0 && R >= 1 && R <= 16, "rows per wave");
    constexpr int kRope = (R * 8 + 63) / 64;     // 16-byte RoPE pieces per lane
    const int b = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * R;
    const int64_t blk = p0 / kBlock;
    const int len = seq_lens[b];
    const int64_t w0 = (int64_t)ws_starts[b] + p0;
    const int base = blk < max_blocks ? bt[(size_t)b * max_blocks + blk] : -1;
    const int n = (int)min((int64_t)R, len - p0);
    if (n <= 0)
        return;
    if (base < 0 || (int64_t)base >= num_blocks) {
        for (int r = 0; r < n; ++r) {
            const int64_t w = w0 + r;
            if (w >= 0 && w < ws_rows) {
                uint4 *dst = (uint4 *)(ws + w * kDqk);
                dst[lane] = make_uint4(0u, 0u, 0u, 0u);
                if (lane < 8)
                    dst[64 + lane] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        return;
    }
    // rows n .. R - 1 (the end of the context) re-read row n - 1 and are not stored
    const uint8_t *rows = cache + ((int64_t)base * kBlock + p0 % kBlock) * kFp8RowBytes;
    uint2 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        v[r] = *(const uint2 *)(rows + (int64_t)min(r, n - 1) * kFp8RowBytes + 8 * lane);
    float sc_all = 0.f;
    if (lane < 4 * R)
        sc_all = *(const float *)(rows + (int64_t)min(lane >> 2, n - 1) * kFp8RowBytes + 512 + 4 * (lane & 3));
    uint4 rope[kRope];
#pragma unroll
    for (int j = 0; j < kRope; ++j) {
        const int i = min(j * 64 + lane, R * 8 - 1);
        rope[j] = *(const uint4 *)(rows + (int64_t)min(i >> 3, n - 1) * kFp8RowBytes + 528 + 16 * (i & 7));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float sc = __shfl(sc_all, 4 * r + (lane >> 4));
        const int64_t w = w0 + r;
        if (r < n && w >= 0 && w < ws_rows) {
            const f32x2 x[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[r].x, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[r].x, 1.0f, true),
                                __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[r].y, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[r].y, 1.0f, true)};
            uint32_t h[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                h[k] = bf16_of_product(x[k][0], sc) | (bf16_of_product(x[k][1], sc) << 16);
            ((uint4 *)(ws + w * kDqk))[lane] = make_uint4(h[0], h[1], h[2], h[3]);
        }
    }
#pragma unroll
    for (int j = 0; j < kRope; ++j) {
        const int i = j * 64 + lane;
        const int64_t w = w0 + (i >> 3);
        if (i < R * 8 && (i >> 3) < n && w >= 0 && w < ws_rows)
            ((uint4 *)(ws + w * kDqk))[64 + (i & 7)] = rope[j];
    }
}

// The same gather over an nvfp4_ds_mla cache [pull-request page "Support
// nvfp4_ds_mla on FLASHINFER_MLA_SPARSE, with native NVFP4 decode": prefill is
// staged through a context gather per request and chunk]. The staged rows hold
// the exact values: lane l turns latent codes 8l .. 8l + 7 (one dword, block
// l / 2) into fp32, multiplies by the block's E4M3 scale and packs to bf16, and
// lanes 0..7 turn 8 E4M3 RoPE bytes each into bf16; no step rounds (E2M1 x E4M3
// has at most 6 significant bits). Wave layout, the zero rows of a bad block and
// the workspace bounds as upconvert_kernel; every load is issued before the
// first conversion.
template <int R>
__global__ __launch_bounds__(256) void upconvert_nvfp4_kernel(const uint8_t *__restrict__ cache, int64_t num_blocks,
                                                              const int32_t *__restrict__ bt, int max_blocks,
                                                              const int32_t *__restrict__ seq_lens,
                                                              const int32_t *__restrict__ ws_starts,
                                                              uint16_t *__restrict__ ws, int64_t ws_rows)
{
    static_assert(kBlock % R == 0 && R >= 1 && R <= 16, "rows per wave");
    using F = RowFmt<kCacheNvfp4>;
    const int b = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * R;
    const int64_t blk = p0 / kBlock;
    const int len = seq_lens[b];
    const int64_t w0 = (int64_t)ws_starts[b] + p0;
    const int base = blk < max_blocks ? bt[(size_t)b * max_blocks + blk] : -1;
    const int n = (int)min((int64_t)R, len - p0);
    if (n <= 0)
        return;
    if (base < 0 || (int64_t)base >= num_blocks) {
        for (int r = 0; r < n; ++r) {
            const int64_t w = w0 + r;
            if (w >= 0 && w < ws_rows) {
                uint4 *dst = (uint4 *)(ws + w * kDqk);
                dst[lane] = make_uint4(0u, 0u, 0u, 0u);
                if (lane < 8)
                    dst[64 + lane] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        return;
    }
    // rows n .. R - 1 (the end of the context) re-read row n - 1 and are not stored
    const uint8_t *rows = cache + ((int64_t)base * kBlock + p0 % kBlock) * kNvfp4RowBytes;
    uint32_t codes[R], sc_byte[R];
    uint2 rope[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint8_t *row = rows + (int64_t)min(r, n - 1) * kNvfp4RowBytes;
        codes[r] = *(const uint32_t *)(row + 4 * lane);
        sc_byte[r] = row[F::kScales + (lane >> 1)];
        rope[r] = *(const uint2 *)(row + F::kRope + 8 * (lane & 7));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t w = w0 + r;
        if (r < n && w >= 0 && w < ws_rows) {
            const float sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc_byte[r], 1.0f, false)[0];
            const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[r], 1.0f, 0);
            const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[r], 1.0f, 1);
            const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[r], 1.0f, 2);
            const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[r], 1.0f, 3);
            uint4 *dst = (uint4 *)(ws + w * kDqk);
            dst[lane] = make_uint4(pack_bf16(f0[0] * sc, f0[1] * sc), pack_bf16(f1[0] * sc, f1[1] * sc),
                                   pack_bf16(f2[0] * sc, f2[1] * sc), pack_bf16(f3[0] * sc, f3[1] * sc));
            if (lane < 8)
                dst[64 + lane] = __builtin_bit_cast(uint4, e4m3x8_to_bf16x8(rope[r]));
        }
    }
}

template <int FMT, int NHH>
hipError_t launch_one(const KParams &p, hipStream_t stream)
{
    using C = Cfg<FMT, NHH>;
    const int64_t tq = (p.T + 7) / 8;
    const dim3 grid((unsigned)(tq * 8 * p.S * p.HB));
    hipLaunchKernelGGL((attn_kernel<FMT, NHH>), grid, dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_pc(const KParams &p, hipStream_t stream)
{
    const int64_t tq = (p.T + 7) / 8;
    const dim3 grid((unsigned)(tq * 8 * p.S * p.HB));
    hipLaunchKernelGGL(attn_pc_kernel, grid, dim3(CfgPC::kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const KParams &p, hipStream_t stream)
{
    if constexpr (FMT == kCacheNvfp4) {
        return launch_one<FMT, 1>(p, stream);     // 16 heads: one workgroup per head block
    } else {
        const int heads = p.H / p.HB;     // heads per workgroup: 128 (bf16), 64, 32 or 16
        if constexpr (FMT == kCacheBf16) {
            if (heads == 128)
                return launch_attn128(p, stream);
        }
        if constexpr (FMT == kCacheFp8) {
            // fp8 cache, 64 heads per workgroup: QK^T waves and PV waves
            if (heads == 64)
                return launch_pc(p, stream);
            if (heads == 32)
                return launch_one<FMT, 2>(p, stream);
            return launch_one<FMT, 1>(p, stream);
        }
        if (heads == 64)
            return launch_one<FMT, 4>(p, stream);
        if (heads == 32)
            return launch_one<FMT, 2>(p, stream);
        return launch_one<FMT, 1>(p, stream);
    }
}

}  // namespace

// The split workspace of the allocation-free entry point: each device holds
// its own copy for the life of the process. In host code the array's name is
// only a stand-in for the symbol; kernels get the device address that
// hipGetSymbolAddress returns, never the name.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (p == nullptr || ((uintptr_t)p & 255u) != 0)
            return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_convert(const int32_t *req_id, const int32_t *block_table, const int32_t *topk,
                          int32_t *out, int num_tokens, int topk_len, int num_reqs, int max_blocks,
                          int64_t num_blocks, hipStream_t stream)
{
    const int64_t total = (int64_t)num_tokens * topk_len;
    const int64_t blocks = (total + 255) / 256;
    const int grid = (int)(blocks < 16384 ? blocks : 16384);
    hipLaunchKernelGGL(convert_kernel, dim3(grid), dim3(256), 0, stream, req_id, block_table, topk,
                       out, total, topk_len, num_reqs, max_blocks, num_blocks);
    return hipGetLastError();
}

hipError_t launch_convert_ws(const int32_t *req_id, const int32_t *block_table, const int32_t *topk,
                             const int32_t *prefill_rid, const int32_t *ws_starts, int32_t *out,
                             int num_tokens, int topk_len, int num_reqs, int max_blocks, int64_t num_blocks,
                             int num_prefills, hipStream_t stream)
{
    const int64_t total = (int64_t)num_tokens * topk_len;
    const int64_t blocks = (total + 255) / 256;
    const int grid = (int)(blocks < 16384 ? blocks : 16384);
    hipLaunchKernelGGL(convert_ws_kernel, dim3(grid), dim3(256), 0, stream, req_id, block_table, topk,
                       prefill_rid, ws_starts, out, total, topk_len, num_reqs, max_blocks, num_blocks,
                       num_prefills);
    return hipGetLastError();
}

hipError_t launch_upconvert(CacheFormat fmt, const void *cache, int64_t num_blocks, const int32_t *block_table,
                            int max_blocks, const int32_t *seq_lens, const int32_t *ws_starts, int batch,
                            int max_seq_len, void *workspace, int64_t workspace_rows, hipStream_t stream)
{
    const dim3 grid((unsigned)(((int64_t)max_seq_len + 4 * kUpRows - 1) / (4 * kUpRows)), (unsigned)batch);
    if (fmt == kCacheNvfp4)
        hipLaunchKernelGGL(upconvert_nvfp4_kernel<kUpRows>, grid, dim3(256), 0, stream, (const uint8_t *)cache,
                           num_blocks, block_table, max_blocks, seq_lens, ws_starts, (uint16_t *)workspace,
                           workspace_rows);
    else
        hipLaunchKernelGGL(upconvert_kernel<kUpRows>, grid, dim3(256), 0, stream, (const uint8_t *)cache,
                           num_blocks, block_table, max_blocks, seq_lens, ws_starts, (uint16_t *)workspace,
                           workspace_rows);
    return hipGetLastError();
}

hipError_t launch_cache_write(CacheFormat fmt, const void *k_c, const void *k_pe, const int64_t *slot_mapping,
                             void *cache, int64_t num_tokens, int64_t num_slots, hipStream_t stream)
{
    const dim3 grid((unsigned)((num_tokens + 3) / 4));
    if (fmt == kCacheNvfp4)
        hipLaunchKernelGGL(cache_write_kernel<kCacheNvfp4>, grid, dim3(256), 0, stream, (const uint16_t *)k_c,
                           (const uint16_t *)k_pe, slot_mapping, (uint8_t *)cache, num_tokens, num_slots);
    else if (fmt == kCacheFp8)
        hipLaunchKernelGGL(cache_write_kernel<kCacheFp8>, grid, dim3(256), 0, stream, (const uint16_t *)k_c,
                           (const uint16_t *)k_pe, slot_mapping, (uint8_t *)cache, num_tokens, num_slots);
    else
        hipLaunchKernelGGL(cache_write_kernel<kCacheBf16>, grid, dim3(256), 0, stream, (const uint16_t *)k_c,
                           (const uint16_t *)k_pe, slot_mapping, (uint8_t *)cache, num_tokens, num_slots);
    return hipGetLastError();
}

template <bool BF>
void launch_merge_as(const float *part_lse, const float *part_o, const int32_t *part_exact, uint16_t *o,
                     float *lse, int T, int H, int S, dim3 grid, hipStream_t stream)
{
    switch (S) {
    case 2: hipLaunchKernelGGL((merge_kernel<2, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    case 3: hipLaunchKernelGGL((merge_kernel<3, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    case 4: hipLaunchKernelGGL((merge_kernel<4, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    case 5: hipLaunchKernelGGL((merge_kernel<5, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    case 6: hipLaunchKernelGGL((merge_kernel<6, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    case 8: hipLaunchKernelGGL((merge_kernel<8, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    default: hipLaunchKernelGGL((merge_kernel<0, BF>), grid, dim3(256), 0, stream, part_o, part_lse, part_exact, o, lse, T, H, S); break;
    }
}

hipError_t launch_merge(const float *part_lse, const float *part_o, const int32_t *part_exact, void *out,
                        float *lse, int T, int H, int S, hipStream_t stream)
{
    // whole workgroups per token (h_q * 64 threads for bf16 partials, h_q * 128
    // for fp32, h_q in {16, 32, 64, 128}), tokens padded to a multiple of 8 for
    // the XCD mapping
    const bool bf = part_exact != nullptr;
    const int64_t wpt = (int64_t)H * (kDv / (bf ? 8 : 4)) / 256;
    const dim3 grid((unsigned)((T + 7) / 8 * 8 * wpt));
    if (bf)
        launch_merge_as<true>(part_lse, part_o, part_exact, (uint16_t *)out, lse, T, H, S, grid, stream);
    else
        launch_merge_as<false>(part_lse, part_o, part_exact, (uint16_t *)out, lse, T, H, S, grid, stream);
    return hipGetLastError();
}

hipError_t launch_attention(CacheFormat fmt, const AttnArgs &a, const Plan &pl, bool partials_only,
                            AttnStage stage, hipStream_t stream)
{
    KParams p;
    p.q = (const uint16_t *)a.q;
    p.cache = (const uint8_t *)a.cache;
    p.bt = a.block_table;
    p.req_id = a.req_id;
    p.topk = a.topk;
    p.out = (uint16_t *)a.out;
    p.lse = a.lse;
    p.phys_out = a.phys_out;
    const bool split = pl.num_splits > 1 || partials_only;
    p.part_o = split ? (float *)((char *)a.workspace + pl.part_o_off) : nullptr;
    p.part_lse = split ? (float *)((char *)a.workspace + pl.part_lse_off) : nullptr;
    // workgroups per (token, part) along heads: two 64-head attn_pc_kernel
    // workgroups for fp8 with h_q = 128, one 16-head workgroup per head block
    // for nvfp4, else one covering every head
    const int hb = fmt == kCacheNvfp4 ? a.h_q / 16 : fmt == kCacheFp8 && a.h_q == 128 ? 2 : 1;
    // bf16 split partials: attn_pc_kernel (fp8 cache, 64-head workgroups) in a
    // call that merges its own splits
    const bool pc = fmt == kCacheFp8 && a.h_q / hb == 64;
    p.part_exact = split && !partials_only && pc ? (int32_t *)((char *)a.workspace + pl.part_exact_off) : nullptr;
    p.log2e_scale = a.sm_scale * 1.4426950408889634f;
    p.T = a.num_tokens;
    p.H = a.h_q;
    p.K = a.topk_len;
    p.R = a.num_reqs;
    p.MB = a.max_blocks;
    p.NB = a.num_blocks;
    p.S = pl.num_splits;
    p.split_len = pl.split_len;
    p.HB = hb;
    p.partials = split ? 1 : 0;
    p.slot_in = a.slot_indices ? 1 : 0;
    if (stage == AttnStage::kMergeOnly && (!split || partials_only))
        return hipSuccess;
    if (stage != AttnStage::kMergeOnly) {
        const hipError_t err = fmt == kCacheFp8     ? launch_fmt<kCacheFp8>(p, stream)
                               : fmt == kCacheNvfp4 ? launch_fmt<kCacheNvfp4>(p, stream)
                                                    : launch_fmt<kCacheBf16>(p, stream);
        if (err != hipSuccess || !split || partials_only || stage == AttnStage::kAttentionOnly)
            return err;
    }
    return launch_merge(p.part_lse, p.part_o, p.part_exact, p.out, p.lse, p.T, p.H, p.S, stream);
}

}  // namespace smla
