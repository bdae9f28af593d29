// smla_kernels.hip -- CDNA4 (gfx950) kernels for sparse MLA forward over top-k
// indices: index conversion, and the fused gather -> QK^T -> online softmax ->
// PV attention kernel with an in-kernel log-sum-exp merge of top-k splits.
//
// What is computed follows the vLLM page "vllm/v1/attention/backends/mla/
// flashmla_sparse.py" (FLASHMLA_SPARSE backend): the index conversion of
// triton_convert_req_index_to_global_index (docstring and kernel), the
// fp8_ds_mla row format of the module note, and the multi-query attention with
// 576-wide keys and 512-wide values that FlashMLASparseImpl.forward runs for
// both cache formats. How it is computed here is this library's own design for
// 64-wide wavefronts, MFMA and the 160 KB LDS of a gfx950 compute unit:
//
//  * Workgroup = one query token x up to 64 heads x one part ("split") of the
//    token's top-k list. Waves: two halves of the 576 columns ("dh") x one or
//    two groups of up to 32 heads ("hh"). Every wave sees every row.
//  * Prologue: the workgroup converts its part of the top-k list to cache
//    slots and compacts the valid ones into LDS (whole runs of -1 cost
//    nothing; only the last tile is ragged).
//  * Gather: global_load_lds_dwordx4 copies the cache rows of a 32-row tile,
//    as stored (fp8_ds_mla 656 B or bf16 1152 B), straight into one of a ring
//    of LDS buffers; the next tiles are in flight while this one is used.
//  * QK^T runs transposed, S^T = K q^T, on v_mfma_f32_16x16x32_bf16 with q in
//    registers. Each wave reads its half of the columns for 16-row blocks
//    (ds_read_b64 of fp8 bytes or ds_read_b128 of bf16), converts fp8 to bf16
//    exactly in registers (every e4m3 value is a bf16 value) and feeds one
//    fragment to the MFMAs of both its 16-head blocks. fp8 partial sums of each
//    128-column group are multiplied by that group's row scales in fp32. The
//    two column halves exchange their partial S^T through LDS.
//  * Softmax: the S^T accumulator layout gives a lane one head and four rows
//    per block, so row max / row sum take two cross-lane steps, and the weights
//    are already in the B-operand layout of O^T += V^T P^T. The running max is
//    only moved (and O rescaled) when the tile max exceeds it by 2^8.
//  * PV reads V straight from the row-major raw tile with the gfx950 LDS
//    transpose loads (ds_read_b64_tr_b8 for fp8, ds_read_b64_tr_b16 for bf16).
//    For fp8 the weights of each 128-wide output group carry that group's row
//    scales, so dequantisation adds no rounding anywhere.
//  * A short list (few valid rows) puts large weights on few rows; then P goes
//    into PV as two bf16 terms, hi + lo.
//  * Splits of one token run on one XCD (workgroup id mod 8). Each writes fp32
//    partials; the last to finish (atomic counter) merges them by log-sum-exp
//    weights and writes the bf16 output, so no separate merge pass runs.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef int i32x2 __attribute__((__vector_size__(8)));
typedef float f32x4 __attribute__((__vector_size__(16)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int kTile = 32;             // cache rows per tile
constexpr int kRB = kTile / 16;       // 16-row MFMA blocks per tile
constexpr int kMaxChunk = 2048;       // top-k positions compacted into LDS per round
constexpr int kExactPRows = 128;      // lists this short feed P to PV as hi + lo bf16
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max moves

template <int FMT> struct RowFmt;
template <> struct RowFmt<kCacheFp8> {
    static constexpr int kBytes = kFp8RowBytes;   // 512 e4m3 | 4 x fp32 scale | 64 x bf16 RoPE
    static constexpr int kRope = 528;
};
template <> struct RowFmt<kCacheBf16> {
    static constexpr int kBytes = kBf16RowBytes;  // 512 x bf16 latent | 64 x bf16 RoPE
    static constexpr int kRope = 1024;
};

// Compile-time shape of one kernel instantiation.
template <int FMT, int HPW, int NHH>
struct Cfg {
    static constexpr int kWaves = 2 * NHH;                 // (dh, hh)
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kHBW = HPW / 16;                  // 16-head blocks per wave
    static constexpr int kHeads = HPW * NHH;               // heads per workgroup
    static constexpr int kRowBytes = RowFmt<FMT>::kBytes;
    static constexpr int kChunksPerRow = kRowBytes / 16;
    static constexpr int kTileChunks = kTile * kChunksPerRow;
    static constexpr int kDmaInstr = (kTileChunks + 63) / 64;        // wave instructions per tile
    static constexpr int kBufBytes = kDmaInstr * 1024;               // ring buffer stride
    // Four waves hold one workgroup per CU: deep ring. Two waves: two
    // workgroups per CU share the LDS.
    static constexpr int kNBuf = FMT == kCacheFp8 ? (NHH == 2 ? 4 : 3) : (NHH == 2 ? 3 : 2);
    static constexpr int kXchgBytes = kWaves * kRB * kHBW * 1024;    // partial S^T exchange
    static constexpr int kSlotsBytes = kMaxChunk * 4;
    static constexpr int kOffXchg = kNBuf * kBufBytes;
    static constexpr int kOffSlots = kOffXchg + kXchgBytes;
    static constexpr int kOffMisc = kOffSlots + kSlotsBytes;
    static constexpr int kLdsBytes = kOffMisc + 512;   // flags + per-wave counts of compaction
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one gfx950 workgroup");
    static_assert(kHeads * kDv * 2 <= kOffSlots, "bf16 output staging fits the ring + exchange");
};

struct KParams {
    const uint16_t *q;
    const uint8_t *cache;
    const int32_t *bt;
    const int32_t *req_id;
    const int32_t *topk;
    uint16_t *out;
    float *lse;
    int32_t *phys_out;
    float *part_o;        // [T][S][H][512] fp32, O / l of each split
    float *part_lse;      // [T][S][H]
    int32_t *counters;    // [T][HB] arrivals of a token's splits
    float sm_scale;
    float log2e_scale;    // sm_scale * log2(e): logits are kept in log2 units
    int T, H, K, R, MB;
    int64_t NB;
    int S, split_len, HB;
};

__device__ __forceinline__ int convert_slot(int req, int idx, const int32_t *__restrict__ bt,
                                            int num_reqs, int max_blocks, int64_t num_blocks)
{
    if ((unsigned)req >= (unsigned)num_reqs || idx < 0)
        return -1;
    const int blk = idx >> 6;
    if (blk >= max_blocks)
        return -1;
    const int base = bt[(size_t)req * max_blocks + blk];
    if (base < 0 || (int64_t)base >= num_blocks)
        return -1;
    return base * kBlock + (idx & (kBlock - 1));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v;
    v[0] = (__bf16)a;   // round to nearest even (v_cvt_pk_bf16_f32)
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight e4m3 bytes -> eight bf16 values, exactly (scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint2 v)
{
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
    return __builtin_bit_cast(bf16x8, r);
}

// P^T block (two 16-row blocks x 4 rows of one head) as the bf16 B operand of a
// 16x16x32 MFMA, plus the bf16 rounding of its residual.
__device__ __forceinline__ void pack_p(const f32x4 &p0, const f32x4 &p1, bf16x8 &hi, bf16x8 &lo)
{
    const uint4 w = make_uint4(pack_bf16(p0[0], p0[1]), pack_bf16(p0[2], p0[3]),
                               pack_bf16(p1[0], p1[1]), pack_bf16(p1[2], p1[3]));
    hi = __builtin_bit_cast(bf16x8, w);
    const uint4 r = make_uint4(pack_bf16(p0[0] - bf16_lo(w.x), p0[1] - bf16_hi(w.x)),
                               pack_bf16(p0[2] - bf16_lo(w.y), p0[3] - bf16_hi(w.y)),
                               pack_bf16(p1[0] - bf16_lo(w.z), p1[1] - bf16_hi(w.z)),
                               pack_bf16(p1[2] - bf16_lo(w.w), p1[3] - bf16_hi(w.w)));
    lo = __builtin_bit_cast(bf16x8, r);
}

// Wait until at most n of this wave's vector-memory instructions are pending
// (n is wave-uniform; values above 31 wait for all).
__device__ __forceinline__ void wait_vmcnt(int n)
{
#define SMLA_VMCNT_CASE(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    switch (n) {
        SMLA_VMCNT_CASE(1) SMLA_VMCNT_CASE(2) SMLA_VMCNT_CASE(3)
        SMLA_VMCNT_CASE(4) SMLA_VMCNT_CASE(5) SMLA_VMCNT_CASE(6) SMLA_VMCNT_CASE(7)
        SMLA_VMCNT_CASE(8) SMLA_VMCNT_CASE(9) SMLA_VMCNT_CASE(10) SMLA_VMCNT_CASE(11)
        SMLA_VMCNT_CASE(12) SMLA_VMCNT_CASE(13) SMLA_VMCNT_CASE(14) SMLA_VMCNT_CASE(15)
        SMLA_VMCNT_CASE(16) SMLA_VMCNT_CASE(17) SMLA_VMCNT_CASE(18) SMLA_VMCNT_CASE(19)
        SMLA_VMCNT_CASE(20) SMLA_VMCNT_CASE(21) SMLA_VMCNT_CASE(22) SMLA_VMCNT_CASE(23)
        SMLA_VMCNT_CASE(24) SMLA_VMCNT_CASE(25) SMLA_VMCNT_CASE(26) SMLA_VMCNT_CASE(27)
        SMLA_VMCNT_CASE(28) SMLA_VMCNT_CASE(29) SMLA_VMCNT_CASE(30) SMLA_VMCNT_CASE(31)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef SMLA_VMCNT_CASE
}

// Copy the rows of one tile, as stored, into an LDS ring buffer (row-major,
// row stride = row bytes). Wave w issues instructions w, w + W, ...; each moves
// 64 consecutive 16-byte pieces. Rows past the tile's valid count repeat the
// tile's first row (finite data whose weights are masked to zero).
template <class C>
__device__ __forceinline__ void issue_tile(const uint8_t *__restrict__ cache, const int32_t *slots,
                                           int n_tile, uint8_t *buf, int wave, int lane)
{
    for (int j = wave; j < C::kDmaInstr; j += C::kWaves) {
        const int piece = j * 64 + lane;
        if (piece < C::kTileChunks) {
            const int r = piece / C::kChunksPerRow;
            const int c = piece - r * C::kChunksPerRow;
            const int slot = slots[r < n_tile ? r : 0];
            const uint8_t *src = cache + (size_t)slot * C::kRowBytes + 16 * c;
            __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, buf + j * 1024), 16, 0, 0);
        }
    }
}

// ------------------------------------------------------------- attention

// Device-scope (sc1) stores and loads, visible to every compute unit once they
// have completed. Used for the split partials, so publishing them needs no
// L2-wide write-back. The stores are relaxed agent-scope atomics (the compiler
// tracks their hazards); the loads carry their own wait.
__device__ __forceinline__ void store_dev_x4(float *addr, const f32x4 &v)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        __hip_atomic_store(addr + e, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two device-scope 16-byte loads; the wait is inside the same statement, so no
// use of the results can be scheduled before the data has arrived.
__device__ __forceinline__ void load_dev_2x4(const float *a0, const float *a1, f32x4 &v0, f32x4 &v1)
{
    asm volatile("global_load_dwordx4 %0, %2, off sc1\n\t"
                 "global_load_dwordx4 %1, %3, off sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(v0), "=&v"(v1)
                 : "v"(a0), "v"(a1)
                 : "memory");
}

template <int FMT, int HPW, int NHH>
__global__ __launch_bounds__(128 * NHH, 1) void attn_kernel(const KParams p)
{
    using C = Cfg<FMT, HPW, NHH>;
    constexpr int HBW = C::kHBW;
    constexpr int RB = kRB;
    constexpr int ROWB = C::kRowBytes;
    constexpr int kPer = kMaxChunk / C::kThreads;    // top-k positions per thread per round

    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLdsBytes];
    uint8_t *ring = smem;
    f32x4 *xchg = (f32x4 *)(smem + C::kOffXchg);
    int32_t *lds_slots = (int32_t *)(smem + C::kOffSlots);
    int32_t *lds_misc = (int32_t *)(smem + C::kOffMisc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, n16 = lane & 15;
    const int dh = wave & 1, hh = wave >> 1;

    // Workgroup id -> (token, split, head block); all workgroups of one token
    // get the same id mod 8, i.e. the same XCD and L2.
    int bid = blockIdx.x;
    const int xcd = bid & 7;
    bid >>= 3;
    const int hb_wg = bid % p.HB;
    bid /= p.HB;
    const int s = bid % p.S;
    const int t = (bid / p.S) * 8 + xcd;
    if (t >= p.T)
        return;

    const int head0 = hb_wg * C::kHeads + hh * HPW;     // first head of this wave
    const float c2 = p.log2e_scale;
    const int pos_begin = s * p.split_len;
    const int pos_end = min(p.K, pos_begin + p.split_len);
    const int32_t *topk_row = p.topk + (size_t)t * p.K;
    // one workgroup of the token's head blocks writes the converted slots
    const bool write_phys = p.phys_out != nullptr && hb_wg == 0;

    // Issue the first round's index loads, the request id and q together.
    int idxv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = pos_begin + tid + C::kThreads * j;
        idxv[j] = i < min(pos_end, pos_begin + kMaxChunk) ? topk_row[i] : -1;
    }
    const int req = p.req_id[t];

    // q^T B operands: lane (head n16 of block hb, group g) holds 8 columns per
    // k-step: latent 256*dh + 32k + 8g (k < 8), RoPE 512 + 32*dh + 8g (k = 8).
    bf16x8 qb[HBW][9];
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
        const uint16_t *qrow = p.q + ((size_t)t * p.H + head0 + 16 * hb + n16) * kDqk;
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            const int col = k < 8 ? 256 * dh + 32 * k + 8 * g : 512 + 32 * dh + 8 * g;
            qb[hb][k] = __builtin_bit_cast(bf16x8, *(const uint4 *)(qrow + col));
        }
    }

    f32x4 o[16][HBW];                   // O^T: dims 256*dh + 16*db + 4g + i, head n16 of hb
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int hb = 0; hb < HBW; ++hb)
            o[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // log2-domain running max (shared by the 4 lanes of a head) and this lane's
    // share of the running sum (its rows), per head
    float m_run[HBW], l_part[HBW];
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
        m_run[hb] = -INFINITY;
        l_part[hb] = 0.f;
    }

    for (int chunk0 = pos_begin; chunk0 < pos_end; chunk0 += kMaxChunk) {
        const int chunk_n = min(kMaxChunk, pos_end - chunk0);

        // ---- convert (all lookups in flight together), then compact the valid
        //      slots in list order with one exchange of per-wave counts
        int slotv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            slotv[j] = convert_slot(req, idxv[j], p.bt, p.R, p.MB, p.NB);
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
        int n_valid = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
#pragma unroll
            for (int w = 0; w < C::kWaves; ++w) {
                const int cw = lds_misc[16 + j * C::kWaves + w];
                if (w == wave && slotv[j] >= 0)
                    lds_slots[n_valid + __popcll(masks[j] & ((1ull << lane) - 1ull))] = slotv[j];
                n_valid += cw;
            }
        }
        __syncthreads();
        const bool exact_p = n_valid <= kExactPRows;
        const int n_tiles = (n_valid + kTile - 1) / kTile;
        // from here on the only vector-memory instructions in flight are tile copies
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // this wave's copy instructions per tile
        const int dma_w = (C::kDmaInstr - wave + C::kWaves - 1) / C::kWaves;

        for (int i = 0; i < min(C::kNBuf - 1, n_tiles); ++i)
            issue_tile<C>(p.cache, lds_slots + i * kTile, min(kTile, n_valid - i * kTile),
                          ring + i * C::kBufBytes, wave, lane);

        for (int it = 0; it < n_tiles; ++it) {
            const int n_tile = min(kTile, n_valid - it * kTile);
            const uint8_t *buf = ring + (it % C::kNBuf) * C::kBufBytes;
            wait_vmcnt(dma_w * min(C::kNBuf - 2, n_tiles - 1 - it));
            __syncthreads();     // every wave's pieces of tile `it` landed; tile it-1 is done
            if (it + C::kNBuf - 1 < n_tiles) {
                const int nt = it + C::kNBuf - 1;
                issue_tile<C>(p.cache, lds_slots + nt * kTile, min(kTile, n_valid - nt * kTile),
                              ring + (nt % C::kNBuf) * C::kBufBytes, wave, lane);
            }

            // ---- read this wave's K fragments (rows 16*rb + n16), all at once
            f32x4 acc[RB][HBW];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb)
                    acc[rb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 sc[2][RB];            // fp8: scales of rows 16*rb + 4g + i, groups 2*dh + gi
            if constexpr (FMT == kCacheFp8) {
                uint2 kf[2][4][RB];
                bf16x8 rf[RB];
#pragma unroll
                for (int gi = 0; gi < 2; ++gi)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
                            kf[gi][kk][rb] = *(const uint2 *)(buf + (16 * rb + n16) * ROWB +
                                                              128 * (2 * dh + gi) + 32 * kk + 8 * g);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    rf[rb] = *(const bf16x8 *)(buf + (16 * rb + n16) * ROWB + RowFmt<FMT>::kRope + 64 * dh + 16 * g);
#pragma unroll
                for (int gi = 0; gi < 2; ++gi)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sc[gi][rb][i] = *(const float *)(buf + (16 * rb + 4 * g + i) * ROWB + 512 + 4 * (2 * dh + gi));
                // S^T = K q^T: each 128-column group's partial sum times its row scales
#pragma unroll
                for (int gi = 0; gi < 2; ++gi) {
                    f32x4 part[RB][HBW];
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int hb = 0; hb < HBW; ++hb)
                            part[rb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            const bf16x8 a = e4m3x8_to_bf16x8(kf[gi][kk][rb]);
#pragma unroll
                            for (int hb = 0; hb < HBW; ++hb)
                                part[rb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    a, qb[hb][4 * gi + kk], part[rb][hb], 0, 0, 0);
                        }
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int hb = 0; hb < HBW; ++hb)
                            acc[rb][hb] += sc[gi][rb] * part[rb][hb];
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int hb = 0; hb < HBW; ++hb)
                        acc[rb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf[rb], qb[hb][8], acc[rb][hb], 0, 0, 0);
            } else {
#pragma unroll
                for (int k = 0; k < 9; ++k) {
                    const int col = k < 8 ? 2 * (256 * dh + 32 * k + 8 * g) : RowFmt<FMT>::kRope + 64 * dh + 16 * g;
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const bf16x8 a = *(const bf16x8 *)(buf + (16 * rb + n16) * ROWB + col);
#pragma unroll
                        for (int hb = 0; hb < HBW; ++hb)
                            acc[rb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[hb][k], acc[rb][hb], 0, 0, 0);
                    }
                }
            }

            // ---- V^T fragments for PV (independent of the softmax): read them now,
            //      so their latency hides behind the exchange barrier
            uint2 vf8[16];
            if constexpr (FMT == kCacheFp8) {
#pragma unroll
                for (int db = 0; db < 16; ++db) {
                    // source lane n16 = 2k + h: row k of {4g..4g+3, 16+4g..16+4g+3}, bytes 8h..8h+7
                    const int k = n16 >> 1;
                    const int row = (k < 4 ? 4 * g + k : 16 + 4 * g + (k - 4));
                    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        LDS_PTR(i32x2, buf + row * ROWB + 256 * dh + 16 * db + 8 * (n16 & 1)));
                    vf8[db] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
                }
            }

            // ---- add the other column half's partial S^T (same lane slots)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb)
                    xchg[((wave * RB + rb) * HBW + hb) * 64 + lane] = acc[rb][hb];
            __syncthreads();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb)
                    acc[rb][hb] += xchg[(((wave ^ 1) * RB + rb) * HBW + hb) * 64 + lane];

            // ---- online softmax in log2 units (rows 16*rb + 4g + i >= n_tile masked).
            //      The running max moves only when some row exceeds it by 2^8; the
            //      test uses each lane's own rows, the move uses the whole head's max.
            bool need = false;
            float lmax[HBW];
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb) {
                lmax[hb] = -INFINITY;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = 16 * rb + 4 * g + i < n_tile ? acc[rb][hb][i] * c2 : -INFINITY;
                        acc[rb][hb][i] = v;
                        lmax[hb] = fmaxf(lmax[hb], v);
                    }
                need |= lmax[hb] > m_run[hb] + kLazyRescale;
            }
            if (__ballot(need) != 0) {
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb) {
                    float mx = lmax[hb];
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    if (mx > m_run[hb] + kLazyRescale) {
                        const float alpha = m_run[hb] == -INFINITY ? 0.f : exp2f(m_run[hb] - mx);
                        l_part[hb] *= alpha;
#pragma unroll
                        for (int db = 0; db < 16; ++db)
                            o[db][hb] *= alpha;
                        m_run[hb] = mx;
                    }
                }
            }
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[rb][hb][i] = exp2f(acc[rb][hb][i] - m_run[hb]);
                        l_part[hb] += acc[rb][hb][i];
                    }

            // ---- O^T += V^T P^T over this wave's 256 output dims. fp8: the weights
            //      of output group 2*dh + gi carry that group's row scales.
            bf16x8 pb[2][HBW], pl[2][HBW];
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb) {
                    f32x4 p0 = acc[0][hb], p1 = acc[1][hb];
                    if constexpr (FMT == kCacheFp8) {
                        p0 *= sc[gi][0];
                        p1 *= sc[gi][1];
                    }
                    if (exact_p)
                        pack_p(p0, p1, pb[gi][hb], pl[gi][hb]);
                    else
                        pb[gi][hb] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(p0[0], p0[1]), pack_bf16(p0[2], p0[3]),
                                                                           pack_bf16(p1[0], p1[1]), pack_bf16(p1[2], p1[3])));
                }
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const int gi = db >> 3;
                bf16x8 a;
                if constexpr (FMT == kCacheFp8) {
                    a = e4m3x8_to_bf16x8(vf8[db]);
                } else {
                    // source lane n16 = 4k + a: row 4g + k (then 16 + 4g + k), dims 4a..4a+3
                    const int k = n16 >> 2;
                    const int colb = 2 * (256 * dh + 16 * db + 4 * (n16 & 3));
                    const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, buf + (4 * g + k) * ROWB + colb)));
                    const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        LDS_PTR(i16x4, buf + (16 + 4 * g + k) * ROWB + colb)));
                    a = __builtin_bit_cast(bf16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
                }
#pragma unroll
                for (int hb = 0; hb < HBW; ++hb)
                    o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[gi][hb], o[db][hb], 0, 0, 0);
                if (exact_p) {
#pragma unroll
                    for (int hb = 0; hb < HBW; ++hb)
                        o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[gi][hb], o[db][hb], 0, 0, 0);
                }
            }
        }
        __syncthreads();     // ring, exchange and slot list are free for the next round
        // the next round's indices
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = chunk0 + kMaxChunk + tid + C::kThreads * j;
            idxv[j] = i < pos_end ? topk_row[i] : -1;
        }
    }

    // ---- epilogue. m_run and the row sums are identical in both column halves.
    float inv_l[HBW], lse_v[HBW];
#pragma unroll
    for (int hb = 0; hb < HBW; ++hb) {
        float l = l_part[hb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        inv_l[hb] = l > 0.f ? 1.f / l : 0.f;
        lse_v[hb] = l > 0.f ? (m_run[hb] + log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
    const int wg_head0 = hb_wg * C::kHeads;

    if (p.S == 1) {
        // stage bf16 rows [head][512] in LDS, then write them out coalesced
        uint16_t *stage = (uint16_t *)smem;
#pragma unroll
        for (int db = 0; db < 16; ++db)
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb) {
                const f32x4 v = o[db][hb] * inv_l[hb];
                *(uint2 *)(stage + (hh * HPW + 16 * hb + n16) * kDv + 256 * dh + 16 * db + 4 * g) =
                    make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
            }
        if (dh == 0 && g == 0 && p.lse != nullptr)
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb)
                p.lse[(size_t)t * p.H + head0 + 16 * hb + n16] = lse_v[hb];
        __syncthreads();
        uint16_t *dst = p.out + ((size_t)t * p.H + wg_head0) * kDv;
        for (int u = tid; u < C::kHeads * kDv / 8; u += C::kThreads)
            *(uint4 *)(dst + 8 * u) = *(const uint4 *)(stage + 8 * u);
        return;
    }

    // ---- top-k split: publish the fp32 partial (O / l) and lse with device-scope
    //      stores, count this arrival; the last of the token's splits merges.
    {
        float *po = p.part_o + (((size_t)t * p.S + s) * p.H + head0) * kDv;
#pragma unroll
        for (int db = 0; db < 16; ++db)
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb)
                store_dev_x4(po + (16 * hb + n16) * kDv + 256 * dh + 16 * db + 4 * g, o[db][hb] * inv_l[hb]);
        if (dh == 0 && g == 0)
#pragma unroll
            for (int hb = 0; hb < HBW; ++hb)
                __hip_atomic_store(p.part_lse + ((size_t)t * p.S + s) * p.H + head0 + 16 * hb + n16, lse_v[hb],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // this thread's partial stores completed
    __syncthreads();
    if (tid == 0) {
        const int prev = atomicAdd(p.counters + (size_t)t * p.HB + hb_wg, 1);
        lds_misc[0] = prev == p.S - 1;
    }
    __syncthreads();
    if (!lds_misc[0])
        return;
    for (int u = tid; u < C::kHeads * (kDv / 8); u += C::kThreads) {
        const int hl = u / (kDv / 8);
        const int d0 = (u % (kDv / 8)) * 8;
        const int head = wg_head0 + hl;
        const size_t base = (size_t)t * p.S * p.H + head;
        float M = -INFINITY;
        for (int s2 = 0; s2 < p.S; ++s2)
            M = fmaxf(M, __hip_atomic_load(p.part_lse + base + (size_t)s2 * p.H, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
        if (M != -INFINITY) {
            for (int s2 = 0; s2 < p.S; ++s2) {
                const float w = expf(__hip_atomic_load(p.part_lse + base + (size_t)s2 * p.H, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT) - M);
                const float *src = p.part_o + (base + (size_t)s2 * p.H) * kDv + d0;
                f32x4 a, b;
                load_dev_2x4(src, src + 4, a, b);
                W += w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] += w * a[e];
                    v[4 + e] += w * b[e];
                }
            }
        }
        const float inv = W > 0.f ? 1.f / W : 0.f;
        *(uint4 *)(p.out + ((size_t)t * p.H + head) * kDv + d0) =
            make_uint4(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv),
                       pack_bf16(v[4] * inv, v[5] * inv), pack_bf16(v[6] * inv, v[7] * inv));
        if (d0 == 0 && p.lse != nullptr)
            p.lse[(size_t)t * p.H + head] = W > 0.f ? M + logf(W) : -INFINITY;
    }
}

__global__ __launch_bounds__(256) void zero_kernel(int32_t *__restrict__ p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        p[i] = 0;
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

template <int FMT, int HPW, int NHH>
hipError_t launch_one(const KParams &p, hipStream_t stream)
{
    using C = Cfg<FMT, HPW, NHH>;
    const int64_t tq = (p.T + 7) / 8;
    const dim3 grid((unsigned)(tq * 8 * p.S * p.HB));
    hipLaunchKernelGGL((attn_kernel<FMT, HPW, NHH>), grid, dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const KParams &p, hipStream_t stream)
{
    if (p.H >= 64)
        return launch_one<FMT, 32, 2>(p, stream);
    if (p.H == 32)
        return launch_one<FMT, 32, 1>(p, stream);
    return launch_one<FMT, 16, 1>(p, stream);
}

}  // namespace

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

hipError_t launch_attention(CacheFormat fmt, const AttnArgs &a, const Plan &pl, hipStream_t stream)
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
    const bool split = pl.num_splits > 1;
    p.part_o = split ? (float *)((char *)a.workspace + pl.part_o_off) : nullptr;
    p.part_lse = split ? (float *)((char *)a.workspace + pl.part_lse_off) : nullptr;
    p.counters = split ? (int32_t *)((char *)a.workspace + pl.counters_off) : nullptr;
    p.sm_scale = a.sm_scale;
    p.log2e_scale = a.sm_scale * 1.4426950408889634f;
    p.T = a.num_tokens;
    p.H = a.h_q;
    p.K = a.topk_len;
    p.R = a.num_reqs;
    p.MB = a.max_blocks;
    p.NB = a.num_blocks;
    p.S = pl.num_splits;
    p.split_len = pl.split_len;
    p.HB = pl.head_blocks;
    if (split) {
        const int n = a.num_tokens * pl.head_blocks;
        const int blocks = (n + 255) / 256;
        hipLaunchKernelGGL(zero_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, stream,
                           p.counters, n);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return fmt == kCacheFp8 ? launch_fmt<kCacheFp8>(p, stream) : launch_fmt<kCacheBf16>(p, stream);
}

}  // namespace smla
