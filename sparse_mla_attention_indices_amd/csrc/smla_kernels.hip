// smla_kernels.hip -- CDNA4 (gfx950) kernels for sparse MLA forward over top-k
// indices: index conversion, the fused gather(+dequant) -> QK^T -> online
// softmax -> PV attention core, and the log-sum-exp merge of top-k splits.
//
// What is computed follows the vLLM page "vllm/v1/attention/backends/mla/
// flashmla_sparse.py" (FLASHMLA_SPARSE backend): the index conversion of
// triton_convert_req_index_to_global_index (docstring and kernel), the
// fp8_ds_mla row format of the module note, and the multi-query attention with
// 576-wide keys and 512-wide values that FlashMLASparseImpl.forward runs for
// both cache formats. How it is computed here is this library's own design for
// 64-wide wavefronts, MFMA and a 160 KB LDS:
//
//  * One workgroup = 4 waves = one query token x up to 64 heads x one top-k
//    split. Every head of the token shares each gathered 64-row tile.
//  * The workgroup first converts its part of the token's top-k list to cache
//    slots and compacts the valid ones into LDS, so whole tiles of -1 cost
//    nothing and only the last tile is ragged.
//  * Gather: each thread loads 16-byte pieces of four rows, converts e4m3 to
//    bf16 exactly (or takes bf16 as is), and writes the tile twice into LDS:
//    row-major (the K operand of QK^T) and transposed (the V operand of PV,
//    whose contraction runs over rows). The fp8 rows' per-128 scales are kept
//    apart in fp32 and applied to the 128-column partial sums of QK^T and to
//    the softmax weights of each 128-wide output group, so the dequantisation
//    itself adds no rounding.
//  * QK^T is computed transposed, S^T = K q^T, with v_mfma_f32_16x16x32_bf16,
//    q held in registers for the whole workgroup. The accumulator layout of
//    S^T gives every lane one head and 4 rows per 16-row block, which is
//    exactly the B-operand layout of O^T += V^T P^T: softmax weights go from
//    the S^T accumulators to the PV MFMA without an LDS round trip, and the
//    row max / row sum need only two cross-lane exchanges.
//  * O^T (16 heads x 512 per wave) stays in registers; at the end the waves
//    stage it through LDS, merge the row splits of small-head configurations,
//    and write coalesced bf16 output (or fp32 partials for a top-k split).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef float f32x2 __attribute__((__vector_size__(8)));

constexpr int kThreads = 256;                 // 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 64;                     // cache rows per tile
constexpr int kKSteps = kDqk / 32;            // 18 MFMA k-steps over the 576 columns
constexpr int kMaxChunk = 2048;               // top-k positions compacted per round
constexpr int kKStride = kDqk * 2 + 16;       // bytes per row of the row-major K tile
constexpr int kVtStride = kTile * 2 + 16;     // bytes per row of the transposed V tile
constexpr int kLdsK = kTile * kKStride;       // 74752
constexpr int kLdsVt = kDv * kVtStride;       // 73728
constexpr int kLdsSlots = kMaxChunk * 4;      // 8192
constexpr int kLdsScale = 4 * kTile * 4;     // fp8 scales of the tile, [group][row] fp32
constexpr int kLdsMisc = 64;
constexpr int kLdsBytes = kLdsK + kLdsVt + kLdsSlots + kLdsScale + kLdsMisc;
constexpr int kOStride = kDv + 4;             // floats per staged output row (padded)
constexpr int kExactPRows = 128;              // lists this short take P as hi + lo bf16 terms
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
static_assert(kWaves * 16 * (kOStride + 2) * 4 <= kLdsK + kLdsVt, "output staging fits the tile region");

struct KParams {
    const uint16_t *q;
    const uint8_t *cache;
    const int32_t *bt;
    const int32_t *req_id;
    const int32_t *topk;
    uint16_t *out;
    float *lse;
    int32_t *phys_out;
    float *part_o;
    float *part_lse;
    float sm_scale;
    float log2e_scale;   // sm_scale * log2(e): softmax runs on exp2
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

// bf16 rounding of what is left of four fp32 values after their bf16 rounding
// `w` (two packed pairs): the low term of a two-term bf16 split.
__device__ __forceinline__ uint2 bf16_residual2(const f32x4 &v, uint2 w)
{
    return make_uint2(pack_bf16(v[0] - bf16_lo(w.x), v[1] - bf16_hi(w.x)),
                      pack_bf16(v[2] - bf16_lo(w.y), v[3] - bf16_hi(w.y)));
}

// Position of tile row 4*rq .. 4*rq+3 in a row of the transposed V tile.
// Within every 32-row chunk, rows 4a+i (a < 4) go to 8a+i and rows 16+4a+i to
// 8a+4+i, so the 8 values one lane feeds to a 16x16x32 MFMA (two S^T blocks'
// worth of rows 4g..4g+3 and 16+4g..16+4g+3) are 16 contiguous bytes.
__device__ __forceinline__ int vt_pos(int rq)
{
    const int q8 = rq & 7;
    return 32 * (rq >> 3) + (q8 < 4 ? 8 * q8 : 8 * (q8 - 4) + 4);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int w)
{
    return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// ---------------------------------------------------------------- gather

// fp8_ds_mla rows. Every e4m3 value is exactly a bf16 value, so the latent
// bytes are converted exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and
// the row's four fp32 scales go to lds_scale[group][row]; they are applied in
// fp32 to the QK^T partial sums and to the softmax weights, never rounded into
// the tile. RoPE (bf16) is copied as is.
template <bool kHighHalf>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t word)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, kHighHalf));
}

__device__ __forceinline__ void load_tile_fp8(const uint8_t *__restrict__ cache,
                                              const int32_t *slots, int n_tile,
                                              uint8_t *lds_k, uint8_t *lds_vt, float *lds_scale,
                                              int tid)
{
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
        const int u = tid + kThreads * ui;       // 16 row-quads x 32 pieces of 16 bytes
        const int rq = u >> 5, c = u & 31;
        uint4 raw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * rq + j;
            const int slot = r < n_tile ? slots[r] : -1;
            raw[j] = slot >= 0 ? *(const uint4 *)(cache + (size_t)slot * kFp8RowBytes + 16 * c)
                               : make_uint4(0, 0, 0, 0);
        }
        uint32_t b[4][8];                        // row j: bf16 pairs (dims 2e, 2e+1)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                b[j][2 * w] = e4m3x2_to_bf16x2<false>(word_of(raw[j], w));
                b[j][2 * w + 1] = e4m3x2_to_bf16x2<true>(word_of(raw[j], w));
            }
            uint4 *dst = (uint4 *)(lds_k + (4 * rq + j) * kKStride + 32 * c);
            dst[0] = make_uint4(b[j][0], b[j][1], b[j][2], b[j][3]);
            dst[1] = make_uint4(b[j][4], b[j][5], b[j][6], b[j][7]);
        }
        const int vpos = vt_pos(rq);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int w = e >> 1;
            uint2 v;
            if (e & 1) {
                v.x = (b[0][w] >> 16) | (b[1][w] & 0xFFFF0000u);
                v.y = (b[2][w] >> 16) | (b[3][w] & 0xFFFF0000u);
            } else {
                v.x = (b[0][w] & 0xFFFFu) | (b[1][w] << 16);
                v.y = (b[2][w] & 0xFFFFu) | (b[3][w] << 16);
            }
            *(uint2 *)(lds_vt + (16 * c + e) * kVtStride + 2 * vpos) = v;
        }
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
        const int u = tid + kThreads * ui;       // 64 rows x 8 RoPE pieces of 16 bytes
        const int r = u >> 3, rc = u & 7;
        const int slot = r < n_tile ? slots[r] : -1;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (slot >= 0)
            v = *(const uint4 *)(cache + (size_t)slot * kFp8RowBytes + 528 + 16 * rc);
        *(uint4 *)(lds_k + r * kKStride + 1024 + 16 * rc) = v;
        if (rc == 0) {
            float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (slot >= 0)
                sc = *(const float4 *)(cache + (size_t)slot * kFp8RowBytes + 512);
            lds_scale[0 * kTile + r] = sc.x;
            lds_scale[1 * kTile + r] = sc.y;
            lds_scale[2 * kTile + r] = sc.z;
            lds_scale[3 * kTile + r] = sc.w;
        }
    }
}

// bf16 rows: copied to the row-major tile, transposed into the V tile.
__device__ __forceinline__ void load_tile_bf16(const uint8_t *__restrict__ cache,
                                               const int32_t *slots, int n_tile,
                                               uint8_t *lds_k, uint8_t *lds_vt, int tid)
{
#pragma unroll
    for (int ui = 0; ui < 4; ++ui) {
        const int u = tid + kThreads * ui;       // 16 row-quads x 64 pieces of 8 values
        const int rq = u >> 6, c = u & 63;
        uint4 raw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * rq + j;
            const int slot = r < n_tile ? slots[r] : -1;
            raw[j] = slot >= 0 ? *(const uint4 *)(cache + (size_t)slot * kBf16RowBytes + 16 * c)
                               : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(uint4 *)(lds_k + (4 * rq + j) * kKStride + 16 * c) = raw[j];
        const int vpos = vt_pos(rq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const uint32_t a0 = word_of(raw[0], w), a1 = word_of(raw[1], w);
            const uint32_t a2 = word_of(raw[2], w), a3 = word_of(raw[3], w);
            uint2 v;
            if (e & 1) {
                v.x = (a0 >> 16) | (a1 & 0xFFFF0000u);
                v.y = (a2 >> 16) | (a3 & 0xFFFF0000u);
            } else {
                v.x = (a0 & 0xFFFFu) | (a1 << 16);
                v.y = (a2 & 0xFFFFu) | (a3 << 16);
            }
            *(uint2 *)(lds_vt + (8 * c + e) * kVtStride + 2 * vpos) = v;
        }
    }
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
        const int u = tid + kThreads * ui;
        const int r = u >> 3, rc = u & 7;
        const int slot = r < n_tile ? slots[r] : -1;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (slot >= 0)
            v = *(const uint4 *)(cache + (size_t)slot * kBf16RowBytes + 1024 + 16 * rc);
        *(uint4 *)(lds_k + r * kKStride + 1024 + 16 * rc) = v;
    }
}

// ------------------------------------------------------------- attention

// KW = waves sharing one group of 16 heads (they split each tile's rows):
// 1 for h_q >= 64, 2 for h_q = 32, 4 for h_q = 16.
template <int FMT, int KW>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(const KParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
    uint8_t *lds_k = smem;
    uint8_t *lds_vt = smem + kLdsK;
    int32_t *lds_slots = (int32_t *)(smem + kLdsK + kLdsVt);
    float *lds_scale = (float *)(smem + kLdsK + kLdsVt + kLdsSlots);
    int32_t *lds_misc = (int32_t *)(smem + kLdsK + kLdsVt + kLdsSlots + kLdsScale);

    constexpr int HG = kWaves / KW;      // groups of 16 heads in this workgroup
    constexpr int RW = kTile / KW;       // tile rows per wave
    constexpr int NBLK = RW / 16;        // 16-row S^T blocks per wave

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, n16 = lane & 15;
    const int hg = wave / KW, kw = wave % KW;

    int bid = blockIdx.x;
    const int s = bid % p.S;
    bid /= p.S;
    const int hb = bid % p.HB;
    const int t = bid / p.HB;

    const int head_base = hb * kHeadsPerGroup;
    const int h = head_base + hg * 16 + n16;
    const int req = p.req_id[t];

    // q^T as the B operand of S^T = K q^T: lane (head n16, group g) holds columns
    // 32k + 8g .. 32k + 8g + 7 for k = 0..17.
    bf16x8 qb[kKSteps];
    {
        const uint4 *qp = (const uint4 *)(p.q + ((size_t)t * p.H + h) * kDqk + 8 * g);
#pragma unroll
        for (int k = 0; k < kKSteps; ++k)
            qb[k] = __builtin_bit_cast(bf16x8, qp[4 * k]);
    }

    f32x4 o[32];                         // O^T: dims 16*db + 4g + i, head n16
#pragma unroll
    for (int i = 0; i < 32; ++i)
        o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;             // running max of raw (unscaled) logits
    float l_run = 0.f;
    const float c2 = p.log2e_scale;

    const int pos_begin = s * p.split_len;
    const int pos_end = min(p.K, pos_begin + p.split_len);
    const int32_t *topk_row = p.topk + (size_t)t * p.K;

    for (int chunk0 = pos_begin; chunk0 < pos_end; chunk0 += kMaxChunk) {
        const int chunk_n = min(kMaxChunk, pos_end - chunk0);

        // ---- convert this chunk's positions and compact the valid slots
        int n_valid = 0;
        for (int i0 = 0; i0 < chunk_n; i0 += kThreads) {
            const int i = i0 + tid;
            int slot = -1;
            if (i < chunk_n) {
                slot = convert_slot(req, topk_row[chunk0 + i], p.bt, p.R, p.MB, p.NB);
                if (p.phys_out != nullptr && hb == 0)
                    p.phys_out[(size_t)t * p.K + chunk0 + i] = slot;
            }
            const bool valid = slot >= 0;
            const uint64_t mask = __ballot(valid);
            const int rank = __popcll(mask & ((1ull << lane) - 1ull));
            if (lane == 0)
                lds_misc[wave] = __popcll(mask);
            __syncthreads();
            int before = 0, total = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const int cw = lds_misc[w];
                before += w < wave ? cw : 0;
                total += cw;
            }
            if (valid)
                lds_slots[n_valid + before + rank] = slot;
            n_valid += total;
            __syncthreads();
        }

        // A short list puts large weights on few rows: use the two-term P.
        const bool exact_p = n_valid <= kExactPRows;

        // ---- tiles of 64 gathered rows
        for (int tile0 = 0; tile0 < n_valid; tile0 += kTile) {
            const int n_tile = min(kTile, n_valid - tile0);
            if (FMT == kCacheFp8)
                load_tile_fp8(p.cache, lds_slots + tile0, n_tile, lds_k, lds_vt, lds_scale, tid);
            else
                load_tile_bf16(p.cache, lds_slots + tile0, n_tile, lds_k, lds_vt, tid);
            __syncthreads();

            const int row_base = kw * RW;
            f32x4 acc[NBLK];
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
                acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (FMT == kCacheFp8) {
                // latent columns in four 128-wide groups, each partial sum times its
                // rows' scale (lane rows row_base + 16b + 4g + i), then RoPE unscaled
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    f32x4 part[NBLK];
#pragma unroll
                    for (int b = 0; b < NBLK; ++b)
                        part[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int k = 4 * grp + kk;
#pragma unroll
                        for (int b = 0; b < NBLK; ++b) {
                            const bf16x8 a = *(const bf16x8 *)(lds_k + (row_base + 16 * b + n16) * kKStride +
                                                               (32 * k + 8 * g) * 2);
                            part[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[k], part[b], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int b = 0; b < NBLK; ++b) {
                        const f32x4 sc = *(const f32x4 *)(lds_scale + grp * kTile + row_base + 16 * b + 4 * g);
                        acc[b] += sc * part[b];
                    }
                }
#pragma unroll
                for (int k = 16; k < kKSteps; ++k) {
#pragma unroll
                    for (int b = 0; b < NBLK; ++b) {
                        const bf16x8 a = *(const bf16x8 *)(lds_k + (row_base + 16 * b + n16) * kKStride +
                                                           (32 * k + 8 * g) * 2);
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[k], acc[b], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < kKSteps; ++k) {
#pragma unroll
                    for (int b = 0; b < NBLK; ++b) {
                        const bf16x8 a = *(const bf16x8 *)(lds_k + (row_base + 16 * b + n16) * kKStride +
                                                           (32 * k + 8 * g) * 2);
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[k], acc[b], 0, 0, 0);
                    }
                }
            }

            // online softmax over this wave's rows (lane: head n16, rows 16b + 4g + i)
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (row_base + 16 * b + 4 * g + i >= n_tile)
                        acc[b][i] = -INFINITY;
                    mx = fmaxf(mx, acc[b][i]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            float alpha = 1.f, rs = 0.f;
            if (m_new != -INFINITY) {
                alpha = exp2f((m_run - m_new) * c2);
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[b][i] = exp2f((acc[b][i] - m_new) * c2);
                        rs += acc[b][i];
                    }
            } else {
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
                    acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            rs += __shfl_xor(rs, 16);
            rs += __shfl_xor(rs, 32);
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                o[i] *= alpha;

            // O^T += V^T P^T. Output dims 128*grp .. 128*grp+127 take the weights
            // times their rows' scale of group grp (fp8; 1 for bf16 rows). For a
            // short list (exact_p) every weight is large and its bf16 rounding would
            // show in the output, so P goes in as two bf16 terms, hi + lo, against the
            // same V^T operand.
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                if constexpr (KW == 4) {
                    f32x4 pv = acc[0];
                    if constexpr (FMT == kCacheFp8)
                        pv *= *(const f32x4 *)(lds_scale + grp * kTile + row_base + 4 * g);
                    const uint2 pw = make_uint2(pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]));
                    const i16x4 pb = __builtin_bit_cast(i16x4, pw);
                    const i16x4 pl = __builtin_bit_cast(i16x4, bf16_residual2(pv, pw));
                    const int col = 32 * (kw >> 1) + 8 * g + 4 * (kw & 1);
#pragma unroll
                    for (int d8 = 0; d8 < 8; ++d8) {
                        const int db = 8 * grp + d8;
                        const i16x4 a = *(const i16x4 *)(lds_vt + (16 * db + n16) * kVtStride + 2 * col);
                        o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[db], 0, 0, 0);
                        if (exact_p)
                            o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, o[db], 0, 0, 0);
                    }
                } else {
                    constexpr int NCH = NBLK / 2;
                    bf16x8 pb[NCH], pl[NCH];
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) {
                        f32x4 p0 = acc[2 * ch], p1 = acc[2 * ch + 1];
                        if constexpr (FMT == kCacheFp8) {
                            const float *sg = lds_scale + grp * kTile + row_base + 32 * ch + 4 * g;
                            p0 *= *(const f32x4 *)sg;
                            p1 *= *(const f32x4 *)(sg + 16);
                        }
                        const uint4 pw = make_uint4(pack_bf16(p0[0], p0[1]), pack_bf16(p0[2], p0[3]),
                                                    pack_bf16(p1[0], p1[1]), pack_bf16(p1[2], p1[3]));
                        pb[ch] = __builtin_bit_cast(bf16x8, pw);
                        const uint2 r0 = bf16_residual2(p0, make_uint2(pw.x, pw.y));
                        const uint2 r1 = bf16_residual2(p1, make_uint2(pw.z, pw.w));
                        pl[ch] = __builtin_bit_cast(bf16x8, make_uint4(r0.x, r0.y, r1.x, r1.y));
                    }
#pragma unroll
                    for (int d8 = 0; d8 < 8; ++d8) {
                        const int db = 8 * grp + d8;
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch) {
                            const int chunk = KW == 1 ? ch : kw;
                            const bf16x8 a = *(const bf16x8 *)(lds_vt + (16 * db + n16) * kVtStride +
                                                               2 * (32 * chunk + 8 * g));
                            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[ch], o[db], 0, 0, 0);
                            if (exact_p)
                                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[ch], o[db], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();
        }
    }

    // ---- stage O^T and (m, l) of every wave, merge row splits, write out
    float *ofin = (float *)smem;                       // [wave][16 heads][kOStride]
    float *mlfin = ofin + kWaves * 16 * kOStride;      // [wave][16 heads][m, l]
#pragma unroll
    for (int db = 0; db < 32; ++db)
        *(f32x4 *)(ofin + (wave * 16 + n16) * kOStride + 16 * db + 4 * g) = o[db];
    if (g == 0) {
        mlfin[(wave * 16 + n16) * 2 + 0] = m_run;
        mlfin[(wave * 16 + n16) * 2 + 1] = l_run;
    }
    __syncthreads();

    for (int u = tid; u < HG * 16 * 64; u += kThreads) {
        const int hh = u >> 6, d0 = (u & 63) * 8;
        const int j = hh & 15, w0 = (hh >> 4) * KW;
        float M = -INFINITY;
#pragma unroll
        for (int k2 = 0; k2 < KW; ++k2)
            M = fmaxf(M, mlfin[((w0 + k2) * 16 + j) * 2]);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int k2 = 0; k2 < KW; ++k2) {
                const int w = w0 + k2;
                const float sc = exp2f((mlfin[(w * 16 + j) * 2] - M) * c2);
                L += sc * mlfin[(w * 16 + j) * 2 + 1];
                const float *src = ofin + (w * 16 + j) * kOStride + d0;
                const f32x4 a = *(const f32x4 *)src, b = *(const f32x4 *)(src + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] += sc * a[e];
                    v[4 + e] += sc * b[e];
                }
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float lse_v = L > 0.f ? M * p.sm_scale + logf(L) : -INFINITY;
        const int head = head_base + hh;
        if (p.S == 1) {
            *(uint4 *)(p.out + ((size_t)t * p.H + head) * kDv + d0) =
                make_uint4(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv),
                           pack_bf16(v[4] * inv, v[5] * inv), pack_bf16(v[6] * inv, v[7] * inv));
            if (d0 == 0 && p.lse != nullptr)
                p.lse[(size_t)t * p.H + head] = lse_v;
        } else {
            float *dst = p.part_o + (((size_t)t * p.S + s) * p.H + head) * kDv + d0;
            *(f32x4 *)dst = f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
            *(f32x4 *)(dst + 4) = f32x4{v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv};
            if (d0 == 0)
                p.part_lse[((size_t)t * p.S + s) * p.H + head] = lse_v;
        }
    }
}

// Combine the top-k splits of every (token, head): weights exp(lse_s - max).
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ part_o,
                                                    const float *__restrict__ part_lse,
                                                    uint16_t *__restrict__ out, float *__restrict__ lse,
                                                    int T, int H, int S)
{
    const int64_t units = (int64_t)T * H * 64;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * 256) {
        const int64_t th = u >> 6;
        const int d0 = (int)(u & 63) * 8;
        const int t = (int)(th / H), h = (int)(th % H);
        float M = -INFINITY;
        for (int s = 0; s < S; ++s)
            M = fmaxf(M, part_lse[((size_t)t * S + s) * H + h]);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < S; ++s) {
                const float w = expf(part_lse[((size_t)t * S + s) * H + h] - M);
                W += w;
                const float *src = part_o + (((size_t)t * S + s) * H + h) * kDv + d0;
                const f32x4 a = *(const f32x4 *)src, b = *(const f32x4 *)(src + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] += w * a[e];
                    v[4 + e] += w * b[e];
                }
            }
        }
        const float inv = W > 0.f ? 1.f / W : 0.f;
        *(uint4 *)(out + ((size_t)t * H + h) * kDv + d0) =
            make_uint4(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv),
                       pack_bf16(v[4] * inv, v[5] * inv), pack_bf16(v[6] * inv, v[7] * inv));
        if (d0 == 0 && lse != nullptr)
            lse[(size_t)t * H + h] = W > 0.f ? M + logf(W) : -INFINITY;
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

template <int FMT>
hipError_t launch_attn_fmt(const KParams &p, int kw, dim3 grid, hipStream_t stream)
{
    if (kw == 1)
        hipLaunchKernelGGL((attn_kernel<FMT, 1>), grid, dim3(kThreads), 0, stream, p);
    else if (kw == 2)
        hipLaunchKernelGGL((attn_kernel<FMT, 2>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_kernel<FMT, 4>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
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
    p.part_o = pl.num_splits > 1 ? (float *)((char *)a.workspace + pl.part_o_off) : nullptr;
    p.part_lse = pl.num_splits > 1 ? (float *)((char *)a.workspace + pl.part_lse_off) : nullptr;
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
    const int kw = a.h_q >= kHeadsPerGroup ? 1 : (a.h_q == 32 ? 2 : 4);
    const dim3 grid((unsigned)((int64_t)a.num_tokens * pl.head_blocks * pl.num_splits));
    hipError_t err = fmt == kCacheFp8 ? launch_attn_fmt<kCacheFp8>(p, kw, grid, stream)
                                      : launch_attn_fmt<kCacheBf16>(p, kw, grid, stream);
    if (err != hipSuccess || pl.num_splits == 1)
        return err;
    const int64_t units = (int64_t)a.num_tokens * a.h_q * 64;
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                       stream, p.part_o, p.part_lse, p.out, p.lse, p.T, p.H, p.S);
    return hipGetLastError();
}

}  // namespace smla
