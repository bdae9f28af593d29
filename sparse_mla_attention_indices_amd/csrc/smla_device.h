// smla_device.h -- device-side pieces shared by the attention kernels of
// smla_kernels.hip and smla_attn128.hip: vector types, tile constants, the
// fp8_ds_mla / bf16 row formats, the kernel parameter block, index conversion,
// bf16 and e4m3 conversions, the explicit vector-memory waits and the
// copy-into-LDS helpers. Everything is file-local (anonymous namespace), so
// each kernel file gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {

// Parameter block of the attention kernels (one launch).
struct KParams {
    const uint16_t *q;
    const uint8_t *cache;
    const int32_t *bt;
    const int32_t *req_id;
    const int32_t *topk;
    uint16_t *out;
    float *lse;
    int32_t *phys_out;
    float *part_o;        // [T][S][H][512] fp32 partial output (O / l) of each split
    float *part_lse;      // [T][S][H] natural-log lse of each split
    // non-null (attn_pc_kernel inside a split call): each split's O / l goes out
    // as bf16 rows in the first half of its fp32 slot ((t, s) holds [2][H][512]
    // bf16), and a split with at most kExactPRows valid rows also writes the
    // bf16 residual rows (O / l - hi) into the second half and sets its flag
    int32_t *part_exact;  // [T][S]
    float log2e_scale;    // sm_scale * log2(e): logits are kept in log2 units
    int T, H, K, R, MB;
    int64_t NB;
    int S, split_len, HB;
    int partials;         // write fp32 partials (O / l) and lse instead of the bf16 output
    int slot_in;          // topk holds cache slots: no request id, no block-table lookup
};

// bf16-cache attention with all 128 heads of a token in one workgroup
// (smla_attn128.hip).
hipError_t launch_attn128(const KParams &p, hipStream_t stream);

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef int i32x2 __attribute__((__vector_size__(8)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef float f32x2 __attribute__((__vector_size__(8)));
typedef int i32x8 __attribute__((__vector_size__(32)));
typedef short s16x2 __attribute__((__vector_size__(4)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int kTile = 32;             // cache rows per tile
constexpr int kRB = kTile / 16;       // 16-row MFMA blocks per tile
// Each kernel compacts a list into LDS in rounds of kChunk positions (its
// configuration's constant). Smaller rounds measured faster on most batch
// shapes (2048 -> 1024: the 16-head decode at top-k 512 and 1024 by 5 %, the
// headline decode, 128-head prefill and mixed batches by 1-3 %): each thread
// handles fewer positions, and a long list's extra rounds cost less than that
// saves, except where a round boundary drains a shallow ring.
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
template <> struct RowFmt<kCacheNvfp4> {
    static constexpr int kBytes = kNvfp4RowBytes; // 256 B E2M1 latent | 32 x E4M3 scale | 64 x E4M3 RoPE
    static constexpr int kScales = 256;
    static constexpr int kRope = 288;
};

// Byte offset of tile row r in a ring buffer.
template <class C>
__device__ __forceinline__ int lds_row(int r)
{
    return (r >> 4) * C::kRowBlockBytes + (r & 15) * C::kRowStride;
}



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

// convert_slot in two steps and without branches: lookup_block always issues
// the block-table load (entry 0 stands in for an invalid position; it exists
// since num_reqs and max_blocks_per_req are >= 1), so the compiler can count
// the loads in flight and wait for earlier ones while these are outstanding;
// finish_slot turns the entry into the slot. Same results as convert_slot.
__device__ __forceinline__ bool slot_position_ok(int req, int idx, int num_reqs, int max_blocks)
{
    return (unsigned)req < (unsigned)num_reqs && idx >= 0 && (idx >> 6) < max_blocks;
}

__device__ __forceinline__ int lookup_block(int req, int idx, const int32_t *__restrict__ bt,
                                            int num_reqs, int max_blocks)
{
    return bt[slot_position_ok(req, idx, num_reqs, max_blocks) ? (size_t)req * max_blocks + (idx >> 6) : 0];
}

__device__ __forceinline__ int finish_slot(int base, int req, int idx, int num_reqs, int max_blocks,
                                           int64_t num_blocks)
{
    return slot_position_ok(req, idx, num_reqs, max_blocks) && base >= 0 && (int64_t)base < num_blocks
               ? base * kBlock + (idx & (kBlock - 1))
               : -1;
}

// A position that already holds a cache slot: valid when inside the cache.
__device__ __forceinline__ int given_slot(int idx, int64_t num_blocks)
{
    return idx >= 0 && (int64_t)idx < num_blocks * kBlock ? idx : -1;
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
// 16x16x32 MFMA.
__device__ __forceinline__ bf16x8 pack_p(const f32x4 &p0, const f32x4 &p1)
{
    return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(p0[0], p0[1]), pack_bf16(p0[2], p0[3]),
                                                 pack_bf16(p1[0], p1[1]), pack_bf16(p1[2], p1[3])));
}

// bf16 rounding of what p0 | p1 lose in their rounding `hi`.
__device__ __forceinline__ bf16x8 pack_p_residual(const f32x4 &p0, const f32x4 &p1, const bf16x8 &hi)
{
    const uint4 w = __builtin_bit_cast(uint4, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(p0[0] - bf16_lo(w.x), p0[1] - bf16_hi(w.x)),
                                                 pack_bf16(p0[2] - bf16_lo(w.y), p0[3] - bf16_hi(w.y)),
                                                 pack_bf16(p1[0] - bf16_lo(w.z), p1[1] - bf16_hi(w.z)),
                                                 pack_bf16(p1[2] - bf16_lo(w.w), p1[3] - bf16_hi(w.w))));
}

// The compaction of a round of the top-k list (valid slots into LDS in list
// order): position tid + kThreads j of the round is thread tid's j-th, so the
// list order is (j, wave, lane). Each wave has counted its valid positions of
// part j, and count j * kWaves + w sits in lane j * kWaves + w of my_count.
// Gives in base[j] the list index of this wave's first valid position of part
// j and returns the round's total: scalar reads of the counts and selects on
// a uniform wave index, no branch per count.
template <int kPer, int kWaves>
__device__ __forceinline__ int compaction_bases(int my_count, int wave, int (&base)[kPer])
{
    static_assert(kPer * kWaves <= 32, "the counts fit lanes 0..31");
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int run = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        base[j] = 0;
#pragma unroll
    for (int k = 0; k < kPer * kWaves; ++k) {
        if (k % kWaves == wv)
            base[k / kWaves] = run;
        run += __builtin_amdgcn_readlane(my_count, k);
    }
    return run;
}

// Lanes below this one whose bit is set in mask.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wait until at most n of this wave's vector-memory instructions are pending
// (n is wave-uniform; values above 63, the counter's range, wait for all).
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
        SMLA_VMCNT_CASE(32) SMLA_VMCNT_CASE(33) SMLA_VMCNT_CASE(34) SMLA_VMCNT_CASE(35)
        SMLA_VMCNT_CASE(36) SMLA_VMCNT_CASE(37) SMLA_VMCNT_CASE(38) SMLA_VMCNT_CASE(39)
        SMLA_VMCNT_CASE(40) SMLA_VMCNT_CASE(41) SMLA_VMCNT_CASE(42) SMLA_VMCNT_CASE(43)
        SMLA_VMCNT_CASE(44) SMLA_VMCNT_CASE(45) SMLA_VMCNT_CASE(46) SMLA_VMCNT_CASE(47)
        SMLA_VMCNT_CASE(48) SMLA_VMCNT_CASE(49) SMLA_VMCNT_CASE(50) SMLA_VMCNT_CASE(51)
        SMLA_VMCNT_CASE(52) SMLA_VMCNT_CASE(53) SMLA_VMCNT_CASE(54) SMLA_VMCNT_CASE(55)
        SMLA_VMCNT_CASE(56) SMLA_VMCNT_CASE(57) SMLA_VMCNT_CASE(58) SMLA_VMCNT_CASE(59)
        SMLA_VMCNT_CASE(60) SMLA_VMCNT_CASE(61) SMLA_VMCNT_CASE(62) SMLA_VMCNT_CASE(63)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef SMLA_VMCNT_CASE
}

// The value of v, opaque to the optimiser from here on: addresses derived from
// it are computed where they are used instead of being hoisted to the kernel's
// start and kept (or spilled) across the tile loop.
__device__ __forceinline__ int late(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// global_load_lds_dwordx4: 16 bytes per active lane from `src` into LDS at
// lds_base + 16 * lane. Written as inline assembly on purpose: the compiler
// cannot see that the LDS reads which follow touch a different ring buffer,
// and for the builtin it waits for the whole copy before the next LDS read,
// which would serialise every gather with the compute on the previous tile.
// Completion is ordered by the explicit vmcnt waits and barriers around the
// ring instead.
__device__ __forceinline__ void dma16(const uint8_t *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// dma16 for the lanes set in `lanes` only, without a branch: the mask goes into
// EXEC for the one copy and the wave's mask is restored after it, so the copy
// can sit in a straight run of MFMAs (a divergent branch there splits the
// accumulators' live ranges and makes the compiler spill them).
__device__ __forceinline__ void dma16_lanes(const uint8_t *src, uint32_t lds_base, uint64_t lanes)
{
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %3\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(lds_base), "s"(lanes)
                 : "memory", "m0");
}

// Cross-lane max and sum with the lane l xor 16 (same 32-lane half) or l xor 32,
// through v_permlane16_swap / v_permlane32_swap instead of an LDS round trip
// (ds_bpermute). Each swap with itself returns, for every lane, its own value
// in one result and its partner's in the other, so a symmetric op of the two
// results is the op with the partner.
__device__ __forceinline__ float xor16_max(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// global_load_lds_dword: 4 bytes per active lane from `src` into LDS at
// lds_base + 4 * lane (inline assembly for the same reason as dma16).
__device__ __forceinline__ void dma4(const void *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// Copy the rows of one tile, as stored, into an LDS ring buffer in the layout
// lds_row() describes. Wave w copies rows w * kRowsPerWave ...: one lane reads
// the slots of those rows from the compacted list, each row's slot is then a
// scalar, and each copy instruction needs a single per-lane address add (lane
// c moves bytes 16c .. 16c + 15 of the row). Rows past the tile's valid count
// repeat the tile's first row (finite data whose weights are masked to zero).
// Every instruction has at least one active lane, so a wave always issues
// kDmaPerWave of them per tile.
template <class C>
__device__ __forceinline__ void issue_tile(const uint8_t *__restrict__ cache, const int32_t *slots,
                                           int n_tile, uint8_t *buf, int wave, int lane)
{
    // recomputed per tile: kept across the tile loop they would be spilled, and a
    // reload from scratch waits for every copy in flight
    lane = late(lane);
    const int r0 = wave * C::kRowsPerWave;
    const int ri = r0 + lane % C::kRowsPerWave;
    const int my_slot = slots[ri < n_tile ? ri : 0];
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)LDS_PTR(uint8_t, buf) +
                                                         (uint32_t)lds_row<C>(r0));
    if constexpr (C::kInstrPerRow == 1) {
        // one instruction per row (fp8): the rows' addresses first, then all the
        // copies under one lane mask
        const uint8_t *rowp[C::kRowsPerWave];
        uint32_t ldsp[C::kRowsPerWave];
#pragma unroll
        for (int i = 0; i < C::kRowsPerWave; ++i) {
            const int slot = __builtin_amdgcn_readlane(my_slot, i);
            rowp[i] = cache + (size_t)(uint32_t)slot * C::kRowBytes + 16 * lane;
            ldsp[i] = __builtin_amdgcn_readfirstlane(base + (uint32_t)(lds_row<C>(r0 + i) - lds_row<C>(r0)));
        }
        if (lane < C::kChunksPerRow) {
#pragma unroll
            for (int i = 0; i < C::kRowsPerWave; ++i)
                dma16(rowp[i], ldsp[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::kRowsPerWave; ++i) {
            const int r = r0 + i;
            const int slot = __builtin_amdgcn_readlane(my_slot, i);
            const uint8_t *row = cache + (size_t)(uint32_t)slot * C::kRowBytes;
            // lds_row(r) - lds_row(r0): r0 is a multiple of kRowsPerWave, so whether
            // row r crosses into the next 16-row block is known from i alone when
            // kRowsPerWave divides 16; otherwise it is computed
            const uint32_t lds = base + (uint32_t)(lds_row<C>(r) - lds_row<C>(r0));
#pragma unroll
            for (int k = 0; k < C::kInstrPerRow; ++k) {
                const int chunk = 64 * k + lane;
                if (chunk < C::kChunksPerRow)
                    dma16(row + 16 * chunk, __builtin_amdgcn_readfirstlane(lds + 1024u * k));
            }
        }
    }
}

}  // namespace
}  // namespace smla
