/*
 * smla_oracle.c -- plain CPU oracle for sparse MLA forward over top-k indices.
 *
 * TEST INFRASTRUCTURE. This file exists to check the GPU library, not to be
 * part of it. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it. The GPU path shares no code, header, table or helper
 * with it, and it includes nothing from the GPU path.
 *
 * It is deliberately slow and literal: every step is the plain definition,
 * computed in double precision, one query token per OpenMP iteration, no
 * tiling, no fusion, no online softmax.
 *
 * Sources (the pages this build follows). Every citation below names the
 * "flashmla_sparse.py page": the package-diff page of the vllm-cpu-avx512bf16
 * 0.14.0 wheel that shows vllm/v1/attention/backends/mla/flashmla_sparse.py,
 * the vLLM FLASHMLA_SPARSE backend source. From it:
 *          - the module note on the fp8_ds_mla cache format (656-byte rows:
 *            512 float8_e4m3, 4 float32 scales per 128 values, 64 bfloat16
 *            RoPE values);
 *          - triton_convert_req_index_to_global_index and its docstring
 *            (logical top-k index -> physical cache slot through the block
 *            table, -1 kept as -1, out-of-table blocks mapped to -1);
 *          - FlashMLASparseImpl.forward (its note that both sparse kernels
 *            run multi-query attention with 576-wide keys and 512-wide
 *            values: every head of a token attends to the same rows, and the
 *            value is the first 512 columns), _fp8_flash_mla_kernel (head_dim_v=512),
 *            and the softmax_scale the backend passes to the kernels.
 *   The OCP 8-bit floating point specification (the E4M3FN encoding) for the
 *   value of an e4m3 byte, and its round-to-nearest-even encoding.
 *   flashmla_sparse.py page, FlashMLASparseImpl.forward: the concat_and_cache_mla call that writes
 *   a token's latent (k_c_normed) and RoPE (k_pe) into the cache slot given by
 *   slot_mapping, in the cache's dtype ("auto" = bf16 or "fp8_ds_mla").
 *   vLLM pull-request page "Support nvfp4_ds_mla on FLASHINFER_MLA_SPARSE, with
 *   native NVFP4 decode" (its description and design notes): an nvfp4_ds_mla
 *   row takes 352 bytes per token against 576 for the fp8 cache, and native
 *   decode attends over the exact dequantised values of the rows as stored
 *   (no staging copy, no re-rounding to e4m3). The OCP Microscaling (MX)
 *   specification for the value of an FP4 E2M1 code, and the NVFP4 block
 *   form: E2M1 values with one E4M3 scale per 16 values.
 *   flashmla_sparse.py page, the separate-prefill mode of an fp8 cache:
 *   _convert_req_index_to_global_index_kernel with HAS_PREFILL
 *   (a prefill token's index maps to its request's workspace start plus the
 *   index), _build_fp8_separate_prefill_decode (workspace starts are the
 *   running sum of the prefill sequence lengths, cut into chunks that fit the
 *   workspace, each chunk's starts made chunk-local; the worked example there:
 *   lengths [10, 15, 20, 5] in chunks [0, 2) and [2, 4) give starts
 *   [0, 10, 0, 20]), get_prefill_workspace_size (5 x max_model_len rows), and
 *   _forward_fp8_kv_separate_prefill_decode (each chunk's context rows are
 *   gathered from the fp8 cache and upconverted into a bf16 workspace, then
 *   the bf16 kernel runs over the workspace).
 *
 * Readings where the pages are silent:
 *   - the second kernel return value is the natural-log log-sum-exp of the
 *     scaled logits;
 *   - a token with no valid slot gets o = 0 and lse = -inf;
 *   - a duplicated index counts once per occurrence (plain sum over the list);
 *   - a request id outside [0, num_reqs) or a block-table entry outside
 *     [0, num_blocks) yields slot -1 (the page's kernel would read out of
 *     bounds there);
 *   - the per-128 scales multiply the decoded e4m3 values;
 *   - cache writer (the pages give the row layout, not the quantisation): each
 *     128-value group's scale is amax / 448 in float32 (1.0 for an all-zero
 *     group), and each byte is the e4m3 value nearest to x / scale (float32
 *     division), ties to the even code, saturating at +-448; a negative slot,
 *     or one past the cache, writes nothing.
 *   - nvfp4_ds_mla row (the page gives its size only): 352 = 256 + 32 + 64
 *     bytes, the one split of that size into standard NVFP4 pieces: bytes
 *     0..255 hold the 512 latent values as E2M1 codes, two per byte, value 2i
 *     in the low nibble of byte i and 2i + 1 in the high nibble; bytes
 *     256..287 hold 32 E4M3FN scales, scale b multiplying latent values
 *     16b .. 16b + 15; bytes 288..351 hold the 64 RoPE values as E4M3FN bytes.
 *     A latent value is its E2M1 value times its block's scale; there is no
 *     per-tensor factor (the page's k_scale belongs to its fp8 staging copy,
 *     which native decode does not make).
 *   - nvfp4_ds_mla writer: a block's scale is the E4M3 value nearest to
 *     amax / 6 (float32 division), ties to even, saturating at 448; each latent
 *     value becomes the E2M1 code nearest to x / scale (float32 division), ties
 *     to the even code, saturating at +-6; a block whose scale is zero stores
 *     zero codes; RoPE values become the nearest E4M3 bytes, saturating.
 *   - separate-prefill mode: the upconverted value of a latent element is the
 *     exact product e4m3 x scale rounded once to the nearest bfloat16, ties to
 *     even (the RoPE part is copied); chunks are formed greedily in request
 *     order, a new chunk starting when the next request would overflow the
 *     workspace; a context position whose block lies outside the table (or
 *     whose table entry lies outside the cache) upconverts to a row of zeros;
 *     a prefill request id past the prefill count converts to -1.
 *
 * Parity pins for every function here live in the CPU test suite
 * (tests/test_oracle_pins.py); none of them re-types these formulas.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 64   /* paged-cache block size (kernel supports 64 only) */
#define ORACLE_DQK 576    /* 512 latent (NoPE) + 64 RoPE                     */
#define ORACLE_DV 512     /* value width = latent part                       */
#define ORACLE_FP8_ROW 656
#define ORACLE_NVFP4_ROW 352

/* Threads an OpenMP parallel region of this library will use. */
int smla_oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* ---------------------------------------------------------------- values */

/* OCP E4M3FN byte -> value. Sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is
 * no infinity. */
double smla_oracle_e4m3fn(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> value (the upper half of a float32). */
double smla_oracle_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One 656-byte fp8_ds_mla row -> 576 values [flashmla_sparse.py page, cache format note]:
 * bytes 0..511 are e4m3 latent values, bytes 512..527 four little-endian
 * float32 scales (scale i covers latent values 128*i .. 128*i+127), bytes
 * 528..655 sixty-four bfloat16 RoPE values, not quantized. */
void smla_oracle_decode_fp8_row(const uint8_t *row, double *out)
{
    float scale[4];
    memcpy(scale, row + 512, sizeof scale);
    for (int i = 0; i < 512; ++i)
        out[i] = smla_oracle_e4m3fn(row[i]) * (double)scale[i / 128];
    for (int r = 0; r < 64; ++r) {
        uint16_t b;
        memcpy(&b, row + 528 + 2 * r, sizeof b);
        out[512 + r] = smla_oracle_bf16(b);
    }
}

/* One bf16 cache row (576 values) -> values. */
void smla_oracle_decode_bf16_row(const uint16_t *row, double *out)
{
    for (int i = 0; i < ORACLE_DQK; ++i)
        out[i] = smla_oracle_bf16(row[i]);
}

/* OCP FP4 E2M1 code (low 4 bits) -> value. Sign bit 3, 2 exponent bits (bias
 * 1), 1 mantissa bit; exponent field 0 is subnormal (m * 2^-1); there is no
 * infinity and no NaN. */
double smla_oracle_e2m1(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 0x3;
    int m = code & 0x1;
    double v;
    if (e == 0)
        v = ldexp((double)m, -1);
    else
        v = ldexp(1.0 + (double)m / 2.0, e - 1);
    return sign ? -v : v;
}

/* One 352-byte nvfp4_ds_mla row -> 576 values (layout in the readings above):
 * latent value i is E2M1 code i (low nibble of byte i / 2 for even i, high
 * nibble for odd i) times the E4M3 scale in byte 256 + i / 16; RoPE value r is
 * the E4M3 byte 288 + r. */
void smla_oracle_decode_nvfp4_row(const uint8_t *row, double *out)
{
    for (int i = 0; i < ORACLE_DV; ++i) {
        const uint8_t byte = row[i / 2];
        const uint8_t code = (i % 2 == 0) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4);
        out[i] = smla_oracle_e2m1(code) * smla_oracle_e4m3fn(row[256 + i / 16]);
    }
    for (int r = 0; r < 64; ++r)
        out[ORACLE_DV + r] = smla_oracle_e4m3fn(row[288 + r]);
}

/* ------------------------------------------------------------ cache write */

/* float -> OCP E4M3FN byte: the finite code whose value is nearest to x, ties
 * to the code with an even mantissa (RNE); magnitudes beyond the largest finite
 * value (448) take 448; NaN gives 0x7F. Found by scanning the 127 non-negative
 * finite codes with the decoder above: slow on purpose, no bit manipulation. */
uint8_t smla_oracle_e4m3fn_encode(float x)
{
    if (isnan(x))
        return 0x7F;
    const double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(smla_oracle_e4m3fn((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(signbit(x) ? (0x80 | best) : best);
}

/* float -> FP4 E2M1 code: the code whose value is nearest to x, ties to the
 * code with an even mantissa bit (RNE); magnitudes beyond 6 take 6; NaN gives
 * 0. Found by scanning the 8 non-negative codes with the decoder above. */
uint8_t smla_oracle_e2m1_encode(float x)
{
    if (isnan(x))
        return 0;
    const double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 7; ++c) {
        const double d = fabs(smla_oracle_e2m1((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(signbit(x) ? (0x8 | best) : best);
}

/* Write num_tokens token rows into a paged cache [flashmla_sparse.py page, FlashMLASparseImpl.forward:
 * concat_and_cache_mla; cache format note]. k_c: bfloat16 [T][512] latent,
 * k_pe: bfloat16 [T][64] RoPE, slot_mapping: int64 [T] (flat slot = block * 64
 * + offset). cache_format 0: bf16 rows [slots][576] (latent then RoPE, copied);
 * 1: fp8_ds_mla rows [slots][656]; 2: nvfp4_ds_mla rows [slots][352] (both as
 * the readings above state). num_slots bounds the
 * cache; slots outside [0, num_slots) are skipped. */
void smla_oracle_cache_write(int cache_format, const uint16_t *k_c, const uint16_t *k_pe,
                             const int64_t *slot_mapping, int64_t num_tokens, void *cache,
                             int64_t num_slots)
{
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        const uint16_t *lat = k_c + t * ORACLE_DV;
        const uint16_t *rope = k_pe + t * (ORACLE_DQK - ORACLE_DV);
        if (cache_format == 0) {
            uint16_t *row = (uint16_t *)cache + slot * ORACLE_DQK;
            memcpy(row, lat, ORACLE_DV * sizeof(uint16_t));
            memcpy(row + ORACLE_DV, rope, (ORACLE_DQK - ORACLE_DV) * sizeof(uint16_t));
            continue;
        }
        if (cache_format == 2) {
            uint8_t *row = (uint8_t *)cache + slot * ORACLE_NVFP4_ROW;
            for (int b = 0; b < 32; ++b) {
                float amax = 0.0f;
                for (int i = 16 * b; i < 16 * b + 16; ++i) {
                    const float v = fabsf((float)smla_oracle_bf16(lat[i]));
                    if (v > amax)
                        amax = v;
                }
                const uint8_t sc = smla_oracle_e4m3fn_encode(amax / 6.0f);
                const float scale = (float)smla_oracle_e4m3fn(sc);
                row[256 + b] = sc;
                for (int i = 16 * b; i < 16 * b + 16; ++i) {
                    const uint8_t code =
                        scale > 0.0f ? smla_oracle_e2m1_encode((float)smla_oracle_bf16(lat[i]) / scale) : 0;
                    if (i % 2 == 0)
                        row[i / 2] = code;
                    else
                        row[i / 2] = (uint8_t)(row[i / 2] | (code << 4));
                }
            }
            for (int r = 0; r < 64; ++r)
                row[288 + r] = smla_oracle_e4m3fn_encode((float)smla_oracle_bf16(rope[r]));
            continue;
        }
        uint8_t *row = (uint8_t *)cache + slot * ORACLE_FP8_ROW;
        for (int g = 0; g < 4; ++g) {
            float amax = 0.0f;
            for (int i = 128 * g; i < 128 * g + 128; ++i) {
                const float v = fabsf((float)smla_oracle_bf16(lat[i]));
                if (v > amax)
                    amax = v;
            }
            const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            for (int i = 128 * g; i < 128 * g + 128; ++i)
                row[i] = smla_oracle_e4m3fn_encode((float)smla_oracle_bf16(lat[i]) / scale);
            memcpy(row + 512 + 4 * g, &scale, sizeof scale);
        }
        memcpy(row + 528, rope, 64 * sizeof(uint16_t));
    }
}

/* --------------------------------------------------------- index convert */

/* Logical per-request top-k index -> physical cache slot [flashmla_sparse.py page,
 * triton_convert_req_index_to_global_index docstring and kernel]:
 *   slot = block_table[req, idx / 64] * 64 + idx % 64,
 * with -1 for a negative index and for a block position outside the table
 * width. Safety readings: bad request id or bad table entry -> -1. */
int32_t smla_oracle_convert_one(int32_t req, int32_t idx, const int32_t *block_table,
                                int64_t num_reqs, int64_t max_blocks_per_req,
                                int64_t num_blocks)
{
    if (req < 0 || req >= num_reqs)
        return -1;
    if (idx < 0)
        return -1;
    int64_t blk = idx / ORACLE_BLOCK;
    int64_t off = idx % ORACLE_BLOCK;
    if (blk >= max_blocks_per_req)
        return -1;
    int64_t base = block_table[(int64_t)req * max_blocks_per_req + blk];
    if (base < 0 || base >= num_blocks)
        return -1;
    return (int32_t)(base * ORACLE_BLOCK + off);
}

void smla_oracle_convert_indices(const int32_t *req_id_per_token, const int32_t *block_table,
                                 const int32_t *topk_indices, int32_t *out, int64_t num_tokens,
                                 int64_t topk, int64_t num_reqs, int64_t max_blocks_per_req,
                                 int64_t num_blocks)
{
    for (int64_t t = 0; t < num_tokens; ++t)
        for (int64_t j = 0; j < topk; ++j)
            out[t * topk + j] = smla_oracle_convert_one(
                req_id_per_token[t], topk_indices[t * topk + j], block_table, num_reqs,
                max_blocks_per_req, num_blocks);
}

/* ------------------------------------------------ separate-prefill mode */

/* Index conversion with a prefill workspace [flashmla_sparse.py page,
 * _convert_req_index_to_global_index_kernel with HAS_PREFILL]: a token whose
 * prefill request id r is >= 0 maps a valid index to workspace_starts[r] + idx;
 * other tokens convert as smla_oracle_convert_one. Invalid either way: a
 * negative index and a block position outside the table width. */
int32_t smla_oracle_convert_one_ws(int32_t req, int32_t idx, const int32_t *block_table,
                                   int64_t num_reqs, int64_t max_blocks_per_req, int64_t num_blocks,
                                   int32_t prefill_req, const int32_t *workspace_starts,
                                   int64_t num_prefills)
{
    if (prefill_req < 0)
        return smla_oracle_convert_one(req, idx, block_table, num_reqs, max_blocks_per_req,
                                       num_blocks);
    if (prefill_req >= num_prefills || idx < 0 || idx / ORACLE_BLOCK >= max_blocks_per_req)
        return -1;
    return workspace_starts[prefill_req] + idx;
}

void smla_oracle_convert_indices_ws(const int32_t *req_id_per_token, const int32_t *block_table,
                                    const int32_t *topk_indices, const int32_t *prefill_request_id,
                                    const int32_t *workspace_starts, int32_t *out, int64_t num_tokens,
                                    int64_t topk, int64_t num_reqs, int64_t max_blocks_per_req,
                                    int64_t num_blocks, int64_t num_prefills)
{
    for (int64_t t = 0; t < num_tokens; ++t)
        for (int64_t j = 0; j < topk; ++j)
            out[t * topk + j] = smla_oracle_convert_one_ws(
                req_id_per_token[t], topk_indices[t * topk + j], block_table, num_reqs,
                max_blocks_per_req, num_blocks, prefill_request_id[t], workspace_starts,
                num_prefills);
}

/* A finite value with at most 53 significant bits -> the bfloat16 bit pattern
 * of the nearest bfloat16 value, ties to even (8 significant bits for normal
 * values, a fixed quantum of 2^-133 below 2^-126), infinity past the largest
 * finite bfloat16. */
uint16_t smla_oracle_bf16_rne(double x)
{
    if (x == 0.0)
        return signbit(x) ? 0x8000u : 0u;
    int e;
    frexp(x, &e);                        /* |x| in [2^(e-1), 2^e) */
    int q = e - 8;                       /* quantum exponent: 8 significant bits */
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(x, -q)), q);     /* nearbyint: ties to even */
    float f = (float)r;                                /* exact: <= 8 significant bits */
    if (fabs(r) >= 0x1.0p128)
        f = r > 0 ? INFINITY : -INFINITY;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Gather and upconvert the context rows of a batch of prefill requests into a
 * bf16 workspace: for request b and position p < seq_lens[b], workspace row
 * workspace_starts[b] + p (when inside [0, workspace_rows)) receives the row at
 * slot block_table[b, p / 64] * 64 + p % 64 of the cache; a position whose
 * block lies outside the table, or whose table entry lies outside the cache,
 * gets a row of zeros.
 * - fp8_ds_mla (cache_format 1) [flashmla_sparse.py page,
 *   _forward_fp8_kv_separate_prefill_decode: the cp_gather_and_upconvert_fp8_kv_cache
 *   call]: each latent value e4m3 x scale rounded to bfloat16, the RoPE values copied.
 * - nvfp4_ds_mla (cache_format 2) [pull-request page "Support nvfp4_ds_mla on
 *   FLASHINFER_MLA_SPARSE, with native NVFP4 decode": prefill is staged through a
 *   context gather per request and chunk]: every value is its exact decoded
 *   value, which bfloat16 holds exactly (E2M1 x E4M3 has at most 6 significant
 *   bits; E4M3 RoPE values 4). */
static void gather_upconvert(int cache_format, const uint8_t *cache, int64_t num_blocks,
                             const int32_t *block_table, int64_t max_blocks_per_req, const int32_t *seq_lens,
                             const int32_t *workspace_starts, int64_t batch, uint16_t *workspace,
                             int64_t workspace_rows)
{
    const int64_t row_bytes = cache_format == 1 ? ORACLE_FP8_ROW : ORACLE_NVFP4_ROW;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t pos = 0; pos < seq_lens[b]; ++pos) {
            int64_t w = (int64_t)workspace_starts[b] + pos;
            if (w < 0 || w >= workspace_rows)
                continue;
            uint16_t *dst = workspace + w * ORACLE_DQK;
            int64_t blk = pos / ORACLE_BLOCK;
            int64_t base = blk < max_blocks_per_req ? block_table[b * max_blocks_per_req + blk] : -1;
            if (base < 0 || base >= num_blocks) {
                memset(dst, 0, ORACLE_DQK * sizeof(uint16_t));
                continue;
            }
            const uint8_t *row = cache + (base * ORACLE_BLOCK + pos % ORACLE_BLOCK) * row_bytes;
            double v[ORACLE_DQK];
            if (cache_format == 1) {
                smla_oracle_decode_fp8_row(row, v);
                for (int i = 0; i < ORACLE_DV; ++i)
                    dst[i] = smla_oracle_bf16_rne(v[i]);
                memcpy(dst + ORACLE_DV, row + 528, 64 * sizeof(uint16_t));
            } else {
                smla_oracle_decode_nvfp4_row(row, v);
                for (int i = 0; i < ORACLE_DQK; ++i)
                    dst[i] = smla_oracle_bf16_rne(v[i]);
            }
        }
    }
}

void smla_oracle_gather_upconvert(const uint8_t *cache, int64_t num_blocks, const int32_t *block_table,
                                  int64_t max_blocks_per_req, const int32_t *seq_lens,
                                  const int32_t *workspace_starts, int64_t batch, uint16_t *workspace,
                                  int64_t workspace_rows)
{
    gather_upconvert(1, cache, num_blocks, block_table, max_blocks_per_req, seq_lens, workspace_starts, batch,
                     workspace, workspace_rows);
}

void smla_oracle_gather_upconvert_nvfp4(const uint8_t *cache, int64_t num_blocks, const int32_t *block_table,
                                        int64_t max_blocks_per_req, const int32_t *seq_lens,
                                        const int32_t *workspace_starts, int64_t batch, uint16_t *workspace,
                                        int64_t workspace_rows)
{
    gather_upconvert(2, cache, num_blocks, block_table, max_blocks_per_req, seq_lens, workspace_starts, batch,
                     workspace, workspace_rows);
}

/* Cut consecutive prefill requests into chunks whose total sequence length fits
 * max_rows workspace rows [flashmla_sparse.py page, _build_fp8_separate_prefill_decode]: greedy in
 * request order. Writes chunk_ends[c] (one past the chunk's last request) and,
 * for every request, its chunk-local workspace start. Returns the chunk count,
 * or -1 if a single request is longer than max_rows or a length is negative. */
int64_t smla_oracle_plan_prefill_chunks(const int32_t *seq_lens, int64_t num_prefills, int64_t max_rows,
                                        int32_t *chunk_ends, int32_t *workspace_starts)
{
    int64_t n = 0, used = 0;
    for (int64_t r = 0; r < num_prefills; ++r) {
        if (seq_lens[r] < 0 || seq_lens[r] > max_rows)
            return -1;
        if (r > 0 && used + seq_lens[r] > max_rows) {
            chunk_ends[n++] = (int32_t)r;
            used = 0;
        }
        workspace_starts[r] = (int32_t)used;
        used += seq_lens[r];
    }
    if (num_prefills > 0)
        chunk_ends[n++] = (int32_t)num_prefills;
    return n;
}

/* -------------------------------------------------------------- attention */

/* Sparse MQA-576/512 attention for the listed query tokens [flashmla_sparse.py page,
 * FlashMLASparseImpl.forward and the two kernel wrappers]:
 *   for token t, head h and valid slots j of t's list,
 *     s_j      = sm_scale * <q[t,h,0:576], K_j>
 *     lse[t,h] = ln sum_j exp(s_j)
 *     p_j      = exp(s_j - lse[t,h])
 *     o[t,h,:] = sum_j p_j * K_j[0:512]
 *
 * cache_format: 0 = bf16 rows [num_blocks, 64, 576] (uint16 bit patterns),
 *               1 = 656-byte fp8_ds_mla rows [num_blocks, 64, 656],
 *               2 = 352-byte nvfp4_ds_mla rows [num_blocks, 64, 352].
 * q: bf16 bit patterns [num_tokens, h_q, 576].
 * tokens: which query tokens to compute (NULL = all, in order); output row i
 *         belongs to token tokens[i].
 * out: [n, h_q, 512]; lse: [n, h_q]; weights (nullable): [n, h_q, topk], the
 *      softmax weight of every list position (0 for invalid positions).
 * Returns 0, or -1 on a bad argument or allocation failure. */
int smla_oracle_attention(int cache_format, const uint16_t *q, const void *cache,
                          const int32_t *block_table, const int32_t *req_id_per_token,
                          const int32_t *topk_indices, double sm_scale, int64_t num_tokens,
                          int64_t h_q, int64_t topk, int64_t num_reqs,
                          int64_t max_blocks_per_req, int64_t num_blocks,
                          const int64_t *tokens, int64_t n, double *out, double *lse,
                          double *weights)
{
    if (cache_format != 0 && cache_format != 1 && cache_format != 2)
        return -1;
    if (tokens == NULL)
        n = num_tokens;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        double *rows = malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1) * ORACLE_DQK);
        int32_t *slot = malloc(sizeof(int32_t) * (size_t)(topk > 0 ? topk : 1));
        double *s = malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
        double *qh = malloc(sizeof(double) * ORACLE_DQK);
        if (!rows || !slot || !s || !qh || t < 0 || t >= num_tokens) {
#pragma omp atomic write
            failed = 1;
            free(rows); free(slot); free(s); free(qh);
            continue;
        }

        /* 1. every list position -> physical slot; decode the valid rows. */
        for (int64_t j = 0; j < topk; ++j) {
            slot[j] = smla_oracle_convert_one(req_id_per_token[t], topk_indices[t * topk + j],
                                              block_table, num_reqs, max_blocks_per_req,
                                              num_blocks);
            if (slot[j] < 0)
                continue;
            if (cache_format == 1)
                smla_oracle_decode_fp8_row((const uint8_t *)cache + (int64_t)slot[j] * ORACLE_FP8_ROW,
                                           rows + j * ORACLE_DQK);
            else if (cache_format == 2)
                smla_oracle_decode_nvfp4_row((const uint8_t *)cache + (int64_t)slot[j] * ORACLE_NVFP4_ROW,
                                             rows + j * ORACLE_DQK);
            else
                smla_oracle_decode_bf16_row((const uint16_t *)cache + (int64_t)slot[j] * ORACLE_DQK,
                                            rows + j * ORACLE_DQK);
        }

        for (int64_t h = 0; h < h_q; ++h) {
            const uint16_t *qrow = q + (t * h_q + h) * ORACLE_DQK;
            double *o = out + (i * h_q + h) * ORACLE_DV;
            double *w = weights ? weights + (i * h_q + h) * topk : NULL;
            for (int d = 0; d < ORACLE_DQK; ++d)
                qh[d] = smla_oracle_bf16(qrow[d]);

            /* 2. logits of the valid positions, and their maximum. */
            double m = -INFINITY;
            int64_t nvalid = 0;
            for (int64_t j = 0; j < topk; ++j) {
                if (slot[j] < 0)
                    continue;
                double dot = 0.0;
                for (int d = 0; d < ORACLE_DQK; ++d)
                    dot += qh[d] * rows[j * ORACLE_DQK + d];
                s[j] = sm_scale * dot;
                if (s[j] > m)
                    m = s[j];
                ++nvalid;
            }

            for (int d = 0; d < ORACLE_DV; ++d)
                o[d] = 0.0;
            if (w)
                for (int64_t j = 0; j < topk; ++j)
                    w[j] = 0.0;
            if (nvalid == 0) {
                lse[i * h_q + h] = -INFINITY;
                continue;
            }

            /* 3. softmax normaliser and log-sum-exp. */
            double l = 0.0;
            for (int64_t j = 0; j < topk; ++j)
                if (slot[j] >= 0)
                    l += exp(s[j] - m);
            double lse_th = m + log(l);
            lse[i * h_q + h] = lse_th;

            /* 4. weighted sum of the latent (first 512) columns. */
            for (int64_t j = 0; j < topk; ++j) {
                if (slot[j] < 0)
                    continue;
                double p = exp(s[j] - lse_th);
                if (w)
                    w[j] = p;
                for (int d = 0; d < ORACLE_DV; ++d)
                    o[d] += p * rows[j * ORACLE_DQK + d];
            }
        }
        free(rows); free(slot); free(s); free(qh);
    }
    return failed ? -1 : 0;
}
