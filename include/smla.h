/*
 * smla.h -- C ABI of libsmla.so: sparse Multi-head Latent Attention (MLA)
 * forward over per-token top-k KV indices, for AMD Instinct MI355X (gfx950).
 *
 * What it computes. For query token t, head h (h_q heads share ONE latent KV
 * head), and every valid position j of t's top-k list:
 *
 *   slot_j   = block_table[req_id_per_token[t], idx[t,j] / 64] * 64 + idx[t,j] % 64
 *   K_j      = the 576-wide cache row at slot_j   (512 latent + 64 RoPE values)
 *   s_j      = sm_scale * <q[t,h,0:576], K_j>
 *   out[t,h] = sum_j softmax(s)_j * K_j[0:512]    (value = the latent part)
 *   lse[t,h] = ln sum_j exp(s_j)
 *
 * Sources: the vLLM page "vllm/v1/attention/backends/mla/flashmla_sparse.py"
 * (FLASHMLA_SPARSE backend): triton_convert_req_index_to_global_index and its
 * docstring (index conversion), the module note on the fp8_ds_mla format
 * (656-byte rows), FlashMLASparseImpl.forward (both sparse kernels run
 * multi-query attention with 576-wide keys and 512-wide values),
 * _fp8_flash_mla_kernel and _bf16_flash_mla_kernel (shapes, head_dim_v 512,
 * softmax_scale, the second returned value), FlashMLASparseBackend
 * (block size 64, head size 576, output buffer supplied by the caller).
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers to contiguous row-major memory
 *     owned by the caller. The library never allocates, frees, or keeps a
 *     pointer after the call returns. `options` and the output arguments of
 *     the query functions (smla_plan, smla_workspace_size) are HOST pointers.
 *   - Calls are asynchronous on `stream` (0 = the null stream). The library does
 *     not synchronize and never reads device memory from the host.
 *   - Every argument is validated before any HIP call; on an error nothing is
 *     launched and nothing is written.
 *   - A logical index < 0, a block position >= max_blocks_per_req, a request id
 *     outside [0, num_reqs) and a block-table entry outside [0, num_blocks) all
 *     mark the position invalid (slot -1); invalid positions contribute
 *     nothing. A token/head with no valid position gets out = 0, lse = -inf.
 *   - Duplicate positions in a list count once per occurrence.
 *   - Block size is fixed at 64 tokens, q/key width at 576, value width at 512.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 8
#define SMLA_BLOCK_SIZE 64
#define SMLA_HEAD_DIM_QK 576
#define SMLA_HEAD_DIM_V 512
#define SMLA_FP8_ROW_BYTES 656
#define SMLA_NVFP4_ROW_BYTES 352
#define SMLA_MAX_TOPK (1 << 20)

typedef enum smla_status {
    SMLA_OK = 0,
    SMLA_ERR_NULL = 1,      /* a required pointer is NULL                        */
    SMLA_ERR_SHAPE = 2,     /* unsupported size (h_q, topk, counts, pool size)   */
    SMLA_ERR_ALIGN = 3,     /* a pointer is not aligned as documented            */
    SMLA_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
    SMLA_ERR_HIP = 5,       /* a HIP runtime call or kernel launch failed        */
    SMLA_ERR_ARG = 6        /* invalid scalar argument or option                 */
} smla_status;

/* Bits of smla_options.flags. */
#define SMLA_FLAG_PARTIALS_ONLY 0x1u
    /* The call stops before the merge: it writes every top-k part's result into
       the workspace (layout at smla_merge_partials) and neither out nor lse.
       The workspace is required even when the list is not split (one part).
       smla_merge_partials then finishes the result; it also merges parts that
       were computed by separate calls, e.g. on different devices. */
#define SMLA_FLAG_SLOT_INDICES 0x2u
    /* topk_indices already hold cache slots (row numbers of kv_cache seen as
       [num_blocks * 64] rows; -1 or any value outside [0, num_blocks * 64) is an
       invalid position), e.g. the output of smla_convert_indices or the
       workspace rows of smla_convert_indices_workspace. block_table and
       req_id_per_token are not read and may be NULL; num_reqs and
       max_blocks_per_req are ignored. */
#define SMLA_FLAG_DEFER_MERGE 0x4u
    /* A call whose lists are split launches its attention kernel only and
       leaves the call's own per-part results in the workspace (their form may
       differ from what SMLA_FLAG_PARTIALS_ONLY writes). The same call repeated
       with SMLA_FLAG_MERGE_ONLY and the same workspace, out and lse finishes
       it: together the two write what one ordinary call writes, bit for bit.
       An unsplit call writes its result at once. */
#define SMLA_FLAG_MERGE_ONLY 0x8u
    /* Only the merge of a call made with SMLA_FLAG_DEFER_MERGE and the same
       arguments (a no-op when the call is not split); it reads the workspace,
       not the inputs. DEFER_MERGE and MERGE_ONLY together, or either with
       PARTIALS_ONLY, is SMLA_ERR_ARG. */
#define SMLA_FLAG_ALL (SMLA_FLAG_PARTIALS_ONLY | SMLA_FLAG_SLOT_INDICES | SMLA_FLAG_DEFER_MERGE | \
                       SMLA_FLAG_MERGE_ONLY)

/* Tuning options (host struct, may be NULL for defaults). */
typedef struct smla_options {
    int32_t num_splits;     /* 0 = automatic; > 0 = split every token's top-k
                               list into this many parts (capped at topk and at
                               32), each part computed by its own workgroups and
                               merged by log-sum-exp weights in a second kernel
                               on the same stream. */
    uint32_t flags;         /* SMLA_FLAG_* bits; any other bit is SMLA_ERR_ARG */
    int32_t reserved[6];    /* must be zero */
} smla_options;

/* Human-readable name of a status code (static string). */
const char *smla_status_string(smla_status status);

/* SMLA_ABI_VERSION of the loaded library. */
int32_t smla_abi_version(void);

/* Split plan and workspace size for an attention call, by host arithmetic
 * alone (no HIP call): num_cus is the device's compute-unit count (256 on
 * MI355X). Writes the number of top-k splits per token and the workspace bytes
 * an attention call with these sizes needs. Errors: SMLA_ERR_NULL,
 * SMLA_ERR_SHAPE, SMLA_ERR_ARG as for the attention calls. */
smla_status smla_plan(int32_t num_tokens, int32_t h_q, int32_t topk, int32_t num_cus,
                      const smla_options *options, int32_t *num_splits,
                      size_t *workspace_bytes);

/* Workspace bytes an attention call with these sizes and options needs on the
 * CURRENT device (its compute-unit count enters the split plan). Writes 0 when
 * no top-k split is planned. Errors as for the attention calls; SMLA_ERR_HIP if
 * the device cannot be queried. */
smla_status smla_workspace_size(int32_t num_tokens, int32_t h_q, int32_t topk,
                                const smla_options *options, size_t *workspace_bytes);

/* Log-sum-exp merge of per-part results into the final output
 * [flashmla_sparse.py page, FlashMLASparseImpl.forward: the sparse kernels return
 * the output and its log-sum-exp; parts of one list combine by the usual
 * log-sum-exp weights].
 *
 *   partials   device buffer, 256-B aligned, in this layout (F = num_parts):
 *                byte 0:               fp32 lse[num_tokens][F][h_q], natural log
 *                byte align256(T*F*h_q*4): fp32 o[num_tokens][F][h_q][512], each
 *                                      part's output normalised by its own sum
 *              (what an attention call with SMLA_FLAG_PARTIALS_ONLY writes into its
 *              workspace, F = its number of splits from smla_plan). A part with
 *              lse = -inf contributes nothing.
 *   partials_bytes  capacity of `partials` (SMLA_ERR_WORKSPACE if too small)
 *   out        bf16 [num_tokens, h_q, 512], 16-B aligned, every element written
 *   lse        fp32 [num_tokens, h_q] merged natural-log lse; may be NULL
 * h_q as for the attention calls; 1 <= num_parts <= 4096; num_tokens == 0 is a
 * no-op. Parts are added in index order, so results do not depend on timing.
 */
smla_status smla_merge_partials(const void *partials, size_t partials_bytes, int32_t num_tokens,
                                int32_t h_q, int32_t num_parts, void *out, float *lse,
                                hipStream_t stream);

/* Cache formats of smla_concat_and_cache_mla. */
#define SMLA_CACHE_BF16 0         /* bf16 rows [num_blocks, 64, 576] ("auto" on the page) */
#define SMLA_CACHE_FP8_DS_MLA 1   /* 656-byte fp8_ds_mla rows [num_blocks, 64, 656]     */
#define SMLA_CACHE_NVFP4_DS_MLA 2 /* 352-byte nvfp4_ds_mla rows [num_blocks, 64, 352]   */

/* Write tokens' latent and RoPE values into their slots of a paged cache
 * [flashmla_sparse.py page, FlashMLASparseImpl.forward: the concat_and_cache_mla
 * call before attention; module note on the fp8_ds_mla format].
 *
 *   k_c_normed    bf16 [num_tokens, 512] latent values, 16-B aligned
 *   k_pe          bf16 [num_tokens, 64] RoPE values, 16-B aligned
 *   slot_mapping  int64 [num_tokens]: flat slot (block * 64 + offset) of each
 *                 token; a slot < 0 or >= num_blocks * 64 writes nothing. Each
 *                 slot at most once per call (two tokens with one slot race).
 *   kv_cache      the cache, 16-B aligned, cache_format:
 *                 SMLA_CACHE_BF16: row = latent ++ RoPE, copied.
 *                 SMLA_CACHE_FP8_DS_MLA: row = 512 e4m3 bytes, 4 fp32 scales, 64
 *                 bf16 RoPE. Scale g = max |latent[128g .. 128g+127]| / 448 in
 *                 fp32 (1.0 for an all-zero group); byte i = latent[i] / scale g
 *                 (fp32 division) rounded to the nearest e4m3 value, ties to
 *                 even. (The page passes a k_scale here as well; the per-group
 *                 scales of this format do not use it.)
 *                 SMLA_CACHE_NVFP4_DS_MLA: row as at smla_decode_nvfp4. Scale b
 *                 = the e4m3 value nearest to max |latent[16b .. 16b+15]| / 6
 *                 (fp32 division, ties to even, at most 448); each code = the
 *                 E2M1 value nearest to latent / scale (fp32 division, ties to
 *                 even, saturating at 6), all codes 0 when the scale is 0; RoPE
 *                 = nearest e4m3 bytes, saturating at 448.
 * Only the rows of the given slots are written. num_tokens == 0 is a no-op.
 * Errors: SMLA_ERR_ARG (format), SMLA_ERR_SHAPE, SMLA_ERR_NULL, SMLA_ERR_ALIGN,
 * SMLA_ERR_HIP. */
smla_status smla_concat_and_cache_mla(const void *k_c_normed, const void *k_pe,
                                      const int64_t *slot_mapping, int32_t num_tokens, void *kv_cache,
                                      int64_t num_blocks, int32_t cache_format, hipStream_t stream);

/* Logical-to-physical index conversion alone [flashmla_sparse.py page,
 * triton_convert_req_index_to_global_index and docstring]:
 *   out[t,j] = block_table[req_id_per_token[t], topk_indices[t,j] / 64] * 64
 *              + topk_indices[t,j] % 64,  or -1 for an invalid position.
 * req_id_per_token int32 [num_tokens]; block_table int32 [num_reqs,
 * max_blocks_per_req]; topk_indices int32 [num_tokens, topk]; out int32
 * [num_tokens, topk]. All 4-byte aligned. num_blocks (the pool size in blocks)
 * must satisfy num_blocks * 64 <= INT32_MAX. Any topk >= 1 (no multiple-of-128
 * restriction). num_tokens == 0 is a no-op. */
smla_status smla_convert_indices(const int32_t *req_id_per_token, const int32_t *block_table,
                                 const int32_t *topk_indices, int32_t *out,
                                 int32_t num_tokens, int32_t topk, int32_t num_reqs,
                                 int32_t max_blocks_per_req, int64_t num_blocks,
                                 hipStream_t stream);

/* ---- separate-prefill mode of an fp8_ds_mla cache [flashmla_sparse.py page as
 * changed for this mode: _build_fp8_separate_prefill_decode,
 * _forward_fp8_kv_separate_prefill_decode, get_prefill_workspace_size]. Decode
 * tokens attend over the fp8 cache (smla_decode_fp8); prefill requests are cut
 * into chunks whose context fits a bf16 workspace, each chunk's context rows are
 * upconverted into the workspace (smla_gather_upconvert_fp8) and its tokens run
 * smla_prefill_bf16 over the workspace with SMLA_FLAG_SLOT_INDICES, their indices
 * converted to workspace rows (smla_convert_indices_workspace). */

/* Workspace rows the page reserves for a model: 5 * max_model_len (bf16 rows
 * of 576 values, 1152 bytes each). Host arithmetic; 0 for a negative length. */
int64_t smla_prefill_workspace_rows(int64_t max_model_len);

/* Chunk plan of the prefill requests (host arithmetic, host pointers): requests
 * are taken in order and a new chunk starts when the next request's length
 * would take the chunk past max_rows workspace rows (the page's worked example:
 * lengths [10, 15, 20, 5] give chunks [0, 2) and [2, 4) and starts
 * [0, 10, 0, 20] for any max_rows from 25 to 34).
 *   seq_lens          host int32 [num_prefills], context + query length of each
 *                     prefill request, each in [0, max_rows]
 *   chunk_ends        host int32 [num_prefills]: chunk c covers requests
 *                     [chunk_ends[c-1], chunk_ends[c]) (chunk_ends[-1] = 0)
 *   workspace_starts  host int32 [num_prefills]: each request's first workspace
 *                     row, counted from its chunk's start
 *   num_chunks        host out
 * Errors: SMLA_ERR_NULL, SMLA_ERR_SHAPE (a negative count or length, a request
 * longer than max_rows). num_prefills == 0 gives 0 chunks. */
smla_status smla_plan_prefill_chunks(const int32_t *seq_lens, int32_t num_prefills, int64_t max_rows,
                                     int32_t *chunk_ends, int32_t *workspace_starts, int32_t *num_chunks);

/* Index conversion with a prefill workspace [flashmla_sparse.py page,
 * _convert_req_index_to_global_index_kernel with HAS_PREFILL]: token t with
 * prefill_request_id[t] = r >= 0 maps a valid index i to workspace_starts[r] + i
 * (a workspace row); a token with r < 0 converts exactly as smla_convert_indices.
 * Either way an index is invalid (-1) when negative or when i / 64 >=
 * max_blocks_per_req; r >= num_prefills also gives -1.
 *   prefill_request_id  int32 [num_tokens], -1 for decode tokens
 *   workspace_starts    int32 [num_prefills] (chunk-local, as planned above);
 *                       may be NULL when num_prefills == 0
 * Other arguments as for smla_convert_indices. num_tokens == 0 is a no-op. */
smla_status smla_convert_indices_workspace(const int32_t *req_id_per_token, const int32_t *block_table,
                                           const int32_t *topk_indices, const int32_t *prefill_request_id,
                                           const int32_t *workspace_starts, int32_t *out,
                                           int32_t num_tokens, int32_t topk, int32_t num_reqs,
                                           int32_t max_blocks_per_req, int64_t num_blocks,
                                           int32_t num_prefills, hipStream_t stream);

/* Gather the context rows of a chunk of prefill requests from an fp8_ds_mla
 * cache and upconvert them into a bf16 workspace [flashmla_sparse.py page,
 * _forward_fp8_kv_separate_prefill_decode: cp_gather_and_upconvert_fp8_kv_cache]:
 * for request b < batch and position p < seq_lens[b], workspace row
 * workspace_starts[b] + p receives the cache row at slot
 * block_table[b, p / 64] * 64 + p % 64: latent value i is e4m3 byte i times
 * scale i / 128, rounded once to the nearest bf16 (ties to even); the 64 RoPE
 * values are copied. A position whose block lies outside the table, or whose
 * table entry lies outside [0, num_blocks), gives a row of zeros.
 *   kv_cache          uint8 [num_blocks, 64, 656], 16-B aligned
 *   block_table       int32 [batch, max_blocks_per_req]: the chunk's requests' rows
 *   seq_lens          int32 [batch], each <= max_seq_len
 *   workspace_starts  int32 [batch]
 *   max_seq_len       host bound on seq_lens (positions past it are not read)
 *   workspace         bf16 [workspace_rows, 576], 16-B aligned; rows outside
 *                     [0, workspace_rows) are never written, rows no request
 *                     covers keep their contents
 * Errors: SMLA_ERR_NULL, SMLA_ERR_SHAPE (also for batch > 65535: cut larger
 * chunks into several calls), SMLA_ERR_ALIGN, SMLA_ERR_HIP. batch == 0 or
 * max_seq_len == 0 is a no-op. */
smla_status smla_gather_upconvert_fp8(const void *kv_cache, int64_t num_blocks, const int32_t *block_table,
                                      int32_t max_blocks_per_req, const int32_t *seq_lens,
                                      const int32_t *workspace_starts, int32_t batch, int32_t max_seq_len,
                                      void *workspace, int64_t workspace_rows, hipStream_t stream);

/* The same gather over an nvfp4_ds_mla cache (rows as at smla_decode_nvfp4)
 * [pull-request page "Support nvfp4_ds_mla on FLASHINFER_MLA_SPARSE, with native
 * NVFP4 decode": prefill is staged through a context gather per request and
 * chunk]. Every staged value is exact: latent value i is its E2M1 code times its
 * block's E4M3 scale, and the 64 RoPE values are their E4M3 values; bf16 holds
 * all of them exactly. So the separate-prefill mode over an nvfp4 cache (this
 * call, smla_convert_indices_workspace and smla_prefill_bf16 with
 * SMLA_FLAG_SLOT_INDICES, decode tokens through smla_decode_nvfp4) gives what
 * smla_decode_nvfp4 gives over the whole batch, up to the kernels' own rounding.
 *   kv_cache  uint8 [num_blocks, 64, 352], 16-B aligned
 * Every other argument, the zero rows and the errors as for
 * smla_gather_upconvert_fp8. */
smla_status smla_gather_upconvert_nvfp4(const void *kv_cache, int64_t num_blocks, const int32_t *block_table,
                                        int32_t max_blocks_per_req, const int32_t *seq_lens,
                                        const int32_t *workspace_starts, int32_t batch, int32_t max_seq_len,
                                        void *workspace, int64_t workspace_rows, hipStream_t stream);

/* Sparse MLA forward over a bf16 paged cache [flashmla_sparse.py page,
 * _bf16_flash_mla_kernel / flash_mla_sparse_prefill].
 *
 *   q                 bf16 [num_tokens, h_q, 576]   (absorbed latent 512 ++ RoPE 64), 16-B aligned
 *   kv_cache          bf16 [num_blocks, 64, 576]    16-B aligned
 *   block_table       int32 [num_reqs, max_blocks_per_req]
 *   req_id_per_token  int32 [num_tokens]
 *   topk_indices      int32 [num_tokens, topk], logical positions, -1 = invalid
 *   sm_scale          softmax scale, finite and > 0 (e.g. 1/sqrt(576))
 *   h_q               16, 32, 64 or 128
 *   out               bf16 [num_tokens, h_q, 512], 16-B aligned, every element written
 *                     (may be NULL with SMLA_FLAG_PARTIALS_ONLY, which does not write it)
 *   lse               fp32 [num_tokens, h_q] natural-log LSE of the scaled logits; may be NULL
 *   phys_indices_out  int32 [num_tokens, topk] converted slots (-1 = invalid), bit-identical
 *                     to smla_convert_indices; may be NULL
 *   workspace         device scratch for the per-part results of a top-k split (partial
 *                     outputs, their lse and, for a call that merges its own parts, one
 *                     int32 flag per token and part), 256-B aligned; may be NULL when
 *                     smla_workspace_size reports 0 bytes for these sizes. Its contents
 *                     need not be initialised; they are written before they are read
 *                     within the call. Calls that overlap in time (other streams) must
 *                     not share a workspace.
 *   workspace_bytes   capacity of `workspace` in bytes (SMLA_ERR_WORKSPACE if too small)
 *   options           host pointer or NULL; the same options must be given to
 *                     smla_workspace_size
 * Any mix of decode, speculative-decode and prefill tokens may share one call.
 */
smla_status smla_prefill_bf16(const void *q, const void *kv_cache, const int32_t *block_table,
                              const int32_t *req_id_per_token, const int32_t *topk_indices,
                              float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                              int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                              void *out, float *lse, int32_t *phys_indices_out,
                              void *workspace, size_t workspace_bytes,
                              const smla_options *options, hipStream_t stream);

/* Sparse MLA forward over an fp8_ds_mla paged cache [flashmla_sparse.py page,
 * module note on the 656-byte format, _fp8_flash_mla_kernel /
 * flash_mla_with_kvcache with is_fp8_kvcache and indices].
 *
 *   kv_cache  uint8 [num_blocks, 64, 656], 16-B aligned; each row is 512 OCP E4M3FN latent
 *             bytes, 4 little-endian fp32 scales (scale i multiplies latent values
 *             128*i .. 128*i+127), 64 bf16 RoPE values.
 * Every other argument as for smla_prefill_bf16. The rows are dequantised inside
 * the kernel as they are gathered; no staging copy of the cache is made.
 */
smla_status smla_decode_fp8(const void *q, const void *kv_cache, const int32_t *block_table,
                            const int32_t *req_id_per_token, const int32_t *topk_indices,
                            float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                            int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                            void *out, float *lse, int32_t *phys_indices_out,
                            void *workspace, size_t workspace_bytes,
                            const smla_options *options, hipStream_t stream);

/* Sparse MLA forward over an nvfp4_ds_mla paged cache, decoded natively: the
 * rows are read as stored and attended over with their exact values, with no
 * staging copy and no re-rounding [vLLM pull-request page "Support nvfp4_ds_mla
 * on FLASHINFER_MLA_SPARSE, with native NVFP4 decode", description and design
 * notes: 352 bytes per token, native decode at 16 heads and top-k 512, 1024,
 * 2048].
 *
 *   kv_cache  uint8 [num_blocks, 64, 352], 16-B aligned. The page gives the
 *             row size only; the layout is the split of 352 bytes into NVFP4
 *             pieces: bytes 0..255 hold the 512 latent values as OCP E2M1
 *             codes, two per byte, value 2i in the low nibble of byte i and
 *             2i+1 in the high nibble; bytes 256..287 hold 32 OCP E4M3FN
 *             scales, scale b multiplying latent values 16b .. 16b+15; bytes
 *             288..351 hold the 64 RoPE values as E4M3FN bytes. A latent value
 *             is E2M1 x scale (no per-tensor factor: the page's k_scale belongs
 *             to its fp8 staging copy, which this call never makes).
 * Every h_q of smla_prefill_bf16 is accepted; each 16 heads of a token are one
 * workgroup, which gathers the token's rows itself. Every other argument,
 * the workspace contract and the errors as for smla_prefill_bf16.
 */
smla_status smla_decode_nvfp4(const void *q, const void *kv_cache, const int32_t *block_table,
                              const int32_t *req_id_per_token, const int32_t *topk_indices,
                              float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                              int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                              void *out, float *lse, int32_t *phys_indices_out,
                              void *workspace, size_t workspace_bytes,
                              const smla_options *options, hipStream_t stream);

/* Split workspace of smla_decode_fp8_noalloc: 64 MiB of device memory that the
 * library holds on each device it runs on, until the process ends. */
#define SMLA_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* smla_decode_fp8 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same computation, arguments and results as smla_decode_fp8, minus the
 * workspace: a call whose top-k lists are split keeps its per-part results in a
 * library-owned array of SMLA_STATIC_WORKSPACE_BYTES on the current device
 * (found once per device with hipGetSymbolAddress), and the call makes no
 * allocation of any kind. Nothing in that array needs initialising: each call
 * writes every entry it later reads. Every call on one device shares the
 * device's array, so calls that may overlap on one device (other streams,
 * other host threads) race; order them on one stream or use smla_decode_fp8
 * with workspaces of their own.
 * Errors: as smla_decode_fp8; SMLA_ERR_WORKSPACE if the split plan needs more
 * than SMLA_STATIC_WORKSPACE_BYTES (smla_workspace_size reports the need);
 * SMLA_ERR_ARG for SMLA_FLAG_PARTIALS_ONLY, SMLA_FLAG_DEFER_MERGE or
 * SMLA_FLAG_MERGE_ONLY (their parts would live in the shared array);
 * SMLA_ERR_HIP if the array's address cannot be found. Nothing is launched
 * or written on an error. */
smla_status smla_decode_fp8_noalloc(const void *q, const void *kv_cache, const int32_t *block_table,
                                    const int32_t *req_id_per_token, const int32_t *topk_indices,
                                    float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                                    int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                                    void *out, float *lse, int32_t *phys_indices_out,
                                    const smla_options *options, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
