// smla_internal.h -- shared between the C-ABI layer (smla_api.cpp) and the HIP
// kernels (smla_kernels.hip). Not installed; the public interface is
// include/smla.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace smla {

constexpr int kBlock = 64;        // paged-cache block size (tokens per block)
constexpr int kDqk = 576;         // query/key width: 512 latent + 64 RoPE
constexpr int kDv = 512;          // value width: the latent part of the row
constexpr int kFp8RowBytes = 656; // 512 e4m3 + 4 fp32 scales + 64 bf16
constexpr int kBf16RowBytes = kDqk * 2;
constexpr int kNvfp4RowBytes = 352;  // 512 E2M1 codes + 32 E4M3 block scales + 64 E4M3 RoPE

enum CacheFormat { kCacheBf16 = 0, kCacheFp8 = 1, kCacheNvfp4 = 2 };

// A workgroup covers all h_q heads of its token (128: four waves of 32 heads
// for the bf16 cache; 64: eight waves; 32 or 16), except fp8 with h_q = 128,
// which takes two 64-head workgroups per token and part, and nvfp4, which
// takes one 16-head workgroup per head block.
constexpr int kHeadsPerGroup = 64;

// Most top-k parts one token's list is cut into.
constexpr int kMaxSplits = 32;

// Bytes of the split workspace that the allocation-free entry point takes from
// a library-owned device array (one per device, held until the process ends).
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;

struct Plan {
    int num_splits;          // top-k parts per token
    int split_len;           // top-k positions per part (the last part may be shorter)
    size_t workspace;        // bytes needed (0 when num_splits == 1)
    size_t part_lse_off;     // byte offsets inside the workspace: [T][S][H] fp32 lse,
    size_t part_o_off;       // [T][S][H][512] fp32 partial outputs (or bf16 rows in them)
    size_t part_exact_off;   // and, for a call that merges its own splits, [T][S] int32 flags
};

// Host arithmetic only. partials: the call writes per-part results (workspace
// needed even for one part).
Plan make_plan(int num_tokens, int h_q, int topk, int num_cus, int forced_splits, bool partials);

// Byte offset of the partial outputs in a partials buffer of T x F x H entries.
size_t partials_o_offset(size_t rows);

struct AttnArgs {
    const void *q;
    const void *cache;
    const int32_t *block_table;
    const int32_t *req_id;
    const int32_t *topk;
    void *out;
    float *lse;
    int32_t *phys_out;
    void *workspace;
    float sm_scale;
    int num_tokens, h_q, topk_len, num_reqs, max_blocks;
    int64_t num_blocks;
    bool slot_indices;       // topk holds cache slots (no request / table lookup)
};

// Kernel launchers (smla_kernels.hip). Return hipSuccess or the launch error.
hipError_t launch_convert(const int32_t *req_id, const int32_t *block_table, const int32_t *topk,
                          int32_t *out, int num_tokens, int topk_len, int num_reqs,
                          int max_blocks, int64_t num_blocks, hipStream_t stream);

// convert_kernel with a prefill workspace: tokens with prefill_request_id >= 0
// map valid indices to workspace_starts[id] + index.
hipError_t launch_convert_ws(const int32_t *req_id, const int32_t *block_table, const int32_t *topk,
                             const int32_t *prefill_rid, const int32_t *ws_starts, int32_t *out,
                             int num_tokens, int topk_len, int num_reqs, int max_blocks, int64_t num_blocks,
                             int num_prefills, hipStream_t stream);

// upconvert_kernel / upconvert_nvfp4_kernel: context rows of `batch` prefill
// requests from an fp8_ds_mla or nvfp4_ds_mla cache into a bf16 workspace.
hipError_t launch_upconvert(CacheFormat fmt, const void *cache, int64_t num_blocks, const int32_t *block_table,
                            int max_blocks, const int32_t *seq_lens, const int32_t *ws_starts, int batch,
                            int max_seq_len, void *workspace, int64_t workspace_rows, hipStream_t stream);

// The attention kernel and, when the plan splits the top-k lists (and
// partials_only is false), the merge kernel after it on the same stream.
// Which kernels of a call run: both, the attention kernel only (a split
// call's merge deferred), or the merge only.
enum class AttnStage { kBoth, kAttentionOnly, kMergeOnly };

hipError_t launch_attention(CacheFormat fmt, const AttnArgs &a, const Plan &p, bool partials_only,
                            AttnStage stage, hipStream_t stream);

// cache_write_kernel: rows of num_tokens tokens into their slots (< num_slots).
hipError_t launch_cache_write(CacheFormat fmt, const void *k_c, const void *k_pe, const int64_t *slot_mapping,
                             void *cache, int64_t num_tokens, int64_t num_slots, hipStream_t stream);

// Device address of this device's static split workspace (kStaticWorkspaceBytes,
// 256-byte aligned), looked up once per device; the current device must be set.
hipError_t static_workspace(void **ptr);

// merge_kernel alone over a partials buffer of T x S x H entries; part_exact
// null: fp32 partials, else bf16 rows and their flags (attn_pc_kernel's form).
hipError_t launch_merge(const float *part_lse, const float *part_o, const int32_t *part_exact, void *out,
                        float *lse, int T, int H, int S, hipStream_t stream);

}  // namespace smla
