// smla_api.cpp -- the C ABI declared in include/smla.h: argument validation,
// the split planner and the workspace contract. Every check runs before the
// first HIP call, so invalid calls fail without touching a device.

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/smla.h"
#include "smla_internal.h"

namespace smla {

static_assert(SMLA_STATIC_WORKSPACE_BYTES == kStaticWorkspaceBytes, "static workspace size in the header");

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t partials_o_offset(size_t rows) { return align_up(rows * sizeof(float), 256); }

Plan make_plan(int num_tokens, int h_q, int topk, int num_cus, int forced_splits, bool partials)
{
    Plan p{};
    int splits = 1;
    if (forced_splits > 0) {
        splits = std::min(std::min(forced_splits, topk), kMaxSplits);
    } else {
        // One workgroup per token when that fills the chip; otherwise cut each
        // token's list so the grid covers every workgroup slot once: 64- and
        // 128-head workgroups take a CU each, 32- and 16-head ones fit two per
        // CU. (fp8 with h_q = 128 runs two 64-head workgroups per token and
        // part under the same plan, so the plan and the workspace it sizes do
        // not depend on the cache format.)
        // A list of at most kShortList positions is not cut once every CU has a
        // workgroup: the merge launch then costs more than the second
        // workgroup per CU gains.
        const int64_t units = num_tokens;
        const int64_t slots = (int64_t)num_cus * (h_q >= kHeadsPerGroup ? 1 : 2);
        const int64_t tiles = (topk + kBlock - 1) / kBlock;
        constexpr int kShortList = 512;
        if (units > 0 && units < slots && !(units >= num_cus && topk <= kShortList))
            splits = (int)std::min<int64_t>(std::min<int64_t>(tiles, kMaxSplits), (slots + units - 1) / units);
        splits = std::max(splits, 1);
    }
    p.split_len = (topk + splits - 1) / splits;
    p.num_splits = (topk + p.split_len - 1) / p.split_len;
    if (p.num_splits > 1 || partials) {
        const size_t rows = (size_t)num_tokens * p.num_splits * h_q;
        p.part_lse_off = 0;
        p.part_o_off = partials_o_offset(rows);
        p.workspace = align_up(p.part_o_off + rows * kDv * sizeof(float), 256);
        if (!partials) {
            p.part_exact_off = p.workspace;
            p.workspace = align_up(p.part_exact_off + (size_t)num_tokens * p.num_splits * sizeof(int32_t), 256);
        }
    }
    return p;
}

namespace {

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

smla_status check_options(const smla_options *o)
{
    if (o == nullptr)
        return SMLA_OK;
    if (o->num_splits < 0 || (o->flags & ~(uint32_t)SMLA_FLAG_ALL) != 0)
        return SMLA_ERR_ARG;
    const uint32_t stages = o->flags & (SMLA_FLAG_DEFER_MERGE | SMLA_FLAG_MERGE_ONLY);
    if (stages == (SMLA_FLAG_DEFER_MERGE | SMLA_FLAG_MERGE_ONLY) ||
        (stages != 0 && (o->flags & SMLA_FLAG_PARTIALS_ONLY)))
        return SMLA_ERR_ARG;
    for (int i = 0; i < 6; ++i)
        if (o->reserved[i] != 0)
            return SMLA_ERR_ARG;
    return SMLA_OK;
}

smla_status check_sizes(int32_t num_tokens, int32_t h_q, int32_t topk)
{
    if (h_q != 16 && h_q != 32 && h_q != 64 && h_q != 128)
        return SMLA_ERR_SHAPE;
    if (num_tokens < 0 || topk < 1 || topk > SMLA_MAX_TOPK)
        return SMLA_ERR_SHAPE;
    return SMLA_OK;
}

smla_status check_pool(int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks)
{
    if (num_reqs < 1 || max_blocks_per_req < 1 || num_blocks < 1)
        return SMLA_ERR_SHAPE;
    if (num_blocks > (int64_t)INT32_MAX / kBlock)   // slots are int32
        return SMLA_ERR_SHAPE;
    return SMLA_OK;
}

// Compute units of the current device, cached per device id.
smla_status device_cus(int *cus)
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return SMLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 64 && cache[dev] > 0) {
        *cus = cache[dev];
        return SMLA_OK;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return SMLA_ERR_HIP;
    if (dev < 64)
        cache[dev] = n;
    *cus = n;
    return SMLA_OK;
}

smla_status attention_entry(CacheFormat fmt, const void *q, const void *kv_cache,
                            const int32_t *block_table, const int32_t *req_id_per_token,
                            const int32_t *topk_indices, float sm_scale, int32_t num_tokens,
                            int32_t h_q, int32_t topk, int32_t num_reqs,
                            int32_t max_blocks_per_req, int64_t num_blocks, void *out, float *lse,
                            int32_t *phys_indices_out, void *workspace, size_t workspace_bytes,
                            const smla_options *options, hipStream_t stream, bool static_ws = false)
{
    smla_status st = check_options(options);
    if (st != SMLA_OK)
        return st;
    // the static workspace holds one call's own parts: no staged or parts-only calls
    if (static_ws && options &&
        (options->flags & (SMLA_FLAG_PARTIALS_ONLY | SMLA_FLAG_DEFER_MERGE | SMLA_FLAG_MERGE_ONLY)))
        return SMLA_ERR_ARG;
    if (!(sm_scale > 0.f) || !isfinite(sm_scale))
        return SMLA_ERR_ARG;
    if ((st = check_sizes(num_tokens, h_q, topk)) != SMLA_OK)
        return st;
    const bool slot_in = options && (options->flags & SMLA_FLAG_SLOT_INDICES);
    if (slot_in) {
        // indices are cache slots: no request or table is read
        block_table = nullptr;
        req_id_per_token = nullptr;
        num_reqs = 1;
        max_blocks_per_req = 1;
    }
    if ((st = check_pool(num_reqs, max_blocks_per_req, num_blocks)) != SMLA_OK)
        return st;
    if (num_tokens == 0)
        return SMLA_OK;
    const bool partials_only = options && (options->flags & SMLA_FLAG_PARTIALS_ONLY);
    if (!q || !kv_cache || (!slot_in && (!block_table || !req_id_per_token)) || !topk_indices ||
        (!out && !partials_only))
        return SMLA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16))
        return SMLA_ERR_ALIGN;
    if (!aligned(block_table, 4) || !aligned(req_id_per_token, 4) || !aligned(topk_indices, 4) ||
        !aligned(lse, 4) || !aligned(phys_indices_out, 4) || !aligned(workspace, 256))
        return SMLA_ERR_ALIGN;
    const int forced = options ? options->num_splits : 0;

    int cus = 0;
    if ((st = device_cus(&cus)) != SMLA_OK)
        return st;
    const Plan plan = make_plan(num_tokens, h_q, topk, cus, forced, partials_only);
    if (static_ws) {
        // no allocation: the device's static array, or an error if the plan needs more
        if (plan.workspace > kStaticWorkspaceBytes)
            return SMLA_ERR_WORKSPACE;
        workspace = nullptr;
        if (plan.workspace > 0 && static_workspace(&workspace) != hipSuccess)
            return SMLA_ERR_HIP;
        workspace_bytes = plan.workspace;
    }
    if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
        return SMLA_ERR_WORKSPACE;

    AttnArgs a;
    a.q = q;
    a.cache = kv_cache;
    a.block_table = block_table;
    a.req_id = req_id_per_token;
    a.topk = topk_indices;
    a.out = out;
    a.lse = lse;
    a.phys_out = phys_indices_out;
    a.workspace = workspace;
    a.sm_scale = sm_scale;
    a.num_tokens = num_tokens;
    a.h_q = h_q;
    a.topk_len = topk;
    a.num_reqs = num_reqs;
    a.max_blocks = max_blocks_per_req;
    a.num_blocks = num_blocks;
    a.slot_indices = slot_in;
    const AttnStage stage = !options                                      ? AttnStage::kBoth
                            : (options->flags & SMLA_FLAG_DEFER_MERGE) ? AttnStage::kAttentionOnly
                            : (options->flags & SMLA_FLAG_MERGE_ONLY)  ? AttnStage::kMergeOnly
                                                                       : AttnStage::kBoth;
    return launch_attention(fmt, a, plan, partials_only, stage, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

}  // namespace
}  // namespace smla

extern "C" {

const char *smla_status_string(smla_status status)
{
    switch (status) {
    case SMLA_OK: return "SMLA_OK";
    case SMLA_ERR_NULL: return "SMLA_ERR_NULL: a required pointer is NULL";
    case SMLA_ERR_SHAPE: return "SMLA_ERR_SHAPE: unsupported size";
    case SMLA_ERR_ALIGN: return "SMLA_ERR_ALIGN: pointer not aligned as required";
    case SMLA_ERR_WORKSPACE: return "SMLA_ERR_WORKSPACE: workspace too small";
    case SMLA_ERR_HIP: return "SMLA_ERR_HIP: HIP runtime or launch failure";
    case SMLA_ERR_ARG: return "SMLA_ERR_ARG: invalid scalar argument or option";
    }
    return "unknown smla_status";
}

int32_t smla_abi_version(void) { return SMLA_ABI_VERSION; }

smla_status smla_plan(int32_t num_tokens, int32_t h_q, int32_t topk, int32_t num_cus,
                      const smla_options *options, int32_t *num_splits, size_t *workspace_bytes)
{
    if (num_splits == nullptr || workspace_bytes == nullptr)
        return SMLA_ERR_NULL;
    smla_status st = smla::check_options(options);
    if (st != SMLA_OK)
        return st;
    if ((st = smla::check_sizes(num_tokens, h_q, topk)) != SMLA_OK)
        return st;
    if (num_cus < 1)
        return SMLA_ERR_ARG;
    if (num_tokens == 0) {
        *num_splits = 1;
        *workspace_bytes = 0;
        return SMLA_OK;
    }
    const smla::Plan p = smla::make_plan(num_tokens, h_q, topk, num_cus, options ? options->num_splits : 0,
                                         options && (options->flags & SMLA_FLAG_PARTIALS_ONLY));
    *num_splits = p.num_splits;
    *workspace_bytes = p.workspace;
    return SMLA_OK;
}

smla_status smla_workspace_size(int32_t num_tokens, int32_t h_q, int32_t topk,
                                const smla_options *options, size_t *workspace_bytes)
{
    if (workspace_bytes == nullptr)
        return SMLA_ERR_NULL;
    smla_status st = smla::check_options(options);
    if (st != SMLA_OK)
        return st;
    if ((st = smla::check_sizes(num_tokens, h_q, topk)) != SMLA_OK)
        return st;
    if (num_tokens == 0) {
        *workspace_bytes = 0;
        return SMLA_OK;
    }
    int cus = 0;
    if ((st = smla::device_cus(&cus)) != SMLA_OK)
        return st;
    *workspace_bytes =
        smla::make_plan(num_tokens, h_q, topk, cus, options ? options->num_splits : 0,
                        options && (options->flags & SMLA_FLAG_PARTIALS_ONLY))
            .workspace;
    return SMLA_OK;
}

smla_status smla_merge_partials(const void *partials, size_t partials_bytes, int32_t num_tokens,
                                int32_t h_q, int32_t num_parts, void *out, float *lse,
                                hipStream_t stream)
{
    if (h_q != 16 && h_q != 32 && h_q != 64 && h_q != 128)
        return SMLA_ERR_SHAPE;
    if (num_tokens < 0 || num_parts < 1 || num_parts > 4096)
        return SMLA_ERR_SHAPE;
    if (num_tokens == 0)
        return SMLA_OK;
    if (!partials || !out)
        return SMLA_ERR_NULL;
    if (!smla::aligned(partials, 256) || !smla::aligned(out, 16) || !smla::aligned(lse, 4))
        return SMLA_ERR_ALIGN;
    const size_t rows = (size_t)num_tokens * num_parts * h_q;
    const size_t o_off = smla::partials_o_offset(rows);
    if (partials_bytes < o_off + rows * smla::kDv * sizeof(float))
        return SMLA_ERR_WORKSPACE;
    const float *base = (const float *)partials;
    return smla::launch_merge(base, (const float *)((const char *)partials + o_off), nullptr, out, lse,
                              num_tokens, h_q, num_parts, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

smla_status smla_concat_and_cache_mla(const void *k_c_normed, const void *k_pe,
                                      const int64_t *slot_mapping, int32_t num_tokens, void *kv_cache,
                                      int64_t num_blocks, int32_t cache_format, hipStream_t stream)
{
    if (cache_format != SMLA_CACHE_BF16 && cache_format != SMLA_CACHE_FP8_DS_MLA &&
        cache_format != SMLA_CACHE_NVFP4_DS_MLA)
        return SMLA_ERR_ARG;
    if (num_tokens < 0 || num_blocks < 1 || num_blocks > INT64_MAX / (smla::kBlock * smla::kBf16RowBytes))
        return SMLA_ERR_SHAPE;
    if (num_tokens == 0)
        return SMLA_OK;
    if (!k_c_normed || !k_pe || !slot_mapping || !kv_cache)
        return SMLA_ERR_NULL;
    if (!smla::aligned(k_c_normed, 16) || !smla::aligned(k_pe, 16) || !smla::aligned(slot_mapping, 8) ||
        !smla::aligned(kv_cache, 16))
        return SMLA_ERR_ALIGN;
    const smla::CacheFormat fmt = cache_format == SMLA_CACHE_FP8_DS_MLA     ? smla::kCacheFp8
                                  : cache_format == SMLA_CACHE_NVFP4_DS_MLA ? smla::kCacheNvfp4
                                                                            : smla::kCacheBf16;
    return smla::launch_cache_write(fmt, k_c_normed, k_pe, slot_mapping, kv_cache, num_tokens,
                                    num_blocks * smla::kBlock, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

int64_t smla_prefill_workspace_rows(int64_t max_model_len)
{
    return max_model_len > 0 && max_model_len <= INT64_MAX / 5 ? 5 * max_model_len : 0;
}

smla_status smla_plan_prefill_chunks(const int32_t *seq_lens, int32_t num_prefills, int64_t max_rows,
                                     int32_t *chunk_ends, int32_t *workspace_starts, int32_t *num_chunks)
{
    if (num_chunks == nullptr)
        return SMLA_ERR_NULL;
    if (num_prefills < 0 || max_rows < 0 || max_rows > INT32_MAX)
        return SMLA_ERR_SHAPE;
    if (num_prefills > 0 && (!seq_lens || !chunk_ends || !workspace_starts))
        return SMLA_ERR_NULL;
    for (int32_t r = 0; r < num_prefills; ++r)
        if (seq_lens[r] < 0 || seq_lens[r] > max_rows)
            return SMLA_ERR_SHAPE;
    // a request starts a new chunk when it would not fit the current one
    int32_t n = 0;
    int64_t used = 0;
    for (int32_t r = 0; r < num_prefills; ++r) {
        if (r > 0 && used + seq_lens[r] > max_rows) {
            chunk_ends[n++] = r;
            used = 0;
        }
        workspace_starts[r] = (int32_t)used;
        used += seq_lens[r];
    }
    if (num_prefills > 0)
        chunk_ends[n++] = num_prefills;
    *num_chunks = n;
    return SMLA_OK;
}

smla_status smla_convert_indices_workspace(const int32_t *req_id_per_token, const int32_t *block_table,
                                           const int32_t *topk_indices, const int32_t *prefill_request_id,
                                           const int32_t *workspace_starts, int32_t *out,
                                           int32_t num_tokens, int32_t topk, int32_t num_reqs,
                                           int32_t max_blocks_per_req, int64_t num_blocks,
                                           int32_t num_prefills, hipStream_t stream)
{
    if (num_tokens < 0 || topk < 1 || topk > SMLA_MAX_TOPK || num_prefills < 0)
        return SMLA_ERR_SHAPE;
    smla_status st = smla::check_pool(num_reqs, max_blocks_per_req, num_blocks);
    if (st != SMLA_OK)
        return st;
    if (num_tokens == 0)
        return SMLA_OK;
    if (!req_id_per_token || !block_table || !topk_indices || !prefill_request_id || !out ||
        (num_prefills > 0 && !workspace_starts))
        return SMLA_ERR_NULL;
    if (!smla::aligned(req_id_per_token, 4) || !smla::aligned(block_table, 4) ||
        !smla::aligned(topk_indices, 4) || !smla::aligned(prefill_request_id, 4) ||
        !smla::aligned(workspace_starts, 4) || !smla::aligned(out, 4))
        return SMLA_ERR_ALIGN;
    return smla::launch_convert_ws(req_id_per_token, block_table, topk_indices, prefill_request_id,
                                   workspace_starts, out, num_tokens, topk, num_reqs, max_blocks_per_req,
                                   num_blocks, num_prefills, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

// requests of one upconvert call: the second grid dimension of its launch
constexpr int32_t kMaxUpconvertBatch = 65535;

namespace smla {
namespace {

smla_status gather_upconvert(CacheFormat fmt, const void *kv_cache, int64_t num_blocks, const int32_t *block_table,
                             int32_t max_blocks_per_req, const int32_t *seq_lens, const int32_t *workspace_starts,
                             int32_t batch, int32_t max_seq_len, void *workspace, int64_t workspace_rows,
                             hipStream_t stream)
{
    if (batch < 0 || batch > kMaxUpconvertBatch || max_seq_len < 0 || workspace_rows < 0 ||
        max_blocks_per_req < 1 || num_blocks < 1 || num_blocks > (int64_t)INT32_MAX / kBlock)
        return SMLA_ERR_SHAPE;
    if (batch == 0 || max_seq_len == 0)
        return SMLA_OK;
    if (!kv_cache || !block_table || !seq_lens || !workspace_starts || !workspace)
        return SMLA_ERR_NULL;
    if (!aligned(kv_cache, 16) || !aligned(workspace, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(workspace_starts, 4))
        return SMLA_ERR_ALIGN;
    return launch_upconvert(fmt, kv_cache, num_blocks, block_table, max_blocks_per_req, seq_lens,
                            workspace_starts, batch, max_seq_len, workspace, workspace_rows, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

}  // namespace
}  // namespace smla

smla_status smla_gather_upconvert_fp8(const void *kv_cache, int64_t num_blocks, const int32_t *block_table,
                                      int32_t max_blocks_per_req, const int32_t *seq_lens,
                                      const int32_t *workspace_starts, int32_t batch, int32_t max_seq_len,
                                      void *workspace, int64_t workspace_rows, hipStream_t stream)
{
    return smla::gather_upconvert(smla::kCacheFp8, kv_cache, num_blocks, block_table, max_blocks_per_req, seq_lens,
                                  workspace_starts, batch, max_seq_len, workspace, workspace_rows, stream);
}

smla_status smla_gather_upconvert_nvfp4(const void *kv_cache, int64_t num_blocks, const int32_t *block_table,
                                        int32_t max_blocks_per_req, const int32_t *seq_lens,
                                        const int32_t *workspace_starts, int32_t batch, int32_t max_seq_len,
                                        void *workspace, int64_t workspace_rows, hipStream_t stream)
{
    return smla::gather_upconvert(smla::kCacheNvfp4, kv_cache, num_blocks, block_table, max_blocks_per_req,
                                  seq_lens, workspace_starts, batch, max_seq_len, workspace, workspace_rows,
                                  stream);
}

smla_status smla_convert_indices(const int32_t *req_id_per_token, const int32_t *block_table,
                                 const int32_t *topk_indices, int32_t *out, int32_t num_tokens,
                                 int32_t topk, int32_t num_reqs, int32_t max_blocks_per_req,
                                 int64_t num_blocks, hipStream_t stream)
{
    if (num_tokens < 0 || topk < 1 || topk > SMLA_MAX_TOPK)
        return SMLA_ERR_SHAPE;
    smla_status st = smla::check_pool(num_reqs, max_blocks_per_req, num_blocks);
    if (st != SMLA_OK)
        return st;
    if (num_tokens == 0)
        return SMLA_OK;
    if (!req_id_per_token || !block_table || !topk_indices || !out)
        return SMLA_ERR_NULL;
    if (!smla::aligned(req_id_per_token, 4) || !smla::aligned(block_table, 4) ||
        !smla::aligned(topk_indices, 4) || !smla::aligned(out, 4))
        return SMLA_ERR_ALIGN;
    return smla::launch_convert(req_id_per_token, block_table, topk_indices, out, num_tokens, topk,
                                num_reqs, max_blocks_per_req, num_blocks, stream) == hipSuccess
               ? SMLA_OK
               : SMLA_ERR_HIP;
}

smla_status smla_prefill_bf16(const void *q, const void *kv_cache, const int32_t *block_table,
                              const int32_t *req_id_per_token, const int32_t *topk_indices,
                              float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                              int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                              void *out, float *lse, int32_t *phys_indices_out, void *workspace,
                              size_t workspace_bytes, const smla_options *options,
                              hipStream_t stream)
{
    return smla::attention_entry(smla::kCacheBf16, q, kv_cache, block_table, req_id_per_token,
                                 topk_indices, sm_scale, num_tokens, h_q, topk, num_reqs,
                                 max_blocks_per_req, num_blocks, out, lse, phys_indices_out,
                                 workspace, workspace_bytes, options, stream);
}

smla_status smla_decode_fp8(const void *q, const void *kv_cache, const int32_t *block_table,
                            const int32_t *req_id_per_token, const int32_t *topk_indices,
                            float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                            int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                            void *out, float *lse, int32_t *phys_indices_out, void *workspace,
                            size_t workspace_bytes, const smla_options *options,
                            hipStream_t stream)
{
    return smla::attention_entry(smla::kCacheFp8, q, kv_cache, block_table, req_id_per_token,
                                 topk_indices, sm_scale, num_tokens, h_q, topk, num_reqs,
                                 max_blocks_per_req, num_blocks, out, lse, phys_indices_out,
                                 workspace, workspace_bytes, options, stream);
}

smla_status smla_decode_nvfp4(const void *q, const void *kv_cache, const int32_t *block_table,
                              const int32_t *req_id_per_token, const int32_t *topk_indices,
                              float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                              int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                              void *out, float *lse, int32_t *phys_indices_out, void *workspace,
                              size_t workspace_bytes, const smla_options *options,
                              hipStream_t stream)
{
    return smla::attention_entry(smla::kCacheNvfp4, q, kv_cache, block_table, req_id_per_token,
                                 topk_indices, sm_scale, num_tokens, h_q, topk, num_reqs,
                                 max_blocks_per_req, num_blocks, out, lse, phys_indices_out,
                                 workspace, workspace_bytes, options, stream);
}

smla_status smla_decode_fp8_noalloc(const void *q, const void *kv_cache, const int32_t *block_table,
                                    const int32_t *req_id_per_token, const int32_t *topk_indices,
                                    float sm_scale, int32_t num_tokens, int32_t h_q, int32_t topk,
                                    int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_blocks,
                                    void *out, float *lse, int32_t *phys_indices_out,
                                    const smla_options *options, hipStream_t stream)
{
    return smla::attention_entry(smla::kCacheFp8, q, kv_cache, block_table, req_id_per_token,
                                 topk_indices, sm_scale, num_tokens, h_q, topk, num_reqs,
                                 max_blocks_per_req, num_blocks, out, lse, phys_indices_out, nullptr, 0,
                                 options, stream, true);
}

}  // extern "C"
