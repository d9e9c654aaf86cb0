// C ABI of the paged-KV decode library: host-side validation and dispatch.
// Declarations and the argument contract are in include/pkv.h.
#include "../../include/pkv.h"

#include <cmath>
#include <cstdint>

#include "pkv_internal.h"

namespace {

constexpr int kAbiVersion = 11;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool known_dtype(int dt) { return dt == PKV_DTYPE_F32 || dt == PKV_DTYPE_BF16 || dt == PKV_DTYPE_FP8_E4M3; }

}  // namespace

extern "C" {

int pkv_abi_version(void) { return kAbiVersion; }

const char* pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported combination";
    case PKV_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
    case PKV_ERR_SCRATCH: return "the no-allocation decode's static scratch is too small for these sizes";
    default: return "unknown status";
    }
}

int paged_kv_write(const void* k_new, const void* v_new, int in_dtype,
                   void* k_cache, void* v_cache, int cache_dtype,
                   const int32_t* slot_mapping, int32_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t num_blocks, float k_scale, float v_scale,
                   void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
        return PKV_ERR_INVALID_ARG;
    if (!known_dtype(in_dtype) || !known_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
    if (block_size != pkv::kBlockTokens || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
    const bool quant = in_dtype != cache_dtype;
    if (quant && !(cache_dtype == PKV_DTYPE_FP8_E4M3 && (in_dtype == PKV_DTYPE_F32 || in_dtype == PKV_DTYPE_BF16)))
        return PKV_ERR_UNSUPPORTED;
    if (quant && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return PKV_ERR_INVALID_ARG;
    if (int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 4))
        return PKV_ERR_ALIGNMENT;
    if (num_blocks == 0) return PKV_OK;  // every slot is out of range: nothing can be written

    pkv::WriteArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.num_slots = num_blocks * pkv::kBlockTokens;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    const hipError_t e = pkv::launch_kv_write(in_dtype, cache_dtype, head_dim, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_dim <= 0 ||
        max_blocks_per_seq < 0 || block_size != pkv::kBlockTokens)
        return 0;
    if (partition_size < 0 || partition_size % pkv::kBlockTokens != 0) return 0;
    return size_t(pkv::workspace_floats(pkv::run_heads(num_heads / num_kv_heads), head_dim)) * sizeof(float);
}

}  // extern "C"

namespace {

// Sequences whose heads share one prefix run's matrix columns.
int prefix_members(int rh) { return pkv::kMaxRunHeads / rh; }

int64_t cascade_extra_floats(int64_t num_seqs, int num_heads, int head_dim) {
    return 2 * pkv::align_floats(num_seqs * num_heads * pkv::state_row_floats(head_dim));
}

int decode_impl(void* out, const void* q, int q_dtype, const void* k_cache, const void* v_cache, int cache_dtype,
                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                float scale, float k_scale, float v_scale, int32_t partition_size, const int32_t* prefix_leader,
                const int32_t* prefix_blocks, bool cascade, const int32_t* cu_q, int32_t num_q_rows, bool multi,
                void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0 || max_blocks_per_seq < 0)
        return PKV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
    if (!known_dtype(q_dtype) || !known_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
    if (partition_size < 0 || partition_size % pkv::kBlockTokens != 0) return PKV_ERR_INVALID_ARG;
    if (block_size != pkv::kBlockTokens || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
    const bool pair_ok = (q_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_F32) ||
                         (q_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_BF16) ||
                         (q_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_FP8_E4M3);
    if (!pair_ok) return PKV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype == PKV_DTYPE_FP8_E4M3;
    if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return PKV_ERR_INVALID_ARG;
    if (int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (int64_t(max_blocks_per_seq) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    const int rh = pkv::run_heads(num_heads / num_kv_heads);
    const int runs = num_heads / rh;
    // units (sequence, run, block) are counted in 32 bits; a prefix run adds at most one sequence's worth,
    // and with several queries every token group of a sequence reads at most its whole table row
    const int64_t groups = multi ? int64_t(num_q_rows) / prefix_members(rh) + num_seqs : num_seqs;
    if (multi && num_q_rows < 0) return PKV_ERR_INVALID_ARG;
    if (groups * runs * max_blocks_per_seq * (cascade ? 2 : 1) >= (int64_t(1) << 31)) return PKV_ERR_UNSUPPORTED;
    if (multi && int64_t(num_q_rows) * num_heads * head_dim >= (int64_t(1) << 31)) return PKV_ERR_UNSUPPORTED;
    const int64_t state_bytes = int64_t(num_seqs) * num_heads * pkv::state_row_floats(head_dim) * 4;
    if (cascade && state_bytes >= (int64_t(1) << 31))
        return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !context_lens || (!block_table && max_blocks_per_seq > 0))
        return PKV_ERR_INVALID_ARG;
    if (cascade && (!prefix_leader || !prefix_blocks)) return PKV_ERR_INVALID_ARG;
    if (multi && !cu_q) return PKV_ERR_INVALID_ARG;
    if (multi && num_q_rows == 0) return PKV_OK;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(context_lens, 4) || !aligned(block_table, 4) || !aligned(workspace, 16) ||
        !aligned(prefix_leader, 4) || !aligned(prefix_blocks, 4) || !aligned(cu_q, 4))
        return PKV_ERR_ALIGNMENT;

    if (noalloc) {
        // The plain decode with the library's static scratch as its workspace: the counters, then two
        // partial-state slots per wave the launch runs.  Sizes whose slots do not fit are refused here,
        // before anything is launched.
        const int64_t need = (pkv::kSlotBase + 2 * int64_t(pkv::decode_waves(cache_dtype, head_dim)) *
                                                   pkv::slot_floats(rh, head_dim)) * int64_t(sizeof(float));
        if (need > int64_t(pkv::kNoAllocScratchBytes)) return PKV_ERR_SCRATCH;
        float* ws = nullptr;
        if (pkv::noalloc_scratch(&ws, static_cast<hipStream_t>(stream)) != hipSuccess) return PKV_ERR_HIP;
        workspace = ws;
    } else {
        const size_t need =
            cascade ? paged_attention_cascade_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                              max_blocks_per_seq, block_size, partition_size)
            : multi ? paged_attention_varlen_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                             max_blocks_per_seq, block_size, partition_size)
                    : paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                      max_blocks_per_seq, block_size, partition_size);
        if (workspace == nullptr || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    }

    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.ws = static_cast<float*>(workspace);
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    a.group = num_heads / num_kv_heads;
    a.rh = rh;
    a.runs = runs;
    a.part_blocks = partition_size / pkv::kBlockTokens;
    const float log2e = 1.4426950408889634f;
    a.score_scale = scale * (fp8 ? k_scale : 1.0f) * log2e;
    a.v_scale = fp8 ? v_scale : 1.0f;
    if (cascade) {
        // a prefix run's columns hold `members` sequences' heads, so its slots are that wide
        const int members = prefix_members(rh);
        const int64_t base = pkv::workspace_floats(members * rh, head_dim);
        a.slot_floats = int32_t(pkv::slot_floats(members * rh, head_dim));
        a.prefix_leader = prefix_leader;
        a.prefix_blocks = prefix_blocks;
        a.members = members;
        a.pstate = a.ws + base;
        a.sstate = a.pstate + pkv::align_floats(int64_t(num_seqs) * num_heads * pkv::state_row_floats(head_dim));
        a.state_bytes = int32_t(state_bytes);
    } else if (multi) {
        // a run's columns hold `members` new tokens of one sequence times rh heads
        const int members = prefix_members(rh);
        a.slot_floats = int32_t(pkv::slot_floats(members * rh, head_dim));
        a.members = members;
        a.cu_q = cu_q;
        a.num_q_rows = num_q_rows;
    } else {
        a.slot_floats = int32_t(pkv::slot_floats(rh, head_dim));
    }
    const hipError_t e = pkv::launch_decode(cache_dtype, head_dim, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attention_decode(void* out,
                           const void* q, int q_dtype,
                           const void* k_cache, const void* v_cache, int cache_dtype,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           float scale, float k_scale, float v_scale,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream) {
    return decode_impl(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale, v_scale,
                       partition_size, nullptr, nullptr, false, nullptr, 0, false, workspace, workspace_bytes,
                       stream);
}

int paged_attention_decode_noalloc(void* out,
                                   const void* q, int q_dtype,
                                   const void* k_cache, const void* v_cache, int cache_dtype,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   float scale, float k_scale, float v_scale,
                                   int32_t partition_size,
                                   void* stream) {
    return decode_impl(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale, v_scale,
                       partition_size, nullptr, nullptr, false, nullptr, 0, false, nullptr, 0, stream, true);
}

size_t paged_attention_cascade_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                               int32_t partition_size) {
    if (paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                                        partition_size) == 0)
        return 0;
    const int rh = pkv::run_heads(num_heads / num_kv_heads);
    const int64_t f = pkv::workspace_floats(prefix_members(rh) * rh, head_dim) +
                      cascade_extra_floats(num_seqs, num_heads, head_dim);
    return size_t(f) * sizeof(float);
}

int paged_attention_decode_cascade(void* out,
                                   const void* q, int q_dtype,
                                   const void* k_cache, const void* v_cache, int cache_dtype,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens,
                                   const int32_t* prefix_leader, const int32_t* prefix_blocks,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   float scale, float k_scale, float v_scale,
                                   int32_t partition_size,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
    return decode_impl(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale, v_scale,
                       partition_size, prefix_leader, prefix_blocks, true, nullptr, 0, false, workspace,
                       workspace_bytes, stream);
}

size_t paged_attention_varlen_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t partition_size) {
    if (paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                                        partition_size) == 0)
        return 0;
    const int rh = pkv::run_heads(num_heads / num_kv_heads);
    return size_t(pkv::workspace_floats(prefix_members(rh) * rh, head_dim)) * sizeof(float);
}

int paged_attention_varlen(void* out,
                           const void* q, int q_dtype, const int32_t* cu_seqlens_q, int32_t num_q_rows,
                           const void* k_cache, const void* v_cache, int cache_dtype,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           float scale, float k_scale, float v_scale,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream) {
    return decode_impl(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_table, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale, v_scale,
                       partition_size, nullptr, nullptr, false, cu_seqlens_q, num_q_rows, true, workspace,
                       workspace_bytes, stream);
}

int paged_attention_prefill(void* out,
                            const void* q, int q_dtype, const int32_t* cu_seqlens_q, int32_t num_q_rows,
                            int32_t max_q_len,
                            const void* k_cache, const void* v_cache, int cache_dtype,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            float scale, float k_scale, float v_scale,
                            void* stream) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0 || max_blocks_per_seq < 0 || num_q_rows < 0 || max_q_len < 0)
        return PKV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
    if (!known_dtype(q_dtype) || !known_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
    if (block_size != pkv::kBlockTokens || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
    const bool pair_ok = (q_dtype == PKV_DTYPE_F32 && cache_dtype == PKV_DTYPE_F32) ||
                         (q_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_BF16) ||
                         (q_dtype == PKV_DTYPE_BF16 && cache_dtype == PKV_DTYPE_FP8_E4M3);
    if (!pair_ok) return PKV_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype == PKV_DTYPE_FP8_E4M3;
    if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return PKV_ERR_INVALID_ARG;
    if (int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (int64_t(max_blocks_per_seq) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    const int group = num_heads / num_kv_heads;
    if (group > pkv::kPrefillWaveCols) return PKV_ERR_UNSUPPORTED;  // a wave holds at least one token
    if (int64_t(num_q_rows) * num_heads * head_dim >= (int64_t(1) << 31)) return PKV_ERR_UNSUPPORTED;
    const int tpw = pkv::kPrefillWaveCols / group;
    const int64_t items = int64_t(num_seqs) * num_kv_heads * ((int64_t(max_q_len) + tpw - 1) / tpw);
    // the grid deals pairs (sequence, KV head) to the 8 XCDs in equal numbers
    if ((int64_t(num_seqs) * num_kv_heads + 7) / 8 * 8 * ((int64_t(max_q_len) + tpw - 1) / tpw) >= (int64_t(1) << 31))
        return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_q_rows == 0 || max_q_len == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !context_lens || !cu_seqlens_q || (!block_table && max_blocks_per_seq > 0))
        return PKV_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(context_lens, 4) || !aligned(block_table, 4) || !aligned(cu_seqlens_q, 4))
        return PKV_ERR_ALIGNMENT;
    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    a.group = group;
    const float log2e = 1.4426950408889634f;
    a.score_scale = scale * (fp8 ? k_scale : 1.0f) * log2e;
    a.v_scale = fp8 ? v_scale : 1.0f;
    a.cu_q = cu_seqlens_q;
    a.num_q_rows = num_q_rows;
    a.max_q = max_q_len;
    const hipError_t e =
        pkv::launch_prefill(cache_dtype, head_dim, a, int(items), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, int cache_dtype, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, const int32_t* src, const int32_t* dst, int32_t n,
                         void* stream) {
    if (n < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
    if (!known_dtype(cache_dtype)) return PKV_ERR_INVALID_ARG;
    if (block_size != pkv::kBlockTokens || (head_dim != 64 && head_dim != 128)) return PKV_ERR_UNSUPPORTED;
    if (int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (n == 0) return PKV_OK;
    if (!k_cache || !v_cache || !src || !dst) return PKV_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src, 4) || !aligned(dst, 4)) return PKV_ERR_ALIGNMENT;
    pkv::CopyArgs a;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.src = src;
    a.dst = dst;
    a.n = n;
    a.num_blocks = num_blocks;
    a.block_bytes = int64_t(num_kv_heads) * pkv::kBlockTokens * head_dim * pkv::dtype_bytes(cache_dtype);
    const hipError_t e = pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_check_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs,
                     const int32_t* slot_mapping, int32_t num_tokens,
                     int32_t num_blocks, int32_t* counts, void* stream) {
    if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return PKV_ERR_INVALID_ARG;
    if (!counts) return PKV_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_table))) return PKV_ERR_INVALID_ARG;
    if (num_tokens > 0 && !slot_mapping) return PKV_ERR_INVALID_ARG;
    if (int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (int64_t(max_blocks_per_seq) * pkv::kBlockTokens >= (int64_t(1) << 31)) return PKV_ERR_INVALID_ARG;
    if (!aligned(counts, 16) || !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(slot_mapping, 4))
        return PKV_ERR_ALIGNMENT;
    pkv::CheckArgs a;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.slot_mapping = slot_mapping;
    a.counts = counts;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_blocks = num_blocks;
    const hipError_t e = pkv::launch_check(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
