// Internal declarations shared by the C ABI layer and the kernel files.
// Not installed; the public interface is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;       // tokens per physical block
constexpr int kDefaultPartition = 512; // tokens per split-K work unit

enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

inline int dtype_bytes(int dt) { return dt == kF32 ? 4 : dt == kBF16 ? 2 : dt == kFP8 ? 1 : 0; }

struct WriteArgs {
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int32_t* slot_mapping;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t num_slots;  // num_blocks * 16
    float k_scale;
    float v_scale;
};

hipError_t launch_kv_write(int in_dtype, int cache_dtype, int head_dim, const WriteArgs& a, hipStream_t stream);

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* context_lens;
    float* ws_acc;       // [B][H][max_parts][D]  (unused when max_parts == 1)
    float* ws_m;         // [B][H][max_parts]
    float* ws_l;         // [B][H][max_parts]
    int32_t max_blocks;  // block_table row length
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t part_blocks; // partition size in blocks
    int32_t max_parts;   // ceil(max_blocks / part_blocks): workspace slots per (seq, head)
    int32_t splits;      // workgroups per (seq, kv-head group), 1 <= splits <= max_parts
    float score_scale;   // scale * k_scale * log2(e): scores are kept in base-2 units
    float v_scale;       // 1 for f32 / bf16 pools
};

hipError_t launch_decode(int cache_dtype, int head_dim, int group, const DecodeArgs& a, hipStream_t stream);

}  // namespace pkv
