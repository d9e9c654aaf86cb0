// Internal declarations shared by the C ABI layer and the kernel files.
// Not installed; the public interface is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;  // tokens per physical block
constexpr int kMaxRunHeads = 16;  // query heads one wave serves (matrix-core tile width)
constexpr int kMaxWaves = 4096;   // persistent waves per launch (16 per CU on a 256-CU MI355X)


enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

inline int dtype_bytes(int dt) { return dt == kF32 ? 4 : dt == kBF16 ? 2 : dt == kFP8 ? 1 : 0; }

// Pool layouts (elements; X = 16 / element bytes):
//   K[block][kv_head][d / X][offset][d % X]   (16-byte chunks of a token row, chunk-major)
//   V[block][kv_head][d][offset]              (dimension-major)
inline int k_chunk_elems(int dt) { return 16 / dtype_bytes(dt); }

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

struct CopyArgs {
    void* k_cache;
    void* v_cache;
    const int32_t* src;
    const int32_t* dst;
    int32_t n;
    int32_t num_blocks;
    int64_t block_bytes;  // bytes of one block in one pool (all KV heads), a multiple of 16
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

// Query heads of one run: the largest divisor of the GQA group that is at
// most kMaxRunHeads.  A run is (sequence, group of run_heads query heads that
// share one KV head); each KV tile of the run is read once for all its heads.
inline int run_heads(int group) {
    for (int g = group < kMaxRunHeads ? group : kMaxRunHeads; g > 1; --g)
        if (group % g == 0) return g;
    return 1;
}

// Workspace (caller-owned, zero-filled before its first use; every call that
// completes leaves its counters at zero again):
//   kWsHeader reserved words;
//   kMergeLevels x kMaxWaves int32 arrival counters (one per merge group);
//   two partial-state slots per wave: slot 0 for the run the wave continues
//   from the wave before it, slot 1 for the run it hands on to the waves
//   after it.  Slot layout (floats): m[16], l[16], acc[columns][D].
// Every counter sits at the same place for every entry point and shape, so
// one zero-filled buffer serves any sequence of calls; slots and state rows
// hold data only and need no clearing.
constexpr int kWsHeader = 16;
constexpr int kMergeFanIn = 8;   // states one merge step combines
constexpr int kMergeLevels = 4;  // kMergeFanIn^kMergeLevels >= kMaxWaves
constexpr int kSlotHead = 2 * kMaxRunHeads;
constexpr int64_t kSlotBase = kWsHeader + int64_t(kMergeLevels) * kMaxWaves;
inline int64_t slot_floats(int columns, int head_dim) { return kSlotHead + int64_t(columns) * head_dim; }
inline int64_t workspace_floats(int columns, int head_dim) {
    return kSlotBase + 2 * int64_t(kMaxWaves) * slot_floats(columns, head_dim);
}

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* context_lens;
    float* ws;           // workspace (header, counters, partial-state slots)
    int32_t max_blocks;  // block_table row length
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t group;       // num_heads / num_kv_heads
    int32_t rh;          // query heads per run
    int32_t runs;        // runs per sequence = num_heads / rh
    int32_t part_blocks; // > 0: partitions of at most this many blocks, each with its own softmax state
    int32_t slot_floats; // floats per partial slot
    float score_scale;   // scale * k_scale * log2(e): scores are kept in base-2 units
    float v_scale;       // 1 for f32 / bf16 pools
    // shared-prefix decode only (null / 0 otherwise)
    const int32_t* prefix_leader;  // [num_seqs] first sequence of each sequence's sharing group
    const int32_t* prefix_blocks;  // [num_seqs] leading blocks shared with that group
    float* pstate;                 // [num_seqs * num_heads] state rows of the prefix part
    float* sstate;                 // [num_seqs * num_heads] state rows of the suffix part
    int32_t members;               // sequences (shared prefix) or new tokens (several queries) per run's columns
    int32_t state_bytes;           // bytes of pstate (and of sstate)
    // several new query tokens per sequence only (null / 0 otherwise)
    const int32_t* cu_q;           // [num_seqs + 1] first query row of each sequence
    int32_t num_q_rows;            // rows of q and out
    // tiled prefill only
    int32_t max_q;                 // new tokens of the longest sequence (tokens past it are not computed)
};

// What the decode kernel computes: one query token per sequence, the same
// with shared prefixes read once, or several new query tokens per sequence.
enum Mode : int { kModePlain = 0, kModeShared = 1, kModeMulti = 2 };

// Shared-prefix state rows, after the slots: two arrays (prefix, suffix), each
// sized num_seqs * num_heads rows of head_dim + 4 floats.  Each holds the first
// part of every row (row = sequence * num_heads + head) -- acc[head_dim] in f32
// for f32 queries, acc / l in bf16 for bf16 queries -- then the (m, l) float
// pair of every row; the rest is unused.
inline int64_t align_floats(int64_t n) { return (n + 63) / 64 * 64; }
inline int64_t state_row_floats(int head_dim) { return int64_t(head_dim) + 4; }

hipError_t launch_decode(int cache_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);

// Persistent waves a plain decode launch runs for this pool type and head_dim
// (its partial-state slots are 2 per wave).
int decode_waves(int cache_dtype, int head_dim);

// The no-allocation decode's static scratch: its size, and its device address
// on the current device (taken, and its counters cleared on `stream`, by the
// first call on each device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;  // PKV_NOALLOC_SCRATCH_BYTES
hipError_t noalloc_scratch(float** out, hipStream_t stream);

// Query columns of one prefill wave: floor(kPrefillWaveCols / G) new tokens
// times the G query heads of one KV head (G at most kPrefillWaveCols; columns
// past the last whole token stay empty).
#ifndef PKV_PREFILL_COLS
#define PKV_PREFILL_COLS 32
#endif
constexpr int kPrefillWaveCols = PKV_PREFILL_COLS;
// Tiled prefill over `items` = num_seqs * num_kv_heads * ceil(max_q / floor(kPrefillWaveCols / G)) waves.
hipError_t launch_prefill(int cache_dtype, int head_dim, const DecodeArgs& a, int items, hipStream_t stream);

struct CheckArgs {
    const int32_t* block_table;
    const int32_t* context_lens;
    const int32_t* slot_mapping;
    int32_t* counts;  // 4 int32, overwritten
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t num_tokens;
    int32_t num_blocks;
};

hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

}  // namespace pkv
