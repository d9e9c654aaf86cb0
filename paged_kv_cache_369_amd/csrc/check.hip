// Input check: counts the contents of the index arrays that the write and
// decode kernels treat as invalid.  The kernels stay memory-safe for any
// contents (an out-of-range table entry is an empty block, a length is
// clamped, an out-of-range slot is skipped); this launch tells a caller when
// that has happened.  What is valid follows the block-table lookup of the
// ipipp.com vLLM/PagedAttention article (section 二) and the slot_mapping of
// the bytelighting wiki "vLLM" (Flattened 布局与 slot_mapping).
#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckArgs a) {
    __shared__ int cnt[4];
    const int tid = threadIdx.x;
    if (tid < 4) cnt[tid] = 0;
    __syncthreads();
    int bad_len = 0, bad_entry = 0, bad_slot = 0, dup_slot = 0;
    // context lengths
    for (int s = tid; s < a.num_seqs; s += kCheckThreads) {
        const int L = a.context_lens[s];
        bad_len += (L < 0 || int64_t(L) > int64_t(a.max_blocks) * kBlockTokens) ? 1 : 0;
    }
    // the table entries the decode reads: j < ceil(L/16), L clamped as the decode clamps it
    const int64_t entries = int64_t(a.num_seqs) * a.max_blocks;
    for (int64_t k = tid; k < entries; k += kCheckThreads) {
        const int s = int(k / a.max_blocks), j = int(k % a.max_blocks);
        int L = a.context_lens[s];
        L = L < 0 ? 0 : L;
        L = L > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : L;
        if (a.num_blocks <= 0) L = 0;
        if (j < (L + kBlockTokens - 1) / kBlockTokens) {
            const int id = a.block_table[k];
            bad_entry += (id < 0 || id >= a.num_blocks) ? 1 : 0;
        }
    }
    // slots: -1 or in range; an in-range slot equal to an earlier one is a repeat
    const int64_t nslots = int64_t(a.num_blocks) * kBlockTokens;
    for (int i = tid; i < a.num_tokens; i += kCheckThreads) {
        const int sl = a.slot_mapping[i];
        bad_slot += (sl == -1 || (sl >= 0 && sl < nslots)) ? 0 : 1;
        if (sl >= 0) {
            for (int j = 0; j < i; ++j) {
                if (a.slot_mapping[j] == sl) {
                    ++dup_slot;
                    break;
                }
            }
        }
    }
    atomicAdd(&cnt[0], bad_len);
    atomicAdd(&cnt[1], bad_entry);
    atomicAdd(&cnt[2], bad_slot);
    atomicAdd(&cnt[3], dup_slot);
    __syncthreads();
    if (tid < 4) a.counts[tid] = cnt[tid];
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv

// ---- a plain streaming read (measurement aid) ----
//
// Reads a buffer once with 16-byte loads.  Each of 8192 workgroups (32 per
// compute unit) streams its own contiguous share, four loads in flight per
// thread, and folds the words into one value that is stored only if it
// matches a constant (so the loads are kept and almost nothing is written).
// Of the shapes timed (grid-stride or contiguous shares, 2048 to 8192
// workgroups, 4 to 16 loads in flight) this one read fastest.  Its rate is
// the same-GPU reference the decode's KV bandwidth is set beside.
namespace pkv {
namespace {

constexpr int kStreamBlocks = PKV_STREAM_SINK_WORDS;
constexpr int kStreamThreads = 256;
constexpr int kStreamInFlight = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                     uint32_t* sink) {
    uint32_t acc = 0;
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = int64_t(blockIdx.x) * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    int64_t i = b0 + threadIdx.x;
    for (; i + (kStreamInFlight - 1) * kStreamThreads < b1; i += kStreamInFlight * kStreamThreads) {
        uint4 v[kStreamInFlight];
#pragma unroll
        for (int k = 0; k < kStreamInFlight; ++k) v[k] = p[i + k * kStreamThreads];
#pragma unroll
        for (int k = 0; k < kStreamInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < b1; i += kStreamThreads) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return PKV_OK;
    if (!buf || !sink) return PKV_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return PKV_ERR_ALIGNMENT;
    hipLaunchKernelGGL(pkv::stream_read_kernel, dim3(pkv::kStreamBlocks), dim3(pkv::kStreamThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
