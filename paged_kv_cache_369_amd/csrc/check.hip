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
    int bad_len = 0, bad_entry = 0, bad_slot = 0;
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
    // slots: -1 or in range (repeats are counted by repeat_kernel, launched after this one)
    const int64_t nslots = int64_t(a.num_blocks) * kBlockTokens;
    for (int i = tid; i < a.num_tokens; i += kCheckThreads) {
        const int sl = a.slot_mapping[i];
        bad_slot += (sl == -1 || (sl >= 0 && sl < nslots)) ? 0 : 1;
    }
    atomicAdd(&cnt[0], bad_len);
    atomicAdd(&cnt[1], bad_entry);
    atomicAdd(&cnt[2], bad_slot);
    __syncthreads();
    if (tid < 4) a.counts[tid] = cnt[tid];  // counts[3] = 0 here; repeat_kernel adds to it
}

// Repeated slots.  The values >= 0 are split into `parts` classes by a hash;
// workgroup p reads every slot, inserts those of class p into an LDS hash
// table (linear probing, compare-and-swap), and counts an insertion that
// finds its value already there.  Each value with k occurrences thus adds
// k - 1, the number of entries that repeat an earlier one.  The host picks
// parts so that a class holds about kRepeatLoad distinct values, well under
// the table's kRepeatTable entries.  A value that finds the table full
// (possible only if the hash is defeated) is checked by a scan of the
// entries before it instead, which gives the same count: a value is then
// absent from the table for good, so all its occurrences take that path.
constexpr int kRepeatTable = 16384;  // LDS entries (64 KiB)
constexpr uint32_t kEmpty = 0xffffffffu;

__device__ __forceinline__ uint32_t mix32(uint32_t x, uint32_t seed) {  // murmur3 finaliser of x ^ seed
    x ^= seed;
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(kCheckThreads) void repeat_kernel(const int32_t* slots, int32_t n, uint32_t parts,
                                                               int32_t* counts) {
    __shared__ uint32_t tab[kRepeatTable];
    __shared__ int dup;
    const int tid = threadIdx.x;
    for (int k = tid; k < kRepeatTable; k += kCheckThreads) tab[k] = kEmpty;
    if (tid == 0) dup = 0;
    __syncthreads();
    int mine = 0;
    for (int i = tid; i < n; i += kCheckThreads) {
        const int sl = slots[i];
        if (sl < 0 || mix32(uint32_t(sl), 0x9e3779b9u) % parts != blockIdx.x) continue;
        const uint32_t v = uint32_t(sl);
        uint32_t b = mix32(v, 0x7f4a7c15u) & (kRepeatTable - 1);
        bool placed = false;
        for (int probe = 0; probe < kRepeatTable; ++probe, b = (b + 1) & (kRepeatTable - 1)) {
            const uint32_t old = atomicCAS(&tab[b], kEmpty, v);
            if (old == kEmpty || old == v) {
                mine += old == v ? 1 : 0;
                placed = true;
                break;
            }
        }
        if (!placed) {  // the table is full and does not hold v: an exact scan of the earlier entries
            for (int j = 0; j < i; ++j) {
                if (slots[j] == sl) {
                    ++mine;
                    break;
                }
            }
        }
    }
    atomicAdd(&dup, mine);
    __syncthreads();
    if (tid == 0 && dup > 0) atomicAdd(&counts[3], dup);
}

}  // namespace

constexpr int kRepeatLoad = 4096;  // distinct values per hash class the host aims for

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, stream, a);
    if (a.num_tokens > 0) {
        const uint32_t parts = uint32_t((int64_t(a.num_tokens) + kRepeatLoad - 1) / kRepeatLoad);
        hipLaunchKernelGGL(repeat_kernel, dim3(parts), dim3(kCheckThreads), 0, stream, a.slot_mapping, a.num_tokens,
                           parts, a.counts);
    }
    return hipGetLastError();
}

}  // namespace pkv

// ---- a plain streaming read (measurement aid) ----
//
// Reads a buffer once with 16-byte nontemporal loads (the streaming hint: on
// MI355X a once-read stream moves about 12 % more bytes per second with it
// than with ordinary loads).  Each of 8192 workgroups (32 per compute unit)
// streams its own contiguous share, four loads in flight per thread, and
// folds the words into one value that is stored only if it matches a
// constant (so the loads are kept and almost nothing is written).  Of the
// shapes timed (grid-stride or contiguous shares, 2048 to 8192 workgroups,
// 4 to 16 loads in flight) this one read fastest.  Its rate is the same-GPU
// reference the decode's KV bandwidth is set beside.
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
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    for (; i + (kStreamInFlight - 1) * kStreamThreads < b1; i += kStreamInFlight * kStreamThreads) {
        u32x4 v[kStreamInFlight];
#pragma unroll
        for (int k = 0; k < kStreamInFlight; ++k) v[k] = __builtin_nontemporal_load(q + i + k * kStreamThreads);
#pragma unroll
        for (int k = 0; k < kStreamInFlight; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < b1; i += kStreamThreads) {
        const u32x4 a = __builtin_nontemporal_load(q + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
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

// ---- a gathered-tile read (measurement aid) ----
//
// The decode's access pattern without its arithmetic: 2048 one-wave
// workgroups (two per SIMD, the decode's occupancy for bf16 and fp8 at
// head_dim 128) each read an equal share of a list of tile ids, K tile then V
// tile of each id from two pools, `depth` tiles in flight, nontemporal loads.
// K is read with 16-byte lane loads and V with 4-, 8- or 16-byte ones, so
// the rate of each V load width can be set beside the others.  Each wave
// folds what it read into one word, stored only if it matches a constant.
namespace pkv {
namespace {

constexpr int kTileReadWaves = 2048;

template <int VW>
struct TileWord;
template <>
struct TileWord<4> {
    typedef uint32_t T;
    __device__ static uint32_t fold(T x) { return x; }
};
template <>
struct TileWord<8> {
    typedef unsigned T __attribute__((ext_vector_type(2)));
    __device__ static uint32_t fold(T x) { return x[0] ^ x[1]; }
};
template <>
struct TileWord<16> {
    typedef unsigned T __attribute__((ext_vector_type(4)));
    __device__ static uint32_t fold(T x) { return x[0] ^ x[1] ^ x[2] ^ x[3]; }
};

template <int TILE, int VW, int P>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void tile_read_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, const int32_t* __restrict__ ids, int32_t n,
    int32_t num_tiles, uint32_t* sink) {
    constexpr int NK = TILE / 1024, NV = TILE / (64 * VW);
    typedef typename TileWord<16>::T K16;
    typedef typename TileWord<VW>::T VT;
    const int lane = threadIdx.x;
    const int64_t w = blockIdx.x, nw = gridDim.x;
    const int64_t lo = w * n / nw, hi = (w + 1) * n / nw;
    if (lo >= hi) return;
    K16 kb[P][NK];
    VT vb[P][NV];
    uint32_t acc = 0;
    auto issue = [&](int s, int64_t pos) {
        int id = ids[pos < hi ? pos : lo];
        id = id < 0 ? 0 : (id >= num_tiles ? num_tiles - 1 : id);  // any contents stay in the pools
        const uint8_t* kp = k + int64_t(id) * TILE + lane * 16;
        const uint8_t* vp = v + int64_t(id) * TILE + lane * VW;
#pragma unroll
        for (int u = 0; u < NK; ++u) kb[s][u] = __builtin_nontemporal_load(reinterpret_cast<const K16*>(kp + u * 1024));
#pragma unroll
        for (int u = 0; u < NV; ++u)
            vb[s][u] = __builtin_nontemporal_load(reinterpret_cast<const VT*>(vp + u * 64 * VW));
    };
#pragma unroll
    for (int s = 0; s < P - 1; ++s) issue(s, lo + s);
    for (int64_t t = lo; t < hi; t += P) {
#pragma unroll
        for (int s = 0; s < P; ++s) {
            if (t + s < hi) {
                issue((s + P - 1) % P, t + s + P - 1);
#pragma unroll
                for (int u = 0; u < NK; ++u) acc ^= TileWord<16>::fold(kb[s][u]);
#pragma unroll
                for (int u = 0; u < NV; ++u) acc ^= TileWord<VW>::fold(vb[s][u]);
            }
        }
    }
    if (acc == 0x9e3779b9u) sink[w] = acc;
}

template <int TILE, int VW, int P>
hipError_t tile_read_t(const void* k, const void* v, const int32_t* ids, int32_t n, int32_t num_tiles, uint32_t* sink,
                       hipStream_t stream) {
    hipLaunchKernelGGL((tile_read_kernel<TILE, VW, P>), dim3(kTileReadWaves), dim3(64), 0, stream,
                       static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), ids, n, num_tiles, sink);
    return hipGetLastError();
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_tile_read(const void* k, const void* v, const int32_t* ids, int32_t n, int32_t num_tiles,
                             int32_t tile_bytes, int32_t v_load_bytes, int32_t depth, uint32_t* sink, void* stream) {
    if (n < 0 || num_tiles < 0) return PKV_ERR_INVALID_ARG;
    if (n == 0) return PKV_OK;
    if (!k || !v || !ids || !sink || num_tiles == 0) return PKV_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(k) & 15) || (reinterpret_cast<uintptr_t>(v) & 15) ||
        (reinterpret_cast<uintptr_t>(ids) & 3) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return PKV_ERR_ALIGNMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipErrorInvalidValue;
    const int key = tile_bytes * 1000 + v_load_bytes * 10 + depth;
    switch (key) {
        case 2048 * 1000 + 40 + 3: e = pkv::tile_read_t<2048, 4, 3>(k, v, ids, n, num_tiles, sink, s); break;
        case 2048 * 1000 + 80 + 3: e = pkv::tile_read_t<2048, 8, 3>(k, v, ids, n, num_tiles, sink, s); break;
        case 2048 * 1000 + 160 + 3: e = pkv::tile_read_t<2048, 16, 3>(k, v, ids, n, num_tiles, sink, s); break;
        case 2048 * 1000 + 40 + 4: e = pkv::tile_read_t<2048, 4, 4>(k, v, ids, n, num_tiles, sink, s); break;
        case 2048 * 1000 + 160 + 4: e = pkv::tile_read_t<2048, 16, 4>(k, v, ids, n, num_tiles, sink, s); break;
        case 4096 * 1000 + 40 + 2: e = pkv::tile_read_t<4096, 4, 2>(k, v, ids, n, num_tiles, sink, s); break;
        case 4096 * 1000 + 80 + 2: e = pkv::tile_read_t<4096, 8, 2>(k, v, ids, n, num_tiles, sink, s); break;
        case 4096 * 1000 + 160 + 2: e = pkv::tile_read_t<4096, 16, 2>(k, v, ids, n, num_tiles, sink, s); break;
        default: return PKV_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
