// KV cache write through slot_mapping (gfx950).
//
// Source: bytelighting wiki "vLLM", 核心机制 / 工作原理, "Flattened 布局与
// slot_mapping" -- every new token's logical position is sent to a physical
// slot of the flattened block pool; ipipp.com vLLM article §二 -- blocks hold
// 16 tokens.  Slot sl is offset sl % 16 of physical block sl / 16.  Inside a
// (block, KV head) tile the K pool keeps each token row as 16-byte chunks of
// consecutive dimensions, chunk-major ([d / X][offset][d % X], X = 16 bytes of
// elements), and the V pool is dimension-major ([d][offset]) -- the layouts
// the decode kernel's matrix-core operands load directly.
//
// One thread per 16-byte K chunk of a (token, head) row: consecutive threads
// take consecutive chunks and then consecutive heads, so the reads of the new
// tokens are fully coalesced and every K store is one aligned 16-byte write.
// The same thread scatters the chunk's dimensions into the V tile (one element
// per dimension row).  The fp8 variant reads 16 input elements per thread and
// quantises them with a bit-exact round-to-nearest-even, saturating E4M3
// encoder.
#include <algorithm>

#include "pkv_internal.h"

namespace pkv {
namespace {

// OCP E4M3 encode of an fp32 value (already divided by the pool scale).
// Integer formulation: normal results keep the top three mantissa bits with
// round-to-nearest-even on the fp32 bit pattern; results below 2^-6 are the
// round-to-nearest-even integer value of |y| * 2^9 (codes 0..8).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;    // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;   // |y| >= 448 or inf: saturate
    const int e = int(a >> 23);                  // biased binary32 exponent
    if (e >= 121) {                              // |y| >= 2^-6: normal E4M3
        const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));         // rebias 127 -> 7
    }
    if (e < 117) return sign;                    // |y| < 2^-10: rounds to zero
    const uint32_t mant = (a & 0x7fffffu) | 0x800000u;
    const int sh = 141 - e;                      // |y| * 2^9 = mant * 2^-sh, sh in [21, 24]
    uint32_t q = mant >> sh;
    const uint32_t rem = mant & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    return sign | q;
}

template <int IN>
__device__ __forceinline__ float load_elem(const uint8_t* p, int i) {
    if constexpr (IN == kF32) {
        return reinterpret_cast<const float*>(p)[i];
    } else {
        const uint32_t b = reinterpret_cast<const uint16_t*>(p)[i];
        return __uint_as_float(b << 16);
    }
}

// Byte offset of the 16-byte K chunk `c` of (slot, head) and of V element
// (slot, head, dim) for a tile of CH chunks / D dims of ELT-byte elements.
__device__ __forceinline__ int64_t k_chunk_offset(int sl, int h, int c, int num_kv_heads, int CH) {
    return ((int64_t(sl >> 4) * num_kv_heads + h) * CH + c) * (kBlockTokens * 16) + (sl & 15) * 16;
}
__device__ __forceinline__ int64_t v_elem_offset(int sl, int h, int d, int num_kv_heads, int D, int ELT) {
    return ((int64_t(sl >> 4) * num_kv_heads + h) * D + d) * (kBlockTokens * ELT) + (sl & 15) * ELT;
}

// Cache stores are nontemporal.  A new token touches 16-byte pieces of many
// cache lines (each K chunk, and one element per dimension in the
// dimension-major V tile); ordinary stores leave all of them dirty in L2, and
// writing them back at the kernel boundary slowed the decode launched right
// after by about 12 us (bf16 GQA batch of 256).  Nontemporal stores do not
// keep them.
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_chunk(uint8_t* p, uint4 v) {
    __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}

// Copy (same dtype): one 16-byte chunk (X elements) per thread.  D = head_dim.
template <int ELT, int D>
__global__ __launch_bounds__(256) void kv_copy_kernel(const uint8_t* __restrict__ k_new,
                                                      const uint8_t* __restrict__ v_new,
                                                      uint8_t* __restrict__ k_cache,
                                                      uint8_t* __restrict__ v_cache,
                                                      const int32_t* __restrict__ slots,
                                                      int64_t total_chunks, int num_kv_heads, int num_slots) {
    constexpr int ROW = D * ELT;
    constexpr int CH = ROW / 16;
    constexpr int X = 16 / ELT;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= total_chunks) return;
    const int c = int(idx % CH);
    const int64_t th = idx / CH;                 // token * heads + head
    const int h = int(th % num_kv_heads);
    const int64_t tok = th / num_kv_heads;
    const int sl = slots[tok];
    if (sl < 0 || sl >= num_slots) return;
    const int64_t src = th * ROW + c * 16;
    const uint4 kx = *reinterpret_cast<const uint4*>(k_new + src);
    const uint4 vx = *reinterpret_cast<const uint4*>(v_new + src);
    store_chunk(k_cache + k_chunk_offset(sl, h, c, num_kv_heads, CH), kx);
    const uint32_t w[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
    for (int e = 0; e < X; ++e) {
        const int64_t dst = v_elem_offset(sl, h, c * X + e, num_kv_heads, D, ELT);
        if constexpr (ELT == 4) {
            __builtin_nontemporal_store(w[e], reinterpret_cast<uint32_t*>(v_cache + dst));
        } else if constexpr (ELT == 2) {
            __builtin_nontemporal_store(uint16_t(w[e / 2] >> (16 * (e % 2))), reinterpret_cast<uint16_t*>(v_cache + dst));
        } else {
            __builtin_nontemporal_store(uint8_t(w[e / 4] >> (8 * (e % 4))), v_cache + dst);
        }
    }
}

// Quantise: 16 output codes (one 16-byte K chunk) per thread.  D = head_dim.
template <int IN, int D>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint8_t* __restrict__ k_new,
                                                       const uint8_t* __restrict__ v_new,
                                                       uint8_t* __restrict__ k_cache,
                                                       uint8_t* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slots,
                                                       int64_t total_chunks, int num_kv_heads, int num_slots,
                                                       float k_scale, float v_scale) {
    constexpr int CH = D / 16;
    constexpr int IN_ELT = IN == kF32 ? 4 : 2;
    constexpr int IN_ROW = D * IN_ELT;
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= total_chunks) return;
    const int c = int(idx % CH);
    const int64_t th = idx / CH;
    const int h = int(th % num_kv_heads);
    const int64_t tok = th / num_kv_heads;
    const int sl = slots[tok];
    if (sl < 0 || sl >= num_slots) return;
    const uint8_t* ks = k_new + th * IN_ROW + c * 16 * IN_ELT;
    const uint8_t* vs = v_new + th * IN_ROW + c * 16 * IN_ELT;
    uint32_t kw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t kb = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) kb |= e4m3_encode(load_elem<IN>(ks, w * 4 + e) / k_scale) << (8 * e);
        kw[w] = kb;
    }
    store_chunk(k_cache + k_chunk_offset(sl, h, c, num_kv_heads, CH), make_uint4(kw[0], kw[1], kw[2], kw[3]));
#pragma unroll
    for (int e = 0; e < 16; ++e)
        __builtin_nontemporal_store(uint8_t(e4m3_encode(load_elem<IN>(vs, e) / v_scale)),
                                    v_cache + v_elem_offset(sl, h, c * 16 + e, num_kv_heads, D, 1));
}

inline unsigned grid_for(int64_t n) { return unsigned((n + 255) / 256); }

}  // namespace

hipError_t launch_kv_write(int in_dtype, int cache_dtype, int head_dim, const WriteArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const auto* kn = static_cast<const uint8_t*>(a.k_new);
    const auto* vn = static_cast<const uint8_t*>(a.v_new);
    auto* kc = static_cast<uint8_t*>(a.k_cache);
    auto* vc = static_cast<uint8_t*>(a.v_cache);
    const int64_t rows = int64_t(a.num_tokens) * a.num_kv_heads;
    if (in_dtype == cache_dtype) {
        const int64_t n = rows * (head_dim * dtype_bytes(cache_dtype) / 16);
        const unsigned g = grid_for(n);
#define PKV_COPY(ELT, D) kv_copy_kernel<ELT, D><<<g, 256, 0, stream>>>(kn, vn, kc, vc, a.slot_mapping, n, a.num_kv_heads, a.num_slots)
        if (cache_dtype == kF32 && head_dim == 64) PKV_COPY(4, 64);
        else if (cache_dtype == kF32 && head_dim == 128) PKV_COPY(4, 128);
        else if (cache_dtype == kBF16 && head_dim == 64) PKV_COPY(2, 64);
        else if (cache_dtype == kBF16 && head_dim == 128) PKV_COPY(2, 128);
        else if (cache_dtype == kFP8 && head_dim == 64) PKV_COPY(1, 64);
        else if (cache_dtype == kFP8 && head_dim == 128) PKV_COPY(1, 128);
        else return hipErrorInvalidValue;
#undef PKV_COPY
    } else {
        const int64_t n = rows * (head_dim / 16);
        const unsigned g = grid_for(n);
#define PKV_QUANT(IN, D) kv_quant_kernel<IN, D><<<g, 256, 0, stream>>>(kn, vn, kc, vc, a.slot_mapping, n, a.num_kv_heads, a.num_slots, a.k_scale, a.v_scale)
        if (in_dtype == kF32 && head_dim == 64) PKV_QUANT(kF32, 64);
        else if (in_dtype == kF32 && head_dim == 128) PKV_QUANT(kF32, 128);
        else if (in_dtype == kBF16 && head_dim == 64) PKV_QUANT(kBF16, 64);
        else if (in_dtype == kBF16 && head_dim == 128) PKV_QUANT(kBF16, 128);
        else return hipErrorInvalidValue;
#undef PKV_QUANT
    }
    return hipGetLastError();
}

namespace {

// Block copies of a copy-on-write: one grid row per (src, dst) pair; a block
// of one pool (all KV heads) is contiguous, so each pair is two plain copies
// of block_bytes, done in 16-byte chunks.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a, int pair0) {
    const int pair = pair0 + int(blockIdx.y);
    const int src = a.src[pair], dst = a.dst[pair];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
    const int64_t n16 = a.block_bytes / 16;
    const uint4* ks = static_cast<const uint4*>(a.k_cache) + int64_t(src) * n16;
    const uint4* vs = static_cast<const uint4*>(a.v_cache) + int64_t(src) * n16;
    uint4* kd = static_cast<uint4*>(a.k_cache) + int64_t(dst) * n16;
    uint4* vd = static_cast<uint4*>(a.v_cache) + int64_t(dst) * n16;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += int64_t(gridDim.x) * blockDim.x) {
        const uint4 k = ks[i];
        const uint4 v = vs[i];
        kd[i] = k;
        vd[i] = v;
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
    const int64_t n16 = a.block_bytes / 16;
    const unsigned gx = unsigned(std::min<int64_t>((n16 + 255) / 256, 16));
    for (int pair0 = 0; pair0 < a.n; pair0 += 65535) {
        const unsigned gy = unsigned(std::min(a.n - pair0, 65535));
        hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream, a, pair0);
    }
    return hipGetLastError();
}

}  // namespace pkv
