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
// One workgroup per group of consecutive new tokens and one KV head.  K
// chunks are loaded along the token rows (coalesced) and stored as aligned
// 16-byte writes.  V rows go through LDS, transposed to the pool's
// dimension-major order, and tokens whose slots are consecutive inside a block
// (a sequence writing several tokens) are stored as 16-byte pieces of each
// dimension row; any other token's V elements are stored one by one.  The fp8
// variant quantises with a bit-exact round-to-nearest-even, saturating E4M3
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

// One 16-byte chunk of cache elements from X = 16 / CELT input elements at
// `src` (copied when the input is the cache dtype, else E4M3-quantised).
template <int IN, int CT>
__device__ __forceinline__ uint4 cache_chunk(const uint8_t* src, float scale) {
    if constexpr (IN == CT) {
        return *reinterpret_cast<const uint4*>(src);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t b = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) b |= e4m3_encode(load_elem<IN>(src, i * 4 + e) / scale) << (8 * e);
            w[i] = b;
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// A group of kGroup consecutive tokens of one KV head per workgroup.
//  1. The slots of the group, with CW - 1 tokens of context on each side
//     (CW = 16 / CELT tokens fill 16 bytes of a dimension row of the V tile),
//     requested together with the rows of step 2.
//  2. Every K chunk of the group's tokens is loaded (coalesced along the
//     token rows), converted and stored as one 16-byte write; the group's V
//     rows (and the next CW - 1 tokens') are converted and transposed into
//     LDS, dimension-major.
//  3. A token is *covered* when the CW tokens around it whose slots would
//     fill its aligned 16-byte piece of the dimension rows (slot % CW == 0 ..
//     CW - 1) really hold those consecutive slots -- the usual case when a
//     sequence writes several new tokens (prefill chunks, speculative tokens).
//     The first token of such a piece (its head) writes each dimension's
//     piece as one 16-byte store; the group holding the head writes it.
//  4. Tokens that are not covered store their elements one by one.
// Every element of a token with a valid slot is written exactly once, by
// step 2 (K), 3 or 4 (V).
#ifndef PKV_WRITE_GROUP
#define PKV_WRITE_GROUP 64
#endif
constexpr int kGroup = PKV_WRITE_GROUP;  // at most 64: step 3a runs in one wave

template <int IN, int CT, int D>
__global__ __launch_bounds__(256) void kv_write_kernel(const uint8_t* __restrict__ k_new,
                                                       const uint8_t* __restrict__ v_new,
                                                       uint8_t* __restrict__ k_cache,
                                                       uint8_t* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slots,
                                                       int num_tokens, int num_kv_heads, int num_slots,
                                                       float k_scale, float v_scale) {
    constexpr int IELT = IN == kF32 ? 4 : (IN == kBF16 ? 2 : 1);
    constexpr int CELT = CT == kF32 ? 4 : (CT == kBF16 ? 2 : 1);
    constexpr int X = 16 / CELT;        // cache elements per 16-byte chunk (= CW)
    constexpr int CW = X;
    constexpr int CH = D / X;           // K chunks per token row
    constexpr int HALO = CW - 1;
    constexpr int NSL = kGroup + 2 * HALO;  // slots: [t0 - HALO, t0 + kGroup + HALO)
    constexpr int NVT = kGroup + HALO;      // V tokens held: [t0, t0 + kGroup + HALO)
    constexpr int PITCH = NVT * CELT;       // bytes of one dimension row in LDS
    __shared__ int sl[NSL];
    __shared__ int heads[kGroup];
    __shared__ int nheads;
    __shared__ uint8_t kind[kGroup];  // 0: no slot, 1: element stores, 2: head of a piece, 3: inside a piece
    __shared__ __align__(16) uint8_t vt[D * PITCH];

    const int t0 = int(blockIdx.x) * kGroup;
    const int h = int(blockIdx.y);
    const int tid = int(threadIdx.x);
    // 1. the slots (-1: none, past the batch, or outside the pool) and 2. the
    // K/V chunks are all requested before anything waits on them, so the
    // slot reads and the row reads share one round trip
    static_assert(NSL <= 256, "one slot per thread");
    const int stok = t0 - HALO + tid;
    const int sraw = (tid < NSL && stok >= 0 && stok < num_tokens) ? slots[stok] : -1;
    constexpr int NIT = (NVT * CH + 255) / 256;  // chunk rows per thread
    const int nv = min(NVT, num_tokens - t0);
    uint4 kx[NIT], vx[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = tid + 256 * it;
        if (i < nv * CH) {
            const int tt = i / CH, c = i % CH;
            const int64_t row = int64_t(t0 + tt) * num_kv_heads + h;
            const int64_t src = (row * D + c * X) * IELT;
            if (tt < kGroup) kx[it] = cache_chunk<IN, CT>(k_new + src, k_scale);
            vx[it] = cache_chunk<IN, CT>(v_new + src, v_scale);
        }
    }
    if (tid < NSL) sl[tid] = (sraw >= 0 && sraw < num_slots) ? sraw : -1;
    __syncthreads();
    // 2. K chunks of the group's tokens stored; V chunks of the group's tokens and the halo after it into LDS
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = tid + 256 * it;
        if (i < nv * CH) {
            const int tt = i / CH, c = i % CH;
            const int s = sl[tt + HALO];
            if (tt < kGroup && s >= 0) store_chunk(k_cache + k_chunk_offset(s, h, c, num_kv_heads, CH), kx[it]);
            const uint32_t w[4] = {vx[it].x, vx[it].y, vx[it].z, vx[it].w};
#pragma unroll
            for (int e = 0; e < X; ++e) {
                uint8_t* dst = vt + (c * X + e) * PITCH + tt * CELT;
                if constexpr (CELT == 4) *reinterpret_cast<uint32_t*>(dst) = w[e];
                else if constexpr (CELT == 2) *reinterpret_cast<uint16_t*>(dst) = uint16_t(w[e / 2] >> (16 * (e % 2)));
                else *dst = uint8_t(w[e / 4] >> (8 * (e % 4)));
            }
        }
    }
    // 3a. what each token of the group does with its V elements; heads listed in token order
    if (tid < kGroup) {
        const int s = sl[tid + HALO];
        int k = 0;
        if (s >= 0) {
            const int e = s % CW;
            bool cov = true;
#pragma unroll
            for (int j = 0; j < CW; ++j) cov = cov && sl[tid - e + j + HALO] == s - e + j;
            k = cov ? (e == 0 ? 2 : 3) : 1;
        }
        kind[tid] = uint8_t(k);
        const unsigned long long m = __ballot(k == 2);  // kGroup <= 64: one wave
        if (k == 2) heads[__builtin_popcountll(m & ((1ull << tid) - 1))] = tid;
        if (tid == 0) nheads = __builtin_popcountll(m);
    }
    __syncthreads();
    // 3b. one 16-byte store per (head, dimension); consecutive threads take the
    // two heads of one block's rows, then the next dimension
    const int np = (nheads + 1) / 2;
    for (int i = tid; i < np * 2 * D; i += 256) {
        const int pr = i / (2 * D), r = i % (2 * D);
        const int d = r / 2, j = 2 * pr + (r & 1);
        if (j >= nheads) continue;
        const int tt = heads[j];
        const uint8_t* p = vt + d * PITCH + tt * CELT;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (CELT == 4) {
                w[q] = *reinterpret_cast<const uint32_t*>(p + 4 * q);
            } else if constexpr (CELT == 2) {
                w[q] = uint32_t(*reinterpret_cast<const uint16_t*>(p + 4 * q)) |
                       (uint32_t(*reinterpret_cast<const uint16_t*>(p + 4 * q + 2)) << 16);
            } else {
                w[q] = uint32_t(p[4 * q]) | (uint32_t(p[4 * q + 1]) << 8) | (uint32_t(p[4 * q + 2]) << 16) |
                       (uint32_t(p[4 * q + 3]) << 24);
            }
        }
        store_chunk(v_cache + v_elem_offset(sl[tt + HALO], h, d, num_kv_heads, D, CELT),
                    make_uint4(w[0], w[1], w[2], w[3]));
    }
    // 4. tokens not covered by a piece: one store per element
    const int ng = min(kGroup, num_tokens - t0);
    for (int i = tid; i < ng * D; i += 256) {
        const int tt = i / D, d = i % D;
        if (kind[tt] != 1) continue;
        const uint8_t* p = vt + d * PITCH + tt * CELT;
        uint8_t* dst = v_cache + v_elem_offset(sl[tt + HALO], h, d, num_kv_heads, D, CELT);
        if constexpr (CELT == 4) __builtin_nontemporal_store(*reinterpret_cast<const uint32_t*>(p), reinterpret_cast<uint32_t*>(dst));
        else if constexpr (CELT == 2) __builtin_nontemporal_store(*reinterpret_cast<const uint16_t*>(p), reinterpret_cast<uint16_t*>(dst));
        else __builtin_nontemporal_store(*p, dst);
    }
}

}  // namespace

hipError_t launch_kv_write(int in_dtype, int cache_dtype, int head_dim, const WriteArgs& a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const auto* kn = static_cast<const uint8_t*>(a.k_new);
    const auto* vn = static_cast<const uint8_t*>(a.v_new);
    auto* kc = static_cast<uint8_t*>(a.k_cache);
    auto* vc = static_cast<uint8_t*>(a.v_cache);
    const dim3 grid(unsigned((a.num_tokens + kGroup - 1) / kGroup), unsigned(a.num_kv_heads));
#define PKV_WRITE(IN, CT, D)                                                                                         \
    kv_write_kernel<IN, CT, D><<<grid, 256, 0, stream>>>(kn, vn, kc, vc, a.slot_mapping, a.num_tokens, a.num_kv_heads, \
                                                         a.num_slots, a.k_scale, a.v_scale)
    if (in_dtype == cache_dtype && cache_dtype == kF32 && head_dim == 64) PKV_WRITE(kF32, kF32, 64);
    else if (in_dtype == cache_dtype && cache_dtype == kF32 && head_dim == 128) PKV_WRITE(kF32, kF32, 128);
    else if (in_dtype == cache_dtype && cache_dtype == kBF16 && head_dim == 64) PKV_WRITE(kBF16, kBF16, 64);
    else if (in_dtype == cache_dtype && cache_dtype == kBF16 && head_dim == 128) PKV_WRITE(kBF16, kBF16, 128);
    else if (in_dtype == cache_dtype && cache_dtype == kFP8 && head_dim == 64) PKV_WRITE(kFP8, kFP8, 64);
    else if (in_dtype == cache_dtype && cache_dtype == kFP8 && head_dim == 128) PKV_WRITE(kFP8, kFP8, 128);
    else if (in_dtype == kF32 && cache_dtype == kFP8 && head_dim == 64) PKV_WRITE(kF32, kFP8, 64);
    else if (in_dtype == kF32 && cache_dtype == kFP8 && head_dim == 128) PKV_WRITE(kF32, kFP8, 128);
    else if (in_dtype == kBF16 && cache_dtype == kFP8 && head_dim == 64) PKV_WRITE(kBF16, kFP8, 64);
    else if (in_dtype == kBF16 && cache_dtype == kFP8 && head_dim == 128) PKV_WRITE(kBF16, kFP8, 128);
    else return hipErrorInvalidValue;
#undef PKV_WRITE
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
