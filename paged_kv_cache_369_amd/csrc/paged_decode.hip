// Paged-attention decode for gfx950 (CDNA4): an HBM-bandwidth-bound VALU kernel.
//
// What it computes (ipipp.com vLLM/PagedAttention article, §二
// "PagedAttention分页原理深度剖析"): for every sequence s and query head h,
// softmax(scale * q . K^T) V over the context_lens[s] cached tokens, where the
// tokens of logical block j live in physical block block_table[s][j] (16
// tokens per block).  The kernel walks the logical blocks, resolves each one
// through the table and reads that block's K/V tile; the result is the same as
// attention over contiguous memory.  Long contexts are split into partitions
// whose partial softmax states are merged with the online-softmax rule
// (bytelighting wiki "vLLM", 参考来源 names online softmax).
//
// Work decomposition: one workgroup (4 wave64s) per (group of G query heads
// sharing one KV head, sequence s, split z).  All G heads are served from one
// read of each K/V tile, so every KV byte is fetched from HBM once.  The
// context is cut into partitions of part_blocks blocks; split z takes
// partitions z, z + splits, z + 2*splits, ... and carries one online-softmax
// state across them.  The head group is the fastest grid dimension, so the
// round-robin placement of workgroups over the eight XCDs gives every XCD the
// same share of KV heads (and the same share of the work); splits are the
// slowest dimension, so the workgroups of splits a short sequence does not
// need come last and exit at once.  Inside a partition the waves take
// logical blocks round-robin, in chunks of up to 8 blocks per wave.  Per
// chunk a wave
//   1. streams its K tiles through a software pipeline (the next tile's
//      16-byte loads are in flight while the current one is consumed; 4 lanes
//      per token, each holding a quarter of the row) and forms G scores per
//      token with packed bf16 dot products (v_dot2_f32_bf16) or fp32 FMAs,
//      reduced across the 4 lanes of a token with DPP quad permutes; one lane
//      per token parks the G scores in the wave's LDS slice;
//   2. updates its running per-head maxima, rescales its accumulators and
//      exponentiates the parked scores in place (one v_exp per weight);
//   3. streams its V tiles (row-contiguous loads, each lane owning a fixed
//      slice of head_dim) and accumulates weight * value in fp32.
// The block ids of a chunk are fetched with one vector load and read back
// with v_readlane, so the loads of a tile never wait on a table read.  The
// four waves' (max, sum, accumulator) states are merged through LDS; when a
// sequence needs a single split the workgroup writes the output directly,
// otherwise its state goes to the workspace and paged_reduce_kernel merges
// the splits.
//
// Scores are kept in base-2 units (scale * k_scale * log2 e folded into one
// factor).  Masking of the partial last block selects -inf scores and zero
// value rows (never multiplies garbage by zero); padding table entries are
// never read; out-of-range block ids are treated as empty blocks.
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int NW = 4;  // waves per workgroup
constexpr int CB = 8;  // blocks per wave per chunk
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int KV, int D>
struct Shape {
    static constexpr int ELT = KV == kF32 ? 4 : (KV == kBF16 ? 2 : 1);
    static constexpr int ROW = D * ELT;             // bytes per token row
    static constexpr int TILE = kBlockTokens * ROW; // bytes per (block, kv head) tile
    // K mapping: lane = 4 * token + c; lane holds bytes i*64 + c*16 .. +16 of its row
    static constexpr int NK = ROW / 64;             // 16-byte K loads per lane per tile
    static constexpr int EK = 16 / ELT;             // elements per 16-byte K load
    static constexpr int QW = EK / 2 > 4 ? EK / 2 : 4; // q words per K load (bf16 pairs or f32)
    // V mapping: lane reads VB contiguous bytes; consecutive lanes cover a row
    static constexpr int VB = (KV == kFP8) ? 8 : 16;
    static constexpr int LPR = ROW / VB;            // lanes per row
    static constexpr int RPI = 64 / LPR;            // rows per load instruction
    static constexpr int NV = kBlockTokens / RPI;   // V loads per lane per tile
    static constexpr int EV = VB / ELT;             // elements per V load
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// fp8 (E4M3, two codes in the low or high half of a word) -> bf16 pair; exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// DPP quad permutes: xor 1 = [1,0,3,2], xor 2 = [2,3,0,1]
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float bf16_word_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_word_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // v_cvt_pk_bf16_f32: nearest even
}

template <int QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
    if constexpr (QT == kF32) {
        static_cast<float*>(out)[idx] = v;
    } else {
        static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
    }
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Context length as the kernels use it: clamped into [0, max_blocks * 16].
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int s) {
    int L = a.context_lens[s];
    L = L < 0 ? 0 : L;
    L = L > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : L;
    return a.num_blocks <= 0 ? 0 : L;  // no pool: every block is out of range
}

template <int KV, int D, int G>
struct Lds {
    static constexpr int SCORES = CB * kBlockTokens * G;  // scores / weights of one chunk
    static constexpr int MERGE = 2 * G + G * D;          // m, l, acc of one wave
    static constexpr int REGION = SCORES > MERGE ? SCORES : MERGE;
};

template <int KV, int D, int G>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(DecodeArgs a) {
    using S = Shape<KV, D>;
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    using VT = typename std::conditional<S::VB == 16, uint4, uint2>::type;
    __shared__ float lds[NW][Lds<KV, D, G>::REGION];

    const int hg = blockIdx.x;
    const int s = blockIdx.y;
    const int z = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int head0 = hg * G;
    const int group = a.num_heads / a.num_kv_heads;
    const int kvh = head0 / group;

    const int L = clamped_len(a, s);
    const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

    if (L == 0) {  // empty context: the output row is zero
        if (z == 0) {
            for (int i = threadIdx.x; i < G * D; i += NW * 64)
                store_out<QT>(a.out, (int64_t(s) * a.num_heads + head0) * D + i, 0.0f);
        }
        return;
    }
    if (z >= nparts) return;

    const int32_t* bt_row = a.block_table + int64_t(s) * a.max_blocks;
    const int64_t block_stride = int64_t(a.num_kv_heads) * S::TILE;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + int64_t(kvh) * S::TILE;
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + int64_t(kvh) * S::TILE;

    // ---- query registers (K mapping: lane = 4 * token + kc) ----
    const int kt = lane >> 2;
    const int kc = lane & 3;
    uint32_t qreg[G][S::NK][S::QW];
    {
        const int qelt = (QT == kF32) ? 4 : 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + ((int64_t(s) * a.num_heads + head0 + h) * D) * qelt;
#pragma unroll
            for (int i = 0; i < S::NK; ++i) {
                const int dim0 = (i * 64 + kc * 16) / S::ELT;
#pragma unroll
                for (int w = 0; w < S::QW; w += 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(qrow + (int64_t(dim0) * qelt) + w * 4);
                    qreg[h][i][w + 0] = v.x;
                    qreg[h][i][w + 1] = v.y;
                    qreg[h][i][w + 2] = v.z;
                    qreg[h][i][w + 3] = v.w;
                }
            }
        }
    }

    // ---- per-wave running softmax state ----
    // m_run: per head, wave-uniform.  l_lane: partial sum of the weights this
    // lane exponentiated (always head lane % G).  acc: this lane's V slice.
    float m_run[G];
    float l_lane = 0.0f;
    float acc[S::EV][G];
#pragma unroll
    for (int h = 0; h < G; ++h) m_run[h] = kNegInf;
#pragma unroll
    for (int e = 0; e < S::EV; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[e][h] = 0.0f;

    float* my_lds = lds[wave];
    const int hl = lane % G;                        // head of the weights this lane exponentiates
    const int vrow = lane / S::LPR;                 // V mapping row within a load
    const int vcol = (lane % S::LPR) * S::VB;       // byte offset within the row

    for (int p = z; p < nparts; p += a.splits) {
    const int b0 = p * a.part_blocks;
    const int b1 = min(nblk, b0 + a.part_blocks);
    for (int c0 = b0; c0 < b1; c0 += NW * CB) {
        // blocks of this wave in this chunk: j = first + b * NW, b < nb
        const int first = c0 + wave;
        const int nb = first < b1 ? min(CB, (b1 - first + NW - 1) / NW) : 0;
        if (nb == 0) continue;
        // one table read per chunk: lane b holds the physical id of block b
        int idl = bt_row[first + min(lane, nb - 1) * NW];
        idl = (idl >= 0 && idl < a.num_blocks) ? idl : -1;
        auto block_id = [&](int b) { return __builtin_amdgcn_readlane(idl, b); };
        auto nvalid = [&](int b, int id) {
            return id < 0 ? 0 : min(kBlockTokens, L - (first + b * NW) * kBlockTokens);
        };
        auto k_ptr = [&](int b) {
            const int id = block_id(b);
            return kbase + int64_t(id < 0 ? 0 : id) * block_stride + kt * S::ROW + kc * 16;
        };
        auto v_ptr = [&](int b) {
            const int id = block_id(b);
            return vbase + int64_t(id < 0 ? 0 : id) * block_stride + vrow * S::ROW + vcol;
        };
        auto load_k = [&](uint4* dst, const uint8_t* ptr) {
#pragma unroll
            for (int i = 0; i < S::NK; ++i) dst[i] = *reinterpret_cast<const uint4*>(ptr + i * 64);
        };
        auto load_v = [&](VT* dst, const uint8_t* ptr) {
#pragma unroll
            for (int i = 0; i < S::NV; ++i) dst[i] = *reinterpret_cast<const VT*>(ptr + i * S::RPI * S::ROW);
        };

        // ---- phase 1: K tiles -> scores (LDS) and running maxima ----
        float cmax[G];
#pragma unroll
        for (int h = 0; h < G; ++h) cmax[h] = kNegInf;
        auto score_block = [&](const uint4* kr, int b) {
            const int nv = nvalid(b, block_id(b));
            float dot[G];
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] = 0.0f;
#pragma unroll
            for (int i = 0; i < S::NK; ++i) {
                const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if constexpr (KV == kBF16) {
#pragma unroll
                        for (int h = 0; h < G; ++h) dot[h] = dot2_bf16(qreg[h][i][w], kw[w], dot[h]);
                    } else if constexpr (KV == kFP8) {
                        const uint32_t lo = fp8x2_to_bf16x2<false>(kw[w]);
                        const uint32_t hi = fp8x2_to_bf16x2<true>(kw[w]);
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            dot[h] = dot2_bf16(qreg[h][i][2 * w], lo, dot[h]);
                            dot[h] = dot2_bf16(qreg[h][i][2 * w + 1], hi, dot[h]);
                        }
                    } else {
                        const float kf = __uint_as_float(kw[w]);
#pragma unroll
                        for (int h = 0; h < G; ++h) dot[h] = fmaf(__uint_as_float(qreg[h][i][w]), kf, dot[h]);
                    }
                }
            }
            const bool valid = kt < nv;
            float sv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = quad_sum(dot[h]) * a.score_scale;
                asm volatile("" : "+v"(d));  // keep the dot products unconditional (no exec-masked branch)
                sv[h] = valid ? d : kNegInf;
                cmax[h] = fmaxf(cmax[h], sv[h]);
            }
            if (kc == 0) {  // one lane per token parks the token's G scores
                float* dst = my_lds + (b * kBlockTokens + kt) * G;
#pragma unroll
                for (int h = 0; h < G; ++h) dst[h] = sv[h];
            }
        };
        // Two tile buffers used in turn (no register copies, so the loads of the
        // next tile stay in flight while the current one is consumed).  Loads
        // always target a valid tile: past the wave's last block they repeat it.
        uint4 ka[S::NK], kb[S::NK];
        load_k(ka, k_ptr(0));
        int b = 0;
        for (; b + 2 <= nb; b += 2) {
            load_k(kb, k_ptr(b + 1));
            score_block(ka, b);
            load_k(ka, k_ptr(min(b + 2, nb - 1)));
            score_block(kb, b + 1);
        }
        VT va[S::NV], vb[S::NV];
        load_v(va, v_ptr(0));  // the first V tile streams in while the maxima are formed
        if (b < nb) score_block(ka, b);

        // ---- phase 2: chunk maxima, rescale, exponentiate in place ----
        float alpha_hl = 1.0f, m_hl = 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = cmax[h];
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float m_new = fmaxf(m_run[h], mx);
            const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
            m_run[h] = m_new;
            if (alpha != 1.0f) {
#pragma unroll
                for (int e = 0; e < S::EV; ++e) acc[e][h] *= alpha;
            }
            alpha_hl = (hl == h) ? alpha : alpha_hl;
            m_hl = (hl == h) ? m_new : m_hl;
        }
        l_lane *= alpha_hl;
        wave_lds_sync();
        for (int idx = lane; idx < nb * kBlockTokens * G; idx += 64) {
            const float sv = my_lds[idx];
            const float pw = (sv == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv - m_hl);
            my_lds[idx] = pw;
            l_lane += pw;
        }
        wave_lds_sync();

        // ---- phase 3: V tiles -> accumulators ----
        auto accum_block = [&](const VT* vr, int b) {
            const int nv = nvalid(b, block_id(b));
#pragma unroll
            for (int i = 0; i < S::NV; ++i) {
                const int r = i * S::RPI + vrow;
                const bool rv = r < nv;
                const float* pp = my_lds + (b * kBlockTokens + r) * G;
                float pw[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pw[h] = rv ? pp[h] : 0.0f;
                float vf[S::EV];
                if constexpr (KV == kBF16) {
                    const uint32_t w4[4] = {rv ? vr[i].x : 0u, rv ? vr[i].y : 0u, rv ? vr[i].z : 0u,
                                            rv ? vr[i].w : 0u};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        vf[2 * w] = bf16_word_lo(w4[w]);
                        vf[2 * w + 1] = bf16_word_hi(w4[w]);
                    }
                } else if constexpr (KV == kFP8) {
                    const uint32_t w2[2] = {rv ? vr[i].x : 0u, rv ? vr[i].y : 0u};
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        const f32x2 lo = fp8x2_to_f32x2<false>(w2[w]);
                        const f32x2 hi = fp8x2_to_f32x2<true>(w2[w]);
                        vf[4 * w + 0] = lo.x;
                        vf[4 * w + 1] = lo.y;
                        vf[4 * w + 2] = hi.x;
                        vf[4 * w + 3] = hi.y;
                    }
                } else {
                    const uint32_t w4[4] = {rv ? vr[i].x : 0u, rv ? vr[i].y : 0u, rv ? vr[i].z : 0u,
                                            rv ? vr[i].w : 0u};
#pragma unroll
                    for (int w = 0; w < 4; ++w) vf[w] = __uint_as_float(w4[w]);
                }
#pragma unroll
                for (int e = 0; e < S::EV; ++e)
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[e][h] = fmaf(pw[h], vf[e], acc[e][h]);
            }
        };
        for (b = 0; b + 2 <= nb; b += 2) {
            load_v(vb, v_ptr(b + 1));
            accum_block(va, b);
            load_v(va, v_ptr(min(b + 2, nb - 1)));
            accum_block(vb, b + 1);
        }
        if (b < nb) accum_block(va, b);
        wave_lds_sync();
    }
    }

    // ---- wave-level reductions ----
#pragma unroll
    for (int off = G; off < 64; off <<= 1) l_lane += __shfl_xor(l_lane, off);
#pragma unroll
    for (int e = 0; e < S::EV; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int off = S::LPR; off < 64; off <<= 1) acc[e][h] += __shfl_xor(acc[e][h], off);

    // wave state -> LDS: [m[G] | l[G] | acc[G][D]]
    {
        float* st = my_lds;
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) st[h] = m_run[h];
        }
        if (lane < G) st[G + lane] = l_lane;
        if (lane < S::LPR) {
            const int d0 = lane * S::EV;
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < S::EV; ++e) st[2 * G + h * D + d0 + e] = acc[e][h];
        }
    }
    __syncthreads();

    // ---- merge the waves and emit ----
    const bool single = (nparts == 1 || a.splits == 1);
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int h = idx / D;
        const int d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, lds[w][h]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = lds[w][h];
            if (mw != kNegInf) {
                const float f = __builtin_amdgcn_exp2f(mw - M);
                num = fmaf(f, lds[w][2 * G + h * D + d], num);
                den = fmaf(f, lds[w][G + h], den);
            }
        }
        const int head = head0 + h;
        if (single) {
            store_out<QT>(a.out, (int64_t(s) * a.num_heads + head) * D + d, (num / den) * a.v_scale);
        } else {
            const int64_t slot = (int64_t(s) * a.num_heads + head) * a.max_parts + z;
            a.ws_acc[slot * D + d] = num;
            if (d == 0) {
                a.ws_m[slot] = M;
                a.ws_l[slot] = den;
            }
        }
    }
}

// Merge the splits of each (sequence, head): M = max m_p,
// out = v_scale * sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// One wave per (head, sequence); split weights go through LDS.  Grid x walks
// the heads in the order (head % G, head / G) so that, like the decode grid,
// consecutive workgroups (and hence XCDs) follow the KV-head group, and the
// partial states are read on the XCD that wrote them.
template <int QT, int D>
__global__ __launch_bounds__(64) void paged_reduce_kernel(DecodeArgs a, int G) {
    constexpr int MAXP = 256;   // splits merged per pass
    constexpr int DPL = D / 64; // dims per lane
    __shared__ float wgt[MAXP];
    const int ngroups = a.num_heads / G;
    const int head = (blockIdx.x % ngroups) * G + blockIdx.x / ngroups;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = clamped_len(a, s);
    const int nblk = (L + kBlockTokens - 1) / kBlockTokens;
    const int nparts = min((nblk + a.part_blocks - 1) / a.part_blocks, a.splits);
    if (nparts <= 1) return;
    const int64_t base = (int64_t(s) * a.num_heads + head) * a.max_parts;
    float M = kNegInf;
    for (int pp = lane; pp < nparts; pp += 64) M = fmaxf(M, a.ws_m[base + pp]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    float den = 0.0f;
    float num[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] = 0.0f;
    for (int p0 = 0; p0 < nparts; p0 += MAXP) {
        const int pn = min(MAXP, nparts - p0);
        for (int pp = lane; pp < pn; pp += 64) {
            const float mp = a.ws_m[base + p0 + pp];
            const float f = (mp == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
            wgt[pp] = f;
            den = fmaf(f, a.ws_l[base + p0 + pp], den);
        }
        __syncthreads();
        for (int pp = 0; pp < pn; ++pp) {
            const float f = wgt[pp];
            const float* src = a.ws_acc + (base + p0 + pp) * D;
#pragma unroll
            for (int k = 0; k < DPL; ++k) num[k] = fmaf(f, src[lane + 64 * k], num[k]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off);
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        store_out<QT>(a.out, (int64_t(s) * a.num_heads + head) * D + lane + 64 * k, (num[k] / den) * a.v_scale);
}

template <int KV, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    dim3 grid(a.num_heads / G, a.num_seqs, a.splits);
    paged_decode_kernel<KV, D, G><<<grid, NW * 64, 0, stream>>>(a);
    if (a.splits > 1) {
        dim3 rgrid(a.num_heads, a.num_seqs);
        paged_reduce_kernel<QT, D><<<rgrid, 64, 0, stream>>>(a, G);
    }
    return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_g(int g, const DecodeArgs& a, hipStream_t stream) {
    switch (g) {
    case 1: return launch_t<KV, D, 1>(a, stream);
    case 2: return launch_t<KV, D, 2>(a, stream);
    case 4: return launch_t<KV, D, 4>(a, stream);
    case 8: return launch_t<KV, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides the GQA
// group (f32 pools with head_dim 128 stop at 4 to bound register use).
static int heads_per_workgroup(int cache_dtype, int head_dim, int group) {
    const int cap = (cache_dtype == kF32 && head_dim == 128) ? 4 : 8;
    for (int g = cap; g > 1; g >>= 1)
        if (group % g == 0) return g;
    return 1;
}

// Splits per (sequence, head group): enough workgroups to fill the chip
// several times over (about 8192), at least 4 so that one long sequence
// cannot hold the whole launch, and never more than the partitions a row of
// the block table can hold.
static int splits_for(int num_seqs, int num_groups, int max_parts) {
    const int64_t pairs = int64_t(num_seqs) * num_groups;
    int64_t z = (8192 + pairs - 1) / pairs;
    z = z < 4 ? 4 : z;
    return int(z < max_parts ? z : max_parts);
}

hipError_t launch_decode(int cache_dtype, int head_dim, int group, const DecodeArgs& args, hipStream_t stream) {
    if (args.num_seqs == 0) return hipSuccess;
    const int g = heads_per_workgroup(cache_dtype, head_dim, group);
    DecodeArgs a = args;
    if (a.splits <= 0) a.splits = splits_for(a.num_seqs, a.num_heads / g, a.max_parts);
    if (cache_dtype == kF32 && head_dim == 64) return launch_g<kF32, 64>(g, a, stream);
    if (cache_dtype == kF32 && head_dim == 128) return launch_g<kF32, 128>(g, a, stream);
    if (cache_dtype == kBF16 && head_dim == 64) return launch_g<kBF16, 64>(g, a, stream);
    if (cache_dtype == kBF16 && head_dim == 128) return launch_g<kBF16, 128>(g, a, stream);
    if (cache_dtype == kFP8 && head_dim == 64) return launch_g<kFP8, 64>(g, a, stream);
    if (cache_dtype == kFP8 && head_dim == 128) return launch_g<kFP8, 128>(g, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
