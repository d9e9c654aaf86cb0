// Paged-attention decode for gfx950 (CDNA4): an HBM-bandwidth-bound kernel
// whose two small contractions run on the matrix cores.
//
// What it computes (ipipp.com vLLM/PagedAttention article, section 二
// "PagedAttention分页原理深度剖析"): for every sequence s and query head h,
// softmax(scale * q . K^T) V over the context_lens[s] cached tokens, where the
// tokens of logical block j live in physical block block_table[s][j] (16
// tokens per block).  The kernel walks the logical blocks, resolves each one
// through the table and reads that block's K/V tile; the result is the same as
// attention over contiguous memory.  Work split over several waves is merged
// with the online-softmax rule (bytelighting wiki "vLLM", 参考来源 names online
// softmax): states (m, l, acc) combine as M = max m_i,
// out = sum 2^(m_i - M) acc_i / sum 2^(m_i - M) l_i.
//
// Work decomposition (balanced split, no idle workgroups).  A "run" is one
// sequence together with the rh query heads that share one KV head; it needs
// every block of that sequence's KV head once.  Units are (sequence, run,
// logical block) in that order; U is their total.  The launch is a persistent
// grid of one-wave workgroups sized to the chip, and the unit line is cut
// into nwv ranges of equal length (floor(v U / nwv) .. floor((v+1) U / nwv)),
// range v going to wave v mod grid.  So every wave streams the same number of
// KV tiles whatever the length mix, there is no tail of long sequences, and
// short sequences cost no empty workgroups.  A range covers whole runs in its
// middle (written out directly) and at most two partial runs at its ends,
// whose states go to the workspace; paged_fixup_kernel merges them.
//
// Per block a wave
//   1. loads the K tile (16-byte loads; the chunked K layout makes each load
//      instruction one contiguous KiB) and the V tile (dimension-major: each
//      lane reads 4 consecutive tokens of one dimension);
//   2. forms the scores of its 16 tokens for all rh heads with matrix-core
//      steps S^T = K Q^T (tokens on rows, heads on columns; unused head
//      columns hold zero queries);
//   3. updates the per-head running maximum (lanes of one column hold one
//      head, so the maximum needs two cross-row exchanges), rescales the
//      accumulators when it grew and exponentiates (base 2, scale folded in);
//   4. accumulates O^T += V^T P^T with matrix-core steps; the exponentiated
//      scores come out of step 2 already in the operand layout step 4 needs.
// Tiles are software-pipelined P blocks deep (loads of later blocks are in
// flight while a block is consumed).  bf16 pools use bf16 matrix steps with P
// rounded to bf16 (the normaliser sums the same rounded weights); fp8 pools are
// widened to bf16 exactly before the same steps; f32 pools use fp32 steps.
//
// Masking: tokens past the context length (and all tokens of a block whose id
// is outside the pool) get score -inf and their V entries are zeroed by a
// select, so poisoned memory never reaches an accumulator.  Padding table
// entries are never read.
#include <algorithm>
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KV, int D>
struct Geo {
    static constexpr int ELT = KV == kF32 ? 4 : (KV == kBF16 ? 2 : 1);
    static constexpr int TILE = kBlockTokens * D * ELT;  // bytes of one (block, KV head) tile
    static constexpr int NKL = TILE / (64 * 16);         // 16-byte K loads per lane per tile
    static constexpr int NVC = D / 16;                    // 16-dimension V chunks
    static constexpr int NQ = KV == kF32 ? 4 * NKL : (KV == kFP8 ? 2 * NKL : NKL);  // QK steps
};

template <int KV>
using VLoad = typename std::conditional<KV == kF32, uint4, typename std::conditional<KV == kBF16, uint2, uint32_t>::type>::type;
template <int KV>
using QOp = typename std::conditional<KV == kF32, float, bf16x8>::type;

template <int KV, int D>
struct Tile {
    uint4 k[Geo<KV, D>::NKL];
    VLoad<KV> v[Geo<KV, D>::NVC];
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// Two E4M3 codes (low or high half of a word) -> two bf16; exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t a, uint32_t b) {
    const uint4 r = make_uint4(fp8x2_to_bf16x2<false>(a), fp8x2_to_bf16x2<true>(a), fp8x2_to_bf16x2<false>(b),
                               fp8x2_to_bf16x2<true>(b));
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {  // inclusive prefix sum over the wave
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(x, off);
        if (lane >= off) x += t;
    }
    return x;
}

// Context length as the kernels use it: clamped into [0, max_blocks * 16].
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int s) {
    int L = a.context_lens[s];
    L = L < 0 ? 0 : L;
    L = L > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : L;
    return a.num_blocks <= 0 ? 0 : L;  // no pool: every block is out of range
}

__device__ __forceinline__ int* slot_ptr(const DecodeArgs& a, int v, int k) {
    return reinterpret_cast<int*>(a.ws + kWsHeader + (int64_t(v) * 2 + k) * a.slot_floats);
}

template <int QT, int D>
__device__ void zero_rows(const DecodeArgs& a, int s) {
    const int n = a.num_heads * D;
    if constexpr (QT == kF32) {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(a.out) + int64_t(s) * n);
        for (int i = lane_id(); i < n / 4; i += 64) o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        uint2* o = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + int64_t(s) * n);
        for (int i = lane_id(); i < n / 4; i += 64) o[i] = make_uint2(0u, 0u);
    }
}

// Forward cursor over the sequences, 64 at a time: lane i holds sequence
// base + i.  Units of a sequence = runs * blocks.
struct Cursor {
    int base;        // first sequence of the chunk
    int len;         // lane: clamped context length (0 past the batch)
    uint32_t inc;    // lane: inclusive prefix of units over the chunk
    uint32_t start;  // units before the chunk
    uint32_t tot;    // units in the chunk
};

__device__ __forceinline__ void cursor_load(Cursor& c, const DecodeArgs& a, int base) {
    const int s = base + lane_id();
    c.base = base;
    c.len = s < a.num_seqs ? clamped_len(a, s) : 0;
    c.inc = wave_scan(uint32_t((c.len + kBlockTokens - 1) / kBlockTokens) * uint32_t(a.runs));
    c.tot = __builtin_amdgcn_readlane(c.inc, 63);
}

__device__ __forceinline__ void cursor_advance(Cursor& c, const DecodeArgs& a) {
    c.start += c.tot;
    cursor_load(c, a, c.base + 64);
}

// Lane of the chunk holding the sequence that contains unit u (u < U).
__device__ __forceinline__ int cursor_find(Cursor& c, const DecodeArgs& a, uint32_t u) {
    while (c.start + c.tot <= u) cursor_advance(c, a);
    return __builtin_ctzll(__ballot(c.start + c.inc > u));
}

// Lane of the next non-empty sequence after lane i (one exists).
__device__ __forceinline__ int cursor_next(Cursor& c, const DecodeArgs& a, int i) {
    unsigned long long m = __ballot(lane_id() > i && c.len > 0);
    while (m == 0) {
        cursor_advance(c, a);
        m = __ballot(c.len > 0);
    }
    return __builtin_ctzll(m);
}

// One segment: blocks [j0, j1) of run (s, hg).  slot < 0: the segment is the
// whole run and the wave writes the output; otherwise the partial state goes
// to workspace slot `slot` (range v, end k) with its header.
template <int KV, int D, int P>
__device__ void run_segment(const DecodeArgs& a, int s, int L, int hg, int j0, int j1, int slot_v, int slot_k,
                            bool complete) {
    using GE = Geo<KV, D>;
    using T = Tile<KV, D>;
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    const int lane = lane_id();
    const int g = lane >> 4;    // row group of the matrix-core operands
    const int col = lane & 15;  // head column (QK output, PV output) / token row (K operand)
    const int head0 = hg * a.rh;
    const int kvh = head0 / a.group;
    const bool hv = col < a.rh;

    // ---- query operand: Q^T, heads on columns, zero for unused columns ----
    QOp<KV> qop[GE::NQ];
    {
        const int qelt = (QT == kF32) ? 4 : 2;
        const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                              (int64_t(s) * a.num_heads + head0 + (hv ? col : 0)) * D * qelt;
        if constexpr (KV == kBF16) {
#pragma unroll
            for (int u = 0; u < GE::NQ; ++u) {
                const uint4 x = hv ? *reinterpret_cast<const uint4*>(qrow + (32 * u + 8 * g) * 2) : make_uint4(0, 0, 0, 0);
                qop[u] = __builtin_bit_cast(bf16x8, x);
            }
        } else if constexpr (KV == kFP8) {
#pragma unroll
            for (int u = 0; u < GE::NKL; ++u)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4 x = hv ? *reinterpret_cast<const uint4*>(qrow + (64 * u + 16 * g + 8 * e) * 2)
                                       : make_uint4(0, 0, 0, 0);
                    qop[2 * u + e] = __builtin_bit_cast(bf16x8, x);
                }
        } else {
#pragma unroll
            for (int u = 0; u < GE::NKL; ++u) {
                const float4 x = hv ? *reinterpret_cast<const float4*>(qrow + (16 * u + 4 * g) * 4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                qop[4 * u + 0] = x.x;
                qop[4 * u + 1] = x.y;
                qop[4 * u + 2] = x.z;
                qop[4 * u + 3] = x.w;
            }
        }
    }

    const int32_t* bt_row = a.block_table + int64_t(s) * a.max_blocks;
    const int64_t block_stride = int64_t(a.num_kv_heads) * GE::TILE;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + int64_t(kvh) * GE::TILE + lane * 16;
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + int64_t(kvh) * GE::TILE +
                           (col * kBlockTokens + 4 * g) * GE::ELT;

    // block ids, 64 per vector register: idc covers [j0 + 64 cq, +64), idn the next 64
    auto load_ids = [&](int grp) -> int {
        const int j = j0 + grp * 64 + lane;
        return j < j1 ? bt_row[j] : -1;
    };
    int cq = 0;
    int idc = load_ids(0);
    int idn = load_ids(1);

    T buf[P];
    int nvb[P];  // valid tokens of the buffered block (0: the block contributes nothing)
    auto issue = [&](T& t, int& nv, int ji) {
        const int jj = ji - j0;
        if ((jj >> 6) != cq) {
            idc = idn;
            ++cq;
            idn = load_ids(cq + 1);
        }
        int id = __builtin_amdgcn_readlane(idc, jj & 63);
        const bool ok = id >= 0 && id < a.num_blocks;
        nv = ok ? min(kBlockTokens, L - ji * kBlockTokens) : 0;
        id = ok ? id : 0;
        const uint8_t* kt = kbase + int64_t(id) * block_stride;
        const uint8_t* vt = vbase + int64_t(id) * block_stride;
#pragma unroll
        for (int u = 0; u < GE::NKL; ++u) t.k[u] = *reinterpret_cast<const uint4*>(kt + u * 1024);
#pragma unroll
        for (int c = 0; c < GE::NVC; ++c)
            t.v[c] = *reinterpret_cast<const VLoad<KV>*>(vt + c * 16 * kBlockTokens * GE::ELT);
    };

    float m = kNegInf;  // running maximum of head `col` (base-2 units)
    float lsum = 0.0f;  // this lane's share of the running normaliser of head `col`
    f32x4 acc[GE::NVC];
#pragma unroll
    for (int c = 0; c < GE::NVC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](const T& t, int nv) {
        // 2. scores: sacc[r] = S^T[token 4g + r][head col]
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KV == kBF16) {
#pragma unroll
            for (int u = 0; u < GE::NKL; ++u)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[u]), qop[u], sacc, 0, 0, 0);
        } else if constexpr (KV == kFP8) {
#pragma unroll
            for (int u = 0; u < GE::NKL; ++u) {
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(t.k[u].x, t.k[u].y), qop[2 * u], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(t.k[u].z, t.k[u].w), qop[2 * u + 1], sacc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < GE::NKL; ++u) {
                sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].x), qop[4 * u + 0], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].y), qop[4 * u + 1], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].z), qop[4 * u + 2], sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].w), qop[4 * u + 3], sacc, 0, 0, 0);
            }
        }
        // 3. online softmax for head `col`
        const int cnt = min(max(nv - 4 * g, 0), 4);  // valid tokens among this lane's four
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = r < cnt ? sacc[r] * a.score_scale : kNegInf;
        float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m, bm);
        const bool live = mn != kNegInf;
        const float alpha = live ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
        m = mn;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = live ? __builtin_amdgcn_exp2f(sv[r] - mn) : 0.0f;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int c = 0; c < GE::NVC; ++c) acc[c] *= alpha;
        }
        // 4. O^T += V^T P^T
        if constexpr (KV == kF32) {
            lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
            for (int c = 0; c < GE::NVC; ++c) {
                const uint4 vv = t.v[c];
                const float v0 = cnt > 0 ? __uint_as_float(vv.x) : 0.0f;
                const float v1 = cnt > 1 ? __uint_as_float(vv.y) : 0.0f;
                const float v2 = cnt > 2 ? __uint_as_float(vv.z) : 0.0f;
                const float v3 = cnt > 3 ? __uint_as_float(vv.w) : 0.0f;
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v0, p[0], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v1, p[1], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v2, p[2], acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v3, p[3], acc[c], 0, 0, 0);
            }
        } else {
            const uint32_t p01 = pack_bf16(p[0], p[1]);
            const uint32_t p23 = pack_bf16(p[2], p[3]);
            // the normaliser sums the rounded weights the products use
            lsum = lsum * alpha + ((__uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xffff0000u)) +
                                   (__uint_as_float(p23 << 16) + __uint_as_float(p23 & 0xffff0000u)));
            const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
            // keep-masks for this lane's four tokens (16 bits per bf16 token)
            const uint32_t mlo = cnt >= 2 ? 0xffffffffu : (cnt == 1 ? 0x0000ffffu : 0u);
            const uint32_t mhi = cnt >= 4 ? 0xffffffffu : (cnt == 3 ? 0x0000ffffu : 0u);
#pragma unroll
            for (int c = 0; c < GE::NVC; ++c) {
                uint2 vv;
                if constexpr (KV == kBF16) {
                    vv = t.v[c];
                } else {
                    vv = make_uint2(fp8x2_to_bf16x2<false>(t.v[c]), fp8x2_to_bf16x2<true>(t.v[c]));
                }
                vv.x &= mlo;
                vv.y &= mhi;
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vv), pb, acc[c], 0, 0, 0);
            }
        }
    };

    // ---- software pipeline, P blocks deep ----
#pragma unroll
    for (int i = 0; i < P - 1; ++i) issue(buf[i], nvb[i], min(j0 + i, j1 - 1));
    for (int jb = j0; jb < j1; jb += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            issue(buf[(i + P - 1) % P], nvb[(i + P - 1) % P], min(jb + i + P - 1, j1 - 1));
            if (jb + i < j1) consume(buf[i], nvb[i]);
        }
    }

    // ---- segment result ----
    float lt = lsum + __shfl_xor(lsum, 16);
    lt += __shfl_xor(lt, 32);
    if (complete) {
        if (hv) {
            const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
            const int64_t o = (int64_t(s) * a.num_heads + head0 + col) * D + 4 * g;
#pragma unroll
            for (int c = 0; c < GE::NVC; ++c) {
                const f32x4 r = acc[c] * inv;
                if constexpr (QT == kF32) {
                    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o + 16 * c) = make_float4(r[0], r[1], r[2], r[3]);
                } else {
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o + 16 * c) =
                        make_uint2(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]));
                }
            }
        }
        if (slot_k == 0 && lane == 0) {  // the range's first segment was a whole run
            int* h = slot_ptr(a, slot_v, 0);
            h[0] = s; h[1] = hg; h[2] = j0; h[3] = j1; h[4] = kSlotComplete;
        }
    } else {
        int* h = slot_ptr(a, slot_v, slot_k);
        float* f = reinterpret_cast<float*>(h);
        if (lane == 0) {
            h[0] = s; h[1] = hg; h[2] = j0; h[3] = j1; h[4] = kSlotPartial;
        }
        if (hv) {
            if (g == 0) {
                f[8 + col] = m;
                f[8 + kMaxRunHeads + col] = lt;
            }
            float* ab = f + kSlotHead + col * D + 4 * g;
#pragma unroll
            for (int c = 0; c < GE::NVC; ++c)
                *reinterpret_cast<float4*>(ab + 16 * c) = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
        }
    }
}

// Range geometry, identical in every wave: the unit line [0, U) is cut into
// n equal ranges (range v = [floor(v U / n), floor((v+1) U / n))), one per
// persistent wave or, under a partition cap, as many as keep every range
// within part_blocks units; every range holds at least one unit.
struct Ranges {
    uint32_t U, n;
    __device__ uint32_t count() const { return n; }
    __device__ void bounds(uint32_t v, uint32_t& lo, uint32_t& hi) const {
        lo = uint32_t(uint64_t(v) * U / n);
        hi = uint32_t(uint64_t(v + 1) * U / n);
    }
};

__device__ __forceinline__ Ranges make_ranges(const DecodeArgs& a, uint32_t U, uint32_t nwt) {
    Ranges r;
    r.U = U;
    uint32_t n = nwt;
    if (a.part_blocks > 0) {
        const uint32_t need = (U + uint32_t(a.part_blocks) - 1) / uint32_t(a.part_blocks);
        n = need > n ? need : n;
    }
    n = n < uint32_t(a.nwv_cap) ? n : uint32_t(a.nwv_cap);
    r.n = n < U ? n : U;
    return r;
}

// Process one work range: its segments in unit order.
template <int KV, int D, int P>
__device__ void run_range(const DecodeArgs& a, Cursor& cur, const Ranges& rg, uint32_t v) {
    uint32_t lo, hi;
    rg.bounds(v, lo, hi);
    int i = cursor_find(cur, a, lo);
    int L = __builtin_amdgcn_readlane(cur.len, i);
    int nb = (L + kBlockTokens - 1) / kBlockTokens;
    const uint32_t first_unit = cur.start + __builtin_amdgcn_readlane(cur.inc, i) - uint32_t(nb * a.runs);
    const uint32_t rem = lo - first_unit;
    int hg = int(rem / uint32_t(nb));
    int j = int(rem % uint32_t(nb));
    uint32_t u = lo;
    int k = 0;
    while (true) {
        const int j1 = int(min(uint32_t(nb), uint32_t(j) + (hi - u)));
        const bool complete = (j == 0 && j1 == nb);
        run_segment<KV, D, P>(a, cur.base + i, L, hg, j, j1, int(v), k, complete);
        u += uint32_t(j1 - j);
        if (u >= hi) break;
        k = 1;
        j = 0;
        if (++hg == a.runs) {
            hg = 0;
            i = cursor_next(cur, a, i);
            L = __builtin_amdgcn_readlane(cur.len, i);
            nb = (L + kBlockTokens - 1) / kBlockTokens;
        }
    }
}

template <int KV, int D, int P>
__global__ __launch_bounds__(64) void paged_decode_kernel(DecodeArgs a) {
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    const int w = blockIdx.x;
    const int nwt = gridDim.x;

    // total units; rows of empty sequences are zeroed (sequence s by wave s mod grid)
    Cursor cur;
    cur.start = 0;
    uint32_t U = 0;
    for (int base = 0; base < a.num_seqs; base += 64) {
        cursor_load(cur, a, base);
        U += cur.tot;
        unsigned long long empty = __ballot(base + lane_id() < a.num_seqs && cur.len == 0);
        while (empty) {
            const int se = base + __builtin_ctzll(empty);
            empty &= empty - 1;
            if (se % nwt == w) zero_rows<QT, D>(a, se);
        }
    }
    const Ranges rg = make_ranges(a, U, uint32_t(nwt));
    if (w == 0 && lane_id() == 0) {
        int* h = reinterpret_cast<int*>(a.ws);
        h[0] = int(U);
        h[1] = int(rg.count());
    }
    if (U == 0) return;

    cur.start = 0;
    cursor_load(cur, a, 0);
    for (uint32_t v = uint32_t(w); v < rg.count(); v += uint32_t(nwt)) run_range<KV, D, P>(a, cur, rg, v);
}

// Merge the partial states of each run cut by a range boundary:
// M = max_i m_i, out = v_scale * sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i
// (taken online over the contributions, all heads of the run at once).
// Workgroup v - 1 handles the boundary at the first unit of range v when that
// unit is inside a run and no earlier boundary cuts the same run; the
// contributions are the previous range's last segment, then the first
// segments of ranges v, v+1, ... while they continue the run.  The headers of
// the next few ranges and then all contributions' states are requested
// together, so a merge costs two memory round trips (plus one per further
// batch of ranges for runs spread over many ranges).
constexpr int kFixBatch = 4;  // ranges examined per round trip

template <int QT, int D>
__global__ __launch_bounds__(64) void paged_fixup_kernel(DecodeArgs a) {
    constexpr int EPL = D / 64;  // dimensions per lane
    const int lane = lane_id();
    const int nwv = reinterpret_cast<const int*>(a.ws)[1];
    const int v = blockIdx.x + 1;
    if (v >= nwv) return;
    // headers: previous range (both slots) and ranges v .. v+kFixBatch-1 (slot 0)
    const int4 p0 = *reinterpret_cast<const int4*>(slot_ptr(a, v - 1, 0));
    const int pk0 = slot_ptr(a, v - 1, 0)[4];
    int4 hb[kFixBatch];
    int kb[kFixBatch];
#pragma unroll
    for (int i = 0; i < kFixBatch; ++i) {
        const int x = min(v + i, nwv - 1);
        hb[i] = *reinterpret_cast<const int4*>(slot_ptr(a, x, 0));
        kb[i] = slot_ptr(a, x, 0)[4];
    }
    const int s = hb[0].x, hg = hb[0].y;
    if (kb[0] != kSlotPartial || hb[0].z == 0) return;  // range v starts a run (or holds none cut)
    const bool prev_same = pk0 == kSlotPartial && p0.x == s && p0.y == hg;
    if (prev_same && p0.z > 0) return;  // an earlier boundary cuts this run

    float M[kMaxRunHeads], den[kMaxRunHeads], num[kMaxRunHeads][EPL];
#pragma unroll
    for (int h = 0; h < kMaxRunHeads; ++h) {
        M[h] = kNegInf;
        den[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[h][e] = 0.0f;
    }
    auto merge = [&](const float* f) {
        float mx[kMaxRunHeads], lx[kMaxRunHeads], ax[kMaxRunHeads][EPL];
#pragma unroll
        for (int h = 0; h < kMaxRunHeads; ++h) {
            if (h < a.rh) {
                mx[h] = f[8 + h];
                lx[h] = f[8 + kMaxRunHeads + h];
#pragma unroll
                for (int e = 0; e < EPL; ++e) ax[h][e] = f[kSlotHead + h * D + lane + 64 * e];
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxRunHeads; ++h) {
            if (h < a.rh && mx[h] != kNegInf) {
                const float Mn = fmaxf(M[h], mx[h]);
                const float so = __builtin_amdgcn_exp2f(M[h] - Mn);  // 0 while M is -inf
                const float sn = __builtin_amdgcn_exp2f(mx[h] - Mn);
                den[h] = den[h] * so + lx[h] * sn;
#pragma unroll
                for (int e = 0; e < EPL; ++e) num[h][e] = num[h][e] * so + ax[h][e] * sn;
                M[h] = Mn;
            }
        }
    };
    merge(reinterpret_cast<const float*>(slot_ptr(a, v - 1, prev_same ? 0 : 1)));
    // ranges v, v+1, ... whose first segment continues the run
    int x = v;
    while (true) {
        int n = 0;  // continuing ranges in this batch
#pragma unroll
        for (int i = 0; i < kFixBatch; ++i)
            if (n == i && x + i < nwv && kb[i] == kSlotPartial && hb[i].x == s && hb[i].y == hg) n = i + 1;
#pragma unroll
        for (int i = 0; i < kFixBatch; ++i)
            if (i < n) merge(reinterpret_cast<const float*>(slot_ptr(a, x + i, 0)));
        if (n < kFixBatch) break;
        x += kFixBatch;
#pragma unroll
        for (int i = 0; i < kFixBatch; ++i) {
            const int y = min(x + i, nwv - 1);
            hb[i] = *reinterpret_cast<const int4*>(slot_ptr(a, y, 0));
            kb[i] = slot_ptr(a, y, 0)[4];
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxRunHeads; ++h) {
        if (h < a.rh) {
            const int64_t o = (int64_t(s) * a.num_heads + hg * a.rh + h) * D + lane;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float r = den[h] > 0.0f ? (num[h][e] / den[h]) * a.v_scale : 0.0f;
                if constexpr (QT == kF32) {
                    static_cast<float*>(a.out)[o + 64 * e] = r;
                } else {
                    static_cast<uint16_t*>(a.out)[o + 64 * e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
                }
            }
        }
    }
}

// Pipeline depth per pool type: enough K/V tiles in flight per wave to cover
// HBM latency at the occupancy the register budget allows.
template <int KV, int D>
struct Depth {
    static constexpr int BYTES = Geo<KV, D>::TILE * 2;  // K + V bytes of one block
#ifdef PKV_DEPTH
    static constexpr int P = PKV_DEPTH;
#else
    static constexpr int P = BYTES >= 8192 ? 2 : 3;
#endif
};

int device_cus() {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cached = n;
        else
            return 256;
    }
    return cached;
}

template <int KV, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    constexpr int P = Depth<KV, D>::P;
    auto kern = paged_decode_kernel<KV, D, P>;
    static int waves_per_cu = 0;  // occupancy of this instance (64-thread workgroups)
    if (waves_per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64, 0) != hipSuccess || n <= 0) n = 8;
        waves_per_cu = n;
    }
#ifdef PKV_MAX_WAVES_PER_CU
    waves_per_cu = waves_per_cu < PKV_MAX_WAVES_PER_CU ? waves_per_cu : PKV_MAX_WAVES_PER_CU;
#endif
    int nwt = waves_per_cu * device_cus();
    nwt = nwt < kMaxWaves ? nwt : kMaxWaves;
    nwt = nwt < a.nwv_cap ? nwt : a.nwv_cap;
    hipLaunchKernelGGL(kern, dim3(nwt), dim3(64), 0, stream, a);
    // one fix-up workgroup per range boundary the decode may create
    int64_t ranges = nwt;
    if (a.part_blocks > 0) {
        const int64_t umax = int64_t(a.num_seqs) * a.runs * a.max_blocks;
        ranges = std::max<int64_t>(ranges, (umax + a.part_blocks - 1) / a.part_blocks);
    }
    ranges = std::min<int64_t>(ranges, a.nwv_cap);
    if (ranges > 1)
        hipLaunchKernelGGL((paged_fixup_kernel<QT, D>), dim3(unsigned(ranges - 1)), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int cache_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (cache_dtype == kF32 && head_dim == 64) return launch_t<kF32, 64>(a, stream);
    if (cache_dtype == kF32 && head_dim == 128) return launch_t<kF32, 128>(a, stream);
    if (cache_dtype == kBF16 && head_dim == 64) return launch_t<kBF16, 64>(a, stream);
    if (cache_dtype == kBF16 && head_dim == 128) return launch_t<kBF16, 128>(a, stream);
    if (cache_dtype == kFP8 && head_dim == 64) return launch_t<kFP8, 64>(a, stream);
    if (cache_dtype == kFP8 && head_dim == 128) return launch_t<kFP8, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
