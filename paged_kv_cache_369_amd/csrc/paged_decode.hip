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
// grid of one-wave workgroups sized to the chip, and wave w takes the
// contiguous stretch [floor(w U / nw), floor((w+1) U / nw)) of the unit line.
// So every wave streams the same number of KV tiles whatever the length mix,
// there is no tail of long sequences, and short sequences cost no empty
// workgroups.  With a partition size, the stretch is further cut into equal
// partitions of at most that many blocks; each partition of a run gets its
// own softmax state and the states are merged in order.
//
// Split-K reduction without a second launch.  A run that crosses a stretch
// boundary gets one partial state from each wave it touches.  Those waves
// combine their states in a tree of fan-in kMergeFanIn: a wave stores its
// state in the workspace and counts itself in its group's arrival counter;
// the wave that completes a group merges the group's states (in index order,
// so the result does not depend on arrival order) and carries the merged
// state to the next level, and the last one writes the output.
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
#include <mutex>
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kNegInf = -__builtin_inff();

// Per-wave timeline, compiled only into the instrumented library (PKV_TIMELINE):
// for each decode wave the real-time clock (100 MHz) at entry, after its first
// tile, after 1/4, 1/2 and 3/4 of its tiles and at its end, then its hardware
// wave id | XCD << 32 | tile count << 40, then the clock after its last tile
// (before the state it closes is merged and written).  Lane 0 writes the eight
// words once, at the end; waves without a stretch write nothing.
#ifdef PKV_TIMELINE
__device__ unsigned long long g_timeline[kMaxWaves * 8];
#define PKV_TL(...) __VA_ARGS__
#else
#define PKV_TL(...)
#endif

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

// Partial-state slot k (0, 1) of wave w, and arrival counter idx of merge level lvl.
__device__ __forceinline__ float* slot_ptr(const DecodeArgs& a, uint32_t w, int k) {
    return a.ws + kSlotBase + (int64_t(w) * 2 + k) * a.slot_floats;
}

__device__ __forceinline__ int* counter_ptr(const DecodeArgs& a, int lvl, uint32_t idx) {
    return reinterpret_cast<int*>(a.ws) + kWsHeader + lvl * kMaxWaves + idx;
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

// Softmax state of a run over some of its tokens, in the matrix-core output
// layout: lane (col, g) holds head col's running maximum m (base 2) and
// normaliser l, both replicated over g, and acc[c] = dimensions 16c + 4g ..
// 16c + 4g + 3 of the unnormalised output.  Lanes with col >= rh carry no head.
template <int NVC>
struct State {
    float m, l;
    f32x4 acc[NVC];
};

template <int NVC>
__device__ __forceinline__ void state_clear(State<NVC>& s) {
    s.m = kNegInf;
    s.l = 0.0f;
#pragma unroll
    for (int c = 0; c < NVC; ++c) s.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// s <- merge(s, t): M = max(m_s, m_t), each side weighted by 2^(m - M)
// (weight 0 for a side without scores).  Merging into a cleared state copies
// t exactly.
template <int NVC>
__device__ __forceinline__ void state_merge(State<NVC>& s, const State<NVC>& t) {
    const float M = fmaxf(s.m, t.m);
    const float ws = s.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(s.m - M);
    const float wt = t.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(t.m - M);
    s.m = M;
    // explicit fused products, so that the same states merge to the same bits wherever this is inlined
    s.l = __builtin_fmaf(t.l, wt, s.l * ws);
#pragma unroll
    for (int c = 0; c < NVC; ++c) s.acc[c] = __builtin_elementwise_fma(t.acc[c], f32x4(wt), s.acc[c] * ws);
}

// Slot traffic between waves uses agent-coherent accesses (SC1: stores write
// through and loads miss in the caches that are not coherent across the
// device), so a state is published by waiting for its stores before the
// arrival is counted, with no cache-wide write-back or invalidation.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kAgentCoherent = 16;  // SC1 cache-policy bit
constexpr unsigned kRawBufferWord3 = 0x00020000u;

// A slot holds m[16], l[16], then D values per head: acc in f32 for f32
// queries; acc / l in bf16 for bf16 queries (a partial result rounded as an
// output would be, half the bytes written through and read back), which the
// load scales by l again.  In bf16 a lane moves chunks c and c + 1 in one
// 16-byte access, and the four lanes of a column fill one 64-byte line per
// access (lane (col, g) at col * D + 16 c + 8 g), so that the stores, which
// write through, are whole lines.
// Two chunks of a state's acc as stored in a bf16 slot (acc * inv, rounded to
// nearest even), and back (times l).
__device__ __forceinline__ u32x4 slot_pack(const f32x4& a, const f32x4& b, float inv) {
    const f32x4 o0 = a * inv, o1 = b * inv;
    return u32x4{pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3]), pack_bf16(o1[0], o1[1]), pack_bf16(o1[2], o1[3])};
}

__device__ __forceinline__ void slot_unpack(const u32x4& v, float l, f32x4& a, f32x4& b) {
    const f32x4 o0 = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                      __uint_as_float(v[1] & 0xffff0000u)};
    const f32x4 o1 = {__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xffff0000u), __uint_as_float(v[3] << 16),
                      __uint_as_float(v[3] & 0xffff0000u)};
    a = o0 * l;
    b = o1 * l;
}

__device__ __forceinline__ float slot_inv(float l) { return l > 0.0f ? 1.0f / l : 0.0f; }

template <int QT, int D, int NVC>
__device__ __forceinline__ void state_store(float* f, int slot_bytes, const State<NVC>& s, bool hv) {
    const int lane = lane_id(), g = lane >> 4, col = lane & 15;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(f, 0, slot_bytes, kRawBufferWord3);
    if (!hv) return;
    if (g == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s.m), r, col * 4, 0, kAgentCoherent);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s.l), r, (kMaxRunHeads + col) * 4, 0, kAgentCoherent);
    }
    if constexpr (QT == kF32) {
        const int ab = (kSlotHead + col * D + 4 * g) * 4;
#pragma unroll
        for (int c = 0; c < NVC; ++c)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s.acc[c]), r, ab + 64 * c, 0,
                                                   kAgentCoherent);
    } else {
        const int ab = kSlotHead * 4 + (col * D + 8 * g) * 2;
        const float inv = slot_inv(s.l);
#pragma unroll
        for (int c = 0; c < NVC; c += 2)
            __builtin_amdgcn_raw_buffer_store_b128(slot_pack(s.acc[c], s.acc[c + 1], inv), r, ab + 32 * c, 0,
                                                   kAgentCoherent);
    }
}

// A member's slot as loaded, before it is widened into a State: its m, l and
// its values (f32 acc, or bf16 acc / l two chunks per access), so that the
// loads of the next members can be in flight while one is merged.
template <int QT, int NVC>
struct SlotRead {
    static constexpr int NQ = QT == kF32 ? NVC : NVC / 2;  // 16-byte accesses per lane
    float m, l;
    u32x4 v[NQ];
};

template <int QT, int D, int NVC>
__device__ __forceinline__ void slot_fetch(const float* f, int slot_bytes, bool hv, SlotRead<QT, NVC>& x) {
    const int lane = lane_id(), g = lane >> 4;
    const int col = hv ? (lane & 15) : 0;  // lanes without a head read head 0's data and never store it
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(f), 0, slot_bytes, kRawBufferWord3);
    x.m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, col * 4, 0, kAgentCoherent));
    x.l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (kMaxRunHeads + col) * 4, 0, kAgentCoherent));
    const int ab = QT == kF32 ? (kSlotHead + col * D + 4 * g) * 4 : kSlotHead * 4 + (col * D + 8 * g) * 2;
#pragma unroll
    for (int q = 0; q < SlotRead<QT, NVC>::NQ; ++q)
        x.v[q] = __builtin_amdgcn_raw_buffer_load_b128(r, ab + 64 * q, 0, kAgentCoherent);
}

// res <- merge(res, x), x widened one access at a time (the same operations as
// state_merge on the state a slot load gives).
template <int QT, int NVC>
__device__ __forceinline__ void merge_slot(State<NVC>& res, const SlotRead<QT, NVC>& x) {
    const float M = fmaxf(res.m, x.m);
    const float ws = res.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(res.m - M);
    const float wt = x.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(x.m - M);
    res.m = M;
    res.l = __builtin_fmaf(x.l, wt, res.l * ws);
#pragma unroll
    for (int q = 0; q < SlotRead<QT, NVC>::NQ; ++q) {
        if constexpr (QT == kF32) {
            res.acc[q] = __builtin_elementwise_fma(__builtin_bit_cast(f32x4, x.v[q]), f32x4(wt), res.acc[q] * ws);
        } else {
            f32x4 a, b;
            slot_unpack(x.v[q], x.l, a, b);
            res.acc[2 * q] = __builtin_elementwise_fma(a, f32x4(wt), res.acc[2 * q] * ws);
            res.acc[2 * q + 1] = __builtin_elementwise_fma(b, f32x4(wt), res.acc[2 * q + 1] * ws);
        }
    }
}

// The dimension held at position p of a bf16 slot column or state row: 16-byte
// group p / 8 holds chunk 2 (p / 32) + (p / 4) % 2 of lane g = (p / 8) % 4.
__device__ __forceinline__ int row_dim(int p) { return 16 * (2 * (p / 32) + (p / 4) % 2) + 4 * ((p / 8) % 4) + p % 4; }

// State rows of the shared-prefix decode: for `rows` = num_seqs * num_heads
// (row = sequence * num_heads + head), the output-shaped part of every row
// first, then the (m, l) pairs of every row, so that each row's first part is
// whole 64-byte lines.  With f32 queries the first part is acc[D] in f32; with
// bf16 queries it is acc / l in bf16 (the partial result rounded as an output
// would be, half the bytes to write and read again), in a slot column's order.
// Each lane moves its column's row; the same agent-coherent accesses as the
// slots.
template <int QT, int D, int NVC>
__device__ __forceinline__ void row_store(float* base, int bytes, int64_t rows, int64_t row, const State<NVC>& s,
                                          bool on) {
    constexpr int EB = QT == kF32 ? 4 : 2;  // bytes per element of the first part
    const int g = lane_id() >> 4;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kRawBufferWord3);
    if (!on) return;
    const int off = int(row) * D * EB;
    if constexpr (QT == kF32) {
#pragma unroll
        for (int c = 0; c < NVC; ++c)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s.acc[c]), r,
                                                   off + (16 * c + 4 * g) * 4, 0, kAgentCoherent);
    } else {  // the order of a bf16 slot column (row_dim gives a position's dimension)
        const float inv = slot_inv(s.l);
#pragma unroll
        for (int c = 0; c < NVC; c += 2)
            __builtin_amdgcn_raw_buffer_store_b128(slot_pack(s.acc[c], s.acc[c + 1], inv), r, off + (16 * c + 8 * g) * 2,
                                                   0, kAgentCoherent);
    }
    if (g == 0) {
        const int mo = int(rows * D * EB + 8 * row);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s.m), r, mo, 0, kAgentCoherent);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s.l), r, mo + 4, 0, kAgentCoherent);
    }
}

// A wave's merged state of the partitions it has finished of the current run
// waits in LDS (lane-major, conflict-free) while the next partition streams,
// so it occupies no registers in the streaming loop.
template <int NVC>
struct LdsState {
    float m[64], l[64], acc[4 * NVC][64];
};

template <int NVC>
__device__ __forceinline__ void lds_put(LdsState<NVC>& x, const State<NVC>& s) {
    const int lane = lane_id();
    x.m[lane] = s.m;
    x.l[lane] = s.l;
#pragma unroll
    for (int c = 0; c < NVC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) x.acc[4 * c + r][lane] = s.acc[c][r];
}

// s <- merge(x, s) with x read from LDS one accumulator at a time (the
// earlier state first, as state_merge(x, s) would compute it).
template <int NVC>
__device__ __forceinline__ void lds_merge_into(const LdsState<NVC>& x, State<NVC>& s) {
    const int lane = lane_id();
    const float xm = x.m[lane];
    const float M = fmaxf(xm, s.m);
    const float wx = xm == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(xm - M);
    const float ws = s.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(s.m - M);
    s.m = M;
    s.l = x.l[lane] * wx + s.l * ws;
#pragma unroll
    for (int c = 0; c < NVC; ++c) {
        const f32x4 xa = {x.acc[4 * c][lane], x.acc[4 * c + 1][lane], x.acc[4 * c + 2][lane], x.acc[4 * c + 3][lane]};
        s.acc[c] = xa * wx + s.acc[c] * ws;
    }
}

template <int NVC>
__device__ __forceinline__ void lds_get(const LdsState<NVC>& x, State<NVC>& s) {
    const int lane = lane_id();
    s.m = x.m[lane];
    s.l = x.l[lane];
#pragma unroll
    for (int c = 0; c < NVC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) s.acc[c][r] = x.acc[4 * c + r][lane];
}

// Output row `row` (sequence * num_heads + head) of this lane's column:
// v_scale * acc / l (0 for a row without scores).
template <int QT, int D, int NVC>
__device__ __forceinline__ void state_output(const DecodeArgs& a, int64_t row, const State<NVC>& st, bool hv) {
    const int g = lane_id() >> 4;
    if (!hv) return;
    const float inv = st.l > 0.0f ? a.v_scale / st.l : 0.0f;
    const int64_t o = row * D + 4 * g;
#pragma unroll
    for (int c = 0; c < NVC; ++c) {
        const f32x4 r = st.acc[c] * inv;
        if constexpr (QT == kF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o + 16 * c) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o + 16 * c) =
                make_uint2(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]));
        }
    }
}

// How sequence s is decoded.  Plain: its runs read blocks [0, nb).  Shared
// prefix: its first pbe blocks are read by the prefix runs of sequence cl
// (the first of the consecutive sequences of s's sharing group that one
// prefix run serves), whose columns hold the heads of `members` sequences;
// its own suffix runs read blocks [pbe, nb), and the two states are merged.
// The test is made from s's and cl's entries alone, so every sequence is
// covered by exactly one prefix run or by none, whatever the arrays hold.
struct SeqInfo {
    int len;  // clamped context length (0 past the batch)
    int pbe;  // blocks read by a prefix run (0: plain)
    int cl;   // sequence whose prefix runs cover s (-1: plain)
    int nq;   // several queries: new query tokens, clamped into [0, len]
    int q0;   // several queries: first query row
};

// Several queries: blocks the run of token group g needs (through its last
// token, at position len - nq + min((g + 1) tpr, nq)).
__device__ __forceinline__ int group_blocks(int len, int nq, int tpr, int g) {
    const int last = min((g + 1) * tpr, nq);
    return (len - nq + last + kBlockTokens - 1) / kBlockTokens;
}

__device__ __forceinline__ int shared_blocks(const DecodeArgs& a, int s, int L) {
    const int pb = a.prefix_blocks[s];
    const int full = L / kBlockTokens;  // only whole blocks are shared
    return pb < 0 ? 0 : (pb > full ? full : pb);
}

template <int M>
__device__ __forceinline__ SeqInfo seq_info(const DecodeArgs& a, int s) {
    SeqInfo r{0, 0, -1, 0, 0};
    if (s >= a.num_seqs) return r;
    r.len = clamped_len(a, s);
    if constexpr (M == kModeMulti) {
        r.q0 = a.cu_q[s];
        const int n = a.cu_q[s + 1] - r.q0;
        r.nq = n < 0 ? 0 : (n > r.len ? r.len : n);
    }
    if constexpr (M == kModeShared) {
        const int pbs = shared_blocks(a, s, r.len);
        const int ld = a.prefix_leader[s];
        const bool led = ld >= 0 && ld <= s;
        const int c = led ? ld + (s - ld) / a.members * a.members : s;  // in [0, s]
        // c's entries are read whatever s's say (c is a valid sequence), so that the two sets of reads are
        // two round trips, not a chain of four
        const int ldc = a.prefix_leader[c];
        const int pbc = shared_blocks(a, c, clamped_len(a, c));
        const bool ok = c == s || (ldc == ld && pbc == pbs);
        if (pbs > 0 && led && ok) {
            r.pbe = pbs;
            r.cl = c;
        }
    }
    return r;
}

// Units of sequence s: its suffix (or plain) runs, plus the prefix runs it
// leads; with several queries, the runs of every token group.
template <int M>
__device__ __forceinline__ uint32_t seq_units(const DecodeArgs& a, const SeqInfo& si, int s) {
    if constexpr (M == kModeMulti) {
        uint32_t b = 0;
        for (int g = 0; g * a.members < si.nq; ++g) b += uint32_t(group_blocks(si.len, si.nq, a.members, g));
        return b * uint32_t(a.runs);
    }
    const int nb = (si.len + kBlockTokens - 1) / kBlockTokens;
    return uint32_t(nb - si.pbe + (si.cl == s ? si.pbe : 0)) * uint32_t(a.runs);
}

// The same count in 64 bits, for the guard against totals the 32-bit unit
// line cannot hold (possible only for contents the host does not check, such
// as a cu_seqlens_q that decreases).
template <int M>
__device__ __forceinline__ uint64_t seq_units64(const DecodeArgs& a, const SeqInfo& si, int s) {
    if constexpr (M == kModeMulti) {
        uint64_t b = 0;
        for (int g = 0; g * a.members < si.nq; ++g) b += uint64_t(group_blocks(si.len, si.nq, a.members, g));
        return b * uint64_t(a.runs);
    }
    const int nb = (si.len + kBlockTokens - 1) / kBlockTokens;
    return uint64_t(nb - si.pbe + (si.cl == s ? si.pbe : 0)) * uint64_t(a.runs);
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor(uint32_t(x), off), hi = __shfl_xor(uint32_t(x >> 32), off);
        x += (uint64_t(hi) << 32) | lo;
    }
    return x;
}

// Unit totals at or above this bound are refused by the kernel (every wave
// returns without a write): the unit line and its cursors use 32-bit
// positions, and the host's size check keeps valid inputs below it.
constexpr uint64_t kMaxUnits = uint64_t(1) << 31;

// Forward cursor over the sequences, 64 at a time: lane i holds sequence
// base + i.
struct Cursor {
    int base;        // first sequence of the chunk
    SeqInfo si;      // lane: its sequence
    uint32_t inc;    // lane: inclusive prefix of units over the chunk
    uint32_t start;  // units before the chunk
    uint32_t tot;    // units in the chunk
};

template <int M>
__device__ __forceinline__ void cursor_set(Cursor& c, const DecodeArgs& a, int base, const SeqInfo& si) {
    c.base = base;
    c.si = si;
    c.inc = wave_scan(seq_units<M>(a, c.si, base + lane_id()));
    c.tot = __builtin_amdgcn_readlane(c.inc, 63);
}
template <int M>
__device__ __forceinline__ void cursor_load(Cursor& c, const DecodeArgs& a, int base) {
    cursor_set<M>(c, a, base, seq_info<M>(a, base + lane_id()));
}

template <int M>
__device__ __forceinline__ void cursor_advance(Cursor& c, const DecodeArgs& a) {
    c.start += c.tot;
    cursor_load<M>(c, a, c.base + 64);
}

// Lane of the chunk holding the sequence that contains unit u (u < U).
template <int M>
__device__ __forceinline__ int cursor_find(Cursor& c, const DecodeArgs& a, uint32_t u) {
    while (c.start + c.tot <= u) cursor_advance<M>(c, a);
    return __builtin_ctzll(__ballot(c.start + c.inc > u));
}

// Lane of the next sequence with units after lane i (one exists).
template <int M>
__device__ __forceinline__ int cursor_next(Cursor& c, const DecodeArgs& a, int i) {
    if constexpr (M == kModePlain) {  // a sequence has units exactly when it has tokens
        unsigned long long m = __ballot(lane_id() > i && c.si.len > 0);
        while (m == 0) {
            cursor_advance<M>(c, a);
            m = __ballot(c.si.len > 0);
        }
        return __builtin_ctzll(m);
    }
    const uint32_t prev = __shfl_up(c.inc, 1);
    unsigned long long m = __ballot(lane_id() > i && c.inc != (lane_id() == 0 ? 0u : prev));
    while (m == 0) {
        cursor_advance<M>(c, a);
        const uint32_t p = __shfl_up(c.inc, 1);
        m = __ballot(c.inc != (lane_id() == 0 ? 0u : p));
    }
    return __builtin_ctzll(m);
}

// Lane `lane`'s query / output row and column state for one run.
struct Cols {
    int64_t row;  // sequence * num_heads + head (a valid row for lanes without a head)
    bool hv;      // the column holds a head
    bool sne;     // prefix runs: that head's sequence also has suffix runs
};

// Columns of prefix run (s, hg): column col serves head hg * rh + col % rh of
// sequence s + col / rh, if that sequence is covered by s's prefix runs.
template <int M>
__device__ __forceinline__ Cols prefix_cols(const DecodeArgs& a, const Cursor& cur, int i, int s, int hg, int pbe) {
    const int col = lane_id() & 15;
    const int member = col / a.rh;
    const int sm = s + member;
    const int src = min(i + member, 63);
    SeqInfo x{__shfl(cur.si.len, src), 0, __shfl(cur.si.cl, src), 0, 0};
    if (i + member >= 64) x = seq_info<M>(a, sm);  // in the next chunk of the cursor
    const bool hv = col < a.members * a.rh && x.cl == s;
    const bool sne = (x.len + kBlockTokens - 1) / kBlockTokens > pbe;
    return Cols{int64_t(hv ? sm : s) * a.num_heads + hg * a.rh + col % a.rh, hv, sne};
}

// ---- the per-block steps, shared by every run kind ----

// Query operand Q^T of one run: this lane's column holds query row `qr` (heads
// on columns; zero for columns without a head).
template <int KV, int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int64_t qr, bool hv, QOp<KV> (&qop)[Geo<KV, D>::NQ]) {
    using GE = Geo<KV, D>;
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    const int g = lane_id() >> 4;
    const int qelt = (QT == kF32) ? 4 : 2;
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + qr * D * qelt;
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
                const uint4 x =
                    hv ? *reinterpret_cast<const uint4*>(qrow + (64 * u + 16 * g + 8 * e) * 2) : make_uint4(0, 0, 0, 0);
                qop[2 * u + e] = __builtin_bit_cast(bf16x8, x);
            }
    } else {
#pragma unroll
        for (int u = 0; u < GE::NKL; ++u) {
            const float4 x =
                hv ? *reinterpret_cast<const float4*>(qrow + (16 * u + 4 * g) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            qop[4 * u + 0] = x.x;
            qop[4 * u + 1] = x.y;
            qop[4 * u + 2] = x.z;
            qop[4 * u + 3] = x.w;
        }
    }
}

// A load of 4, 8 or 16 bytes, plain or nontemporal.  Nontemporal loads carry
// the streaming hint to the caches: a KV tile is read once per call, and on
// MI355X a chip-wide stream of 8 KiB tiles read this way moves about 12 % more
// bytes per second than with ordinary loads (6.7 against 6.0 TB/s).
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

template <typename T, bool NT>
__device__ __forceinline__ T load_as(const uint8_t* p) {
    if constexpr (!NT) {
        return *reinterpret_cast<const T*>(p);
    } else if constexpr (sizeof(T) == 16) {
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p)));
    } else if constexpr (sizeof(T) == 8) {
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p)));
    } else {
        static_assert(sizeof(T) == 4, "4, 8 or 16 bytes");
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p)));
    }
}

// Step 1: the K and V tiles of physical block `id`, KV head kvh (NT: with the
// streaming hint, for tiles no other wave of the call reads).
template <int KV, int D, bool NT>
__device__ __forceinline__ void load_tile(const DecodeArgs& a, int kvh, int id, Tile<KV, D>& t) {
    using GE = Geo<KV, D>;
    const int lane = lane_id(), g = lane >> 4, col = lane & 15;
    const int64_t off = (int64_t(id) * a.num_kv_heads + kvh) * GE::TILE;
    const uint8_t* kt = static_cast<const uint8_t*>(a.k_cache) + off + lane * 16;
    const uint8_t* vt = static_cast<const uint8_t*>(a.v_cache) + off + (col * kBlockTokens + 4 * g) * GE::ELT;
#pragma unroll
    for (int u = 0; u < GE::NKL; ++u) t.k[u] = load_as<uint4, NT>(kt + u * 1024);
#pragma unroll
    for (int c = 0; c < GE::NVC; ++c) t.v[c] = load_as<VLoad<KV>, NT>(vt + c * 16 * kBlockTokens * GE::ELT);
}

// Combine x over the four lanes of this lane's column (lanes lane % 16 + 16 r):
// the gfx950 row swaps exchange rows 0<->1 and 2<->3 of 16 lanes, then the
// two halves of 32 lanes, in the vector ALU (no trip through the LDS
// crossbar).  The second operand of each swap goes through an opaque copy so
// that the compiler cannot merge the two operands of the swap into one value.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t x) {
    uint32_t y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

__device__ __forceinline__ float column_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), opaque_copy(__float_as_uint(m)), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The sum over the column as (r0 + r1) + (r2 + r3), the same in every lane.
__device__ __forceinline__ float column_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
    const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), opaque_copy(__float_as_uint(m)), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Running softmax state of one run inside the streaming loop, in the
// matrix-core output layout (see State); lsum is this lane's share of the
// normaliser (its four rows), summed over the row groups when the state closes.
template <int NVC>
struct Run {
    float m, lsum;
    f32x4 acc[NVC];
};

template <int NVC>
__device__ __forceinline__ void run_reset(Run<NVC>& r) {
    r.m = kNegInf;
    r.lsum = 0.0f;
#pragma unroll
    for (int c = 0; c < NVC; ++c) r.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int NVC>
__device__ __forceinline__ void run_close(const Run<NVC>& r, State<NVC>& st) {
    st.m = r.m;
    st.l = column_sum(r.lsum);
#pragma unroll
    for (int c = 0; c < NVC; ++c) st.acc[c] = r.acc[c];
}

// Steps 2-4 for one block with nv valid tokens, for CT query-column tiles
// at once: every score product first, then each column tile's softmax
// update, then every value product (K and V widened, and V masked, once for
// all column tiles).  With CAUSAL, this lane's column of tile c scores only
// the block's first upto[c] tokens (its token's position is upto[c] - 1
// relative to the block); the values stay masked by nv only.
template <int KV, int D, int CT, bool CAUSAL>
__device__ __forceinline__ void consume_tiles(const DecodeArgs& a, const Tile<KV, D>& t, int nv, const int (&upto)[CT],
                                              const QOp<KV> (&qop)[CT][Geo<KV, D>::NQ],
                                              Run<Geo<KV, D>::NVC> (&rs)[CT]) {
    using GE = Geo<KV, D>;
    const int g = lane_id() >> 4;
    f32x4 sacc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) sacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == kBF16) {
#pragma unroll
        for (int u = 0; u < GE::NKL; ++u)
#pragma unroll
            for (int c = 0; c < CT; ++c)
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[u]), qop[c][u], sacc[c],
                                                                  0, 0, 0);
    } else if constexpr (KV == kFP8) {
#pragma unroll
        for (int u = 0; u < GE::NKL; ++u) {
            const bf16x8 k0 = fp8x8_to_bf16x8(t.k[u].x, t.k[u].y);
            const bf16x8 k1 = fp8x8_to_bf16x8(t.k[u].z, t.k[u].w);
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[c][2 * u], sacc[c], 0, 0, 0);
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[c][2 * u + 1], sacc[c], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < GE::NKL; ++u)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].x), qop[c][4 * u + 0], sacc[c], 0, 0, 0);
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].y), qop[c][4 * u + 1], sacc[c], 0, 0, 0);
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].z), qop[c][4 * u + 2], sacc[c], 0, 0, 0);
                sacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[u].w), qop[c][4 * u + 3], sacc[c], 0, 0, 0);
            }
    }
    const int cnt = min(max(nv - 4 * g, 0), 4);  // valid tokens among this lane's four
    float sv[CT][4], bm[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const int scnt = CAUSAL ? min(cnt, max(upto[c] - 4 * g, 0)) : cnt;  // ... that this column may see
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[c][r] = r < scnt ? sacc[c][r] * a.score_scale : kNegInf;
        bm[c] = fmaxf(fmaxf(sv[c][0], sv[c][1]), fmaxf(sv[c][2], sv[c][3]));
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) bm[c] = column_max(bm[c]);
    float alpha[CT], pw[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const float mn = fmaxf(rs[c].m, bm[c]);
        const bool live = mn != kNegInf;
        alpha[c] = live ? __builtin_amdgcn_exp2f(rs[c].m - mn) : 1.0f;
        rs[c].m = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[c][r] = live ? __builtin_amdgcn_exp2f(sv[c][r] - mn) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        if (__ballot(alpha[c] != 1.0f)) {
#pragma unroll
            for (int v = 0; v < GE::NVC; ++v) rs[c].acc[v] *= alpha[c];
        }
    }
    if constexpr (KV == kF32) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
            rs[c].lsum = rs[c].lsum * alpha[c] + ((pw[c][0] + pw[c][1]) + (pw[c][2] + pw[c][3]));
#pragma unroll
        for (int v = 0; v < GE::NVC; ++v) {
            const uint4 vv = t.v[v];
            const float v0 = cnt > 0 ? __uint_as_float(vv.x) : 0.0f;
            const float v1 = cnt > 1 ? __uint_as_float(vv.y) : 0.0f;
            const float v2 = cnt > 2 ? __uint_as_float(vv.z) : 0.0f;
            const float v3 = cnt > 3 ? __uint_as_float(vv.w) : 0.0f;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                rs[c].acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(v0, pw[c][0], rs[c].acc[v], 0, 0, 0);
                rs[c].acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(v1, pw[c][1], rs[c].acc[v], 0, 0, 0);
                rs[c].acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(v2, pw[c][2], rs[c].acc[v], 0, 0, 0);
                rs[c].acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(v3, pw[c][3], rs[c].acc[v], 0, 0, 0);
            }
        }
    } else {
        i16x4 pb[CT];
        const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const uint32_t p01 = pack_bf16(pw[c][0], pw[c][1]);
            const uint32_t p23 = pack_bf16(pw[c][2], pw[c][3]);
            // the normaliser sums the rounded weights the value product uses
            rs[c].lsum = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2, p23), ones,
                __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01), ones, rs[c].lsum * alpha[c], false),
                false);
            pb[c] = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
        }
        // V entries of tokens past the block's valid ones are zeroed (their
        // weights are 0, but the memory may hold any bits); a full block,
        // the usual case, needs no mask
        auto pv = [&](auto masked) {
            const uint32_t mlo = cnt >= 2 ? 0xffffffffu : (cnt == 1 ? 0x0000ffffu : 0u);
            const uint32_t mhi = cnt >= 4 ? 0xffffffffu : (cnt == 3 ? 0x0000ffffu : 0u);
#pragma unroll
            for (int v = 0; v < GE::NVC; ++v) {
                uint2 vv;
                if constexpr (KV == kBF16) {
                    vv = t.v[v];
                } else {
                    vv = make_uint2(fp8x2_to_bf16x2<false>(t.v[v]), fp8x2_to_bf16x2<true>(t.v[v]));
                }
                if constexpr (decltype(masked)::value) {
                    vv.x &= mlo;
                    vv.y &= mhi;
                }
                const i16x4 va = __builtin_bit_cast(i16x4, vv);
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    rs[c].acc[v] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[c], rs[c].acc[v], 0, 0, 0);
            }
        };
        if (nv >= kBlockTokens)
            pv(std::false_type{});
        else
            pv(std::true_type{});
    }
}

template <int KV, int D, bool CAUSAL>
__device__ __forceinline__ void consume_tile(const DecodeArgs& a, const Tile<KV, D>& t, int nv, int upto,
                                             const QOp<KV> (&qop)[Geo<KV, D>::NQ], Run<Geo<KV, D>::NVC>& rs) {
    const int up[1] = {upto};
    consume_tiles<KV, D, 1, CAUSAL>(a, t, nv, up, reinterpret_cast<const QOp<KV>(&)[1][Geo<KV, D>::NQ]>(qop),
                                    reinterpret_cast<Run<Geo<KV, D>::NVC>(&)[1]>(rs));
}

// Stretch geometry, identical in every wave.  Stretch t of nw covers units
// [lo(t), lo(t + 1)); every stretch holds at least one unit.  When nw is a
// multiple of 8, the line is cut into 8 regions, one per XCD (workgroup w runs
// on XCD w mod 8 and takes stretch (w mod 8) * nw / 8 + w / 8), sized in
// proportion to the XCD's weight and split evenly among its nw / 8 waves;
// otherwise the split is even.  One region per XCD keeps the sequences that
// share a prompt prefix (consecutive in the batch) on one XCD's L2.  On
// MI355X the odd-numbered XCDs stream 16- and 32-bit tiles about 10 % slower
// than the even ones (measured per wave; not so for 8-bit tiles), so their
// regions weigh 14 against 16.
#ifndef PKV_ODD_XCD_WEIGHT
#define PKV_ODD_XCD_WEIGHT 14
#endif
#ifndef PKV_ODD_XCD_WEIGHT8
#define PKV_ODD_XCD_WEIGHT8 16
#endif
struct Split {
    uint32_t U, nw;
    uint32_t m;    // waves per region (0: even split, no regions)
    uint32_t odd;  // weight of an odd XCD's region (an even one weighs 16)
    __device__ void init(uint32_t units, uint32_t waves, uint32_t odd_weight) {
        U = units;
        nw = waves;
        odd = odd_weight;
        m = (waves % 8 == 0 && units >= 2 * waves) ? waves / 8 : 0;
    }
    // first unit of region x (weights alternate 16, odd, 16, odd, ...)
    __device__ uint32_t rb(uint32_t x) const {
        const uint64_t acc = 16 * ((x + 1) / 2) + uint64_t(odd) * (x / 2);
        return uint32_t(uint64_t(U) * acc / (64 + 4 * uint64_t(odd)));
    }
    __device__ uint32_t lo(uint32_t t) const {
        if (m == 0) return uint32_t(uint64_t(t) * U / nw);
        const uint32_t x = t / m, k = t % m;
        if (x >= 8) return U;
        const uint32_t r0 = rb(x);
        return r0 + uint32_t(uint64_t(k) * (rb(x + 1) - r0) / m);
    }
    // the stretch that holds unit u: the largest t with lo(t) <= u
    __device__ uint32_t wave_of(uint32_t u) const {
        if (m == 0) return uint32_t((uint64_t(u + 1) * nw - 1) / U);
        uint32_t x = 0;
        while (x < 7 && u >= rb(x + 1)) ++x;
        const uint32_t r0 = rb(x);
        return x * m + uint32_t((uint64_t(u - r0 + 1) * m - 1) / (rb(x + 1) - r0));
    }
};

// Combine the partial states of a run cut between waves and write its output.
// The run's units [run_first, run_last] touch waves w0..w1; the wave with index
// i = w - w0 among them holds state st.  Contributor i keeps its state in slot
// 0 of wave w0 + i, except contributor 0 when the run starts after w0's first
// unit (then the run is w0's last, not its first, run: slot 1).  A level-l node
// n of the tree lives in the slot of contributor n * kMergeFanIn^l: the node
// that completes group n at level l - 1 has merged that slot's previous
// contents before it stores there.
struct Contrib {
    uint32_t w0, w1;
    bool first_in_slot1;
};

__device__ __forceinline__ Contrib contributors(const Split& sp, uint32_t run_first, uint32_t run_last) {
    const uint32_t w0 = sp.wave_of(run_first);
    return Contrib{w0, sp.wave_of(run_last), run_first != sp.lo(w0)};
}

// Arrivals already counted in this wave's first merge group, read while the
// wave still streams its last segment of the run (lane 0; -1: no group).
__device__ __forceinline__ int peek_arrivals(const DecodeArgs& a, const Contrib& c, uint32_t w) {
    const uint32_t idx = w - c.w0;
    const uint32_t first = idx / kMergeFanIn * kMergeFanIn;
    const uint32_t cnt = c.w1 - c.w0 + 1;
    if (min(cnt, first + kMergeFanIn) - first <= 1) return -1;
    int seen = -1;
    if (lane_id() == 0)
        seen = __hip_atomic_load(counter_ptr(a, 0, c.w0 + first), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return seen;
}

// The state a wave keeps in LDS, in the form its slot would hold (so that a
// merge gives the same bits whichever member kept its state).
template <int QT, int NVC>
__device__ __forceinline__ void slot_own(const LdsState<NVC>& o, SlotRead<QT, NVC>& x) {
    const int lane = lane_id();
    x.m = o.m[lane];
    x.l = o.l[lane];
    auto chunk = [&](int c) {
        return f32x4{o.acc[4 * c][lane], o.acc[4 * c + 1][lane], o.acc[4 * c + 2][lane], o.acc[4 * c + 3][lane]};
    };
#pragma unroll
    for (int q = 0; q < SlotRead<QT, NVC>::NQ; ++q) {
        if constexpr (QT == kF32)
            x.v[q] = __builtin_bit_cast(u32x4, chunk(q));
        else
            x.v[q] = slot_pack(chunk(2 * q), chunk(2 * q + 1), slot_inv(x.l));
    }
}

// Returns true in the one wave that ends up with the run's whole state (left
// in own_state).
template <int QT, int D, int NVC>
__device__ bool merge_across(const DecodeArgs& a, const Contrib& c, uint32_t w, const State<NVC>& mine,
                             LdsState<NVC>& own_state, bool hv, int seen) {
    auto slot = [&](uint32_t i) { return slot_ptr(a, c.w0 + i, (i == 0 && c.first_in_slot1) ? 1 : 0); };
    const int slot_bytes = a.slot_floats * 4;
    seen = __builtin_amdgcn_readfirstlane(seen);
    lds_put(own_state, mine);  // this wave's node state waits in LDS between the steps below
    uint32_t idx = w - c.w0, cnt = c.w1 - c.w0 + 1, span = 1;
    for (int lvl = 0; cnt > 1; ++lvl) {
        const uint32_t first = idx / kMergeFanIn * kMergeFanIn;
        const uint32_t members = min(cnt, first + kMergeFanIn) - first;
        if (members > 1) {
            int* ctr = counter_ptr(a, lvl, c.w0 + first * span);
            // Every other member had counted itself before this wave's last
            // segment began: it is the last arrival and need not publish.
            bool last = lvl == 0 && uint32_t(seen) == members - 1;
            if (!last) {
                {
                    State<NVC> t;
                    lds_get(own_state, t);
                    state_store<QT, D>(slot(idx * span), slot_bytes, t, hv);
                }
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_s_waitcnt(0);  // the state has reached the coherent level before it is counted
                int old = 0;
                if (lane_id() == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __builtin_amdgcn_readfirstlane(old);
                last = uint32_t(old) == members - 1;
            }
            if (!last) return false;  // a later arrival completes the group
            if (lane_id() == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the loads below are issued after the count was seen

            // Members in index order, this wave's own from LDS; the slots of the
            // next two members load while one merges.  Every pass issues its
            // loads (past the group they read the last member's slot again,
            // unused), so the loads never sit behind a branch.
            const uint32_t own = idx - first;
            auto fetch = [&](SlotRead<QT, NVC>& x, uint32_t k) {
                slot_fetch<QT, D>(slot((first + min(k, members - 1)) * span), slot_bytes, hv, x);
            };
            State<NVC> res;
            state_clear(res);
            SlotRead<QT, NVC> xa, xb;
            fetch(xa, 0);
            fetch(xb, 1);
#pragma unroll 1
            for (uint32_t k = 0; k < members; k += 2) {
                if (k == own) slot_own(own_state, xa);
                merge_slot(res, xa);
                fetch(xa, k + 2);
                if (k + 1 < members) {
                    if (k + 1 == own) slot_own(own_state, xb);
                    merge_slot(res, xb);
                }
                fetch(xb, k + 3);
            }
            lds_put(own_state, res);
        }
        idx /= kMergeFanIn;
        cnt = (cnt + kMergeFanIn - 1) / kMergeFanIn;
        span *= kMergeFanIn;
    }
    return true;
}

// Shared-prefix decode: the finished state of a covered (sequence, head) row
// from its prefix run and from its own (suffix) runs are both stored as state
// rows; cascade_merge_kernel, launched after the decode on the same stream,
// combines them with the merge rule and writes the output.  Rows whose
// sequence has no suffix runs (its context ends inside the shared blocks) are
// written straight from the prefix run; uncovered sequences are plain runs.
template <int QT, int D, int NVC>
__device__ void finish_suffix(const DecodeArgs& a, const Cols& cm, const State<NVC>& st) {
    row_store<QT, D>(a.sstate, a.state_bytes, int64_t(a.num_seqs) * a.num_heads, cm.row, st, cm.hv);
}

template <int QT, int D, int NVC>
__device__ void finish_prefix(const DecodeArgs& a, const Cols& cm, const State<NVC>& st) {
    // rows whose sequence has suffix runs
    row_store<QT, D>(a.pstate, a.state_bytes, int64_t(a.num_seqs) * a.num_heads, cm.row, st, cm.hv && cm.sne);
    state_output<QT, D>(a, cm.row, st, cm.hv && !cm.sne);               // the rest: the prefix state is whole
}

constexpr int kLenChunks = 8;  // 64-sequence chunks of lengths read per round trip

// A piece: consecutive units of one run inside one partition of a wave's
// stretch, at most 64 blocks, so that its block ids fit in one vector
// register.  The walker plans pieces a few ahead of the tile being consumed.
enum PieceFlags : int {
    kNewRun = 1,    // the first piece of a run in this wave: new query operand
    kNewState = 2,  // starts a softmax state (a new run, or after a partition boundary)
    kClose = 4,     // the state ends with this piece
    kEndsPart = 8,  // ... and so does this wave's part of the run
    kLocal = 16,    // the whole run lies in this wave's stretch
    kReread = 32,   // other runs of the call read the same tiles (ordinary loads, so the L2 keeps them)
};

struct Piece {
    uint32_t p0, p1;  // positions [p0, p1) of its tiles in the wave's stream (p0 == p1: no piece)
    int s;            // sequence whose table row holds the blocks
    int lim0;         // tokens of the run at and after the piece's first block
    int info;         // head group (bits 0-15) | kind << 16 (0 plain, 1 prefix, 2 suffix) | flags << 20
    uint32_t contrib; // a cut run's waves: w0 | (w1 << 13) | first_in_slot1 << 26
    uint32_t cols;    // bit c: column c holds a head; bit 16 + c: its sequence has suffix runs (prefix runs)
    int ids;          // lane l < p1 - p0: physical block of the piece's l-th block
    int kvh;          // KV head of the piece's run
    int qrow0;        // several queries: query row of column 0's token
    int cpos0;        // several queries: column 0's token position + 1 - context length (<= 0)
};

static_assert(kMaxWaves <= (1 << 13), "wave indices are packed in 13 bits");

__device__ __forceinline__ uint32_t pack_contrib(const Contrib& c) {
    return c.w0 | (c.w1 << 13) | (c.first_in_slot1 ? 1u << 26 : 0u);
}

__device__ __forceinline__ Contrib unpack_contrib(uint32_t v) {
    return Contrib{v & 0x1fffu, (v >> 13) & 0x1fffu, ((v >> 26) & 1u) != 0};
}

__device__ __forceinline__ int piece_hg(const Piece& p) { return p.info & 0xffff; }
__device__ __forceinline__ int piece_kind(const Piece& p) { return (p.info >> 16) & 3; }
__device__ __forceinline__ int piece_flags(const Piece& p) { return p.info >> 20; }

// This lane's column of the piece's run (see Cols).
__device__ __forceinline__ Cols piece_cols(const DecodeArgs& a, const Piece& p) {
    const int col = lane_id() & 15;
    const bool hv = (p.cols >> col) & 1u;
    const bool sne = (p.cols >> (16 + col)) & 1u;
    const int hg = piece_hg(p);
    if (piece_kind(p) == 1)
        return Cols{int64_t(p.s + (hv ? col / a.rh : 0)) * a.num_heads + hg * a.rh + col % a.rh, hv, sne};
    if (piece_kind(p) == 3)  // several queries: column col is token col / rh of the group, head col % rh
        return Cols{int64_t(hv ? p.qrow0 + col / a.rh : 0) * a.num_heads + hg * a.rh + col % a.rh, hv, false};
    return Cols{int64_t(p.s) * a.num_heads + hg * a.rh + (hv ? col : 0), hv, sne};
}

// Waves per SIMD the register allocation must allow: two for the 16-bit and
// 8-bit pools (the streaming loop fits in 256 registers), one for fp32 pools
// of head_dim 128, whose tiles are twice as large.
#ifdef PKV_WAVES_PER_SIMD
template <int KV, int D>
constexpr int kWavesPerSimd = PKV_WAVES_PER_SIMD;
#else
template <int KV, int D>
constexpr int kWavesPerSimd = (KV == kF32 && D == 128) ? 1 : 2;
#endif

template <int KV, int D, int P, int M>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<KV, D>))) void paged_decode_kernel(
    DecodeArgs a) {
    using GE = Geo<KV, D>;
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    constexpr int NVC = GE::NVC;
    const uint32_t w = blockIdx.x;
    const uint32_t nwt = gridDim.x;
    const int lane = lane_id();
    PKV_TL(const unsigned long long tl_entry = __builtin_amdgcn_s_memrealtime();)

    // ---- total units; per-chunk totals of the first kLenChunks chunks; rows
    //      of empty sequences are zeroed (sequence s by wave s mod grid) ----
    uint32_t U = 0;
    uint64_t U64 = 0;  // the same total, without wrap-around
    uint32_t ctot[kLenChunks];
    SeqInfo sfirst[kLenChunks];  // the first kLenChunks chunks' entries, kept for the cursor
#pragma unroll
    for (int c = 0; c < kLenChunks; ++c) ctot[c] = 0;
    for (int base = 0; base < a.num_seqs; base += 64 * kLenChunks) {
        SeqInfo si[kLenChunks];
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) si[c] = seq_info<M>(a, base + 64 * c + lane);
        if (base == 0) {
#pragma unroll
            for (int c = 0; c < kLenChunks; ++c) sfirst[c] = si[c];
        }
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) {
            const int cb = base + 64 * c;
            if (cb >= a.num_seqs) break;
            const uint32_t t = __builtin_amdgcn_readlane(wave_scan(seq_units<M>(a, si[c], cb + lane)), 63);
            U64 += wave_sum64(seq_units64<M>(a, si[c], cb + lane));
            if (base == 0) ctot[c] = t;
            U += t;
            unsigned long long empty = __ballot(M != kModeMulti && cb + lane < a.num_seqs && si[c].len == 0);
            while (empty) {
                const int se = cb + __builtin_ctzll(empty);
                empty &= empty - 1;
                if (uint32_t(se) % nwt == w) zero_rows<QT, D>(a, se);
            }
        }
    }
    // Past the bound the 32-bit positions below could wrap: every wave returns
    // here.  Only several-query calls can get here (their per-sequence counts
    // come from cu_seqlens_q), and those write nothing before this point, so
    // the output and the workspace stay untouched.
    if (U64 >= kMaxUnits) return;
    Split sp;
    sp.init(U, U < nwt ? U : nwt, KV == kFP8 ? uint32_t(PKV_ODD_XCD_WEIGHT8) : uint32_t(PKV_ODD_XCD_WEIGHT));
    if (w >= sp.nw) return;
    const uint32_t sw = sp.m ? (w % 8) * sp.m + w / 8 : w;  // this wave's stretch
    const uint32_t lo = sp.lo(sw), hi = sp.lo(sw + 1);

    // ---- the sequence holding unit lo: skip whole cached chunks, then walk ----
    Cursor cur;
    cur.start = 0;
    int chunk = 0;
    {
        bool go = true;
#pragma unroll
        for (int c = 0; c < kLenChunks; ++c) {
            go = go && cur.start + ctot[c] <= lo;
            if (go) {
                cur.start += ctot[c];
                chunk = c + 1;
            }
        }
    }
    if (chunk < kLenChunks) {  // the chunk's entries are still in registers: no second round trip
        SeqInfo x = sfirst[0];
#pragma unroll
        for (int c = 1; c < kLenChunks; ++c)
            if (c == chunk) x = sfirst[c];
        cursor_set<M>(cur, a, 64 * chunk, x);
    } else {
        cursor_load<M>(cur, a, 64 * chunk);
    }
    int i = 0;
    // Runs of a sequence: npre prefix runs over blocks [0, pbe) (when it leads
    // a prefix group), then its runs over blocks [pbe, nb).
    // With several queries, a sequence's runs are its token groups (of
    // a.members new tokens) times its head groups, run r being group r / runs.
    int L = 0, nb = 0, pbe = 0, npre = 0, nq = 0, q0 = 0;
    auto enter = [&]() {
        L = __builtin_amdgcn_readlane(cur.si.len, i);
        nb = (L + kBlockTokens - 1) / kBlockTokens;
        if constexpr (M == kModeShared) {
            pbe = __builtin_amdgcn_readlane(cur.si.pbe, i);
            npre = __builtin_amdgcn_readlane(cur.si.cl, i) == cur.base + i ? a.runs : 0;
        }
        if constexpr (M == kModeMulti) {
            nq = __builtin_amdgcn_readlane(cur.si.nq, i);
            q0 = __builtin_amdgcn_readlane(cur.si.q0, i);
        }
    };
    auto nruns = [&]() -> int {
        if constexpr (M == kModeMulti) return (nq + a.members - 1) / a.members * a.runs;
        return npre + (nb > pbe ? a.runs : 0);
    };
    int r = 0, j = 0;
    uint32_t run_first = 0;
    uint32_t len = 0, kk = 1, part = 1, cut = 0;
    uint32_t u = 0;      // first unit not yet planned
    bool fresh = true;   // the next piece starts a new softmax state
    // position the walker at unit `at` (the start of the stretch)
    auto seek = [&](uint32_t at) {
        i = cursor_find<M>(cur, a, at);
        enter();
        const uint32_t prev = i > 0 ? uint32_t(__builtin_amdgcn_readlane(cur.inc, i - 1)) : 0u;
        uint32_t o = at - (cur.start + prev);
        const uint32_t pre_units = uint32_t(npre * pbe);
        if constexpr (M == kModeMulti) {
            int g = 0;
            while (true) {
                const uint32_t gb = uint32_t(group_blocks(L, nq, a.members, g));
                if (o < gb * uint32_t(a.runs)) {
                    r = g * a.runs + int(o / gb);
                    j = int(o % gb);
                    break;
                }
                o -= gb * uint32_t(a.runs);
                ++g;
            }
            run_first = at - uint32_t(j);
        } else if (o < pre_units) {
            r = int(o / uint32_t(pbe));
            j = int(o % uint32_t(pbe));
            run_first = at - uint32_t(j);
        } else {
            o -= pre_units;
            const uint32_t sl = uint32_t(nb - pbe);
            r = npre + int(o / sl);
            j = pbe + int(o % sl);
            run_first = at - uint32_t(j - pbe);
        }
        // partitions: kk equal parts of the stretch, each <= part_blocks
        len = hi - lo;
        kk = a.part_blocks > 0 ? (len + uint32_t(a.part_blocks) - 1) / uint32_t(a.part_blocks) : 1u;
        part = 1;
        cut = lo + uint32_t(uint64_t(len) / kk);
        u = at;
        fresh = true;
    };
    seek(lo);

    // ---- pieces, planned in order: the walker's next piece of the stream ----
    uint32_t spos = 0;  // stream position (tiles planned so far)
    auto plan = [&](Piece& pc) {
        if (u >= hi) {
            pc.p0 = pc.p1 = spos;
            pc.info = 0;
            pc.cols = 0;
            pc.ids = -1;
            pc.kvh = 0;
            return;
        }
        const int s = cur.base + i;
        const bool pre = r < npre;
        const int grp = M == kModeMulti ? r / a.runs : 0;  // several queries: the token group
        const int hg = M == kModeMulti ? r % a.runs : (pre ? r : r - npre);
        const int rlen = M == kModeMulti ? group_blocks(L, nq, a.members, grp) : (pre ? pbe : nb - pbe);
        const uint32_t run_end = run_first + uint32_t(rlen);
        const uint32_t seg_end = run_end < cut ? run_end : cut;
        const uint32_t pe = seg_end < u + 64u ? seg_end : u + 64u;
        const bool close = pe == seg_end;
        int f = 0;
        if (u == run_first || u == lo) f |= kNewRun | kNewState;
        if (fresh) f |= kNewState;
        if (close) f |= kClose;
        if (close && (seg_end == run_end || seg_end == hi)) f |= kEndsPart;
        if (run_first >= lo && pe == run_end) f |= kLocal;
        // the prefix runs of a sharing group, and the token groups of a sequence with several, read
        // tiles that other runs read again
        if (pre || (M == kModeMulti && nq > a.members)) f |= kReread;
        pc.p0 = spos;
        pc.p1 = spos + (pe - u);
        pc.s = s;
        pc.lim0 = (pre ? pbe * kBlockTokens : L) - j * kBlockTokens;
        pc.info = hg | ((M == kModeMulti ? 3 : (pre ? 1 : (pbe > 0 ? 2 : 0))) << 16) | (f << 20);
        pc.contrib = (f & kEndsPart) && !(f & kLocal) ? pack_contrib(contributors(sp, run_first, run_end - 1)) : 0u;
        pc.cols = (1u << a.rh) - 1u;
        if constexpr (M == kModeMulti) {
            // columns: a.members tokens of the group (those that exist) times rh heads
            const int first = grp * a.members;
            const int ntok = min(a.members, nq - first);
            const bool rows_ok = q0 >= 0 && int64_t(q0) + first + ntok <= int64_t(a.num_q_rows);
            pc.cols = rows_ok ? (ntok * a.rh >= 32 ? 0xffffffffu : (1u << (ntok * a.rh)) - 1u) & 0xffffu : 0u;
            pc.qrow0 = q0 + first;
            pc.cpos0 = first + 1 - nq;
        }
        if constexpr (M == kModeShared) {
            if (pre) {
                const Cols x = prefix_cols<M>(a, cur, i, s, hg, pbe);
                const uint32_t hvm = uint32_t(__ballot(x.hv)) & 0xffffu;  // row group 0 holds every column
                const uint32_t snem = uint32_t(__ballot(x.hv && x.sne)) & 0xffffu;
                pc.cols = hvm | (snem << 16);
            }
        }
        pc.ids = lane < int(pe - u) ? a.block_table[int64_t(s) * a.max_blocks + j + lane] : -1;
        pc.kvh = hg * a.rh / a.group;
        // advance the walker past the piece
        spos = pc.p1;
        j += int(pe - u);
        u = pe;
        fresh = close;
        if (u == cut && u < hi) {
            ++part;
            cut = lo + uint32_t(uint64_t(part) * len / kk);
        }
        if (close && seg_end == run_end && u < hi) {  // the next run
            run_first = run_end;
            if (++r == nruns()) {
                i = cursor_next<M>(cur, a, i);
                enter();
                r = 0;
            }
            j = r < npre ? 0 : pbe;
        }
    };

    // Slot 0 holds the piece being consumed; the tile P - 1 ahead lies in one
    // of slots 0..P-1 (a slot is planned when the piece before it is
    // consumed, so its block ids are loading while that piece's last tiles
    // are consumed).
    constexpr int NS = P;
    Piece sl[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) plan(sl[k]);

    using T = Tile<KV, D>;
    QOp<KV> qop[GE::NQ], qn[GE::NQ];  // the query operand of slot 0's run, and of slot 1's
    {
        const Cols c0 = piece_cols(a, sl[0]);
        load_q<KV, D>(a, c0.row, c0.hv, qop);
        const Cols c1 = piece_cols(a, sl[1]);
        load_q<KV, D>(a, c1.row, c1.hv, qn);
    }
    Run<NVC> rs;
    run_reset(rs);
    // several queries: this lane's column token position + 1 - context length;
    // a tile with `lim` tokens left of the context shows it lim + crel of them
    int crel = 0;
    auto set_crel = [&]() {
        if constexpr (M == kModeMulti) crel = sl[0].cpos0 + (lane & 15) / a.rh;
    };
    set_crel();

    // the tile at stream position pos: its piece's block id and valid tokens
    // (a position past the stream loads block 0 of KV head 0 and counts no tokens)
    auto issue = [&](T& tb, int& nv, int& lraw, uint32_t pos) {
        int id = 0, kvh = 0, lim = 0;
        bool real = false, shared = false;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            if (!real && pos < sl[k].p1) {
                const int off = int(pos - sl[k].p0);
                id = __builtin_amdgcn_readlane(sl[k].ids, off);
                kvh = sl[k].kvh;
                lim = sl[k].lim0 - off * kBlockTokens;
                shared = (piece_flags(sl[k]) & kReread) != 0;
                real = true;
            }
        }
        const bool ok = real && id >= 0 && id < a.num_blocks;
        nv = ok ? min(kBlockTokens, lim) : 0;
        lraw = lim;
        if (M != kModePlain && shared)
            load_tile<KV, D, false>(a, ok ? kvh : 0, ok ? id : 0, tb);
        else
            load_tile<KV, D, true>(a, ok ? kvh : 0, ok ? id : 0, tb);
    };

    __shared__ LdsState<NVC> held;  // merged state of the current run's finished partitions
    bool holding = false;
    int seen = -1;  // arrivals seen before the last piece of a cut run (see peek_arrivals)
    auto peek = [&]() {
        seen = -1;
        const int f = piece_flags(sl[0]);
        if ((f & kEndsPart) && !(f & kLocal))
            seen = peek_arrivals(a, unpack_contrib(sl[0].contrib), sw);
    };
    peek();

    // the piece in slot 0 is consumed: close its state as flagged, then move
    // the slots up, plan the next piece and load what it needs
    auto next_piece = [&]() {
        const int f = piece_flags(sl[0]);
        if (f & kClose) {
            const Cols cm = piece_cols(a, sl[0]);
            State<NVC> st;
            run_close(rs, st);
            if (holding) lds_merge_into(held, st);  // earlier partitions first
            if (!(f & kEndsPart)) {
                lds_put(held, st);  // a partition boundary inside the run
                holding = true;
            } else {
                holding = false;
                bool whole = (f & kLocal) != 0;
                if (!whole &&
                    merge_across<QT, D>(a, unpack_contrib(sl[0].contrib), sw, st, held, cm.hv, seen)) {
                    lds_get(held, st);
                    whole = true;
                }
                if (whole) {
                    if constexpr (M == kModeShared) {
                        if (piece_kind(sl[0]) == 1)
                            finish_prefix<QT, D>(a, cm, st);
                        else if (piece_kind(sl[0]) == 2)
                            finish_suffix<QT, D>(a, cm, st);
                        else
                            state_output<QT, D>(a, cm.row, st, cm.hv);
                    } else {
                        state_output<QT, D>(a, cm.row, st, cm.hv);
                    }
                }
            }
            run_reset(rs);  // a closed state is always followed by a new one
        }
        if (piece_flags(sl[1]) & kNewRun) {
#pragma unroll
            for (int q = 0; q < GE::NQ; ++q) qop[q] = qn[q];
        }
#pragma unroll
        for (int k = 0; k < NS - 1; ++k) sl[k] = sl[k + 1];
        plan(sl[NS - 1]);
        if (piece_flags(sl[1]) & kNewRun) {
            const Cols c1 = piece_cols(a, sl[1]);
            load_q<KV, D>(a, c1.row, c1.hv, qn);
        }
        set_crel();
        peek();
    };

    // ---- the tile stream: consume position t while position t + P - 1 loads ----
    T buf[P];
    int nvb[P];  // valid tokens of the buffered block (0: the block contributes nothing)
    int lrb[P];  // tokens of the context at and after the buffered block's first token
#pragma unroll
    for (int k = 0; k < P - 1; ++k) issue(buf[k], nvb[k], lrb[k], uint32_t(k));
    PKV_TL(unsigned long long tl[6] = {tl_entry, 0, 0, 0, 0, 0}; const uint32_t tl_n = hi - lo; int tl_k = 0;
           uint32_t tl_next = 1; unsigned long long tl_last = 0;)
    bool more = true;
    for (uint32_t t = 0; more; t += P) {
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const uint32_t tp = t + uint32_t(k);
            more = more && tp < sl[0].p1;
            if (more) {
                issue(buf[(k + P - 1) % P], nvb[(k + P - 1) % P], lrb[(k + P - 1) % P], tp + uint32_t(P - 1));
                consume_tile<KV, D, M == kModeMulti>(a, buf[k], nvb[k], lrb[k] + crel, qop, rs);
                PKV_TL(if (tp + 1 == tl_next && tl_k < 4) {
                    tl[1 + tl_k] = __builtin_amdgcn_s_memrealtime();
                    ++tl_k;
                    tl_next = max(tl_next + 1, uint32_t(uint64_t(tl_n) * uint32_t(tl_k) / 4));
                } if (tp + 1 == tl_n) tl_last = __builtin_amdgcn_s_memrealtime();)
                if (tp + 1 == sl[0].p1) next_piece();
            }
        }
    }
    PKV_TL({
        tl[5] = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            const uint32_t hwid = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_ID
            const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
            unsigned long long* o = g_timeline + uint64_t(w) * 8;
            for (int e = 0; e < 6; ++e) o[e] = tl[e];
            o[6] = uint64_t(hwid) | (uint64_t(xcc & 0xf) << 32) | (uint64_t(tl_n) << 40);
            o[7] = tl_last;
        }
    })
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

// Persistent waves one launch of this instance runs: its occupancy (one-wave
// workgroups per CU) times the CUs, at most kMaxWaves.
template <int KV, int D, int M>
int waves_t() {
    constexpr int P = Depth<KV, D>::P;
    static int waves_per_cu = 0;
    if (waves_per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, paged_decode_kernel<KV, D, P, M>, 64, 0) != hipSuccess ||
            n <= 0)
            n = 8;
        waves_per_cu = n;
    }
#ifdef PKV_MAX_WAVES_PER_CU
    waves_per_cu = waves_per_cu < PKV_MAX_WAVES_PER_CU ? waves_per_cu : PKV_MAX_WAVES_PER_CU;
#endif
    const int nwt = waves_per_cu * device_cus();
    return nwt < kMaxWaves ? nwt : kMaxWaves;
}

template <int KV, int D, int M>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int P = Depth<KV, D>::P;
    hipLaunchKernelGGL((paged_decode_kernel<KV, D, P, M>), dim3(waves_t<KV, D, M>()), dim3(64), 0, stream, a);
    return hipGetLastError();
}

// ---- tiled prefill: many new query tokens of one sequence against its context ----
//
// The same attention as the several-queries mode (a new token at position p
// sees positions 0..p of its sequence), in a shape for long chunks of new
// tokens: one wave owns kPrefillCols (32) query columns -- kPrefillCols / G
// consecutive new tokens times the G query heads of one KV head -- as two
// matrix-core column tiles, and walks the context once for all of them.
// Each K/V tile read feeds twice the matrix steps of a decode run, and waves
// holding neighbouring token tiles of one (sequence, KV head) are placed on
// one XCD so their context reads meet in its L2.  No split over the
// context: a wave keeps the softmax states of its columns to the end.
#ifndef PKV_PREFILL_NT
#define PKV_PREFILL_NT false
#endif
constexpr int kPrefillCols = kPrefillWaveCols;
constexpr int kPrefillTiles = kPrefillCols / 16;

// Two waves per SIMD (one for fp32 pools of head_dim 128, whose tiles and
// query operands are twice as large): the matrix steps of one wave overlap the
// softmax of the other.
template <int KV, int D>
constexpr int kPrefillWaves = (KV == kF32 && D == 128) ? 1 : 2;

template <int KV, int D, int P>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kPrefillWaves<KV, D>))) void paged_prefill_kernel(DecodeArgs a) {
    using GE = Geo<KV, D>;
    using T = Tile<KV, D>;
    constexpr int QT = (KV == kF32) ? kF32 : kBF16;
    constexpr int NVC = GE::NVC;
    constexpr int CT = kPrefillTiles;
    const int lane = lane_id(), col = lane & 15;
    const int G = a.group;
    const int tpw = kPrefillCols / G;  // new tokens per wave (columns past tpw * G hold none)
    // Work item: (pair, token tile), a pair being (sequence, KV head).
    // Workgroup w runs on XCD w mod 8 and is the (w / 8)-th item that XCD
    // receives.  XCD x takes pairs x, x + 8, x + 16, ... in turn, all token
    // tiles of a pair one after the other, so the waves reading one pair's
    // context share an L2, and the pairs (the heads of a sequence included)
    // are dealt round the XCDs rather than in contiguous ranges: XCDs given
    // the long sequences no longer run on after the others.  A pair's last
    // token tile, which sees the most context, goes first.
    const uint32_t ntt = uint32_t((a.max_q + tpw - 1) / tpw);
    const uint32_t k = blockIdx.x / 8;
    const uint32_t pair = blockIdx.x % 8 + 8 * (k / ntt);
    const int tt = int(ntt - 1 - k % ntt);
    if (pair >= uint32_t(a.num_seqs) * uint32_t(a.num_kv_heads)) return;
    const int kvh = int(pair % uint32_t(a.num_kv_heads));
    const int s = int(pair / uint32_t(a.num_kv_heads));
    const int L = clamped_len(a, s);
    const int q0 = a.cu_q[s];
    const int nq = min(max(a.cu_q[s + 1] - q0, 0), L);
    const int t0 = tt * tpw;
    if (t0 >= nq) return;
    const int tend = min(min(t0 + tpw, nq), a.max_q);  // tokens at index >= max_q are not computed
    const int ctx = L - nq + tend;  // positions the wave's last token sees
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;

    // columns: column tile c, lane column col -> token t0 + k / G, head kvh * G + k % G (k = 16 c + col)
    QOp<KV> qop[CT][GE::NQ];
    int vis[CT];      // positions this lane's column sees
    int64_t row[CT];  // its output row (query row * num_heads + head)
    bool hv[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const int k = 16 * c + col;
        const int tok = t0 + k / G;
        const bool ok = tok < tend && q0 >= 0 && int64_t(q0) + tok < int64_t(a.num_q_rows);
        hv[c] = ok;
        row[c] = (ok ? int64_t(q0) + tok : 0) * a.num_heads + kvh * G + k % G;
        vis[c] = ok ? L - nq + tok + 1 : ctx;
        load_q<KV, D>(a, row[c], ok, qop[c]);
    }
    Run<NVC> rs[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) run_reset(rs[c]);

    // block ids of the next 64 blocks to load (lane l: block jb + l), and of the 64 after them
    const int32_t* bt = a.block_table + int64_t(s) * a.max_blocks;
    int jb = 0;
    int ids = lane < nblk ? bt[lane] : -1;
    int idsn = 64 + lane < nblk ? bt[64 + lane] : -1;
    auto issue = [&](T& tb, int& nv, int j) {
        if (j - jb >= 64) {  // positions only grow: move to the next window
            jb += 64;
            ids = idsn;
            idsn = jb + 64 + lane < nblk ? bt[jb + 64 + lane] : -1;
        }
        const int id = j < nblk ? __builtin_amdgcn_readlane(ids, j - jb) : -1;
        const bool ok = id >= 0 && id < a.num_blocks;
        nv = ok ? min(kBlockTokens, L - j * kBlockTokens) : 0;
        load_tile<KV, D, PKV_PREFILL_NT>(a, ok ? kvh : 0, ok ? id : 0, tb);
    };
    T buf[P];
    int nvb[P];
#pragma unroll
    for (int k = 0; k < P - 1; ++k) issue(buf[k], nvb[k], k);
    for (int j = 0; j < nblk; j += P) {
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int jj = j + k;
            if (jj < nblk) {
                issue(buf[(k + P - 1) % P], nvb[(k + P - 1) % P], jj + P - 1);
                int upto[CT];
#pragma unroll
                for (int c = 0; c < CT; ++c) upto[c] = vis[c] - jj * kBlockTokens;
                consume_tiles<KV, D, CT, true>(a, buf[k], nvb[k], upto, qop, rs);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        State<NVC> st;
        run_close(rs[c], st);
        state_output<QT, D>(a, row[c], st, hv[c]);
    }
}

// ---- tiled prefill for 16- and 8-bit pools: two blocks per step on 32x32 matrix steps ----
//
// The columns of paged_prefill_kernel (a wave owns 32 / G new tokens of one
// (sequence, KV head), 32 query columns), with the scores of 32 context
// tokens (two blocks) per step held as one 32x32 tile S^T = K Q^T (tokens
// on rows, columns on columns) and the values taken with 32x32x16 steps,
// O^T += V^T P^T, so both products run at the matrix cores' full bf16 rate.
//
// Token order.  Row i of a step's score tile is block i / 16, token
// swap_quads(i % 16), where swap_quads exchanges tokens 4-7 and 8-11 of a
// block.  The output layout of a 32x32 step gives lane (column n, half h)
// rows 8b + 4h + r (b, r < 4); with this order those are tokens 8h .. 8h + 7
// of block 0 (registers 0-7) and of block 1 (registers 8-15).  That is
// exactly the operand a 32x32x16 value step takes from lane (n, h) for one
// block (its k index 8h + e), so the exponentiated scores feed the value
// products in place, and each lane's V operand is 8 consecutive tokens of
// one dimension row of the dimension-major V tile: one 16-byte load (bf16)
// or 8-byte load (fp8).
//
// Softmax per step: the raw scores' column maximum (in-lane, then lane
// n + 32), one fused multiply-add and one exponential per score with the
// scale folded in, bf16 packing, and the normaliser summed from the packed
// weights with a two-term dot product.  The running maximum that the
// weights are taken against is moved only when a column's maximum passes it
// by more than kLazyMax (base-2 units): weights then stay below 2^kLazyMax,
// far inside bf16 and fp32 range, and the accumulators are rescaled far
// less often; the normaliser is taken against the same reference, so the
// result is unchanged.
constexpr float kLazyMax = 8.0f;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swap_quads(int u) { return u ^ ((((u >> 2) ^ (u >> 3)) & 1) * 12); }

// x of this lane combined with x of lane ^ 32 (the other half of the same
// column), by the gfx950 swap of 32-lane halves (operands as in column_max).
__device__ __forceinline__ float halves_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int KV>
__device__ __forceinline__ bf16x8 widen8(const typename std::conditional<KV == kBF16, uint4, uint2>::type& x) {
    if constexpr (KV == kBF16) {
        return __builtin_bit_cast(bf16x8, x);
    } else {
        return fp8x8_to_bf16x8(x.x, x.y);
    }
}

// ---- the same prefill with K/V staged in LDS and shared by a workgroup of four waves ----
//
// A workgroup serves four consecutive token tiles (4 * 32 / G new tokens) of one (sequence, KV head); the
// waves walk the same context, so each stage's K and V tiles (kPfSub 32-token steps, two blocks each) are
// brought in once for all four: each wave copies a quarter of them straight into LDS (gfx950 load-to-LDS,
// 16 bytes per lane, no registers), and each wave reads its matrix operands from LDS.  Two LDS buffers
// alternate: stage s + 1's tiles are in flight while stage s is computed, and one barrier per stage
// separates the two uses of a buffer.  V tiles are copied permuted, so that lane (n, h)'s operand
// (dimension row n of a 32-row tile, tokens 8h .. 8h + 7) sits at 16 * lane within its 1 KiB
// (conflict-free reads); fp8 V tiles are copied as they are.
#ifndef PKV_PF_WAVES
#define PKV_PF_WAVES 4
#endif
#ifndef PKV_PF_SUB
#define PKV_PF_SUB 2
#endif
constexpr int kPfWaves = PKV_PF_WAVES;  // waves per workgroup
constexpr int kPfSub = PKV_PF_SUB;      // 32-token steps per LDS stage (one barrier per stage)

template <int KV, int D>
#ifndef PKV_PF_OCC
#define PKV_PF_OCC 2
#endif
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(PKV_PF_OCC))) void paged_prefill_lds_kernel(
    DecodeArgs a) {
    constexpr int ELT = KV == kBF16 ? 2 : 1;
    constexpr int TILE = kBlockTokens * D * ELT;  // one block of one KV head, bytes
    constexpr int NK = D / 16, NT = D / 32;
    constexpr int CHUNKS = TILE / 1024;           // 16-byte-per-lane copies per tile
    using KOp = typename std::conditional<KV == kBF16, uint4, uint2>::type;
    constexpr int NB = 2 * kPfSub;  // blocks per stage
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * NB * TILE];  // [buffer][K of NB blocks, V of NB blocks]
    const int wv = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5;
    const int G = a.group;
    const int tpw = 32 / G;          // new tokens per wave
    const int tpg = kPfWaves * tpw;  // ... per workgroup
    // work item: (pair, token group), pairs dealt round the XCDs, a pair's last group first
    const uint32_t ngrp = uint32_t((a.max_q + tpg - 1) / tpg);
    const uint32_t kq = blockIdx.x / 8;
    const uint32_t pair = blockIdx.x % 8 + 8 * (kq / ngrp);
    const int tg = int(ngrp - 1 - kq % ngrp);
    if (pair >= uint32_t(a.num_seqs) * uint32_t(a.num_kv_heads)) return;  // the whole workgroup
    const int kvh = int(pair % uint32_t(a.num_kv_heads));
    const int s = int(pair / uint32_t(a.num_kv_heads));
    const int L = clamped_len(a, s);
    const int q0 = a.cu_q[s];
    const int nq = min(max(a.cu_q[s + 1] - q0, 0), L);
    const int g0 = tg * tpg;
    if (g0 >= nq) return;  // the whole workgroup
    const int ctx = L - nq + min(min(g0 + tpg, nq), a.max_q);  // positions the group's last token sees
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int nstage = (nblk + NB - 1) / NB;
    // this wave's tokens (possibly none: it still copies its tiles and meets the barriers)
    const int t0 = g0 + wv * tpw;
    const int tend = min(min(t0 + tpw, nq), a.max_q);  // tokens at index >= max_q are not computed
    const int vis_min = L - nq + t0 + 1;
    const int tok = t0 + n / G;
    const bool hv = n < tpw * G && tok < tend && q0 >= 0 && int64_t(q0) + tok < int64_t(a.num_q_rows);
    const int64_t row = (hv ? int64_t(q0) + tok : 0) * a.num_heads + kvh * G + n % G;
    const int vis = hv ? L - nq + tok + 1 : 0;
    bf16x8 qop[NK];
    {
        const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + row * D * 2;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const uint4 x = hv ? *reinterpret_cast<const uint4*>(qrow + (16 * i + 8 * h) * 2) : make_uint4(0, 0, 0, 0);
            qop[i] = __builtin_bit_cast(bf16x8, x);
        }
    }
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float mref = kNegInf, thr = kNegInf, lsum = 0.0f;

    const int32_t* bt = a.block_table + int64_t(s) * a.max_blocks;
    auto table_entry = [&](int j) -> int { return j < nblk ? bt[j] : -1; };
    auto valid_tokens = [&](int j, int id) -> int {
        return (id >= 0 && id < a.num_blocks) ? min(kBlockTokens, L - j * kBlockTokens) : 0;
    };
    // The stage's 2 * NB tiles (K of its blocks, then V) are copied in 1 KiB pieces, PER consecutive
    // pieces per wave.  An absent block copies block 0 (its tokens are masked).
    constexpr int PIECES = 2 * NB * CHUNKS;
    constexpr int PER = (PIECES + kPfWaves - 1) / kPfWaves;  // pieces per wave, consecutive
    auto copy_tiles = [&](int buf, const int (&ent)[NB]) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int c = wv * PER + r;
            if (PIECES % kPfWaves != 0 && c >= PIECES) break;
            const int tile = c / CHUNKS, u = c % CHUNKS;
            const bool isv = tile >= NB;
            const int e = ent[isv ? tile - NB : tile];
            const int id = (e >= 0 && e < a.num_blocks) ? e : 0;
            const uint8_t* src = static_cast<const uint8_t*>(isv ? a.v_cache : a.k_cache) +
                                 (int64_t(id) * a.num_kv_heads + kvh) * TILE;
            int off = u * 1024 + lane * 16;
            if (KV == kBF16 && isv) off = (32 * u + n) * 32 + 16 * h;  // V: operand order
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src + off),
                                             reinterpret_cast<uint32_t*>(&lds[buf][tile * TILE + u * 1024]), 16, 0, 0);
        }
    };
    const int ktok = swap_quads(n & 15);
    const float cs = a.score_scale;
    const float inv_cs = 1.0f / cs;
    const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    int ent[NB], nxt[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) ent[b] = table_entry(b);
    copy_tiles(0, ent);
#pragma unroll
    for (int b = 0; b < NB; ++b) nxt[b] = table_entry(NB + b);
    for (int sg = 0; sg < nstage; ++sg) {
        const int buf = sg & 1;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of stage sg have landed ...
        __syncthreads();                // ... and everyone's; everyone is done with the other buffer
        if (sg + 1 < nstage) copy_tiles(buf ^ 1, nxt);
        int vt[NB];  // valid tokens of the stage's blocks
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            vt[b] = valid_tokens(NB * sg + b, ent[b]);
            ent[b] = nxt[b];
            nxt[b] = table_entry(NB * (sg + 2) + b);
        }
        // scores S^T = K Q^T of every step of the stage first (K operands from LDS), so that the matrix
        // cores work on the later steps' scores while the earlier steps' softmax runs
        f32x16 saccs[kPfSub];
#pragma unroll
        for (int sb = 0; sb < kPfSub; ++sb) saccs[sb] = f32x16{};
        // the steps' products interleaved, so that consecutive matrix steps use different accumulators
#pragma unroll
        for (int i = 0; i < NK; ++i) {
#pragma unroll
            for (int sb = 0; sb < kPfSub; ++sb) {
                const uint8_t* kt = &lds[buf][2 * sb * TILE] + (n < 16 ? 0 : TILE);
                bf16x8 kop;
                if constexpr (KV == kBF16)
                    kop = __builtin_bit_cast(bf16x8,
                                             *reinterpret_cast<const uint4*>(kt + ((2 * i + h) * kBlockTokens + ktok) * 16));
                else
                    kop = widen8<KV>(*reinterpret_cast<const uint2*>(kt + (i * kBlockTokens + ktok) * 16 + 8 * h));
                saccs[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[i], saccs[sb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int sb = 0; sb < kPfSub; ++sb) {
        const int st = kPfSub * sg + sb;
        const int nv0 = vt[2 * sb], nv1 = vt[2 * sb + 1];
        const uint8_t* vl = &lds[buf][(NB + 2 * sb) * TILE];
        const int k0 = 32 * st;
        f32x16& sacc = saccs[sb];
        // V operands of this step (masked below when tokens are absent)
        KOp vv[NT][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (KV == kBF16)
                    vv[t][b] = *reinterpret_cast<const uint4*>(vl + b * TILE + t * 1024 + lane * 16);
                else
                    vv[t][b] = *reinterpret_cast<const uint2*>(vl + b * TILE + ((32 * t + n) * kBlockTokens + 8 * h));
            }
        const bool whole = nv0 == kBlockTokens && nv1 == kBlockTokens && k0 + 32 <= vis_min;
        if (!whole) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tk = 8 * h + (i & 7);
                const int pos = k0 + 16 * (i >> 3) + tk;
                const bool ok = tk < (i < 8 ? nv0 : nv1) && pos < vis;
                sacc[i] = ok ? sacc[i] : kNegInf;
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int cnt = min(max((b == 0 ? nv0 : nv1) - 8 * h, 0), 8);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if constexpr (KV == kBF16) {
                        uint4& x = vv[t][b];
                        x.x = cnt >= 2 ? x.x : (cnt == 1 ? x.x & 0xffffu : 0u);
                        x.y = cnt >= 4 ? x.y : (cnt == 3 ? x.y & 0xffffu : 0u);
                        x.z = cnt >= 6 ? x.z : (cnt == 5 ? x.z & 0xffffu : 0u);
                        x.w = cnt >= 8 ? x.w : (cnt == 7 ? x.w & 0xffffu : 0u);
                    } else {
                        uint2& x = vv[t][b];
                        const uint32_t mlo = cnt >= 4 ? 0xffffffffu : (0xffffffffu >> (32 - 8 * cnt)) * (cnt > 0);
                        const uint32_t mhi = cnt >= 8 ? 0xffffffffu : cnt > 4 ? (0xffffffffu >> (32 - 8 * (cnt - 4))) : 0u;
                        x.x &= mlo;
                        x.y &= mhi;
                    }
                }
            }
        }
        // lazy reference (see the notes on the 32x32 steps above)
        bool over = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) over = over || sacc[i] > thr;
        if (__ballot(over)) {
            float bm = fmaxf(fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3])),
                             fmaxf(fmaxf(sacc[4], sacc[5]), fmaxf(sacc[6], sacc[7])));
            bm = fmaxf(bm, fmaxf(fmaxf(fmaxf(sacc[8], sacc[9]), fmaxf(sacc[10], sacc[11])),
                                 fmaxf(fmaxf(sacc[12], sacc[13]), fmaxf(sacc[14], sacc[15]))));
            bm = halves_max(bm);
            const float mnew = bm * cs;
            const bool move = mnew > mref + kLazyMax;
            const float mto = move ? mnew : mref;
            const float alpha = !move ? 1.0f : mref == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mref - mto);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] *= alpha;
            lsum *= alpha;
            mref = mto;
            thr = mto == kNegInf ? kNegInf : (mto + kLazyMax) * inv_cs;
        }
        const float mm = mref == kNegInf ? 0.0f : mref;
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pk[e] = pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * e], cs, -mm)),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * e + 1], cs, -mm)));
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), one2, lsum, false);
        const bf16x8 p0 = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        const bf16x8 p1 = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8<KV>(vv[t][0]), p0, acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8<KV>(vv[t][1]), p1, acc[t], 0, 0, 0);
        }
    }
    const float lt = halves_sum(lsum);
    if (!hv) return;
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    uint16_t* o = static_cast<uint16_t*>(a.out) + row * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            *reinterpret_cast<uint2*>(o + 32 * t + 8 * b + 4 * h) =
                make_uint2(pack_bf16(acc[t][4 * b] * inv, acc[t][4 * b + 1] * inv),
                           pack_bf16(acc[t][4 * b + 2] * inv, acc[t][4 * b + 3] * inv));
}

template <int KV, int D>
hipError_t launch_prefill_t(const DecodeArgs& a, int items, hipStream_t stream) {
    // three tiles in flight (two for fp32 pools of head_dim 128, tiles of 16 KiB): deeper buys nothing,
    // the wave is bound by its matrix and softmax steps
#ifdef PKV_PREFILL_DEPTH
    constexpr int P = PKV_PREFILL_DEPTH;
#else
    constexpr int P = (KV == kF32 && D == 128) ? 2 : 3;
#endif
    const int pairs = a.num_seqs * a.num_kv_heads;  // items = pairs * token tiles per pair
    if constexpr (KV == kF32) {
        const int grid = (pairs + 7) / 8 * 8 * (items / pairs);
        hipLaunchKernelGGL((paged_prefill_kernel<KV, D, P>), dim3(grid), dim3(64), 0, stream, a);
    } else {
        const int tpg = kPfWaves * (32 / a.group);
        const int grid = (pairs + 7) / 8 * 8 * ((a.max_q + tpg - 1) / tpg);
        hipLaunchKernelGGL((paged_prefill_lds_kernel<KV, D>), dim3(grid), dim3(64 * kPfWaves), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

// ---- shared-prefix decode, second pass: merge(prefix, suffix) of every covered row with suffix runs ----
//
// 32 threads per (sequence, head) row, each taking D / 32 consecutive dimensions.  A row's two states
// (m, l, acc) combine as M = max(m_p, m_s), out = v_scale * (2^(m_p - M) acc_p + 2^(m_s - M) acc_s) /
// (2^(m_p - M) l_p + 2^(m_s - M) l_s), a side without scores (m = -inf) weighing 0.  Which rows are covered
// is decided from the sharing arrays exactly as in the decode (seq_info), so each row is written once.
constexpr int kMergeRows = 8;  // rows per 256-thread workgroup

template <int QT, int D>
__global__ __launch_bounds__(32 * kMergeRows) void cascade_merge_kernel(DecodeArgs a) {
    constexpr int E = D / 32;  // dimensions per thread
    const int64_t row = int64_t(blockIdx.x) * kMergeRows + threadIdx.x / 32;
    const int t = threadIdx.x % 32;
    if (row >= int64_t(a.num_seqs) * a.num_heads) return;
    const int s = int(row / a.num_heads);
    // the two rows are read before the sharing arrays are (both are in bounds for any row), so that
    // their loads overlap the dependent reads that decide whether the row is merged at all
    // a row's first part: E f32 of acc (f32 queries) or E bf16 of acc / l (bf16 queries) per thread
    constexpr int EB = QT == kF32 ? 4 : 2;
    using VE = typename std::conditional<E * EB == 16, uint4, typename std::conditional<E * EB == 8, uint2, uint32_t>::type>::type;
    const int64_t rows = int64_t(a.num_seqs) * a.num_heads;
    const char* pb = reinterpret_cast<const char*>(a.pstate);
    const char* sb = reinterpret_cast<const char*>(a.sstate);
    const VE pv = *reinterpret_cast<const VE*>(pb + (row * D + E * t) * EB);
    const VE sv = *reinterpret_cast<const VE*>(sb + (row * D + E * t) * EB);
    const float2 pml = *reinterpret_cast<const float2*>(pb + rows * D * EB + 8 * row);
    const float2 sml = *reinterpret_cast<const float2*>(sb + rows * D * EB + 8 * row);
    const SeqInfo si = seq_info<kModeShared>(a, s);
    const int nb = (si.len + kBlockTokens - 1) / kBlockTokens;
    if (si.cl < 0 || nb <= si.pbe) return;  // not covered, or no suffix runs: written by the decode
    const float mp = pml.x, lp = pml.y, ms = sml.x, ls = sml.y;
    float pa[E], sa[E];
    if constexpr (QT == kF32) {
        __builtin_memcpy(pa, &pv, sizeof(pa));
        __builtin_memcpy(sa, &sv, sizeof(sa));
    } else {
        uint16_t ph[E], sh[E];
        __builtin_memcpy(ph, &pv, sizeof(ph));
        __builtin_memcpy(sh, &sv, sizeof(sh));
#pragma unroll
        for (int e = 0; e < E; ++e) {
            pa[e] = __uint_as_float(uint32_t(ph[e]) << 16);
            sa[e] = __uint_as_float(uint32_t(sh[e]) << 16);
        }
    }
    const float M = fmaxf(mp, ms);
    // the weight of each part: exp(m - M) times what its first part was divided by (1 for acc)
    const float wp = mp == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mp - M) * (QT == kF32 ? 1.0f : lp);
    const float ws = ms == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(ms - M) * (QT == kF32 ? 1.0f : ls);
    const float l = QT == kF32 ? lp * wp + ls * ws : wp + ws;
    const float inv = l > 0.0f ? a.v_scale / l : 0.0f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (pa[e] * wp + sa[e] * ws) * inv;
    if constexpr (QT == kF32) {
        float* out = static_cast<float*>(a.out) + row * D + E * t;
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = o[e];
    } else {  // positions E t .. E t + E - 1 of a bf16 row are E consecutive dimensions
        uint16_t* out = static_cast<uint16_t*>(a.out) + row * D + row_dim(E * t);
#pragma unroll
        for (int e = 0; e < E; e += 2) *reinterpret_cast<uint32_t*>(out + e) = pack_bf16(o[e], o[e + 1]);
    }
}

template <int M>
hipError_t launch_c(int cache_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
    if (cache_dtype == kF32 && head_dim == 64) return launch_t<kF32, 64, M>(a, stream);
    if (cache_dtype == kF32 && head_dim == 128) return launch_t<kF32, 128, M>(a, stream);
    if (cache_dtype == kBF16 && head_dim == 64) return launch_t<kBF16, 64, M>(a, stream);
    if (cache_dtype == kBF16 && head_dim == 128) return launch_t<kBF16, 128, M>(a, stream);
    if (cache_dtype == kFP8 && head_dim == 64) return launch_t<kFP8, 64, M>(a, stream);
    if (cache_dtype == kFP8 && head_dim == 128) return launch_t<kFP8, 128, M>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(int cache_dtype, int head_dim, const DecodeArgs& a, int items, hipStream_t stream) {
    if (items == 0) return hipSuccess;
    if (cache_dtype == kF32 && head_dim == 64) return launch_prefill_t<kF32, 64>(a, items, stream);
    if (cache_dtype == kF32 && head_dim == 128) return launch_prefill_t<kF32, 128>(a, items, stream);
    if (cache_dtype == kBF16 && head_dim == 64) return launch_prefill_t<kBF16, 64>(a, items, stream);
    if (cache_dtype == kBF16 && head_dim == 128) return launch_prefill_t<kBF16, 128>(a, items, stream);
    if (cache_dtype == kFP8 && head_dim == 64) return launch_prefill_t<kFP8, 64>(a, items, stream);
    if (cache_dtype == kFP8 && head_dim == 128) return launch_prefill_t<kFP8, 128>(a, items, stream);
    return hipErrorInvalidValue;
}

int decode_waves(int cache_dtype, int head_dim) {
    if (cache_dtype == kF32 && head_dim == 64) return waves_t<kF32, 64, kModePlain>();
    if (cache_dtype == kF32 && head_dim == 128) return waves_t<kF32, 128, kModePlain>();
    if (cache_dtype == kBF16 && head_dim == 64) return waves_t<kBF16, 64, kModePlain>();
    if (cache_dtype == kBF16 && head_dim == 128) return waves_t<kBF16, 128, kModePlain>();
    if (cache_dtype == kFP8 && head_dim == 64) return waves_t<kFP8, 64, kModePlain>();
    if (cache_dtype == kFP8 && head_dim == 128) return waves_t<kFP8, 128, kModePlain>();
    return kMaxWaves;
}

hipError_t launch_decode(int cache_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.cu_q) return launch_c<kModeMulti>(cache_dtype, head_dim, a, stream);
    if (a.prefix_leader) {
        const hipError_t e = launch_c<kModeShared>(cache_dtype, head_dim, a, stream);
        if (e != hipSuccess) return e;
        const int64_t rows = int64_t(a.num_seqs) * a.num_heads;
        const dim3 grid(uint32_t((rows + kMergeRows - 1) / kMergeRows));
        if (cache_dtype == kF32 && head_dim == 64) hipLaunchKernelGGL((cascade_merge_kernel<kF32, 64>), grid, dim3(256), 0, stream, a);
        else if (cache_dtype == kF32) hipLaunchKernelGGL((cascade_merge_kernel<kF32, 128>), grid, dim3(256), 0, stream, a);
        else if (head_dim == 64) hipLaunchKernelGGL((cascade_merge_kernel<kBF16, 64>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((cascade_merge_kernel<kBF16, 128>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    return launch_c<kModePlain>(cache_dtype, head_dim, a, stream);
}

}  // namespace pkv

// ---- static scratch of the no-allocation decode ----
//
// paged_attention_decode_noalloc runs the plain decode with its workspace
// (arrival counters, then the partial-state slots of the waves) in this
// file-scope device array instead of a caller's buffer.  Every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to a kernel.
namespace pkv {
namespace {

__device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(float** out, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
        // The counters must start at zero (every call that completes leaves them so): cleared once, by a
        // fill kernel on the first call's stream, ahead of that call's decode.
        hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                           int64_t(kSlotBase));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace pkv

#ifdef PKV_TIMELINE
// Instrumented library only: copy the first n_waves rows of eight words of the
// last decode call's timeline to host memory (after the call has finished).
extern "C" int pkv_timeline_read(unsigned long long* host, int n_waves) {
    if (!host || n_waves < 0 || n_waves > pkv::kMaxWaves) return 1;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(pkv::g_timeline), size_t(n_waves) * 64, 0, hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? 0
               : 2;
}

extern "C" int pkv_timeline_clear() {
    static unsigned long long zeros[pkv::kMaxWaves * 8];
    return hipMemcpyToSymbol(HIP_SYMBOL(pkv::g_timeline), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) ==
                   hipSuccess
               ? 0
               : 2;
}
#endif
