// vwc_kernels.hip -- gfx950 kernels for selected-token log-probabilities,
// entropy and the logit gradient.
//
// Method (web pages, cited by title and section):
//  * "fix: chunk target logprobs without tensor parallelism (long-context
//    OOM)", "Changes": forward = float32 logsumexp of each row plus a gather
//    of the target logit; backward = recompute the softmax and write
//    (onehot - softmax) * grad_output in the logits' dtype.
//  * "[megatron] feat: add memory-efficient chunked top-k KL computation",
//    "Design & Code Changes": the backward keeps the low-precision logits and
//    a per-token fp32 logZ and recomputes the probabilities from them.
//  * "feat: Reduce reference model memory with with parallel logprob
//    computation", "Implementation": per-shard max, per-shard sum of
//    exp(x - max), target logit from the owning shard, then one merge.  Here
//    the same merge joins the segments of one row inside one GPU, and the
//    vocabulary slices of the split-vocabulary entry points.
//
// Design for gfx950 (a bandwidth-bound streaming reduction, no MFMA):
//  * One 256-thread workgroup streams one segment (<= 128 KiB) of one row.
//    Consecutive lanes read consecutive 16-byte vectors, so every wave load
//    instruction covers 1 KiB of contiguous HBM; each lane keeps U loads in
//    flight.  The vectors start at the row's first 16-byte boundary; the few
//    elements before it and past the last whole vector go one per thread.
//  * Each lane keeps (K, s, w) in fp32 registers: K is a shift in log2
//    units, s = sum 2^u and w = sum 2^u * u with u = x * c - K, c = log2(e)/tau
//    (one FMA and one v_exp_f32 per element).  K only moves when a chunk's sum
//    would leave [1, 2^64] -- the first chunk, or a new maximum more than
//    44 nats above the current reference -- so the common path carries no
//    per-element max and no per-chunk rescale.  Every quantity is kept
//    relative to the K it was accumulated with, so the lag costs no accuracy.
//  * Lane states merge through DPP (quad_perm, row mirrors) and ds_swizzle
//    within the wave, then through LDS across the 4 waves, in a fixed order.
//  * Rows of 2-3 segments are reduced by one workgroup of 256 threads per
//    segment, whose partials merge in LDS; longer rows write one 16-byte
//    partial per segment and a second small kernel merges them.  Both merge
//    in segment order in fp64 with the same code (the pages' shard merge), so
//    the two shapes give the same bits.  The epilogue arithmetic (partials,
//    merge, log) is fp64, once per row.
//  * The backward streams each row once more: one 1024-thread workgroup per
//    segment reads 16-byte vectors and writes each one's gradient with one
//    non-temporal 16-byte store; rows without loss are written as +0.0
//    without being read.
#include <math.h>
#include <type_traits>
#include <stdint.h>

#include "vwc_internal.h"
#include "vwc_lane.h"

namespace vwc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr double kLog2e = 1.44269504088896340736;
// A chunk whose sum of 2^u exceeds this re-centres K (u > 64 means the logit
// is more than 64 * ln 2 = 44.4 nats above the reference).
constexpr float kChunkBound = 0x1p64f;
// In the slow path, entropy terms use max(u, -256) so a -inf logit adds
// 0 * (-256) = 0 to w instead of 0 * (-inf) = NaN; 2^-256 is 0 in fp32.
constexpr float kUFloor = -256.0f;

// Loads in flight per lane in the forward: the in-block shape (two 768-thread
// workgroups per compute unit, at most 80 VGPRs) holds 8; the one-workgroup-
// per-segment shape holds 16, so a 128 KiB bf16 segment streams in two rounds
// (145 VGPRs, three 256-thread workgroups per compute unit): 573 against
// 589 us on the default step's forward, A/B in one process.
#ifndef VWC_FWD_UNROLL
#define VWC_FWD_UNROLL 8
#endif
#ifndef VWC_FWD_UNROLL_SEG
#define VWC_FWD_UNROLL_SEG 16
#endif
#ifndef VWC_BWD_UNROLL
#define VWC_BWD_UNROLL 4
#endif
// Cache policy of the streaming loads/stores: non-temporal (1) or default (0).
#ifndef VWC_NT_LOAD
#define VWC_NT_LOAD 1
#endif
#ifndef VWC_NT_STORE
#define VWC_NT_STORE 1
#endif
// Optional occupancy attributes, e.g. __attribute__((amdgpu_waves_per_eu(8, 8))).
#ifndef VWC_FWD_ATTR
#define VWC_FWD_ATTR
#endif
#ifndef VWC_BWD_ATTR
#define VWC_BWD_ATTR
#endif
constexpr int kFwdU = VWC_FWD_UNROLL;
constexpr int kFwdUSeg = VWC_FWD_UNROLL_SEG;
constexpr int kBwdU = VWC_BWD_UNROLL;

template <class T>
__device__ __forceinline__ T stream_load(const T *p) {
#if VWC_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <class T>
__device__ __forceinline__ void stream_store(T v, T *p) {
#if VWC_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ float bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b); }

// Gradient vectors leave through buffer stores on a resource that spans the
// bytes one workgroup writes (a segment of a gradient row), with the cache
// policy bits of gfx950 (sc0 = 1, nt = 2, sc1 = 16).  Non-temporal at device
// scope (nt | sc1) ran the backward 0.9-1.7 % faster on MI355X (a copy probe
// of its traffic 2-3 %) than the non-temporal global store (nt alone), which
// __builtin_nontemporal_store emits; the stronger scope changes no result.
// VWC_BUF_STORE 0 keeps the global stores.
#ifndef VWC_BUF_STORE
#define VWC_BUF_STORE 1
#endif
#ifndef VWC_STORE_CPOL
#define VWC_STORE_CPOL 18
#endif

// A buffer resource over `bytes` bytes from `base` (raw, untyped access; the
// range check drops stores past the end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                             0x00020000);
}

// Where a vector store goes: byte voff (per lane) of the resource rs, which
// the global pointer dst also addresses.  The stores never take an SGPR
// offset: with one, the compiler lets the next VALU instruction overwrite the
// store's data registers at once, and on MI355X such 16-byte stores were seen
// to write a stale first dword in some lanes; with the offset field 0 it
// inserts the wait state.  A uniform part of the offset goes into the
// resource's base instead.
struct VecDst {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff;
    char *dst;
};

// One 16- or 8-byte vector store.
__device__ __forceinline__ void vec_store(u32x4 v, const VecDst &d) {
#if VWC_BUF_STORE
    __builtin_amdgcn_raw_buffer_store_b128(v, d.rs, static_cast<int>(d.voff), 0, VWC_STORE_CPOL);
#else
    stream_store(v, reinterpret_cast<u32x4 *>(d.dst));
#endif
}
__device__ __forceinline__ void vec_store(u32x2 v, const VecDst &d) {
#if VWC_BUF_STORE
    __builtin_amdgcn_raw_buffer_store_b64(v, d.rs, static_cast<int>(d.voff), 0, VWC_STORE_CPOL);
#else
    stream_store(v, reinterpret_cast<u32x2 *>(d.dst));
#endif
}

// ---------------------------------------------------------------- load units
// A load unit is a 16-byte vector (vector path) or one element (any layout).

template <int DT, bool VEC>
struct Unit;

template <>
struct Unit<VWC_BF16, true> {
    using T = u32x4;
    static constexpr int N = 8;
    static __device__ __forceinline__ T load(const T *p) { return stream_load(p); }
    // Element k of 8 bf16 packed little-endian in 4 dwords.
    static __device__ __forceinline__ float get(const T &v, int k) {
        uint32_t w = v[k >> 1];
        return bits_to_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

template <>
struct Unit<VWC_FP32, true> {
    using T = f32x4;
    static constexpr int N = 4;
    static __device__ __forceinline__ T load(const T *p) { return stream_load(p); }
    static __device__ __forceinline__ float get(const T &v, int k) { return v[k]; }
};

template <>
struct Unit<VWC_BF16, false> {
    using T = uint16_t;
    static constexpr int N = 1;
    static __device__ __forceinline__ T load(const T *p) { return *p; }
    static __device__ __forceinline__ float get(const T &v, int) {
        return bits_to_float(static_cast<uint32_t>(v) << 16);
    }
};

template <>
struct Unit<VWC_FP32, false> {
    using T = float;
    static constexpr int N = 1;
    static __device__ __forceinline__ T load(const T *p) { return *p; }
    static __device__ __forceinline__ float get(const T &v, int) { return v; }
};

template <int DT>
__device__ __forceinline__ float load_element(const char *row, int64_t j) {
    return Unit<DT, false>::get(reinterpret_cast<const typename Unit<DT, false>::T *>(row)[j], 0);
}

// Elements of a row before its first 16-byte boundary (the row starts on an
// element boundary), at most the row's length.
template <int64_t kE>
__device__ __forceinline__ int32_t row_head(const void *row, int32_t vocab) {
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row)) & 15u;
    return min(static_cast<int32_t>(((16u - mis) & 15u) / kE), vocab);
}

// Column of edge element `k` of a row whose whole vectors cover columns
// [head, head + body): the head columns first, then the tail past the body;
// -1 past the last edge element.
__device__ __forceinline__ int32_t edge_column(int32_t head, int32_t body, int32_t vocab,
                                               int32_t k) {
    if (k < head) return k;
    const int32_t j = head + body + (k - head);
    return j < vocab ? j : -1;
}

// Re-centre a lane on a chunk (units [0, nvalid) of v, still in registers)
// and return the chunk's (sum, w) relative to the new K.  Rare: a new maximum
// far above the reference, or NaN/-inf data.
template <int DT, bool VEC, int U, bool W>
__device__ __forceinline__ f32x2 recentre(const typename Unit<DT, VEC>::T (&v)[U], int nvalid,
                                          float c, Lane &L) {
    using Un = Unit<DT, VEC>;
    float cm = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        if (j < nvalid) {
#pragma unroll
            for (int k = 0; k < Un::N; ++k) {
                const float x = Un::get(v[j], k);
                cm = fmaxf(cm, x);
                nan |= (x != x);
            }
        }
    }
    const float Kn = cm * c;
    if (Kn > L.K) {
        if (L.s != 0.f) {  // move the mass seen so far (possibly NaN) onto Kn
            const float d = L.K - Kn;
            const float r = __builtin_amdgcn_exp2f(d);
            L.w = r * __builtin_fmaf(d, L.s, L.w);
            L.s = r * L.s;
        }
        L.K = Kn;
        L.m = cm;
    }
    if (L.K == -INFINITY) return f32x2{nan ? NAN : 0.f, 0.f};  // nothing finite yet
    float cs = 0.f, cw = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        if (j < nvalid) {
#pragma unroll
            for (int k = 0; k < Un::N; ++k) {
                const float u = __builtin_fmaf(Un::get(v[j], k), c, -L.K);
                const float e = __builtin_amdgcn_exp2f(u);
                cs += e;
                if (W) cw = __builtin_fmaf(e, fmaxf(u, kUFloor), cw);
            }
        }
    }
    return f32x2{cs, cw};
}

// Fold one chunk (U units per lane, the first `nvalid` valid) into the lane.
template <int DT, bool VEC, int U, bool W>
__device__ __forceinline__ void fold_chunk(const typename Unit<DT, VEC>::T (&v)[U], int nvalid,
                                           float c, Lane &L) {
    using Un = Unit<DT, VEC>;
    // A lane's first chunk seeds the shift with its first logit, so the common
    // case never enters the re-centre path (nor re-reads the chunk).  NaN and
    // -inf seeds are left to that path.
    if (L.K == -INFINITY) {
        const float x0 = Un::get(v[0], 0);
        if (x0 > -INFINITY) {
            L.m = x0;
            L.K = x0 * c;
        }
    }
    float s0 = 0.f, s1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        if (j < nvalid) {
#pragma unroll
            for (int k = 0; k < Un::N; ++k) {
                float u = __builtin_fmaf(Un::get(v[j], k), c, -L.K);
                float e = __builtin_amdgcn_exp2f(u);
                if (((j * Un::N + k) & 1) == 0) {
                    s0 += e;
                    if (W) w0 = __builtin_fmaf(e, u, w0);
                } else {
                    s1 += e;
                    if (W) w1 = __builtin_fmaf(e, u, w1);
                }
            }
        }
    }
    float cs = s0 + s1;
    float cw = w0 + w1;
    // Leave the fast path when the chunk needs a new shift, or when a -inf
    // logit made w NaN (2^-inf * -inf); the slow path clamps u for w.  NaN
    // logits also land there and stay NaN through s.
    if (!(cs <= kChunkBound) || (W && cw != cw)) {
        const f32x2 r = recentre<DT, VEC, U, W>(v, nvalid, c, L);
        cs = r[0];
        cw = r[1];
    }
    L.s += cs;
    if (W) L.w += cw;
}

// Stream units [u0, u1) of a row (thread `tid` of the segment's kFwdBlock
// threads takes u0 + tid, u0 + tid + kFwdBlock, ...).
// With prefetch on, the loads of chunk k+1 are issued before chunk k is folded,
// so each wave keeps loads in flight while its ALU work runs.
#ifndef VWC_FWD_PREFETCH
#define VWC_FWD_PREFETCH 0
#endif
template <int DT, bool VEC, int U, bool W>
__device__ __forceinline__ void stream_units(const char *row, int32_t u0, int32_t u1, float c,
                                             int32_t tid, Lane &L) {
    using Un = Unit<DT, VEC>;
    using T = typename Un::T;
    const T *p = reinterpret_cast<const T *>(row);
    int32_t b = u0 + tid;
#if VWC_FWD_PREFETCH
    if (b + (U - 1) * kFwdBlock < u1) {
        T cur[U];
#pragma unroll
        for (int j = 0; j < U; ++j) cur[j] = Un::load(p + b + j * kFwdBlock);
        for (;;) {
            const int32_t nb = b + U * kFwdBlock;
            const bool more = nb + (U - 1) * kFwdBlock < u1;
            T nxt[U];
            if (more) {
#pragma unroll
                for (int j = 0; j < U; ++j) nxt[j] = Un::load(p + nb + j * kFwdBlock);
            }
            fold_chunk<DT, VEC, U, W>(cur, U, c, L);
            b = nb;
            if (!more) break;
#pragma unroll
            for (int j = 0; j < U; ++j) cur[j] = nxt[j];
        }
    }
#else
    for (; b + (U - 1) * kFwdBlock < u1; b += U * kFwdBlock) {
        T v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = Un::load(p + b + j * kFwdBlock);
        fold_chunk<DT, VEC, U, W>(v, U, c, L);
    }
#endif
    if (b < u1) {
        T v[U];
        int nv = 0;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            v[j] = T{};
            if (b + j * kFwdBlock < u1) {
                v[j] = Un::load(p + b + j * kFwdBlock);
                nv = j + 1;
            }
        }
        fold_chunk<DT, VEC, U, W>(v, nv, c, L);
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return bits_to_float(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(__builtin_bit_cast(uint32_t, v)), CTRL, 0xf, 0xf, false)));
}

template <int PATTERN>
__device__ __forceinline__ float swz(float v) {
    return bits_to_float(static_cast<uint32_t>(
        __builtin_amdgcn_ds_swizzle(static_cast<int>(__builtin_bit_cast(uint32_t, v)), PATTERN)));
}

template <int CTRL>
__device__ __forceinline__ void wave_step_dpp(Lane &L) {
    Lane o{dpp<CTRL>(L.K), dpp<CTRL>(L.m), dpp<CTRL>(L.s), dpp<CTRL>(L.w)};
    merge(L, o);
}

template <int PATTERN>
__device__ __forceinline__ void wave_step_swz(Lane &L) {
    Lane o{swz<PATTERN>(L.K), swz<PATTERN>(L.m), swz<PATTERN>(L.s), swz<PATTERN>(L.w)};
    merge(L, o);
}

// Reduce the lane states of each group of kFwdBlock threads of a workgroup
// (NG groups at most; `grp` is the caller's group); every thread of a group
// gets its group's state.
template <int NG>
__device__ __forceinline__ Lane block_reduce(Lane L, int grp) {
    // Within a wave: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
    // row_mirror (all lanes of a row of 16 then hold the row's state), then a
    // swizzle exchanging rows 0<->1 and 2<->3 (xor 16 inside each 32-lane half).
    wave_step_dpp<0xB1>(L);
    wave_step_dpp<0x4E>(L);
    wave_step_dpp<0x141>(L);
    wave_step_dpp<0x140>(L);
    wave_step_swz<0x401F>(L);
    // Lanes 0 and 32 now hold the two halves.
    Lane hi{bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.K), 32)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.m), 32)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.s), 32)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.w), 32))};
    Lane lo{bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.K), 0)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.m), 0)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.s), 0)),
            bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, L.w), 0))};
    merge(lo, hi);
    constexpr int kW = kFwdBlock / 64;
    __shared__ Lane wave_state[NG * kW];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wave_state[wave] = lo;
    __syncthreads();
    const Lane *g = wave_state + grp * kW;
    Lane acc = g[0];
#pragma unroll
    for (int q = 1; q < kW; ++q) merge(acc, g[q]);
    return acc;
}

// Lane states of a whole wave reduced the cheap way: the largest shift K and
// reference m first (maxima through DPP and ds_swizzle; K = fl(m c) is monotone
// in m, so the two maxima belong together), then every lane's sums rescaled to
// that K and added over the same exchange tree.  Empty lanes (s = 0) add 0; NaN
// sums propagate.  Every lane gets the wave's state.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) { return fmaxf(v, dpp<CTRL>(v)); }
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) { return v + dpp<CTRL>(v); }

__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xB1>(v);
    v = dpp_max<0x4E>(v);
    v = dpp_max<0x141>(v);
    v = dpp_max<0x140>(v);
    v = fmaxf(v, swz<0x401F>(v));
    return fmaxf(bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)),
                 bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x141>(v);
    v = dpp_add<0x140>(v);
    v = v + swz<0x401F>(v);
    return bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
           bits_to_float(__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
}

__device__ __forceinline__ Lane wave_reduce_rescaled(const Lane &L) {
    Lane o;
    o.K = wave_max(L.K);
    o.m = wave_max(L.m);
    const float d = L.K - o.K;  // <= 0
    const float r = __builtin_amdgcn_exp2f(d);
    const bool has = L.s != 0.f;  // true for NaN too
    o.s = wave_sum(has ? r * L.s : 0.f);
    o.w = wave_sum(has ? r * __builtin_fmaf(d, L.s, L.w) : 0.f);
    return o;
}

// Merge partials in order (formulas in the vwc_partial comment).
struct Merged {
    double M, S, W, T;
};

// Two passes, slices in order: the global reference first (the pages' MAX
// step), then the rescaled sums (their SUM steps).  `at(q)` yields partial q.
template <class At>
__device__ __forceinline__ Merged merge_partials(At at, int k, double tau) {
    double M = -INFINITY;
    for (int q = 0; q < k; ++q) {
        const P64 v = at(q);
        if (v.s != 0.0 && v.m > M) M = v.m;
    }
    double S = 0.0, W = 0.0, T = -INFINITY;
    bool tnan = false;
    for (int q = 0; q < k; ++q) {
        const P64 v = at(q);
        if (v.t != v.t)
            tnan = true;
        else if (v.t > T)
            T = v.t;
        if (v.s != 0.0) {  // empty slices add nothing; NaN partials poison S
            const double d = (v.m - M) / tau;
            const double f = exp(d);
            S += v.s * f;
            W += f * (v.w + d * v.s);
        }
    }
    return Merged{M, S, W, tnan ? NAN : T};
}

__device__ __forceinline__ void write_final(const Merged &g, double tau, int64_t i, float *logprob,
                                            float *lse, float *entropy) {
    const double lnS = log(g.S);
    if (lse) lse[i] = static_cast<float>(g.M / tau + lnS);
    if (logprob) logprob[i] = static_cast<float>((g.T - g.M) / tau - lnS);
    if (entropy) entropy[i] = static_cast<float>(lnS - g.W / g.S);
}

__device__ __forceinline__ vwc_partial to_f32(const Merged &g) {
    return vwc_partial{static_cast<float>(g.M), static_cast<float>(g.S), static_cast<float>(g.T),
                       static_cast<float>(g.W)};
}

// ---------------------------------------------------------------- forward

// A row of nseg segments, each reduced by kFwdBlock threads into one partial.
// Two launch shapes give the same bits:
//   INBLOCK = false: one workgroup per (row, segment); with nseg > 1 the
//     partials go to the workspace ([nseg][m]) and combine_kernel merges them;
//   INBLOCK = true (2 <= nseg <= kFwdMaxSegPerBlock): one workgroup of
//     nseg * kFwdBlock threads per row; group q reduces segment q, the groups'
//     fp32 partials meet in LDS and thread 0 merges them with the combine's
//     own code, in segment order.  No workspace, no second launch.
// The in-block kernel asks the compiler for few enough registers that this many
// waves share a SIMD (6: two workgroups of three segments per compute unit).
#ifndef VWC_FWD_INBLOCK_WAVES
#define VWC_FWD_INBLOCK_WAVES 6
#endif
template <int DT, bool VEC, bool W, bool INBLOCK>
__global__ __launch_bounds__(INBLOCK ? kFwdBlock * kFwdMaxSegPerBlock : kFwdBlock,
                              INBLOCK ? VWC_FWD_INBLOCK_WAVES : 1) VWC_FWD_ATTR
    void fwd_segment_kernel(FwdPlan p) {
    using Un = Unit<DT, VEC>;
    constexpr int64_t kE = DT == VWC_BF16 ? 2 : 4;
    const int32_t tid = static_cast<int32_t>(threadIdx.x) & (kFwdBlock - 1);
    const int grp = INBLOCK ? static_cast<int>(threadIdx.x) / kFwdBlock : 0;
    const int64_t i = INBLOCK ? static_cast<int64_t>(blockIdx.x)
                              : static_cast<int64_t>(blockIdx.x) / p.nseg;
    const int q = INBLOCK ? grp : static_cast<int>(blockIdx.x - i * p.nseg);
    const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
    const bool bad = r < 0 || r >= p.n_rows;  // row id outside the tensor: NaN, no reads
    if (!INBLOCK && bad) {
        if (threadIdx.x == 0) {
            const vwc_partial nan4{NAN, NAN, NAN, NAN};
            if (p.nseg > 1)
                p.seg_part[static_cast<int64_t>(q) * p.m + i] = nan4;
            else if (p.partial_out)
                p.partial_out[i] = nan4;
            else {
                if (p.logprob && p.target_mode != kTargetNone) p.logprob[i] = NAN;
                if (p.lse) p.lse[i] = NAN;
                if (p.entropy) p.entropy[i] = NAN;
            }
        }
        return;
    }

    vwc_partial mine{NAN, NAN, NAN, NAN};
    if (!bad) {  // uniform over the workgroup
        const char *row = static_cast<const char *>(p.logits) + r * p.ld * kE;
        // The whole vectors start at the row's first 16-byte boundary, `head`
        // elements in (0 when the row starts on one); the elements before it
        // and past the last whole vector are the row's edges.
        const int32_t head = VEC ? row_head<kE>(row, p.vocab) : 0;
        const int32_t nunits = (p.vocab - head) / Un::N;
        const int32_t u0 = q * p.seg_units;
        const int32_t u1 = min(u0 + p.seg_units, nunits);
        const bool last = q == p.nseg - 1;

        Lane L = lane_init();
        if (u0 < u1)
            stream_units<DT, VEC, INBLOCK ? kFwdU : kFwdUSeg, W>(row + head * kE, u0, u1, p.c, tid, L);
        if (VEC && last) {  // the edge elements, one per thread
            const int32_t j = edge_column(head, nunits * Un::N, p.vocab, tid);
            if (j >= 0) {
                using Us = Unit<DT, false>;
                typename Us::T v[1];
                v[0] = reinterpret_cast<const typename Us::T *>(row)[j];
                fold_chunk<DT, false, 1, W>(v, 1, p.c, L);
            }
        }
        const Lane B = block_reduce<INBLOCK ? kFwdMaxSegPerBlock : 1>(L, grp);
        if (!INBLOCK && threadIdx.x != 0) return;

        if (tid == 0) {
            // Target logit from the segment that owns its column.
            double t = -INFINITY;
            if (p.target_mode != kTargetNone) {
                const int64_t tl = static_cast<int64_t>(p.targets[r]) - p.v_start;
                const int64_t span = static_cast<int64_t>(p.seg_units) * Un::N;
                const bool in_range = tl >= 0 && tl < p.vocab;
                if (in_range) {
                    const int64_t owner = min(tl / span, static_cast<int64_t>(p.nseg - 1));
                    if (owner == q) t = load_element<DT>(row, tl);
                } else if (p.target_mode == kTargetFull && q == 0) {
                    t = NAN;
                }
            }
            const P64 part = to_partial(B, p.c, t);
            if (!INBLOCK && p.nseg == 1 && !p.partial_out) {
                const Merged g = merge_partials([&](int) { return part; }, 1, p.tau);
                write_final(g, p.tau, i, p.target_mode == kTargetNone ? nullptr : p.logprob,
                            p.lse, p.entropy);
                return;
            }
            mine = vwc_partial{static_cast<float>(part.m), static_cast<float>(part.s),
                               static_cast<float>(part.t), static_cast<float>(part.w)};
        }
    }

    if (!INBLOCK) {  // thread 0 of a (row, segment) workgroup
        if (p.nseg > 1)
            p.seg_part[static_cast<int64_t>(q) * p.m + i] = mine;
        else
            p.partial_out[i] = mine;
        return;
    }
    __shared__ vwc_partial seg_parts[kFwdMaxSegPerBlock];
    if (tid == 0) seg_parts[grp] = mine;
    __syncthreads();
    if (threadIdx.x != 0) return;
    const Merged g = merge_partials(
        [&](int k) {
            const vwc_partial v = seg_parts[k];
            return P64{v.m, v.s, v.t, v.w};
        },
        p.nseg, p.tau);
    if (p.partial_out)
        p.partial_out[i] = to_f32(g);
    else
        write_final(g, p.tau, i, p.target_mode == kTargetNone ? nullptr : p.logprob, p.lse,
                    p.entropy);
}

// One thread per row: merge k partials ([k][stride]) in slice order.
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(CombinePlan p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kCombineBlock + threadIdx.x;
    if (i >= p.rows) return;
    const vwc_partial *base = p.parts + i;
    const int64_t stride = p.stride;
    const Merged g = merge_partials(
        [=](int q) {
            const vwc_partial v = base[static_cast<int64_t>(q) * stride];
            return P64{v.m, v.s, v.t, v.w};
        },
        p.k, p.tau);
    if (p.partial_out)
        p.partial_out[i] = to_f32(g);
    else
        write_final(g, p.tau, i, p.logprob, p.lse, p.entropy);
}

// One wave per row: merge k partials stored row-major ([rows][k], so a row's
// partials are contiguous).  Each lane folds partials lane, lane + 64, ...
// into a running fp64 (M, S, W) (rescaled whenever its reference rises), then
// the 64 lane states merge over a fixed xor tree.  Used for rows with many
// segments (the fused LM head), where one thread per row would serialise.
constexpr int kCombineRowsBlock = 256;

__device__ __forceinline__ void merge64(double &M, double &S, double &W, double m, double s,
                                        double w, double tau) {
    if (!(s != 0.0)) return;  // empty (NaN states are not empty and poison S)
    if (m > M) {
        if (S != 0.0) {
            const double d = (M - m) / tau;
            const double f = exp(d);
            W = f * (W + d * S);
            S = f * S;
        }
        M = m;
    }
    const double d = (m - M) / tau;
    const double f = exp(d);
    S += s * f;
    W += f * (w + d * s);
}

__global__ __launch_bounds__(kCombineRowsBlock) void combine_rows_kernel(CombinePlan p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * (kCombineRowsBlock / 64) +
                      (threadIdx.x >> 6);
    if (i >= p.rows) return;  // whole waves
    const int lane = threadIdx.x & 63;
    const vwc_partial *row = p.parts + i * p.k;
    double M = -INFINITY, S = 0.0, W = 0.0, T = -INFINITY;
    bool tnan = false;
    for (int q = lane; q < p.k; q += 64) {
        const vwc_partial v = row[q];
        if (v.t != v.t)
            tnan = true;
        else if (v.t > T)
            T = v.t;
        merge64(M, S, W, v.m, v.s, v.w, p.tau);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double m = __shfl_xor(M, off), s = __shfl_xor(S, off), w = __shfl_xor(W, off);
        const double t = __shfl_xor(T, off);
        tnan |= __shfl_xor(static_cast<int>(tnan), off) != 0;
        // Lane pairs merge in the same (lower-lane-first) order on both sides.
        double Ma = M, Sa = S, Wa = W;
        double Mb = m, Sb = s, Wb = w;
        if (lane & off) {
            Ma = m; Sa = s; Wa = w;
            Mb = M; Sb = S; Wb = W;
        }
        merge64(Ma, Sa, Wa, Mb, Sb, Wb, p.tau);
        M = Ma;
        S = Sa;
        W = Wa;
        if (t > T) T = t;
    }
    if (lane != 0) return;
    // An all-empty row keeps M = -inf and S = 0 (outputs -inf / NaN as in the
    // per-thread merge).
    const Merged g{M, S, W, tnan ? NAN : T};
    write_final(g, p.tau, i, p.logprob, p.lse, p.entropy);
}

// ---------------------------------------------------------------- backward

template <int GDT, int N>
struct GradStore;

// N gradients to bf16 (round to nearest-even through v_cvt_pk_bf16_f32) or fp32.
template <int N>
struct GradStore<VWC_BF16, N> {
    static __device__ __forceinline__ void store(char *dst, const float (&o)[N]) {
        if constexpr (N == 1) {
            const bf16x2 b = __builtin_convertvector((f32x2{o[0], 0.f}), bf16x2);
            *reinterpret_cast<uint16_t *>(dst) =
                static_cast<uint16_t>(__builtin_bit_cast(uint32_t, b) & 0xffffu);
        } else {
            uint32_t packed[N / 2];
#pragma unroll
            for (int k = 0; k < N / 2; ++k) {
                const bf16x2 b = __builtin_convertvector((f32x2{o[2 * k], o[2 * k + 1]}), bf16x2);
                packed[k] = __builtin_bit_cast(uint32_t, b);
            }
            if constexpr (N == 8)
                stream_store(u32x4{packed[0], packed[1], packed[2], packed[3]},
                                            reinterpret_cast<u32x4 *>(dst));
            else
                stream_store(u32x2{packed[0], packed[1]},
                                            reinterpret_cast<u32x2 *>(dst));
        }
    }
    // The same vector (N > 1) at d.
    static __device__ __forceinline__ void store(const VecDst &d, const float (&o)[N]) {
        static_assert(N == 4 || N == 8, "vector units");
        uint32_t packed[N / 2];
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const bf16x2 b = __builtin_convertvector((f32x2{o[2 * k], o[2 * k + 1]}), bf16x2);
            packed[k] = __builtin_bit_cast(uint32_t, b);
        }
        if constexpr (N == 8)
            vec_store(u32x4{packed[0], packed[1], packed[2], packed[3]}, d);
        else
            vec_store(u32x2{packed[0], packed[1]}, d);
    }
};

template <int N>
struct GradStore<VWC_FP32, N> {
    static __device__ __forceinline__ void store(char *dst, const float (&o)[N]) {
        if constexpr (N == 1) {
            *reinterpret_cast<float *>(dst) = o[0];
        } else {
#pragma unroll
            for (int k = 0; k < N; k += 4)
                stream_store(f32x4{o[k], o[k + 1], o[k + 2], o[k + 3]},
                                            reinterpret_cast<f32x4 *>(dst + 4 * k));
        }
    }
    static __device__ __forceinline__ void store(const VecDst &d, const float (&o)[N]) {
        static_assert(N == 4 || N == 8, "vector units");
#pragma unroll
        for (int k = 0; k < N; k += 4)
            vec_store(__builtin_bit_cast(u32x4, (f32x4{o[k], o[k + 1], o[k + 2], o[k + 3]})),
                      VecDst{d.rs, d.voff + 4u * k, d.dst + 4 * k});
    }
};

// Top-k KL gradient per row, with p_tail = max(0, 1 - P) and q_tail = 1 - Q:
//   dL/dz_j = alpha q_j              for j outside the payload,
//           = beta q_j - kappa p_j   for j in it,
// tail (guard off): alpha = P - p_tail Q / q_tail, beta = P + p_tail, kappa = 1
// (q - p inside, q (P - Q)/(1 - Q) outside when P < 1); tail with the eps guard
// on, or truncated: alpha = beta = P; a truncated row whose sum S < 0 was
// clamped and has no gradient.
struct KlCoef {
    double alpha, beta, kappa;
    bool dead;
};

__device__ __forceinline__ KlCoef kl_coef(int mode, double eps, double P, double Q, double S) {
    KlCoef c{P, P, 1.0, false};
    if (mode == VWC_KL_TRUNCATED) {
        c.dead = S < 0.0;
    } else {
        const double pt = P < 1.0 ? 1.0 - P : 0.0;
        const double qt = 1.0 - Q;
        if (qt >= eps) {
            c.alpha = P - pt * Q / qt;
            c.beta = P + pt;
        }
    }
    return c;
}

// Gradient of payload column n of a row whose student logit is x:
// (beta q - kappa p_n) g / tau with q = exp(x / tau - lse), p_n = exp(a_n), in
// fp64 (the two terms cancel when the student matches the teacher).
__device__ __forceinline__ float kl_payload_value(double q, double pn, double gt, double beta,
                                                  double kappa) {
    return static_cast<float>(gt * (beta * q - kappa * pn));
}

__device__ __forceinline__ float kl_payload_grad(double x, double tau, double lse, double gt,
                                                 const KlCoef &c, float tlp) {
    const double q = exp(x / tau - lse);
    const double pn = exp(static_cast<double>(tlp));
    return kl_payload_value(q, pn, gt, c.beta, c.kappa);
}

// The payload columns of one backward segment, in LDS.  An open-addressing
// table keyed by the segment-relative 16-byte unit (the row's tail past its
// last whole vector has a key of its own) holds which columns of the unit are
// payload columns and their final gradients; the streaming pass overwrites
// those lanes of the unit before its one store.  A per-thread mask marks the
// thread's units that have an entry (bit `it`: unit u0 + thread + it * kBwdBlock),
// so the common unit costs one bit test.
struct KlSlot {
    int32_t unit;   // -1: empty
    uint32_t cols;  // bit k: column k of the unit is a payload column
    float val[8];   // its gradient
};
constexpr int32_t kKlTailKey = 0x7fffffff;

__device__ __forceinline__ uint32_t kl_hash(int32_t key) {
    return (static_cast<uint32_t>(key) * 0x9E3779B1u) >> 23;  // 9 bits: kKlSlots = 512
}
static_assert(kKlSlots == 512, "kl_hash yields 9 bits");

// Slot of `key`, or -1 when it is absent (a probe ends at an empty slot; the
// table is at most half full).
__device__ __forceinline__ int kl_find(const KlSlot *tab, int32_t key) {
    uint32_t h = kl_hash(key);
    for (int probe = 0; probe < kKlSlots; ++probe) {
        const int32_t u = tab[h].unit;
        if (u == key) return static_cast<int>(h);
        if (u == -1) return -1;
        h = (h + 1) & (kKlSlots - 1);
    }
    return -1;
}

template <int N>
__device__ __forceinline__ void kl_patch(const KlSlot *tab, int32_t key, float (&o)[N]) {
    const int h = kl_find(tab, key);
    if (h < 0) return;
    const uint32_t cols = tab[h].cols;
#pragma unroll
    for (int k = 0; k < N; ++k)
        if ((cols >> k) & 1u) o[k] = tab[h].val[k];
}

// Uniform per-row constants of the backward.
struct RowGrad {
    float c_hi, c_lo;  // log2(e) / tau as a float pair
    float B;       // lse * log2(e), the float nearest to its fp64 value
    float gs;      // 2^-B_lo times the factor of p: -g / tau (top-k KL: alpha g / tau)
    float a, b;    // entropy gradient: o = p' (a + b u'), both times 2^-B_lo
    double gt;     // g / tau
    double hs;     // -h / tau
    double H;      // the saved entropy, widened
    double lse;    // the saved logZ, widened
    double tau;
    int32_t t;     // target column (-1: no logprob term)
};

// Row constants from the saved fp32 lse.  The probability is
// p_j = 2^(x_j c - B) with c = log2(e)/tau and B = lse log2(e).  Held as single
// floats, c and B would move the exponent by |x| ulp(c)/2 + ulp(B)/2, which is
// several 1e-6 at |lse| of 16 to 64 and becomes the same absolute error in a
// gradient where p_j -> 1.  So the kernel computes u' = (x c_hi - B_hi) + x c_lo
// = x c - B + B_lo, accurate to about ulp(u'), and the factor 2^-B_lo that
// p' = 2^u' carries in excess goes into the per-row factors, once per row in
// fp64.  `coef` is the factor of p before that: -g/tau, or alpha g/tau.
__device__ __forceinline__ RowGrad row_grad(float c_hi, float c_lo, double tau, float lse,
                                            float g, float h, double H, double coef) {
    RowGrad R;
    R.c_hi = c_hi;
    R.c_lo = c_lo;
    R.tau = tau;
    R.gt = static_cast<double>(g) / tau;
    R.lse = static_cast<double>(lse);
    const double B = R.lse * kLog2e;
    R.B = static_cast<float>(B);
    // Non-finite lse: no split (u' = x c - B as before, inf / NaN propagate).
    const double B_lo = isfinite(R.B) ? B - static_cast<double>(R.B) : 0.0;
    const double f = exp2(-B_lo);
    R.hs = -static_cast<double>(h) / tau;
    R.H = H;
    R.gs = static_cast<float>(coef * f);
    // o = p (a + b u) with u = u' - B_lo, a = -(g + h H)/tau, b = -h ln2/tau.
    const double a = -R.gt + R.hs * H, b = R.hs * kLn2;
    R.a = static_cast<float>(f * (a - b * B_lo));
    R.b = static_cast<float>(f * b);
    R.t = -1;
    return R;
}

// Whether a row's exponent needs the float pair.  An fp32 gradient always
// does.  A bf16 gradient is rounded to 8 bits, and dropping x c_lo moves
// u' by at most |x| c_lo < |x| c 2^-23; every element above 2^-126 has
// |x| c <= |B| + 126, so for |B| < 4096 that is below 3.5e-4 relative in p,
// a tenth of a bf16 step: such rows take x c_hi - B alone (one FMA less per
// element), others (and non-finite B) keep the pair.
__device__ __forceinline__ bool exponent_pair(bool fp32_grad, float B) {
    return fp32_grad || !(fabsf(B) < 4096.f);
}

// Gradient of one unit.  Logprob only: o_k = gs p'_k with p'_k = 2^u'_k.
// With the entropy term (WH):
//   o_k = p_k (-g/tau - h/tau (z_k - lse + H)) = p'_k (a + b u'_k).
// The target column adds g/tau (1 - p_t), computed as -expm1(x_t/tau - lse) in
// fp64 so that p_t -> 1 does not cancel.
// v_exp_f32 flushes results below 2^-126, which exp2f rescales at five more
// instructions per element.  EXP picks how p' is evaluated:
//   kExpRescale: exp2f everywhere;
//   kExpPerUnit: a unit whose exponents all lie at or above -126 (nearly every
//     unit) takes the bare instruction, which gives exp2f's bits there, and a
//     unit with a smaller one (or NaN) takes exp2f: the same results for fewer
//     VALU cycles, at the cost of a branch per unit;
//   kExpBare: the caller has shown that every exponent lies at or above -126.
// The streaming backward, bound by memory, runs fastest with kExpRescale; the
// one-call kernel, whose compute phases run between its memory phases, decides
// once per thread.  PAIR: the exponent with the float pair (x c_hi - B) + x c_lo,
// else x c_hi - B alone (see exponent_pair).  TGT: add the target column's
// one-hot term here (callers that write that element themselves pass false).
constexpr int kExpRescale = 0, kExpPerUnit = 1, kExpBare = 2;

template <int DT, bool VEC, bool WH, int EXP = kExpRescale, bool PAIR = true, bool TGT = true>
__device__ __forceinline__ void unit_grad(const typename Unit<DT, VEC>::T &v, int32_t col0,
                                          const RowGrad &R, float (&o)[Unit<DT, VEC>::N]) {
    using Un = Unit<DT, VEC>;
    float u[Un::N];
#pragma unroll
    for (int k = 0; k < Un::N; ++k) {
        const float x = Un::get(v, k);
        u[k] = PAIR ? __builtin_fmaf(x, R.c_lo, __builtin_fmaf(x, R.c_hi, -R.B))
                    : __builtin_fmaf(x, R.c_hi, -R.B);
    }
    float umin = u[0];
#pragma unroll
    for (int k = 1; k < Un::N; ++k) umin = fminf(umin, u[k]);
    if (EXP == kExpBare || (EXP == kExpPerUnit && __builtin_expect(umin >= -126.f, 1))) {
#pragma unroll
        for (int k = 0; k < Un::N; ++k) {
            const float pk = __builtin_amdgcn_exp2f(u[k]);
            o[k] = WH ? pk * __builtin_fmaf(R.b, u[k], R.a) : pk * R.gs;
        }
    } else {
        // Here u may be -inf (a -inf logit): its p is 0, and the entropy factor
        // takes max(u, -256) so that the term is 0, not 0 * inf (2^-256 is 0 in
        // fp32, so no finite term changes).
#pragma unroll
        for (int k = 0; k < Un::N; ++k) {
            const float pk = exp2f(u[k]);
            o[k] = WH ? pk * __builtin_fmaf(R.b, fmaxf(u[k], kUFloor), R.a) : pk * R.gs;
        }
    }
    if (TGT && static_cast<uint32_t>(R.t - col0) < static_cast<uint32_t>(Un::N)) {
#pragma unroll
        for (int k = 0; k < Un::N; ++k)
            if (col0 + k == R.t) {
                const double d = static_cast<double>(Un::get(v, k)) / R.tau - R.lse;
                double ot = R.gt * -expm1(d);
                const double pt = exp(d);
                if (WH && pt != 0.0) ot += R.hs * pt * (d + R.H);
                o[k] = static_cast<float>(ot);
            }
    }
}

// Gradient of segment q of output row i.  KLF: top-k KL with the payload
// columns written in the same pass (16-byte units, no entropy term).
template <int DT, int GDT, bool VEC, bool WH, bool KLF>
__device__ __forceinline__ void bwd_item(const BwdPlan &p, int64_t i, int q) {
    static_assert(!KLF || (VEC && !WH), "fused payload columns: vector rows, no entropy term");
    using Un = Unit<DT, VEC>;
    using T = typename Un::T;
    constexpr int N = Un::N;
    constexpr int U = kBwdU;
    constexpr int64_t kE = DT == VWC_BF16 ? 2 : 4;
    constexpr int64_t kGE = GDT == VWC_BF16 ? 2 : 4;
    const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
    if (r < 0 || r >= p.n_rows) return;  // row id outside the tensor: nothing is written
    const char *row = static_cast<const char *>(p.logits) + r * p.ld * kE;
    char *grow = static_cast<char *>(p.grad) + (p.grad_by_row_id ? r : i) * p.ld_grad * kGE;
    // Whole vectors from the row's first 16-byte boundary on (the host checked
    // that it falls on a vector boundary of the gradient row too; the fused
    // top-k KL path takes rows that start on one); the edges go element-wise.
    const int32_t head = (VEC && !KLF) ? row_head<kE>(row, p.vocab) : 0;
    const char *vrow = row + head * kE;
    char *vgrow = grow + head * kGE;
    const int32_t nunits = (p.vocab - head) / N;
    const int32_t u0 = q * p.seg_units;
    const int32_t u1 = min(u0 + p.seg_units, nunits);
    const bool last = q == p.nseg - 1;
    // Unit b + j kBwdBlock of this thread (j uniform): byte (b - u0) N kGE of a
    // buffer resource over this segment's whole gradient vectors from unit
    // u0 + j kBwdBlock on.
    const int64_t seg_bytes = static_cast<int64_t>(max(u1 - u0, 0)) * N * kGE;
    auto put = [&](int32_t b, int j, const float (&o)[N]) {
        char *dst = vgrow + static_cast<int64_t>(b + j * kBwdBlock) * N * kGE;
        if constexpr (VEC) {
            const int64_t lead = static_cast<int64_t>(j) * kBwdBlock * N * kGE;
            const __amdgpu_buffer_rsrc_t rs =
                span_rsrc(vgrow + static_cast<int64_t>(u0) * N * kGE + lead,
                          static_cast<uint32_t>(max(seg_bytes - lead, int64_t{0})));
            GradStore<GDT, N>::store(VecDst{rs, static_cast<uint32_t>((b - u0) * N * kGE), dst}, o);
        } else {
            GradStore<GDT, N>::store(dst, o);
        }
    };
    const float g = p.grad_out ? p.grad_out[i] : 0.f;
    const float h = WH ? p.grad_ent[i] : 0.f;
    const bool kl = p.kl_P != nullptr;
    KlCoef klc{0.0, 0.0, 0.0, false};
    if (kl && g != 0.f)
        klc = kl_coef(p.kl_mode, p.kl_eps, static_cast<double>(p.kl_P[i]),
                      static_cast<double>(p.kl_Q[i]), static_cast<double>(p.kl_S[i]));

    if ((g == 0.f && h == 0.f) || klc.dead) {
        // Rows without loss: +0.0, no logits read.
        float z[N];
#pragma unroll
        for (int k = 0; k < N; ++k) z[k] = 0.f;
        for (int32_t b = u0 + static_cast<int32_t>(threadIdx.x); b < u1; b += kBwdBlock) put(b, 0, z);
        if (VEC && last) {
            const int32_t j = edge_column(head, nunits * N, p.vocab,
                                          static_cast<int32_t>(threadIdx.x));
            if (j >= 0) {
                float z1[1] = {0.f};
                GradStore<GDT, 1>::store(grow + static_cast<int64_t>(j) * kGE, z1);
            }
        }
        return;
    }

    const double gt = static_cast<double>(g) / p.tau;
    RowGrad R = row_grad(p.c_hi, p.c_lo, p.tau, p.lse[i], g, h,
                         WH ? static_cast<double>(p.entropy[i]) : 0.0,
                         kl ? gt * klc.alpha : -gt);  // top-k KL: o = q (g alpha / tau)
    R.t = (g != 0.f && !kl) ? p.targets[r] : -1;
    const T *src = reinterpret_cast<const T *>(vrow);

    __shared__ KlSlot kl_tab[KLF ? kKlSlots : 1];
    __shared__ uint32_t kl_lane[KLF ? kBwdBlock : 1];
    uint32_t kl_mine = 0;  // bit it: this thread's unit u0 + tid + it * kBwdBlock has payload columns
    if constexpr (KLF) {
        const int tid = static_cast<int>(threadIdx.x);
        for (int h = tid; h < kKlSlots; h += kBwdBlock) {
            kl_tab[h].unit = -1;
            kl_tab[h].cols = 0u;
        }
        kl_lane[tid] = 0u;
        __syncthreads();
        // This segment's payload columns: its whole vectors, and in the last
        // segment the tail past them.
        const int32_t vc0 = u0 * N, vc1 = u1 * N;
        for (int n = tid; n < p.kl_k; n += kBwdBlock) {
            const int32_t j = p.kl_idx[i * p.kl_k + n];
            const bool vec_col = j >= vc0 && j < vc1;
            const bool tail_col = last && j >= nunits * N && j < p.vocab;
            if (!vec_col && !tail_col) continue;  // another segment's, or outside the row
            const int32_t key = vec_col ? j / N - u0 : kKlTailKey;
            const int kk = j % N;
            const float val = kl_payload_grad(static_cast<double>(load_element<DT>(row, j)),
                                              R.tau, R.lse, R.gt, klc, p.kl_tlp[i * p.kl_k + n]);
            uint32_t h = kl_hash(key);
            for (int probe = 0; probe < kKlSlots; ++probe) {  // at most half full: ends early
                const int32_t old = atomicCAS(&kl_tab[h].unit, -1, key);
                if (old == -1 || old == key) break;
                h = (h + 1) & (kKlSlots - 1);
            }
            atomicOr(&kl_tab[h].cols, 1u << kk);
            kl_tab[h].val[kk] = val;
            if (vec_col) atomicOr(&kl_lane[key % kBwdBlock], 1u << (key / kBwdBlock));
        }
        __syncthreads();
        kl_mine = kl_lane[tid];
    }

    auto stream = [&](auto pair_tag) {
        constexpr bool kPair = decltype(pair_tag)::value;
        int32_t b = u0 + static_cast<int32_t>(threadIdx.x);
        for (; b + (U - 1) * kBwdBlock < u1; b += U * kBwdBlock) {
            T v[U];
#pragma unroll
            for (int j = 0; j < U; ++j) v[j] = Un::load(src + b + j * kBwdBlock);
            // All U loads go out before any arithmetic (the scheduler may
            // otherwise start unpacking after the first and hold the rest back).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int32_t unit = b + j * kBwdBlock;
                float o[N];
                unit_grad<DT, VEC, WH, kExpRescale, kPair>(v[j], head + unit * N, R, o);
                if (KLF && ((kl_mine >> ((unit - u0) / kBwdBlock)) & 1u))
                    kl_patch<N>(kl_tab, unit - u0, o);
                put(b, j, o);
            }
        }
        // The last (at most U - 1) units of this thread: all loads first, as above.
        if (b < u1) {
            T v[U - 1];
#pragma unroll
            for (int j = 0; j < U - 1; ++j)
                v[j] = b + j * kBwdBlock < u1 ? Un::load(src + b + j * kBwdBlock) : T{};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < U - 1; ++j) {
                const int32_t unit = b + j * kBwdBlock;
                if (unit >= u1) break;
                float o[N];
                unit_grad<DT, VEC, WH, kExpRescale, kPair>(v[j], head + unit * N, R, o);
                if (KLF && ((kl_mine >> ((unit - u0) / kBwdBlock)) & 1u))
                    kl_patch<N>(kl_tab, unit - u0, o);
                put(b, j, o);
            }
        }
        if (VEC && last) {
            const int32_t j = edge_column(head, nunits * N, p.vocab, static_cast<int32_t>(threadIdx.x));
            if (j >= 0) {
                using Us = Unit<DT, false>;
                const typename Us::T v = reinterpret_cast<const typename Us::T *>(row)[j];
                float o[1];
                unit_grad<DT, false, WH, kExpRescale, kPair>(v, j, R, o);
                if constexpr (KLF) {  // column j - nunits * N (< N) of the tail
                    const int h = kl_find(kl_tab, kKlTailKey);
                    const int kk = static_cast<int>(threadIdx.x);
                    if (h >= 0 && ((kl_tab[h].cols >> kk) & 1u)) o[0] = kl_tab[h].val[kk];
                }
                GradStore<GDT, 1>::store(grow + static_cast<int64_t>(j) * kGE, o);
            }
        }
    };
    if (GDT == VWC_FP32 || exponent_pair(false, R.B))
        stream(std::true_type{});
    else if constexpr (GDT != VWC_FP32)
        stream(std::false_type{});
}

// One workgroup per (row, segment) item.
template <int DT, int GDT, bool VEC, bool WH, bool KLF = false>
__global__ __launch_bounds__(kBwdBlock) VWC_BWD_ATTR void bwd_segment_kernel(BwdPlan p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) / p.nseg;
    bwd_item<DT, GDT, VEC, WH, KLF>(p, i, static_cast<int>(blockIdx.x - i * p.nseg));
}

// ---------------------------------------------------------------- top-k KL

constexpr int kTopkBlock = 64;  // one wave per row

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

// Per row: gather the k payload columns of the student row and reduce P, Q and
// S = sum p (a - log q) in fp64 (lane-strided, then a fixed butterfly).
template <int DT>
__global__ __launch_bounds__(kTopkBlock) void topk_fwd_kernel(TopkPlan p) {
    const int64_t i = blockIdx.x;
    const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
    if (r < 0 || r >= p.n_rows) {  // row id outside the logits: NaN outputs, no reads
        if (threadIdx.x == 0) {
            if (p.loss) p.loss[i] = NAN;
            if (p.Q) p.Q[i] = NAN;
            if (p.P) p.P[i] = NAN;
            if (p.S) p.S[i] = NAN;
        }
        return;
    }
    const char *row = static_cast<const char *>(p.logits) + r * p.ld * (DT == VWC_BF16 ? 2 : 4);
    const double lse = static_cast<double>(p.lse[i]);
    double P = 0.0, Q = 0.0, S = 0.0, bad = 0.0;
    for (int n = threadIdx.x; n < p.k; n += kTopkBlock) {
        const int32_t j = p.idx[i * p.k + n];
        if (j < 0 || j >= p.vocab) {
            bad = 1.0;
            continue;
        }
        const double a = static_cast<double>(p.tlp[i * p.k + n]);
        const double lq = static_cast<double>(load_element<DT>(row, j)) / p.tau - lse;
        const double pn = exp(a);
        P += pn;
        Q += exp(lq);
        S += pn * (a - lq);
    }
    P = wave_sum(P);
    Q = wave_sum(Q);
    S = wave_sum(S);
    bad = wave_sum(bad);
    if (threadIdx.x != 0) return;
    double L;
    if (p.mode == VWC_KL_TRUNCATED) {
        L = S < 0.0 ? 0.0 : S;
    } else {
        const double pt = P < 1.0 ? 1.0 - P : 0.0;
        const double qt = fmax(1.0 - Q, p.eps);
        L = S + (pt == 0.0 ? 0.0 : pt * (log(pt) - log(qt)));
    }
    if (bad != 0.0) L = P = Q = S = NAN;
    if (p.loss) p.loss[i] = static_cast<float>(L);
    if (p.Q) p.Q[i] = static_cast<float>(Q);
    if (p.P) p.P[i] = static_cast<float>(P);
    if (p.S) p.S[i] = static_cast<float>(S);
}

// After the streaming backward wrote alpha q_j g / tau everywhere: overwrite
// the k payload columns with (beta q_j - kappa p_j) g / tau.
template <int DT, int GDT>
__global__ __launch_bounds__(kTopkBlock) void topk_fixup_kernel(TopkPlan p) {
    const int64_t i = blockIdx.x;
    const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
    if (r < 0 || r >= p.n_rows) return;  // the streaming pass wrote nothing for it either
    const float g = p.grad_loss[i];
    if (g == 0.f) return;
    const KlCoef c = kl_coef(p.mode, p.eps, static_cast<double>(p.inP[i]),
                             static_cast<double>(p.inQ[i]), static_cast<double>(p.inS[i]));
    if (c.dead) return;
    const char *row = static_cast<const char *>(p.logits) + r * p.ld * (DT == VWC_BF16 ? 2 : 4);
    char *grow = static_cast<char *>(p.grad) +
                 (p.grad_by_row_id ? r : i) * p.ld_grad * (GDT == VWC_BF16 ? 2 : 4);
    const double lse = static_cast<double>(p.lse[i]);
    const double gt = static_cast<double>(g) / p.tau;
    for (int n = threadIdx.x; n < p.k; n += kTopkBlock) {
        const int32_t j = p.idx[i * p.k + n];
        if (j < 0 || j >= p.vocab) continue;
        const float o[1] = {kl_payload_grad(static_cast<double>(load_element<DT>(row, j)), p.tau,
                                            lse, gt, c, p.tlp[i * p.k + n])};
        GradStore<GDT, 1>::store(grow + static_cast<int64_t>(j) * (GDT == VWC_BF16 ? 2 : 4), o);
    }
}

// ---------------------------------------------------------------- fused forward + backward

// One 1024-thread workgroup per row (one per compute unit: the row fills its
// LDS and most of its registers), the whole row kept on chip between the
// reduction and the gradient.  Unit u = tid + k * 1024 (16 bytes from the
// row's first 16-byte boundary) sits in LDS for k < kFusedLds (staged by
// buffer_load ... lds) and in registers after that.  Phase 1 reads the row once
// and reduces it (four groups of 256 threads, their partials merged in fp64 as
// in the segmented forward); thread 0 writes logprob / lse / entropy and
// shares the fp32 lse; phase 2 computes every gradient element from the held
// values with the backward's own per-unit code and writes it.  Every read of
// the row ends before the barrier that starts phase 2, so the gradient may
// replace the logits.
//
// KL: the same row pass for the top-k KL objective instead of the target's
// logprob (the tail-aware / truncated objective of "[megatron] feat: add
// memory-efficient chunked top-k KL computation", with the per-row weight
// known up front).  Each thread below k also loads one payload entry: its
// column id and teacher log-prob first (parked in LDS once the row's loads
// are out, so that no register holds them through the fold), the student
// logit at that column after the row, as the logprob mode loads the target's.  Once the row's lse is known, those
// threads sum P, Q and S (a fixed butterfly per wave, then the waves in
// order), thread 0 writes P, Q and S and turns their float values into the
// gradient's coefficients exactly as the separate backward reads them, and
// every payload thread computes its column's gradient and files it, in LDS,
// under the thread that stores that column's unit, which writes it after the
// unit (same thread, later store).  The loss, which the gradient does not
// need, is written at the end.
template <int DT, bool W, bool KL = false, bool WH = false>
__global__ __launch_bounds__(kFusedBlock) void fused_row_kernel(FusedPlan p) {
    static_assert(!(KL && W), "the top-k KL call writes no entropy");
    static_assert(!WH || (W && !KL), "the entropy gradient needs the entropy, no top-k KL");
    using Un = Unit<DT, true>;
    using T = typename Un::T;
    using Us = Unit<DT, false>;
    constexpr int N = Un::N;
    constexpr int64_t kE = DT == VWC_BF16 ? 2 : 4;
    constexpr int kStride = kFusedBlock * 16;  // bytes between a thread's units
    __shared__ __attribute__((aligned(16))) char stage[kFusedLds * kStride];
    __shared__ Lane wave_state[kFusedBlock / 64];
    __shared__ double row_gt;
    __shared__ float row_lse, row_B, row_gs;
    // the entropy gradient's row constants (WH): o = p' (a + b u'), and for the
    // target column -h/tau and the saved entropy
    __shared__ float row_a, row_b;
    __shared__ double row_hs, row_H;
    // KL: the waves' payload sums (P, Q, S, bad), the row's coefficients, the
    // payload gradients and, per thread, the list of those its units hold.
    constexpr int kKlN = KL ? kKlMaxK : 1;
    constexpr int kKlTid0 = 64;  // payload entry n is thread kKlTid0 + n (waves 1-4)
    constexpr int kKlWaves = kKlMaxK / 64;
    static_assert(!KL || kKlTid0 + kKlMaxK <= kFusedBlock, "payload threads");
    __shared__ double kl_sums[KL ? kKlWaves * 3 : 1];
    __shared__ double kl_pn[kKlN], kl_q[kKlN];  // p_n = exp(a_n), q at the payload column
    __shared__ double kl_beta, kl_kappa;
    __shared__ int kl_zero;
    __shared__ int kl_head[KL ? kFusedBlock : 1];
    __shared__ int kl_next[kKlN];
    __shared__ int kl_col[kKlN];   // the payload column ids
    __shared__ float kl_val[kKlN];  // the teacher log-probs, then the payload gradients

    const int64_t i = blockIdx.x;  // output row
    const int32_t tid = static_cast<int32_t>(threadIdx.x);
    const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
    if (r < 0 || r >= p.n_rows) {  // row id outside the tensor: NaN outputs, nothing written
        if (tid == 0) {
            if (!KL && p.logprob) p.logprob[i] = NAN;
            p.lse[i] = NAN;
            if (W && p.entropy) p.entropy[i] = NAN;
            if (KL) {
                if (p.kl_loss) p.kl_loss[i] = NAN;
                p.kl_P[i] = NAN;
                p.kl_Q[i] = NAN;
                p.kl_S[i] = NAN;
            }
        }
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const char *row = static_cast<const char *>(p.logits) + r * p.ld * kE;
    char *grow = static_cast<char *>(p.grad) + (p.grad_by_row_id ? r : i) * p.ld_grad * kE;
    const int32_t head = row_head<kE>(row, p.vocab);
    const int32_t nunits = (p.vocab - head) / N;
    // This thread's units: tid + k * kFusedBlock; the LDS ones (k < kFusedLds)
    // and the register ones (k = kFusedLds + kr, kr < nreg) that lie in the row.
    const int32_t nreg = min(max((nunits - tid - kFusedLds * kFusedBlock + kFusedBlock - 1) /
                                     kFusedBlock, 0), kFusedReg);
    char *vgrow = grow + head * kE + tid * 16;  // this thread's unit 0 of the gradient

    // Phase 1.  This thread's edge element is read first, then the LDS units
    // through the DMA path and the register units through plain buffer loads,
    // both from one buffer resource that ends at the row's last whole vector:
    // units past it read as zero (the whole offset sits in the per-lane offset,
    // which the range check covers), so every wave issues the same loads in the
    // same order.  Only then come the loss weight, the target id and the target
    // logit, whose dependent round trips would otherwise delay the row's
    // loads.  Loads complete in order, so once at most kFusedReg + 1 are
    // outstanding the wave's LDS units have landed, and they are folded while
    // the register units still arrive.  Each thread reads back only what its
    // own wave's loads wrote.  The edge and target loads are unconditional
    // (clamped to the row) so that no branch makes the compiler wait for them.
    // KL: this thread's payload entry (threads past k load entry k - 1 and
    // ignore it, so that every wave issues the same loads).
    int32_t kj = 0;
    float ka = 0.f;
    if constexpr (KL) {
        const int64_t n = i * p.kl_k + min(max(tid - kKlTid0, 0), p.kl_k - 1);
        kj = p.kl_idx[n];
        ka = p.kl_tlp[n];
        kl_head[tid] = -1;
    }
    const int32_t edge = edge_column(head, nunits * N, p.vocab, tid);
    typename Us::T ev[1] = {reinterpret_cast<const typename Us::T *>(row)[max(edge, 0)]};
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(row + head * kE), 0, nunits * 16, 0x00020000);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kFusedLds; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, stage + k * kStride + wave * 64 * 16, 16,
            static_cast<uint32_t>(tid * 16 + k * kStride), 0, 0, 0);
    T v[kFusedReg];
#pragma unroll
    for (int kr = 0; kr < kFusedReg; ++kr)  // cache policy: non-temporal
        v[kr] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(
                                          rsrc, static_cast<uint32_t>(tid * 16 + (kFusedLds + kr) * kStride),
                                          0, 2));
    __builtin_amdgcn_sched_barrier(0);
    const float g = (!WH || p.grad_out) ? p.grad_out[i] : 0.f;  // WH: g may be absent
    const float h = WH ? p.grad_ent[i] : 0.f;
    // The target (logprob mode), or this thread's payload column (KL): one more
    // load each, after the row's.
    const int32_t t = (KL || (WH && !p.targets)) ? -1 : p.targets[r];
    const bool t_ok = t >= 0 && t < p.vocab;
    const bool kj_ok = kj >= 0 && kj < p.vocab;
    const typename Us::T t_raw =
        reinterpret_cast<const typename Us::T *>(row)[KL ? (kj_ok ? kj : 0) : (t_ok ? t : 0)];
    if constexpr (KL) {  // the payload entry's id and log-prob wait in LDS
        const int32_t n = tid - kKlTid0;
        if (n >= 0 && n < p.kl_k) {
            kl_col[n] = kj_ok ? kj : -1;
            kl_val[n] = ka;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // s_waitcnt vmcnt(kFusedReg + 1) (6-bit count: low 4 bits at [3:0], high 2
    // at [15:14]; expcnt and lgkmcnt not waited on).
    constexpr int kAfterLds = kFusedReg + 1;
    static_assert(kAfterLds < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt(((kAfterLds >> 4) << 14) | 0x0F70 | (kAfterLds & 15));
    __builtin_amdgcn_sched_barrier(0);

    Lane L = lane_init();
    float xmin = INFINITY;  // this thread's smallest whole-vector logit (NaN ignored)
    auto unit_min = [&](const T &x) {
#pragma unroll
        for (int k = 0; k < N; ++k) xmin = fminf(xmin, Un::get(x, k));
    };
#pragma unroll 1
    for (int k = 0; k < kFusedLds; ++k) {
        if (tid + k * kFusedBlock >= nunits) break;
        const T x[1] = {*reinterpret_cast<const T *>(stage + k * kStride + tid * 16)};
        fold_chunk<DT, true, 1, W>(x, 1, p.c, L);
        unit_min(x[0]);
    }
    // The register units in short chunks (few unpacked values live at a time
    // while every unit stays held for phase 2).
    constexpr int kChunk = 2;
    static_assert(kFusedReg % kChunk == 0, "whole chunks of register units");
#pragma unroll
    for (int k0 = 0; k0 < kFusedReg; k0 += kChunk) {
        const int nv = min(max(nreg - k0, 0), kChunk);
        if (nv > 0) {
            fold_chunk<DT, true, kChunk, W>(*reinterpret_cast<const T(*)[kChunk]>(&v[k0]), nv,
                                            p.c, L);
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
                if (j < nv) unit_min(v[k0 + j]);
        }
    }
    if (edge >= 0) fold_chunk<DT, false, 1, W>(ev, 1, p.c, L);

    // The row's state: each wave's lanes, then the 16 wave states (lanes 0-15
    // of wave 0), reduced by rescaling to the largest shift (fp32); thread 0
    // turns it into the row's outputs in fp64 as the segment forward does for
    // one segment, and the gradient's per-row constants (computed once, shared
    // through LDS).
    const Lane Wv = wave_reduce_rescaled(L);
    if ((tid & 63) == 0) wave_state[wave] = Wv;
    __syncthreads();
    // KL, while wave 0 forms the row's lse: the payload's sums that do not need
    // it, P = sum p_n, D = sum p_n (a_n - x_n / tau) and
    // E = sum exp((x_n - mr) / tau) against the row's largest logit mr, so that
    // Q = exp(mr / tau - lse) E and S = D + lse P once lse is known.  An entry
    // outside the row adds NaN to P, which then makes P, Q and S NaN.
    if constexpr (KL) {
        if (wave >= 1 && wave <= kKlWaves) {
            const int32_t n = tid - kKlTid0;
            const bool mine = n < p.kl_k;
            float mr = -INFINITY;
            for (int w = 0; w < kFusedBlock / 64; ++w) mr = fmaxf(mr, wave_state[w].m);
            double sP = 0.0, sD = 0.0, sE = 0.0;
            if (mine) {
                if (kl_col[n] < 0) {
                    sP = NAN;
                } else {
                    const double a = static_cast<double>(kl_val[n]);
                    const double x = static_cast<double>(Us::get(t_raw, 0)) / p.tau;
                    const double pn = exp(a);
                    kl_pn[n] = pn;
                    sP = pn;
                    sD = pn * (a - x);
                    sE = exp(x - static_cast<double>(mr) / p.tau);
                }
            }
            sP = wave_sum(sP);
            sD = wave_sum(sD);
            sE = wave_sum(sE);
            if ((tid & 63) == 0) {
                double *o = kl_sums + (wave - 1) * 3;
                o[0] = sP;
                o[1] = sD;
                o[2] = sE;
            }
        }
    }
    if (wave == 0) {
        const Lane Lw = (tid < kFusedBlock / 64) ? wave_state[tid] : lane_init();
        const Lane Rw = wave_reduce_rescaled(Lw);
        if (tid == 0) {
            const double tx = KL ? -INFINITY : !t_ok ? NAN : static_cast<double>(Us::get(t_raw, 0));
            const P64 part = to_partial(Rw, p.c, tx);
            const Merged mg = merge_partials([&](int) { return part; }, 1, p.tau);
            write_final(mg, p.tau, i, KL ? nullptr : p.logprob, p.lse, W ? p.entropy : nullptr);
            const float lse32 = static_cast<float>(mg.M / p.tau + log(mg.S));  // lse[i]
            row_lse = lse32;
            if constexpr (!KL) {
                // WH: the entropy as written (its float), as the separate backward reads it
                const double H32 = WH ? static_cast<double>(static_cast<float>(
                                            log(mg.S) - mg.W / mg.S))
                                      : 0.0;
                const RowGrad R0 = row_grad(p.gc_hi, p.gc_lo, p.tau, lse32, g, h, H32,
                                            -static_cast<double>(g) / p.tau);
                row_B = R0.B;
                row_gs = R0.gs;
                row_gt = R0.gt;
                if constexpr (WH) {
                    row_a = R0.a;
                    row_b = R0.b;
                    row_hs = R0.hs;
                    row_H = R0.H;
                }
            }
        }
    }
    __syncthreads();

    if constexpr (KL) {
        const double lse = static_cast<double>(row_lse);
        const int32_t n = tid - kKlTid0;
        const bool mine = n >= 0 && n < p.kl_k;
        if (tid == 0) {
            // P, Q and S in the top-k forward's definitions; bad entries make
            // them NaN.  Then the gradient's coefficients from their float
            // values, as the separate backward reads them back.
            double P = 0.0, D = 0.0, E = 0.0;
            for (int w = 0; w < kKlWaves; ++w) {
                P += kl_sums[w * 3 + 0];
                D += kl_sums[w * 3 + 1];
                E += kl_sums[w * 3 + 2];
            }
            float mr = -INFINITY;
            for (int w = 0; w < kFusedBlock / 64; ++w) mr = fmaxf(mr, wave_state[w].m);
            double Q = exp(static_cast<double>(mr) / p.tau - lse) * E;
            double S = D + lse * P;
            if (P != P) P = Q = S = NAN;  // an entry outside the row
            kl_sums[0] = P;  // kept for the loss at the end
            kl_sums[1] = Q;
            kl_sums[2] = S;
            const float Pf = static_cast<float>(P), Qf = static_cast<float>(Q),
                        Sf = static_cast<float>(S);
            p.kl_P[i] = Pf;
            p.kl_Q[i] = Qf;
            p.kl_S[i] = Sf;
            KlCoef kc{0.0, 0.0, 0.0, false};
            if (g != 0.f)
                kc = kl_coef(p.kl_mode, p.kl_eps, static_cast<double>(Pf),
                             static_cast<double>(Qf), static_cast<double>(Sf));
            const double gt = static_cast<double>(g) / p.tau;
            const RowGrad R0 = row_grad(p.gc_hi, p.gc_lo, p.tau, row_lse, g, 0.f, 0.0,
                                        gt * kc.alpha);
            row_B = R0.B;
            row_gs = R0.gs;
            row_gt = R0.gt;
            kl_beta = kc.beta;
            kl_kappa = kc.kappa;
            kl_zero = (g == 0.f || kc.dead) ? 1 : 0;
        } else if (mine && kl_col[n] >= 0) {
            // q at the payload column, as the separate backward forms it.
            kl_q[n] = exp(static_cast<double>(Us::get(t_raw, 0)) / p.tau - lse);
        }
        __syncthreads();
        // Each payload column's gradient (beta q - kappa p_n) g / tau, filed under
        // the thread that stores its unit (or, outside the whole vectors, its
        // edge element).
        if (mine && kl_zero == 0) {
            const int32_t pj = kl_col[n];
            if (pj >= 0) {
                kl_val[n] = kl_payload_value(kl_q[n], kl_pn[n], row_gt, kl_beta, kl_kappa);
                const int32_t body = nunits * N;
                const int32_t owner = pj < head          ? pj
                                      : pj >= head + body ? pj - body
                                                          : ((pj - head) / N) % kFusedBlock;
                kl_next[n] = atomicExch(&kl_head[owner], n);
            }
        }
        __syncthreads();
    }

    // Phase 2: the gradient, as the backward computes it from the saved fp32 lse
    // (the row constants row_grad gives for it).
    RowGrad R;
    R.c_hi = p.gc_hi;
    R.c_lo = p.gc_lo;
    R.B = row_B;
    R.gs = row_gs;
    R.a = WH ? row_a : 0.f;
    R.b = WH ? row_b : 0.f;
    R.gt = row_gt;
    R.hs = WH ? row_hs : 0.0;
    R.H = WH ? row_H : 0.0;
    R.lse = static_cast<double>(row_lse);
    R.tau = p.tau;
    R.t = g != 0.f ? t : -1;  // no one-hot term without a logprob weight, as in the backward
    // A row without loss (or a clamped truncated KL row): +0.0, nothing computed.
    const bool zero = KL ? kl_zero != 0 : (g == 0.f && h == 0.f);
    // p' = 2^u' with u' increasing in x, so the thread's smallest logit gives
    // its smallest exponent: when that one lies at or above -126 every unit of
    // the thread takes the bare exp2 (exp2f's bits there), else every unit takes
    // exp2f, one decision per thread instead of one per unit.  The units are
    // stored without the target column's one-hot term; the thread that owns that
    // column writes its element afterwards.
    auto phase2 = [&](auto pair_tag, auto bare_tag) {
        constexpr bool kPair = decltype(pair_tag)::value;
        constexpr int kExp = decltype(bare_tag)::value ? kExpBare : kExpRescale;
        auto emit = [&](const T &x, int32_t u, char *dst) {
            float o[N];
            if (zero) {
#pragma unroll
                for (int k = 0; k < N; ++k) o[k] = 0.f;
            } else {
                unit_grad<DT, true, WH, kExp, kPair, false>(x, head + u * N, R, o);
            }
            GradStore<DT, N>::store(dst, o);
        };
#pragma unroll
        for (int kr = 0; kr < kFusedReg; ++kr)
            if (kr < nreg)
                emit(v[kr], tid + (kFusedLds + kr) * kFusedBlock, vgrow + (kFusedLds + kr) * kStride);
        // The register units are spent, so the LDS units are all read up front
        // (slots past the row hold zeros and are not stored).
        T xl[kFusedLds];
#pragma unroll
        for (int k = 0; k < kFusedLds; ++k)
            xl[k] = *reinterpret_cast<const T *>(stage + k * kStride + tid * 16);
#pragma unroll
        for (int k = 0; k < kFusedLds; ++k) {
            const int32_t u = tid + k * kFusedBlock;
            if (u < nunits) emit(xl[k], u, vgrow + k * kStride);
        }
    };
    const bool pair = exponent_pair(DT == VWC_FP32, R.B);
    const float umin = pair ? __builtin_fmaf(xmin, R.c_lo, __builtin_fmaf(xmin, R.c_hi, -R.B))
                            : __builtin_fmaf(xmin, R.c_hi, -R.B);
    if constexpr (DT == VWC_FP32) {
        if (umin >= -126.f)
            phase2(std::true_type{}, std::true_type{});
        else
            phase2(std::true_type{}, std::false_type{});
    } else if (!pair) {
        if (umin >= -126.f)
            phase2(std::false_type{}, std::true_type{});
        else
            phase2(std::false_type{}, std::false_type{});
    } else {
        // A row whose exponent keeps the float pair (|B| >= 4096, far outside any
        // trained model's logits) re-reads its units from memory in a plain loop
        // instead of a third unrolled copy of the above: each unit is read before
        // this thread stores it, and no other thread touches it, so an in-place
        // gradient is still safe.  exp2f's bits equal the bare exp2 where both apply.
        const T *src = reinterpret_cast<const T *>(row + head * kE);
#pragma unroll 1
        for (int k = 0; k < kFusedLds + kFusedReg; ++k) {
            const int32_t u = tid + k * kFusedBlock;
            if (u >= nunits) break;
            float o[N];
            if (zero) {
#pragma unroll
                for (int e = 0; e < N; ++e) o[e] = 0.f;
            } else {
                unit_grad<DT, true, WH, kExpRescale, true, false>(Un::load(src + u), head + u * N, R, o);
            }
            GradStore<DT, N>::store(vgrow + k * kStride, o);
        }
    }
    // The target column, when it lies in the whole vectors: its unit went out
    // above from this thread; this later store from the same thread replaces
    // the element with the one-hot term included.
    const int32_t tcol = t_ok && R.t >= 0 ? t - head : -1;
    if (!KL && !zero && tcol >= 0 && tcol < nunits * N && (tcol / N) % kFusedBlock == tid) {
        const double d = static_cast<double>(Us::get(t_raw, 0)) / R.tau - R.lse;
        double ot = R.gt * -expm1(d);  // as unit_grad forms the target column
        if constexpr (WH) {
            const double pt = exp(d);
            if (pt != 0.0) ot += R.hs * pt * (d + R.H);
        }
        float o[1] = {static_cast<float>(ot)};
        GradStore<DT, 1>::store(grow + static_cast<int64_t>(t) * kE, o);
    }
    if (edge >= 0) {
        float o[1] = {0.f};
        if (!zero) {
            if (pair)
                unit_grad<DT, false, WH, kExpPerUnit, true>(ev[0], edge, R, o);
            else
                unit_grad<DT, false, WH, kExpPerUnit, false>(ev[0], edge, R, o);
        }
        GradStore<DT, 1>::store(grow + static_cast<int64_t>(edge) * kE, o);
    }
    // KL: the payload columns this thread's units (or edge element) hold, after
    // those stores.  The list holds at most k entries.
    if constexpr (KL) {
        if (!zero)
            for (int e = kl_head[tid]; e >= 0; e = kl_next[e]) {
                const float o[1] = {kl_val[e]};
                GradStore<DT, 1>::store(grow + static_cast<int64_t>(kl_col[e]) * kE, o);
            }
        if (tid == 0 && p.kl_loss) {  // the loss, as the top-k forward defines it
            const double P = kl_sums[0], Q = kl_sums[1], S = kl_sums[2];
            double Lk;
            if (p.kl_mode == VWC_KL_TRUNCATED) {
                Lk = S < 0.0 ? 0.0 : S;
            } else {
                const double pt = P < 1.0 ? 1.0 - P : 0.0;
                const double qt = fmax(1.0 - Q, p.kl_eps);
                Lk = S + (pt == 0.0 ? 0.0 : pt * (log(pt) - log(qt)));
            }
            p.kl_loss[i] = static_cast<float>(Lk);
        }
    }
}

// ---------------------------------------------------------------- mask -> index

constexpr int kScanBlock = 1024;
constexpr int kScanItems = 16;

__global__ __launch_bounds__(kScanBlock) void mask_to_index_kernel(const uint8_t *mask, int64_t n,
                                                                   int32_t *idx, int32_t *count) {
    __shared__ int32_t wave_tot[kScanBlock / 64];
    __shared__ int32_t wave_off[kScanBlock / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool aligned = (reinterpret_cast<uintptr_t>(mask) & 15) == 0;
    int32_t carry = 0;
    for (int64_t base = 0; base < n; base += static_cast<int64_t>(kScanBlock) * kScanItems) {
        const int64_t b = base + static_cast<int64_t>(threadIdx.x) * kScanItems;
        uint32_t bits = 0;
        if (aligned && b + kScanItems <= n) {
            // one 16-byte load: bit k is set when byte k is nonzero
            const u32x4 q = *reinterpret_cast<const u32x4 *>(mask + b);
#pragma unroll
            for (int k = 0; k < kScanItems; ++k)
                if ((q[k >> 2] >> (8 * (k & 3))) & 0xffu) bits |= 1u << k;
        } else {
#pragma unroll
            for (int k = 0; k < kScanItems; ++k)
                if (b + k < n && mask[b + k] != 0) bits |= 1u << k;
        }
        const int32_t c = __builtin_popcount(bits);
        // Inclusive scan of c across the wave.
        int32_t x = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t acc = 0;
            for (int w = 0; w < kScanBlock / 64; ++w) {
                wave_off[w] = acc;
                acc += wave_tot[w];
            }
            wave_tot[0] = acc;  // block total (read after the barrier below)
        }
        __syncthreads();
        int32_t off = carry + wave_off[wave] + x - c;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k)
            if (bits & (1u << k)) idx[off++] = static_cast<int32_t>(b + k);
        carry += wave_tot[0];
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = carry;
}

// Long masks: three launches over tiles of kTileItems entries.  Each tile's
// nonzero count goes to the workspace, one workgroup turns the counts into
// exclusive offsets (and the total), then every tile writes its ascending ids
// from its offset.  The same ids as the one-workgroup scan, in parallel over
// the tiles.
constexpr int kTileBlock = 256;
constexpr int kTileItems = kTileBlock * kScanItems;  // 4096

// Bits k of the returned word: entry b + k of the mask is nonzero (k < 16).
__device__ __forceinline__ uint32_t mask_bits(const uint8_t *mask, int64_t n, int64_t b,
                                              bool aligned) {
    uint32_t bits = 0;
    if (aligned && b + kScanItems <= n) {
        const u32x4 q = *reinterpret_cast<const u32x4 *>(mask + b);
#pragma unroll
        for (int k = 0; k < kScanItems; ++k)
            if ((q[k >> 2] >> (8 * (k & 3))) & 0xffu) bits |= 1u << k;
    } else {
#pragma unroll
        for (int k = 0; k < kScanItems; ++k)
            if (b + k < n && mask[b + k] != 0) bits |= 1u << k;
    }
    return bits;
}

// Exclusive prefix of v over the workgroup's threads (kTileBlock of them) and
// the workgroup's total.
__device__ __forceinline__ int32_t tile_exclusive_scan(int32_t v, int32_t *total) {
    __shared__ int32_t wave_tot[kTileBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTileBlock / 64; ++w) {
        if (w < wave) off += wave_tot[w];
        tot += wave_tot[w];
    }
    *total = tot;
    return off + x - v;
}

__global__ __launch_bounds__(kTileBlock) void mask_tile_count_kernel(const uint8_t *mask,
                                                                     int64_t n, int32_t *tiles) {
    const bool aligned = (reinterpret_cast<uintptr_t>(mask) & 15) == 0;
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kTileItems +
                      static_cast<int64_t>(threadIdx.x) * kScanItems;
    int32_t tot;
    tile_exclusive_scan(__builtin_popcount(mask_bits(mask, n, b, aligned)), &tot);
    if (threadIdx.x == 0) tiles[blockIdx.x] = tot;
}

// One workgroup: tiles[0..ntiles) -> exclusive offsets, *count = the total.
__global__ __launch_bounds__(kScanBlock) void mask_tile_scan_kernel(int32_t *tiles,
                                                                    int64_t ntiles,
                                                                    int32_t *count) {
    __shared__ int32_t wave_tot[kScanBlock / 64];
    __shared__ int32_t wave_off[kScanBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t carry = 0;
    for (int64_t base = 0; base < ntiles; base += kScanBlock) {
        const int64_t k = base + threadIdx.x;
        const int32_t c = k < ntiles ? tiles[k] : 0;
        int32_t x = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t acc = 0;
            for (int w = 0; w < kScanBlock / 64; ++w) {
                wave_off[w] = acc;
                acc += wave_tot[w];
            }
            wave_tot[0] = acc;
        }
        __syncthreads();
        if (k < ntiles) tiles[k] = carry + wave_off[wave] + x - c;
        carry += wave_tot[0];
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = carry;
}

__global__ __launch_bounds__(kTileBlock) void mask_tile_write_kernel(const uint8_t *mask,
                                                                     int64_t n,
                                                                     const int32_t *tiles,
                                                                     int32_t *idx) {
    const bool aligned = (reinterpret_cast<uintptr_t>(mask) & 15) == 0;
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kTileItems +
                      static_cast<int64_t>(threadIdx.x) * kScanItems;
    const uint32_t bits = mask_bits(mask, n, b, aligned);
    int32_t tot;
    int32_t off = tiles[blockIdx.x] + tile_exclusive_scan(__builtin_popcount(bits), &tot);
#pragma unroll
    for (int k = 0; k < kScanItems; ++k)
        if (bits & (1u << k)) idx[off++] = static_cast<int32_t>(b + k);
}

// ---------------------------------------------------------------- launch helpers

// Every row streams 16-byte vectors from its first 16-byte boundary on.
template <int DT, bool INBLOCK>
void launch_fwd_shape(const FwdPlan &p, dim3 grid, dim3 block, hipStream_t s) {
    if (p.want_entropy)
        hipLaunchKernelGGL((fwd_segment_kernel<DT, true, true, INBLOCK>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((fwd_segment_kernel<DT, true, false, INBLOCK>), grid, block, 0, s, p);
}

template <int DT>
hipError_t launch_fwd_dt(const FwdPlan &p, hipStream_t s) {
    if (p.nseg > 1 && !fwd_needs_workspace(p.nseg))
        launch_fwd_shape<DT, true>(p, dim3(static_cast<uint32_t>(p.m)),
                                   dim3(static_cast<uint32_t>(p.nseg * kFwdBlock)), s);
    else
        launch_fwd_shape<DT, false>(p, dim3(static_cast<uint32_t>(p.m * p.nseg)),
                                    dim3(kFwdBlock), s);
    return hipGetLastError();
}

template <int DT, int GDT>
hipError_t launch_bwd_dt(const BwdPlan &p, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(p.m * p.nseg)), block(kBwdBlock);
    const bool wh = p.grad_ent != nullptr;
    if (p.kl_fused) {  // the host checked: vector rows, no entropy term
        hipLaunchKernelGGL((bwd_segment_kernel<DT, GDT, true, false, true>), grid, block, 0, s,
                           p);
    } else if (p.vector) {
        if (wh)
            hipLaunchKernelGGL((bwd_segment_kernel<DT, GDT, true, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((bwd_segment_kernel<DT, GDT, true, false>), grid, block, 0, s, p);
    } else {
        if (wh)
            hipLaunchKernelGGL((bwd_segment_kernel<DT, GDT, false, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((bwd_segment_kernel<DT, GDT, false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdPlan &p, int dt, hipStream_t stream) {
    hipError_t e = dt == VWC_BF16 ? launch_fwd_dt<VWC_BF16>(p, stream)
                                  : launch_fwd_dt<VWC_FP32>(p, stream);
    if (e != hipSuccess || !fwd_needs_workspace(p.nseg)) return e;
    CombinePlan c{};
    c.parts = p.seg_part;
    c.k = p.nseg;
    c.stride = p.m;
    c.rows = p.m;
    c.tau = p.tau;
    c.logprob = p.target_mode == kTargetNone ? nullptr : p.logprob;
    c.lse = p.lse;
    c.entropy = p.entropy;
    c.partial_out = p.partial_out;
    return launch_combine(c, stream);
}

hipError_t launch_combine(const CombinePlan &p, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>((p.rows + kCombineBlock - 1) / kCombineBlock)),
        block(kCombineBlock);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_combine_rows(const CombinePlan &p, hipStream_t stream) {
    constexpr int rows_per_block = kCombineRowsBlock / 64;
    const dim3 grid(static_cast<uint32_t>((p.rows + rows_per_block - 1) / rows_per_block)),
        block(kCombineRowsBlock);
    hipLaunchKernelGGL(combine_rows_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdPlan &p, hipStream_t stream) {
    if (p.dt == VWC_BF16)
        return p.gdt == VWC_BF16 ? launch_bwd_dt<VWC_BF16, VWC_BF16>(p, stream)
                                 : launch_bwd_dt<VWC_BF16, VWC_FP32>(p, stream);
    return p.gdt == VWC_BF16 ? launch_bwd_dt<VWC_FP32, VWC_BF16>(p, stream)
                             : launch_bwd_dt<VWC_FP32, VWC_FP32>(p, stream);
}

hipError_t launch_fused(const FusedPlan &p, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.m)), block(kFusedBlock);
    const bool w = p.entropy != nullptr;
    if (p.kl_idx) {
        if (p.dt == VWC_BF16)
            hipLaunchKernelGGL((fused_row_kernel<VWC_BF16, false, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fused_row_kernel<VWC_FP32, false, true>), grid, block, 0, stream, p);
    } else if (p.grad_ent) {  // the host checked: the entropy output is requested
        if (p.dt == VWC_BF16)
            hipLaunchKernelGGL((fused_row_kernel<VWC_BF16, true, false, true>), grid, block, 0,
                               stream, p);
        else
            hipLaunchKernelGGL((fused_row_kernel<VWC_FP32, true, false, true>), grid, block, 0,
                               stream, p);
    } else if (p.dt == VWC_BF16) {
        if (w)
            hipLaunchKernelGGL((fused_row_kernel<VWC_BF16, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fused_row_kernel<VWC_BF16, false>), grid, block, 0, stream, p);
    } else {
        if (w)
            hipLaunchKernelGGL((fused_row_kernel<VWC_FP32, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fused_row_kernel<VWC_FP32, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_topk_fwd(const TopkPlan &p, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.m)), block(kTopkBlock);
    if (p.dt == VWC_BF16)
        hipLaunchKernelGGL(topk_fwd_kernel<VWC_BF16>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(topk_fwd_kernel<VWC_FP32>, grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_topk_fixup(const TopkPlan &p, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.m)), block(kTopkBlock);
    if (p.dt == VWC_BF16) {
        if (p.gdt == VWC_BF16)
            hipLaunchKernelGGL((topk_fixup_kernel<VWC_BF16, VWC_BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((topk_fixup_kernel<VWC_BF16, VWC_FP32>), grid, block, 0, stream, p);
    } else {
        if (p.gdt == VWC_BF16)
            hipLaunchKernelGGL((topk_fixup_kernel<VWC_FP32, VWC_BF16>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((topk_fixup_kernel<VWC_FP32, VWC_FP32>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_mask_to_index(const uint8_t *mask, int64_t n, int32_t *idx, int32_t *count,
                                hipStream_t stream) {
    hipLaunchKernelGGL(mask_to_index_kernel, dim3(1), dim3(kScanBlock), 0, stream, mask, n, idx,
                       count);
    return hipGetLastError();
}

int64_t mask_tiles(int64_t n) { return (n + kTileItems - 1) / kTileItems; }

hipError_t launch_mask_to_index_tiled(const uint8_t *mask, int64_t n, int32_t *idx,
                                      int32_t *count, int32_t *tiles, hipStream_t stream) {
    const int64_t nt = mask_tiles(n);
    if (nt == 0) {  // empty mask: the count only
        hipLaunchKernelGGL(mask_tile_scan_kernel, dim3(1), dim3(kScanBlock), 0, stream, tiles,
                           nt, count);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(mask_tile_count_kernel, dim3(static_cast<uint32_t>(nt)), dim3(kTileBlock),
                       0, stream, mask, n, tiles);
    hipLaunchKernelGGL(mask_tile_scan_kernel, dim3(1), dim3(kScanBlock), 0, stream, tiles, nt,
                       count);
    hipLaunchKernelGGL(mask_tile_write_kernel, dim3(static_cast<uint32_t>(nt)),
                       dim3(kTileBlock), 0, stream, mask, n, tiles, idx);
    return hipGetLastError();
}

}  // namespace vwc
