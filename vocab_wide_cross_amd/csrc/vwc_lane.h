// vwc_lane.h -- the per-lane log-sum-exp state and the row partial, shared by
// the streaming kernels and the fused LM-head kernel.
//
// A lane state (K, m, s, w) summarises a set of logits x_j of one row:
// s = sum 2^u_j and w = sum 2^u_j * u_j with u_j = x_j * c - K, c = log2(e)/tau,
// and K = fl(m * c) for a reference logit m.  Two states merge exactly up to
// rounding; a state becomes the 16-byte row partial (vwc_partial: reference,
// scaled sum, target logit, entropy sum) that the pages' shard merge joins
// ("feat: Reduce reference model memory with with parallel logprob
// computation", "Implementation").
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace vwc {

constexpr double kLn2 = 0.69314718055994530942;

// ---------------------------------------------------------------- lane state

struct Lane {
    float K;  // shift, log2 units; -inf until the first finite logit
    float m;  // reference logit: K == fl(m * c)
    float s;  // sum of 2^u, u = fl(x * c - K)
    float w;  // sum of 2^u * u (terms with 2^u == 0 add 0)
};

__device__ __forceinline__ Lane lane_init() { return Lane{-INFINITY, -INFINITY, 0.f, 0.f}; }

// Merge lane state b into a (fixed, commutative rule: the larger K is kept).
__device__ __forceinline__ void merge(Lane &a, const Lane &b) {
    const bool swap = b.K > a.K;
    const Lane &big = swap ? b : a;
    const Lane &sml = swap ? a : b;
    const float d = sml.K - big.K;  // <= 0 (NaN when both are empty)
    const float r = __builtin_amdgcn_exp2f(d);
    const bool has = sml.s != 0.f;  // true for NaN too, so NaN propagates
    const float add_s = has ? r * sml.s : 0.f;
    const float add_w = has ? r * __builtin_fmaf(d, sml.s, sml.w) : 0.f;
    Lane o;
    o.K = big.K;
    o.m = (a.K == b.K) ? fmaxf(a.m, b.m) : big.m;
    o.s = big.s + add_s;
    o.w = big.w + add_w;
    a = o;
}

// fp64 view of a partial.
struct P64 {
    double m, s, t, w;
};

// Lane state -> partial relative to its reference logit m (see vwc_partial).
__device__ __forceinline__ P64 to_partial(const Lane &L, float c, double t) {
    P64 p;
    p.t = t;
    if (!(L.s != 0.f)) {  // empty segment
        p.m = -INFINITY;
        p.s = 0.0;
        p.w = 0.0;
        return p;
    }
    // sum 2^{(x - m) c} = 2^rho * s with rho = K - m c, exact in fp64.
    const double rho = static_cast<double>(L.K) - static_cast<double>(L.m) * static_cast<double>(c);
    const double f = exp2(rho);
    p.m = L.m;
    p.s = static_cast<double>(L.s) * f;
    p.w = kLn2 * f * (static_cast<double>(L.w) + rho * static_cast<double>(L.s));
    return p;
}

}  // namespace vwc
