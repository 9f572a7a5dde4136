// vwc_lmhead.hip -- fused LM head for gfx950: the logits of the kept hidden
// rows against the output-layer weight, computed on MFMA and folded straight
// into log-sum-exp lane states, so no logit ever reaches HBM.
//
// Method (web pages, cited by title and section):
//  * "[Bug] Training/log-prob forward materializes full-vocab fp32 logits over
//    the entire packed sequence ...", maintainer comment: keep only the
//    loss-mask rows of the final hidden state before the vocabulary
//    projection, then compute log-probability and entropy on those rows.
//  * "[RL][Performance] Avoid full-vocabulary TP gather for selected-token
//    logprobs", "Alternatives considered": a fused LM-head / cross-entropy
//    kernel.
//  * "feat: Reduce reference model memory with with parallel logprob
//    computation", "Implementation": per-shard max / sum of exponentials /
//    owned target logit, merged once per row.  Here the shards are the
//    vocabulary segments of one workgroup each.
//
// Design for gfx950:
//  * The kept hidden rows are compacted first (gather_rows_kernel), so a tile
//    of 256 of them is contiguous.
//  * One 512-thread workgroup owns a tile of 256 kept rows (tokens) and a
//    segment of kLmSegTiles vocabulary tiles of 256 rows of the weight.  Its
//    8 waves (2 per SIMD, so each hides the other's stalls) split the
//    256 x 256 logit tile 2 x 4; each wave holds a 128 x 64 block as 4 x 2
//    accumulators of v_mfma_f32_32x32x16_bf16 (128 fp32 per lane).  The
//    product is weight_tile x hidden_tile^T, so in every accumulator lane l
//    holds 16 vocabulary rows of token l % 32.
//  * The hidden dimension streams through LDS in stages of kLmK columns.
//    buffer_load ... lds writes every lane's 16 bytes straight into LDS, from
//    a buffer resource per tile whose size stops at the last valid row, so
//    rows past the vocabulary or past the kept rows read as zero.  Weight
//    tiles use a 3-slot ring and stream in two stages ahead, a few load
//    instructions per k-step; hidden tiles use a 2-slot ring.  Staged rows are
//    128 bytes whose 16-byte chunks are XOR-swizzled, so the MFMA fragment
//    reads (ds_read_b128) hit distinct banks.  One barrier per stage; the
//    fragments of the next k-step are read ahead of the MFMAs of this one.
//  * After the last stage of a vocabulary tile each lane folds its 64 logits
//    per token into the token's lane state (K, m, s, w) with one FMA and one
//    v_exp_f32 per logit; lanes l and l ^ 32 and the two vocabulary halves
//    merge at the end of the segment, and the workgroup writes one 16-byte
//    partial per row.  The split-V combine merges a row's segment partials in
//    segment order in fp64.
//  * Workgroups go to the 8 XCDs in turn; each XCD takes a contiguous block
//    of a work list grouped by a few token tiles, so the workgroups it runs at
//    once share token and weight tiles in its L2.
#include <math.h>
#include <stdint.h>

#include "vwc_internal.h"
#include "vwc_lane.h"

namespace vwc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef VWC_LM_WAVES
#define VWC_LM_WAVES 8
#endif
constexpr int kWaves = VWC_LM_WAVES;              // waves per workgroup: 4 or 8
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                   // token groups (the 2 vocabulary halves
                                                  // times kWN token groups = the waves)
constexpr int kJ = kLmTok / kWN / 32;             // 32-token accumulator columns per wave
constexpr int kRowsPerWave = kLmTok / kWaves;     // staged rows each wave loads per tile
#ifndef VWC_LM_GROUP
#define VWC_LM_GROUP 4
#endif
constexpr int kLmGroup = VWC_LM_GROUP;            // token tiles per group of the work order
constexpr int kRowBytes = kLmK * 2;               // one staged tile row
constexpr int kTileBytes = kLmVoc * kRowBytes;    // one staged operand tile
constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per staged row
constexpr int kRowsPerInst = 1024 / kRowBytes;    // rows one wave load instruction fills
constexpr int kInstPerTile = kRowsPerWave / kRowsPerInst;  // per wave and operand tile
constexpr int kSteps = kLmK / 16;                 // MFMA k-steps per stage
constexpr int kWPerStep = kInstPerTile / kSteps;  // weight load instructions per k-step
// LDS rings of operand tiles, kDist stages deep.  The weight tile of stage
// g + kDist streams in during stage g, kWPerStep load instructions per k-step,
// into the unit stage g - 1 freed; the hidden tile of stage g + kDist goes out
// in stage g's last k-step, into the unit stage g frees.  Spreading the loads
// keeps each wave's memory queue short: a load that cannot issue would hold up
// the MFMAs behind it.
#ifndef VWC_LM_DIST
#define VWC_LM_DIST 2
#endif
constexpr int kDist = VWC_LM_DIST;
constexpr int kWS = kDist + 1;
constexpr int kHS = kDist;
static_assert(kLmTok == kLmVoc, "the staging assumes square tiles");
static_assert(kWaves == 4 || kWaves == 8, "4 waves (1 per SIMD) or 8 (2 per SIMD)");
static_assert(kLmK == 32 || kLmK == 64, "stage widths of 64 or 128 bytes per row");
static_assert(kDist >= 2 && (kWS + kHS) * kTileBytes <= 160 * 1024, "LDS rings too large");
static_assert(kSteps >= 2 && kWPerStep * kSteps == kInstPerTile, "weight loads per k-step");
static_assert((kDist - 1) * 2 * kInstPerTile < 64, "vmcnt range");
constexpr float kUFloor = -256.0f;

// Chunk c (16 bytes) of staged row r sits at chunk position c ^ swz(r), so
// that the rows one group of lanes reads in a cycle (one logical chunk of 8 or
// 16 consecutive rows) land on distinct banks.  swz depends only on r % 16.
__device__ __forceinline__ int swz(int r) {
    if constexpr (kChunks == 8)
        return (r >> 1) & 7;
    else
        return ((r >> 1) ^ (r >> 2)) & 3;
}

// s_waitcnt vmcnt(n), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32); }

// Workgroup barrier without the memory fences of __syncthreads(): the fences
// would also wait for the LDS loads that are meant to stay in flight.  The
// waves' own LDS reads are waited for first (lgkmcnt(0)), so no slot is
// refilled under a read; the loads the barrier must cover are waited for
// explicitly (vmcnt) before it.
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// Fold the logits of token column j of the accumulators into lane state L.
// Row (i, r) of the wave's 128 vocabulary rows is i * 32 + (r / 4) * 8 +
// (l / 32) * 4 + r % 4; with MASK, rows at or past vlim (relative to the
// lane's half) are outside the vocabulary and skipped.
//
// One pass with the lane's current shift K: u = x c - K, s += 2^u, w += 2^u u.
// K is seeded from the lane's first logit and only moves (an exact-maximum
// re-centre over the tile, rarely taken) when the tile's sum leaves
// [0, 2^64] or turns NaN, as in the streaming forward.
constexpr float kTileBound = 0x1p64f;

template <bool MASK, bool ENT>
__device__ __forceinline__ void fold_recentre(const f32x16 (&acc)[4][kJ], int j, float c, int vlim,
                                              Lane &L, float &cs, float &cw) {
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + (r & 3);
            if (!MASK || row < vlim) cm = fmaxf(cm, acc[i][j][r]);
        }
    const float Kn = cm * c;
    if (Kn > L.K) {
        if (L.s != 0.f) {
            const float d = L.K - Kn;
            const float rr = __builtin_amdgcn_exp2f(d);
            L.w = rr * __builtin_fmaf(d, L.s, L.w);
            L.s = rr * L.s;
        }
        L.K = Kn;
        L.m = cm;
    }
    cs = 0.f;
    cw = 0.f;
    if (L.K == -INFINITY) return;  // nothing finite in this lane yet
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + (r & 3);
            if (MASK && row >= vlim) continue;
            const float u = __builtin_fmaf(acc[i][j][r], c, -L.K);
            const float e = __builtin_amdgcn_exp2f(u);
            cs += e;
            if (ENT) cw = __builtin_fmaf(e, fmaxf(u, kUFloor), cw);
        }
}

template <bool MASK, bool ENT>
__device__ __forceinline__ void fold_column(const f32x16 (&acc)[4][kJ], int j, float c, int vlim,
                                            Lane &L) {
    if (L.K == -INFINITY && (!MASK || vlim > 0)) {  // seed with the lane's first logit
        const float x0 = acc[0][j][0];
        if (x0 > -INFINITY) {
            L.m = x0;
            L.K = x0 * c;
        }
    }
    float s0 = 0.f, s1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + (r & 3);
            const float u = __builtin_fmaf(acc[i][j][r], c, -L.K);
            float e = __builtin_amdgcn_exp2f(u);
            if (MASK && row >= vlim) e = 0.f;
            if (r & 1) {
                s1 += e;
                if (ENT) w1 = __builtin_fmaf(e, u, w1);
            } else {
                s0 += e;
                if (ENT) w0 = __builtin_fmaf(e, u, w0);
            }
        }
    }
    float cs = s0 + s1;
    float cw = w0 + w1;
    // Re-centre when the tile needs a new shift, or when masked rows (u
    // possibly infinite while the lane has no shift yet) or -inf logits left a
    // NaN; NaN logits also land there and stay NaN through s.
    if (!(cs <= kTileBound) || (ENT && cw != cw)) fold_recentre<MASK, ENT>(acc, j, c, vlim, L, cs, cw);
    L.s += cs;
    if (ENT) L.w += cw;
}

template <bool ENT, bool RAGGED>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void lmhead_fwd_kernel(LmPlan p) {
    __shared__ __attribute__((aligned(16))) char lds[(kWS + kHS) * kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
    const int wm = wave / kWN;  // vocabulary half of the tile
    const int wn = wave % kWN;  // token group of the tile
    // Work order.  Consecutive workgroups go to the 8 XCDs in turn, and each
    // XCD has its own L2, so XCD x (blockIdx % 8) takes one contiguous block of
    // the work list; the list runs over groups of kLmGroup token tiles, and
    // over the vocabulary segments inside a group.  The workgroups an XCD runs
    // at once then share a few token tiles and a few weight tiles in its L2.
    int tb, seg;
    {
        const int T = p.ntb * p.nseg;
        const int b = static_cast<int>(blockIdx.x);
        const int per = T / 8, rem = T % 8;  // XCDs below rem take per + 1 items
        const int x = b % 8, r = b / 8;
        const int v = r < per ? (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + r
                              : x * (per + 1) + per;
        const int G = min(kLmGroup, p.ntb);
        const int grp = v / (G * p.nseg);
        const int g0 = grp * G;
        const int gs = min(G, p.ntb - g0);  // token tiles in this group
        const int w = v - grp * G * p.nseg;
        seg = w / gs;
        tb = g0 + w % gs;
    }
    const int vt0 = seg * kLmSegTiles;
    const int vt1 = min(vt0 + kLmSegTiles, p.nvt);

    // Staging role.  Stages go from global memory straight into LDS
    // (buffer_load ... lds, 16 bytes per lane): one wave instruction fills
    // 1 KiB, i.e. kRowsPerInst staged rows, lane L writing chunk position
    // L % kChunks of row L / kChunks.  Wave w fills kRowsPerWave rows of both
    // tiles from row kRowsPerWave w on, kRowsPerInst per instruction q, so lane
    // L fetches logical chunk cq[q] = (L % kChunks) ^ swz(row) of row
    // kRowsPerWave w + kRowsPerInst q + L / kChunks.
    const int srow = wave * kRowsPerWave + lane / kChunks;
    int cq[kInstPerTile];
    // Both operands come through buffer resources whose size stops at the last
    // valid row (vocabulary rows of the weight tile, kept rows of the token
    // tile), so rows past it read as zero; chunks past the hidden size are sent
    // out of range too.  The token tile is row tb * 256 of p.hidden, which
    // holds the kept rows in order (compacted beforehand when a row list is
    // given).  Offsets stay below 256 * ld * 2 < 2^31.
    uint32_t aoff[kInstPerTile], hoff[kInstPerTile];
#pragma unroll
    for (int q = 0; q < kInstPerTile; ++q) {
        const int row = srow + kRowsPerInst * q;
        cq[q] = (lane % kChunks) ^ swz(row);
        aoff[q] = static_cast<uint32_t>(row * p.ldw * 2 + cq[q] * 16);
        hoff[q] = static_cast<uint32_t>(row * p.ldh * 2 + cq[q] * 16);
    }
    const int trows = static_cast<int>(min(static_cast<int64_t>(kLmTok),
                                           p.m - static_cast<int64_t>(tb) * kLmTok));
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.hidden + static_cast<int64_t>(tb) * kLmTok * p.ldh), 0,
        static_cast<int>(trows * p.ldh * 2), 0x00020000);

    // MFMA role: fragment rows and the swizzled chunk of each 16-column step.
    const int fr = lane & 31;
    const int fh = lane >> 5;
    const int a_off = (wm * 128 + fr) * kRowBytes;
    const int b_off = (wn * 32 * kJ + fr) * kRowBytes;
    int koff[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) koff[s] = ((2 * s + fh) ^ swz(fr)) << 4;

    // Targets of the lane's kJ token columns (-1: none, or outside the vocabulary).
    int tg[kJ];
    float tv[kJ];
    Lane L[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int64_t i = static_cast<int64_t>(tb) * kLmTok + wn * 32 * kJ + j * 32 + fr;
        tg[j] = -1;
        if (p.targets && i < p.m) {
            const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
            if (r >= 0 && r < p.n_rows) {
                const int32_t t = p.targets[r];
                if (t >= 0 && t < p.vocab) tg[j] = t;
            }
        }
        tv[j] = -INFINITY;
        L[j] = lane_init();
    }

    // Stages run over (vocabulary tile, kLmK-column step) pairs.
    const int nk = (p.d + kLmK - 1) / kLmK;
    const int nstage = (vt1 - vt0) * nk;
    // LDS: kWS weight units, then kHS hidden units, one operand tile each.
    char *const wlds = lds + wave * kRowsPerWave * kRowBytes;   // this wave's rows of unit 0
    char *const hlds = wlds + kWS * kTileBytes;
    const int64_t wtile = static_cast<int64_t>(kLmVoc) * p.ldw;  // elements per weight tile
    // Issue the loads of one operand tile: step k0 of the tile at base `rsrc`,
    // into LDS at `dst` (this wave's rows).  With a hidden size that is not a
    // multiple of kLmK, chunks past it get the top offset bit, which sends them
    // out of range (read as zero).
    auto load_tile = [&](const __amdgpu_buffer_rsrc_t rsrc, const uint32_t (&off)[kInstPerTile],
                         char *dst, int k0, int q0, int nq) {
        const uint32_t kb = static_cast<uint32_t>(k0 * 2);
#pragma unroll
        for (int q = q0; q < q0 + nq; ++q) {
            uint32_t o = off[q] + kb;
            if (RAGGED) o |= k0 + cq[q] * 8 < p.d ? 0u : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + q * kRowsPerInst * kRowBytes, 16,
                                                     o, 0, 0, 0);
        }
    };
    // Weight tiles: a buffer resource per tile (rows of the tile inside the
    // vocabulary).  A stage past the segment's last (its loads are issued to
    // keep the loop free of branches) gets an empty range: no memory is read
    // and the unit, which no later stage uses, receives zeros.
    auto w_rsrc = [&](int vt, bool live) {
        const int rows = live ? min(p.vocab - vt * kLmVoc, kLmVoc) : 0;
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(p.weight + (live ? vt * wtile : 0)), 0,
            rows * static_cast<int>(p.ldw) * 2, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t hr_none = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.hidden), 0, 0, 0x00020000);
    auto load_h = [&](int k, int u, bool live) {
        load_tile(live ? hr : hr_none, hoff, hlds + u * kTileBytes, k * kLmK, 0, kInstPerTile);
    };
    // Fragments of k-step s from weight unit wu and hidden unit hu.
    auto read_frags = [&](int wu, int hu, int s, bf16x8 (&a)[4], bf16x8 (&b)[kJ]) {
        const char *SA = lds + wu * kTileBytes;
        const char *SB = lds + (kWS + hu) * kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const bf16x8 *>(SA + a_off + i * 32 * kRowBytes + koff[s]);
#pragma unroll
        for (int j = 0; j < kJ; ++j)
            b[j] = *reinterpret_cast<const bf16x8 *>(SB + b_off + j * 32 * kRowBytes + koff[s]);
    };

    f32x16 acc[4][kJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kJ; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][4], fb[2][kJ];

    // Prologue: stages 0 .. kDist - 1 whole (hidden tile, then weight tile; the
    // ones past the last stage read nothing), then wait for stage 0.  Every
    // stage issues the same loads, so the counts the waits rely on are exact.
    // (hk) is the step of the next hidden load, (wt, wk) the tile and step of
    // the next weight load.
    int hk = 0, wk = 0, wt = vt0;
    auto step_h = [&]() { hk = hk + 1 == nk ? 0 : hk + 1; };
    auto step_w = [&]() {
        const bool wrap = wk + 1 == nk;
        wk = wrap ? 0 : wk + 1;
        wt += wrap ? 1 : 0;
    };
#pragma unroll
    for (int i = 0; i < kDist; ++i) {
        load_h(hk, i, i < nstage);
        step_h();
        load_tile(w_rsrc(wt, i < nstage), aoff, wlds + i * kTileBytes, wk * kLmK, 0,
                  kInstPerTile);
        step_w();
    }
    wait_vmcnt<(kDist - 1) * 2 * kInstPerTile>();
    __syncthreads();
    if (nstage > 0) read_frags(0, 0, 0, fa[0], fb[0]);

    int g = 0;               // stage being computed
    int wu = 0, hu = 0;      // its units
    for (int vt = vt0; vt < vt1; ++vt) {
        for (int kt = 0; kt < nk; ++kt, ++g) {
            const int nwu = wu + 1 == kWS ? 0 : wu + 1;
            const int nhu = hu + 1 == kHS ? 0 : hu + 1;
            const bool more = g + 1 < nstage;
            // The weight tile of stage g + kDist, unit (g + kDist) % kWS: the one
            // before wu, which stage g - 1 used.
            const __amdgpu_buffer_rsrc_t wr = w_rsrc(wt, g + kDist < nstage);
            char *const wdst = wlds + (wu == 0 ? kWS - 1 : wu - 1) * kTileBytes;
            const int wk0 = wk * kLmK;
            step_w();
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                // Step s of stage g.  The fragments of the next step (step 0 of
                // stage g + 1 after the last step) and this step's share of the
                // weight loads are issued ahead of the step's MFMAs; in the last
                // step, so are the hidden loads that refill stage g's unit.  The
                // fence keeps each step's group in order; the two waves of a
                // SIMD interleave with each other.  (After the last stage the
                // reads touch units nobody refills.)
                const bool next_here = s + 1 < kSteps;
                const bool last = s + 1 == kSteps;
                if (next_here)
                    read_frags(wu, hu, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
                else
                    read_frags(nwu, nhu, 0, fa[0], fb[0]);
                load_tile(wr, aoff, wdst, wk0, s * kWPerStep, kWPerStep);
                if (last) {
                    load_h(hk, hu, g + kHS < nstage);
                    step_h();
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < kJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fa[s & 1][i], fb[s & 1][j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (s == kSteps - 2) {
                    // Every read of stage g's units has been issued by now (the
                    // last step's fragments were read during this step) and the
                    // barrier waits for them.  Stage g + 1's tiles went out in
                    // earlier stages; only the tiles of stages g + 2 .. g +
                    // kDist - 1 and this stage's weight loads (for stage g +
                    // kDist) may still be in flight.
                    if (more)
                        wait_vmcnt<(kDist - 2) * 2 * kInstPerTile + kWPerStep * (kSteps - 1)>();
                    block_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            wu = nwu;
            hu = nhu;
        }

        // Fold the tile's logits into the lane states (the next stages' loads
        // are in flight meanwhile).
        const int vbase = vt * kLmVoc + wm * 128;  // vocabulary id of the wave's row 0
        // Target logits: the lane holding row tg - vbase of its token keeps it.
        bool mine = false;
#pragma unroll
        for (int j = 0; j < kJ; ++j) mine |= static_cast<unsigned>(tg[j] - vbase) < 128u;
        if (__ballot(mine)) {
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const int tl = tg[j] - vbase - fh * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (tl == i * 32 + (r >> 2) * 8 + (r & 3)) tv[j] = acc[i][j][r];
            }
        }
        const int vlim = p.vocab - vbase - fh * 4;
        if (vbase + 128 > p.vocab) {
#pragma unroll
            for (int j = 0; j < kJ; ++j) fold_column<true, ENT>(acc, j, p.c, vlim, L[j]);
        } else {
#pragma unroll
            for (int j = 0; j < kJ; ++j) fold_column<false, ENT>(acc, j, p.c, vlim, L[j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kJ; ++j) acc[i][j] = f32x16{};
    }

    // The last loads (of stages past the segment) must land before the LDS is
    // reused below.
    wait_vmcnt<0>();
    __syncthreads();

    // Lanes l and l ^ 32 hold other rows of the same tokens.
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const Lane o{shfl_xor32(L[j].K), shfl_xor32(L[j].m), shfl_xor32(L[j].s),
                     shfl_xor32(L[j].w)};
        merge(L[j], o);
        tv[j] = fmaxf(tv[j], shfl_xor32(tv[j]));
    }
    // The two vocabulary halves meet in LDS (the stage buffers are free now).
    float *fin = reinterpret_cast<float *>(lds);
    if (wm == 1 && lane < 32) {
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            float *f = fin + ((wn * kJ + j) * 32 + lane) * 5;
            f[0] = L[j].K;
            f[1] = L[j].m;
            f[2] = L[j].s;
            f[3] = L[j].w;
            f[4] = tv[j];
        }
    }
    __syncthreads();
    if (wm != 0 || lane >= 32) return;
    const int64_t v_lo = static_cast<int64_t>(vt0) * kLmVoc;
    const int64_t v_hi = min(static_cast<int64_t>(vt1) * kLmVoc, static_cast<int64_t>(p.vocab));
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const float *f = fin + ((wn * kJ + j) * 32 + lane) * 5;
        merge(L[j], Lane{f[0], f[1], f[2], f[3]});
        const float t_here = fmaxf(tv[j], f[4]);
        const int64_t i = static_cast<int64_t>(tb) * kLmTok + wn * 32 * kJ + j * 32 + lane;
        if (i >= p.m) continue;
        const int64_t r = p.row_idx ? static_cast<int64_t>(p.row_idx[i]) : i;
        vwc_partial out;
        if (r < 0 || r >= p.n_rows) {  // row id outside the hidden rows
            out = vwc_partial{NAN, NAN, NAN, NAN};
        } else {
            double t = -INFINITY;
            if (p.targets) {
                const int64_t tt = p.targets[r];
                if (tt < 0 || tt >= p.vocab) {
                    if (seg == 0) t = NAN;
                } else if (tt >= v_lo && tt < v_hi) {
                    t = t_here;
                }
            }
            const P64 q = to_partial(L[j], p.c, t);
            out = vwc_partial{static_cast<float>(q.m), static_cast<float>(q.s),
                              static_cast<float>(q.t), static_cast<float>(q.w)};
        }
        p.seg_part[i * p.nseg + seg] = out;  // row-major: a row's segments are contiguous
    }
}

// Kept rows of the hidden states, in row-list order, into a dense [m, d]
// array (the pages' compaction at the hidden-state boundary).  Row ids outside
// [0, n_rows) give zero rows; their outputs are written as NaN later.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *hidden, int64_t ldh,
                                                          int64_t n_rows, const int32_t *row_idx,
                                                          int64_t m, int32_t d, uint16_t *out) {
    const int64_t chunks = d / 8;  // 16-byte chunks per row
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= m * chunks) return;
    const int64_t i = t / chunks;
    const int64_t c = t - i * chunks;
    const int64_t r = row_idx[i];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0 && r < n_rows) v = *reinterpret_cast<const u32x4 *>(hidden + r * ldh + c * 8);
    *reinterpret_cast<u32x4 *>(out + i * d + c * 8) = v;
}

}  // namespace

hipError_t launch_gather_rows(const uint16_t *hidden, int64_t ldh, int64_t n_rows,
                              const int32_t *row_idx, int64_t m, int32_t d, uint16_t *out,
                              hipStream_t stream) {
    const int64_t work = m * (d / 8);
    const dim3 grid(static_cast<unsigned>((work + 255) / 256));
    hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, stream, hidden, ldh, n_rows,
                       row_idx, m, d, out);
    return hipGetLastError();
}

hipError_t launch_lmhead_fwd(const LmPlan &p, bool want_entropy, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.ntb) * p.nseg));
    const dim3 block(kThreads);
    const bool ragged = p.d % kLmK != 0;
    if (want_entropy) {
        if (ragged)
            hipLaunchKernelGGL((lmhead_fwd_kernel<true, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((lmhead_fwd_kernel<true, false>), grid, block, 0, stream, p);
    } else {
        if (ragged)
            hipLaunchKernelGGL((lmhead_fwd_kernel<false, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((lmhead_fwd_kernel<false, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace vwc
