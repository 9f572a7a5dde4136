// vwc_internal.h -- launch plans shared by the C-ABI layer and the kernels.
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "vwc.h"

namespace vwc {

// Workgroup sizes (multiples of the 64-lane wave).
#ifndef VWC_FWD_BLOCK
#define VWC_FWD_BLOCK 256
#endif
#ifndef VWC_BWD_BLOCK
#define VWC_BWD_BLOCK 1024
#endif
constexpr int kFwdBlock = VWC_FWD_BLOCK;
constexpr int kBwdBlock = VWC_BWD_BLOCK;
constexpr int kCombineBlock = 64;

// Bytes of one row that one forward workgroup reduces.  A row of `vocab`
// elements is cut into ceil(vocab * e / kFwdSegBytes) segments, a function of
// (vocab, dtype) only, so a row's reduction order never depends on how many
// rows a call covers.  The backward has no reduction; its segment size only
// sets the work per workgroup: rows are cut into ceil(vocab * e /
// kBwdSegBytes) pieces (kBwdSegBytesKL for the top-k KL, kBwdSegBytesWH for
// bf16 rows with the entropy-gradient term, whose heavier arithmetic favours
// longer pieces).  Sizes and rules were chosen by timing on MI355X: with
// 64 KiB pieces a 1024-thread workgroup issues all its loads in one round (at
// most four 16-byte loads per lane), which streamed the default step's bf16
// backward 6.5 % and an fp32 one 7 % faster than pieces of 128-256 KiB.
#ifndef VWC_FWD_SEG_BYTES
#define VWC_FWD_SEG_BYTES (128 * 1024)
#endif
#ifndef VWC_BWD_SEG_BYTES
#define VWC_BWD_SEG_BYTES (64 * 1024)
#endif
#ifndef VWC_BWD_SEG_BYTES_WH
#define VWC_BWD_SEG_BYTES_WH (128 * 1024)
#endif
#ifndef VWC_BWD_SEG_BYTES_KL
#define VWC_BWD_SEG_BYTES_KL (128 * 1024)
#endif
// Segment boundaries fall on multiples of this many 16-byte units from the
// row's first 16-byte boundary, so that every wave's 1 KiB load or store
// covers whole 128-byte lines when the row is so aligned.
#ifndef VWC_SEG_ALIGN_UNITS
#define VWC_SEG_ALIGN_UNITS 64
#endif
constexpr int64_t kSegAlignUnits = VWC_SEG_ALIGN_UNITS;
constexpr int64_t kFwdSegBytes = VWC_FWD_SEG_BYTES;
constexpr int64_t kBwdSegBytes = VWC_BWD_SEG_BYTES;
constexpr int64_t kBwdSegBytesWH = VWC_BWD_SEG_BYTES_WH;  // bf16 rows with the entropy-gradient term
// Rows of the top-k KL backward, whose workgroups each first table the
// payload columns of their segment.
constexpr int64_t kBwdSegBytesKL = VWC_BWD_SEG_BYTES_KL;

// Rows of at most this many forward segments are reduced by one workgroup of
// nseg * kFwdBlock threads that also merges the segment partials (no
// workspace, no second launch); longer rows use one workgroup per segment and
// a combine launch.  Both give the same bits.  1 turns the in-block merge off.
// Timed on MI355X: three segments (768 threads, two workgroups per compute
// unit) beat the two-launch form; four (1024 threads, one workgroup per
// compute unit) lose 6 % on 248320-column bf16 rows to the lower occupancy.
#ifndef VWC_FWD_INBLOCK_MAX
#define VWC_FWD_INBLOCK_MAX 3
#endif
constexpr int kFwdMaxSegPerBlock = VWC_FWD_INBLOCK_MAX;
static_assert(kFwdMaxSegPerBlock >= 1 && kFwdMaxSegPerBlock * VWC_FWD_BLOCK <= 1024,
              "in-block merge exceeds the workgroup size limit");

// Whether a forward over rows of nseg segments needs a workspace.
constexpr bool fwd_needs_workspace(int64_t nseg) {
    return nseg > 1 && nseg > kFwdMaxSegPerBlock;
}

enum TargetMode : int {
    kTargetNone = 0,   // entropy only
    kTargetFull = 1,   // targets index the full row; out of range -> NaN
    kTargetSlice = 2,  // global targets, owned by this slice or -inf
};

// One forward (or partial) launch.
struct FwdPlan {
    const void *logits;       // column 0 of row 0 of the (slice of the) rows
    int64_t ld;               // elements between rows
    int32_t vocab;            // columns handled per row (slice width for partials)
    int64_t v_start;          // global id of column 0 (slice calls), else 0
    const int32_t *targets;   // by row id; null in kTargetNone
    const int32_t *row_idx;   // null: output i is row i
    int64_t n_rows;           // rows of the tensor (row ids are checked against it)
    int64_t m;                // output rows
    int target_mode;
    float c;                  // log2(e) / tau rounded to float
    double tau;               // the float temperature widened
    int nseg;                 // segments per row
    int32_t seg_units;        // 16-byte load units per segment (rows stream from their
                              // first 16-byte boundary; the edges go element-wise)
    bool want_entropy;
    // Final outputs (nseg == 1 and !partial_out), compact [m]:
    float *logprob, *lse, *entropy;
    // Segment partials, [nseg][m] in workspace (when fwd_needs_workspace(nseg)):
    vwc_partial *seg_part;
    // Slice partial output [m] (vwc_vocab_partial):
    vwc_partial *partial_out;
};

struct BwdPlan {
    const void *logits;
    int64_t ld;
    int32_t vocab;
    int dt;                   // vwc_dtype of logits
    int gdt;                  // vwc_dtype of the gradient
    const int32_t *targets;   // by row id
    const int32_t *row_idx;   // null: dense
    int64_t n_rows;
    int64_t m;
    float c_hi, c_lo;         // log2(e) / tau as a float pair (split_scale)
    double tau;
    const float *lse;         // [m]
    const float *grad_out;    // [m] incoming d/d logprob, or null (0)
    const float *entropy;     // [m] the forward's entropy (entropy gradient only)
    const float *grad_ent;    // [m] incoming d/d entropy, or null (0)
    // Top-k KL coefficient mode (kl_P non-null): o_j = q_j * g alpha / tau,
    // alpha from (P, Q, S) of the row; no target column.
    const float *kl_P, *kl_Q, *kl_S;
    int kl_mode;
    double kl_eps;
    // Fused payload columns (kl_fused): the k payload columns of each row
    // (kl_idx, kl_tlp: [m][kl_k]) get beta q_j - kappa p_j in the same pass,
    // so no fix-up launch follows.
    bool kl_fused;
    const int32_t *kl_idx;
    const float *kl_tlp;
    int32_t kl_k;
    void *grad;
    int64_t ld_grad;
    bool grad_by_row_id;      // true: gradient row = row id; false: = output index
    int nseg;
    int32_t seg_units;
    bool vector;              // 16-byte units from each row's first 16-byte boundary
                              // (else one element per unit)
};

// log2(e) / tau as a float pair for the backward's exponent u = x c - B:
// hi is rounded down and lo = c - hi > 0 in float, so x hi + x lo carries c to
// about 2^-48 relative, and a -inf logit gives -inf in both products (never
// -inf + inf).  A lo of exactly 0 becomes a negligible positive value.
struct ScaleSplit {
    float hi, lo;
};
inline ScaleSplit split_scale(double tau) {
    const double c = 1.44269504088896340736 / tau;
    float hi = static_cast<float>(c);
    if (static_cast<double>(hi) > c) hi = nextafterf(hi, 0.f);
    float lo = static_cast<float>(c - static_cast<double>(hi));
    if (!(lo > 0.f)) lo = hi * 0x1p-60f;
    return ScaleSplit{hi, lo};
}

// Forward and backward of one row in one workgroup, the row held on chip
// between them (grad_out known before the forward).  Rows of at most
// kFusedMaxUnits 16-byte units, the gradient in the logits' dtype with rows on
// the same 16-byte phase (the host checks; other calls take fwd + bwd).
constexpr int kFusedBlock = 1024;
constexpr int kFusedLds = 9;    // units per thread staged in LDS (144 KiB)
constexpr int kFusedReg = 22;   // units per thread held in registers
constexpr int64_t kFusedMaxUnits = static_cast<int64_t>(kFusedLds + kFusedReg) * kFusedBlock;

struct FusedPlan {
    const void *logits;
    int64_t ld;
    int32_t vocab;
    int dt;                   // logits and gradient dtype
    const int32_t *targets;   // by row id
    const int32_t *row_idx;   // null: output i is row i
    int64_t n_rows;           // rows of the tensor (row ids are checked against it)
    int64_t m;                // output rows
    float c;                  // log2(e) / tau rounded to float (the reduction)
    float gc_hi, gc_lo;       // log2(e) / tau as a float pair (the gradient; split_scale)
    double tau;
    const float *grad_out;    // [m]
    const float *grad_ent;    // [m] incoming d/d entropy (the entropy-gradient term), or null
    float *logprob, *lse, *entropy;  // [m]; lse non-null, the others nullable
    void *grad;
    int64_t ld_grad;
    bool grad_by_row_id;      // gradient row = row id (dense, scatter) or output index
    // Top-k KL instead of the target's logprob (kl_idx non-null): the payload
    // [m][kl_k] (student columns, teacher log-probs), the objective, and its
    // outputs ([m]; loss nullable); grad_out is then the loss weight.
    const int32_t *kl_idx;
    const float *kl_tlp;
    int32_t kl_k;
    int kl_mode;
    double kl_eps;
    float *kl_loss, *kl_P, *kl_Q, *kl_S;
};

// The fused top-k KL backward keeps a segment's payload columns in an LDS hash
// table of kKlSlots entries, so it takes rows of at most kKlMaxK payload
// columns (load factor <= 1/2), and each thread's units of a segment are
// flagged in one 32-bit mask.
constexpr int kKlSlots = 512;
constexpr int kKlMaxK = kKlSlots / 2;
constexpr int64_t kKlMaxSegUnits = 32 * static_cast<int64_t>(VWC_BWD_BLOCK);

struct CombinePlan {
    const vwc_partial *parts;   // [k][stride]
    int k;
    int64_t stride;
    int64_t rows;
    double tau;
    float *logprob, *lse, *entropy;
    vwc_partial *partial_out;   // merge into partials instead of final outputs
};

// Top-k KL per-row pieces: gathers k student logits per output row.  Output
// i is row row_idx[i] of the logits (row i when row_idx is null); the payload
// and the per-row values are indexed by output.
struct TopkPlan {
    const void *logits;
    int64_t ld;
    int32_t vocab;
    int dt, gdt;
    int64_t n_rows;
    const int32_t *row_idx;    // [m] or null
    int64_t m;                 // output rows
    const int32_t *idx;        // [m][k]
    const float *tlp;          // [m][k]
    int32_t k;
    int mode;
    double eps;
    double tau;
    const float *lse;          // [m]
    // forward outputs (nullable)
    float *loss, *Q, *P, *S;
    // backward (fix-up) inputs/outputs
    const float *inP, *inQ, *inS, *grad_loss;
    void *grad;
    int64_t ld_grad;
    bool grad_by_row_id;       // gradient row = row id (scatter) or output index (compact)
};

// Fused LM head: logits of a tile of kept hidden rows against a tile of the
// output-layer weight on MFMA, folded straight into lane states.
constexpr int kLmTok = 256;        // hidden rows (tokens) per workgroup tile
constexpr int kLmVoc = 256;        // vocabulary rows per tile
#ifndef VWC_LM_K
#define VWC_LM_K 64
#endif
constexpr int kLmK = VWC_LM_K;     // hidden columns per pipeline stage
#ifndef VWC_LM_SEG_TILES
#define VWC_LM_SEG_TILES 4
#endif
// Vocabulary tiles one workgroup folds into one partial; fixed, so the
// reduction order of a row never depends on how many rows a call covers.
constexpr int kLmSegTiles = VWC_LM_SEG_TILES;

struct LmPlan {
    const uint16_t *hidden;   // bf16 kept rows in output order: row i is output i
    int64_t ldh;              // elements between those rows
    int64_t n_rows;           // rows of the caller's hidden tensor (row ids are checked against it)
    const uint16_t *weight;   // bf16 [vocab, ldw]
    int64_t ldw;
    int32_t vocab;
    int32_t d;
    const int32_t *targets;   // by row id; null: no target
    const int32_t *row_idx;   // null: output i is row i
    int64_t m;
    float c;                  // log2(e) / tau rounded to float
    int ntb;                  // token tiles: ceil(m / kLmTok)
    int nvt;                  // vocabulary tiles: ceil(vocab / kLmVoc)
    int nseg;                 // ceil(nvt / kLmSegTiles)
    vwc_partial *seg_part;    // [m][nseg], row-major
};

hipError_t launch_lmhead_fwd(const LmPlan &p, bool want_entropy, hipStream_t stream);
hipError_t launch_gather_rows(const uint16_t *hidden, int64_t ldh, int64_t n_rows,
                              const int32_t *row_idx, int64_t m, int32_t d, uint16_t *out,
                              hipStream_t stream);
hipError_t launch_fwd(const FwdPlan &p, int dt, hipStream_t stream);
hipError_t launch_topk_fwd(const TopkPlan &p, hipStream_t stream);
hipError_t launch_topk_fixup(const TopkPlan &p, hipStream_t stream);
hipError_t launch_bwd(const BwdPlan &p, hipStream_t stream);
hipError_t launch_fused(const FusedPlan &p, hipStream_t stream);
hipError_t launch_combine(const CombinePlan &p, hipStream_t stream);
// Row-major partials ([rows][k]), one wave per row (rows with many segments).
hipError_t launch_combine_rows(const CombinePlan &p, hipStream_t stream);
hipError_t launch_mask_to_index(const uint8_t *mask, int64_t n, int32_t *idx, int32_t *count,
                                hipStream_t stream);
// Tiles of the multi-workgroup scan (one int32 of workspace each).
int64_t mask_tiles(int64_t n);
hipError_t launch_mask_to_index_tiled(const uint8_t *mask, int64_t n, int32_t *idx,
                                      int32_t *count, int32_t *tiles, hipStream_t stream);

}  // namespace vwc
