// vwc_api.cpp -- the extern "C" boundary: argument checks (host only, before
// any HIP call), launch planning, status codes.  The arithmetic is in
// vwc_kernels.hip.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "vwc.h"
#include "vwc_internal.h"

namespace {

thread_local std::string g_last_error;

vwc_status fail(vwc_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

vwc_status ok() {
    g_last_error.clear();
    return VWC_OK;
}

vwc_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(VWC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The allocation-free forward's segment partials: one array per GPU in this
// library's code object, held until the process ends.  Host code uses the
// per-device address from hipGetSymbolAddress, never the array's name.
static __device__ __align__(256) unsigned char scratch[VWC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
vwc_status scratch_address(const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(VWC_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(VWC_ERR_UNSUPPORTED, "%s: device ordinal %d beyond %d", fn, dev, kMaxDevices);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(VWC_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn,
                            hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return VWC_OK;
}

bool dtype_ok(int dt) { return dt == VWC_BF16 || dt == VWC_FP32; }
int64_t esize(int dt) { return dt == VWC_BF16 ? 2 : 4; }

// Row segments of a `vocab`-wide row: a function of (vocab, dtype) only.
int64_t segments(int64_t vocab, int dt, int64_t seg_bytes) {
    const int64_t bytes = vocab * esize(dt);
    const int64_t s = (bytes + seg_bytes - 1) / seg_bytes;
    return s < 1 ? 1 : s;
}

// Backward segments: ceil(row bytes / kBwdSegBytes), or kBwdSegBytesKL for
// the top-k KL, or kBwdSegBytesWH for bf16 rows with the entropy-gradient
// term (fp32 rows with that term stream fastest in kBwdSegBytes pieces too).
int64_t bwd_segments(int64_t vocab, int dt, bool entropy_term, bool topk_kl) {
    return segments(vocab, dt,
                    topk_kl                              ? vwc::kBwdSegBytesKL
                    : (entropy_term && dt == VWC_BF16) ? vwc::kBwdSegBytesWH
                                                         : vwc::kBwdSegBytes);
}

// Units per segment: the row's units split into nseg parts, rounded up to a
// multiple of kSegAlignUnits (element-wise rows: no rounding).  The last
// segment takes what is left (possibly nothing but the row's edge elements).
int32_t seg_units_of(int64_t nunits, int64_t nseg, bool vector) {
    int64_t s = (nunits + nseg - 1) / nseg;
    if (vector) s = (s + vwc::kSegAlignUnits - 1) / vwc::kSegAlignUnits * vwc::kSegAlignUnits;
    return static_cast<int32_t>(s < 1 ? 1 : s);
}

bool rows_aligned16(const void *p, int64_t ld, int64_t e) {
    return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((ld * e) % 16 == 0);
}

// The backward streams 16-byte vectors of each logits row from its first
// 16-byte boundary on (`head` elements in) and stores each vector's gradient
// with one store, so that boundary must fall on a 16-byte boundary of the
// row's gradient too.  It does when every row has the same phase on both
// sides (row strides of whole 16-byte multiples and matching bases), or when
// both sides shift by the same bytes from row to row (equal element size and
// stride, the gradient row indexed like the logits row, equal base phase).
bool vector_rows(const void *x, int64_t ld, int64_t e, const void *g, int64_t ld_grad,
                 int64_t ge, bool same_row) {
    const uintptr_t bx = reinterpret_cast<uintptr_t>(x), bg = reinterpret_cast<uintptr_t>(g);
    if ((ld * e) % 16 == 0 && (ld_grad * ge) % 16 == 0) {
        const uintptr_t head = ((16 - bx % 16) % 16) / static_cast<uintptr_t>(e);
        return (bg + head * static_cast<uintptr_t>(ge)) % 16 == 0;
    }
    return same_row && e == ge && ld == ld_grad && bx % 16 == bg % 16;
}

// Common checks of a logits operand.
vwc_status check_logits(const char *fn, const void *logits, int dt, int64_t n_rows, int64_t vocab,
                        int64_t ld, float temperature) {
    if (!dtype_ok(dt)) return fail(VWC_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
    if (n_rows < 0) return fail(VWC_ERR_INVALID_ARG, "%s: n_rows < 0", fn);
    if (vocab <= 0) return fail(VWC_ERR_INVALID_ARG, "%s: vocab must be positive", fn);
    if (ld < vocab) return fail(VWC_ERR_INVALID_ARG, "%s: ld < vocab", fn);
    if (!(temperature > 0.f) || !isfinite(temperature))
        return fail(VWC_ERR_INVALID_ARG, "%s: temperature must be finite and > 0", fn);
    if (vocab > INT32_MAX / 4 || ld > INT64_MAX / 16 / (n_rows > 0 ? n_rows : 1))
        return fail(VWC_ERR_UNSUPPORTED, "%s: vocab or tensor too large", fn);
    if (n_rows > 0 && !logits) return fail(VWC_ERR_INVALID_ARG, "%s: logits is null", fn);
    if (reinterpret_cast<uintptr_t>(logits) % esize(dt) != 0)
        return fail(VWC_ERR_UNSUPPORTED, "%s: logits not aligned to its dtype", fn);
    return VWC_OK;
}

vwc_status check_workspace(const char *fn, int64_t rows, int64_t nseg, const void *ws,
                           size_t ws_bytes) {
    if (!vwc::fwd_needs_workspace(nseg)) return VWC_OK;
    const size_t need = static_cast<size_t>(rows) * static_cast<size_t>(nseg) * sizeof(vwc_partial);
    if (!ws || ws_bytes < need)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    ws ? ws_bytes : static_cast<size_t>(0));
    if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    return VWC_OK;
}

vwc_status check_grid(const char *fn, int64_t rows, int64_t nseg) {
    if (rows > INT32_MAX / nseg)
        return fail(VWC_ERR_UNSUPPORTED, "%s: %lld rows x %lld segments exceed one launch", fn,
                    static_cast<long long>(rows), static_cast<long long>(nseg));
    return VWC_OK;
}

// Shared body of the forward, entropy and partial calls.
vwc_status forward_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                          int64_t vocab, int64_t ld, int64_t v_start, const int32_t *targets,
                          int target_mode, const int32_t *row_idx, int64_t m, float temperature,
                          float *logprob, float *lse, float *entropy, vwc_partial *partial_out,
                          void *workspace, size_t workspace_bytes, hipStream_t stream,
                          bool use_scratch = false) {
    vwc_status st = check_logits(fn, logits, dt, n_rows, vocab, ld, temperature);
    if (st != VWC_OK) return st;
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    if (m == 0) return ok();  // empty row sets: nothing to do (pointers may be null)
    if (!row_idx && m != n_rows)
        return fail(VWC_ERR_INVALID_ARG, "%s: without row_idx, m must equal n_rows", fn);
    if (target_mode == vwc::kTargetFull && !targets && logprob)
        return fail(VWC_ERR_INVALID_ARG, "%s: targets is null", fn);
    if (!partial_out && !logprob && !lse && !entropy)
        return fail(VWC_ERR_INVALID_ARG, "%s: no output requested", fn);
    if (n_rows == 0) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx given but n_rows == 0", fn);

    const int64_t nseg = segments(vocab, dt, vwc::kFwdSegBytes);
    if ((st = check_grid(fn, m, nseg)) != VWC_OK) return st;  // first: bounds m for the sizes below
    if (use_scratch && vwc::fwd_needs_workspace(nseg)) {
        // Every partial the merge reads is written by the same call, so the
        // array needs no clearing.  Its address is the first HIP call.
        const size_t need =
            static_cast<size_t>(m) * static_cast<size_t>(nseg) * sizeof(vwc_partial);
        if (need > VWC_NOALLOC_SCRATCH_BYTES)
            return fail(VWC_ERR_UNSUPPORTED,
                        "%s: %lld rows of %lld segments need %zu bytes of scratch; the "
                        "library holds %zu per GPU (use vwc_selected_logprob_fwd with a "
                        "workspace, or fewer rows per call)",
                        fn, static_cast<long long>(m), static_cast<long long>(nseg), need,
                        static_cast<size_t>(VWC_NOALLOC_SCRATCH_BYTES));
        if ((st = scratch_address(fn, &workspace)) != VWC_OK) return st;
        workspace_bytes = VWC_NOALLOC_SCRATCH_BYTES;
    }
    if ((st = check_workspace(fn, m, nseg, workspace, workspace_bytes)) != VWC_OK) return st;

    vwc::FwdPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.v_start = v_start;
    p.targets = targets;
    p.row_idx = row_idx;
    p.n_rows = n_rows;
    p.m = m;
    // The target logit is read only when a log-probability (or a slice
    // partial with targets) is asked for.
    p.target_mode = target_mode;
    if (target_mode == vwc::kTargetFull && !logprob) p.target_mode = vwc::kTargetNone;
    if (target_mode == vwc::kTargetSlice && !targets) p.target_mode = vwc::kTargetNone;
    p.tau = static_cast<double>(temperature);
    p.c = static_cast<float>(1.44269504088896340736 / p.tau);
    // Every row streams 16-byte vectors from its first 16-byte boundary on.
    const int64_t nunits = vocab / (16 / esize(dt));
    p.nseg = static_cast<int>(nseg);
    p.seg_units = seg_units_of(nunits, nseg, true);
    p.want_entropy = entropy != nullptr || partial_out != nullptr;
    p.logprob = logprob;
    p.lse = lse;
    p.entropy = entropy;
    p.seg_part = vwc::fwd_needs_workspace(nseg) ? static_cast<vwc_partial *>(workspace) : nullptr;
    p.partial_out = partial_out;
    return hip_status(vwc::launch_fwd(p, dt, stream), fn);
}

// The gradient buffer [grad_rows, ld_grad] of grad_dt: aligned, addressable,
// and either exactly the logits (same pointer, dtype and row stride: each
// element is read and then written by the same thread) or disjoint from them.
vwc_status check_grad_buffer(const char *fn, const void *logits, int dt, int64_t n_rows,
                             int64_t vocab, int64_t ld, const void *grad_logits, int grad_dt,
                             int64_t ld_grad, int64_t grad_rows, bool *in_place) {
    if (reinterpret_cast<uintptr_t>(grad_logits) % esize(grad_dt) != 0)
        return fail(VWC_ERR_UNSUPPORTED, "%s: grad_logits not aligned to its dtype", fn);
    if (ld_grad > INT64_MAX / 16 / grad_rows)
        return fail(VWC_ERR_UNSUPPORTED, "%s: gradient tensor too large", fn);
    *in_place = grad_logits == logits && grad_dt == dt && ld_grad == ld;
    if (*in_place) return VWC_OK;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(logits);
    const uintptr_t x1 = x0 + static_cast<uintptr_t>(((n_rows - 1) * ld + vocab) * esize(dt));
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(grad_logits);
    const uintptr_t g1 =
        g0 + static_cast<uintptr_t>(((grad_rows - 1) * ld_grad + vocab) * esize(grad_dt));
    if (g0 < x1 && x0 < g1)
        return fail(VWC_ERR_INVALID_ARG, "%s: grad_logits overlaps logits", fn);
    return VWC_OK;
}

struct KlArgs {
    const float *P, *Q, *S;
    int mode;
    double eps;
    const int32_t *idx;  // payload columns [n_rows][k] and teacher log-probs
    const float *tlp;
    int32_t k;
    bool fused;          // set by backward_common: the payload columns were written too
};

vwc_status backward_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                           int64_t vocab, int64_t ld, const int32_t *targets,
                           const int32_t *row_idx, int64_t m, float temperature, const float *lse,
                           const float *entropy, const float *grad_logprob,
                           const float *grad_entropy, void *grad_logits, int grad_dt,
                           int64_t ld_grad, bool by_row_id, hipStream_t stream,
                           KlArgs *kl = nullptr) {
    vwc_status st = check_logits(fn, logits, dt, n_rows, vocab, ld, temperature);
    if (st != VWC_OK) return st;
    if (!dtype_ok(grad_dt)) return fail(VWC_ERR_INVALID_ARG, "%s: unknown grad dtype", fn);
    if (ld_grad < vocab) return fail(VWC_ERR_INVALID_ARG, "%s: ld_grad < vocab", fn);
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    if (m == 0) return ok();
    if (!row_idx && m != n_rows)
        return fail(VWC_ERR_INVALID_ARG, "%s: without row_idx, m must equal n_rows", fn);
    if (n_rows == 0) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx given but n_rows == 0", fn);
    if (!grad_logprob && !grad_entropy)
        return fail(VWC_ERR_INVALID_ARG, "%s: no incoming gradient", fn);
    if (grad_logprob && !targets && !kl)
        return fail(VWC_ERR_INVALID_ARG, "%s: targets is null", fn);
    if (grad_entropy && !entropy) return fail(VWC_ERR_INVALID_ARG, "%s: entropy is null", fn);
    if (!lse || !grad_logits)
        return fail(VWC_ERR_INVALID_ARG, "%s: null lse or grad_logits", fn);
    const int64_t nseg = bwd_segments(vocab, dt, grad_entropy != nullptr, kl != nullptr);
    if ((st = check_grid(fn, m, nseg)) != VWC_OK) return st;  // first: bounds m for the sizes below
    const int64_t grad_rows = by_row_id ? n_rows : m;
    bool in_place = false;
    st = check_grad_buffer(fn, logits, dt, n_rows, vocab, ld, grad_logits, grad_dt, ld_grad,
                           grad_rows, &in_place);
    if (st != VWC_OK) return st;
    if (in_place && row_idx && !by_row_id)
        return fail(VWC_ERR_INVALID_ARG,
                    "%s: an in-place gradient needs gradient rows indexed by row id", fn);

    vwc::BwdPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.dt = dt;
    p.gdt = grad_dt;
    p.targets = targets;
    p.row_idx = row_idx;
    p.n_rows = n_rows;
    p.m = m;
    p.tau = static_cast<double>(temperature);
    const vwc::ScaleSplit cs = vwc::split_scale(p.tau);
    p.c_hi = cs.hi;
    p.c_lo = cs.lo;
    p.lse = lse;
    p.grad_out = grad_logprob;
    p.entropy = entropy;
    p.grad_ent = grad_entropy;
    if (kl) {
        p.kl_P = kl->P;
        p.kl_Q = kl->Q;
        p.kl_S = kl->S;
        p.kl_mode = kl->mode;
        p.kl_eps = kl->eps;
    }
    p.grad = grad_logits;
    p.ld_grad = ld_grad;
    p.grad_by_row_id = by_row_id;
    const bool aligned = rows_aligned16(logits, ld, esize(dt)) &&
                         rows_aligned16(grad_logits, ld_grad, esize(grad_dt));
    p.vector = vector_rows(logits, ld, esize(dt), grad_logits, ld_grad, esize(grad_dt),
                           !row_idx || by_row_id);
    const int64_t unit = p.vector ? 16 / esize(dt) : 1;
    const int64_t nunits = vocab / unit;
    p.nseg = static_cast<int>(nseg);
    p.seg_units = seg_units_of(nunits, nseg, p.vector);
    if (kl) {
        // The payload columns go into the same pass when the rows are 16-byte
        // vectors and a segment's payload fits the in-LDS table; otherwise the
        // caller runs the fix-up launch.
        kl->fused = aligned && kl->k <= vwc::kKlMaxK && p.seg_units <= vwc::kKlMaxSegUnits;
        // The fix-up launch re-reads payload logits after the stream wrote them.
        if (in_place && !kl->fused)
            return fail(VWC_ERR_UNSUPPORTED,
                        "%s: an in-place top-k KL gradient needs rows on 16 bytes and k <= %d",
                        fn, vwc::kKlMaxK);
        p.kl_fused = kl->fused;
        p.kl_idx = kl->idx;
        p.kl_tlp = kl->tlp;
        p.kl_k = kl->k;
    }
    return hip_status(vwc::launch_bwd(p, stream), fn);
}

}  // namespace

extern "C" {

size_t vwc_workspace_bytes(int64_t rows, int64_t vocab, vwc_dtype dt) {
    if (rows <= 0 || vocab <= 0 || !dtype_ok(dt)) return 0;
    const int64_t nseg = segments(vocab, dt, vwc::kFwdSegBytes);
    if (!vwc::fwd_needs_workspace(nseg)) return 0;
    return static_cast<size_t>(rows) * static_cast<size_t>(nseg) * sizeof(vwc_partial);
}

vwc_status vwc_selected_logprob_fwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *targets,
                                    float temperature, float *logprob, float *lse,
                                    float *entropy, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    return forward_common("vwc_selected_logprob_fwd", logits, dt, n_rows, vocab, ld, 0, targets,
                          vwc::kTargetFull, nullptr, n_rows, temperature, logprob, lse, entropy,
                          nullptr, workspace, workspace_bytes, stream);
}

vwc_status vwc_selected_logprob_fwd_noalloc(const void *logits, vwc_dtype dt, int64_t n_rows,
                                            int64_t vocab, int64_t ld, const int32_t *targets,
                                            float temperature, float *logprob, float *lse,
                                            float *entropy, hipStream_t stream) {
    return forward_common("vwc_selected_logprob_fwd_noalloc", logits, dt, n_rows, vocab, ld, 0,
                          targets, vwc::kTargetFull, nullptr, n_rows, temperature, logprob, lse,
                          entropy, nullptr, nullptr, 0, stream, /*use_scratch=*/true);
}

vwc_status vwc_selected_logprob_fwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                         int64_t vocab, int64_t ld, const int32_t *targets,
                                         const int32_t *row_idx, int64_t m, float temperature,
                                         float *logprob, float *lse, float *entropy,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    if (m > 0 && !row_idx)
        return fail(VWC_ERR_INVALID_ARG, "vwc_selected_logprob_fwd_rows: row_idx is null");
    return forward_common("vwc_selected_logprob_fwd_rows", logits, dt, n_rows, vocab, ld, 0,
                          targets, vwc::kTargetFull, row_idx, m, temperature, logprob, lse,
                          entropy, nullptr, workspace, workspace_bytes, stream);
}

vwc_status vwc_entropy(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                       int64_t ld, float temperature, float *entropy, float *lse,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n_rows > 0 && !entropy) return fail(VWC_ERR_INVALID_ARG, "vwc_entropy: entropy is null");
    return forward_common("vwc_entropy", logits, dt, n_rows, vocab, ld, 0, nullptr,
                          vwc::kTargetNone, nullptr, n_rows, temperature, nullptr, lse, entropy,
                          nullptr, workspace, workspace_bytes, stream);
}

vwc_status vwc_entropy_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                            int64_t ld, const int32_t *row_idx, int64_t m, float temperature,
                            float *entropy, float *lse, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "vwc_entropy_rows: row_idx is null");
    if (m > 0 && !entropy) return fail(VWC_ERR_INVALID_ARG, "vwc_entropy_rows: entropy is null");
    return forward_common("vwc_entropy_rows", logits, dt, n_rows, vocab, ld, 0, nullptr,
                          vwc::kTargetNone, row_idx, m, temperature, nullptr, lse, entropy,
                          nullptr, workspace, workspace_bytes, stream);
}

vwc_status vwc_selected_logprob_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *targets,
                                    float temperature, const float *lse,
                                    const float *grad_logprob, void *grad_logits,
                                    vwc_dtype grad_dt, int64_t ld_grad, hipStream_t stream) {
    if (n_rows > 0 && !grad_logprob)
        return fail(VWC_ERR_INVALID_ARG, "vwc_selected_logprob_bwd: grad_logprob is null");
    return backward_common("vwc_selected_logprob_bwd", logits, dt, n_rows, vocab, ld, targets,
                           nullptr, n_rows, temperature, lse, nullptr, grad_logprob, nullptr,
                           grad_logits, grad_dt, ld_grad, true, stream);
}

// Shared body of the one-call forward + backward, dense (row_idx null) or over
// a row set (outputs and grad_logprob compact [m]; the gradient row is the row
// id with by_row_id, else the output index).
static vwc_status fwd_bwd_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                                 int64_t vocab, int64_t ld, const int32_t *targets,
                                 const int32_t *row_idx, int64_t m, float temperature,
                                 const float *grad_logprob, const float *grad_entropy,
                                 float *logprob, float *lse, float *entropy, void *grad_logits,
                                 int grad_dt, int64_t ld_grad, bool by_row_id, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    vwc_status st = check_logits(fn, logits, dt, n_rows, vocab, ld, temperature);
    if (st != VWC_OK) return st;
    if (!dtype_ok(grad_dt)) return fail(VWC_ERR_INVALID_ARG, "%s: unknown grad dtype", fn);
    if (ld_grad < vocab) return fail(VWC_ERR_INVALID_ARG, "%s: ld_grad < vocab", fn);
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    if (m == 0) return ok();
    if (!row_idx && m != n_rows)
        return fail(VWC_ERR_INVALID_ARG, "%s: without row_idx, m must equal n_rows", fn);
    if (n_rows == 0) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx given but n_rows == 0", fn);
    if (!grad_entropy) {
        if (!targets || !grad_logprob || !lse || !grad_logits)
            return fail(VWC_ERR_INVALID_ARG,
                        "%s: null targets, grad_logprob, lse or grad_logits", fn);
    } else {
        // The entropy-gradient term: g may be absent (0), and then the targets too
        // unless logprob is asked for; the entropy is an output the gradient needs.
        if (!lse || !entropy || !grad_logits)
            return fail(VWC_ERR_INVALID_ARG, "%s: null lse, entropy or grad_logits", fn);
        if ((grad_logprob || logprob) && !targets)
            return fail(VWC_ERR_INVALID_ARG, "%s: targets is null", fn);
    }
    if (m > INT32_MAX) return fail(VWC_ERR_UNSUPPORTED, "%s: too many rows", fn);
    const int64_t e = esize(dt);
    bool in_place = false;
    st = check_grad_buffer(fn, logits, dt, n_rows, vocab, ld, grad_logits, grad_dt, ld_grad,
                           by_row_id ? n_rows : m, &in_place);
    if (st != VWC_OK) return st;
    if (in_place && row_idx && !by_row_id)
        return fail(VWC_ERR_INVALID_ARG,
                    "%s: an in-place gradient needs gradient rows indexed by row id", fn);
    // One workgroup holds a whole row on chip when it fits and each gradient
    // row shares its logits row's dtype and 16-byte phase; otherwise the
    // forward and the backward run as their own calls (same results, one more
    // read of the rows).
    const bool fused = grad_dt == dt && vocab / (16 / e) <= vwc::kFusedMaxUnits &&
                       vector_rows(logits, ld, e, grad_logits, ld_grad, e, !row_idx || by_row_id);
    if (!fused) {
        st = forward_common(fn, logits, dt, n_rows, vocab, ld, 0, targets, vwc::kTargetFull,
                            row_idx, m, temperature, logprob, lse, entropy, nullptr, workspace,
                            workspace_bytes, stream);
        if (st != VWC_OK) return st;
        return backward_common(fn, logits, dt, n_rows, vocab, ld, targets, row_idx, m,
                               temperature, lse, grad_entropy ? entropy : nullptr, grad_logprob,
                               grad_entropy, grad_logits, grad_dt, ld_grad, by_row_id, stream);
    }
    vwc::FusedPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.dt = dt;
    p.targets = targets;
    p.row_idx = row_idx;
    p.n_rows = n_rows;
    p.m = m;
    p.tau = static_cast<double>(temperature);
    p.c = static_cast<float>(1.44269504088896340736 / p.tau);
    const vwc::ScaleSplit cs = vwc::split_scale(p.tau);
    p.gc_hi = cs.hi;
    p.gc_lo = cs.lo;
    p.grad_out = grad_logprob;
    p.grad_ent = grad_entropy;
    p.logprob = logprob;
    p.lse = lse;
    p.entropy = entropy;
    p.grad = grad_logits;
    p.ld_grad = ld_grad;
    p.grad_by_row_id = by_row_id;
    return hip_status(vwc::launch_fused(p, stream), fn);
}

vwc_status vwc_selected_logprob_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                        int64_t vocab, int64_t ld, const int32_t *targets,
                                        float temperature, const float *grad_logprob,
                                        float *logprob, float *lse, float *entropy,
                                        void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return fwd_bwd_common("vwc_selected_logprob_fwd_bwd", logits, dt, n_rows, vocab, ld, targets,
                          nullptr, n_rows, temperature, grad_logprob, nullptr, logprob, lse,
                          entropy, grad_logits, grad_dt, ld_grad, true, workspace,
                          workspace_bytes, stream);
}

vwc_status vwc_logprob_entropy_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                       int64_t vocab, int64_t ld, const int32_t *targets,
                                       float temperature, const float *grad_logprob,
                                       const float *grad_entropy, float *logprob, float *lse,
                                       float *entropy, void *grad_logits, vwc_dtype grad_dt,
                                       int64_t ld_grad, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    const char *fn = "vwc_logprob_entropy_fwd_bwd";
    if (!grad_entropy) return fail(VWC_ERR_INVALID_ARG, "%s: grad_entropy is null", fn);
    return fwd_bwd_common(fn, logits, dt, n_rows, vocab, ld, targets, nullptr, n_rows,
                          temperature, grad_logprob, grad_entropy, logprob, lse, entropy,
                          grad_logits, grad_dt, ld_grad, true, workspace, workspace_bytes,
                          stream);
}

vwc_status vwc_selected_logprob_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                             int64_t vocab, int64_t ld, const int32_t *targets,
                                             const int32_t *row_idx, int64_t m,
                                             float temperature, const float *grad_logprob,
                                             float *logprob, float *lse, float *entropy,
                                             void *grad_logits, vwc_dtype grad_dt,
                                             int64_t ld_grad, vwc_grad_layout layout,
                                             void *workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
    const char *fn = "vwc_selected_logprob_fwd_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    return fwd_bwd_common(fn, logits, dt, n_rows, vocab, ld, targets, row_idx, m, temperature,
                          grad_logprob, nullptr, logprob, lse, entropy, grad_logits, grad_dt,
                          ld_grad, layout == VWC_GRAD_SCATTER, workspace, workspace_bytes,
                          stream);
}

vwc_status vwc_logprob_entropy_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                            int64_t vocab, int64_t ld, const int32_t *targets,
                                            const int32_t *row_idx, int64_t m, float temperature,
                                            const float *grad_logprob, const float *grad_entropy,
                                            float *logprob, float *lse, float *entropy,
                                            void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                            vwc_grad_layout layout, void *workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_logprob_entropy_fwd_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    if (!grad_entropy) return fail(VWC_ERR_INVALID_ARG, "%s: grad_entropy is null", fn);
    return fwd_bwd_common(fn, logits, dt, n_rows, vocab, ld, targets, row_idx, m, temperature,
                          grad_logprob, grad_entropy, logprob, lse, entropy, grad_logits, grad_dt,
                          ld_grad, layout == VWC_GRAD_SCATTER, workspace, workspace_bytes,
                          stream);
}

vwc_status vwc_selected_logprob_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                         int64_t vocab, int64_t ld, const int32_t *targets,
                                         const int32_t *row_idx, int64_t m, float temperature,
                                         const float *lse, const float *grad_logprob,
                                         void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                         vwc_grad_layout layout, hipStream_t stream) {
    const char *fn = "vwc_selected_logprob_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    if (m > 0 && !grad_logprob) return fail(VWC_ERR_INVALID_ARG, "%s: grad_logprob is null", fn);
    return backward_common(fn, logits, dt, n_rows, vocab, ld, targets, row_idx, m, temperature,
                           lse, nullptr, grad_logprob, nullptr, grad_logits, grad_dt, ld_grad,
                           layout == VWC_GRAD_SCATTER, stream);
}

vwc_status vwc_logprob_entropy_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                   int64_t ld, const int32_t *targets, float temperature,
                                   const float *lse, const float *entropy,
                                   const float *grad_logprob, const float *grad_entropy,
                                   void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                   hipStream_t stream) {
    return backward_common("vwc_logprob_entropy_bwd", logits, dt, n_rows, vocab, ld, targets,
                           nullptr, n_rows, temperature, lse, entropy, grad_logprob, grad_entropy,
                           grad_logits, grad_dt, ld_grad, true, stream);
}

vwc_status vwc_logprob_entropy_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                        int64_t vocab, int64_t ld, const int32_t *targets,
                                        const int32_t *row_idx, int64_t m, float temperature,
                                        const float *lse, const float *entropy,
                                        const float *grad_logprob, const float *grad_entropy,
                                        void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                        vwc_grad_layout layout, hipStream_t stream) {
    const char *fn = "vwc_logprob_entropy_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    return backward_common(fn, logits, dt, n_rows, vocab, ld, targets, row_idx, m, temperature,
                           lse, entropy, grad_logprob, grad_entropy, grad_logits, grad_dt,
                           ld_grad, layout == VWC_GRAD_SCATTER, stream);
}

static vwc_status check_topk(const char *fn, const int32_t *topk_idx, const float *tlp, int32_t k,
                             int64_t vocab, int mode, float eps, int64_t n_rows) {
    if (k <= 0 || k > vocab) return fail(VWC_ERR_INVALID_ARG, "%s: k must be in [1, vocab]", fn);
    if (mode != VWC_KL_TRUNCATED && mode != VWC_KL_TAIL)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown mode %d", fn, mode);
    if (mode == VWC_KL_TAIL && !(eps > 0.f && eps < 1.f))
        return fail(VWC_ERR_INVALID_ARG, "%s: tail_mass_eps must lie in (0, 1)", fn);
    if (n_rows > 0 && (!topk_idx || !tlp))
        return fail(VWC_ERR_INVALID_ARG, "%s: null topk_idx or teacher_logprob", fn);
    if (n_rows > INT32_MAX) return fail(VWC_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (static_cast<int64_t>(k) * n_rows > INT64_MAX / 8)
        return fail(VWC_ERR_UNSUPPORTED, "%s: payload too large", fn);
    return VWC_OK;
}

// Shared bodies of the dense and row-set top-k KL calls: row_idx null means
// output i is row i (m == n_rows); the payload and the per-row values are
// indexed by output.
static vwc_status topk_fwd_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                                  int64_t vocab, int64_t ld, const int32_t *row_idx, int64_t m,
                                  const int32_t *topk_idx, const float *teacher_logprob,
                                  int32_t k, int mode, float tail_mass_eps, float temperature,
                                  float *loss, float *student_mass, float *teacher_mass,
                                  float *topk_sum, float *lse, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    vwc_status st = check_logits(fn, logits, dt, n_rows, vocab, ld, temperature);
    if (st != VWC_OK) return st;
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    if ((st = check_topk(fn, topk_idx, teacher_logprob, k, vocab, mode, tail_mass_eps, m)) !=
        VWC_OK)
        return st;
    if (m == 0) return ok();
    if (!lse) return fail(VWC_ERR_INVALID_ARG, "%s: lse is null", fn);
    st = forward_common(fn, logits, dt, n_rows, vocab, ld, 0, nullptr, vwc::kTargetNone, row_idx,
                        m, temperature, nullptr, lse, nullptr, nullptr, workspace,
                        workspace_bytes, stream);
    if (st != VWC_OK) return st;
    vwc::TopkPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.dt = dt;
    p.n_rows = n_rows;
    p.row_idx = row_idx;
    p.m = m;
    p.idx = topk_idx;
    p.tlp = teacher_logprob;
    p.k = k;
    p.mode = mode;
    p.eps = tail_mass_eps;
    p.tau = temperature;
    p.lse = lse;
    p.loss = loss;
    p.Q = student_mass;
    p.P = teacher_mass;
    p.S = topk_sum;
    return hip_status(vwc::launch_topk_fwd(p, stream), fn);
}

static vwc_status topk_bwd_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                                  int64_t vocab, int64_t ld, const int32_t *row_idx, int64_t m,
                                  const int32_t *topk_idx, const float *teacher_logprob,
                                  int32_t k, int mode, float tail_mass_eps, float temperature,
                                  const float *lse, const float *student_mass,
                                  const float *teacher_mass, const float *topk_sum,
                                  const float *grad_loss, void *grad_logits, int grad_dt,
                                  int64_t ld_grad, bool by_row_id, hipStream_t stream) {
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    vwc_status st = check_topk(fn, topk_idx, teacher_logprob, k, vocab, mode, tail_mass_eps, m);
    if (st != VWC_OK) return st;
    if (m > 0 && (!student_mass || !teacher_mass || !topk_sum || !grad_loss))
        return fail(VWC_ERR_INVALID_ARG,
                    "%s: null student_mass, teacher_mass, topk_sum or grad_loss", fn);
    KlArgs kl{teacher_mass, student_mass, topk_sum, mode, tail_mass_eps,
              topk_idx, teacher_logprob, k, false};
    st = backward_common(fn, logits, dt, n_rows, vocab, ld, nullptr, row_idx, m, temperature, lse,
                         nullptr, grad_loss, nullptr, grad_logits, grad_dt, ld_grad, by_row_id,
                         stream, &kl);
    if (st != VWC_OK || m == 0 || kl.fused) return st;
    vwc::TopkPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.dt = dt;
    p.gdt = grad_dt;
    p.n_rows = n_rows;
    p.row_idx = row_idx;
    p.m = m;
    p.grad_by_row_id = by_row_id;
    p.idx = topk_idx;
    p.tlp = teacher_logprob;
    p.k = k;
    p.mode = mode;
    p.eps = tail_mass_eps;
    p.tau = temperature;
    p.lse = lse;
    p.inP = teacher_mass;
    p.inQ = student_mass;
    p.inS = topk_sum;
    p.grad_loss = grad_loss;
    p.grad = grad_logits;
    p.ld_grad = ld_grad;
    return hip_status(vwc::launch_topk_fixup(p, stream), fn);
}

vwc_status vwc_topk_kl_fwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                           int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                           int32_t k, vwc_kl_mode mode, float tail_mass_eps, float temperature,
                           float *loss, float *student_mass, float *teacher_mass, float *topk_sum,
                           float *lse, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    return topk_fwd_common("vwc_topk_kl_fwd", logits, dt, n_rows, vocab, ld, nullptr, n_rows,
                           topk_idx, teacher_logprob, k, mode, tail_mass_eps, temperature, loss,
                           student_mass, teacher_mass, topk_sum, lse, workspace, workspace_bytes,
                           stream);
}

vwc_status vwc_topk_kl_fwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                int64_t ld, const int32_t *row_idx, int64_t m,
                                const int32_t *topk_idx, const float *teacher_logprob, int32_t k,
                                vwc_kl_mode mode, float tail_mass_eps, float temperature,
                                float *loss, float *student_mass, float *teacher_mass,
                                float *topk_sum, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_topk_kl_fwd_rows";
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    return topk_fwd_common(fn, logits, dt, n_rows, vocab, ld, row_idx, m, topk_idx,
                           teacher_logprob, k, mode, tail_mass_eps, temperature, loss,
                           student_mass, teacher_mass, topk_sum, lse, workspace, workspace_bytes,
                           stream);
}

vwc_status vwc_topk_kl_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                           int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                           int32_t k, vwc_kl_mode mode, float tail_mass_eps, float temperature,
                           const float *lse, const float *student_mass, const float *teacher_mass,
                           const float *topk_sum, const float *grad_loss, void *grad_logits,
                           vwc_dtype grad_dt, int64_t ld_grad, hipStream_t stream) {
    return topk_bwd_common("vwc_topk_kl_bwd", logits, dt, n_rows, vocab, ld, nullptr, n_rows,
                           topk_idx, teacher_logprob, k, mode, tail_mass_eps, temperature, lse,
                           student_mass, teacher_mass, topk_sum, grad_loss, grad_logits, grad_dt,
                           ld_grad, true, stream);
}

vwc_status vwc_topk_kl_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                int64_t ld, const int32_t *row_idx, int64_t m,
                                const int32_t *topk_idx, const float *teacher_logprob, int32_t k,
                                vwc_kl_mode mode, float tail_mass_eps, float temperature,
                                const float *lse, const float *student_mass,
                                const float *teacher_mass, const float *topk_sum,
                                const float *grad_loss, void *grad_logits, vwc_dtype grad_dt,
                                int64_t ld_grad, vwc_grad_layout layout, hipStream_t stream) {
    const char *fn = "vwc_topk_kl_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    return topk_bwd_common(fn, logits, dt, n_rows, vocab, ld, row_idx, m, topk_idx,
                           teacher_logprob, k, mode, tail_mass_eps, temperature, lse,
                           student_mass, teacher_mass, topk_sum, grad_loss, grad_logits, grad_dt,
                           ld_grad, layout == VWC_GRAD_SCATTER, stream);
}

static vwc_status topk_fwd_bwd_common(const char *fn, const void *logits, int dt, int64_t n_rows,
                                      int64_t vocab, int64_t ld, const int32_t *row_idx,
                                      int64_t m, const int32_t *topk_idx,
                                      const float *teacher_logprob, int32_t k, int mode,
                                      float tail_mass_eps, float temperature,
                                      const float *grad_loss, float *loss, float *student_mass,
                                      float *teacher_mass, float *topk_sum, float *lse,
                                      void *grad_logits, int grad_dt, int64_t ld_grad,
                                      bool by_row_id, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    vwc_status st = check_logits(fn, logits, dt, n_rows, vocab, ld, temperature);
    if (st != VWC_OK) return st;
    if (m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: m < 0", fn);
    if ((st = check_topk(fn, topk_idx, teacher_logprob, k, vocab, mode, tail_mass_eps, m)) !=
        VWC_OK)
        return st;
    if (!dtype_ok(grad_dt)) return fail(VWC_ERR_INVALID_ARG, "%s: unknown grad dtype", fn);
    if (ld_grad < vocab) return fail(VWC_ERR_INVALID_ARG, "%s: ld_grad < vocab", fn);
    if (m == 0) return ok();
    if (!row_idx && m != n_rows)
        return fail(VWC_ERR_INVALID_ARG, "%s: without row_idx, m must equal n_rows", fn);
    if (n_rows == 0) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx given but n_rows == 0", fn);
    if (!grad_loss || !lse || !student_mass || !teacher_mass || !topk_sum || !grad_logits)
        return fail(VWC_ERR_INVALID_ARG,
                    "%s: null grad_loss, lse, student_mass, teacher_mass, topk_sum or grad_logits",
                    fn);
    const int64_t e = esize(dt);
    bool in_place = false;
    st = check_grad_buffer(fn, logits, dt, n_rows, vocab, ld, grad_logits, grad_dt, ld_grad,
                           by_row_id ? n_rows : m, &in_place);
    if (st != VWC_OK) return st;
    if (in_place && row_idx && !by_row_id)
        return fail(VWC_ERR_INVALID_ARG,
                    "%s: an in-place gradient needs gradient rows indexed by row id", fn);
    // One workgroup per row with the row on chip, as the logprob one-call;
    // otherwise the forward and the backward as their own calls.
    const bool fused = grad_dt == dt && k <= vwc::kKlMaxK &&
                       vocab / (16 / e) <= vwc::kFusedMaxUnits &&
                       vector_rows(logits, ld, e, grad_logits, ld_grad, e, !row_idx || by_row_id);
    if (!fused) {
        // In place, the separate backward must write the payload columns in its
        // own pass (checked here, before anything runs).
        if (in_place && !(k <= vwc::kKlMaxK && rows_aligned16(logits, ld, e) &&
                          rows_aligned16(grad_logits, ld_grad, esize(grad_dt))))
            return fail(VWC_ERR_UNSUPPORTED,
                        "%s: an in-place top-k KL gradient needs rows on 16 bytes and k <= %d",
                        fn, vwc::kKlMaxK);
        st = topk_fwd_common(fn, logits, dt, n_rows, vocab, ld, row_idx, m, topk_idx,
                             teacher_logprob, k, mode, tail_mass_eps, temperature, loss,
                             student_mass, teacher_mass, topk_sum, lse, workspace,
                             workspace_bytes, stream);
        if (st != VWC_OK) return st;
        return topk_bwd_common(fn, logits, dt, n_rows, vocab, ld, row_idx, m, topk_idx,
                               teacher_logprob, k, mode, tail_mass_eps, temperature, lse,
                               student_mass, teacher_mass, topk_sum, grad_loss, grad_logits,
                               grad_dt, ld_grad, by_row_id, stream);
    }
    if (m > INT32_MAX) return fail(VWC_ERR_UNSUPPORTED, "%s: too many rows", fn);
    vwc::FusedPlan p{};
    p.logits = logits;
    p.ld = ld;
    p.vocab = static_cast<int32_t>(vocab);
    p.dt = dt;
    p.row_idx = row_idx;
    p.n_rows = n_rows;
    p.m = m;
    p.tau = static_cast<double>(temperature);
    p.c = static_cast<float>(1.44269504088896340736 / p.tau);
    const vwc::ScaleSplit cs = vwc::split_scale(p.tau);
    p.gc_hi = cs.hi;
    p.gc_lo = cs.lo;
    p.grad_out = grad_loss;
    p.lse = lse;
    p.grad = grad_logits;
    p.ld_grad = ld_grad;
    p.grad_by_row_id = by_row_id;
    p.kl_idx = topk_idx;
    p.kl_tlp = teacher_logprob;
    p.kl_k = k;
    p.kl_mode = mode;
    p.kl_eps = tail_mass_eps;
    p.kl_loss = loss;
    p.kl_P = teacher_mass;
    p.kl_Q = student_mass;
    p.kl_S = topk_sum;
    return hip_status(vwc::launch_fused(p, stream), fn);
}

vwc_status vwc_topk_kl_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                               int32_t k, vwc_kl_mode mode, float tail_mass_eps,
                               float temperature, const float *grad_loss, float *loss,
                               float *student_mass, float *teacher_mass, float *topk_sum,
                               float *lse, void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return topk_fwd_bwd_common("vwc_topk_kl_fwd_bwd", logits, dt, n_rows, vocab, ld, nullptr,
                               n_rows, topk_idx, teacher_logprob, k, mode, tail_mass_eps,
                               temperature, grad_loss, loss, student_mass, teacher_mass,
                               topk_sum, lse, grad_logits, grad_dt, ld_grad, true, workspace,
                               workspace_bytes, stream);
}

vwc_status vwc_topk_kl_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *row_idx, int64_t m,
                                    const int32_t *topk_idx, const float *teacher_logprob,
                                    int32_t k, vwc_kl_mode mode, float tail_mass_eps,
                                    float temperature, const float *grad_loss, float *loss,
                                    float *student_mass, float *teacher_mass, float *topk_sum,
                                    float *lse, void *grad_logits, vwc_dtype grad_dt,
                                    int64_t ld_grad, vwc_grad_layout layout, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_topk_kl_fwd_bwd_rows";
    if (layout != VWC_GRAD_COMPACT && layout != VWC_GRAD_SCATTER)
        return fail(VWC_ERR_INVALID_ARG, "%s: unknown layout %d", fn, static_cast<int>(layout));
    if (m > 0 && !row_idx) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx is null", fn);
    return topk_fwd_bwd_common(fn, logits, dt, n_rows, vocab, ld, row_idx, m, topk_idx,
                               teacher_logprob, k, mode, tail_mass_eps, temperature, grad_loss,
                               loss, student_mass, teacher_mass, topk_sum, lse, grad_logits,
                               grad_dt, ld_grad, layout == VWC_GRAD_SCATTER, workspace,
                               workspace_bytes, stream);
}

vwc_status vwc_vocab_partial(const void *logits_slice, vwc_dtype dt, int64_t n_rows,
                             int64_t v_local, int64_t ld, int64_t v_start,
                             const int32_t *targets, const int32_t *row_idx, int64_t m,
                             float temperature, vwc_partial *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_vocab_partial";
    if (v_start < 0) return fail(VWC_ERR_INVALID_ARG, "%s: v_start < 0", fn);
    if (m > 0 && !out) return fail(VWC_ERR_INVALID_ARG, "%s: out is null", fn);
    return forward_common(fn, logits_slice, dt, n_rows, v_local, ld, v_start, targets,
                          vwc::kTargetSlice, row_idx, m, temperature, nullptr, nullptr, nullptr,
                          out, workspace, workspace_bytes, stream);
}

vwc_status vwc_partial_combine(const vwc_partial *parts, int32_t k, int64_t rows,
                               float temperature, float *logprob, float *lse, float *entropy,
                               hipStream_t stream) {
    const char *fn = "vwc_partial_combine";
    if (k <= 0) return fail(VWC_ERR_INVALID_ARG, "%s: k must be positive", fn);
    if (rows < 0) return fail(VWC_ERR_INVALID_ARG, "%s: rows < 0", fn);
    if (!(temperature > 0.f) || !isfinite(temperature))
        return fail(VWC_ERR_INVALID_ARG, "%s: temperature must be finite and > 0", fn);
    if (rows == 0) return ok();
    if (!parts) return fail(VWC_ERR_INVALID_ARG, "%s: parts is null", fn);
    if (!logprob && !lse && !entropy)
        return fail(VWC_ERR_INVALID_ARG, "%s: no output requested", fn);
    if (rows > INT32_MAX - 256) return fail(VWC_ERR_UNSUPPORTED, "%s: too many rows", fn);
    vwc::CombinePlan p{};
    p.parts = parts;
    p.k = k;
    p.stride = rows;
    p.rows = rows;
    p.tau = static_cast<double>(temperature);
    p.logprob = logprob;
    p.lse = lse;
    p.entropy = entropy;
    return hip_status(vwc::launch_combine(p, stream), fn);
}

static int64_t lmhead_segments(int64_t vocab) {
    const int64_t tiles = (vocab + vwc::kLmVoc - 1) / vwc::kLmVoc;
    return (tiles + vwc::kLmSegTiles - 1) / vwc::kLmSegTiles;
}

// Workspace: the segment partials, then (16-byte aligned) the compacted
// kept hidden rows.
static size_t lmhead_partial_bytes(int64_t rows, int64_t vocab) {
    return static_cast<size_t>(rows) * static_cast<size_t>(lmhead_segments(vocab)) *
           sizeof(vwc_partial);
}

size_t vwc_lmhead_workspace_bytes(int64_t rows, int64_t vocab, int64_t d) {
    if (rows <= 0 || vocab <= 0 || d <= 0) return 0;
    const size_t gather = (static_cast<size_t>(rows) * static_cast<size_t>(d) * 2 + 15) / 16 * 16;
    return lmhead_partial_bytes(rows, vocab) + gather;
}

vwc_status vwc_lmhead_logprob_fwd(const void *hidden, int64_t n_rows, int64_t ldh,
                                  const void *weight, int64_t vocab, int64_t ldw, int64_t d,
                                  const int32_t *targets, const int32_t *row_idx, int64_t m,
                                  float temperature, float *logprob, float *lse, float *entropy,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_lmhead_logprob_fwd";
    if (n_rows < 0 || m < 0) return fail(VWC_ERR_INVALID_ARG, "%s: n_rows < 0 or m < 0", fn);
    if (vocab <= 0) return fail(VWC_ERR_INVALID_ARG, "%s: vocab must be positive", fn);
    if (d <= 0 || ldh < d || ldw < d)
        return fail(VWC_ERR_INVALID_ARG, "%s: need 0 < d <= ldh and d <= ldw", fn);
    if (!(temperature > 0.f) || !isfinite(temperature))
        return fail(VWC_ERR_INVALID_ARG, "%s: temperature must be finite and > 0", fn);
    if (m == 0) return ok();
    if (!row_idx && m != n_rows)
        return fail(VWC_ERR_INVALID_ARG, "%s: without row_idx, m must equal n_rows", fn);
    if (n_rows == 0) return fail(VWC_ERR_INVALID_ARG, "%s: row_idx given but n_rows == 0", fn);
    if (!hidden || !weight) return fail(VWC_ERR_INVALID_ARG, "%s: hidden or weight is null", fn);
    if (logprob && !targets) return fail(VWC_ERR_INVALID_ARG, "%s: targets is null", fn);
    if (!logprob && !lse && !entropy)
        return fail(VWC_ERR_INVALID_ARG, "%s: no output requested", fn);
    if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(weight) % 16 ||
        d % 8 || ldh % 8 || ldw % 8)
        return fail(VWC_ERR_UNSUPPORTED,
                    "%s: hidden and weight must be 16-byte aligned, d, ldh, ldw multiples of 8",
                    fn);
    // Tiles are addressed with 32-bit byte offsets: 256 rows of ldh or ldw
    // elements must stay below 2^31 bytes.
    if (vocab > INT32_MAX - vwc::kLmVoc || ldh >= (int64_t{1} << 22) ||
        ldw >= (int64_t{1} << 22) || n_rows > INT64_MAX / 2 / ldh ||
        vocab > INT64_MAX / 2 / ldw || m > INT64_MAX / 2 / d)
        return fail(VWC_ERR_UNSUPPORTED, "%s: operand too large", fn);
    const int64_t nseg = lmhead_segments(vocab);
    const int64_t ntb = (m + vwc::kLmTok - 1) / vwc::kLmTok;
    // The row gather runs one thread per 16-byte chunk of the kept rows.
    if (row_idx && (m * (d / 8) + 255) / 256 > INT32_MAX)
        return fail(VWC_ERR_UNSUPPORTED, "%s: kept rows too large to gather in one launch", fn);
    if (m > INT32_MAX || ntb > INT32_MAX / nseg)
        return fail(VWC_ERR_UNSUPPORTED, "%s: %lld rows exceed one launch", fn,
                    static_cast<long long>(m));
    const size_t part_bytes = lmhead_partial_bytes(m, vocab);
    const size_t need = row_idx ? vwc_lmhead_workspace_bytes(m, vocab, d) : part_bytes;
    if (!workspace || workspace_bytes < need)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace ? workspace_bytes : static_cast<size_t>(0));
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);

    vwc::LmPlan p{};
    p.hidden = static_cast<const uint16_t *>(hidden);
    p.ldh = ldh;
    p.n_rows = n_rows;
    if (row_idx) {  // keep the listed rows, in order, before the projection
        uint16_t *compact = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + part_bytes);
        hipError_t ge = vwc::launch_gather_rows(p.hidden, ldh, n_rows, row_idx, m,
                                                static_cast<int32_t>(d), compact, stream);
        if (ge != hipSuccess) return hip_status(ge, fn);
        p.hidden = compact;
        p.ldh = d;
    }
    p.weight = static_cast<const uint16_t *>(weight);
    p.ldw = ldw;
    p.vocab = static_cast<int32_t>(vocab);
    p.d = static_cast<int32_t>(d);
    p.targets = logprob ? targets : nullptr;
    p.row_idx = row_idx;
    p.m = m;
    const double tau = static_cast<double>(temperature);
    p.c = static_cast<float>(1.44269504088896340736 / tau);
    p.ntb = static_cast<int>(ntb);
    p.nvt = static_cast<int>((vocab + vwc::kLmVoc - 1) / vwc::kLmVoc);
    p.nseg = static_cast<int>(nseg);
    p.seg_part = static_cast<vwc_partial *>(workspace);
    hipError_t e = vwc::launch_lmhead_fwd(p, entropy != nullptr, stream);
    if (e != hipSuccess) return hip_status(e, fn);
    vwc::CombinePlan cp{};
    cp.parts = p.seg_part;
    cp.k = p.nseg;
    cp.stride = 1;
    cp.rows = m;
    cp.tau = tau;
    cp.logprob = logprob;
    cp.lse = lse;
    cp.entropy = entropy;
    return hip_status(vwc::launch_combine_rows(cp, stream), fn);
}

vwc_status vwc_mask_to_index(const uint8_t *mask, int64_t n, int32_t *row_idx, int32_t *count,
                             hipStream_t stream) {
    const char *fn = "vwc_mask_to_index";
    if (n < 0 || n > INT32_MAX) return fail(VWC_ERR_INVALID_ARG, "%s: n outside [0, 2^31)", fn);
    if (!count) return fail(VWC_ERR_INVALID_ARG, "%s: count is null", fn);
    if (n > 0 && (!mask || !row_idx))
        return fail(VWC_ERR_INVALID_ARG, "%s: null mask or row_idx", fn);
    return hip_status(vwc::launch_mask_to_index(mask, n, row_idx, count, stream), fn);
}

// Masks up to this length take the one-workgroup scan (one launch, no
// workspace); longer ones the tiled scan.
constexpr int64_t kMaskOneGroupMax = 65536;

size_t vwc_mask_to_index_workspace_bytes(int64_t n) {
    if (n <= kMaskOneGroupMax) return 0;
    return static_cast<size_t>(vwc::mask_tiles(n)) * sizeof(int32_t);
}

vwc_status vwc_mask_to_index_ws(const uint8_t *mask, int64_t n, int32_t *row_idx, int32_t *count,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "vwc_mask_to_index_ws";
    if (n < 0 || n > INT32_MAX) return fail(VWC_ERR_INVALID_ARG, "%s: n outside [0, 2^31)", fn);
    if (!count) return fail(VWC_ERR_INVALID_ARG, "%s: count is null", fn);
    if (n > 0 && (!mask || !row_idx))
        return fail(VWC_ERR_INVALID_ARG, "%s: null mask or row_idx", fn);
    const size_t need = vwc_mask_to_index_workspace_bytes(n);
    if (need == 0)
        return hip_status(vwc::launch_mask_to_index(mask, n, row_idx, count, stream), fn);
    if (!workspace || workspace_bytes < need)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace ? workspace_bytes : static_cast<size_t>(0));
    if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
        return fail(VWC_ERR_INVALID_ARG, "%s: workspace must be 4-byte aligned", fn);
    return hip_status(vwc::launch_mask_to_index_tiled(mask, n, row_idx, count,
                                                      static_cast<int32_t *>(workspace), stream),
                      fn);
}

const char *vwc_status_string(vwc_status status) {
    switch (static_cast<int>(status)) {
        case VWC_OK: return "ok";
        case VWC_ERR_INVALID_ARG: return "invalid argument";
        case VWC_ERR_UNSUPPORTED: return "unsupported";
        case VWC_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *vwc_last_error(void) { return g_last_error.c_str(); }

int vwc_abi_version(void) { return VWC_ABI_VERSION; }

}  // extern "C"
