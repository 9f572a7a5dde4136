"""The C-ABI library on a host without a GPU: it loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vwc.h")
# VWC_TEST_LIB points the checks at another build of the library (the
# sanitizer test runs them against an instrumented copy).
LIB = os.environ.get("VWC_TEST_LIB") or os.path.join(ROOT, "vocab_wide_cross_amd", "libvwc.so")

OK, INVALID, UNSUPPORTED = 0, 1, 2
BF16, FP32 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._build_module().build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vwc_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 30
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    lib.vwc_abi_version.restype = ctypes.c_int
    assert lib.vwc_abi_version() == 1
    lib.vwc_status_string.restype = ctypes.c_char_p
    lib.vwc_status_string.argtypes = [ctypes.c_int]
    assert lib.vwc_status_string(0) == b"ok"
    assert lib.vwc_status_string(1) == b"invalid argument"
    assert lib.vwc_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    f = lib.vwc_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    # Rows are cut into segments of <= 128 KiB.  Up to 3 segments, one workgroup
    # reduces and merges a row: no workspace.  Longer rows take one workgroup per
    # segment and 16 bytes per row and segment.
    assert f(8192, 248320, BF16) == 8192 * 4 * 16   # 485 KiB: 4 segments
    assert f(8192, 248320, FP32) == 8192 * 8 * 16
    assert f(4096, 151936, BF16) == 0               # 297 KiB: 3 segments
    assert f(8192, 98304, FP32) == 0                # exactly 3 segments
    assert f(8192, 98305, FP32) == 8192 * 4 * 16
    assert f(16384, 62080, FP32) == 0               # 2 segments
    assert f(3, 1 << 20, BF16) == 3 * 16 * 16
    assert f(64, 2048, FP32) == 0          # one segment: no workspace
    assert f(0, 248320, BF16) == 0
    assert f(10, 0, BF16) == 0
    assert f(10, 10, 7) == 0


def _fwd(lib):
    f = lib.vwc_selected_logprob_fwd
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_float, p, p, p, p, ctypes.c_size_t,
                  p]
    f.restype = ctypes.c_int
    return f


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def test_forward_validation(lib):
    f = _fwd(lib)
    err = lib.vwc_last_error
    err.restype = ctypes.c_char_p
    ws = ctypes.c_void_p(0x200000)
    # unknown dtype
    assert f(FAKE, 7, 4, 16, 16, FAKE, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert b"dtype" in err()
    # ld < vocab, vocab <= 0, n_rows < 0
    assert f(FAKE, BF16, 4, 16, 8, FAKE, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert f(FAKE, BF16, 4, 0, 8, FAKE, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert f(FAKE, BF16, -1, 16, 16, FAKE, 1.0, FAKE, None, None, None, 0, None) == INVALID
    # temperature must be finite and positive
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert f(FAKE, BF16, 4, 16, 16, FAKE, tau, FAKE, None, None, None, 0, None) == INVALID
    # missing targets / no output / null logits
    assert f(FAKE, BF16, 4, 16, 16, None, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 1.0, None, None, None, None, 0, None) == INVALID
    assert f(None, BF16, 4, 16, 16, FAKE, 1.0, FAKE, None, None, None, 0, None) == INVALID
    # misaligned for its dtype
    assert f(ctypes.c_void_p(0x100001), BF16, 4, 16, 16, FAKE, 1.0, FAKE, None, None, None, 0,
             None) == UNSUPPORTED
    # workspace required for rows of more than 4 segments, and must be large enough
    assert f(FAKE, FP32, 4, 248320, 248320, FAKE, 1.0, FAKE, None, None, None, 0,
             None) == INVALID
    assert b"workspace" in err()
    assert f(FAKE, FP32, 4, 248320, 248320, FAKE, 1.0, FAKE, None, None, ws, 4 * 8 * 16 - 1,
             None) == INVALID
    # zero rows: OK, nothing launched (no GPU is touched here)
    assert f(None, BF16, 0, 16, 16, None, 1.0, None, None, None, None, 0, None) == OK
    assert err() == b""


def err_str(lib):
    lib.vwc_last_error.restype = ctypes.c_char_p
    return lib.vwc_last_error()


def test_rows_and_backward_validation(lib):
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    fr = lib.vwc_selected_logprob_fwd_rows
    fr.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, ctypes.c_float, p, p, p, p,
                   ctypes.c_size_t, p]
    # null row_idx with m > 0; m < 0; empty row set is a no-op
    assert fr(FAKE, BF16, 8, 16, 16, FAKE, None, 3, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert fr(FAKE, BF16, 8, 16, 16, FAKE, FAKE, -1, 1.0, FAKE, None, None, None, 0, None) == INVALID
    assert fr(FAKE, BF16, 8, 16, 16, FAKE, FAKE, 0, 1.0, FAKE, None, None, None, 0, None) == OK
    # a row list longer than one launch is refused before any size is computed from it
    # (the workspace and gradient sizes would overflow 64 bits)
    huge = 1 << 62
    assert fr(FAKE, BF16, 8, 1 << 20, 1 << 20, FAKE, FAKE, huge, 1.0, FAKE, None, None, FAKE,
              1 << 30, None) == UNSUPPORTED
    assert b"exceed one launch" in err_str(lib)
    b = lib.vwc_selected_logprob_bwd
    b.argtypes = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_float, p, p, p, ctypes.c_int, i64, p]
    g = ctypes.c_void_p(0x900000)
    # ld_grad < vocab, bad grad dtype, null lse
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, g, BF16, 8, None) == INVALID
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, g, 5, 16, None) == INVALID
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, None, FAKE, g, BF16, 16, None) == INVALID
    # gradient overlapping the logits without being exactly them (in place needs
    # the same pointer, dtype and ld)
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, ctypes.c_void_p(0x100010), BF16, 16,
             None) == INVALID
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, FAKE, FP32, 16, None) == INVALID
    assert b(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, FAKE, BF16, 24, None) == INVALID
    assert b"overlaps" in err_str(lib)
    br = lib.vwc_selected_logprob_bwd_rows
    br.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, ctypes.c_float, p, p, p,
                   ctypes.c_int, i64, ctypes.c_int, p]
    assert br(FAKE, BF16, 4, 16, 16, FAKE, FAKE, 2, 1.0, FAKE, FAKE, g, BF16, 16, 9,
              None) == INVALID
    assert br(FAKE, BF16, 4, 16, 16, FAKE, FAKE, 0, 1.0, FAKE, FAKE, g, BF16, 16, 0, None) == OK
    assert br(FAKE, BF16, 4, 1 << 20, 1 << 20, FAKE, FAKE, huge, 1.0, FAKE, FAKE, g, BF16,
              1 << 20, 0, None) == UNSUPPORTED     # compact gradient of 2^62 rows
    assert b"exceed one launch" in err_str(lib)
    # in place, compact gradient rows (indexed by output, not row id) are refused
    assert br(FAKE, BF16, 4, 16, 16, FAKE, FAKE, 2, 1.0, FAKE, FAKE, FAKE, BF16, 16, 0,
              None) == INVALID
    assert b"row id" in err_str(lib)
    # in place, the top-k KL backward needs the single-pass payload (k <= 256)
    kb = lib.vwc_topk_kl_bwd
    kb.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, ctypes.c_int32, ctypes.c_int,
                   ctypes.c_float, ctypes.c_float, p, p, p, p, p, p, ctypes.c_int, i64, p]
    assert kb(FAKE, BF16, 4, 1000, 1000, FAKE, FAKE, 300, 1, 1e-6, 1.0, FAKE, FAKE, FAKE, FAKE,
              FAKE, FAKE, BF16, 1000, None) == UNSUPPORTED
    assert b"in-place top-k KL" in err_str(lib)
    # row-set top-k KL: a row list is required, the layout must be known
    kfr = lib.vwc_topk_kl_fwd_rows
    kfr.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i64, p, p, ctypes.c_int32, ctypes.c_int,
                    ctypes.c_float, ctypes.c_float, p, p, p, p, p, p, ctypes.c_size_t, p]
    assert kfr(FAKE, BF16, 4, 1000, 1000, None, 2, FAKE, FAKE, 8, 1, 1e-6, 1.0, None, None, None,
               None, FAKE, None, 0, None) == INVALID
    assert b"row_idx" in err_str(lib)
    assert kfr(FAKE, BF16, 4, 1000, 1000, FAKE, 0, FAKE, FAKE, 8, 1, 1e-6, 1.0, None, None, None,
               None, FAKE, None, 0, None) == OK          # empty row set
    kbr = lib.vwc_topk_kl_bwd_rows
    kbr.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i64, p, p, ctypes.c_int32, ctypes.c_int,
                    ctypes.c_float, ctypes.c_float, p, p, p, p, p, p, ctypes.c_int, i64,
                    ctypes.c_int, p]
    assert kbr(FAKE, BF16, 4, 1000, 1000, FAKE, 2, FAKE, FAKE, 8, 1, 1e-6, 1.0, FAKE, FAKE, FAKE,
               FAKE, FAKE, g, BF16, 1000, 7, None) == INVALID
    assert b"layout" in err_str(lib)
    assert kbr(FAKE, BF16, 4, 1000, 1000, FAKE, 2, FAKE, FAKE, 0, 1, 1e-6, 1.0, FAKE, FAKE, FAKE,
               FAKE, FAKE, g, BF16, 1000, 0, None) == INVALID   # k = 0


def test_fused_forward_backward_validation(lib):
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.vwc_selected_logprob_fwd_bwd
    f.argtypes = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_float, p, p, p, p, p, ctypes.c_int,
                  i64, p, ctypes.c_size_t, p]
    f.restype = ctypes.c_int
    g = ctypes.c_void_p(0x900000)
    # lse is required (it is both an output and the backward's saved logZ)
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, FAKE, None, None, g, BF16, 16, None, 0,
             None) == INVALID
    assert b"lse" in err_str(lib)
    # a gradient that overlaps the logits without being them
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, None, FAKE, None,
             ctypes.c_void_p(0x100010), BF16, 16, None, 0, None) == INVALID
    assert b"overlaps" in err_str(lib)
    # no rows: nothing to do; bad temperature and ld as for the other calls
    assert f(FAKE, BF16, 0, 16, 16, None, 1.0, None, None, None, None, None, BF16, 16, None, 0,
             None) == OK
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 0.0, FAKE, None, FAKE, None, g, BF16, 16, None, 0,
             None) == INVALID
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 1.0, FAKE, None, FAKE, None, g, BF16, 8, None, 0,
             None) == INVALID


def test_topk_kl_one_call_validation(lib):
    p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    f = lib.vwc_topk_kl_fwd_bwd
    f.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, ctypes.c_int32, ctypes.c_int, f32, f32, p,
                  p, p, p, p, p, p, ctypes.c_int, i64, p, ctypes.c_size_t, p]
    f.restype = ctypes.c_int
    g = ctypes.c_void_p(0x900000)

    def call(n=4, k=8, mode=1, eps=1e-6, tau=1.0, gl=FAKE, Q=FAKE, P=FAKE, S=FAKE, lse=FAKE,
             grad=g, gdt=BF16, ldg=1000):
        return f(FAKE, BF16, n, 1000, 1000, FAKE, FAKE, k, mode, eps, tau, gl, None, Q, P, S,
                 lse, grad, gdt, ldg, None, 0, None)

    assert call(n=0) == OK                                  # no rows
    for kw in ({"lse": None}, {"Q": None}, {"P": None}, {"S": None}, {"gl": None},
               {"grad": None}):
        assert call(**kw) == INVALID, kw                    # every output but the loss required
    assert b"null grad_loss" in err_str(lib)
    assert call(k=0) == INVALID and call(k=1001) == INVALID  # k in [1, vocab]
    assert call(mode=5) == INVALID
    assert call(eps=0.0) == INVALID                         # the tail guard must lie in (0, 1)
    assert call(tau=0.0) == INVALID
    assert call(ldg=999) == INVALID
    # in place without the single-pass payload (k > 256) runs nothing
    assert call(k=300, grad=FAKE) == UNSUPPORTED
    assert b"in-place top-k KL" in err_str(lib)
    fr = lib.vwc_topk_kl_fwd_bwd_rows
    fr.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i64, p, p, ctypes.c_int32, ctypes.c_int, f32,
                   f32, p, p, p, p, p, p, p, ctypes.c_int, i64, ctypes.c_int, p, ctypes.c_size_t, p]
    fr.restype = ctypes.c_int

    def rows(m=2, idx=FAKE, layout=0, grad=g):
        return fr(FAKE, BF16, 4, 1000, 1000, idx, m, FAKE, FAKE, 8, 1, 1e-6, 1.0, FAKE, None,
                  FAKE, FAKE, FAKE, FAKE, grad, BF16, 1000, layout, None, 0, None)

    assert rows(m=0, idx=None) == OK                         # empty row set
    assert rows(idx=None) == INVALID and b"row_idx" in err_str(lib)
    assert rows(layout=7) == INVALID and b"layout" in err_str(lib)
    # in place needs gradient rows indexed by row id (the scatter layout)
    assert rows(grad=FAKE) == INVALID and b"row id" in err_str(lib)


def test_partial_combine_and_mask_validation(lib):
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    c = lib.vwc_partial_combine
    c.argtypes = [p, ctypes.c_int32, i64, ctypes.c_float, p, p, p, p]
    assert c(FAKE, 0, 4, 1.0, FAKE, None, None, None) == INVALID
    assert c(FAKE, 2, -1, 1.0, FAKE, None, None, None) == INVALID
    assert c(FAKE, 2, 4, 0.0, FAKE, None, None, None) == INVALID
    assert c(FAKE, 2, 4, 1.0, None, None, None, None) == INVALID
    assert c(None, 2, 0, 1.0, None, None, None, None) == OK
    vp = lib.vwc_vocab_partial
    vp.argtypes = [p, ctypes.c_int, i64, i64, i64, i64, p, p, i64, ctypes.c_float, p, p,
                   ctypes.c_size_t, p]
    assert vp(FAKE, FP32, 4, 16, 64, -1, FAKE, None, 4, 1.0, FAKE, None, 0, None) == INVALID
    assert vp(FAKE, FP32, 4, 16, 64, 0, FAKE, None, 4, 1.0, None, None, 0, None) == INVALID
    mk = lib.vwc_mask_to_index
    mk.argtypes = [p, i64, p, p, p]
    assert mk(FAKE, -1, FAKE, FAKE, None) == INVALID
    assert mk(FAKE, 2 ** 31, FAKE, FAKE, None) == INVALID
    assert mk(FAKE, 4, FAKE, None, None) == INVALID
    assert mk(None, 4, FAKE, FAKE, None) == INVALID
    # the tiled scan: 4 bytes per tile of 4096 entries past 65536 entries
    wb = lib.vwc_mask_to_index_workspace_bytes
    wb.argtypes = [i64]
    wb.restype = ctypes.c_size_t
    assert wb(0) == 0 and wb(65536) == 0
    assert wb(65537) == 17 * 4 and wb(160000) == 40 * 4 and wb(1 << 20) == 256 * 4
    mw = lib.vwc_mask_to_index_ws
    mw.argtypes = [p, i64, p, p, p, ctypes.c_size_t, p]
    assert mw(FAKE, -1, FAKE, FAKE, FAKE, 1024, None) == INVALID
    assert mw(FAKE, 2 ** 31, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert mw(FAKE, 1 << 20, FAKE, None, FAKE, 1024, None) == INVALID
    assert mw(FAKE, 1 << 20, FAKE, FAKE, None, 0, None) == INVALID          # no workspace
    assert mw(FAKE, 1 << 20, FAKE, FAKE, FAKE, 256 * 4 - 1, None) == INVALID  # too small
    assert mw(FAKE, 1 << 20, FAKE, FAKE, ctypes.c_void_p(0x100002), 1024, None) == INVALID


def _lmhead(lib):
    f = lib.vwc_lmhead_logprob_fwd
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [p, i64, i64, p, i64, i64, i64, p, p, i64, ctypes.c_float, p, p, p, p,
                  ctypes.c_size_t, p]
    f.restype = ctypes.c_int
    return f


def test_lmhead_workspace_bytes(lib):
    f = lib.vwc_lmhead_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    # 248320 = 970 tiles of 256 -> 243 segments of 4 tiles, then the kept rows
    assert f(8192, 248320, 2560) == 8192 * 243 * 16 + 8192 * 2560 * 2
    assert f(300, 2000, 320) == 300 * 2 * 16 + 300 * 320 * 2
    assert f(1, 1, 8) == 16 + 16
    assert f(0, 2000, 8) == 0
    assert f(5, 0, 8) == 0
    assert f(5, 10, 0) == 0


def test_lmhead_validation(lib):
    f = _lmhead(lib)
    err = lib.vwc_last_error
    err.restype = ctypes.c_char_p
    ws = ctypes.c_void_p(0x200000)
    big = 1 << 40
    H, Wt = FAKE, ctypes.c_void_p(0x300000)

    def call(hidden=H, n=4, ldh=64, weight=Wt, vocab=1000, ldw=64, d=64, targets=FAKE,
             rows=None, m=4, tau=1.0, lp=FAKE, lse=None, ent=None, w=ws, wsb=big):
        return f(hidden, n, ldh, weight, vocab, ldw, d, targets, rows, m, tau, lp, lse, ent, w,
                 wsb, None)

    assert call(n=-1) == INVALID
    assert call(m=-1) == INVALID
    assert call(vocab=0) == INVALID
    assert call(d=0) == INVALID
    assert call(d=72) == INVALID            # d > ldh
    assert call(ldw=56) == INVALID          # d > ldw
    for tau in (0.0, -2.0, float("inf"), float("nan")):
        assert call(tau=tau) == INVALID
    assert call(m=3) == INVALID             # dense call needs m == n_rows
    assert call(n=0, rows=FAKE, m=3) == INVALID
    assert call(hidden=None) == INVALID
    assert call(weight=None) == INVALID
    assert call(targets=None) == INVALID    # logprob needs targets
    assert call(lp=None) == INVALID         # no output at all
    # layout limits
    assert call(hidden=ctypes.c_void_p(0x100008)) == UNSUPPORTED
    assert call(d=60, ldh=64, ldw=64) == UNSUPPORTED
    assert call(ldh=68, d=64) == UNSUPPORTED
    assert call(ldh=1 << 22) == UNSUPPORTED
    # kept rows whose gather would need more than 2^31 workgroups
    wide = 1 << 21
    assert call(n=1 << 31, rows=FAKE, m=1 << 31, d=wide, ldh=wide, ldw=wide) == UNSUPPORTED
    assert b"gather" in err()
    assert call(n=1 << 31, m=1 << 31) == UNSUPPORTED   # more rows than one launch takes
    # workspace: required, large enough, aligned
    assert call(w=None, wsb=0) == INVALID
    assert b"workspace" in err()
    assert call(wsb=4 * 1 * 16 - 1) == INVALID  # 4 rows x 1 segment
    assert call(w=ctypes.c_void_p(0x200008)) == INVALID
    # nothing to do: OK without touching any pointer
    assert call(hidden=None, weight=None, targets=None, lp=None, m=0, n=0, w=None,
                wsb=0) == OK
    assert err() == b""


def _signatures():
    """(name, [(type, parameter)]) of every entry point that takes a logits tensor,
    read from the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = []
    for name, params in re.findall(r"\bvwc_status\s+(vwc_[a-z_0-9]+)\s*\((.*?)\);", text, flags=re.S):
        ps = []
        for p in " ".join(params.split()).split(","):
            p = p.strip()
            m = re.match(r"(.*?)(\w+)$", p)
            ps.append((m.group(1).replace(" ", ""), m.group(2)))
        if ps[0][1] in ("logits", "logits_slice"):
            out.append((name, ps))
    return out


_CTYPE = {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int, "vwc_dtype": ctypes.c_int,
          "vwc_kl_mode": ctypes.c_int, "vwc_grad_layout": ctypes.c_int, "float": ctypes.c_float,
          "size_t": ctypes.c_size_t, "hipStream_t": ctypes.c_void_p}
_BASE = {"dt": BF16, "grad_dt": BF16, "n_rows": 4, "vocab": 64, "v_local": 64, "ld": 64,
         "ld_grad": 64, "m": 4, "v_start": 0, "temperature": 1.0, "k": 2, "mode": 0,
         "tail_mass_eps": 1e-6, "layout": 0, "workspace_bytes": 0}
# Each of these alone must be refused by the host checks (VWC_ERR_INVALID_ARG, the
# entry point's name in the message) before any HIP call.
_BAD = [("dt", 7), ("n_rows", -1), ("vocab", 0), ("ld", 63), ("temperature", 0.0),
        ("temperature", float("nan")), ("temperature", float("inf")), ("logits", None)]


@pytest.mark.parametrize("name,params", _signatures(), ids=[n for n, _ in _signatures()])
def test_every_logits_entry_point_checks_its_arguments(lib, name, params):
    assert len(params) >= 8
    f = getattr(lib, name)
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p if t.endswith("*") else _CTYPE[t] for t, _ in params]
    lib.vwc_last_error.restype = ctypes.c_char_p
    names = [n for _, n in params]
    for key, val in _BAD:
        key = {"vocab": "v_local", "logits": "logits_slice"}.get(key, key) \
            if key not in names else key
        assert key in names, (name, key)
        args = []
        for t, n in params:
            if n == key:
                args.append(val)
            elif t.endswith("*"):
                args.append(None if n == "workspace" else FAKE)
            elif n == "stream":
                args.append(None)
            else:
                args.append(_BASE[n])
        st = f(*args)
        msg = lib.vwc_last_error().decode()
        assert st == INVALID, (name, key, val, st, msg)
        assert msg.startswith(name), (name, msg)


def test_last_error_is_per_thread(lib):
    """Each host thread reads back its own last failure (the detail is thread-local)."""
    import threading
    f = _fwd(lib)
    lib.vwc_last_error.restype = ctypes.c_char_p
    results = {}

    def worker(name, n_rows, vocab):
        msgs = set()
        for _ in range(2000):
            st = f(FAKE, BF16, n_rows, vocab, max(vocab, 1), FAKE, 1.0, FAKE, FAKE, None, None, 0,
                   None)
            assert st == INVALID
            msgs.add(lib.vwc_last_error().decode())
        results[name] = msgs

    ts = [threading.Thread(target=worker, args=("rows", -1, 64)),
          threading.Thread(target=worker, args=("vocab", 4, 0))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert results["rows"] == {"vwc_selected_logprob_fwd: n_rows < 0"}
    assert results["vocab"] == {"vwc_selected_logprob_fwd: vocab must be positive"}
