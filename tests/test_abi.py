"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the headers declare, sizes workspaces and rejects bad arguments
before enqueuing anything."""
import ctypes
import os
import re

import pytest

import tile_sparse_attention_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(T.LIB_PATH),
                                reason="libtsa.so not built (python tile_sparse_attention_amd/build.py)")


def _declared():
    names = set()
    for h in ("tsa.h", "tsa_workload.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"\b(tsa_[a-z0-9_]+)\s*\(", txt))
    return names


def test_exports_every_declared_symbol():
    lib = T.lib()
    declared = _declared()
    assert declared == set(T.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_row_words():
    assert T.mask_row_words(32760, 8) == 128
    assert T.mask_row_words(75600, 1) == 2363
    assert T.mask_row_words(118800, 16) == 233
    assert T.mask_row_words(512, 16) == 1
    assert T.mask_row_words(0, 8) == 0 and T.mask_row_words(10, 0) == 0


def test_workspace_sizes():
    pr = T.problem(1, 40, 32760, 128, 16, 8)
    # packed V^T, then (bf16, N >= 8) 64 chunk-bitmap words and a flag per
    # work-group of 256 query rows, and a count
    assert T.workspace_size(T.OP_ATTENTION_FWD, pr) == 40 * 129 * 32768 * 2 + (40 * 128 * 65 + 1) * 4
    assert T.workspace_size(T.OP_ATTENTION_FWD, T.problem(1, 40, 32760, 128, 16, 4)) == 40 * 129 * 32768 * 2
    assert T.workspace_size(T.OP_MASK_COMPACT, pr) >= 40 * 2048 * 4
    pp = T.problem(1, 24, 118800, 128, 16, 16)
    ws = T.workspace_size(T.OP_PREDICT_MASK, pp)
    assert 2 * 24 * 7425 * 128 * 4 < ws < 2 * 24 * 7425 * 128 * 4 + (600 << 20)
    with pytest.raises(T.TsaError) as e:
        T.workspace_size(7, pr)
    assert e.value.status == T.ERR_INVALID_ARGUMENT


def _attn(pr, q=1, k=1, v=1, m=1, o=2, scale=1.0):
    # non-null fake addresses: validation must reject before any use of them
    def p(x):
        return ctypes.c_void_p(0x10000 * x) if x else ctypes.c_void_p(0)
    return T.lib().tsa_attention_fwd(ctypes.byref(pr), p(q), p(k), p(v), p(m),
                                     ctypes.c_float(scale), p(o), None, None, 0, None)


@pytest.mark.parametrize("field,value,status", [
    ("M", 8, T.ERR_UNSUPPORTED), ("M", 48, T.ERR_UNSUPPORTED), ("N", 3, T.ERR_UNSUPPORTED),
    ("N", 128, T.ERR_UNSUPPORTED), ("d", 96, T.ERR_UNSUPPORTED), ("dtype", 5, T.ERR_UNSUPPORTED),
    ("L", 0, T.ERR_INVALID_ARGUMENT), ("B", -1, T.ERR_INVALID_ARGUMENT),
    ("L", (1 << 22) + 1, T.ERR_UNSUPPORTED), ("H", 1 << 21, T.ERR_UNSUPPORTED),
])
def test_attention_rejects_bad_problem(field, value, status):
    pr = T.problem(1, 2, 512, 64, 16, 16)
    setattr(pr, field, value)
    assert _attn(pr) == status
    assert T.last_error() != ""


def test_attention_rejects_grids_beyond_one_dispatch():
    # a dispatch holds fewer than 2^32 work-items per dimension, and the
    # attention grids hold 4 per (b, h) and row with 256 rows of padding
    pr = T.problem(1, 1 << 20, 768, 64, 16, 16)     # 2^20 * 1024 * 4 = 2^32
    assert _attn(pr) == T.ERR_UNSUPPORTED and "grid" in T.last_error()
    pr = T.problem(1, 1 << 20, 767, 64, 16, 16)     # one row less: on to the workspace check
    assert _attn(pr) == T.ERR_WORKSPACE_TOO_SMALL


def test_attention_rejects_bad_pointers_and_scale():
    pr = T.problem(1, 2, 512, 64, 16, 16, T.DTYPE_F32)
    assert _attn(pr, q=0) == T.ERR_INVALID_ARGUMENT
    assert _attn(pr, m=0) == T.ERR_INVALID_ARGUMENT
    assert _attn(pr, o=0) == T.ERR_INVALID_ARGUMENT
    assert _attn(pr, o=1) == T.ERR_INVALID_ARGUMENT          # aliases q
    assert _attn(pr, scale=float("inf")) == T.ERR_INVALID_ARGUMENT
    assert _attn(pr, scale=float("nan")) == T.ERR_INVALID_ARGUMENT
    lib = T.lib()
    st = lib.tsa_attention_fwd(ctypes.byref(pr), ctypes.c_void_p(0x10008), ctypes.c_void_p(0x20000),
                               ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
                               ctypes.c_float(1.0), ctypes.c_void_p(0x50000), None, None, 0, None)
    assert st == T.ERR_INVALID_ARGUMENT and "align" in T.last_error()
    assert _attn(pr) == T.ERR_WORKSPACE_TOO_SMALL            # no workspace given


def _bwd(pr, ptrs=None, scale=1.0, ws=(None, 0)):
    # q k v o do lse mask dq dk dv as fake, distinct, aligned addresses
    p = dict(q=1, k=2, v=3, o=4, do=5, lse=6, m=7, dq=8, dk=9, dv=10)
    p.update(ptrs or {})
    a = {n: ctypes.c_void_p(0x10000 * x) if x else ctypes.c_void_p(0) for n, x in p.items()}
    return T.lib().tsa_attention_bwd(ctypes.byref(pr), a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                     a["m"], ctypes.c_float(scale), a["dq"], a["dk"], a["dv"],
                                     ws[0], ws[1], None)


def test_backward_workspace_and_validation():
    pr = T.problem(1, 40, 32760, 128, 16, 8)
    # per (b, h) and 128-row chunk: 128 lse2 and 128 D values (fp32)
    assert T.workspace_size(T.OP_ATTENTION_BWD, pr) == 40 * 256 * 256 * 4
    with pytest.raises(T.TsaError) as e:
        T.workspace_size(T.OP_ATTENTION_BWD, T.problem(1, 2, 512, 64, 16, 16, T.DTYPE_F32))
    assert e.value.status == T.ERR_UNSUPPORTED
    small = T.problem(1, 2, 512, 64, 16, 16)
    assert _bwd(T.problem(1, 2, 512, 64, 16, 16, T.DTYPE_F32)) == T.ERR_UNSUPPORTED
    assert _bwd(T.problem(1, 2, 512, 96, 16, 16)) == T.ERR_UNSUPPORTED
    assert _bwd(T.problem(1, 2, 512, 64, 16, 3)) == T.ERR_UNSUPPORTED
    for name in ("q", "o", "do", "lse", "m", "dq", "dv"):
        assert _bwd(small, {name: 0}) == T.ERR_INVALID_ARGUMENT, name
    assert _bwd(small, {"dq": 1}) == T.ERR_INVALID_ARGUMENT          # dq aliases q
    assert _bwd(small, {"dk": 8}) == T.ERR_INVALID_ARGUMENT          # dk aliases dq
    assert _bwd(small, scale=float("nan")) == T.ERR_INVALID_ARGUMENT
    # every call above and below fails validation, so nothing is launched
    assert _bwd(small) == T.ERR_WORKSPACE_TOO_SMALL                 # no workspace given
    need = T.workspace_size(T.OP_ATTENTION_BWD, small)
    assert need == 2 * 4 * 256 * 4
    assert _bwd(small, ws=(ctypes.c_void_p(0x900000), need - 4)) == T.ERR_WORKSPACE_TOO_SMALL
    assert _bwd(small, ws=(ctypes.c_void_p(0x900010), need)) == T.ERR_WORKSPACE_TOO_SMALL  # misaligned


def test_mask_diff_validation():
    lib = T.lib()
    p = lambda x: ctypes.c_void_p(x)  # noqa: E731  (fake, never dereferenced: every call below fails checks)
    pr = T.problem(1, 2, 512, 0, 16, 8)
    assert lib.tsa_mask_diff(ctypes.byref(pr), p(0), p(0x20000), p(0x30000), None, None) == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_mask_diff(ctypes.byref(pr), p(0x10000), p(0x20000), p(0), None, None) == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_mask_diff(ctypes.byref(pr), p(0x10002), p(0x20000), p(0x30000), None, None) \
        == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_mask_diff(ctypes.byref(pr), p(0x10000), p(0x20000), p(0x30004), None, None) \
        == T.ERR_INVALID_ARGUMENT
    bad = T.problem(1, 2, 512, 0, 8, 8)
    assert lib.tsa_mask_diff(ctypes.byref(bad), p(0x10000), p(0x20000), p(0x30000), None, None) \
        == T.ERR_UNSUPPORTED


def test_compact_and_predict_validation():
    lib = T.lib()
    pr = T.problem(1, 2, 512, 64, 16, 16)
    need = T.workspace_size(T.OP_MASK_COMPACT, pr)
    st = lib.tsa_mask_compact(ctypes.byref(pr), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                              ctypes.c_void_p(0x3000), 10, ctypes.c_void_p(0x4000), need - 1, None)
    assert st == T.ERR_WORKSPACE_TOO_SMALL
    st = lib.tsa_mask_compact(ctypes.byref(pr), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                              None, 10, ctypes.c_void_p(0x4000), need, None)
    assert st == T.ERR_INVALID_ARGUMENT
    st = lib.tsa_mask_compact(ctypes.byref(pr), None, ctypes.c_void_p(0x2000),
                              ctypes.c_void_p(0x3000), 10, ctypes.c_void_p(0x4000), need, None)
    assert st == T.ERR_INVALID_ARGUMENT
    pw = T.workspace_size(T.OP_PREDICT_MASK, pr)
    for sp in (-1, 100):
        st = lib.tsa_predict_mask(ctypes.byref(pr), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                                  sp, ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), pw, None)
        assert st == T.ERR_INVALID_ARGUMENT
    st = lib.tsa_predict_mask(ctypes.byref(pr), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                              85, ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), pw - 1, None)
    assert st == T.ERR_WORKSPACE_TOO_SMALL


def test_maskgen_validation():
    lib = T.lib()
    pr = T.problem(1, 2, 512, 64, 16, 16)
    g = T.MaskgenParams(1, (1 << 24) + 1, 0, 0, 0, 1)
    assert lib.tsa_maskgen_hash(ctypes.byref(pr), ctypes.byref(g), ctypes.c_void_p(0x1000),
                                None) == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_maskgen_hash(ctypes.byref(pr), None, ctypes.c_void_p(0x1000),
                                None) == T.ERR_INVALID_ARGUMENT


def test_structured_maskgen_validation():
    lib = T.lib()
    pr = T.problem(1, 2, 512, 64, 16, 16)
    out = ctypes.c_void_p(0x1000)
    g = T.StructuredParams(10, 4, 64, 2, 16, 4)

    def call(pats, params=g, prob=pr):
        arr = (ctypes.c_int32 * len(pats))(*pats)
        return lib.tsa_maskgen_structured(ctypes.byref(prob), ctypes.byref(params), arr, out, None)

    assert call([0, 5]) == T.ERR_INVALID_ARGUMENT                       # unknown pattern
    assert call([1, -1]) == T.ERR_INVALID_ARGUMENT
    assert call([2, 1], T.StructuredParams(10, 4, 0, 2, 16, 4)) == T.ERR_INVALID_ARGUMENT  # frame 0
    assert call([2, 1], T.StructuredParams(10, 4, 64, 65, 16, 4)) == T.ERR_INVALID_ARGUMENT  # reach
    assert call([3, 1], T.StructuredParams(10, 4, 64, 2, 16, 17)) == T.ERR_INVALID_ARGUMENT  # stripe
    assert call([1, 1], T.StructuredParams(-1, 4, 64, 2, 16, 4)) == T.ERR_INVALID_ARGUMENT
    big = T.problem(1, 129, 512, 64, 16, 16)
    assert call([1] * 129, prob=big) == T.ERR_UNSUPPORTED
    assert lib.tsa_maskgen_structured(ctypes.byref(pr), None, (ctypes.c_int32 * 2)(1, 1), out,
                                      None) == T.ERR_INVALID_ARGUMENT


def test_status_strings():
    assert T.status_string(T.OK) == "success"
    assert T.status_string(T.ERR_HIP) == "HIP runtime error"
    assert T.status_string(99) == "unknown status"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(T, "_lib", None)
    monkeypatch.setattr(T, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        T.lib()


def _noalloc(pr, q=1, k=2, v=3, m=4, o=5, scale=1.0):
    def p(x):
        return ctypes.c_void_p(0x10000 * x) if x else ctypes.c_void_p(0)
    return T.lib().tsa_attention_fwd_noalloc(ctypes.byref(pr), p(q), p(k), p(v), p(m),
                                             ctypes.c_float(scale), p(o), None, None)


def test_noalloc_forward_validates_before_touching_the_gpu():
    pr = T.problem(1, 2, 512, 64, 16, 16, T.DTYPE_F32)
    assert _noalloc(pr, q=0) == T.ERR_INVALID_ARGUMENT
    assert _noalloc(pr, o=1) == T.ERR_INVALID_ARGUMENT          # aliases q
    assert _noalloc(pr, scale=float("nan")) == T.ERR_INVALID_ARGUMENT
    bad = T.problem(1, 2, 512, 96, 16, 16)
    assert _noalloc(bad) == T.ERR_UNSUPPORTED
    # beyond the 64 MiB scratch (about 338 MB of workspace): refused, nothing enqueued
    big = T.problem(1, 40, 32760, 128, 16, 8)
    assert _noalloc(big) == T.ERR_UNSUPPORTED and "scratch" in T.last_error()


def test_timing_events_need_both_or_neither():
    lib = T.lib()
    assert lib.tsa_set_timing_events(ctypes.c_void_p(0x1000), None) == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_set_timing_events(None, ctypes.c_void_p(0x1000)) == T.ERR_INVALID_ARGUMENT
    assert lib.tsa_set_timing_events(None, None) == T.OK
