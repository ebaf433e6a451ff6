"""CPU tests of the C ABI: the library loads, exports every symbol that
include/hq.h declares, and rejects invalid arguments before any device work
(status code + message; no GPU needed, no compute call is made).  Pointers
passed here are never dereferenced: every case fails host validation."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import fp4_gemm_moe_amd as hq  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hq.library_path()):
        from fp4_gemm_moe_amd import build
        build.build(verbose=False)
    return hq.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "hq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_calls():
    names = _declared()
    for n in ["hq_group_wise_quant", "hq_dense_gemm", "hq_batch_gemm", "hq_group_contiguous_gemm",
              "hq_group_masked_gemm", "hq_fused_swiglu_quant", "hq_prefill_permute_to_masked_gemm",
              "hq_last_error"]:
        assert n in names
    assert set(names) == set(hq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
MIS = ctypes.c_void_p(0x10001)    # misaligned
NUL = None


def _dense(lib, mode=0, a=A, sfa=A, b=A, sfb=A, bias=NUL, alpha=NUL, out=A, m=64, n=64, k=64):
    return lib.hq_dense_gemm(None, mode, a, sfa, b, sfb, bias, alpha, out, m, n, k, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=7), -4),
    (dict(k=48), -2),
    (dict(k=0), -2),
    (dict(n=12), -2),
    (dict(m=-1), -2),
    (dict(mode=1, bias=A), -4),
    (dict(mode=2, bias=A, alpha=A), -4),
    (dict(mode=0, alpha=A), -4),
    (dict(mode=1, alpha=A), -4),
    (dict(mode=2), -4),
    (dict(a=NUL), -1),
    (dict(out=NUL), -1),
    (dict(a=MIS), -3),
    (dict(out=MIS), -3),
    (dict(m=1 << 31), -2),
])
def test_dense_rejects(lib, kw, code):
    assert _dense(lib, **kw) == code
    assert hq.hq_last_error() != ""


def test_empty_problem_is_a_noop(lib):
    assert _dense(lib, m=0, a=NUL, sfa=NUL, b=NUL, sfb=NUL, out=NUL) == 0
    assert _dense(lib, n=0) == 0
    assert hq.hq_last_error() == ""


def test_batch_rejects(lib):
    f = lib.hq_batch_gemm
    assert f(None, 0, A, A, A, A, NUL, NUL, A, -1, 8, 8, 32, 0) == -2
    assert f(None, 0, A, A, A, A, NUL, NUL, A, 1 << 20, 1 << 12, 8, 32, 0) == -2
    assert f(None, 1, A, A, A, A, A, NUL, A, 2, 8, 8, 32, 0) == -4
    assert f(None, 0, A, A, A, A, NUL, NUL, A, 0, 8, 8, 32, 0) == 0


def test_grouped_rejects(lib):
    c = lib.hq_group_contiguous_gemm
    assert c(None, 0, A, A, A, A, A, 0, NUL, NUL, A, 64, 64, 64, 0) == -2
    assert c(None, 0, A, A, A, A, A, 1025, NUL, NUL, A, 64, 64, 64, 0) == -2
    assert c(None, 0, A, A, A, A, NUL, 4, NUL, NUL, A, 64, 64, 64, 0) == -1
    assert c(None, 2, A, A, A, A, A, 4, NUL, NUL, A, 64, 64, 64, 0) == -4
    mm = lib.hq_group_masked_gemm
    assert mm(None, 0, A, A, A, A, A, 4, 0, NUL, NUL, A, 64, 64, 0) == -2
    assert mm(None, 0, A, A, A, A, NUL, 4, 16, NUL, NUL, A, 64, 64, 0) == -1
    assert mm(None, 0, A, A, A, A, A, 4, 16, NUL, NUL, A, 64, 40, 0) == -2
    assert mm(None, 1, A, A, A, A, A, 4, 16, A, NUL, A, 64, 64, 0) == -4


def test_quant_rejects(lib):
    q = lib.hq_group_wise_quant
    assert q(None, 0, A, 4, 48, A, A, NUL, 0) == -2
    assert q(None, 3, A, 4, 64, A, A, NUL, 0) == -4
    assert q(None, 0, A, 4, 64, A, A, A, 0) == -4       # global scale is NVFP4-only
    assert q(None, 1, A, 4, 64, A, A, NUL, 1) == -4     # flags are NVFP4-only
    assert q(None, 2, A, 4, 64, A, A, NUL, 0) == -1     # NVFP4 needs a global scale
    assert q(None, 2, A, 4, 64, A, A, A, 4) == -4       # unknown flag
    assert q(None, 0, A, 4, 64, A, A, NUL, 3) == -4     # HQ_GS_INPUT is NVFP4-only, also with HQ_IN_FP16
    assert q(None, 0, MIS, 4, 64, A, A, NUL, 0) == -3
    assert q(None, 0, NUL, 4, 64, A, A, NUL, 0) == -1
    assert q(None, 0, NUL, 0, 64, NUL, NUL, NUL, 0) == 0


def test_swiglu_rejects(lib):
    s = lib.hq_fused_swiglu_quant
    assert s(None, 0, A, 8, 48, 1, NUL, 8, NUL, A, A, NUL, NUL) == -2
    assert s(None, 0, A, 8, 64, 1, NUL, 0, NUL, A, A, NUL, NUL) == -2
    assert s(None, 0, A, 8, 64, 0, NUL, 8, NUL, A, A, NUL, NUL) == -2
    assert s(None, 2, A, 8, 64, 1, NUL, 8, NUL, A, A, NUL, NUL) == -1
    assert s(None, 0, A, 8, 64, 1, NUL, 8, NUL, A, A, A, NUL) == -4
    assert s(None, 0, A, 8, 64, 1, NUL, 8, NUL, A, A, NUL, MIS) == -3
    assert s(None, 0, NUL, 0, 64, 1, NUL, 8, NUL, NUL, NUL, NUL, NUL) == 0


def test_python_binding_checks_buffer_sizes():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hq.hq_group_wise_quant("mxfp8", x, torch.zeros(4, 64, dtype=torch.uint8),
                               torch.zeros(4, 2, dtype=torch.uint8))   # CPU tensor


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(hq, "_lib", None)
    monkeypatch.setattr(hq, "library_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="has not been built"):
        hq.load()


def _permute(lib, x=A, T=8, row_bytes=4096, hidden=2048, scale=A, mode=0, ids=A, topk=8, E=16, M=1024,
             px=A, osf=A, imap=A, nums=A):
    return lib.hq_prefill_permute_to_masked_gemm(None, x, T, row_bytes, hidden, scale, mode, ids, topk, E, M,
                                                 px, osf, imap, nums)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), -4),
    (dict(topk=0), -2),
    (dict(topk=65), -2),
    (dict(E=0), -2),
    (dict(E=1025), -2),
    (dict(M=100), -2),
    (dict(M=0), -2),
    (dict(row_bytes=4100), -2),
    (dict(hidden=2176), -2),            # broadcast mode needs hidden % 512 == 0
    (dict(mode=1, hidden=2112), -2),    # direct mode needs hidden % 128 == 0
    (dict(T=-1), -2),
    (dict(nums=NUL), -1),
    (dict(x=NUL), -1),
    (dict(x=MIS), -3),
    (dict(osf=ctypes.c_void_p(0x10002)), -3),
])
def test_permute_rejects_before_launch(lib, kw, code):
    assert _permute(lib, **kw) == code
    assert len(lib.hq_last_error()) > 0


def test_workspace_calls_reject_before_launch(lib):
    """The workspace forms validate their workspace before any device work:
    a NULL workspace with a byte count, a misaligned one; the size query its
    shape, mode and output pointer."""
    d = lib.hq_dense_gemm_ws
    assert d(None, 0, A, A, A, A, NUL, NUL, A, 64, 64, 64, 0, NUL, 1024) == -1
    assert d(None, 0, A, A, A, A, NUL, NUL, A, 64, 64, 64, 0, MIS, 1024) == -3
    assert d(None, 0, A, A, A, A, NUL, NUL, A, 64, 12, 64, 0, A, 1024) == -2
    assert d(None, 0, A, A, A, A, NUL, NUL, A, 0, 64, 64, 0, NUL, 0) == 0
    b = lib.hq_batch_gemm_ws
    assert b(None, 0, A, A, A, A, NUL, NUL, A, 2, 64, 64, 64, 0, NUL, 16) == -1
    assert b(None, 0, A, A, A, A, NUL, NUL, A, 2, 64, 64, 64, 0, MIS, 16) == -3
    q = lib.hq_gemm_workspace_size
    out = ctypes.c_uint64(99)
    assert q(0, 1, 64, 64, 64, 0, NUL) == -1
    assert q(0, 0, 64, 64, 64, 0, ctypes.byref(out)) == -2
    assert q(0, 1, 64, 12, 64, 0, ctypes.byref(out)) == -2
    assert q(0, 1, 64, 64, 48, 0, ctypes.byref(out)) == -2
    assert q(7, 1, 64, 64, 64, 0, ctypes.byref(out)) == -4
    assert q(0, 1, 0, 64, 64, 0, ctypes.byref(out)) == 0 and out.value == 0


def test_gemm_swiglu_rejects_offsets_past_32_bits(lib):
    """The gate|up GEMM with the SwiGLU epilogue reads a tile's up rows h + 127
    rows past its first gate row with 32-bit offsets: shapes whose
    (h + 256) * k reaches 2^31 are refused on the host (status -2, not a
    device error), before any launch."""
    f = lib.hq_group_contiguous_gemm_swiglu_quant
    h, k = 32768, 65536
    assert f(None, 0, A, A, A, A, A, 4, NUL, NUL, A, A, NUL, 1024, h, k, 0) == -2
    assert "2^31" in hq.hq_last_error()


def test_dswiglu_rejects_before_launch(lib):
    f = lib.hq_group_contiguous_gemm_dswiglu
    args = lambda mode=0, n=64, k=512, c=A, prob=A, dprob=A, d=A, G=4: (
        None, mode, A, A, A, A, A, G, c, NUL, NUL, prob, dprob, d, 64, n, k, 0)
    assert f(*args(mode=2)) == -4              # NVFP4: not this call
    assert f(*args(n=48)) == -2                # n % 32
    assert f(*args(k=48)) == -2                # k % 32
    assert f(*args(k=128)) == -2               # one MXFP8 K step
    assert f(*args(G=0)) == -2
    assert f(*args(c=NUL)) == -1
    assert f(*args(dprob=NUL)) == -1
    assert f(*args(c=MIS)) == -3
    assert f(*args(d=MIS)) == -3


def test_dswiglu_quant_rejects_before_launch(lib):
    f = lib.hq_group_contiguous_gemm_dswiglu_quant
    args = lambda mode=0, n=64, k=512, c=A, dprob=A, dq=A, dsf=A: (
        None, mode, A, A, A, A, A, 4, c, NUL, NUL, A, dprob, dq, dsf, 64, n, k, 0)
    assert f(*args(mode=2)) == -4              # NVFP4: not this call
    assert f(*args(n=48)) == -2                # n % 32
    assert f(*args(k=128)) == -2               # one MXFP8 K step
    assert f(*args(dq=NUL)) == -1
    assert f(*args(dsf=NUL)) == -1
    assert f(*args(c=NUL)) == -1
    assert f(*args(dq=MIS)) == -3
    assert f(*args(c=MIS)) == -3
