"""Python binding of libhq.so, the MI355X (gfx950) block-scaled GEMM library.

The functions carry the names of the C ABI (include/hq.h) and only marshal
arguments: they check that the torch tensors have the dtypes, sizes, device
and contiguity the C call assumes (the C layer cannot see buffer sizes), pass
raw device pointers and the current HIP stream, and raise HQError on a
non-zero status.  Every step of the computation runs in the HIP kernels;
there is no CPU fallback.  If libhq.so has not been built, loading fails
loudly (build it with ``python -m fp4_gemm_moe_amd.build``).

PyTorch is used for device memory and streams only.
"""
import ctypes
import os

import torch

__all__ = [
    "HQ_MXFP8", "HQ_MXFP4", "HQ_NVFP4", "HQ_GS_INPUT", "HQ_IN_FP16", "HQ_OUT_FP16", "HQError",
    "hq_group_wise_quant", "hq_dense_gemm", "hq_batch_gemm", "hq_gemm_workspace_size",
    "gemm_workspace", "ptr_arrays", "hq_dense_gemm_scratch", "HQ_SCRATCH_BYTES",
    "hq_group_contiguous_gemm", "hq_group_masked_gemm", "hq_fused_swiglu_quant",
    "hq_group_contiguous_gemm_swiglu_quant", "hq_group_contiguous_gemm_ptr_array",
    "hq_group_contiguous_gemm_dswiglu", "hq_group_contiguous_gemm_dswiglu_quant",
    "hq_prefill_permute_to_masked_gemm", "prefill_permute_to_masked_gemm",
    "HQ_SCALE_BROADCAST", "HQ_SCALE_DIRECT",
    "hq_last_error", "library_path", "load", "EXPORTED_SYMBOLS",
    "quantize", "group_size", "code_cols",
]

HQ_MXFP8 = 0
HQ_MXFP4 = 1
HQ_NVFP4 = 2
HQ_GS_INPUT = 1
HQ_IN_FP16 = 2
HQ_OUT_FP16 = 0x100      # OR'ed into a GEMM's mode: out is float16, not bfloat16
HQ_SCALE_BROADCAST = 0
HQ_SCALE_DIRECT = 1

MODES = {"mxfp8": HQ_MXFP8, "mxfp4": HQ_MXFP4, "nvfp4": HQ_NVFP4,
         "w8a8-mxfp8": HQ_MXFP8, "w4a4-mxfp4": HQ_MXFP4, "w4a4-nvfp4": HQ_NVFP4}

EXPORTED_SYMBOLS = (
    "hq_last_error", "hq_group_wise_quant", "hq_dense_gemm", "hq_batch_gemm",
    "hq_dense_gemm_ws", "hq_batch_gemm_ws", "hq_gemm_workspace_size", "hq_dense_gemm_scratch",
    "hq_group_contiguous_gemm", "hq_group_masked_gemm", "hq_fused_swiglu_quant",
    "hq_group_contiguous_gemm_swiglu_quant", "hq_group_contiguous_gemm_ptr_array",
    "hq_prefill_permute_to_masked_gemm", "hq_group_contiguous_gemm_dswiglu",
    "hq_group_contiguous_gemm_dswiglu_quant",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class HQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"hq status {status}: {msg}")
        self.status = status


def library_path():
    return os.path.join(_HERE, "libhq.so")


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64

_SIGS = {
    "hq_last_error": ([], ctypes.c_char_p),
    "hq_group_wise_quant": ([_VP, _I32, _VP, _I64, _I64, _VP, _VP, _VP, _U32], _I32),
    "hq_dense_gemm": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32], _I32),
    "hq_batch_gemm": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I32], _I32),
    "hq_dense_gemm_ws": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _VP, _U64],
                         _I32),
    "hq_batch_gemm_ws": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I32, _VP,
                          _U64], _I32),
    "hq_gemm_workspace_size": ([_I32, _I64, _I64, _I64, _I64, _I32, ctypes.POINTER(ctypes.c_uint64)], _I32),
    "hq_dense_gemm_scratch": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32], _I32),
    "hq_group_contiguous_gemm": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP,
                                  _I64, _I64, _I64, _I32], _I32),
    "hq_group_contiguous_gemm_ptr_array": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP,
                                            _I64, _I64, _I64, _I32], _I32),
    "hq_group_contiguous_gemm_swiglu_quant": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP,
                                               _VP, _VP, _VP, _I64, _I64, _I64, _I32], _I32),
    "hq_group_contiguous_gemm_dswiglu": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP,
                                          _VP, _I64, _I64, _I64, _I32], _I32),
    "hq_group_contiguous_gemm_dswiglu_quant": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP,
                                                _VP, _VP, _VP, _I64, _I64, _I64, _I32], _I32),
    "hq_group_masked_gemm": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _VP, _VP, _VP,
                              _I64, _I64, _I32], _I32),
    "hq_fused_swiglu_quant": ([_VP, _I32, _VP, _I64, _I64, _I32, _VP, _I64, _VP, _VP, _VP,
                               _VP, _VP], _I32),
    "hq_prefill_permute_to_masked_gemm": ([_VP, _VP, _I64, _I64, _I64, _VP, _I32, _VP, _I32, _I32,
                                           _I64, _VP, _VP, _VP, _VP], _I32),
}


def load():
    """Loads libhq.so once and declares the C signatures."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: the HIP library has not been built "
                               "(python -m fp4_gemm_moe_amd.build)")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def hq_last_error():
    return load().hq_last_error().decode()


def _mode(mode):
    if isinstance(mode, str):
        return MODES[mode]
    return int(mode)


def group_size(mode):
    return 16 if _mode(mode) == HQ_NVFP4 else 32


def code_cols(mode, k):
    """Bytes per row of the code tensor for logical width k."""
    return k if _mode(mode) == HQ_MXFP8 else k // 2


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(*ts):
    dev = next((t.device for t in ts if t is not None), None)
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, numel=None, shape_last=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _check(status):
    if status != 0:
        raise HQError(status, hq_last_error())


# ---------------------------------------------------------------- the six calls
def hq_group_wise_quant(mode, x, q, sf, global_scale=None, flags=0):
    """x [m, k] bf16 or float16 -> q [m, K'] uint8, sf [m, k/gs] uint8 (in
    place; a float16 x sets HQ_IN_FP16).  NVFP4: global_scale is a float32 [1]
    tensor (read with HQ_GS_INPUT, else written)."""
    mode = _mode(mode)
    m, k = x.shape
    if x.dtype == torch.float16:
        _need(x, "x", torch.float16)
        flags |= HQ_IN_FP16
    else:
        _need(x, "x", torch.bfloat16)
    _need(q, "q", torch.uint8, m * code_cols(mode, k))
    _need(sf, "sf", torch.uint8, m * (k // group_size(mode)))
    _need(global_scale, "global_scale", torch.float32, 1)
    _check(load().hq_group_wise_quant(_stream(x), mode, _p(x), m, k, _p(q), _p(sf),
                                      _p(global_scale), flags))


def _out_mode(mode, out):
    """The mode passed to a GEMM call: HQ_OUT_FP16 added for a float16 out."""
    return mode | (HQ_OUT_FP16 if out is not None and out.dtype == torch.float16 else 0)


def _need_out(out, numel):
    if out is not None and out.dtype == torch.float16:
        _need(out, "out", torch.float16, numel)
    else:
        _need(out, "out", torch.bfloat16, numel)


def _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, rows, n, k, groups, bias_groups):
    _need(a, "a", torch.uint8, rows * code_cols(mode, k))
    _need(sfa, "sfa", torch.uint8, rows * (k // group_size(mode)))
    _need(b, "b", torch.uint8, groups * n * code_cols(mode, k))
    _need(sfb, "sfb", torch.uint8, groups * n * (k // group_size(mode)))
    _need_out(out, rows * n)
    _need(bias, "bias", torch.bfloat16, bias_groups * n)
    _need(alpha, "alpha", torch.float32, bias_groups)


def _workspace(ws):
    """(pointer, bytes) of a caller workspace tensor (any dtype, contiguous,
    on the device), or (None, 0)."""
    if ws is None:
        return None, 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return _p(ws), ws.numel() * ws.element_size()


def hq_gemm_workspace_size(mode, m, n, k, batch=1, cu_limit=0):
    """Bytes of FP32 workspace a dense (batch=1) or batch GEMM of this shape
    uses on the current device (0: it never splits K)."""
    out = ctypes.c_uint64(0)
    _check(load().hq_gemm_workspace_size(_mode(mode), batch, m, n, k, cu_limit, ctypes.byref(out)))
    return int(out.value)


def gemm_workspace(mode, m, n, k, batch=1, cu_limit=0, device=None):
    """Allocates (with torch) the workspace hq_gemm_workspace_size asks for:
    a uint8 device tensor, or None when the shape needs none.  Allocate it
    before graph capture and pass it on every call."""
    nbytes = hq_gemm_workspace_size(mode, m, n, k, batch, cu_limit)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device or torch.device("cuda"))


def hq_dense_gemm(mode, a, sfa, b, sfb, out, bias=None, alpha=None, m=None, n=None, k=None,
                  cu_limit=0, workspace=None):
    """out[m, n] = a[m, k] * b[n, k]^T (+bias[n]) (*alpha[0]) in BF16.  With a
    workspace tensor (gemm_workspace) the call may split K (hq_dense_gemm_ws)."""
    mode = _mode(mode)
    m = out.shape[0] if m is None else m
    n = out.shape[-1] if n is None else n
    k = a.shape[-1] * (1 if mode == HQ_MXFP8 else 2) if k is None else k
    _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, m, n, k, 1, 1)
    wp, wb = _workspace(workspace)
    _check(load().hq_dense_gemm_ws(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(b), _p(sfb),
                                   _p(bias), _p(alpha), _p(out), m, n, k, cu_limit, wp, wb))


HQ_SCRATCH_BYTES = 32 << 20


def hq_dense_gemm_scratch(mode, a, sfa, b, sfb, out, bias=None, alpha=None, cu_limit=0):
    """hq_dense_gemm_ws whose K-split workspace is the library's static
    scratch (HQ_SCRATCH_BYTES per GPU): allocates nothing; shapes whose split
    needs more are refused; calls overlapping on one GPU race."""
    mode = _mode(mode)
    m, n = out.shape[0], out.shape[-1]
    k = a.shape[-1] * (1 if mode == HQ_MXFP8 else 2)
    _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, m, n, k, 1, 1)
    _check(load().hq_dense_gemm_scratch(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(b), _p(sfb),
                                        _p(bias), _p(alpha), _p(out), m, n, k, cu_limit))


def hq_batch_gemm(mode, a, sfa, b, sfb, out, bias=None, alpha=None, cu_limit=0, workspace=None):
    """out[B, m, n] = a[B, m, k] * b[B, n, k]^T per batch item (a workspace:
    hq_batch_gemm_ws)."""
    mode = _mode(mode)
    B, m, kc = a.shape
    n = b.shape[1]
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, B * m, n, k, B, B)
    wp, wb = _workspace(workspace)
    _check(load().hq_batch_gemm_ws(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(b), _p(sfb),
                                   _p(bias), _p(alpha), _p(out), B, m, n, k, cu_limit, wp, wb))


def hq_group_contiguous_gemm(mode, a, sfa, b, sfb, group_end, out, bias=None, alpha=None,
                             cu_limit=0):
    """Group g (rows [group_end[g-1], group_end[g]) of a) times b[g]^T."""
    mode = _mode(mode)
    rows, kc = a.shape
    E, n, _ = b.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    _need(group_end, "group_end", torch.int32, E)
    _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, rows, n, k, E, E)
    _check(load().hq_group_contiguous_gemm(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(b), _p(sfb),
                                           _p(group_end), E, _p(bias), _p(alpha), _p(out),
                                           rows, n, k, cu_limit))


def ptr_arrays(mode, bs, sfbs, n, k):
    """Device arrays (int64) of the addresses of per-expert weight tensors
    bs[g] [n, K'] and sfbs[g] [n, k/gs] (uint8, contiguous, 16-byte aligned),
    checked here (the C layer cannot see them).  Built once -- a blocking
    host-to-device copy -- before any graph capture, then passed to
    hq_group_contiguous_gemm_ptr_array on every call."""
    mode = _mode(mode)
    E = len(bs)
    if len(sfbs) != E:
        raise ValueError("bs and sfbs must have one tensor per group")
    for g in range(E):
        _need(bs[g], f"bs[{g}]", torch.uint8, n * code_cols(mode, k))
        _need(sfbs[g], f"sfbs[{g}]", torch.uint8, n * (k // group_size(mode)))
        if bs[g].data_ptr() % 16 or sfbs[g].data_ptr() % 16:
            raise ValueError(f"bs[{g}] and sfbs[{g}] must be 16-byte aligned")
    dev = bs[0].device if E else torch.device("cuda")
    bp = torch.tensor([t.data_ptr() for t in bs], dtype=torch.int64).to(dev, non_blocking=False)
    sp = torch.tensor([t.data_ptr() for t in sfbs], dtype=torch.int64).to(dev, non_blocking=False)
    return bp, sp


def hq_group_contiguous_gemm_ptr_array(mode, a, sfa, bs, sfbs, group_end, out, n, bias=None,
                                       alpha=None, cu_limit=0):
    """Grouped-contiguous GEMM whose group g uses its own weight tensors.
    bs / sfbs are either lists of the per-expert tensors (the binding then
    builds the address arrays with ptr_arrays: a host-to-device copy, so such
    a call cannot be graph-captured) or the int64 device arrays that
    ptr_arrays returned (no copy; capturable).  Returns the arrays used."""
    mode = _mode(mode)
    rows, kc = a.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    if isinstance(bs, torch.Tensor):
        bp, sp = bs, sfbs
        E = bp.numel()
        _need(bp, "b_ptrs", torch.int64, E)
        _need(sp, "sfb_ptrs", torch.int64, E)
    else:
        bp, sp = ptr_arrays(mode, bs, sfbs, n, k)
        E = len(bs)
    _need(a, "a", torch.uint8, rows * code_cols(mode, k))
    _need(sfa, "sfa", torch.uint8, rows * (k // group_size(mode)))
    _need(group_end, "group_end", torch.int32, E)
    _need_out(out, rows * n)
    _need(bias, "bias", torch.bfloat16, E * n)
    _need(alpha, "alpha", torch.float32, E)
    _check(load().hq_group_contiguous_gemm_ptr_array(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(bp), _p(sp),
                                                     _p(group_end), E, _p(bias), _p(alpha), _p(out),
                                                     rows, n, k, cu_limit))
    return bp, sp     # keep the address arrays alive until the stream has run the call


def hq_group_contiguous_gemm_swiglu_quant(mode, a, sfa, b, sfb, group_end, q, sf, valid=None,
                                          bias=None, y_debug=None, cu_limit=0):
    """The gate|up grouped-contiguous GEMM (b [E, 2h, k]) with SwiGLU and the
    MXFP8 re-quant in its epilogue: q [rows, h], sf [rows, h/32] as
    hq_fused_swiglu_quant would write them from the GEMM's BF16 output."""
    mode = _mode(mode)
    rows, kc = a.shape
    E, n, _ = b.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    h = n // 2
    _need(a, "a", torch.uint8, rows * code_cols(mode, k))
    _need(sfa, "sfa", torch.uint8, rows * (k // group_size(mode)))
    _need(b, "b", torch.uint8, E * n * code_cols(mode, k))
    _need(sfb, "sfb", torch.uint8, E * n * (k // group_size(mode)))
    _need(group_end, "group_end", torch.int32, E)
    _need(valid, "valid", torch.int32, E)
    _need(bias, "bias", torch.bfloat16, E * n)
    _need(q, "q", torch.uint8, rows * h)
    _need(sf, "sf", torch.uint8, rows * (h // 32))
    _need(y_debug, "y_debug", torch.float32, rows * h)
    _check(load().hq_group_contiguous_gemm_swiglu_quant(
        _stream(a), mode, _p(a), _p(sfa), _p(b), _p(sfb), _p(group_end), E, _p(valid), _p(bias),
        _p(q), _p(sf), _p(y_debug), rows, h, k, cu_limit))


def hq_group_contiguous_gemm_dswiglu(mode, a, sfa, b, sfb, group_end, c, prob, dprob, d, alpha=None,
                                     beta=None, cu_limit=0):
    """Backward grouped GEMM with the dSwiGLU epilogue: R = alpha[g]^2 a b[g]^T
    (b [E, n, K']), combined with the forward activations c [rows, 2n] bf16
    (32-column input / gate blocks) scaled by beta[g] and with prob [rows]
    float32 -> d [rows, 2n] bf16; dprob [rows] float32 accumulates the row
    sums (in place)."""
    mode = _mode(mode)
    rows, kc = a.shape
    E, n, _ = b.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    _need(a, "a", torch.uint8, rows * code_cols(mode, k))
    _need(sfa, "sfa", torch.uint8, rows * (k // group_size(mode)))
    _need(b, "b", torch.uint8, E * n * code_cols(mode, k))
    _need(sfb, "sfb", torch.uint8, E * n * (k // group_size(mode)))
    _need(group_end, "group_end", torch.int32, E)
    _need(c, "c", torch.bfloat16, rows * 2 * n)
    _need(prob, "prob", torch.float32, rows)
    _need(dprob, "dprob", torch.float32, rows)
    _need(d, "d", torch.bfloat16, rows * 2 * n)
    _need(alpha, "alpha", torch.float32, E)
    _need(beta, "beta", torch.float32, E)
    _check(load().hq_group_contiguous_gemm_dswiglu(
        _stream(a), mode, _p(a), _p(sfa), _p(b), _p(sfb), _p(group_end), E, _p(c), _p(alpha), _p(beta),
        _p(prob), _p(dprob), _p(d), rows, n, k, cu_limit))


def hq_group_contiguous_gemm_dswiglu_quant(mode, a, sfa, b, sfb, group_end, c, prob, dprob, dq, dsf,
                                           alpha=None, beta=None, cu_limit=0):
    """hq_group_contiguous_gemm_dswiglu with D written row-quantised: dq
    [rows, 2n] uint8 E4M3 codes and dsf [rows, 2n/32] uint8 UE8M0 scales (the
    MXFP8 rule of hq_group_wise_quant on the BF16 D)."""
    mode = _mode(mode)
    rows, kc = a.shape
    E, n, _ = b.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    _need(a, "a", torch.uint8, rows * code_cols(mode, k))
    _need(sfa, "sfa", torch.uint8, rows * (k // group_size(mode)))
    _need(b, "b", torch.uint8, E * n * code_cols(mode, k))
    _need(sfb, "sfb", torch.uint8, E * n * (k // group_size(mode)))
    _need(group_end, "group_end", torch.int32, E)
    _need(c, "c", torch.bfloat16, rows * 2 * n)
    _need(prob, "prob", torch.float32, rows)
    _need(dprob, "dprob", torch.float32, rows)
    _need(dq, "dq", torch.uint8, rows * 2 * n)
    _need(dsf, "dsf", torch.uint8, rows * 2 * n // 32)
    _need(alpha, "alpha", torch.float32, E)
    _need(beta, "beta", torch.float32, E)
    _check(load().hq_group_contiguous_gemm_dswiglu_quant(
        _stream(a), mode, _p(a), _p(sfa), _p(b), _p(sfb), _p(group_end), E, _p(c), _p(alpha), _p(beta),
        _p(prob), _p(dprob), _p(dq), _p(dsf), rows, n, k, cu_limit))


def hq_group_masked_gemm(mode, a, sfa, b, sfb, masked_m, out, max_m, bias=None, alpha=None,
                         cu_limit=0):
    """Expert e: the first masked_m[e] rows of slot [e*max_m, (e+1)*max_m)."""
    mode = _mode(mode)
    rows, kc = a.shape
    E, n, _ = b.shape
    k = kc * (1 if mode == HQ_MXFP8 else 2)
    if rows != E * max_m:
        raise ValueError(f"a has {rows} rows, expected num_groups * max_m = {E * max_m}")
    _need(masked_m, "masked_m", torch.int32, E)
    _gemm_common(mode, a, sfa, b, sfb, out, bias, alpha, rows, n, k, E, E)
    _check(load().hq_group_masked_gemm(_stream(a), _out_mode(mode, out), _p(a), _p(sfa), _p(b), _p(sfb),
                                       _p(masked_m), E, max_m, _p(bias), _p(alpha), _p(out),
                                       n, k, cu_limit))


def hq_fused_swiglu_quant(mode, x, q, sf, num_groups, group_end=None, slot_rows=0, valid=None,
                          global_scale=None, y_debug=None):
    """x [rows, 2h] = [gate | up] -> y = up * silu(gate) quantised into q, sf."""
    mode = _mode(mode)
    rows, h2 = x.shape
    h = h2 // 2
    _need(x, "x", torch.bfloat16)
    _need(q, "q", torch.uint8, rows * code_cols(mode, h))
    _need(sf, "sf", torch.uint8, rows * (h // group_size(mode)))
    _need(group_end, "group_end", torch.int32, num_groups)
    _need(valid, "valid", torch.int32, num_groups)
    _need(global_scale, "global_scale", torch.float32, 1)
    _need(y_debug, "y_debug", torch.float32, rows * h)
    _check(load().hq_fused_swiglu_quant(_stream(x), mode, _p(x), rows, h, num_groups,
                                        _p(group_end), slot_rows, _p(valid), _p(q), _p(sf),
                                        _p(global_scale), _p(y_debug)))


def hq_prefill_permute_to_masked_gemm(x, scale, topk_ids, num_local_experts, max_token_num,
                                      permute_x, out_scale, indice_map, token_nums, hidden=None):
    """Token permute into the masked-GEMM layout, in place: x [T, row_bytes
    as any dtype] rows go to permute_x [E * max_token_num, ...] by topk_ids
    [T, topk] int64; scale is int32 [T, hidden/512] (broadcast mode) or uint8
    [T, hidden/32] (direct mode); out_scale uint8 [E, max_token_num,
    hidden/32]; indice_map int32 [T, topk]; token_nums int32 [E]."""
    T = x.shape[0]
    row_bytes = x[0].numel() * x.element_size() if T > 0 else x.shape[-1] * x.element_size()
    if scale.dtype == torch.int32:
        mode, hidden = HQ_SCALE_BROADCAST, (scale.shape[-1] * 512 if hidden is None else hidden)
    elif scale.dtype == torch.uint8:
        mode, hidden = HQ_SCALE_DIRECT, (scale.shape[-1] * 32 if hidden is None else hidden)
    else:
        raise ValueError("scale must be int32 (broadcast mode) or uint8 (direct mode)")
    topk = topk_ids.shape[-1]
    E, M = int(num_local_experts), int(max_token_num)
    for t, name in ((x, "x"), (permute_x, "permute_x")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if permute_x.numel() * permute_x.element_size() != E * M * row_bytes:
        raise ValueError("permute_x must hold num_local_experts * max_token_num rows of x's width")
    _need(scale, "scale", scale.dtype, T * (hidden // (512 if mode == HQ_SCALE_BROADCAST else 32)))
    _need(topk_ids, "topk_ids", torch.int64, T * topk)
    _need(out_scale, "out_scale", torch.uint8, E * M * (hidden // 32))
    _need(indice_map, "indice_map", torch.int32, T * topk)
    _need(token_nums, "token_nums", torch.int32, E)
    _check(load().hq_prefill_permute_to_masked_gemm(
        _stream(x), _p(x), T, row_bytes, hidden, _p(scale), mode, _p(topk_ids), topk, E, M,
        _p(permute_x), _p(out_scale), _p(indice_map), _p(token_nums)))


def prefill_permute_to_masked_gemm(x, scale, topk_ids, num_local_experts, max_token_num):
    """The page's call: returns (permute_x [E * max_token_num, ...] with x's
    dtype, output_scale [E, max_token_num, hidden/32] uint8, permuted_indice_map
    [T, topk] int32, token_nums_per_expert [E, 1] int32).  Rows of permute_x
    past an expert's count are left uninitialised."""
    E, M = int(num_local_experts), int(max_token_num)
    T, topk = topk_ids.shape
    hidden = scale.shape[-1] * (512 if scale.dtype == torch.int32 else 32)
    dev = x.device
    px = torch.empty((E * M,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
    osf = torch.empty((E, M, hidden // 32), dtype=torch.uint8, device=dev)
    imap = torch.empty((T, topk), dtype=torch.int32, device=dev)
    nums = torch.empty((E, 1), dtype=torch.int32, device=dev)
    hq_prefill_permute_to_masked_gemm(x, scale, topk_ids, E, M, px, osf, imap, nums, hidden)
    return px, osf, imap, nums


# ---------------------------------------------------------------- allocation helper
def quantize(x, mode, global_scale=None):
    """Allocates (q, sf, g) with torch and runs hq_group_wise_quant.  For
    NVFP4, g is computed unless a float32 [1] global_scale is supplied."""
    mode = _mode(mode)
    m, k = x.shape
    q = torch.empty((m, code_cols(mode, k)), dtype=torch.uint8, device=x.device)
    sf = torch.empty((m, k // group_size(mode)), dtype=torch.uint8, device=x.device)
    g = None
    flags = 0
    if mode == HQ_NVFP4:
        if global_scale is not None:
            g = global_scale
            flags = HQ_GS_INPUT
        else:
            g = torch.empty(1, dtype=torch.float32, device=x.device)
    hq_group_wise_quant(mode, x, q, sf, g, flags)
    return q, sf, g
