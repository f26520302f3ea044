"""ctypes binding of ``libfp8rl.so`` (the C ABI declared in include/fp8rl.h).

Argument marshalling only: every function here checks that the tensors are what the C call
expects (device, dtype, row-major with unit column stride), passes raw device pointers, row
pitches and the current HIP stream, and turns a non-zero status into ``Fp8rlError``. All of the
arithmetic runs in the library's HIP kernels. There is no fallback: if the library is missing or
cannot be loaded, every call raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import functools
import inspect
import os
import threading

import torch

from .build import LIB_PATH

FP8RL_OUT_BF16 = 0
FP8RL_OUT_F32 = 1
FP8RL_ACCUM_FP8 = 0
FP8RL_ACCUM_F16 = 1
FP8RL_ACCUM_MX = 2
FP8RL_ACCUM_AUTO = 3
FP8RL_SCALE_FP32 = 0
FP8RL_SCALE_POW2 = 1
FP8RL_OP_GEMM = 0
FP8RL_OP_GROUPED_GEMM = 1
FP8RL_OP_GEMM_ROWSCALED = 2
FP8RL_OP_GEMM_FUSED_ACT = 3
FP8RL_OP_GROUPED_GEMM_FUSED_ACT = 4

class WeightDesc(ctypes.Structure):
    """fp8rl_weight_desc (include/fp8rl.h)."""

    _fields_ = [("w", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("sw", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ld_w", ctypes.c_int64),
                ("ld_wq", ctypes.c_int64)]


class TensorDesc(ctypes.Structure):
    """fp8rl_tensor_desc (include/fp8rl.h)."""

    _fields_ = [("x", ctypes.c_void_p), ("amax", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64)]


class QuantDesc(ctypes.Structure):
    """fp8rl_quant_desc (include/fp8rl.h)."""

    _fields_ = [("x", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("slot_mapping", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64), ("out_rows", ctypes.c_int64),
                ("ld_out", ctypes.c_int64)]


_lock = threading.Lock()
_lib = None


class Fp8rlError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        msg = lib().fp8rl_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{func} failed with status {status}: {msg}")


def declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and result types of every C ABI function on a loaded copy of the
    library (the in-tree build, or another build of the same sources); returns it."""
    i64, vp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "fp8rl_encode_e4m3_f32": (ctypes.c_int, [vp, i64, vp, vp]),
        "fp8rl_quant_weight_blk128": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, vp]),
        "fp8rl_quant_weight_blk128_batched": (ctypes.c_int,
                                              [ctypes.POINTER(WeightDesc), i32, vp]),
        "fp8rl_quant_act_tok128": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, vp]),
        "fp8rl_quant_weight_blk128_ex": (ctypes.c_int,
                                         [vp, i64, i64, i64, vp, i64, vp, ctypes.c_int, vp]),
        "fp8rl_quant_weight_blk128_batched_ex": (
            ctypes.c_int, [ctypes.POINTER(WeightDesc), i32, ctypes.c_int, vp]),
        "fp8rl_quant_act_tok128_ex": (ctypes.c_int,
                                      [vp, i64, i64, i64, vp, i64, vp, ctypes.c_int, vp]),
        "fp8rl_gemm_w8a8_blockscaled": (
            ctypes.c_int,
            [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, i64, ctypes.c_int, vp, sz, vp]),
        "fp8rl_grouped_gemm_w8a8": (
            ctypes.c_int,
            [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, ctypes.c_int, ctypes.c_int, vp, sz, vp]),
        "fp8rl_amax_bf16": (ctypes.c_int, [vp, i64, i64, i64, vp, vp]),
        "fp8rl_amax_bf16_batched": (ctypes.c_int, [ctypes.POINTER(TensorDesc), i32, vp]),
        "fp8rl_scale_from_amax": (ctypes.c_int, [vp, i32, vp, vp]),
        "fp8rl_quant_bf16_per_tensor": (ctypes.c_int,
                                        [vp, i64, i64, i64, vp, vp, i64, i64, vp, vp]),
        "fp8rl_quant_bf16_per_tensor_batched": (ctypes.c_int,
                                                [ctypes.POINTER(QuantDesc), i32, vp]),
        "fp8rl_quant_weight_blk128_t": (
            ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, vp, i64, vp, ctypes.c_int, vp]),
        "fp8rl_quant_act_colwise128": (
            ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, vp, i64, vp, ctypes.c_int, vp]),
        "fp8rl_gemm_w8a8_rowscaled": (
            ctypes.c_int,
            [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, i64, ctypes.c_int, vp, sz, vp]),
        "fp8rl_gemm_w8a8_blockscaled_noalloc": (
            ctypes.c_int,
            [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, i64, ctypes.c_int, vp]),
        "fp8rl_gemm_w8a8_fused_act_quant": (
            ctypes.c_int,
            [vp, i64, vp, vp, i64, i64, i64, vp, ctypes.c_int, i64, ctypes.c_int,
             ctypes.c_int, vp, sz, vp]),
        "fp8rl_grouped_gemm_w8a8_fused_act_quant": (
            ctypes.c_int,
            [vp, i64, i64, vp, vp, vp, vp, i32, i64, i64, i64, vp, ctypes.c_int, ctypes.c_int,
             ctypes.c_int, vp, sz, vp]),
        "fp8rl_workspace_bytes": (sz, [ctypes.c_int, i64, i64, i64, i32]),
        "fp8rl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "fp8rl_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m fp8_blockwise_quantization_amd.build`"
            )
        L = declare(ctypes.CDLL(LIB_PATH))
        _lib = L
        return L


EXPORTED = (
    "fp8rl_encode_e4m3_f32",
    "fp8rl_quant_weight_blk128",
    "fp8rl_quant_weight_blk128_batched",
    "fp8rl_quant_act_tok128",
    "fp8rl_quant_weight_blk128_ex",
    "fp8rl_quant_weight_blk128_batched_ex",
    "fp8rl_quant_act_tok128_ex",
    "fp8rl_gemm_w8a8_blockscaled",
    "fp8rl_grouped_gemm_w8a8",
    "fp8rl_amax_bf16",
    "fp8rl_amax_bf16_batched",
    "fp8rl_scale_from_amax",
    "fp8rl_quant_bf16_per_tensor",
    "fp8rl_quant_bf16_per_tensor_batched",
    "fp8rl_quant_weight_blk128_t",
    "fp8rl_quant_act_colwise128",
    "fp8rl_gemm_w8a8_rowscaled",
    "fp8rl_gemm_w8a8_fused_act_quant",
    "fp8rl_gemm_w8a8_blockscaled_noalloc",
    "fp8rl_grouped_gemm_w8a8_fused_act_quant",
    "fp8rl_workspace_bytes",
    "fp8rl_status_string",
    "fp8rl_version",
)


def _scale_code(scale) -> int:
    """'fp32' / 'pow2' (or the fp8rl_scale_fmt value) -> fp8rl_scale_fmt."""
    codes = {"fp32": FP8RL_SCALE_FP32, "pow2": FP8RL_SCALE_POW2}
    if isinstance(scale, str):
        if scale not in codes:
            raise ValueError(f"scale must be one of {sorted(codes)}")
        return codes[scale]
    return int(scale)


def _check(status: int, func: str) -> None:
    if status != 0:
        raise Fp8rlError(status, func)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@contextlib.contextmanager
def _on_stream(stream):
    """Make `stream` torch's current stream while a binding runs, so that the tensors it
    allocates (outputs, temporary workspaces) and the workspace header's zero fill are ordered on
    the stream the kernels run on, and the caching allocator hands a freed temporary to another
    allocation only behind that stream's work."""
    if stream is None:
        yield
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    with torch.cuda.stream(s):
        yield


def _allocs_on_stream(fn):
    """Run `fn` under _on_stream of its `stream` argument (keyword or positional)."""
    idx = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = kwargs["stream"] if "stream" in kwargs else (args[idx] if len(args) > idx else None)
        with _on_stream(stream):
            return fn(*args, **kwargs)

    return wrapper


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _rows(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int = 2):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    return t.stride(-2) if ndim >= 2 else t.numel()


def _dense(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous cuda {dtype} tensor")


def _blocks(n: int) -> int:
    """128-wide blocks covering n (a dimension that is not a multiple of 128 is left to the C
    call, which rejects it with its own status)."""
    return -(-n // 128)


def _sizes(**want):
    """Raise unless each tensor has the stated element count (int) or shape (tuple): the C calls
    take only pointers and pitches, so a smaller tensor would be read or written past its end."""
    for name, (t, w) in want.items():
        if t is None:
            continue
        ok = t.numel() == w if isinstance(w, int) else tuple(t.shape) == tuple(w)
        if not ok:
            got = t.numel() if isinstance(w, int) else tuple(t.shape)
            raise ValueError(f"{name} has {got}, expected {w}")


# ---------------------------------------------------------------------------------------------
# One Python function per C entry point, same name, tensors in place of pointers.
# ---------------------------------------------------------------------------------------------


@_allocs_on_stream
def fp8rl_encode_e4m3_f32(v: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    _dense(v, "v", torch.float32)
    if out is None:
        out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _dense(out, "out", torch.uint8)
    _check(lib().fp8rl_encode_e4m3_f32(_ptr(v), v.numel(), _ptr(out), _stream(stream)),
           "fp8rl_encode_e4m3_f32")
    return out


@_allocs_on_stream
def fp8rl_quant_weight_blk128(w: torch.Tensor, wq: torch.Tensor | None = None,
                              sw: torch.Tensor | None = None, stream=None, scale="fp32"):
    """bf16 W[N][K] -> (Wq uint8 [N][K], sw float32 [N/128][K/128]); scale 'fp32' or 'pow2'."""
    ld_w = _rows(w, "w", torch.bfloat16)
    N, K = w.shape
    if wq is None:
        wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if sw is None:
        sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    ld_wq = _rows(wq, "wq", torch.uint8)
    _dense(sw, "sw", torch.float32)
    if tuple(wq.shape) != (N, K) or sw.numel() != (N // 128) * (K // 128):
        raise ValueError("output shapes do not match the weight")
    fmt = _scale_code(scale)
    if fmt == FP8RL_SCALE_FP32:
        _check(lib().fp8rl_quant_weight_blk128(_ptr(w), N, K, ld_w, _ptr(wq), ld_wq, _ptr(sw),
                                               _stream(stream)), "fp8rl_quant_weight_blk128")
    else:
        _check(lib().fp8rl_quant_weight_blk128_ex(_ptr(w), N, K, ld_w, _ptr(wq), ld_wq, _ptr(sw),
                                                  fmt, _stream(stream)),
               "fp8rl_quant_weight_blk128_ex")
    return wq, sw


def fp8rl_quant_weight_blk128_ex(w, wq=None, sw=None, scale_fmt=FP8RL_SCALE_FP32, stream=None):
    return fp8rl_quant_weight_blk128(w, wq, sw, stream=stream, scale=scale_fmt)


def weight_descs(ws, wqs, sws):
    """Validate tensors and build the descriptor array for fp8rl_quant_weight_blk128_batched."""
    arr = (WeightDesc * len(ws))()
    for i, (w, wq, sw) in enumerate(zip(ws, wqs, sws)):
        ld_w = _rows(w, "w", torch.bfloat16)
        ld_wq = _rows(wq, "wq", torch.uint8)
        _dense(sw, "sw", torch.float32)
        N, K = w.shape
        if tuple(wq.shape) != (N, K) or sw.numel() != (N // 128) * (K // 128):
            raise ValueError(f"descriptor {i}: output shapes do not match the weight")
        arr[i] = WeightDesc(_ptr(w), _ptr(wq), _ptr(sw), N, K, ld_w, ld_wq)
    return arr


def fp8rl_quant_weight_blk128_batched(ws, wqs, sws, stream=None, descs=None, scale="fp32"):
    """Re-quantize several bf16 weights in ceil(len/32) launches; outputs are given by the caller.

    ``descs`` may be a prebuilt array from ``weight_descs`` (saves re-validating every call)."""
    if descs is None:
        descs = weight_descs(ws, wqs, sws)
    fmt = _scale_code(scale)
    if fmt == FP8RL_SCALE_FP32:
        _check(lib().fp8rl_quant_weight_blk128_batched(descs, len(descs), _stream(stream)),
               "fp8rl_quant_weight_blk128_batched")
    else:
        _check(lib().fp8rl_quant_weight_blk128_batched_ex(descs, len(descs), fmt, _stream(stream)),
               "fp8rl_quant_weight_blk128_batched_ex")


def fp8rl_quant_weight_blk128_batched_ex(ws, wqs, sws, scale_fmt=FP8RL_SCALE_FP32, stream=None,
                                         descs=None):
    return fp8rl_quant_weight_blk128_batched(ws, wqs, sws, stream=stream, descs=descs,
                                             scale=scale_fmt)


@_allocs_on_stream
def fp8rl_quant_act_tok128(x: torch.Tensor, xq: torch.Tensor | None = None,
                           sa: torch.Tensor | None = None, stream=None, scale="fp32"):
    """bf16 X[M][K] -> (Xq uint8 [M][K], sa float32 [M][K/128]); scale 'fp32' or 'pow2'."""
    ld_x = _rows(x, "x", torch.bfloat16)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    ld_xq = _rows(xq, "xq", torch.uint8)
    _dense(sa, "sa", torch.float32)
    if tuple(xq.shape) != (M, K) or sa.numel() != M * (K // 128):
        raise ValueError("output shapes do not match the activation")
    fmt = _scale_code(scale)
    if fmt == FP8RL_SCALE_FP32:
        _check(lib().fp8rl_quant_act_tok128(_ptr(x), M, K, ld_x, _ptr(xq), ld_xq, _ptr(sa),
                                            _stream(stream)), "fp8rl_quant_act_tok128")
    else:
        _check(lib().fp8rl_quant_act_tok128_ex(_ptr(x), M, K, ld_x, _ptr(xq), ld_xq, _ptr(sa), fmt,
                                               _stream(stream)), "fp8rl_quant_act_tok128_ex")
    return xq, sa


def fp8rl_quant_act_tok128_ex(x, xq=None, sa=None, scale_fmt=FP8RL_SCALE_FP32, stream=None):
    return fp8rl_quant_act_tok128(x, xq, sa, stream=stream, scale=scale_fmt)


def fp8rl_workspace_bytes(op: int, M: int, N: int, K: int, E: int = 0) -> int:
    return int(lib().fp8rl_workspace_bytes(op, M, N, K, E))


WORKSPACE_HEADER_BYTES = 4096  # FP8RL_WORKSPACE_HEADER_BYTES: counters that must start at zero


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A GEMM workspace of at least ``nbytes`` whose counter header is zero (ready for any call;
    the library leaves the header zero after each call)."""
    ws = torch.empty(max(int(nbytes), WORKSPACE_HEADER_BYTES), dtype=torch.uint8, device=device)
    ws[:WORKSPACE_HEADER_BYTES].zero_()
    return ws


def _accum_code(accum, out_dtype=None) -> int:
    """None leaves the choice to the library (FP8RL_ACCUM_AUTO: the form that meets the accuracy
    contract for the call's output type and GEMM)."""
    if accum is None or accum in ("auto", FP8RL_ACCUM_AUTO):
        return FP8RL_ACCUM_AUTO
    if accum in ("fp8", FP8RL_ACCUM_FP8):
        return FP8RL_ACCUM_FP8
    if accum in ("f16", FP8RL_ACCUM_F16):
        return FP8RL_ACCUM_F16
    if accum in ("mx", FP8RL_ACCUM_MX):
        return FP8RL_ACCUM_MX
    raise ValueError("accum must be None, 'auto', 'fp8', 'f16' or 'mx'")


def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return FP8RL_OUT_BF16
    if dtype == torch.float32:
        return FP8RL_OUT_F32
    raise TypeError("output dtype must be torch.bfloat16 or torch.float32")


@_allocs_on_stream
def fp8rl_gemm_w8a8_blockscaled(xq, sa, wq, sw, out_dtype=torch.bfloat16, y=None,
                                workspace=None, stream=None, accum=None):
    """Y[M][N] = blockscaled Xq Wq^T (bf16 or float32)."""
    _dense(xq, "xq", torch.uint8)
    _dense(wq, "wq", torch.uint8)
    _dense(sa, "sa", torch.float32)
    _dense(sw, "sw", torch.float32)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("K mismatch between xq and wq")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    ld_y = _rows(y, "y", y.dtype)
    _sizes(sa=(sa, M * _blocks(K)), sw=(sw, _blocks(N) * _blocks(K)), y=(y, (M, N)))
    need = fp8rl_workspace_bytes(FP8RL_OP_GEMM, M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8rl_gemm_w8a8_blockscaled(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sw), M, N, K,
                                             _ptr(y), _out_code(y.dtype), ld_y,
                                             _accum_code(accum, y.dtype), _ptr(workspace),
                                             ws_bytes, _stream(stream)),
           "fp8rl_gemm_w8a8_blockscaled")
    return y


SCRATCH_BYTES = 32 << 20  # FP8RL_SCRATCH_BYTES: the no-allocation GEMM's static scratch per device


@_allocs_on_stream
def fp8rl_gemm_w8a8_blockscaled_noalloc(xq, sa, wq, sw, y, stream=None, accum=None):
    """Y = blockscaled Xq Wq^T into the caller's ``y`` (bf16 or float32), with the library's
    static scratch instead of a workspace: the C call allocates nothing (neither does this
    binding: ``y`` is required)."""
    _dense(xq, "xq", torch.uint8)
    _dense(wq, "wq", torch.uint8)
    _dense(sa, "sa", torch.float32)
    _dense(sw, "sw", torch.float32)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("K mismatch between xq and wq")
    ld_y = _rows(y, "y", y.dtype)
    _sizes(sa=(sa, M * _blocks(K)), sw=(sw, _blocks(N) * _blocks(K)), y=(y, (M, N)))
    _check(lib().fp8rl_gemm_w8a8_blockscaled_noalloc(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sw), M, N,
                                                     K, _ptr(y), _out_code(y.dtype), ld_y,
                                                     _accum_code(accum, y.dtype),
                                                     _stream(stream)),
           "fp8rl_gemm_w8a8_blockscaled_noalloc")
    return y


@_allocs_on_stream
def fp8rl_gemm_w8a8_rowscaled(aq, sa, bq, sb, out_dtype=torch.bfloat16, y=None, workspace=None,
                              stream=None, accum=None):
    """Y[M][N] = sum over 128-wide K slices of sa[m][kb] sb[n][kb] (Aq Bq^T)_kb: both operands
    scaled per row and slice (the weight-gradient GEMM)."""
    _dense(aq, "aq", torch.uint8)
    _dense(bq, "bq", torch.uint8)
    _dense(sa, "sa", torch.float32)
    _dense(sb, "sb", torch.float32)
    M, K = aq.shape
    N = bq.shape[0]
    if bq.shape[1] != K or sb.numel() != N * (K // 128) or sa.numel() != M * (K // 128):
        raise ValueError("shape mismatch between aq, sa, bq and sb")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    ld_y = _rows(y, "y", y.dtype)
    _sizes(y=(y, (M, N)))
    need = fp8rl_workspace_bytes(FP8RL_OP_GEMM_ROWSCALED, M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, aq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8rl_gemm_w8a8_rowscaled(_ptr(aq), _ptr(sa), _ptr(bq), _ptr(sb), M, N, K,
                                           _ptr(y), _out_code(y.dtype), ld_y,
                                           _accum_code(accum, y.dtype), _ptr(workspace), ws_bytes,
                                           _stream(stream)), "fp8rl_gemm_w8a8_rowscaled")
    return y


@_allocs_on_stream
def fp8rl_gemm_w8a8_fused_act_quant(x, wq, sw, out_dtype=torch.bfloat16, y=None, workspace=None,
                                    stream=None, accum=None, scale="fp32"):
    """Y[M][N] for bf16 X: quantize X in 1x128 groups (`scale` format) and multiply, in one call
    (one kernel up to 4 rows); the same bits as quant_act followed by the blockscaled GEMM."""
    ld_x = _rows(x, "x", torch.bfloat16)
    _dense(wq, "wq", torch.uint8)
    _dense(sw, "sw", torch.float32)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("K mismatch between x and wq")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    ld_y = _rows(y, "y", y.dtype)
    _sizes(sw=(sw, _blocks(N) * _blocks(K)), y=(y, (M, N)))
    need = fp8rl_workspace_bytes(FP8RL_OP_GEMM_FUSED_ACT, M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8rl_gemm_w8a8_fused_act_quant(_ptr(x), ld_x, _ptr(wq), _ptr(sw), M, N, K,
                                                 _ptr(y), _out_code(y.dtype), ld_y,
                                                 _accum_code(accum, y.dtype), _scale_code(scale),
                                                 _ptr(workspace), ws_bytes, _stream(stream)),
           "fp8rl_gemm_w8a8_fused_act_quant")
    return y


@_allocs_on_stream
def fp8rl_grouped_gemm_w8a8(xq, sa, wq, sw, expert_offsets, out_dtype=torch.bfloat16, y=None,
                            workspace=None, stream=None, accum=None):
    """Per-expert blockscaled GEMM over row segments given by device int32 ``expert_offsets``."""
    _dense(xq, "xq", torch.uint8)
    _dense(wq, "wq", torch.uint8)
    _dense(sa, "sa", torch.float32)
    _dense(sw, "sw", torch.float32)
    _dense(expert_offsets, "expert_offsets", torch.int32)
    M, K = xq.shape
    E, N, K2 = wq.shape
    if K2 != K or expert_offsets.numel() != E + 1:
        raise ValueError("shape mismatch between xq, wq and expert_offsets")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _dense(y, "y", y.dtype)
    _sizes(sa=(sa, M * _blocks(K)), sw=(sw, E * _blocks(N) * _blocks(K)), y=(y, (M, N)))
    need = fp8rl_workspace_bytes(FP8RL_OP_GROUPED_GEMM, M, N, K, E)
    if workspace is None and need > 0:
        workspace = new_workspace(need, xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8rl_grouped_gemm_w8a8(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sw),
                                         _ptr(expert_offsets), E, M, N, K, _ptr(y),
                                         _out_code(y.dtype), _accum_code(accum, y.dtype),
                                         _ptr(workspace), ws_bytes, _stream(stream)),
           "fp8rl_grouped_gemm_w8a8")
    return y


@_allocs_on_stream
def fp8rl_grouped_gemm_w8a8_fused_act_quant(x, wq, sw, expert_offsets, row_ids=None,
                                            out_dtype=torch.bfloat16, y=None, workspace=None,
                                            stream=None, accum=None, scale="fp32"):
    """Grouped GEMM on bf16 activations: grouped row r multiplies row ``row_ids[r]`` of ``x``
    (device int32; None: row r) quantized in 1x128 groups (`scale` format) with its expert's
    weights. Each row of ``x`` is quantized once; the same bits as quant_act on the gathered rows
    followed by the grouped GEMM."""
    ld_x = _rows(x, "x", torch.bfloat16)
    _dense(wq, "wq", torch.uint8)
    _dense(sw, "sw", torch.float32)
    _dense(expert_offsets, "expert_offsets", torch.int32)
    src_rows, K = x.shape
    E, N, K2 = wq.shape
    if K2 != K or expert_offsets.numel() != E + 1:
        raise ValueError("shape mismatch between x, wq and expert_offsets")
    if row_ids is not None:
        _dense(row_ids, "row_ids", torch.int32)
        M = row_ids.numel()
    else:
        M = src_rows
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _dense(y, "y", y.dtype)
    _sizes(sw=(sw, E * _blocks(N) * _blocks(K)), y=(y, (M, N)))
    need = fp8rl_workspace_bytes(FP8RL_OP_GROUPED_GEMM_FUSED_ACT, max(src_rows, M), N, K, E)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8rl_grouped_gemm_w8a8_fused_act_quant(
        _ptr(x), ld_x, src_rows, _ptr(row_ids), _ptr(wq), _ptr(sw), _ptr(expert_offsets), E, M, N,
        K, _ptr(y), _out_code(y.dtype), _accum_code(accum, y.dtype), _scale_code(scale),
        _ptr(workspace), ws_bytes, _stream(stream)), "fp8rl_grouped_gemm_w8a8_fused_act_quant")
    return y


# ---------------------------------------------------------------- per-tensor (Q/K/V, KV cache)


def _tensor_rows(x: torch.Tensor, name: str = "x") -> int:
    """Row pitch of a 2-D bf16 tensor with unit column stride (e.g. a column slice of a fused QKV
    output)."""
    return _rows(x, name, torch.bfloat16)


def fp8rl_amax_bf16(x: torch.Tensor, amax: torch.Tensor, stream=None):
    """amax (1-element float32) <- max(amax, max|x|) for a 2-D bf16 tensor; set amax to 0 first."""
    ld = _tensor_rows(x)
    _dense(amax, "amax", torch.float32)
    if amax.numel() != 1:
        raise ValueError("amax must hold one float32")
    rows, cols = x.shape
    _check(lib().fp8rl_amax_bf16(_ptr(x), rows, cols, ld, _ptr(amax), _stream(stream)),
           "fp8rl_amax_bf16")
    return amax


def tensor_descs(xs, amax: torch.Tensor):
    """Descriptor array for fp8rl_amax_bf16_batched: tensor i accumulates into amax[i]."""
    _dense(amax, "amax", torch.float32)
    if amax.numel() < len(xs):
        raise ValueError("one amax slot per tensor")
    arr = (TensorDesc * len(xs))()
    for i, x in enumerate(xs):
        ld = _tensor_rows(x, f"xs[{i}]")
        arr[i] = TensorDesc(_ptr(x), amax.data_ptr() + 4 * i, x.shape[0], x.shape[1], ld)
    return arr


def fp8rl_amax_bf16_batched(xs, amax: torch.Tensor, stream=None, descs=None):
    """amax[i] <- max(amax[i], max|xs[i]|) for every tensor, in ceil(len / 32) launches."""
    if descs is None:
        descs = tensor_descs(xs, amax)
    _check(lib().fp8rl_amax_bf16_batched(descs, len(descs), _stream(stream)),
           "fp8rl_amax_bf16_batched")
    return amax


@_allocs_on_stream
def fp8rl_scale_from_amax(amax: torch.Tensor, scale: torch.Tensor | None = None, stream=None):
    """scale[i] = fp32(amax[i] / 448), 1 where amax[i] == 0."""
    _dense(amax, "amax", torch.float32)
    if scale is None:
        scale = torch.empty_like(amax)
    _dense(scale, "scale", torch.float32)
    if scale.numel() != amax.numel():
        raise ValueError("scale and amax must have the same length")
    _check(lib().fp8rl_scale_from_amax(_ptr(amax), amax.numel(), _ptr(scale), _stream(stream)),
           "fp8rl_scale_from_amax")
    return scale


@_allocs_on_stream
def fp8rl_quant_bf16_per_tensor(x: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None,
                                slot_mapping: torch.Tensor | None = None, stream=None):
    """Codes of x / scale (device scalar) into out[slot[r]] (or out[r]); returns out (uint8)."""
    ld_x = _tensor_rows(x)
    rows, cols = x.shape
    if scale.dtype != torch.float32 or not scale.is_cuda or scale.numel() < 1:
        raise ValueError("scale must be a cuda float32 tensor holding the per-tensor scale")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    ld_out = _rows(out, "out", torch.uint8)
    if slot_mapping is not None:
        _dense(slot_mapping, "slot_mapping", torch.int64)
        if slot_mapping.numel() != rows:
            raise ValueError("one slot per row of x")
    _check(lib().fp8rl_quant_bf16_per_tensor(_ptr(x), rows, cols, ld_x, _ptr(scale), _ptr(out),
                                             out.shape[0], ld_out, _ptr(slot_mapping),
                                             _stream(stream)), "fp8rl_quant_bf16_per_tensor")
    return out


def quant_descs(xs, scales, outs, slots=None):
    """Descriptor array for fp8rl_quant_bf16_per_tensor_batched: xs[i] / scales[i] (a one-element
    cuda float32 tensor or view) into outs[i] at rows slots[i] (an int64 cuda tensor or None)."""
    arr = (QuantDesc * len(xs))()
    for i, (x, sc, out) in enumerate(zip(xs, scales, outs)):
        ld_x = _tensor_rows(x, f"xs[{i}]")
        if sc.dtype != torch.float32 or not sc.is_cuda or sc.numel() < 1:
            raise ValueError(f"scales[{i}] must be a cuda float32 tensor")
        ld_out = _rows(out, f"outs[{i}]", torch.uint8)
        sl = None if slots is None else slots[i]
        if sl is not None:
            _dense(sl, "slot_mapping", torch.int64)
            if sl.numel() != x.shape[0]:
                raise ValueError(f"descriptor {i}: one slot per row")
        arr[i] = QuantDesc(_ptr(x), _ptr(sc), _ptr(out), _ptr(sl), x.shape[0], x.shape[1], ld_x,
                           out.shape[0], ld_out)
    return arr


def fp8rl_quant_bf16_per_tensor_batched(xs=None, scales=None, outs=None, slots=None, stream=None,
                                        descs=None):
    """Per-tensor quantization of several tensors in ceil(len / 16) launches."""
    if descs is None:
        descs = quant_descs(xs, scales, outs, slots)
    _check(lib().fp8rl_quant_bf16_per_tensor_batched(descs, len(descs), _stream(stream)),
           "fp8rl_quant_bf16_per_tensor_batched")


# ------------------------------------------------------------------ backward (transposed outputs)


@_allocs_on_stream
def fp8rl_quant_weight_blk128_t(w: torch.Tensor, wqt=None, swt=None, wq=None, sw=None,
                                rowmajor: bool = False, scale="fp32", stream=None):
    """bf16 W[N][K] -> (WqT uint8 [K][N], swT float32 [K/128][N/128]), the block quantization of
    W^T; with ``rowmajor`` also (Wq [N][K], sw [N/128][K/128]) from the same read. Returns
    (wqt, swt, wq, sw) with wq, sw None unless asked for."""
    ld_w = _rows(w, "w", torch.bfloat16)
    N, K = w.shape
    dev = w.device
    if wqt is None:
        wqt = torch.empty((K, N), dtype=torch.uint8, device=dev)
    if swt is None:
        swt = torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev)
    if rowmajor and wq is None:
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if rowmajor and sw is None:
        sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    ld_wqt = _rows(wqt, "wqt", torch.uint8)
    _dense(swt, "swt", torch.float32)
    ld_wq = 0
    if wq is not None:
        ld_wq = _rows(wq, "wq", torch.uint8)
        _dense(sw, "sw", torch.float32)
    _check(lib().fp8rl_quant_weight_blk128_t(_ptr(w), N, K, ld_w, _ptr(wq), ld_wq, _ptr(sw),
                                             _ptr(wqt), ld_wqt, _ptr(swt), _scale_code(scale),
                                             _stream(stream)), "fp8rl_quant_weight_blk128_t")
    return wqt, swt, wq, sw


@_allocs_on_stream
def fp8rl_quant_act_colwise128(x: torch.Tensor, xtq=None, sat=None, xq=None, sa=None,
                               rowwise: bool = False, scale="fp32", stream=None):
    """bf16 X[M][K] (M % 128 == 0) -> (XtQ uint8 [K][M], st float32 [K][M/128]): 128x1 token
    groups stored transposed; with ``rowwise`` also the 1x128 row quantization (Xq, sa) from the
    same read. Returns (xtq, sat, xq, sa)."""
    ld_x = _rows(x, "x", torch.bfloat16)
    M, K = x.shape
    dev = x.device
    if xtq is None:
        xtq = torch.empty((K, M), dtype=torch.uint8, device=dev)
    if sat is None:
        sat = torch.empty((K, M // 128), dtype=torch.float32, device=dev)
    if rowwise and xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if rowwise and sa is None:
        sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    ld_xtq = _rows(xtq, "xtq", torch.uint8)
    _dense(sat, "sat", torch.float32)
    ld_xq = 0
    if xq is not None:
        ld_xq = _rows(xq, "xq", torch.uint8)
        _dense(sa, "sa", torch.float32)
    _check(lib().fp8rl_quant_act_colwise128(_ptr(x), M, K, ld_x, _ptr(xq), ld_xq, _ptr(sa),
                                            _ptr(xtq), ld_xtq, _ptr(sat), _scale_code(scale),
                                            _stream(stream)), "fp8rl_quant_act_colwise128")
    return xtq, sat, xq, sa
