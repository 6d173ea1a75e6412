"""Matryoshka-nested integer matmul on MI355X (gfx950).

A thin Python binding over the C ABI of libmq.so (include/mq.h): argument
marshalling only; every step of the computation runs in the library's HIP
kernels.  torch is used for device memory and streams.

    import nested_int_matmul_amd as mq
    codes, alpha, zero = mq.quantize(w_fp32_cuda, group=128)
    plane = mq.pack(codes, r=4)
    y = mq.gemm(plane, 4, alpha, zero, 128, x_bf16_cuda)
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmq.so")

MQ_OK = 0
STATUS_NAMES = {
    0: "MQ_OK", 1: "MQ_ERR_NULL", 2: "MQ_ERR_SHAPE", 3: "MQ_ERR_PRECISION",
    4: "MQ_ERR_GROUP", 5: "MQ_ERR_ALIGN", 6: "MQ_ERR_WORKSPACE", 7: "MQ_ERR_DEVICE",
    8: "MQ_ERR_HIP",
}

# Every exported symbol of include/mq.h.
EXPORTS = (
    "mq_status_string", "mq_last_hip_error", "mq_version", "mq_packed_bytes",
    "mq_quantize", "mq_pack", "mq_gemv", "mq_gemv_grouped", "mq_gemv_mixed",
    "mq_gemm_workspace_bytes",
    "mq_gemm", "mq_gemm_noalloc", "mq_mixnmatch_workspace_bytes",
    "mq_mixnmatch_workspace_offsets", "mq_mixnmatch_forward", "mq_mixnmatch_forward_inplace",
    "mq_overflow_rows", "mq_overflow_cols", "mq_overflow_apply", "mq_overflow_apply_grouped",
    "mq_bitplanes_bytes", "mq_pack_bitplanes", "mq_gemv_bitplanes",
    "mq_mlp_workspace_bytes", "mq_mlp_decode",
)


class MQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mq_status_string(status).decode()
        if status == 8:
            msg += f" (hipError {lib().mq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


class GemvProblem(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
                ("zero", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("group", ctypes.c_int64)]


class OverflowProblem(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("group", ctypes.c_int64)]


class Linear(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
                ("zero", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("group", ctypes.c_int64)]


LAYER_LINEARS = ("q", "k", "v", "o", "up", "gate", "down")


class Layer(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int)] + [(n, Linear) for n in LAYER_LINEARS]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libmq.so (built in-tree by nested_int_matmul_amd/build.py).  Raises
    if it is missing: there is no fallback implementation."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m nested_int_matmul_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.mq_status_string.restype = ctypes.c_char_p
    L.mq_status_string.argtypes = [i32]
    L.mq_last_hip_error.restype = i32
    L.mq_version.restype = ctypes.c_char_p
    L.mq_packed_bytes.restype = sz
    L.mq_packed_bytes.argtypes = [i64, i64, i32]
    L.mq_quantize.restype = i32
    L.mq_quantize.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    L.mq_pack.restype = i32
    L.mq_pack.argtypes = [vp, i64, i64, i32, vp, vp]
    L.mq_gemv.restype = i32
    L.mq_gemv.argtypes = [vp, i32, vp, vp, i64, i64, i64, vp, i64, vp, vp]
    L.mq_gemv_grouped.restype = i32
    L.mq_gemv_grouped.argtypes = [ctypes.POINTER(GemvProblem), i32, i32, i64, vp]
    L.mq_overflow_rows.restype = i32
    L.mq_overflow_rows.argtypes = [vp, i64, i64, i32, vp, vp]
    L.mq_overflow_cols.restype = i32
    L.mq_overflow_cols.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    L.mq_overflow_apply.restype = i32
    L.mq_overflow_apply.argtypes = [vp, vp, i32, vp, i64, i64, i64, vp, i64, vp, vp]
    L.mq_overflow_apply_grouped.restype = i32
    L.mq_overflow_apply_grouped.argtypes = [ctypes.POINTER(OverflowProblem), i32, i32, i64, vp]
    L.mq_bitplanes_bytes.restype = sz
    L.mq_bitplanes_bytes.argtypes = [i64, i64]
    L.mq_pack_bitplanes.restype = i32
    L.mq_pack_bitplanes.argtypes = [vp, i64, i64, vp, vp]
    L.mq_gemv_bitplanes.restype = i32
    L.mq_gemv_bitplanes.argtypes = [vp, i32, i32, vp, vp, i64, i64, i64, vp, i64, vp, vp]
    L.mq_mlp_workspace_bytes.restype = sz
    L.mq_mlp_workspace_bytes.argtypes = [i64, i64]
    L.mq_mlp_decode.restype = i32
    L.mq_mlp_decode.argtypes = [ctypes.POINTER(Linear), ctypes.POINTER(Linear),
                                ctypes.POINTER(Linear), i32, i32, vp, i64, vp, vp, sz, vp]
    L.mq_gemv_mixed.restype = i32
    L.mq_gemv_mixed.argtypes = [ctypes.POINTER(GemvProblem), ctypes.POINTER(ctypes.c_int), i32,
                                i64, vp]
    L.mq_gemm_workspace_bytes.restype = sz
    L.mq_gemm_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.mq_gemm.restype = i32
    L.mq_gemm.argtypes = [vp, i32, vp, vp, i64, i64, i64, vp, i64, vp, vp, sz, vp]
    L.mq_gemm_noalloc.restype = i32
    L.mq_gemm_noalloc.argtypes = [vp, i32, vp, vp, i64, i64, i64, vp, i64, vp, vp]
    L.mq_mixnmatch_workspace_bytes.restype = sz
    L.mq_mixnmatch_workspace_bytes.argtypes = [ctypes.POINTER(Layer), i32, i64]
    L.mq_mixnmatch_workspace_offsets.restype = i32
    L.mq_mixnmatch_workspace_offsets.argtypes = [ctypes.POINTER(Layer), i32, i64,
                                                 ctypes.POINTER(sz)]
    L.mq_mixnmatch_forward.restype = i32
    L.mq_mixnmatch_forward.argtypes = [ctypes.POINTER(Layer), i32, vp, i64, vp, vp, sz, vp]
    L.mq_mixnmatch_forward_inplace.restype = i32
    L.mq_mixnmatch_forward_inplace.argtypes = [ctypes.POINTER(Layer), i32, vp, i64, vp, sz, vp]
    _LIB = L
    return L


def _check(status: int, where: str):
    if status != MQ_OK:
        raise MQError(status, where)


def _stream(stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    """Device address of a tensor the library reads or writes: it must live
    on the GPU and be contiguous (the library takes plain row-major buffers)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("mq: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("mq: tensors must be contiguous (row-major)")
    return ctypes.c_void_p(t.data_ptr())


def _bits16(x):
    """bf16 activations as a 16-bit view (bf16 or int16/uint16 tensors)."""
    import torch

    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("activations must be bf16 (or their 16-bit patterns)")


# ------------------------------------------------------------- argument checks
# The library sizes its buffer resources from the integer arguments and trusts
# the pointers; these checks make every tensor agree with those arguments
# (dtype, element count, one device) before a pointer is passed.

def _need(t, name, dtypes, numel=None, shape=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"mq: {name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"mq: {name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"mq: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"mq: {name} has {t.numel()} elements, expected {numel}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"mq: tensors on different devices: {sorted(map(str, devs))}")


def _check_weights(packed, alpha, zero, N, K, group, r, planes=False):
    """Sizes of a plane and its scales against N, K, group and r.  A group
    or r the library does not serve is left for the library to refuse
    (MQ_ERR_GROUP / MQ_ERR_PRECISION, before it reads any buffer)."""
    import torch

    nb = N * K if planes else packed_bytes(N, K, r)
    _need(packed, "packed" if not planes else "planes", (torch.uint8,),
          numel=nb if nb > 0 else None)
    g = (K // group) if group in (K, 128) and group > 0 and K % group == 0 else None
    _need(alpha, "alpha", (torch.float32,), numel=None if g is None else N * g)
    _need(zero, "zero", (torch.float32,), numel=None if g is None else N * g)


def _check_xy(x, y, M, N, K):
    import torch

    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), shape=(M, K))
    if y is not None:
        _need(y, "out", (torch.float32,), numel=M * N)


def _check_linear(p, name="linear", r=None):
    """A linear's dict {"packed", "alpha", "zero", "N", "K", "group"} at r."""
    _check_weights(p["packed"], p["alpha"], p["zero"], p["N"], p["K"], p["group"], r)


# ----------------------------------------------------------------- entry points

def packed_bytes(N: int, K: int, r: int) -> int:
    return int(lib().mq_packed_bytes(N, K, r))


def quantize(w, group: int, stream=None):
    """Eq. 1 min-max quantization on the GPU: fp32 [N, K] -> (codes uint8
    [N, K], alpha fp32 [N, K/group], zero fp32 [N, K/group])."""
    import torch

    _need(w, "w", (torch.float32,))
    if w.dim() != 2:
        raise ValueError("mq: w must be [N, K]")
    n, k = w.shape
    g = k // group if group else 0
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    alpha = torch.empty((n, max(g, 1)), dtype=torch.float32, device=w.device)
    zero = torch.empty_like(alpha)
    _check(lib().mq_quantize(_ptr(w), n, k, group, _ptr(codes), _ptr(alpha), _ptr(zero),
                             _stream(stream)), "mq_quantize")
    return codes, alpha, zero


def pack(codes, r: int, out=None, stream=None):
    """Slice uint8 codes [N, K] to r bits and pack: uint8 [N, K*r/8] (for
    r = 3 and 6 the two sub-planes are back to back in that byte array)."""
    import torch

    _need(codes, "codes", (torch.uint8,))
    if codes.dim() != 2:
        raise ValueError("mq: codes must be [N, K]")
    n, k = codes.shape
    if out is None:
        out = torch.empty((n, k * r // 8), dtype=torch.uint8, device=codes.device)
    _need(out, "out", (torch.uint8,), numel=packed_bytes(n, k, r))
    _same_device(codes, out)
    _check(lib().mq_pack(_ptr(codes), n, k, r, _ptr(out), _stream(stream)), "mq_pack")
    return out


def gemv(packed, r: int, alpha, zero, group: int, N: int, K: int, x, out=None, stream=None):
    """y = x @ dequant(S(q, r))^T for M <= 8 rows of bf16 x: fp32 [M, N]."""
    import torch

    x = _bits16(x)
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _check_weights(packed, alpha, zero, N, K, group, r)
    _check_xy(x, out, m, N, K)
    _same_device(packed, alpha, zero, x, out)
    _check(lib().mq_gemv(_ptr(packed), r, _ptr(alpha), _ptr(zero), group, N, K, _ptr(x), m,
                         _ptr(out), _stream(stream)), "mq_gemv")
    return out


def _problem_array(problems, rs):
    arr = (GemvProblem * len(problems))()
    for i, p in enumerate(problems):
        x = _bits16(p["x"])
        _check_weights(p["packed"], p["alpha"], p["zero"], p["N"], p["K"], p["group"], rs[i])
        _check_xy(x, p["y"], x.shape[0], p["N"], p["K"])
        _same_device(p["packed"], p["alpha"], p["zero"], x, p["y"])
        arr[i] = GemvProblem(_ptr(p["packed"]), _ptr(p["alpha"]), _ptr(p["zero"]),
                             _ptr(_bits16(p["x"])), _ptr(p["y"]), p["N"], p["K"], p["group"])
    return arr


def gemv_grouped(problems, r, M: int, stream=None):
    """problems: list of dicts with packed, alpha, zero, x, y (tensors), N, K, group.
    r: one precision for all (mq_gemv_grouped) or a list, one per problem
    (mq_gemv_mixed)."""
    GemvGroupedPlan(problems, r, M, stream)()


class GemvGroupedPlan:
    """A prepared mq_gemv_grouped / mq_gemv_mixed call: the problem array is
    marshalled once, each call is a single C call (for launch-rate-bound
    decode loops).  r is an int (same for all) or a list (one per problem).
    The caller keeps every tensor alive while the plan is in use."""

    def __init__(self, problems, r, M: int, stream=None):
        rs = list(r) if isinstance(r, (list, tuple)) else [r] * len(problems)
        if len(rs) != len(problems):
            raise ValueError("one r per problem")
        for p in problems:
            if p["x"].shape[0] != M:
                raise ValueError(f"mq: x has {p['x'].shape[0]} rows, expected M = {M}")
        self.arr = _problem_array(problems, rs)
        self.count, self.M = len(problems), M
        self.stream = _stream(stream)
        if isinstance(r, (list, tuple)):
            if len(r) != len(problems):
                raise ValueError("one r per problem")
            self.rs = (ctypes.c_int * len(r))(*r)
            self.fn, self.name = lib().mq_gemv_mixed, "mq_gemv_mixed"
            self.args = (self.arr, self.rs, self.count, self.M, self.stream)
        else:
            self.fn, self.name = lib().mq_gemv_grouped, "mq_gemv_grouped"
            self.args = (self.arr, self.count, int(r), self.M, self.stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != MQ_OK:
            raise MQError(st, self.name)


def overflow_lists(codes, r: int, stream=None):
    """Extra-Precision lists of a code matrix at precision r: (row_ptr int32
    [N + 1], col_idx [nnz] of 16-bit column indices, stored as int16 (read
    them as uint16)) on the device.  Synchronizes once to size col_idx (a
    setup step)."""
    import torch

    _need(codes, "codes", (torch.uint8,))
    n, k = codes.shape
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=codes.device)
    _check(lib().mq_overflow_rows(_ptr(codes), n, k, r, _ptr(row_ptr), _stream(stream)),
           "mq_overflow_rows")
    # the count was written on `stream`: wait for it there before reading it
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    nnz = int(row_ptr[n].item())
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int16, device=codes.device)
    _check(lib().mq_overflow_cols(_ptr(codes), n, k, r, _ptr(row_ptr), _ptr(col_idx),
                                  _stream(stream)), "mq_overflow_cols")
    return row_ptr, col_idx[:nnz]


def overflow_apply(row_ptr, col_idx, r: int, alpha, group: int, N: int, K: int, x, y,
                   stream=None):
    """y += the extra-precision correction (after a product at the same r)."""
    import torch

    x = _bits16(x)
    g = (K // group) if group in (K, 128) and group > 0 and K % group == 0 else None
    _need(row_ptr, "row_ptr", (torch.int32,), numel=N + 1)
    _need(col_idx, "col_idx", (torch.int16, torch.uint16))
    _need(alpha, "alpha", (torch.float32,), numel=None if g is None else N * g)
    _check_xy(x, y, x.shape[0], N, K)
    _same_device(row_ptr, col_idx, alpha, x, y)
    ci = col_idx if col_idx.numel() else row_ptr  # any valid pointer when the list is empty
    _check(lib().mq_overflow_apply(_ptr(row_ptr), _ptr(ci), r, _ptr(alpha), group, N, K, _ptr(x),
                                   x.shape[0], _ptr(y), _stream(stream)), "mq_overflow_apply")
    return y


def overflow_apply_grouped(problems, r: int, M: int, stream=None):
    """The sparse addition for several matrices in one launch.  problems: dicts
    with row_ptr, col_idx, alpha, x, y (tensors), N, K, group."""
    import torch

    arr = (OverflowProblem * len(problems))()
    for i, p in enumerate(problems):
        x = _bits16(p["x"])
        N, K, group = p["N"], p["K"], p["group"]
        g = (K // group) if group in (K, 128) and group > 0 and K % group == 0 else None
        _need(p["row_ptr"], "row_ptr", (torch.int32,), numel=N + 1)
        _need(p["col_idx"], "col_idx", (torch.int16, torch.uint16))
        _need(p["alpha"], "alpha", (torch.float32,), numel=None if g is None else N * g)
        _check_xy(x, p["y"], M, N, K)
        _same_device(p["row_ptr"], p["col_idx"], p["alpha"], x, p["y"])
        ci = p["col_idx"] if p["col_idx"].numel() else p["row_ptr"]
        arr[i] = OverflowProblem(_ptr(p["row_ptr"]), _ptr(ci), _ptr(p["alpha"]), _ptr(x),
                                 _ptr(p["y"]), N, K, group)
    _check(lib().mq_overflow_apply_grouped(arr, len(problems), r, M, _stream(stream)),
           "mq_overflow_apply_grouped")


def bitplanes_bytes(N: int, K: int) -> int:
    return int(lib().mq_bitplanes_bytes(N, K))


def pack_bitplanes(codes, out=None, stream=None):
    """The eight bit-planes of uint8 codes [N, K]: uint8 [8, N, K/8]."""
    import torch

    _need(codes, "codes", (torch.uint8,))
    n, k = codes.shape
    if out is None:
        out = torch.empty((8, n, k // 8), dtype=torch.uint8, device=codes.device)
    _need(out, "out", (torch.uint8,), numel=n * k)
    _same_device(codes, out)
    _check(lib().mq_pack_bitplanes(_ptr(codes), n, k, _ptr(out), _stream(stream)),
           "mq_pack_bitplanes")
    return out


def gemv_bitplanes(planes, r: int, alpha, zero, group: int, N: int, K: int, x, extra=False,
                   out=None, stream=None):
    """y = x @ dequant(S(q, r))^T read from bit-planes (unclamped slice with
    extra=True): fp32 [M, N]."""
    import torch

    x = _bits16(x)
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _check_weights(planes, alpha, zero, N, K, group, r, planes=True)
    _check_xy(x, out, m, N, K)
    _same_device(planes, alpha, zero, x, out)
    _check(lib().mq_gemv_bitplanes(_ptr(planes), r, int(bool(extra)), _ptr(alpha), _ptr(zero),
                                   group, N, K, _ptr(x), m, _ptr(out), _stream(stream)),
           "mq_gemv_bitplanes")
    return out


def gemm_workspace_bytes(M: int, N: int, K: int, group: int) -> int:
    return int(lib().mq_gemm_workspace_bytes(M, N, K, group))


def gemm(packed, r: int, alpha, zero, group: int, N: int, K: int, x, out=None, workspace=None,
         stream=None):
    """y = x @ dequant(S(q, r))^T for any M: fp32 [M, N]."""
    import torch

    x = _bits16(x)
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _check_weights(packed, alpha, zero, N, K, group, r)
    _check_xy(x, out, m, N, K)
    _same_device(packed, alpha, zero, x, out, workspace)
    need = gemm_workspace_bytes(m, N, K, group)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mq_gemm(_ptr(packed), r, _ptr(alpha), _ptr(zero), group, N, K, _ptr(x), m,
                         _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)), "mq_gemm")
    return out


GEMM_NOALLOC_MAX_BYTES = 64 << 20  # MQ_GEMM_NOALLOC_MAX_BYTES of mq.h


def gemm_noalloc(packed, r: int, alpha, zero, group: int, N: int, K: int, x, out, stream=None):
    """mq_gemm_noalloc: gemm() with the K-slice partials in the library's
    per-device scratch array (no workspace, nothing allocated; `out` is
    required).  Overlapping calls on one device race on that array."""
    x = _bits16(x)
    m = x.shape[0]
    _check_weights(packed, alpha, zero, N, K, group, r)
    _check_xy(x, out, m, N, K)
    _same_device(packed, alpha, zero, x, out)
    _check(lib().mq_gemm_noalloc(_ptr(packed), r, _ptr(alpha), _ptr(zero), group, N, K, _ptr(x),
                                 m, _ptr(out), _stream(stream)), "mq_gemm_noalloc")
    return out


def make_layers(layers):
    """layers: list of dicts {"r": r, name: {"packed", "alpha", "zero", "N", "K", "group"}}
    -> ctypes array of Layer (keeps no references: the caller keeps the tensors)."""
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        kw = {"r": L["r"]}
        for n in LAYER_LINEARS:
            p = L[n]
            _check_linear(p, n, L["r"])
            kw[n] = Linear(_ptr(p["packed"]), _ptr(p["alpha"]), _ptr(p["zero"]),
                           p["N"], p["K"], p["group"])
        arr[i] = Layer(**kw)
    return arr


MLP_ACTS = {"identity": 0, "silu": 1, "gelu_tanh": 2}


def make_linear(p):
    """{"packed", "alpha", "zero", "N", "K", "group"} -> a ctypes Linear."""
    return Linear(_ptr(p["packed"]), _ptr(p["alpha"]), _ptr(p["zero"]),
                  p["N"], p["K"], p["group"])


def mlp_workspace_bytes(M: int, F: int) -> int:
    return int(lib().mq_mlp_workspace_bytes(M, F))


def mlp_decode(up, gate, down, r: int, x, act="identity", workspace=None, out=None,
               stream=None):
    """y = W_down bf16(W_up x * act(W_gate x)) for M <= 8 rows of bf16 x.
    up, gate, down: dicts as for make_linear.  Returns (y fp32 [M, H],
    workspace), the workspace holding u, g (fp32) and the bf16 product."""
    import torch

    x = _bits16(x)
    m = x.shape[0]
    F, H = up["N"], up["K"]
    for p, nm in ((up, "up"), (gate, "gate"), (down, "down")):
        _check_linear(p, nm, r)
    _check_xy(x, out, m, H, H)
    need = mlp_workspace_bytes(m, F)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((m, H), dtype=torch.float32, device=x.device)
    lu, lg, ld = make_linear(up), make_linear(gate), make_linear(down)
    _check(lib().mq_mlp_decode(ctypes.byref(lu), ctypes.byref(lg), ctypes.byref(ld), r,
                               MLP_ACTS[act], _ptr(x), m, _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "mq_mlp_decode")
    return out, workspace


def mixnmatch_workspace_bytes(layer_arr, M: int) -> int:
    return int(lib().mq_mixnmatch_workspace_bytes(layer_arr, len(layer_arr), M))


def mixnmatch_workspace_offsets(layer_arr, M: int):
    off = (ctypes.c_size_t * 10)()
    _check(lib().mq_mixnmatch_workspace_offsets(layer_arr, len(layer_arr), M, off),
           "mq_mixnmatch_workspace_offsets")
    return list(off)


def _stack_h(layer_arr):
    return int(layer_arr[0].q.N) if len(layer_arr) else 0


def mixnmatch_forward(layer_arr, x, workspace, out=None, stream=None):
    """Run the stack on bf16 x [M, H]: returns the final fp32 residual stream
    h [M, H] (written to `out` when given)."""
    import torch

    x = _bits16(x)
    m, H = x.shape
    if H != _stack_h(layer_arr):
        raise ValueError(f"mq: x has {H} columns, the stack's width is {_stack_h(layer_arr)}")
    if out is None:
        out = torch.empty((m, H), dtype=torch.float32, device=x.device)
    _check_xy(x, out, m, H, H)
    _need(workspace, "workspace", (torch.uint8,))
    _same_device(x, out, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().mq_mixnmatch_forward(layer_arr, len(layer_arr), _ptr(x), m, _ptr(out),
                                      _ptr(workspace), ws_bytes, _stream(stream)),
           "mq_mixnmatch_forward")
    return out


def mixnmatch_forward_inplace(layer_arr, h, workspace, stream=None):
    """Run the stack in place on an fp32 residual stream h [M, H] (to continue
    a stack over several calls)."""
    import torch

    m, H = h.shape
    if H != _stack_h(layer_arr):
        raise ValueError(f"mq: h has {H} columns, the stack's width is {_stack_h(layer_arr)}")
    _need(h, "h", (torch.float32,))
    _need(workspace, "workspace", (torch.uint8,))
    _same_device(h, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().mq_mixnmatch_forward_inplace(layer_arr, len(layer_arr), _ptr(h), m,
                                              _ptr(workspace), ws_bytes, _stream(stream)),
           "mq_mixnmatch_forward_inplace")
    return h
