"""ctypes binding of libgdn (include/gdn.h).

Argument marshalling only: shapes, dtypes and contiguity are checked, output
and workspace buffers are allocated with torch (device memory plumbing),
and the raw device pointers plus the current HIP stream are handed to the C
ABI.  Every step of the computation runs in the library's HIP kernels; there
is no fallback path.  If libgdn.so is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch  # imported before the library so that it binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(5)
GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
_IO_DTYPES = {torch.float32: GDN_DTYPE_F32, torch.bfloat16: GDN_DTYPE_BF16}


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libgdn.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built (%s); run `python -m gated_deltanet_scan_amd.build`"
                               % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        SP = ctypes.POINTER(Shape)
        lib.gdn_prefill_workspace_bytes.argtypes = [SP, i64, i32]
        lib.gdn_prefill_workspace_bytes.restype = sz
        lib.gdn_prefill_workspace_bytes_for.argtypes = [SP, vp, i32]
        lib.gdn_prefill_workspace_bytes_for.restype = sz
        lib.gdn_prefill_chunked.argtypes = [SP, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, sz, vp]
        lib.gdn_prefill_chunked.restype = ctypes.c_int
        lib.gdn_prefill_chunked_noalloc.argtypes = [SP, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, vp]
        lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int
        lib.gdn_prefill_chunked_gated_rmsnorm.argtypes = [SP, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, vp,
                                                          ctypes.c_float, vp, vp, sz, vp]
        lib.gdn_prefill_chunked_gated_rmsnorm.restype = ctypes.c_int
        lib.gdn_decode_step.argtypes = [SP, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        lib.gdn_decode_step.restype = ctypes.c_int
        lib.gdn_state_snapshot.argtypes = [SP, vp, vp, i32, vp, vp, i32, i32, vp]
        lib.gdn_state_snapshot.restype = ctypes.c_int
        lib.gdn_conv_state_snapshot.argtypes = [i64, i32, vp, vp, i32, vp, vp, i32, i32, vp]
        lib.gdn_conv_state_snapshot.restype = ctypes.c_int
        lib.gdn_gated_rmsnorm.argtypes = [SP, vp, vp, vp, vp, i64, ctypes.c_float, vp]
        lib.gdn_gated_rmsnorm.restype = ctypes.c_int
        lib.gdn_conv1d_qkv.argtypes = [SP, vp, vp, i32, vp, i32, i64, vp, vp, i32, i32, ctypes.c_float, vp, vp, vp,
                                       vp]
        lib.gdn_conv1d_qkv.restype = ctypes.c_int
        lib.gdn_status_string.argtypes = [ctypes.c_int]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_last_error.argtypes = []
        lib.gdn_last_error.restype = ctypes.c_char_p
        lib.gdn_profile_enable.argtypes = [i32]
        lib.gdn_profile_enable.restype = ctypes.c_int
        lib.gdn_profile_collect.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
        lib.gdn_profile_collect.restype = ctypes.c_int
        lib.gdn_version.argtypes = []
        lib.gdn_version.restype = i32
        _lib = lib
        return lib


def header_functions():
    """Names of the functions include/gdn.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def _status_name(status: int) -> str:
    names = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_WORKSPACE",
             4: "GDN_ERR_HIP"}
    return names.get(status, "GDN_ERR_%d" % status)


def _check(lib, status: int):
    if status != GDN_OK:
        raise GdnError(status, lib.gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def make_shape(hqk, hv, dk, dv, chunk, io_dtype, scale) -> Shape:
    return Shape(int(hqk), int(hv), int(dk), int(dv), int(chunk), int(io_dtype), float(scale))


def workspace_bytes(shape: Shape, total_tokens: int, num_seqs: int) -> int:
    return int(load_library().gdn_prefill_workspace_bytes(ctypes.byref(shape), int(total_tokens),
                                                          int(num_seqs)))


def workspace_bytes_for(shape: Shape, cu_seqlens_host) -> int:
    """Workspace bytes the prefill uses for a batch whose offsets are known on the host."""
    arr = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    if arr.device.type != "cpu" or arr.dim() != 1 or arr.shape[0] < 1:
        raise ValueError("cu_seqlens_host must be a 1-D host sequence of num_seqs + 1 offsets")
    return int(load_library().gdn_prefill_workspace_bytes_for(ctypes.byref(shape), ctypes.c_void_p(arr.data_ptr()),
                                                              int(arr.shape[0] - 1)))


def _prefill_call(q, k, v, g, beta, cu_seqlens, initial_state, scale, chunk, final_state, out, workspace):
    """Validate and marshal the arguments of gdn_prefill_chunked; returns (lib, args, keep, out, final)."""
    lib = load_library()
    _need(q, "q", ndim=3)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    io = q.dtype
    if io not in _IO_DTYPES:
        raise TypeError("io dtype must be float32 or bfloat16")
    _need(k, "k", io, dev, 3)
    _need(v, "v", io, dev, 3)
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if tuple(k.shape) != (T, hqk, dk) or v.shape[0] != T:
        raise ValueError("q, k, v shapes disagree: %s %s %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    if tuple(g.shape) != (T, hv) or tuple(beta.shape) != (T, hv):
        raise ValueError("g and beta must be [T, HV]")
    cu_host = None
    if cu_seqlens is None:
        cu_host = torch.tensor([0, T], dtype=torch.int32)
        cu_dev = cu_host.to(dev)
    elif isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        cu_dev = cu_seqlens
    else:
        cu_host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous()
        cu_dev = cu_host.to(dev)
    n = cu_dev.shape[0] - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
    if final_state is None:
        final_state = torch.empty(n, hv, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev, 4)
    for st, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if st is not None and tuple(st.shape) != (n, hv, dk, dv):
            raise ValueError("%s must be [N, HV, dk, dv] = %s" % (name, (n, hv, dk, dv)))
    if out is None:
        out = torch.empty(T, hv, dv, dtype=io, device=dev)
    _need(out, "out", io, dev, 3)
    if scale is None:
        scale = dk ** -0.5
    shape = make_shape(hqk, hv, dk, dv, chunk, _IO_DTYPES[io], scale)
    need = workspace_bytes(shape, T, n)
    if need == 0 and n > 0:
        raise GdnError(GDN_ERR_UNSUPPORTED, "no prefill kernel for dk=%d dv=%d chunk=%d %s" % (dk, dv, chunk, io))
    if workspace is None:
        if cu_host is not None:   # the plan for these lengths may need less (segments)
            need = workspace_bytes_for(shape, cu_host) or need
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)
    host_arr = None if cu_host is None else cu_host.numpy()
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_dev), n, T,
            None if host_arr is None else host_arr.ctypes.data_as(ctypes.c_void_p),
            _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace), workspace.numel())
    keep = (shape, cu_dev, host_arr, workspace, q, k, v, g, beta, initial_state)
    return lib, args, keep, dev, out, final_state


def prefill_chunked(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, scale=None, chunk=64,
                    final_state=None, out=None, workspace=None):
    """Chunked prefill over a packed batch (gdn_prefill_chunked).

    q, k [T, HQK, dk] and v [T, HV, dv] in fp32 or bf16 on one GPU; g, beta [T, HV] fp32;
    cu_seqlens [N+1] int32 (a CPU tensor or list is copied to the device and also passed
    as the host copy, which the library validates; None means one sequence);
    initial_state [N, HV, dk, dv] fp32 or None (zeros).  final_state may be the same
    tensor as initial_state (in-place prefix reuse).  Returns (o, final_state).
    """
    lib, args, keep, dev, out, final_state = _prefill_call(q, k, v, g, beta, cu_seqlens, initial_state, scale,
                                                           chunk, final_state, out, workspace)
    _check(lib, lib.gdn_prefill_chunked(*args, _stream(dev)))
    return out, final_state


def prefill_chunked_noalloc(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, scale=None, chunk=64,
                            final_state=None, out=None):
    """gdn_prefill_chunked_noalloc: the chunked prefill with the library's own device scratch in
    place of a workspace (the library allocates nothing).  Arguments and result as for
    prefill_chunked; a batch too large for the scratch raises GdnError (GDN_ERR_WORKSPACE).
    Calls that overlap in time on one device race on the scratch."""
    lib, args, keep, dev, out, final_state = _prefill_call(q, k, v, g, beta, cu_seqlens, initial_state, scale,
                                                           chunk, final_state, out, torch.empty(0, dtype=torch.uint8,
                                                                                                device=q.device))
    # (shape, q, k, v, g, beta, cu, N, T, cu_host, s0, final, o) without (workspace, bytes)
    _check(lib, lib.gdn_prefill_chunked_noalloc(*args[:13], _stream(dev)))
    return out, final_state


def _prefill_norm_call(q, k, v, g, beta, z, norm_weight, cu_seqlens, initial_state, eps, scale, chunk, final_state,
                       out, workspace):
    """gdn_prefill_chunked's arguments with the gate, the norm weight and eps added."""
    lib, args, keep, dev, out, final_state = _prefill_call(q, k, v, g, beta, cu_seqlens, initial_state, scale,
                                                           chunk, final_state, out, workspace)
    _need(z, "z", q.dtype, dev, 3)
    if tuple(z.shape) != tuple(out.shape):
        raise ValueError("z must be shaped like the output, %s" % (tuple(out.shape),))
    _need(norm_weight, "norm_weight", torch.float32, dev, 1)
    if norm_weight.shape[0] != out.shape[2]:
        raise ValueError("norm_weight must be [dv]")
    # (shape, q, k, v, g, beta, cu, N, T, cu_host, s0, final) + (z, weight, eps) + (y, workspace, bytes)
    args = args[:12] + (_ptr(z), _ptr(norm_weight), ctypes.c_float(float(eps))) + args[12:]
    return lib, args, keep + (z, norm_weight), dev, out, final_state


def prefill_chunked_gated_rmsnorm(q, k, v, g, beta, z, norm_weight, cu_seqlens=None, initial_state=None, *,
                                  eps=1e-6, scale=None, chunk=64, final_state=None, out=None, workspace=None):
    """Chunked prefill followed by the gated RMSNorm of its output rows
    (gdn_prefill_chunked_gated_rmsnorm): y = o / sqrt(mean(o^2) + eps) * norm_weight * silu(z)
    per (token, value head) row, in place on y right after the scans.  z [T, HV, dv] in the
    io dtype, norm_weight [dv] fp32; the other arguments as for prefill_chunked.  Returns
    (y, final_state)."""
    lib, args, keep, dev, out, final_state = _prefill_norm_call(q, k, v, g, beta, z, norm_weight, cu_seqlens,
                                                                initial_state, eps, scale, chunk, final_state,
                                                                out, workspace)
    _check(lib, lib.gdn_prefill_chunked_gated_rmsnorm(*args, _stream(dev)))
    return out, final_state


class PreparedCall:
    """A library call whose arguments were validated and marshalled once; calling it enqueues
    the kernels again on the current stream with the same buffers (for timing loops)."""

    def __init__(self, fn, lib, args, keep, dev, result):
        self._fn, self._lib, self._args, self._keep, self._dev = fn, lib, args, keep, dev
        self.result = result
        self._stream = torch.cuda.current_stream(dev)
        self._stream_arg = ctypes.c_void_p(self._stream.cuda_stream)

    def __call__(self):
        status = self._fn(*self._args, self._stream_arg)
        if status != GDN_OK:
            _check(self._lib, status)
        return self.result


def prepare_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, scale=None, chunk=64,
                    final_state=None, out=None, workspace=None) -> PreparedCall:
    lib, args, keep, dev, out, final_state = _prefill_call(q, k, v, g, beta, cu_seqlens, initial_state, scale,
                                                           chunk, final_state, out, workspace)
    return PreparedCall(lib.gdn_prefill_chunked, lib, args, keep, dev, (out, final_state))


def prepare_prefill_gated_rmsnorm(q, k, v, g, beta, z, norm_weight, cu_seqlens=None, initial_state=None, *,
                                  eps=1e-6, scale=None, chunk=64, final_state=None, out=None,
                                  workspace=None) -> PreparedCall:
    lib, args, keep, dev, out, final_state = _prefill_norm_call(q, k, v, g, beta, z, norm_weight, cu_seqlens,
                                                                initial_state, eps, scale, chunk, final_state,
                                                                out, workspace)
    return PreparedCall(lib.gdn_prefill_chunked_gated_rmsnorm, lib, args, keep, dev, (out, final_state))


def _decode_call(q, k, v, g, beta, state, scale, out):
    lib = load_library()
    _need(q, "q", ndim=3)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    io = q.dtype
    if io not in _IO_DTYPES:
        raise TypeError("io dtype must be float32 or bfloat16")
    _need(k, "k", io, dev, 3)
    _need(v, "v", io, dev, 3)
    n, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if tuple(k.shape) != (n, hqk, dk) or v.shape[0] != n:
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    if tuple(g.shape) != (n, hv) or tuple(beta.shape) != (n, hv):
        raise ValueError("g and beta must be [N, HV]")
    _need(state, "state", torch.float32, dev, 4)
    if tuple(state.shape) != (n, hv, dk, dv):
        raise ValueError("state must be [N, HV, dk, dv]")
    if out is None:
        out = torch.empty(n, hv, dv, dtype=io, device=dev)
    _need(out, "out", io, dev, 3)
    if scale is None:
        scale = dk ** -0.5
    shape = make_shape(hqk, hv, dk, dv, 64, _IO_DTYPES[io], scale)
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out), n)
    keep = (shape, q, k, v, g, beta, state)
    return lib, args, keep, dev, out


def decode_step(q, k, v, g, beta, state, *, scale=None, out=None):
    """One token per sequence, state updated in place (gdn_decode_step).

    q, k [N, HQK, dk]; v [N, HV, dv] (fp32 or bf16); g, beta [N, HV] fp32;
    state [N, HV, dk, dv] fp32.  Returns o [N, HV, dv].
    """
    lib, args, keep, dev, out = _decode_call(q, k, v, g, beta, state, scale, out)
    _check(lib, lib.gdn_decode_step(*args, _stream(dev)))
    return out


def prepare_decode(q, k, v, g, beta, state, *, scale=None, out=None) -> PreparedCall:
    lib, args, keep, dev, out = _decode_call(q, k, v, g, beta, state, scale, out)
    return PreparedCall(lib.gdn_decode_step, lib, args, keep, dev, out)


def _snapshot_rows(src, dst, src_rows, dst_rows, num_rows):
    _need(src, "src", torch.float32, None, None)
    dev = src.device
    _need(dst, "dst", torch.float32, dev, None)
    if tuple(src.shape[1:]) != tuple(dst.shape[1:]):
        raise ValueError("src and dst must have the same per-sequence shape")
    for t, name in ((src_rows, "src_rows"), (dst_rows, "dst_rows")):
        if t is not None:
            _need(t, name, torch.int32, dev, 1)
    if num_rows is None:
        if src_rows is not None:
            num_rows = src_rows.numel()
        elif dst_rows is not None:
            num_rows = dst_rows.numel()
        else:
            num_rows = src.shape[0]
    for t, name in ((src_rows, "src_rows"), (dst_rows, "dst_rows")):
        if t is not None and t.numel() < num_rows:
            raise ValueError("%s has fewer than num_rows entries" % name)
    return dev, int(num_rows)


def conv_state_snapshot(src, dst, src_rows=None, dst_rows=None, num_rows=None):
    """dst[dst_rows[i]] = src[src_rows[i]] over whole per-sequence conv states
    (gdn_conv_state_snapshot).

    src, dst [capacity, C, width - 1] fp32; the index tensors are int32 on the same GPU
    (None = identity).  Restore is the same call with src and dst swapped.
    """
    lib = load_library()
    if src.dim() != 3:
        raise ValueError("conv states are [capacity, C, width - 1]")
    dev, num_rows = _snapshot_rows(src, dst, src_rows, dst_rows, num_rows)
    channels, taps = src.shape[1], src.shape[2]
    status = lib.gdn_conv_state_snapshot(int(channels), int(taps) + 1, _ptr(src), _ptr(src_rows), src.shape[0],
                                         _ptr(dst), _ptr(dst_rows), dst.shape[0], num_rows, _stream(dev))
    _check(lib, status)
    return dst


def state_snapshot(src, dst, src_rows=None, dst_rows=None, num_rows=None):
    """dst[dst_rows[i]] = src[src_rows[i]] over whole per-sequence states (gdn_state_snapshot).

    src, dst [capacity, HV, dk, dv] fp32; the index tensors are int32 on the same GPU (None =
    identity).  Restore is the same call with src and dst swapped.
    """
    lib = load_library()
    if src.dim() != 4:
        raise ValueError("states are [capacity, HV, dk, dv]")
    dev, num_rows = _snapshot_rows(src, dst, src_rows, dst_rows, num_rows)
    hv, dk, dv = src.shape[1:]
    shape = make_shape(1, hv, dk, dv, 64, GDN_DTYPE_F32, 1.0)
    status = lib.gdn_state_snapshot(ctypes.byref(shape), _ptr(src), _ptr(src_rows), src.shape[0], _ptr(dst),
                                    _ptr(dst_rows), dst.shape[0], int(num_rows), _stream(dev))
    _check(lib, status)
    return dst


def _norm_call(o, z, weight, eps, out):
    lib = load_library()
    _need(o, "o", ndim=3)
    dev = o.device
    if dev.type != "cuda":
        raise ValueError("o must be on a GPU")
    io = o.dtype
    if io not in _IO_DTYPES:
        raise TypeError("io dtype must be float32 or bfloat16")
    _need(z, "z", io, dev, 3)
    if tuple(z.shape) != tuple(o.shape):
        raise ValueError("z must be shaped like o")
    t, hv, dv = o.shape
    _need(weight, "weight", torch.float32, dev, 1)
    if weight.shape[0] != dv:
        raise ValueError("weight must be [dv]")
    if out is None:
        out = torch.empty_like(o)
    _need(out, "out", io, dev, 3)
    if tuple(out.shape) != tuple(o.shape):
        raise ValueError("out must be shaped like o")
    shape = make_shape(1, hv, dv, dv, 64, _IO_DTYPES[io], 1.0)
    args = (ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(weight), _ptr(out), t, float(eps))
    keep = (shape, o, z, weight)
    return lib, args, keep, dev, out


def gated_rmsnorm(o, z, weight, *, eps=1e-6, out=None):
    """y = o / sqrt(mean(o^2) + eps) * weight * silu(z) per (token, head) row (gdn_gated_rmsnorm).

    o, z [T, HV, dv] (fp32 or bf16); weight [dv] fp32.  `out` may be o or z (in place).
    Returns y [T, HV, dv].
    """
    lib, args, keep, dev, out = _norm_call(o, z, weight, eps, out)
    _check(lib, lib.gdn_gated_rmsnorm(*args, _stream(dev)))
    return out


def prepare_gated_rmsnorm(o, z, weight, *, eps=1e-6, out=None) -> PreparedCall:
    lib, args, keep, dev, out = _norm_call(o, z, weight, eps, out)
    return PreparedCall(lib.gdn_gated_rmsnorm, lib, args, keep, dev, out)


def _conv_call(x, weight, hqk, hv, dk, dv, cu_seqlens, state_in, state_out, silu, l2norm, eps, out):
    lib = load_library()
    _need(x, "x", ndim=2)
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be on a GPU")
    io = x.dtype
    if io not in _IO_DTYPES:
        raise TypeError("io dtype must be float32 or bfloat16")
    T, C = x.shape
    if C != 2 * hqk * dk + hv * dv:
        raise ValueError("x must have 2 * HQK * dk + HV * dv channels")
    _need(weight, "weight", torch.float32, dev, 2)
    if weight.shape[0] != C:
        raise ValueError("weight must be [C, K]")
    K = int(weight.shape[1])
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
    n = cu_seqlens.numel() - 1
    for t, name in ((state_in, "state_in"), (state_out, "state_out")):
        if t is not None:
            _need(t, name, torch.float32, dev, 3)
            if tuple(t.shape) != (n, C, K - 1):
                raise ValueError("%s must be [N, C, K-1]" % name)
    if out is None:
        out = (torch.empty(T, hqk, dk, dtype=io, device=dev), torch.empty(T, hqk, dk, dtype=io, device=dev),
               torch.empty(T, hv, dv, dtype=io, device=dev))
    q, k, v = out
    shape = make_shape(hqk, hv, dk, dv, 64, _IO_DTYPES[io], 1.0)
    args = (ctypes.byref(shape), _ptr(x), _ptr(weight), K, _ptr(cu_seqlens), n, T, _ptr(state_in), _ptr(state_out),
            1 if silu else 0, 1 if l2norm else 0, float(eps), _ptr(q), _ptr(k), _ptr(v))
    keep = (shape, x, weight, cu_seqlens, state_in, state_out)
    return lib, args, keep, dev, out


def conv1d_qkv(x, weight, hqk, hv, dk, dv, cu_seqlens=None, state_in=None, state_out=None, *, silu=False,
               l2norm=True, eps=1e-6, out=None):
    """Depthwise causal conv1d over the packed projections [q heads | k heads | v heads], with
    the conv state, then q and k L2-normalised per head (gdn_conv1d_qkv).

    x [T, 2*HQK*dk + HV*dv] (fp32 or bf16); weight [C, K] fp32; cu_seqlens int32 [N+1] on the GPU
    (None = one sequence); state_in / state_out [N, C, K-1] fp32 or None (state_out may be
    state_in).  Returns (q [T, HQK, dk], k [T, HQK, dk], v [T, HV, dv]).
    """
    lib, args, keep, dev, out = _conv_call(x, weight, hqk, hv, dk, dv, cu_seqlens, state_in, state_out, silu,
                                           l2norm, eps, out)
    _check(lib, lib.gdn_conv1d_qkv(*args, _stream(dev)))
    return out


def prepare_conv1d_qkv(x, weight, hqk, hv, dk, dv, cu_seqlens=None, state_in=None, state_out=None, *, silu=False,
                       l2norm=True, eps=1e-6, out=None) -> PreparedCall:
    lib, args, keep, dev, out = _conv_call(x, weight, hqk, hv, dk, dv, cu_seqlens, state_in, state_out, silu,
                                           l2norm, eps, out)
    return PreparedCall(lib.gdn_conv1d_qkv, lib, args, keep, dev, out)


PROF_CHUNK_TABLE, PROF_PREP, PROF_SCAN, PROF_DECODE, PROF_SNAPSHOT, PROF_NORM, PROF_CONV, PROF_CONV_STATE = range(8)


def profile_enable(on: bool = True):
    """Start (clearing earlier records) or stop per-kernel HIP-event timing in the library."""
    lib = load_library()
    _check(lib, lib.gdn_profile_enable(1 if on else 0))


def profile_collect(kernel: int):
    """(launches, total_ms) of one kernel since profile_enable(True); waits for its events."""
    lib = load_library()
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check(lib, lib.gdn_profile_collect(int(kernel), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def version() -> int:
    return int(load_library().gdn_version())
