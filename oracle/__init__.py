"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, loads or calls anything here, and this package
imports nothing from the product.

`gdn_forward` runs the gated delta rule token by token in the closed form of
the Qwen3.5-9B architecture page (section Gated DeltaNet), expanded as one read
of the old state along the key, the decayed error written back as a rank-one
update, and the output read along the query; for every (sequence, value head)
pair of a packed batch, in fp64, in plain C (gdn_oracle.c).  Decode is the
same call with one token per sequence.

Parity pins for this oracle live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc (-O2, no fast-math) into libgdn_oracle.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            fn = lib.gdn_oracle_forward
            P = ctypes.POINTER
            fn.argtypes = [ctypes.c_int64, ctypes.c_int32, P(ctypes.c_int64),
                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                           P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_double),
                           P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_double),
                           ctypes.c_double, P(ctypes.c_double), P(ctypes.c_double),
                           ctypes.c_int32]
            fn.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x):
    """Exact widening to a C-contiguous fp64 numpy array (accepts torch tensors)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: widen on the CPU (bf16 -> fp32 -> fp64 is exact)
        x = x.detach().to("cpu")
        if not x.dtype.is_floating_point:
            return np.ascontiguousarray(x.numpy()).astype(np.float64)
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def gdn_forward(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=None, threads=None):
    """Sequential fp64 recurrence over a packed batch.

    q, k: [T, HQK, dk]; v: [T, HV, dv]; g, beta: [T, HV];
    cu_seqlens: [N+1] non-decreasing token offsets (None = one sequence);
    initial_state: [N, HV, dk, dv] or None (zeros);
    scale: output multiplier (None = 1/sqrt(dk)).
    Returns (o [T, HV, dv], final_state [N, HV, dk, dv]) as fp64 numpy arrays.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, hv) or beta.shape != (T, hv):
        raise ValueError("inconsistent shapes")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().to("cpu").numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    n = cu.shape[0] - 1
    s0 = _f64(initial_state)
    if s0 is not None and s0.shape != (n, hv, dk, dv):
        raise ValueError("initial_state must be [N, HV, dk, dv]")
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    o = np.zeros((T, hv, dv), dtype=np.float64)
    s_out = np.zeros((n, hv, dk, dv), dtype=np.float64)
    if threads is None:
        threads = default_threads()
    rc = _load().gdn_oracle_forward(
        T, n, _ptr(cu, ctypes.c_int64), hqk, hv, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        float(scale), _ptr(o), _ptr(s_out), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return o, s_out


# Number of fp64 flops the recurrence spends per token per value head:
# decay (dk*dv), read (2*dk*dv), write-back (2*dk*dv), output (2*dk*dv).
def flops_per_token_head(dk: int, dv: int) -> int:
    return 7 * dk * dv
