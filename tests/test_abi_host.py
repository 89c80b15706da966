"""The C ABI on the host: the library loads, exports every function include/gdn.h
declares, sizes its workspace, and rejects bad arguments before any device work.

No call here reaches a kernel launch: every call carries at least one
argument that the host-side validation refuses, and the fake device pointers
are never dereferenced.
"""
import ctypes
import os

import numpy as np
import pytest

import gated_deltanet_scan_amd as gdn
from gated_deltanet_scan_amd import binding

F32, BF16 = binding.GDN_DTYPE_F32, binding.GDN_DTYPE_BF16


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.library_path()):
        from gated_deltanet_scan_amd import build
        build.build()
    return gdn.load_library()


def shape(hqk=16, hv=32, d=128, chunk=64, io=BF16, scale=0.088):
    return gdn.make_shape(hqk, hv, d, d, chunk, io, scale)


# distinct, 256-byte aligned fake device addresses far apart (never dereferenced)
def fake(i):
    return ctypes.c_void_p(0x7f0000000000 + i * (1 << 34))


def prefill(lib, sh, T=128, N=1, cu_host=None, ws_bytes=None, ws=None, q=None, g=None, s0=None, fs=None, o=None):
    cu = np.array([0, T] if N == 1 else np.linspace(0, T, N + 1).astype(np.int32), dtype=np.int32) \
        if cu_host is None else np.asarray(cu_host, dtype=np.int32)
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), T, N)
    return lib.gdn_prefill_chunked(
        ctypes.byref(sh), q if q is not None else fake(1), fake(2), fake(3), g if g is not None else fake(4),
        fake(5), fake(6), N, T, cu.ctypes.data_as(ctypes.c_void_p), s0 if s0 is not None else fake(7),
        fs if fs is not None else fake(8), o if o is not None else fake(9), ws if ws is not None else fake(10),
        need if ws_bytes is None else ws_bytes, None)


def test_every_declared_function_is_exported(lib):
    names = gdn.header_functions()
    assert set(names) >= {"gdn_prefill_chunked", "gdn_decode_step", "gdn_state_snapshot", "gdn_gated_rmsnorm",
                          "gdn_conv1d_qkv", "gdn_conv_state_snapshot", "gdn_prefill_chunked_gated_rmsnorm",
                          "gdn_prefill_workspace_bytes", "gdn_status_string", "gdn_last_error", "gdn_version"}
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.gdn_status_string(0) == b"GDN_OK"
    assert lib.gdn_status_string(3) == b"GDN_ERR_WORKSPACE"
    assert lib.gdn_version() >= 100


def table_bytes(num_seqs, max_chunks):
    """The workspace's table region: chunk table (N + 1 int32), scan order (N int32), then,
    8-byte aligned, a (first token, length) int32 pair per chunk slot; 256-byte aligned."""
    head = -(-(2 * num_seqs + 1) * 4 // 8) * 8
    return -(-(head + 8 * max_chunks) // 256) * 256


def test_workspace_size(lib):
    sh = shape()
    T, N = 1000, 3
    max_chunks = -(-T // 64) + N
    # bf16 at chunk 64 (absorbed form): per chunk slot and value head, W (dk x C) and M (C x C)
    # in bf16 and the decay record (4 C floats)
    expect = table_bytes(N, max_chunks) + max_chunks * 32 * (128 * 64 + 64 * 64) * 2 + max_chunks * 32 * 4 * 64 * 4
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), T, N) == expect
    # fp32 io (direct form): T and A (C x C each)
    sh32 = gdn.make_shape(2, 4, 32, 32, 16, 0, 1.0)
    mc = -(-T // 16) + N
    expect32 = table_bytes(N, mc) + mc * 4 * 2 * 16 * 16 * 4 + mc * 4 * 4 * 16 * 4
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(sh32), T, N) == expect32
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(shape(d=96)), T, N) == 0     # unsupported
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(shape(hqk=3)), T, N) == 0    # 32 % 3 != 0
    assert lib.gdn_prefill_workspace_bytes(None, T, N) == 0


def test_workspace_size_for_host_lengths(lib):
    """gdn_prefill_workspace_bytes_for: the slots of the segment plan for host-known lengths."""
    sh = shape()
    slot = 32 * ((128 + 64) * 64 * 2 + 4 * 64 * 4)          # 819,200 bytes
    cu = np.array([0, 32768], dtype=np.int32)                # 512 chunks: four segments of 128
    got = lib.gdn_prefill_workspace_bytes_for(ctypes.byref(sh), cu.ctypes.data_as(ctypes.c_void_p), 1)
    assert got == table_bytes(1, 513) + 128 * slot
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), 32768, 1) == table_bytes(1, 513) + 513 * slot
    assert gdn.workspace_bytes_for(sh, cu) == got
    # 16 sequences of up to 8192 tokens: single launch over the chunk table, every slot
    from gated_deltanet_scan_amd import synthetic
    lengths = synthetic.varlen_lengths(1004)
    cu16 = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert gdn.workspace_bytes_for(sh, cu16) == lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), int(cu16[-1]), 16)
    # a short batch: one segment as long as its longest sequence
    cu3 = np.array([0, 333, 666, 1000], dtype=np.int32)
    assert gdn.workspace_bytes_for(sh, cu3) == table_bytes(3, -(-1000 // 64) + 3) + 3 * 6 * slot
    # invalid offsets or shapes
    for bad in ([5, 100], [0, 100, 50]):
        arr = np.array(bad, dtype=np.int32)
        assert lib.gdn_prefill_workspace_bytes_for(ctypes.byref(sh), arr.ctypes.data_as(ctypes.c_void_p),
                                                   len(bad) - 1) == 0
    assert lib.gdn_prefill_workspace_bytes_for(ctypes.byref(sh), None, 1) == 0
    assert lib.gdn_prefill_workspace_bytes_for(ctypes.byref(shape(d=96)), cu.ctypes.data_as(ctypes.c_void_p), 1) == 0


def test_prefill_refuses_a_workspace_without_a_chunk_per_sequence(lib):
    """A workspace below the whole batch is cut into segments only with host offsets, and only
    if it holds one chunk of every sequence; otherwise GDN_ERR_WORKSPACE before any launch."""
    sh = shape()
    slot = 32 * ((128 + 64) * 64 * 2 + 4 * 64 * 4)
    N, T = 4, 4000
    cu = np.linspace(0, T, N + 1).astype(np.int32)
    assert prefill(lib, sh, T=T, N=N, cu_host=cu, ws_bytes=256 + N * slot - 1) == binding.GDN_ERR_WORKSPACE
    assert b"one chunk each" in lib.gdn_last_error()
    rc = lib.gdn_prefill_chunked(ctypes.byref(sh), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), N, T, None,
                                 fake(7), fake(8), fake(9), fake(10), 256 + 10 * slot, None)
    assert rc == binding.GDN_ERR_WORKSPACE
    assert b"cu_seqlens_host" in lib.gdn_last_error()


def test_prefill_rejects_bad_shapes(lib):
    assert lib.gdn_prefill_chunked(None, *([None] * 5), None, 1, 1, None, None, None, None, None, 0, None) == 1
    assert prefill(lib, shape(hqk=3)) == binding.GDN_ERR_INVALID_ARG
    assert b"multiple" in lib.gdn_last_error()
    assert prefill(lib, shape(d=96)) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, shape(chunk=32)) == binding.GDN_ERR_UNSUPPORTED
    assert prefill(lib, shape(d=128, chunk=16)) == binding.GDN_ERR_UNSUPPORTED
    # fp32 io at dk = 128 is served (token-recurrent kernel): past the shape check, a misaligned
    # q is the first error (argument checks come before any device work)
    assert prefill(lib, shape(d=128, io=F32), q=ctypes.c_void_p(fake(1).value + 4)) == binding.GDN_ERR_INVALID_ARG
    assert b"aligned" in lib.gdn_last_error()
    assert prefill(lib, shape(io=7)) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, shape(scale=float("nan"))) == binding.GDN_ERR_INVALID_ARG


def test_prefill_rejects_bad_cu_seqlens(lib):
    sh = shape()
    assert prefill(lib, sh, T=100, N=2, cu_host=[1, 50, 100]) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, sh, T=100, N=2, cu_host=[0, 60, 50]) == binding.GDN_ERR_INVALID_ARG
    assert b"decreases" in lib.gdn_last_error()
    assert prefill(lib, sh, T=100, N=2, cu_host=[0, 50, 99]) == binding.GDN_ERR_INVALID_ARG


def prefill_norm(lib, sh, T=128, z=None, w=None, eps=1e-6, y=None):
    cu = np.array([0, T], dtype=np.int32)
    need = lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), T, 1)
    return lib.gdn_prefill_chunked_gated_rmsnorm(
        ctypes.byref(sh), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), 1, T,
        cu.ctypes.data_as(ctypes.c_void_p), fake(7), fake(8), z if z is not None else fake(11),
        w if w is not None else fake(12), ctypes.c_float(eps), y if y is not None else fake(9), fake(10), need, None)


def test_prefill_norm_rejects_bad_arguments(lib):
    sh = shape()
    assert prefill_norm(lib, sh, z=ctypes.c_void_p(fake(11).value + 8)) == binding.GDN_ERR_INVALID_ARG   # alignment
    assert prefill_norm(lib, sh, eps=-1.0) == binding.GDN_ERR_INVALID_ARG
    assert prefill_norm(lib, sh, eps=float("inf")) == binding.GDN_ERR_INVALID_ARG
    assert prefill_norm(lib, sh, y=ctypes.c_void_p(fake(11).value + 256)) == binding.GDN_ERR_INVALID_ARG  # y over z
    assert prefill_norm(lib, sh, w=ctypes.c_void_p(fake(9).value + 16)) == binding.GDN_ERR_INVALID_ARG   # y over w
    assert lib.gdn_prefill_chunked_gated_rmsnorm(
        ctypes.byref(sh), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), 1, 128, None, fake(7), fake(8),
        None, fake(12), ctypes.c_float(1e-6), fake(9), fake(10), 1 << 30, None) == binding.GDN_ERR_INVALID_ARG


def test_prefill_rejects_workspace_and_alignment(lib):
    sh = shape()
    assert prefill(lib, sh, ws_bytes=1024) == binding.GDN_ERR_WORKSPACE
    assert prefill(lib, sh, ws=ctypes.c_void_p(0x7f0000000000 + 10 * (1 << 34) + 64)) == \
        binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, sh, q=ctypes.c_void_p(0x7f0000000000 + (1 << 34) + 2)) == binding.GDN_ERR_INVALID_ARG
    assert prefill(lib, sh, g=ctypes.c_void_p(0x7f0000000000 + 4 * (1 << 34) + 2)) == binding.GDN_ERR_INVALID_ARG


def test_prefill_rejects_overlaps(lib):
    sh = shape()
    # o placed on top of q
    assert prefill(lib, sh, o=fake(1)) == binding.GDN_ERR_INVALID_ARG
    # final state partially overlapping the initial state (exact aliasing is fine, partial is not)
    s0 = fake(7)
    fs_partial = ctypes.c_void_p(s0.value + 4096)
    assert prefill(lib, sh, s0=s0, fs=fs_partial) == binding.GDN_ERR_INVALID_ARG
    assert b"partially" in lib.gdn_last_error()


def test_prefill_with_no_sequences_is_a_no_op(lib):
    sh = shape()
    assert lib.gdn_prefill_chunked(ctypes.byref(sh), None, None, None, None, None, None, 0, 0, None, None, None,
                                   None, None, 0, None) == binding.GDN_OK
    assert lib.gdn_prefill_chunked(ctypes.byref(sh), None, None, None, None, None, None, 0, 5, None, None, None,
                                   None, None, 0, None) == binding.GDN_ERR_INVALID_ARG


def test_decode_rejects_bad_arguments(lib):
    sh = shape()
    args = [fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7)]
    assert lib.gdn_decode_step(ctypes.byref(shape(d=96)), *args, 4, None) == binding.GDN_ERR_UNSUPPORTED
    assert lib.gdn_decode_step(ctypes.byref(sh), *args, -1, None) == binding.GDN_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = None
    assert lib.gdn_decode_step(ctypes.byref(sh), *bad, 4, None) == binding.GDN_ERR_INVALID_ARG
    bad = list(args)
    bad[6] = ctypes.c_void_p(fake(6).value + 8)   # o on top of the state
    assert lib.gdn_decode_step(ctypes.byref(sh), *bad, 4, None) == binding.GDN_ERR_INVALID_ARG
    assert lib.gdn_decode_step(ctypes.byref(sh), *args, 0, None) == binding.GDN_OK


def test_snapshot_rejects_bad_arguments(lib):
    sh = shape()
    assert lib.gdn_state_snapshot(ctypes.byref(sh), fake(1), None, 4, fake(2), None, 4, 5, None) == \
        binding.GDN_ERR_INVALID_ARG   # more rows than capacity
    assert lib.gdn_state_snapshot(ctypes.byref(sh), fake(1), None, 4, ctypes.c_void_p(fake(1).value + 16), None,
                                  4, 2, None) == binding.GDN_ERR_INVALID_ARG   # overlap
    assert lib.gdn_state_snapshot(ctypes.byref(sh), None, None, 4, fake(2), None, 4, 2, None) == \
        binding.GDN_ERR_INVALID_ARG
    assert lib.gdn_state_snapshot(ctypes.byref(sh), fake(1), None, 4, fake(2), None, 4, 0, None) == binding.GDN_OK


def test_conv_state_snapshot_rejects_bad_arguments(lib):
    f = lib.gdn_conv_state_snapshot
    C, W = 768, 4
    assert f(C, W, fake(1), None, 4, fake(2), None, 4, 5, None) == binding.GDN_ERR_INVALID_ARG   # rows > capacity
    assert f(C, W, fake(1), None, 4, ctypes.c_void_p(fake(1).value + 16), None, 4, 2, None) == \
        binding.GDN_ERR_INVALID_ARG   # overlap
    assert f(C, W, ctypes.c_void_p(fake(1).value + 4), None, 4, fake(2), None, 4, 2, None) == \
        binding.GDN_ERR_INVALID_ARG   # misaligned
    assert f(C, W, None, None, 4, fake(2), None, 4, 2, None) == binding.GDN_ERR_INVALID_ARG
    assert f(0, W, fake(1), None, 4, fake(2), None, 4, 2, None) == binding.GDN_ERR_INVALID_ARG
    assert f(C, 9, fake(1), None, 4, fake(2), None, 4, 2, None) == binding.GDN_ERR_UNSUPPORTED
    assert f(6, 2, fake(1), None, 4, fake(2), None, 4, 2, None) == binding.GDN_ERR_UNSUPPORTED   # 6 floats a row
    assert f(C, 1, None, None, 4, None, None, 4, 2, None) == binding.GDN_OK   # width 1: no state
    assert f(C, W, fake(1), None, 4, fake(2), None, 4, 0, None) == binding.GDN_OK


def test_gated_rmsnorm_rejects_bad_arguments(lib):
    sh = shape()
    o, z, w, y = fake(1), fake(2), fake(3), fake(4)
    f = lib.gdn_gated_rmsnorm
    assert f(ctypes.byref(shape(d=96)), o, z, w, y, 4, ctypes.c_float(1e-6), None) == binding.GDN_ERR_UNSUPPORTED
    assert f(ctypes.byref(sh), o, z, w, y, -1, ctypes.c_float(1e-6), None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), o, z, w, y, 4, ctypes.c_float(-1.0), None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), o, z, w, y, 4, ctypes.c_float(float("inf")), None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), o, None, w, y, 4, ctypes.c_float(1e-6), None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), o, z, ctypes.c_void_p(fake(3).value + 4), y, 4, ctypes.c_float(1e-6), None) == \
        binding.GDN_ERR_INVALID_ARG                                             # misaligned weight
    assert f(ctypes.byref(sh), o, z, w, ctypes.c_void_p(fake(1).value + 256), 4, ctypes.c_float(1e-6), None) == \
        binding.GDN_ERR_INVALID_ARG                                             # y partially over o
    assert b"partially" in lib.gdn_last_error()
    assert f(ctypes.byref(sh), o, z, w, y, 0, ctypes.c_float(1e-6), None) == binding.GDN_OK


def test_conv1d_rejects_bad_arguments(lib):
    sh = shape(hqk=2, hv=4, d=64)
    f = lib.gdn_conv1d_qkv
    x, w, cu, si, so, q, k, v = (fake(i) for i in range(1, 9))
    eps = ctypes.c_float(1e-6)
    assert f(ctypes.byref(shape(d=96)), x, w, 4, cu, 1, 10, si, so, 0, 1, eps, q, k, v, None) == \
        binding.GDN_ERR_UNSUPPORTED
    assert f(ctypes.byref(sh), x, w, 9, cu, 1, 10, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_ERR_UNSUPPORTED
    assert f(ctypes.byref(sh), x, w, 0, cu, 1, 10, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_ERR_UNSUPPORTED
    assert f(ctypes.byref(sh), x, w, 4, cu, -1, 10, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), x, w, 4, cu, 0, 10, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), x, w, 4, None, 1, 10, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), x, w, 4, cu, 1, 10, si, so, 0, 1, ctypes.c_float(-1.0), q, k, v, None) == \
        binding.GDN_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), ctypes.c_void_p(fake(1).value + 8), w, 4, cu, 1, 10, si, so, 0, 1, eps, q, k, v,
             None) == binding.GDN_ERR_INVALID_ARG                                 # misaligned x
    assert f(ctypes.byref(sh), x, w, 4, cu, 1, 10, si, so, 0, 1, eps, q, q, v, None) == \
        binding.GDN_ERR_INVALID_ARG                                               # q and k overlap
    assert f(ctypes.byref(sh), x, w, 4, cu, 1, 10, si, ctypes.c_void_p(fake(4).value + 64), 0, 1, eps, q, k, v,
             None) == binding.GDN_ERR_INVALID_ARG                                 # state_out partially over state_in
    assert f(ctypes.byref(sh), x, w, 4, cu, 0, 0, si, so, 0, 1, eps, q, k, v, None) == binding.GDN_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 1, 32)
    with pytest.raises(ValueError):
        gdn.prefill_chunked(x, x, torch.zeros(4, 2, 32), torch.zeros(4, 2), torch.zeros(4, 2))


def test_noalloc_prefill_rejects_batches_beyond_its_scratch(lib):
    """gdn_prefill_chunked_noalloc refuses, on the host and before any device call, a batch whose
    chunk workspace exceeds its 64 MiB scratch when no host offsets are given, and a batch of
    more sequences than the scratch has chunk slots even with them (GDN_ERR_WORKSPACE); and it
    checks its other arguments as gdn_prefill_chunked does."""
    sh = shape()
    T = 12000                                   # 190 chunk slots of 819,200 bytes: 155 MB
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(sh), T, 2) > (64 << 20)
    rc = lib.gdn_prefill_chunked_noalloc(ctypes.byref(sh), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                                         2, T, None, fake(7), fake(8), fake(9), None)
    assert rc == binding.GDN_ERR_WORKSPACE
    assert b"scratch" in lib.gdn_last_error()
    N = 120                                     # more sequences than its 81 chunk slots
    cu = np.arange(0, 70 * (N + 1), 70, dtype=np.int32)
    rc = lib.gdn_prefill_chunked_noalloc(ctypes.byref(sh), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                                         N, int(cu[-1]), cu.ctypes.data_as(ctypes.c_void_p), fake(7), fake(8),
                                         fake(9), None)
    assert rc == binding.GDN_ERR_WORKSPACE
    # argument errors come first, as for the workspace entry point
    rc = lib.gdn_prefill_chunked_noalloc(ctypes.byref(shape(d=96)), fake(1), fake(2), fake(3), fake(4), fake(5),
                                         fake(6), 1, 128, None, fake(7), fake(8), fake(9), None)
    assert rc == binding.GDN_ERR_UNSUPPORTED
    rc = lib.gdn_prefill_chunked_noalloc(ctypes.byref(sh), ctypes.c_void_p(0x7f0000000008), fake(2), fake(3),
                                         fake(4), fake(5), fake(6), 1, 128, None, fake(7), fake(8), fake(9), None)
    assert rc == binding.GDN_ERR_INVALID_ARG
