"""GPU check of what the chunk table launch writes (global mode: offsets on the device only).

At the start of the workspace the table launch writes the chunk table (the first chunk slot
of every sequence, then the number of chunks), the longest-first order of the sequences
(ties by index), and, for every chunk slot the workspace holds, the first token and the
length of that slot's chunk (length 0 past the batch's chunks); the prep reads nothing but
those slot entries.  Every parity case would also catch a wrong entry; this test checks the
integers themselves, exactly, against a host computation of the same definitions.  The
batches cover one and several blocks of 256 sequences, one and several table workgroups of
2048 slots, zero-length sequences, ragged last chunks and slots past the batch's chunks.
The workspace is filled with a stale byte pattern first, so that an entry left unwritten
shows.  A last case checks the table that a windowed call (host offsets, a long sequence in
the row-split scan, windows of local chunks) leaves behind: its last window's.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

C = 64


def _expected(lengths, max_chunks):
    lengths = np.asarray(lengths, dtype=np.int64)
    counts = -(-lengths // C)
    first = np.concatenate([[0], np.cumsum(counts)])
    table = np.minimum(first, max_chunks).astype(np.int32)
    order = np.array(sorted(range(len(lengths)), key=lambda n: (-lengths[n], n)), dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    slots = np.zeros((max_chunks, 2), dtype=np.int32)
    for n, cnt in enumerate(counts):
        for c in range(int(cnt)):
            e = first[n] + c
            if e < max_chunks:
                t0 = starts[n] + c * C
                slots[e] = (t0, min(C, starts[n + 1] - t0))
    return table, order, slots


def _table_region(lengths, seed):
    inp = S.make_inputs(lengths, 1, 1, 32, 32, torch.bfloat16, seed=seed, s0_std=None)
    N, T = len(lengths), int(sum(lengths))
    shape = gdn.make_shape(1, 1, 32, 32, C, 1, 32 ** -0.5)
    need = gdn.workspace_bytes(shape, T, N)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    d = to_dev(inp)
    say("chunk_table", "N=%d" % N, "T=%d" % T, "workspace %d bytes" % need)
    gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], None, chunk=C, workspace=ws)
    torch.cuda.synchronize()
    raw = ws[:4 * (2 * N + 1) + 8 + 8 * (-(-T // C) + N)].cpu().numpy()
    return raw, N, T


@pytest.mark.parametrize("case", ["varlen_16", "300_sequences", "3000_sequences"])
def test_table_order_and_slot_entries(case):
    rng = np.random.default_rng({"varlen_16": 71, "300_sequences": 72, "3000_sequences": 73}[case])
    if case == "varlen_16":
        lengths = [700, 0, 64, 1, 65, 4096, 0, 129, 2000, 63, 128, 5, 3000, 64, 0, 999]
    elif case == "300_sequences":
        lengths = rng.integers(0, 151, size=300).tolist()      # two blocks of 256 sequences
    else:
        lengths = rng.integers(0, 101, size=3000).tolist()     # slots over three table workgroups
    raw, N, T = _table_region(lengths, seed=len(lengths))
    max_chunks = -(-T // C) + N
    table, order, slots = _expected(lengths, max_chunks)
    ints = raw[:4 * (2 * N + 1)].view(np.int32)
    off = (4 * (2 * N + 1) + 7) // 8 * 8
    got_slots = raw[off:off + 8 * max_chunks].view(np.int32).reshape(max_chunks, 2)
    say("chunk_table", case, "chunks %d of %d slots" % (int(table[-1]), max_chunks))
    np.testing.assert_array_equal(ints[:N + 1], table)
    np.testing.assert_array_equal(ints[N + 1:2 * N + 1], order)
    bad = np.nonzero(np.any(got_slots != slots, axis=1))[0]
    assert bad.size == 0, "slot entries differ at %s: got %s, expected %s" % (
        bad[:5].tolist(), got_slots[bad[:5]].tolist(), slots[bad[:5]].tolist())


def test_last_window_table():
    """Windows: one chunk table per window of local chunks [w0, w0 + W), counting only the
    chunks in it.  At 16 QK / 32 V heads, dk = dv = 128, bf16, the 375-chunk sequence below
    takes windows of W = 125 chunks (three launches, checked by the parity case of the same
    batch), so after the call the workspace holds the last window's table (w0 = 250): the
    125 slots of the long sequence's last 125 chunks, every other sequence empty, and the
    longest-first order written by the first window's launch."""
    lengths = [24000, 9000] + [64] * 20 + [37, 0, 1]
    N, T = len(lengths), int(sum(lengths))
    inp = S.make_inputs(lengths, 16, 32, 128, 128, torch.bfloat16, seed=91, s0_std=None)
    shape = gdn.make_shape(16, 32, 128, 128, C, 1, 128 ** -0.5)
    need = gdn.workspace_bytes(shape, T, N)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    d = to_dev(inp)
    say("chunk_table", "windows", "N=%d" % N, "T=%d" % T, "workspace %d bytes" % need)
    gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], inp["cu_seqlens"].cpu(), None, chunk=C,
                        workspace=ws)
    torch.cuda.synchronize()
    W, w0 = 125, 250
    counts = [min(max(-(-n // C) - w0, 0), W) for n in lengths]
    table = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.array(sorted(range(N), key=lambda n: (-lengths[n], n)), dtype=np.int32)
    slots = np.array([(w0 * C + e * C, min(C, lengths[0] - (w0 + e) * C)) for e in range(table[-1])],
                     dtype=np.int32)
    raw = ws[:4 * (2 * N + 1) + 8 + 8 * len(slots)].cpu().numpy()
    ints = raw[:4 * (2 * N + 1)].view(np.int32)
    off = (4 * (2 * N + 1) + 7) // 8 * 8
    got = raw[off:off + 8 * len(slots)].view(np.int32).reshape(-1, 2)
    np.testing.assert_array_equal(ints[:N + 1], table)
    np.testing.assert_array_equal(ints[N + 1:2 * N + 1], order)
    np.testing.assert_array_equal(got, slots)
