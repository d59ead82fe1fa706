"""GPU: the memory-system probes (read-only, write-only, copy) do the work
they are timed for, in every compiled shape and both cache policies, through
the C ABI: the read probe's per-row XOR words match the buffer, the write
probe sets every word, the copy reproduces its source; nothing outside the
target range is written (guard words around each buffer)."""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(64, 2), (64, 4), (64, 8), (64, 16), (128, 4), (256, 1), (256, 2), (256, 4), (256, 8),
          (256, 16), (512, 1), (512, 2), (512, 4), (512, 8), (1024, 1), (1024, 2), (1024, 4),
          (1024, 7), (1024, 8), (1024, 13), (1024, 16)]
GUARD = 64            # int32 words on each side
CANARY = 0x5A5A5A5A


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def guarded(nwords, fill):
    buf = torch.full((nwords + 2 * GUARD,), CANARY, dtype=torch.int32, device=DEV)
    body = buf[GUARD:GUARD + nwords]
    body.fill_(fill)
    return buf, body


def intact(buf):
    g = torch.cat([buf[:GUARD], buf[-GUARD:]]).cpu().numpy()
    return bool(np.all(g == CANARY))


def row_xor(words, row_words):
    """The read probe's expectation: XOR of each row's 32-bit words."""
    per_row = row_words
    rows = -(-len(words) // per_row)
    pad = np.zeros(rows * per_row, dtype=np.uint32)
    pad[:len(words)] = words
    return np.bitwise_xor.reduce(pad.reshape(rows, per_row), axis=1)


@pytest.mark.parametrize("policy", [0, 1, 2, 3])
@pytest.mark.parametrize("threads,vecs", SHAPES)
@pytest.mark.parametrize("short_rows", [False, True])
def test_probes(threads, vecs, policy, short_rows):
    rng = np.random.default_rng(threads * 100 + vecs)
    # full rows of the shape, or rows of an odd number of chunks short of it;
    # several rows and a partial last row (a multiple of 16 bytes)
    row_bytes = threads * vecs * 16 - (16 * 37 if short_rows and threads * vecs > 37 else 0)
    nbytes = 3 * row_bytes + 48 * 16 + 16
    nw = nbytes // 4
    src_np = rng.integers(0, 2**32, size=nw, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(src_np.view(np.int32)).to(DEV)
    rb = row_bytes if short_rows else 0

    rows = fr.fr_stream_probe_rows(nbytes, row_bytes)
    sbuf, sink = guarded(rows, -1)
    fr.fr_stream_probe(fr.PROBE_READ, src=src, sink=sink, nbytes=nbytes, threads=threads,
                       vecs=vecs, policy=policy, row_bytes=rb)
    torch.cuda.synchronize()
    assert intact(sbuf), "read probe wrote outside its sink"
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, row_xor(src_np, row_bytes // 4))

    dbuf, dst = guarded(nw, 0)
    fr.fr_stream_probe(fr.PROBE_WRITE, dst=dst, nbytes=nbytes, value=0x01234567,
                       threads=threads, vecs=vecs, policy=policy, row_bytes=rb)
    torch.cuda.synchronize()
    assert intact(dbuf), "write probe wrote outside its buffer"
    assert bool(torch.all(dst == 0x01234567))

    cbuf, cdst = guarded(nw, 0)
    fr.fr_stream_probe(fr.PROBE_COPY, src=src, dst=cdst, nbytes=nbytes, threads=threads,
                       vecs=vecs, policy=policy, row_bytes=rb)
    torch.cuda.synchronize()
    assert intact(cbuf), "copy probe wrote outside its buffer"
    assert torch.equal(cdst, src)


def test_default_shape_entry_points():
    nbytes = (1 << 20) + 16 * 5
    nw = nbytes // 4
    src_np = np.arange(nw, dtype=np.uint32) * np.uint32(2654435761)
    src = torch.from_numpy(src_np.view(np.int32)).to(DEV)
    sbuf, sink = guarded(fr.fr_stream_probe_rows(nbytes), -1)
    fr.fr_stream_read(src, sink)
    dbuf, dst = guarded(nw, 0)
    fr.fr_stream_write(dst, 0xDEADBEEF)
    cbuf, cdst = guarded(nw, 0)
    fr.fr_stream_copy(src, cdst)
    torch.cuda.synchronize()
    assert intact(sbuf) and intact(dbuf) and intact(cbuf)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32),
                          row_xor(src_np, fr.STREAM_THREADS * fr.STREAM_VECS * 4))
    assert bool(torch.all(dst == np.int32(np.uint32(0xDEADBEEF).view(np.int32))))
    assert torch.equal(cdst, src)
