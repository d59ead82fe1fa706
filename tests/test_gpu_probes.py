"""GPU: the memory-system probes (read-only, write-only, copy) do the work
they are timed for, in every compiled shape and both cache policies, through
the C ABI: the read probe's per-row XOR words match the buffer, the write
probe sets every word, the copy reproduces its source; nothing outside the
target range is written (guard words around each buffer). The matrix-core
probe runs every instruction it is timed for (an exact per-lane sum)."""
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


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (7, 3), (768, 64)])
def test_mfma_probe_runs_every_instruction(workgroups, iters):
    """Constant operands (1/8): every lane's accumulator sum is exactly
    32 * iters (each instruction adds 16 / 64 to each of the 16 elements of
    each accumulator a lane holds, 2 iters instructions per accumulator);
    the sink past the last workgroup is not written."""
    n = workgroups * 256
    buf = torch.full((n + 2 * GUARD,), -1.0, dtype=torch.float32, device=DEV)
    body = buf[GUARD:GUARD + n]
    fr.fr_mfma_probe(workgroups, iters, body, pattern=0)
    torch.cuda.synchronize()
    assert torch.all(body == 32.0 * iters).item()
    assert torch.all(buf[:GUARD] == -1.0).item() and torch.all(buf[GUARD + n:] == -1.0).item()


def probe_operands():
    """The pseudo-random operands of the probe: element e of lane l's vector
    s is the bf16 rounding (nearest, ties to even) of x / 2^23 - 1, with x the
    top 24 bits of the MurmurHash3 32-bit finaliser of h + 1,
    h = (64 s + l) * 8 + e. Returns u, w as [64 lanes, 8] float64 arrays."""
    M = np.uint64(0xFFFFFFFF)
    x = np.arange(1, 2 * 64 * 8 + 1, dtype=np.uint64)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x85EBCA6B)) & M
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & M
    x ^= x >> np.uint64(16)
    v = ((x >> np.uint64(8)).astype(np.float64) * 2.0 ** -23 - 1.0).astype(np.float32)
    b = v.view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    q = r.astype(np.uint32).view(np.float32).astype(np.float64).reshape(2, 64, 8)
    return q[0], q[1]


def test_mfma_probe_random_operands():
    """Pseudo-random operands: every wavefront writes the same 64 sums (same
    operands, same order), and a wavefront's total is the sum of all
    elements of all products it formed: per instruction, sum over the
    k-index of (column sum of A) x (row sum of B), A and B being the lane
    vectors u and w laid out as 32 rows x 16 (lanes 32 h + i hold
    k = 8 h .. 8 h + 7 of row i)."""
    workgroups, iters = 7, 64
    n = workgroups * 256
    buf = torch.full((n + 2 * GUARD,), -1.0, dtype=torch.float32, device=DEV)
    body = buf[GUARD:GUARD + n]
    fr.fr_mfma_probe(workgroups, iters, body, pattern=1)
    torch.cuda.synchronize()
    assert torch.all(buf[:GUARD] == -1.0).item() and torch.all(buf[GUARD + n:] == -1.0).item()
    s = body.cpu().numpy().reshape(workgroups * 4, 64)
    assert np.all(s.view(np.uint32) == s[0].view(np.uint32))
    u, w = probe_operands()
    su, sw = u.reshape(2, 32, 8).sum(axis=1), w.reshape(2, 32, 8).sum(axis=1)
    expected = 8 * iters * float((su * sw).sum())
    au, aw = np.abs(u).reshape(2, 32, 8).sum(axis=1), np.abs(w).reshape(2, 32, 8).sum(axis=1)
    bound = 8 * iters * float((au * aw).sum())
    assert abs(float(s[0].astype(np.float64).sum()) - expected) <= 1e-5 * bound

