"""GPU parity of the attention forward (the online softmax inside attention,
on the bf16 matrix cores) against the double-precision oracle, through the C
ABI.

Tolerances (bf16 inputs are exact; the kernel accumulates in fp32, rounds the
probabilities to bf16 for the value product and the output to bf16 once):
  o_id    |g - o| <= 2^-8 * sum_j p_ij |v_jd| + 2^-8 |o_id|
          (each probability carries a relative rounding error <= 2^-9; the
          output's own rounding <= 2^-9 |o|; a factor 2 of margin on each)
  lse_i   |g - lse| <= 1e-5 (|lse| + scale * max_j sum_d |q_id k_jd|)
          (fp32 accumulation of a D-term dot product: D * 2^-24 < 1e-5)
"""
import numpy as np
import pytest
import torch

import memory_bound_row_pass_amd as fr
import oracle
import workloads
from gpu_buffers import DEV, Guarded, upload
from parity import bf16_bits, bf16_value

pytestmark = pytest.mark.gpu


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    oracle.set_threads(min(16, oracle.threads()))


def run(w, causal, scale, inplace=False, with_lse=True):
    q, k, v = (upload(w[n]) for n in ("q", "k", "v"))
    B, H, Sq, D = w["q"].shape
    lse = Guarded((B, H, Sq), torch.float32) if with_lse else None
    if inplace:
        fr.fr_attention_fwd(q, k, v, q, lse.t if lse else None, causal, scale)
        torch.cuda.synchronize()
        return bf16_bits(q), (lse.t.cpu().numpy() if lse else None)
    o = Guarded((B, H, Sq, D), torch.bfloat16)
    fr.fr_attention_fwd(q, k, v, o.t, lse.t if lse else None, causal, scale)
    torch.cuda.synchronize()
    assert o.canaries_intact() and (lse is None or lse.canaries_intact())
    return bf16_bits(o.t), (lse.t.cpu().numpy() if lse else None)


def expect(w, causal, scale, got, what):
    ob, lg = got
    q, k, v = (oracle.decode(w[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.attention(w["q"], w["k"], w["v"], causal=causal, scale=scale)
    Sq, Sk = q.shape[2], k.shape[2]
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    vis = np.ones((Sq, Sk), bool) if not causal else np.tri(Sq, Sk, Sk - Sq, dtype=bool)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(vis, np.exp(s - lse_ref[..., None]), 0.0)
    p = np.nan_to_num(p)
    bound = 2.0 ** -8 * (p @ np.abs(v)) + 2.0 ** -8 * np.abs(o_ref)
    g = bf16_value(ob).reshape(o_ref.shape)
    err = np.abs(g - o_ref)
    bad = err > bound + 1e-30
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond bound; worst "
                           f"{float((err - bound).max()):.3g}")
    if lg is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lg), ~fin), what + ": -inf lse where no key is visible"
        sabs = abs(scale) * np.einsum("bhid,bhjd->bhij", np.abs(q), np.abs(k))
        sabs = np.where(vis, sabs, 0).max(-1)
        lb = 1e-5 * (np.abs(lse_ref) + sabs)
        assert np.all(np.abs(lg[fin] - lse_ref[fin]) <= lb[fin]), what + " lse"
    return float((err / np.maximum(bound, 1e-30)).max())


SHAPES = [(1, 2, 128, 128, 64), (2, 3, 200, 333, 128), (1, 1, 1, 1, 64), (1, 2, 300, 300, 128),
          (1, 1, 257, 129, 64), (1, 1, 129, 500, 128), (2, 2, 64, 31, 128), (1, 1, 1000, 1000, 64),
          # batch x heads a multiple of 8: workgroups grouped by head per XCD
          (2, 4, 300, 300, 128), (1, 8, 129, 200, 64), (4, 4, 256, 100, 128)]


@pytest.mark.parametrize("B,H,Sq,Sk,D", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_shapes(B, H, Sq, Sk, D, causal):
    w = workloads.make_attention(B, H, Sq, Sk, D, seed=Sq * 7 + Sk + D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    r = expect(w, causal, scale, run(w, causal, scale), f"attn {B}x{H}x{Sq}x{Sk}x{D} causal={causal}")
    print("worst error / bound", round(r, 3))


def test_scales_in_place_and_no_lse():
    w = workloads.make_attention(1, 2, 256, 256, 128, seed=5)
    # 0: every visible score equal, hidden blocks of a query at scale 0;
    # negative: the block max is taken as the min of the raw scores
    for scale in (0.0, 0.02, 0.3, -0.05):
        expect(w, True, scale, run(w, True, scale), f"attn scale {scale}")
    expect(w, False, -0.05, run(w, False, -0.05), "attn scale -0.05 non-causal")
    expect(w, False, 0.0883883, run(w, False, 0.0883883, inplace=True), "attn in place (o = q)")
    ob, lg = run(w, False, 0.0883883, with_lse=False)
    assert lg is None
    expect(w, False, 0.0883883, (ob, None), "attn without lse")


def test_large_sampled():
    # B=2, H=4, S=2048, D=128; oracle on a subset of queries: non-causal any
    # rows, causal the first 256 (their visible keys are the first ones)
    w = workloads.make_attention(2, 4, 2048, 2048, 128, seed=11)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    for causal in (False, True):
        ob, lg = run(w, causal, scale)
        ob = ob.reshape(2, 4, 2048, 128)
        rows = np.array([0, 1, 255, 777, 1500, 2047]) if not causal else np.arange(256)
        sub = workloads.Workload(w.spec, 0, 0, 0, {"q": w["q"][:, :, rows],
                                                   "k": w["k"] if not causal else w["k"][:, :, :256],
                                                   "v": w["v"] if not causal else w["v"][:, :, :256]})
        expect(sub, causal, scale, (ob[:, :, rows], lg[:, :, rows]), f"attn large causal={causal}")


def test_bitwise_determinism():
    w = workloads.make_attention(2, 2, 512, 512, 128, seed=12)
    r = [run(w, True, 0.0883883) for _ in range(3)]
    assert all(np.array_equal(r[0][0], x[0]) and np.array_equal(r[0][1], x[1]) for x in r)


def test_rising_scores_rescale_every_block():
    # scores rise by ~11 (base 2) from one 32-key block to the next, so the
    # running max is raised and the accumulator rescaled on every block
    B, H, S, D = 1, 2, 512, 64
    rng = np.random.default_rng(13)
    q = np.full((B, H, S, D), 4.0, np.float32)
    k = np.repeat((4.0 * np.arange(S) / S).astype(np.float32)[None, None, :, None], D, axis=3)
    k = np.broadcast_to(k, (B, H, S, D)).copy()
    v = rng.normal(0, 1, size=(B, H, S, D)).astype(np.float32)
    w = workloads.Workload(workloads.make_attention(1, 1, 1, 1, 64).spec, 0, 0, 0,
                           {n: oracle.round_bf16(a) for n, a in (("q", q), ("k", k), ("v", v))})
    for causal in (False, True):
        expect(w, causal, 0.125, run(w, causal, 0.125), f"attn rising scores causal={causal}")


def test_bench_shape_sampled():
    # the benchmarked shape (B=4 H=16 S=4096 D=128), every one of the 64
    # (batch, head) pairs (the head-to-XCD grouping deals them out in groups
    # of 8): queries of the first, a middle and the last 128-query block —
    # both ends of each block and one seeded query per block in another
    # wave — against the oracle, causal and not
    w = workloads.make_attention(4, 16, 4096, 4096, 128)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    rng = np.random.default_rng(4096)
    for causal in (False, True):
        ob, lg = run(w, causal, scale)
        ob = ob.reshape(4, 16, 4096, 128)
        for b in range(4):
            for h in range(16):
                rows = []
                for blk in (0, 16, 31):
                    q0 = 128 * blk
                    rows += [q0, q0 + 127, q0 + 32 * int(rng.integers(1, 3)) + int(rng.integers(0, 32))]
                rows = np.array(sorted(set(rows)))
                sub = workloads.Workload(w.spec, 0, 0, 0, {"q": w["q"][b:b + 1, h:h + 1, rows],
                                                           "k": w["k"][b:b + 1, h:h + 1],
                                                           "v": w["v"][b:b + 1, h:h + 1]})
                if causal:
                    # a sampled query i sees keys j <= i: compare query by query
                    for r_i, r in enumerate(rows):
                        one = workloads.Workload(w.spec, 0, 0, 0, {
                            "q": sub["q"][:, :, r_i:r_i + 1], "k": sub["k"][:, :, :r + 1],
                            "v": sub["v"][:, :, :r + 1]})
                        expect(one, False, scale, (ob[b:b + 1, h:h + 1, r:r + 1],
                                                   lg[b:b + 1, h:h + 1, r:r + 1]),
                               f"attn bench shape causal b{b} h{h} q{r}")
                else:
                    expect(sub, False, scale, (ob[b:b + 1, h:h + 1, rows], lg[b:b + 1, h:h + 1, rows]),
                           f"attn bench shape b{b} h{h}")