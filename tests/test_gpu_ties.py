"""GPU parity of the routing tie rules (reading S3: among equal keys the lower
expert id comes first, in the top-K and in the coreset's mass order).

The margin bands of the other parity tests leave every near-tie uncompared.
Here the ties are exact on both sides: two experts get the same router row and
the same bias, so their logits are bit-identical on the GPU (the same products
summed in the same order) and equal in the oracle's float64, and with them
every position's softmax scores and the block masses.  Biases place the tied
pair exactly at the decision: the top-K boundary (K = 2: the lower id is
picked, the higher one is not) or the coreset cut (K = 3, top_p 0.7: equal
masses straddle the cut and the lower id is kept).  Every other decision is
redrawn until it lies outside the margin band, then routing, coreset, union
and y are compared with the oracle.

[P1] aitujian.cn article on Clover-35B-A3B-Preview, section 四 (top-8 of 256
routed experts); [P2] goremy.ai "What is the MoE coreset and why does it
matter?" (experts ranked by block mass, the shortest covering prefix)."""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W
from gpu_helpers import BAND, assert_close, dims_of, f64, oracle_layer

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

A, B1, B2 = 3, 11, 29   # the leading expert and the tied pair (B1 < B2)


def _dims(K):
    return W.Dims(f"ties_k{K}", T=13, H=256, E=40, K=K, I=96, I_s=64, V=16, wdtype="bf16", w_std=0.05,
                  lm_std=0.06)


def _tied_case(K, bias_a, bias_b, top_p, check):
    """The first seed (from 7, counting up by 1000) whose oracle layer passes
    `check` and keeps every decision other than the tie outside the band."""
    d = _dims(K)
    for s in range(7, 40007, 1000):
        layer = W.layer_weights(s, 0, d, device="cpu", bias="flat")
        layer["w_router"][B2] = layer["w_router"][B1]
        layer["router_bias"][A] = bias_a
        layer["router_bias"][B1] = bias_b
        layer["router_bias"][B2] = bias_b
        h = W.block_hidden(s, d)
        xh = O.bf16_round(O.rmsnorm(f64(h)))
        y_ref, info = O.moe_layer(xh, oracle_layer(layer), d.K, top_p)
        l = info["logits"]
        assert np.array_equal(l[:, B1], l[:, B2])   # the tie is exact in the oracle
        order = np.argsort(-l, axis=1, kind="stable")
        # the ranks below the tied pair's ranks (K + 1 of them) are clear of the pair
        # and of each other
        srt = np.take_along_axis(l, order, axis=1)
        gaps_ok = all(srt[t, j] - srt[t, j + 1] >= BAND
                      for t in range(d.T) for j in range(K + 1)
                      if {int(order[t, j]), int(order[t, j + 1])} != {B1, B2})
        if gaps_ok and check(info):
            return d, layer, h, xh, y_ref, info
    pytest.fail("no seed places the tie at the decision with every other decision outside the band")


def _gpu(d, layer, h, top_p):
    lay = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}
    out = bdd.moe_block_forward(dims_of(d), lay, h.to(DEV), top_p)
    torch.cuda.synchronize()
    return out


def _picks(out, t):
    gi = out["topk_idx"].cpu().numpy()[t]
    gw = out["topk_w"].cpu().numpy()[t]
    return {int(e): float(w) for e, w in zip(gi, gw) if e >= 0}


def test_topk_tie_at_the_boundary_takes_the_lower_id():
    # K = 2: the leader first, then the tied pair: only the lower id is picked
    d, layer, h, xh, y_ref, info = _tied_case(
        2, 10.0, 6.0, 1.0, lambda inf: all(sorted(int(e) for e in inf["idx"][t]) == [A, B1] for t in range(13)))
    out = _gpu(d, layer, h, 1.0)
    for t in range(d.T):
        got = _picks(out, t)
        assert sorted(got) == [A, B1], (t, sorted(got))
        ref = {int(e): w for e, w in zip(info["idx"][t], info["w"][t])}
        assert_close([got[e] for e in ref], [ref[e] for e in ref], f"topk_w[{t}]")
    assert int(out["n_distinct"].item()) == 2
    assert_close(f64(out["y"]), y_ref, "y")


def test_coreset_mass_tie_at_the_cut_keeps_the_lower_id():
    # K = 3: every position picks the leader and both tied experts, whose block
    # masses are then exactly equal; top_p 0.7 cuts between them
    top_p = 0.7

    def block_mass(inf):
        first = np.argsort(-inf["logits"], axis=1, kind="stable")[:, :3]
        return O.coreset_select(inf["p"], first, top_p)[1]

    def check(inf):
        c = inf["coreset"]
        if c is None or sorted(int(e) for e in c) != [A, B1]:
            return False
        m = block_mass(inf)
        tot = float(np.sum(m))
        # the cut is clear of the target on both sides (the pair itself is the tie)
        return m[A] < top_p * tot - BAND and m[A] + m[B1] >= top_p * tot + BAND

    d, layer, h, xh, y_ref, info = _tied_case(3, 10.0, 9.0, top_p, check)
    m = block_mass(info)
    assert m[B1] == m[B2] and m[B1] > 0   # the masses tie exactly
    out = _gpu(d, layer, h, top_p)
    bits = out["coreset_bits"].cpu().numpy().view(np.uint32)
    got = [e for e in range(d.E) if bits[e // 32] >> (e % 32) & 1]
    assert got == [A, B1], got
    assert int(out["coreset_size"].item()) == 2
    for t in range(d.T):
        g = _picks(out, t)
        assert sorted(g) == [A, B1], (t, sorted(g))
        ref = {int(e): w for e, w in zip(info["idx"][t], info["w"][t])}
        assert_close([g[e] for e in ref], [ref[e] for e in ref], f"topk_w[{t}]")
    assert int(out["n_distinct"].item()) == 2
    assert_close(f64(out["y"]), y_ref, "y")
