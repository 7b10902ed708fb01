"""GPU parity of a full round through 40 Clover-shaped MoE layers.

Forty independent layers (hidden 2048, 256 routed experts top-8 with Zipf
router bias, intermediate 512, shared expert 512) with the block coreset at
top_p 0.9; identity mixer with RMSNorm before every layer; final RMSNorm;
LM head over a 248320-token vocabulary and the commit.  About 64 GB of bf16
weights are resident.

Every layer is checked against the oracle on the GPU's own normalised input
of that layer (teacher forcing): routing sets bit-exact outside the margin
band, and the residual stream rebuilt in float64 from the oracle's layer
outputs under the routing the GPU took (a legitimate choice inside the band)
must reproduce the GPU's next normalised input."""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W
from gpu_helpers import (BAND, Int4Rows, assert_close, bf16_ulp, commit_check, coreset_in_band, f64,
                         oracle_layer, oracle_layer_int4, packed_layer_int4, top2_gap, topk_gap)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LAYERS = 40
XTOL = 1e-4   # absolute, on unit-RMS normalised states


def _phase1_idx(l, K):
    return np.argsort(-l, axis=1, kind="stable")[:, :K]


def _run_stack(d, layers, oracle_of, lm, wl, x, top_p, wdtype):
    """One round through the layers; every layer checked teacher-forced."""
    T, K = d.T, d.K
    plan = bdd.RoundPlan(bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, wdtype), layers, lm, top_p)
    tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=DEV)
    conf = torch.empty(T, dtype=torch.float32, device=DEV)
    choice = torch.empty(T, dtype=torch.int32, device=DEV)
    ri = torch.empty(4, dtype=torch.int32, device=DEV)
    ltk = torch.empty((LAYERS, T, K), dtype=torch.int32, device=DEV)
    nd = torch.empty(LAYERS, dtype=torch.int32, device=DEV)
    lx = torch.empty((LAYERS, T, d.H), dtype=torch.bfloat16, device=DEV)
    hh = torch.empty((T, d.H), dtype=torch.bfloat16, device=DEV)
    before = tok.cpu().numpy().copy()
    plan(x[0].contiguous().to(DEV), tok, conf, choice, ri, ltk, nd, hh, layer_xhat=lx)
    torch.cuda.synchronize()
    ltk_g, nd_g, lx_g = ltk.cpu().numpy(), nd.cpu().numpy(), f64(lx)

    h = x[0].double().numpy()
    band_layers = 0
    for l in range(LAYERS):
        xg = lx_g[l]
        xr = O.bf16_round(O.rmsnorm(h))
        # two bf16 ulps, plus an absolute term for the float32 residual sum
        # (entries near zero after cancellation carry its ~1e-6 rounding)
        assert np.all(np.abs(xg - xr) <= 2 * bf16_ulp(xr) + XTOL), f"layer {l}: normalised input"
        ol = oracle_of(l)
        _, info = O.moe_layer(xg, ol, K, top_p)
        g = ltk_g[l]
        cband = coreset_in_band(info["p"], _phase1_idx(info["logits"], K), top_p)
        band = topk_gap(info["logits"], K) < BAND
        m = info["coreset"]
        band |= topk_gap(info["logits"][:, m], min(K, len(m))) < BAND
        if cband or band.any():
            band_layers += 1
        if not cband:
            for t in np.nonzero(~band)[0]:
                assert set(int(e) for e in g[t] if e >= 0) == set(int(e) for e in info["idx"][t]), (l, t)
            if not band.any():
                assert int(nd_g[l]) == len(info["union"]), l
        # the layer's output under the routing the GPU took
        p = info["p"]
        wg = np.zeros((T, K))
        for t in range(T):
            live = g[t] >= 0
            wg[t, live] = p[t, g[t][live]] / p[t, g[t][live]].sum()
        y, _ = O.moe_given_routing(xg, ol, g, wg)
        h = h + y
    hr = O.bf16_round(O.rmsnorm(h))
    hg = f64(hh)
    assert np.all(np.abs(hg - hr) <= 2 * bf16_ulp(hr) + XTOL), "LM-head input"

    c_ref, ch_ref, z = O.lm_head_confidence(hg, wl)
    c_gpu, ch_gpu = conf.cpu().numpy(), choice.cpu().numpy()
    assert_close(c_gpu, c_ref, "conf")
    ok = top2_gap(z) >= BAND
    assert np.array_equal(ch_gpu[ok], ch_ref[ok])
    _, exact = commit_check(before, c_ref, ch_ref, ~ok, c_gpu, ch_gpu, tok.cpu().numpy(), ri.cpu().tolist())
    print(f"{LAYERS} layers: distinct experts per layer {nd_g.tolist()}, layers with a band decision "
          f"{band_layers}, round_info {ri.cpu().tolist()}, commit exact {exact}, "
          f"conf range {c_gpu.min():.3f}..{c_gpu.max():.3f}")


def test_stack_40_layers_zipf_coreset():
    seed, d, top_p = 0, W.C1, 0.9
    layers = [W.layer_weights(seed, l, d, device=DEV, bias="zipf", gamma=1.0) for l in range(LAYERS)]
    x, xinfo = W.planted_round_inputs(seed, d, rounds=1, p=0.3, amp_pass=40.0, amp_fail=(14.0, 22.0),
                                      tag="stack")
    w_lm = W.lm_head_weight(seed, d, device=DEV, unit_rows=xinfo["unit_rows"])
    _run_stack(d, layers, lambda l: oracle_layer(layers[l]), bdd.pack_lm_head(w_lm), f64(w_lm), x, top_p,
               bdd.BDD_BF16)


def test_stack_40_layers_int4_zipf_coreset():
    """The same round with 4-bit expert weights (every routed expert and the
    shared expert; router bf16) and the 4-bit LM head (the planted tokens'
    rows the 4-bit rounding of the bf16 head's): about 16 GB of packed
    weights.  The oracle runs on the dequantised weights."""
    seed, d, top_p = 0, W.C1, 0.9
    raw = [W.layer_weights_int4(seed, l, d, device=DEV, bias="zipf", gamma=1.0) for l in range(LAYERS)]
    layers = [packed_layer_int4(w, DEV) for w in raw]
    x, xinfo = W.planted_round_inputs(seed, d, rounds=1, p=0.3, amp_pass=40.0, amp_fail=(14.0, 22.0),
                                      tag="stack")
    codes, scales = W.lm_head_int4(seed, d, device=DEV, unit_rows=xinfo["unit_rows"])
    lm = bdd.pack_lm_head_int4(codes, scales)
    _run_stack(d, layers, lambda l: oracle_layer_int4(raw[l]), lm, Int4Rows(codes, scales), x, top_p,
               bdd.BDD_INT4)
