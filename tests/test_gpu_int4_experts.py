"""GPU parity of MoE layers with 4-bit expert weights against the CPU oracle
on the dequantised weights.

[P3] 10100.com article on Clover-35B-A3B-Preview, part 03 (memory and
quantisation): the model is deployed with INT4 weights; the pages give no
format.  The format read here (the library's BDD_INT4): two 4-bit codes per
byte (low nibble = even column), code n standing for n - 8, one bf16 scale per
row and 128-column group; the router and the activations stay bf16.  The
oracle dequantises every expert matrix in float64 (oracle.int4_dequantize) and
runs its MoE layer on the result; the GPU takes the codes packed by
bdd_pack_int4.  Tolerances are those of the bf16 layers.  Each draw is
redrawn on the CPU until no routing or coreset decision lies inside a margin
band, then routing, coreset, union and y are all compared."""

import dataclasses

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W
from gpu_helpers import (BAND, Int4Rows, assert_close, bf16_ulp, commit_check, commit_in_band, coreset_in_band, f64,
                         oracle_layer_int4, packed_layer_int4, top2_gap, topk_gap)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dims(d):
    return bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, bdd.BDD_INT4)


def _phase1_idx(l, K):
    return np.argsort(-l, axis=1, kind="stable")[:, :K]


def _bands(d, info, top_p):
    band = topk_gap(info["logits"], d.K) < BAND
    if info["coreset"] is not None:
        m = info["coreset"]
        band |= topk_gap(info["logits"][:, m], min(d.K, len(m))) < BAND
    return band, coreset_in_band(info["p"], _phase1_idx(info["logits"], d.K), top_p)


def _layer_case(d, seed, bias, top_p, gen_device="cpu"):
    for s in range(seed, seed + 20000, 1000):
        w = W.layer_weights_int4(s, 0, d, device=gen_device, bias=bias)
        h = W.block_hidden(s, d)
        xh = O.bf16_round(O.rmsnorm(f64(h)))
        ol = oracle_layer_int4(w)
        y_ref, info = O.moe_layer(xh, ol, d.K, top_p)
        band, cband = _bands(d, info, top_p)
        if not (band.any() or cband):
            return s, w, h, xh, y_ref, info
    pytest.fail("no seed with every decision outside the margin band")


def _check_layer(d, out, xh, y_ref, info, top_p):
    gx = f64(out["xhat"])
    assert np.all(np.abs(gx - xh) <= bf16_ulp(xh) * 1.0001)
    gi = out["topk_idx"].cpu().numpy()
    gw = out["topk_w"].cpu().numpy()
    for t in range(d.T):
        ref = {int(e): w for e, w in zip(info["idx"][t], info["w"][t])}
        got = {int(e): float(w) for e, w in zip(gi[t], gw[t]) if e >= 0}
        assert set(got) == set(ref), (t, sorted(got), sorted(ref))
        assert_close([got[e] for e in ref], [ref[e] for e in ref], f"topk_w[{t}]")
    assert int(out["n_distinct"].item()) == len(info["union"])
    members = info["coreset"] if info["coreset"] is not None else np.array(info["union"])
    bits = out["coreset_bits"].cpu().numpy().astype(np.uint32)
    got = [e for e in range(d.E) if (int(bits[e // 32]) >> (e % 32)) & 1]
    assert got == sorted(int(e) for e in members)
    assert_close(f64(out["y"]), y_ref, "y")


SMALL = W.Dims("i4_small", T=13, H=384, E=40, K=6, I=256, I_s=128, V=5003, wdtype="bf16", w_std=0.05,
               lm_std=384 ** -0.5)


@pytest.mark.parametrize("bias,top_p,force,T", [("flat", 1.0, False, 13), ("zipf", 0.7, False, 13),
                                                ("flat", 1.0, True, 13), ("zipf", 0.9, True, 13),
                                                ("flat", 1.0, True, 64), ("zipf", 0.9, False, 50)])
def test_int4_layer_small(bias, top_p, force, T):
    # hidden 384 (3 groups of 128: the waves' group shares are uneven), I 256,
    # I_s 128; `force` sends every position to experts 0..2 (dense experts
    # with all T positions beside token groups); blocks of 50 and 64 positions
    # take four column tiles
    d = SMALL if T == SMALL.T else dataclasses.replace(SMALL, name=f"i4_small_block{T}", T=T)
    for s in range(3, 20003, 1000):
        w = W.layer_weights_int4(s, 0, d, bias=bias)
        if force:
            w["router_bias"][:3] = 10.0
        h = W.block_hidden(s, d)
        xh = O.bf16_round(O.rmsnorm(f64(h)))
        y_ref, info = O.moe_layer(xh, oracle_layer_int4(w), d.K, top_p)
        band, cband = _bands(d, info, top_p)
        if not (band.any() or cband):
            break
    else:
        pytest.fail("no seed with every decision outside the margin band")
    out = bdd.moe_block_forward(_dims(d), packed_layer_int4(w, DEV), h.to(DEV), top_p)
    torch.cuda.synchronize()
    _check_layer(d, out, xh, y_ref, info, top_p)
    n_e = np.bincount(np.asarray(info["idx"]).ravel()[np.asarray(info["idx"]).ravel() >= 0], minlength=d.E)
    print(f"{bias} top_p {top_p} force {force} seed {s}: positions per union expert "
          f"{sorted(n_e[n_e > 0].tolist(), reverse=True)}")
    if force:
        assert (n_e[:3] == d.T).all() or info["coreset"] is not None


@pytest.mark.parametrize("bias,top_p", [("flat", 1.0), ("zipf", 0.9)])
def test_int4_layer_clover_shape(bias, top_p):
    """One Clover-shaped layer (hidden 2048, 256 experts top-8, intermediate
    512, shared expert 512, block 32) with 4-bit experts."""
    d = W.C1
    s, w, h, xh, y_ref, info = _layer_case(d, 0, bias, top_p, gen_device=DEV)
    out = bdd.moe_block_forward(_dims(d), packed_layer_int4(w, DEV), h.to(DEV), top_p)
    torch.cuda.synchronize()
    _check_layer(d, out, xh, y_ref, info, top_p)
    print(f"{bias} top_p {top_p} seed {s}: union {len(info['union'])}, "
          f"coreset {None if info['coreset'] is None else len(info['coreset'])}")


def test_int4_round_two_layers_with_int4_lm_head():
    """A full round: two 4-bit layers (Zipf, coreset 0.9), final norm, the
    4-bit LM head and the commit; each layer teacher-forced on the GPU's own
    normalised input, the head and commit on the GPU's final state."""
    d = SMALL
    L, top_p = 2, 0.9
    for s in range(5, 40005, 1000):
        x, xinfo = W.planted_round_inputs(s, d, rounds=1, p=0.4, amp_pass=40.0, amp_fail=(6.0, 16.0))
        ws = [W.layer_weights_int4(s, l, d, bias="zipf") for l in range(L)]
        ols = [oracle_layer_int4(w) for w in ws]
        hh, infos = O.moe_stack(x[0].double().numpy(), ols, d.K, top_p)
        if any(_bands(d, inf, top_p)[0].any() or _bands(d, inf, top_p)[1] for inf in infos):
            continue
        codes, scales = W.lm_head_int4(s, d, unit_rows=xinfo["unit_rows"])
        wl = Int4Rows(codes, scales)
        c0, _, z0 = O.lm_head_confidence(hh, wl)
        if not commit_in_band(np.full(d.T, O.MASK), c0) and (top2_gap(z0) >= BAND).all():
            break
    else:
        pytest.fail("no seed with every decision outside the margin band")
    lm = bdd.pack_lm_head_int4(codes.to(DEV), scales.to(DEV))
    plan = bdd.RoundPlan(_dims(d), [packed_layer_int4(w, DEV) for w in ws], lm, top_p)
    T = d.T
    tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=DEV)
    conf = torch.empty(T, dtype=torch.float32, device=DEV)
    choice = torch.empty(T, dtype=torch.int32, device=DEV)
    ri = torch.empty(4, dtype=torch.int32, device=DEV)
    ltk = torch.empty((L, T, d.K), dtype=torch.int32, device=DEV)
    lx = torch.empty((L, T, d.H), dtype=torch.bfloat16, device=DEV)
    hh_gpu = torch.empty((T, d.H), dtype=torch.bfloat16, device=DEV)
    plan(x[0].to(DEV), tok, conf, choice, ri, ltk, None, hh_gpu, layer_xhat=lx)
    torch.cuda.synchronize()
    h = x[0].double().numpy()
    g_idx, lx_g = ltk.cpu().numpy(), f64(lx)
    for li in range(L):
        xr = O.bf16_round(O.rmsnorm(h))
        assert np.all(np.abs(lx_g[li] - xr) <= 2 * bf16_ulp(xr) + 1e-4), li
        _, inf = O.moe_layer(lx_g[li], ols[li], d.K, top_p)
        band, cband = _bands(d, inf, top_p)
        assert not cband and band.sum() <= 1
        for t in np.nonzero(~band)[0]:
            assert set(int(e) for e in g_idx[li, t] if e >= 0) == set(int(e) for e in inf["idx"][t]), (li, t)
        g = g_idx[li]
        wg = np.zeros((T, d.K))
        for t in range(T):
            live = g[t] >= 0
            wg[t, live] = inf["p"][t, g[t][live]] / inf["p"][t, g[t][live]].sum()
        y, _ = O.moe_given_routing(lx_g[li], ols[li], g, wg)
        h = h + y
    hr = O.bf16_round(O.rmsnorm(h))
    assert np.all(np.abs(f64(hh_gpu) - hr) <= 2 * bf16_ulp(hr) + 1e-4)
    c_ref, ch_ref, z = O.lm_head_confidence(f64(hh_gpu), wl)
    c_gpu, ch_gpu = conf.cpu().numpy(), choice.cpu().numpy()
    assert_close(c_gpu, c_ref, "conf")
    ok = top2_gap(z) >= BAND
    assert np.array_equal(ch_gpu[ok], ch_ref[ok])
    _, exact = commit_check(np.full(T, O.MASK), c_ref, ch_ref, ~ok, c_gpu, ch_gpu, tok.cpu().numpy(),
                            ri.cpu().tolist())
    print(f"seed {s}: round_info {ri.cpu().tolist()}, committed {int((tok >= 0).sum())} of {T}")
    assert exact


def test_int4_pack_matches_the_lm_head_layout():
    # the expert pack (bdd_pack_int4) lays each matrix out as the 4-bit LM
    # head does (bdd_lmhead_pack_int4), matrix after matrix
    d = W.Dims("p", T=1, H=256, E=3, K=1, I=128, I_s=128, V=48, wdtype="bf16", w_std=0.05, lm_std=0.06)
    mats = [W.int4_matrix((7, "m", j), 48, 256, 0.05) for j in range(3)]
    codes = torch.stack([c for c, _ in mats]).to(DEV)
    scales = torch.stack([s for _, s in mats]).to(DEV)
    packed = bdd.pack_int4(codes, scales)
    torch.cuda.synchronize()
    mb = bdd.int4_packed_bytes(1, 48, 256)
    assert packed.numel() == 3 * mb
    for j in range(3):
        one = bdd.pack_lm_head_int4(codes[j].contiguous(), scales[j].contiguous()).packed
        torch.cuda.synchronize()
        assert torch.equal(packed[j * mb:(j + 1) * mb].cpu(), one.cpu()), j
