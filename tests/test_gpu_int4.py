"""GPU parity of the 4-bit weight-only LM head against the CPU oracle.

[P3] 10100.com article on Clover-35B-A3B-Preview, part 03 (memory and
quantisation): the model is deployed with INT4 weights; the pages give no
format.  The format read here: two 4-bit codes per byte (low nibble = even
column), code n standing for n - 8, one bf16 scale per row and 128-column
group.  The oracle dequantises in float64 and runs its LM head on the result;
the GPU takes the codes through bdd_lmhead_pack_int4 and
bdd_lmhead_confidence_commit(dtype = BDD_INT4).  Tolerances are those of the
bf16 LM head: the GPU forms each group's sum from exact bf16 products
accumulated in fp32.
"""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W
from gpu_helpers import BAND, TAU, Int4Rows, assert_close, commit_in_band, f64, top2_gap

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dims(T, H, V):
    return W.Dims("lm_int4", T=T, H=H, E=1, K=1, I=32, I_s=0, V=V, wdtype="bf16", w_std=0.02, lm_std=H ** -0.5)


def _planted(seed, d, codes, scales, R, p, pass_amp=(14.5, 16.5), fail_amp=(6.0, 10.0)):
    """Hidden states with a peak planted along the code pattern u = n - 8 of a
    random token per position, h = noise + a u with a = amp / (mean scale *
    |u|^2), so that token's logit is near amp: 14.5-16.5 (pass) with
    probability p, else 6-10, over N(0, 0.3) noise (the oracle decides every
    outcome)."""
    rng = np.random.default_rng(seed)
    c = codes.cpu().numpy()
    sm = scales.float().cpu().numpy().mean(axis=1)
    h = 0.3 * rng.standard_normal((R, d.T, d.H))
    for r in range(R):
        for t in range(d.T):
            v = int(rng.integers(d.V))
            u = np.empty(d.H)
            u[0::2] = (c[v] & 15).astype(np.float64) - 8.0
            u[1::2] = (c[v] >> 4).astype(np.float64) - 8.0
            amp = rng.uniform(*pass_amp) if rng.random() < p else rng.uniform(*fail_amp)
            h[r, t] += amp / (sm[v] * max(float(u @ u), 1.0)) * u
    return torch.tensor(h, dtype=torch.float32).to(torch.bfloat16)


def _clear_resolve(h, wl, rounds):
    """True when the oracle's resolve over these inputs has no commit or
    argmax decision inside the margin band in any round it runs."""
    tok = np.full(h.shape[1], O.MASK)
    for r in range(rounds):
        c, ch, z = O.lm_head_confidence(f64(h[r]), wl)
        if commit_in_band(tok, c) or (top2_gap(z)[tok == O.MASK] < BAND).any():
            return False
        tok, _, _, _, done = O.commit(tok, c, ch, TAU)
        if done:
            return True
    return True


def test_int4_pack_layout_matches_the_stated_layout():
    d = _dims(4, 256, 37)                       # 3 tiles, the last with 11 padding rows
    codes, scales = W.lm_head_int4(3, d, device=DEV)
    lm = bdd.pack_lm_head_int4(codes, scales)
    torch.cuda.synchronize()
    got = lm.packed.cpu().numpy()
    c = codes.cpu().numpy()
    G, tiles = d.H // 128, (d.V + 15) // 16
    nib = np.zeros((tiles * 16, d.H), np.uint32)
    nib[:d.V, 0::2] = c & 15
    nib[:d.V, 1::2] = c >> 4
    want = np.zeros(tiles * G * 64 * 4, np.uint32)
    for tau in range(tiles):
        for grp in range(G):
            for lane in range(64):
                li, g = lane & 15, lane >> 4
                for kk in range(4):
                    word = 0
                    for e in range(8):
                        word |= int(nib[tau * 16 + li, (4 * grp + kk) * 32 + 8 * g + e]) << (4 * (e // 2) + 16 * (e % 2))
                    want[((tau * G + grp) * 64 + lane) * 4 + kk] = word
    code_bytes = tiles * 8 * d.H
    assert np.array_equal(got[:code_bytes].view(np.uint32), want)
    s = scales.view(torch.int16).cpu().numpy().astype(np.uint16)
    ws = np.zeros((tiles, G, 16), np.uint16)
    for v in range(d.V):
        ws[v // 16, :, v % 16] = s[v]
    assert np.array_equal(got[code_bytes:].view(np.uint16), ws.ravel())


@pytest.mark.parametrize("T,V,seed", [(7, 5003, 0), (32, 5003, 1), (1, 4099, 2), (16, 16, 3), (64, 5003, 4),
                                      (40, 4099, 5)])
def test_int4_lmhead_commit_multiround(T, V, seed):
    d = _dims(T, 384, V)                        # 3 groups of 128 columns
    codes, scales = W.lm_head_int4(seed, d)
    wl = Int4Rows(codes, scales)
    R = 8
    # the first draw of planted inputs (seed counting up by 1000) whose oracle
    # resolve has no commit or argmax decision inside the margin band
    for s in range(seed, seed + 20000, 1000):
        h = _planted(s, d, codes, scales, R, p=0.3)
        if _clear_resolve(h, wl, R):
            break
    else:
        pytest.fail("no draw with every commit outside the margin band")
    lm = bdd.pack_lm_head_int4(codes.to(DEV), scales.to(DEV))
    tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=DEV)
    tok_ref = np.full(T, O.MASK)
    done = False
    for r in range(R):
        hr = h[r].contiguous().to(DEV)
        prev = tok.cpu().numpy().copy()
        conf, choice, ri = bdd.lmhead_confidence_commit(hr, lm, tok)
        torch.cuda.synchronize()
        c_ref, ch_ref, z = O.lm_head_confidence(f64(hr), wl)
        assert_close(conf.cpu().numpy(), c_ref, f"conf round {r}")
        ok = top2_gap(z) >= BAND
        assert np.array_equal(choice.cpu().numpy()[ok], ch_ref[ok])
        assert not commit_in_band(tok_ref, c_ref)
        tok_ref, acc, fb, left, done = O.commit(tok_ref, c_ref, ch_ref, TAU)
        got = tok.cpu().numpy()
        assert np.array_equal(got, tok_ref), (r, got, tok_ref)
        assert ri.cpu().tolist() == [len(acc), int(fb), left, int(done)]
        assert np.all(got[prev != O.MASK] == prev[prev != O.MASK])
        if done:
            break
    assert done or T > R


def test_int4_zero_codes_and_extreme_codes():
    # all codes 8: every weight 0, conf = 1/V (the logits are all equal in the
    # oracle, so the argmax is a tie, which the margin band leaves uncompared);
    # then codes 0 / 15 (-8 s, +7 s) on one row
    d = _dims(3, 256, 777)
    codes = torch.full((d.V, d.H // 2), 0x88, dtype=torch.uint8, device=DEV)
    scales = torch.full((d.V, d.H // 128), 0.01, dtype=torch.bfloat16, device=DEV)
    h = W.counter_normal(W.key_of(4, "h"), d.T * d.H, 1.0).to(torch.bfloat16).reshape(d.T, d.H).to(DEV)
    tok = torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=DEV)
    conf, choice, _ = bdd.lmhead_confidence_commit(h, bdd.pack_lm_head_int4(codes, scales), tok)
    torch.cuda.synchronize()
    assert_close(conf.cpu().numpy(), np.full(d.T, 1.0 / d.V), "conf", abs_=1e-7, rel=1e-4)
    assert ((choice.cpu().numpy() >= 0) & (choice.cpu().numpy() < d.V)).all()
    codes[500, :64] = 0xF0                      # columns 0..127: -8, +7 alternating
    codes[500, 64:] = 0x0F
    scales[500] = torch.tensor([0.5, 0.25], dtype=torch.bfloat16)
    tok = torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=DEV)
    conf, choice, _ = bdd.lmhead_confidence_commit(h, bdd.pack_lm_head_int4(codes, scales), tok)
    torch.cuda.synchronize()
    c_ref, ch_ref, z = O.lm_head_confidence(f64(h), Int4Rows(codes, scales))
    assert_close(conf.cpu().numpy(), c_ref, "conf")
    ok = top2_gap(z) >= BAND
    assert np.array_equal(choice.cpu().numpy()[ok], ch_ref[ok])


def test_int4_lmhead_full_vocabulary():
    # the Clover LM-head shape, vocabulary 248320 x hidden 2048, block 32, in
    # the launch configuration the benchmark times
    d = _dims(32, 2048, 248320)
    codes, scales = W.lm_head_int4(0, d, device=DEV)
    lm = bdd.pack_lm_head_int4(codes, scales)
    # at this vocabulary conf = 0.95 near a planted logit of 15.4: passing
    # levels 18-20 and failing ones 10-13.5 keep every commit out of the band
    h = _planted(5, d, codes, scales, 1, p=0.5, pass_amp=(18.0, 20.0), fail_amp=(10.0, 13.5))[0]
    h = h.contiguous().to(DEV)
    tok = torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=DEV)
    conf, choice, ri = bdd.lmhead_confidence_commit(h, lm, tok)
    torch.cuda.synchronize()
    c_ref, ch_ref, z = O.lm_head_confidence(f64(h), Int4Rows(codes, scales))
    assert_close(conf.cpu().numpy(), c_ref, "conf")
    ok = top2_gap(z) >= BAND
    assert ok.sum() >= d.T - 2
    assert np.array_equal(choice.cpu().numpy()[ok], ch_ref[ok])
    # (this draw's commit lies outside the margin band: checked on the CPU)
    assert not commit_in_band(np.full(d.T, O.MASK), c_ref)
    tok_ref, acc, fb, left, done = O.commit(np.full(d.T, O.MASK), c_ref, ch_ref, TAU)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
    assert ri.cpu().tolist() == [len(acc), int(fb), left, int(done)]
    print(f"full INT4 head: {int((c_ref >= TAU).sum())} of {d.T} positions pass")
