"""LowConfidence commit statistics on the GPU over 200 blocks.

[P1] aitujian.cn article on Clover-35B-A3B-Preview, section 三 (the commit rule
and its toy fallback model): in every round the masked positions whose
confidence reaches the threshold are written; when none does, the single most
confident masked position is written instead.  With m masked positions that
pass independently with probability p, a round falls back with probability
(1 - p)^m.

Each block is resolved from all-MASK through the LM head + commit entry on the
seeded stub (a passing position's planted logit gives confidence >= 0.99 at
this vocabulary, a failing one <= 0.75, so the planted pattern decides every
pass), and every round is checked against the rule:
- the written positions are exactly the planted passes among the masked ones,
  or, when there are none, the masked position of highest reported confidence
  (lowest position on ties);
- the written tokens are the planted ones and round_info agrees;
- the number of fallback rounds is within 4 standard deviations of
  sum_r (1 - p)^{m_r} over the rounds played (the indicators minus their
  conditional probabilities form a martingale), and the first-round fallback
  count is within 4 standard deviations of 200 (1 - p)^32.
"""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BLOCKS, T, TAU = 200, 32, 0.95
D = W.Dims("lm_stats", T=T, H=256, E=1, K=1, I=32, I_s=0, V=5003, wdtype="bf16", w_std=0.02,
           lm_std=256 ** -0.5)


@pytest.mark.parametrize("p", [0.05, 0.2])
def test_fallback_frequency_over_200_blocks(p):
    seed = 11
    # one stub round per (block, round): block b plays rounds b*T .. b*T + T - 1
    h, info = W.lmhead_stub_inputs(seed, D, BLOCKS * T, p=p, pass_logit=(14.5, 16.5), fail_logit=(6.0, 10.0))
    passed, vocab = info["passed"], info["vocab"]
    lm = bdd.pack_lm_head(W.lm_head_weight(seed, D, device=DEV))
    ws = torch.empty(bdd.lmhead_workspace_bytes(T, D.H, D.V), dtype=torch.uint8, device=DEV)
    hd = h.to(DEV)
    fb_rounds = first_fb = rounds = 0
    expect = var = 0.0
    for b in range(BLOCKS):
        tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=DEV)
        masked = np.ones(T, dtype=bool)
        for r in range(T):
            row = b * T + r
            q = (1.0 - p) ** int(masked.sum())
            expect += q
            var += q * (1.0 - q)
            conf, choice, ri = bdd.lmhead_confidence_commit(hd[row], lm, tok, threshold=TAU, ws=ws)
            info_r = ri.cpu().tolist()
            got = tok.cpu().numpy()
            c = conf.cpu().numpy()
            # the planted pattern decides every pass
            assert np.array_equal(c[masked] >= TAU, passed[row][masked]), (b, r)
            want = masked & passed[row]
            if want.any():
                assert info_r[1] == 0, (b, r, info_r)
            else:
                best = np.where(masked, c, -np.inf)
                i = int(np.flatnonzero(best == best.max())[0])
                want = np.zeros(T, dtype=bool)
                want[i] = True
                assert info_r[1] == 1, (b, r, info_r)
                fb_rounds += 1
                first_fb += int(r == 0)
            newly = masked & (got != bdd.MASK)
            assert np.array_equal(newly, want), (b, r, np.flatnonzero(newly), np.flatnonzero(want))
            assert np.array_equal(got[want], vocab[row][want]), (b, r)
            masked &= ~want
            assert info_r[0] == int(want.sum()) and info_r[2] == int(masked.sum()), (b, r, info_r)
            rounds += 1
            if not masked.any():
                assert info_r[3] == 1
                break
        assert not masked.any(), f"block {b} not resolved within {T} rounds"
    sd = var ** 0.5
    q0 = (1.0 - p) ** T
    sd0 = (BLOCKS * q0 * (1.0 - q0)) ** 0.5
    print(f"p={p}: {rounds} rounds over {BLOCKS} blocks ({rounds / BLOCKS:.2f} per block); fallback rounds "
          f"{fb_rounds} (expected {expect:.1f} +- {sd:.1f}); first-round fallbacks {first_fb} "
          f"(expected {BLOCKS * q0:.1f} +- {sd0:.1f})")
    assert abs(fb_rounds - expect) <= 4.0 * sd + 1.0
    assert abs(first_fb - BLOCKS * q0) <= 4.0 * sd0 + 1.0
