"""GPU parity of the multi-block generation driver (bdd_generate) against the
oracle's generation loop (oracle.generate: the block_decode pseudocode of the
aitujian.cn article, section 三, and the generation controls on the goremy.ai
page): blocks start all-MASK and run rounds until resolved or max_steps, a
resolved block joins the output, generation stops after a block whose last
token is EOS or once max_new_tokens are produced, and requests beyond 131072
tokens are rejected.  Each round's forward is the round of two MoE layers
(Zipf routing), final norm, LM head and commit on the stub's
input for that (block, round); the coreset has parity cases of its own and
is left out here (its cut band would be hit somewhere in ~15 rounds).  The
seed is redrawn on the CPU until no routing, argmax or commit decision of any
round lies inside a margin band, so every block is compared exactly."""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W
from gpu_helpers import BAND, commit_in_band, dims_of, f64, oracle_layer, top2_gap, topk_gap

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D = W.Dims("gen_bf16", T=8, H=256, E=40, K=6, I=96, I_s=64, V=5003, wdtype="bf16", w_std=0.05,
           lm_std=256 ** -0.5)
NB, STEPS, TOP_P, TAU = 3, 8, 1.0, 0.95


class _Forward:
    """The oracle round on the stub input of (block, round); flags any
    decision inside a margin band."""

    def __init__(self, x, layers, w_lm):
        self.x = x
        self.ol = [oracle_layer(w) for w in layers]
        self.wl = f64(w_lm)
        self.band = False

    def __call__(self, b, r, tok, prefix):
        hh, infos = O.moe_stack(self.x[b, r].double().numpy(), self.ol, D.K, TOP_P)
        for inf in infos:
            self.band |= bool((topk_gap(inf["logits"], D.K) < BAND).any())
        c, ch, z = O.lm_head_confidence(hh, self.wl)
        self.band |= commit_in_band(tok, c, TAU) or bool((top2_gap(z)[tok == O.MASK] < BAND).any())
        return c, ch


def _draw(seed):
    x, info = W.planted_round_inputs(seed, D, rounds=NB * STEPS, p=0.3, amp_pass=40.0, amp_fail=(4.0, 16.0),
                                     tag="gen")
    layers = [W.layer_weights(seed, l, D, bias="zipf") for l in range(2)]
    for w in layers:
        # router logits spread 8 times wider (a power of two: exact in bf16), so
        # that over the ~15 rounds of a generation no top-K gap falls in the band
        w["w_router"] = w["w_router"] * 8
    w_lm = W.lm_head_weight(seed, D, unit_rows=info["unit_rows"])
    return x.reshape(NB, STEPS, D.T, D.H), layers, w_lm


@pytest.fixture(scope="module")
def setup():
    for seed in range(3, 60003, 1000):
        x, layers, w_lm = _draw(seed)
        fwd = _Forward(x, layers, w_lm)
        ref = O.generate(fwd, D.T, NB * D.T, eos_token=-7, threshold=TAU, max_steps=STEPS)
        if not fwd.band and ref[2] == "length":
            break
    else:
        pytest.fail("no seed with every decision of the generation outside the margin band")
    layers = [{k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()} for w in layers]
    plan = bdd.RoundPlan(dims_of(D), layers, bdd.pack_lm_head(w_lm.to(DEV)), TOP_P, TAU)
    print(f"seed {seed}: rounds per block {[b['rounds'] for b in ref[1]]}, "
          f"fallbacks {[b['fallbacks'] for b in ref[1]]}", flush=True)
    return plan, x.contiguous().to(DEV), fwd, ref


def _compare(got, ref, nb_expect):
    toks, rounds, n, stop, fbs = got
    out, blocks, stop_ref = ref
    assert stop == stop_ref
    assert n == len(out)
    assert rounds == [b["rounds"] for b in blocks]
    assert fbs == [b["fallbacks"] for b in blocks]
    assert len(rounds) == nb_expect
    for i, blk in enumerate(blocks):
        assert toks[i].cpu().numpy().tolist() == blk["tokens"].tolist(), i
    flat = toks[:len(blocks)].cpu().numpy().ravel().tolist()
    if stop_ref != "unresolved":
        assert flat[:n] == out


@pytest.mark.parametrize("rounds_per_read", [0, 1, 3, 32])   # 32: one read per block
def test_generate_matches_the_oracle(setup, rounds_per_read):
    plan, xr, fwd, ref = setup
    got = bdd.generate(plan, xr, max_new_tokens=NB * D.T, max_steps=STEPS, eos_token=-7,
                       rounds_per_read=rounds_per_read, with_fallbacks=True)
    _compare(got, ref, NB)


def test_generate_stops_after_a_block_ending_in_eos(setup):
    plan, xr, fwd, ref = setup
    blocks = ref[1]
    eos = int(blocks[1]["tokens"][-1])
    first = next(b for b in range(NB) if int(blocks[b]["tokens"][-1]) == eos)
    want = O.generate(fwd, D.T, NB * D.T, eos_token=eos, threshold=TAU, max_steps=STEPS)
    assert want[2] == "eos" and len(want[1]) == first + 1
    got = bdd.generate(plan, xr, max_new_tokens=NB * D.T, max_steps=STEPS, eos_token=eos, with_fallbacks=True)
    _compare(got, want, first + 1)


def test_generate_max_new_tokens_resolves_the_final_block_whole(setup):
    plan, xr, fwd, ref = setup
    want = O.generate(fwd, D.T, D.T + 3, eos_token=-7, threshold=TAU, max_steps=STEPS)
    got = bdd.generate(plan, xr, max_new_tokens=D.T + 3, max_steps=STEPS, eos_token=-7, with_fallbacks=True)
    assert got[2] == D.T + 3 and got[3] == "length"
    _compare(got, want, 2)


def test_generate_unresolved_block_reports_unresolved(setup):
    plan, xr, fwd, ref = setup
    # block 0 of this draw needs more than one round, so one step leaves it unresolved
    assert ref[1][0]["rounds"] > 1
    want = O.generate(fwd, D.T, D.T, eos_token=-7, threshold=TAU, max_steps=1)
    assert want[2] == "unresolved"
    got = bdd.generate(plan, xr[:, :1].contiguous(), max_new_tokens=D.T, max_steps=1, eos_token=-7,
                       with_fallbacks=True)
    _compare(got, want, 1)
    assert (got[0][0] == bdd.MASK).any()


def test_generate_rejects_requests_beyond_the_token_bound(setup):
    plan, xr, fwd, ref = setup
    with pytest.raises(bdd.BddError) as e:
        bdd.generate(plan, xr, max_new_tokens=1, max_steps=STEPS, eos_token=-7, prompt_len=131072 - D.T + 1)
    assert e.value.status == -1
    with pytest.raises(ValueError):
        O.generate(fwd, D.T, 1, eos_token=-7, prompt=range(131072 - D.T + 1))
