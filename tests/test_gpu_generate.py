"""GPU checks of the multi-block generation driver (bdd_generate): the
blocks it produces equal the same rounds run one by one through
bdd_block_denoise_round (each of which is checked against the oracle in
test_gpu_small / test_gpu_full), and its stopping rules follow the
block_decode pseudocode of the aitujian.cn article (section 三): a block
starts all-MASK and runs until resolved or max_steps, generation stops after
a block whose last token is EOS, and max_new_tokens bounds the output."""

import pytest
import torch

import block_diffusion_decode_amd as bdd
import workloads as W
from gpu_helpers import dims_of

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D = W.Dims("gen_bf16", T=8, H=256, E=40, K=6, I=96, I_s=64, V=5003, wdtype="bf16", w_std=0.05,
           lm_std=256 ** -0.5)
NB, STEPS = 3, 8


@pytest.fixture(scope="module")
def setup():
    x, info = W.planted_round_inputs(3, D, rounds=NB * STEPS, p=0.3, amp_pass=40.0, amp_fail=(4.0, 9.0),
                                     tag="gen")
    layers = [W.layer_weights(3, l, D, device=DEV, bias="zipf") for l in range(2)]
    w_lm = W.lm_head_weight(3, D, device=DEV, unit_rows=info["unit_rows"])
    plan = bdd.RoundPlan(dims_of(D), layers, bdd.pack_lm_head(w_lm), 0.9)
    xr = x.reshape(NB, STEPS, D.T, D.H).contiguous().to(DEV)
    # the same rounds one by one
    tok = torch.empty(D.T, dtype=torch.int32, device=DEV)
    conf = torch.empty(D.T, dtype=torch.float32, device=DEV)
    choice = torch.empty(D.T, dtype=torch.int32, device=DEV)
    ri = torch.empty(4, dtype=torch.int32, device=DEV)
    blocks, rounds = [], []
    for b in range(NB):
        tok.fill_(bdd.MASK)
        n = 0
        for r in range(STEPS):
            plan(xr[b, r], tok, conf, choice, ri)
            n += 1
            if ri.cpu().tolist()[3]:
                break
        assert ri.cpu().tolist()[3] == 1, "the stub resolves every block within T rounds"
        blocks.append(tok.cpu().clone())
        rounds.append(n)
    return plan, xr, blocks, rounds


def test_generate_matches_round_loop(setup):
    plan, xr, blocks, rounds = setup
    toks, brounds, n, stop = bdd.generate(plan, xr, max_new_tokens=NB * D.T, max_steps=STEPS, eos_token=-7)
    assert stop == "length" and n == NB * D.T
    assert brounds == rounds
    for b in range(NB):
        assert torch.equal(toks[b].cpu(), blocks[b]), b
    assert all(int(v) >= 0 for blk in blocks for v in blk)


def test_generate_stops_after_a_block_ending_in_eos(setup):
    plan, xr, blocks, rounds = setup
    eos = int(blocks[1][-1])
    # the first block whose last token is eos ends generation
    first = next(b for b in range(NB) if int(blocks[b][-1]) == eos)
    toks, brounds, n, stop = bdd.generate(plan, xr, max_new_tokens=NB * D.T, max_steps=STEPS, eos_token=eos)
    assert stop == "eos" and len(brounds) == first + 1 and n == (first + 1) * D.T
    assert brounds == rounds[:first + 1]


def test_generate_max_new_tokens_resolves_the_final_block_whole(setup):
    plan, xr, blocks, rounds = setup
    toks, brounds, n, stop = bdd.generate(plan, xr, max_new_tokens=D.T + 3, max_steps=STEPS, eos_token=-7)
    assert stop == "length" and n == D.T + 3 and len(brounds) == 2
    assert torch.equal(toks[1].cpu(), blocks[1])


def test_generate_unresolved_block_reports_unresolved(setup):
    plan, xr, blocks, rounds = setup
    # block 0 of this stub needs more than one round, so one step leaves it unresolved
    assert rounds[0] > 1
    toks, brounds, n, stop = bdd.generate(plan, xr[:, :1].contiguous(), max_new_tokens=D.T, max_steps=1,
                                          eos_token=-7)
    assert stop == "unresolved" and brounds == [1]
    assert (toks[0] == bdd.MASK).any()


def test_generate_rejects_requests_beyond_the_token_bound(setup):
    plan, xr, blocks, rounds = setup
    with pytest.raises(bdd.BddError) as e:
        bdd.generate(plan, xr, max_new_tokens=1, max_steps=STEPS, eos_token=-7, prompt_len=131072 - D.T + 1)
    assert e.value.status == -1
