"""GPU check of bdd_block_denoise_round_noalloc (the round without a
workspace, on the library's static per-GPU scratch): through the C ABI, its
outputs equal those of bdd_block_denoise_round on the same inputs, bit for
bit (the same kernels in the same order), for calls in a row, each on a
smaller block or layer stack than the one before (64, 32, then 13 positions)."""

import numpy as np
import pytest
import torch

import block_diffusion_decode_amd as bdd
import workloads as W
from gpu_helpers import dims_of

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

WIDE = W.Dims("noalloc_wide", T=64, H=1024, E=64, K=8, I=256, I_s=256, V=20011, wdtype="bf16", w_std=0.03,
              lm_std=1024 ** -0.5)
BIG = W.Dims("noalloc_big", T=32, H=1024, E=64, K=8, I=256, I_s=256, V=20011, wdtype="bf16", w_std=0.03,
             lm_std=1024 ** -0.5)
SMALL = W.Dims("noalloc_small", T=13, H=256, E=40, K=6, I=96, I_s=64, V=5003, wdtype="bf16", w_std=0.05,
               lm_std=256 ** -0.5)


def _outputs(d, L):
    return {"tok": torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=DEV),
            "conf": torch.empty(d.T, dtype=torch.float32, device=DEV),
            "choice": torch.empty(d.T, dtype=torch.int32, device=DEV),
            "ri": torch.empty(4, dtype=torch.int32, device=DEV),
            "topk": torch.empty((L, d.T, d.K), dtype=torch.int32, device=DEV),
            "nd": torch.empty(L, dtype=torch.int32, device=DEV),
            "hhat": torch.empty((d.T, d.H), dtype=d.torch_wdtype, device=DEV)}


def _case(d, seed, L, top_p, rounds):
    x, info = W.planted_round_inputs(seed, d, rounds=rounds, p=0.4, amp_pass=40.0, amp_fail=(6.0, 16.0))
    layers = [W.layer_weights(seed, l, d, device=DEV, bias="zipf") for l in range(L)]
    w_lm = W.lm_head_weight(seed, d, device=DEV, unit_rows=info["unit_rows"])
    return x.to(DEV), bdd.RoundPlan(dims_of(d), layers, bdd.pack_lm_head(w_lm), top_p, 0.95)


def _run_both(d, x, plan, L, rounds):
    """Rounds of a resolve through both entry points; every output compared."""
    a, b = _outputs(d, L), _outputs(d, L)
    for r in range(rounds):
        plan(x[r], a["tok"], a["conf"], a["choice"], a["ri"], a["topk"], a["nd"], a["hhat"])
        bdd.block_denoise_round_noalloc(plan, x[r], b["tok"], b["conf"], b["choice"], b["ri"], b["topk"], b["nd"],
                                        b["hhat"])
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k], b[k]), (d.name, r, k)
        if a["ri"][3].item():
            break
    return int((a["tok"] >= 0).sum())


def test_noalloc_round_matches_the_workspace_round_twice_in_a_row():
    print("noalloc: wide case (T 64, H 1024, 2 layers, coreset 0.9)", flush=True)
    x0, plan0 = _case(WIDE, 2, 2, 0.9, 3)
    assert bdd.round_workspace_bytes(plan0.d, plan0.V) <= bdd.NOALLOC_SCRATCH_BYTES
    n0 = _run_both(WIDE, x0, plan0, 2, 3)
    print("noalloc: big case (T 32, H 1024, 2 layers, coreset 0.9)", flush=True)
    x, plan = _case(BIG, 0, 2, 0.9, 4)
    assert bdd.round_workspace_bytes(plan.d, plan.V) <= bdd.NOALLOC_SCRATCH_BYTES
    n1 = _run_both(BIG, x, plan, 2, 4)
    print("noalloc: small case (T 13, H 256, 1 layer, no coreset)", flush=True)
    x2, plan2 = _case(SMALL, 1, 1, 1.0, 3)
    n2 = _run_both(SMALL, x2, plan2, 1, 3)
    assert n0 > 0 and n1 > 0 and n2 > 0
