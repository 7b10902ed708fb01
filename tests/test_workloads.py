"""CPU tests of the seeded input generators (shared by both sides)."""

import math

import numpy as np
import torch

import oracle as O
import workloads as W
from workloads import gen as G


def _lowbias32_py(x: int) -> int:
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def test_mix32_matches_python_integers():
    r = np.random.default_rng(0)
    xs = [0, 1, 2, 0xFFFFFFFF, 0x80000000] + r.integers(0, 2 ** 32, size=500).tolist()
    got = G._mix32(torch.tensor(xs, dtype=torch.int64)).tolist()
    assert got == [_lowbias32_py(int(x)) for x in xs]


def test_counter_words_range():
    w = G.counter_words(W.key_of(1, "x"), torch.arange(0, 100000, dtype=torch.int64))
    assert int(w.min()) >= 0 and int(w.max()) < 2 ** 32
    # roughly uniform bits
    assert abs(float((w & 1).double().mean()) - 0.5) < 0.01


def test_normal_subrange_and_determinism():
    k = W.key_of(7, "t")
    a = W.counter_normal(k, 50000, 0.02)
    b = W.counter_normal(k, 50000, 0.02)
    c = W.counter_normal(k, 1000, 0.02, start=12345)
    assert torch.equal(a, b) and torch.equal(a[12345:13345], c)
    assert not torch.equal(a, W.counter_normal(W.key_of(8, "t"), 50000, 0.02))


def test_normal_moments_and_support():
    x = W.counter_normal(W.key_of(3, "m"), 400000, 1.0).double()
    assert abs(float(x.mean())) < 0.01
    assert abs(float(x.std()) - 1.0) < 0.01
    assert float(x.abs().max()) <= 2 * math.sqrt(3) + 1e-6
    # fourth moment of the Irwin-Hall(4) law at unit variance: 3 - 6/(5*4) = 2.7
    assert abs(float((x ** 4).mean()) - 2.7) < 0.05


def test_uniform_range():
    u = W.counter_uniform(W.key_of(3, "u"), 100000)
    assert float(u.min()) > 0 and float(u.max()) < 1 and abs(float(u.mean()) - 0.5) < 0.01


def test_bf16_storage_matches_oracle_rounding():
    x = W.counter_normal(W.key_of(5, "b"), 100000, 0.02)
    assert np.array_equal(x.to(torch.bfloat16).double().numpy(), O.bf16_round(x.double().numpy()))


def test_layer_subset_equals_full():
    d = W.C0
    full = W.layer_weights(0, 0, d)
    sub = W.layer_weights(0, 0, d, experts=[3, 11])
    assert torch.equal(full["w_gate_up"][3], sub["w_gate_up"][0])
    assert torch.equal(full["w_down"][11], sub["w_down"][1])
    assert torch.equal(full["w_router"], sub["w_router"])
    assert full["w_gate_up"].dtype == torch.float32
    assert abs(float(full["w_gate_up"].std()) - 0.02) < 0.001


def test_lm_rows_equal_full_weight():
    d = W.C0
    w = W.lm_head_weight(1, d, unit_rows=[5, 900])
    rows = W.lm_head_rows(1, d, [5, 17, 900], unit_rows=[5, 900])
    assert torch.equal(w[[5, 17, 900]], rows)
    assert abs(float(torch.linalg.vector_norm(w[5].double())) - 1.0) < 1e-6


def test_zipf_bias_is_rank_law():
    b = W.zipf_router_bias(0, 0, 256, 1.1, 1.0).double().numpy()
    ranks = np.exp(-b / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 257), rtol=1e-5)


def test_lmhead_stub_plants_target_logits():
    d = W.Dims("small", T=8, H=256, E=4, K=2, I=8, I_s=8, V=3000, wdtype="bf16",
               w_std=0.02, lm_std=256 ** -0.5)
    h, info = W.lmhead_stub_inputs(0, d, rounds=3, p=0.5)
    assert h.shape == (3, 8, 256) and h.dtype == torch.bfloat16
    rows = W.lm_head_rows(0, d, info["vocab"].ravel().tolist()).double()
    z = (h.double().reshape(-1, 256) * rows).sum(1).numpy().reshape(3, 8)
    assert np.allclose(z, info["target_logit"], atol=0.05)
    assert np.all(np.where(info["passed"], z > 18, z < 14.1))


def test_planted_round_inputs_shape():
    x, info = W.planted_round_inputs(0, W.C0, rounds=2, p=0.4, amp_pass=32.0, amp_fail=(3.0, 6.0))
    assert x.shape == (2, 8, 256) and x.dtype == torch.float32
    assert len(info["unit_rows"]) >= 1
