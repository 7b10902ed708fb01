"""Pins of the CPU oracle to things other than itself: hand-computed values,
closed forms, library routines (scipy, torch, pure-Python math), brute force
on tiny inputs, invariants the pages state, and the toy fallback model."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# bf16 storage rounding
# ---------------------------------------------------------------------------

def test_bf16_hand_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even keep 1.
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,
        -(1.0 + 3 * 2.0 ** -8): -(1.0 + 2.0 ** -6),
        0.1: 205.0 / 2048.0,          # 0x3DCD
        3.0: 3.0,
        255.5: 256.0,                 # 255.5 = 1.99609375 * 2^7 -> rounds up
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.bf16_round(np.array([x]))[0] == want, x


def test_bf16_matches_torch_conversion():
    x = torch.randn(200000, generator=torch.Generator().manual_seed(3)) * 7.0
    x = torch.cat([x, torch.tensor([1e-30, -1e-20, 65504.0, 3.4e37])])
    want = x.to(torch.bfloat16).double().numpy()
    got = O.bf16_round(x.double().numpy())
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# RMSNorm, silu, SwiGLU
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    c = 2.5
    out = O.rmsnorm(np.full((1, 64), c))
    assert np.allclose(out, c / math.sqrt(c * c + 1e-6), rtol=0, atol=1e-15)
    out = O.rmsnorm(np.array([[3.0, 4.0]]))
    assert np.allclose(out, np.array([[3.0, 4.0]]) / math.sqrt(12.5 + 1e-6), rtol=0, atol=1e-15)
    # unit RMS of the output for inputs far above eps
    h = RNG.normal(size=(5, 300)) * 10
    r = np.sqrt(np.mean(O.rmsnorm(h) ** 2, axis=1))
    assert np.allclose(r, 1.0, atol=1e-8)


def test_silu_values():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    assert abs(O.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-15
    z = RNG.normal(size=100) * 5
    # silu(z) - silu(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    assert np.allclose(O.silu(z) - O.silu(-z), z, atol=1e-12)
    assert np.allclose(O.silu(z), z * sps.expit(z), atol=1e-12)


def test_swiglu_hand_example():
    # gate row [0.5, 0.25] -> g = 1; up row [1, -0.25] -> u = 0.5;
    # a = silu(1) * 0.5; down [[2], [-1]] -> y = [2a, -a].
    x = np.array([[1.0, 2.0]])
    gu = np.array([[0.5, 0.25], [1.0, -0.25]])
    dn = np.array([[2.0], [-1.0]])
    a = 0.7310585786300049 * 0.5
    y = O.swiglu_expert(x, gu, dn)
    assert np.allclose(y, [[2 * a, -a]], rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def _router_from_logits(logits):
    """A router whose logits equal ``logits`` exactly: xhat = identity rows,
    W_r = logits^T, zero bias."""
    T, E = logits.shape
    return np.eye(T), logits.T.copy(), np.zeros(E)


def test_route_brute_force_small():
    for trial in range(200):
        T, E, K = 3, int(RNG.integers(2, 8)), 0
        K = int(RNG.integers(1, E + 1))
        l = RNG.integers(-3, 4, size=(T, E)).astype(np.float64)  # many ties
        x, wr, b = _router_from_logits(l)
        ll, p, idx, w = O.route(x, wr, b, K)
        for t in range(T):
            sel = list(idx[t])
            rest = [e for e in range(E) if e not in sel]
            assert len(set(sel)) == K
            # every selected logit >= every unselected one
            assert all(l[t, a] >= l[t, c] for a in sel for c in rest)
            # among equal logits on the boundary, the lower id wins
            for a in sel:
                for c in rest:
                    if l[t, a] == l[t, c]:
                        assert a < c
            assert np.allclose(p[t], sps.softmax(l[t]), atol=1e-15)
            assert np.allclose(w[t], sps.softmax(l[t, sel]), atol=1e-14)
            assert abs(w[t].sum() - 1) < 1e-14


def test_route_two_experts_sigmoid():
    l = np.array([[0.3, -1.2]])
    x, wr, b = _router_from_logits(l)
    _, p, idx, w = O.route(x, wr, b, 1)
    assert idx[0, 0] == 0 and w[0, 0] == 1.0
    assert abs(p[0, 0] - 1 / (1 + math.exp(-1.5))) < 1e-15


def test_route_block_equals_per_token():
    # block_size 1 reduces to per-token routing: each row routed alone
    # equals the same row routed inside the block.
    H, E, K, T = 24, 16, 4, 6
    x = RNG.normal(size=(T, H)); wr = RNG.normal(size=(E, H)); b = RNG.normal(size=E)
    _, p, idx, w = O.route(x, wr, b, K)
    for t in range(T):
        _, p1, i1, w1 = O.route(x[t:t + 1], wr, b, K)
        assert np.array_equal(i1[0], idx[t]) and np.allclose(w1[0], w[t]) and np.allclose(p1[0], p[t])


def test_route_all_experts_uniform():
    T, E = 3, 8
    x, wr, b = _router_from_logits(np.zeros((T, E)))
    _, p, idx, w = O.route(x, wr, b, E)
    assert np.allclose(w, 1.0 / E) and np.array_equal(idx, np.tile(np.arange(E), (T, 1)))


# ---------------------------------------------------------------------------
# coreset
# ---------------------------------------------------------------------------

def _random_routing(T, E, K, scale=1.0, bias=None):
    l = RNG.normal(size=(T, E)) * scale + (0 if bias is None else bias)
    x, wr, b = _router_from_logits(l)
    return O.route(x, wr, b, K)


def test_coreset_hand_example():
    # 2 tokens, 4 experts, top-2.  p rows chosen directly:
    p = np.array([[0.5, 0.3, 0.15, 0.05], [0.1, 0.6, 0.25, 0.05]])
    idx = np.array([[0, 1], [1, 2]])
    # mass: e0 0.5, e1 0.3 + 0.6 = 0.9, e2 0.25, e3 0 -> total 1.65
    members, mass, order = O.coreset_select(p, idx, 0.5)
    assert np.allclose(mass, [0.5, 0.9, 0.25, 0.0])
    assert list(members) == [1]                 # 0.9 >= 0.825
    members, _, _ = O.coreset_select(p, idx, 0.6)
    assert list(members) == [0, 1]              # 0.9 < 0.99 <= 1.4
    members, _, _ = O.coreset_select(p, idx, 1.0)
    assert list(members) == [0, 1, 2]           # every expert with mass


def test_coreset_identity_at_top_p_one():
    for _ in range(50):
        T, E, K = int(RNG.integers(1, 9)), 16, 4
        l, p, idx, w = _random_routing(T, E, K)
        members, _, _ = O.coreset_select(p, idx, 1.0)
        assert set(members) == set(idx.ravel().tolist())
        i2, w2 = O.reroute(l, p, members, K)
        assert np.array_equal(i2, idx) and np.allclose(w2, w, atol=1e-15)


def test_coreset_coverage_minimality_nesting():
    for _ in range(100):
        T, E, K = 8, 16, 4
        bias = -1.1 * np.log(RNG.permutation(E) + 1.0)
        l, p, idx, w = _random_routing(T, E, K, bias=bias)
        prev = None
        for tp in (0.3, 0.5, 0.7, 0.9, 1.0):
            members, mass, order = O.coreset_select(p, idx, tp)
            M = mass.sum()
            assert len(members) >= 1
            assert mass[members].sum() >= tp * M * (1 - 1e-12)
            ranked = [e for e in order if e in set(members)]
            if len(members) > 1:
                assert mass[ranked[:-1]].sum() < tp * M
            if prev is not None:
                assert set(prev) <= set(members)
            prev = members


def test_coreset_brute_force_minimal_size():
    for _ in range(40):
        T, E, K = 4, 9, 3
        l, p, idx, w = _random_routing(T, E, K, scale=2.0)
        tp = float(RNG.uniform(0.2, 0.95))
        members, mass, _ = O.coreset_select(p, idx, tp)
        M = mass.sum()
        best = None
        for r in range(1, E + 1):
            if any(mass[list(c)].sum() >= tp * M for c in itertools.combinations(range(E), r)):
                best = r
                break
        assert len(members) == best


def test_reroute_inside_small_coreset():
    T, E, K = 5, 12, 4
    l, p, idx, w = _random_routing(T, E, K)
    members = np.array([2, 7])
    i2, w2 = O.reroute(l, p, members, K)
    assert i2.shape == (T, 2)
    for t in range(T):
        assert set(i2[t]) == {2, 7}
        assert np.allclose(w2[t], sps.softmax(l[t, i2[t]]), atol=1e-14)


# ---------------------------------------------------------------------------
# MoE layer
# ---------------------------------------------------------------------------

def _layer(E, H, I, seed=0, same=False, zero_down=False):
    r = np.random.default_rng(seed)
    gu0 = r.normal(size=(2 * I, H)) * 0.2
    dn0 = r.normal(size=(H, I)) * 0.2
    ex = {}
    for e in range(E):
        gu = gu0 if same else r.normal(size=(2 * I, H)) * 0.2
        dn = dn0 if same else r.normal(size=(H, I)) * 0.2
        ex[e] = (gu, np.zeros_like(dn) if zero_down else dn)
    return {"w_router": r.normal(size=(E, H)), "router_bias": r.normal(size=E) * 0.1,
            "ws_gate_up": r.normal(size=(2 * I, H)) * 0.2, "ws_down": r.normal(size=(H, I)) * 0.2,
            "experts": ex}


def test_moe_identical_experts_ignore_routing():
    E, H, I, K, T = 6, 10, 5, 3, 4
    L = _layer(E, H, I, same=True)
    x = RNG.normal(size=(T, H))
    y, _ = O.moe_layer(x, L, K)
    gu, dn = L["experts"][0]
    want = O.swiglu_expert(x, gu, dn) + O.swiglu_expert(x, L["ws_gate_up"], L["ws_down"])
    assert np.allclose(y, want, atol=1e-12)


def test_moe_zero_down_is_shared_only_and_linear():
    E, H, I, K, T = 6, 10, 5, 3, 4
    x = RNG.normal(size=(T, H))
    L0 = _layer(E, H, I, seed=4, zero_down=True)
    y0, _ = O.moe_layer(x, L0, K)
    assert np.allclose(y0, O.swiglu_expert(x, L0["ws_gate_up"], L0["ws_down"]), atol=1e-13)
    L = _layer(E, H, I, seed=4)
    y1, _ = O.moe_layer(x, L, K)
    L2 = dict(L, experts={e: (g, 2 * d) for e, (g, d) in L["experts"].items()})
    y2, _ = O.moe_layer(x, L2, K)
    assert np.allclose(y2 - y0, 2 * (y1 - y0), atol=1e-12)


def test_moe_hand_example_single_expert():
    # E=2, K=1: router always picks expert 1 with weight 1; shared expert zero.
    x = np.array([[1.0, 2.0]])
    gu = np.array([[0.5, 0.25], [1.0, -0.25]]); dn = np.array([[2.0], [-1.0]])
    L = {"w_router": np.array([[0.0, 0.0], [1.0, 1.0]]), "router_bias": np.zeros(2),
         "ws_gate_up": np.zeros((2, 2)), "ws_down": np.zeros((2, 1)),
         "experts": {0: (np.zeros((2, 2)), np.zeros((2, 1))), 1: (gu, dn)}}
    y, info = O.moe_layer(x, L, 1)
    a = 0.7310585786300049 * 0.5
    assert info["union"] == [1]
    assert np.allclose(y, [[2 * a, -a]], atol=1e-15)


def test_moe_uniform_router_all_experts():
    E, H, I, T = 5, 8, 4, 3
    L = _layer(E, H, I, seed=9)
    L["w_router"] = np.zeros((E, H)); L["router_bias"] = np.zeros(E)
    x = RNG.normal(size=(T, H))
    y, _ = O.moe_layer(x, L, E)
    want = O.swiglu_expert(x, L["ws_gate_up"], L["ws_down"])
    for e in range(E):
        want = want + O.swiglu_expert(x, *L["experts"][e]) / E
    assert np.allclose(y, want, atol=1e-12)


def test_moe_block_equals_per_token_without_coreset():
    E, H, I, K, T = 8, 12, 6, 2, 5
    L = _layer(E, H, I, seed=2)
    x = RNG.normal(size=(T, H))
    y, _ = O.moe_layer(x, L, K)
    for t in range(T):
        y1, _ = O.moe_layer(x[t:t + 1], L, K)
        assert np.allclose(y1[0], y[t], atol=1e-13)


def test_moe_coreset_restricts_union():
    E, H, I, K, T = 16, 12, 6, 4, 8
    L = _layer(E, H, I, seed=5)
    x = RNG.normal(size=(T, H)) * 3
    y1, i1 = O.moe_layer(x, L, K, top_p=1.0)
    y7, i7 = O.moe_layer(x, L, K, top_p=0.7)
    assert set(i7["union"]) <= set(i7["coreset"].tolist())
    assert len(i7["union"]) <= len(i1["union"])


def test_coreset_equal_masses_at_the_cut_keep_the_lower_id():
    # 2 positions, 4 experts, top-2; probabilities exact in binary.
    #   position 0: p = [0.5, 0.0625, 0.125, 0.3125] -> picks {0, 3}
    #   position 1: p = [0.5, 0.3125, 0.125, 0.0625] -> picks {0, 1}
    # mass: e0 = 1.0, e1 = 0.3125, e3 = 0.3125, e2 = 0; total 1.625.
    # Ranked (mass desc, id asc): e0, e1, e3.  top_p 0.7 -> target 1.1375:
    # cum 1.0 < 1.1375 <= 1.3125, so the cut falls between the two equal
    # masses and the lower id (e1) is kept.
    p = np.array([[0.5, 0.0625, 0.125, 0.3125], [0.5, 0.3125, 0.125, 0.0625]])
    idx = np.array([[0, 3], [0, 1]])
    members, mass, order = O.coreset_select(p, idx, 0.7)
    assert list(mass) == [1.0, 0.3125, 0.0, 0.3125]
    assert list(order[:3]) == [0, 1, 3]
    assert list(members) == [0, 1]
    # the same block with the expert ids of the tied pair swapped keeps e1 again
    p2 = p[:, [0, 3, 2, 1]]
    idx2 = np.array([[0, 1], [0, 3]])
    members2, _, _ = O.coreset_select(p2, idx2, 0.7)
    assert list(members2) == [0, 1]
    # re-routing inside C = {0, 1}: position 0 now takes e0 and e1, weights
    # renormalised over them: 0.5 / 0.5625 and 0.0625 / 0.5625
    l = np.log(p)
    i2, w2 = O.reroute(l, p, members, 2)
    assert [sorted(r) for r in i2.tolist()] == [[0, 1], [0, 1]]
    assert np.allclose(w2[0], [0.5 / 0.5625, 0.0625 / 0.5625], rtol=0, atol=1e-15)


def test_reroute_equal_logits_take_the_lower_id():
    # coreset {1, 2, 5}; one position's logits: e5 = 2, e1 = e2 = 1 (equal),
    # the rest outside the coreset larger still (they must be ignored).
    l = np.array([[9.0, 1.0, 1.0, 9.0, 9.0, 2.0]])
    p = np.exp(l) / np.exp(l).sum()
    members = np.array([5, 2, 1])
    i2, w2 = O.reroute(l, p, members, 2)
    assert i2.tolist() == [[5, 1]]                    # e5 first, then the lower of the tie
    assert np.allclose(w2[0], [math.e / (math.e + 1), 1 / (math.e + 1)], rtol=0, atol=1e-15)
    i1, w1 = O.reroute(l, p, members, 1)
    assert i1.tolist() == [[5]] and w1[0, 0] == 1.0
    # all three equal: the two lowest ids
    l3 = np.array([[0.0, 3.0, 3.0, 0.0, 0.0, 3.0]])
    i3, w3 = O.reroute(l3, np.exp(l3) / np.exp(l3).sum(), members, 2)
    assert i3.tolist() == [[1, 2]] and np.allclose(w3, 0.5, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# layer stack: residual, inter-layer RMSNorm, final RMSNorm, bf16 points
# ---------------------------------------------------------------------------

def _zero_layer(E, H, I, Is):
    return {"w_router": np.zeros((E, H)), "router_bias": np.zeros(E),
            "ws_gate_up": np.zeros((2 * Is, H)), "ws_down": np.zeros((H, Is)),
            "experts": {e: (np.zeros((2 * I, H)), np.zeros((H, I))) for e in range(E)}}


def _bf16_torch(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("n_layers", [1, 2, 5])
def test_stack_of_zero_layers_is_the_final_norm(n_layers):
    # every routed and shared weight zero: each layer adds y = 0, so the
    # stack returns bf16(RMSNorm(x_in)) exactly (RMSNorm written out here,
    # bf16 by torch's conversion)
    T, H, E, K, I = 5, 48, 6, 2, 8
    x = RNG.normal(size=(T, H)) * 3.0
    layers = [_zero_layer(E, H, I, I) for _ in range(n_layers)]
    hh, infos = O.moe_stack(x, layers, K)
    want = _bf16_torch(x / np.sqrt((x * x).sum(axis=1, keepdims=True) / H + 1e-6))
    assert np.array_equal(hh, want)
    assert len(infos) == n_layers
    for inf in infos:                 # every layer saw the same normalised input
        assert np.array_equal(inf["xhat"], want)
    hh_f, _ = O.moe_stack(x, layers, K, round_bf16=False)
    assert np.allclose(hh_f, x / np.sqrt((x * x).mean(axis=1, keepdims=True) + 1e-6), rtol=0, atol=1e-15)
    # scale invariance of the normalised output (eps 0: exact for any c > 0
    # up to the last bit before bf16 rounding)
    for c in (0.25, 3.0, 1024.0):
        hc, _ = O.moe_stack(c * x, layers, K, eps=0.0)
        h1, _ = O.moe_stack(x, layers, K, eps=0.0)
        assert np.array_equal(hc, h1), c


def _hand_layers():
    # H = 2, E = 2, K = 1, I = 1, shared expert I_s = 1; weights [out][in]
    la = {"w_router": np.array([[1.0, 0.0], [0.0, 1.0]]), "router_bias": np.zeros(2),
          "ws_gate_up": np.array([[0.5, 0.5], [1.0, -1.0]]), "ws_down": np.array([[1.0], [0.5]]),
          "experts": {0: (np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([[1.0], [1.0]])),
                      1: (np.array([[0.0, 1.0], [1.0, 0.0]]), np.array([[2.0], [-1.0]]))}}
    lb = {"w_router": np.array([[0.0, 1.0], [1.0, 0.0]]), "router_bias": np.array([0.25, 0.0]),
          "ws_gate_up": np.array([[1.0, 0.0], [1.0, 0.0]]), "ws_down": np.array([[0.0], [1.0]]),
          "experts": {0: (np.array([[1.0, 1.0], [1.0, 0.0]]), np.array([[-1.0], [1.0]])),
                      1: (np.array([[1.0, -1.0], [0.0, 1.0]]), np.array([[0.5], [0.5]]))}}
    return [la, lb]


def test_stack_hand_worked_two_layers():
    # Worked by hand (50-digit decimal arithmetic, one scalar step at a time):
    # x_in rows (3, 4) and (4, -3).
    # Layer A: RMSNorm (eps 1e-6) gives (0.848528..., 1.131371...) and its
    #   mirror; stored as bf16: 0.848528 * 256 = 217.22 -> 217/256 =
    #   0.84765625; 1.131371 * 128 = 144.82 -> 145/128 = 1.1328125.
    #   Router = identity: position 0 picks expert 1, position 1 expert 0
    #   (K = 1, weight 1).  Position 0: expert 1 gate x1 = 1.1328125, up x0,
    #   a = silu(1.1328125) * 0.84765625, down (2, -1) -> (2a, -a); shared:
    #   gate 0.5 (x0 + x1), up x0 - x1, down (1, 0.5).  y0 = (1.24667617...,
    #   -0.82922482...); h = x_in + y.
    # Layer B normalises h (not y) and rounds to bf16: (1.1328125, 0.84765625)
    #   and (0.96875, -1.03125); router logits with bias (0.25, 0): position 0
    #   (1.09765625, 1.1328125) -> expert 1; position 1 (-0.78125, 0.96875)
    #   -> expert 1.
    # Final: RMSNorm of h after layer B, then bf16.
    layers = _hand_layers()
    x = np.array([[3.0, 4.0], [4.0, -3.0]])
    hh, infos = O.moe_stack(x, layers, 1)
    assert np.array_equal(infos[0]["xhat"], [[0.84765625, 1.1328125], [1.1328125, -0.84765625]])
    assert infos[0]["idx"].tolist() == [[1], [0]]
    assert np.array_equal(infos[1]["xhat"], [[1.1328125, 0.84765625], [0.96875, -1.03125]])
    assert np.allclose(infos[1]["logits"], [[1.09765625, 1.1328125], [-0.78125, 0.96875]], rtol=0, atol=1e-15)
    assert infos[1]["idx"].tolist() == [[1], [1]]
    assert np.array_equal(hh, [[1.015625, 0.98828125], [0.76953125, -1.1875]])
    # the layer outputs, from the residual stream: h_B - h_A = y_B
    yA = np.array([[1.2466761722877542, -0.8292248229677873], [-0.5750477095118931, -0.6506645820338626]])
    yB = np.array([[0.06898650733380712, 1.0395930595051959], [-0.9083219866646912, -0.2280482216198391]])
    yA_o, _ = O.moe_layer(infos[0]["xhat"], layers[0], 1)
    yB_o, _ = O.moe_layer(infos[1]["xhat"], layers[1], 1)
    assert np.allclose(yA_o, yA, rtol=0, atol=1e-14)
    assert np.allclose(yB_o, yB, rtol=0, atol=1e-14)
    # without the bf16 storage rounding: every value follows the fp64 chain
    hf, inf_f = O.moe_stack(x, layers, 1, round_bf16=False)
    assert np.allclose(inf_f[0]["xhat"], [[0.8485281034827336, 1.1313708046436448],
                                          [1.1313708046436448, -0.8485281034827336]], rtol=0, atol=1e-15)
    assert np.allclose(inf_f[1]["xhat"], [[1.1331079282161627, 0.8462069963574267],
                                          [0.9674357670102223, -1.0315366581216066]], rtol=0, atol=1e-14)
    assert np.allclose(hf, [[1.0121513503043398, 0.9876991111323001],
                            [0.7693474354809785, -1.1866357219127317]], rtol=0, atol=1e-14)


def test_stack_single_layer_hand_values():
    # the first layer alone: h = x_in + yA, then the final norm and bf16
    # (x_in + yA = (4.24667617..., 3.17077518...), (3.42495229..., -3.65066458...);
    # RMSNorm -> (1.13319..., 0.84610...) and (0.96761..., -1.03138...);
    # bf16 -> 145.05/128 -> 145/128, 216.6/256 -> 217/256, 123.85/128 -> 124/128,
    # -132.02/128 -> -132/128: the input layer B consumed in the two-layer stack)
    hh, _ = O.moe_stack(np.array([[3.0, 4.0], [4.0, -3.0]]), _hand_layers()[:1], 1)
    assert np.array_equal(hh, [[1.1328125, 0.84765625], [0.96875, -1.03125]])


# ---------------------------------------------------------------------------
# LM head confidence
# ---------------------------------------------------------------------------

def test_lmhead_all_equal_logits():
    V, H = 37, 6
    w = np.tile(RNG.normal(size=(1, H)), (V, 1))
    conf, choice, _ = O.lm_head_confidence(RNG.normal(size=(3, H)), w)
    assert np.allclose(conf, 1.0 / V, rtol=1e-14) and np.all(choice == 0)


def test_lmhead_single_peak_closed_form():
    V, H = 1000, 4
    w = np.zeros((V, H)); w[:, 0] = 1.0           # every logit = c = hhat[0]
    w[417, 1] = 1.0                                # row 417 adds hhat[1] = hp
    for c, hp in ((0.0, 3.0), (2.0, 15.87), (-1.0, 20.0)):
        hh = np.array([[c, hp, 0.0, 0.0]])
        conf, choice, _ = O.lm_head_confidence(hh, w)
        want = math.exp(hp) / (math.exp(hp) + (V - 1))
        assert abs(conf[0] - want) < 1e-14 and choice[0] == 417


def test_lmhead_matches_logsumexp_and_brute_force():
    T, H, V = 4, 7, 13
    hh = RNG.normal(size=(T, H)); w = RNG.normal(size=(V, H))
    conf, choice, z = O.lm_head_confidence(hh, w, chunk=5)
    for t in range(T):
        zt = [math.fsum(hh[t, k] * w[v, k] for k in range(H)) for v in range(V)]
        best = max(range(V), key=lambda v: (zt[v], -v))
        assert choice[t] == best
        assert abs(conf[t] - math.exp(max(zt)) / math.fsum(math.exp(a) for a in zt)) < 1e-13
        assert abs(conf[t] - math.exp(max(zt) - sps.logsumexp(zt))) < 1e-13


def test_lmhead_tie_lowest_id():
    w = np.array([[1.0], [2.0], [2.0], [0.5]])
    conf, choice, _ = O.lm_head_confidence(np.array([[1.0]]), w)
    assert choice[0] == 1


def _merge(a, b):
    """Online-softmax merge of two (max, sum of exp(z - max), argmax) partials:
    the larger max wins and the other sum is rescaled onto it; equal maxima
    add their sums and keep the lower index."""
    (m1, s1, i1), (m2, s2, i2) = a, b
    if m2 > m1:
        return m2, s1 * math.exp(m1 - m2) + s2, i2
    if m2 < m1:
        return m1, s1 + s2 * math.exp(m2 - m1), i1
    return m1, s1 + s2, min(i1, i2)


def test_online_softmax_merge_matches_direct_confidence():
    # The LM head reduces each vocabulary tile to (max, sum, argmax) and merges
    # the tiles' partials in whatever order its waves and workgroups meet them.
    # In exact arithmetic the merge is associative and commutative; in fp64 any
    # split and order must give the oracle's confidence and argmax (ties to the
    # lowest id) to 1e-12.
    V, H = 1031, 5
    hh = RNG.normal(size=(3, H)) * 2.0
    w = RNG.normal(size=(V, H))
    w[123] = w[700] = 0.0
    w[123, 0] = w[700, 0] = 10.0                      # an exact tie of two rows ...
    hh[2] = 0.0
    hh[2, 0] = 1.0                                    # ... that is position 2's maximum (10 vs N(0,1))
    conf, choice, z = O.lm_head_confidence(hh, w)
    for t in range(hh.shape[0]):
        for trial in range(6):
            cuts = np.sort(RNG.choice(np.arange(1, V), size=RNG.integers(1, 40), replace=False))
            tiles = np.split(np.arange(V), cuts)
            parts = []
            for tile in tiles:
                zt = z[t, tile]
                j = int(np.argmax(zt))                 # first maximum = lowest id in the tile
                parts.append((float(zt[j]), float(np.sum(np.exp(zt - zt[j]))), int(tile[j])))
            order = RNG.permutation(len(parts))
            acc = parts[order[0]]
            for k in order[1:]:
                acc = _merge(acc, parts[k]) if trial % 2 else _merge(parts[k], acc)
            assert abs(1.0 / acc[1] - conf[t]) <= 1e-12, (t, trial)
            assert acc[2] == choice[t], (t, trial)
    assert choice[2] == 123


# ---------------------------------------------------------------------------
# commit rule
# ---------------------------------------------------------------------------

def _check_commit_properties(tok, conf, choice, tau):
    new, acc, fb, left, done = O.commit(tok, conf, choice, tau)
    masked = [t for t in range(len(tok)) if tok[t] == O.MASK]
    committed = [t for t in range(len(tok)) if tok[t] != O.MASK]
    for t in committed:                              # never rewritten
        assert new[t] == tok[t]
    if not masked:
        assert acc == [] and done
        return
    assert len(acc) >= 1                             # always progresses
    passing = [t for t in masked if conf[t] >= tau]
    if passing:
        assert sorted(acc) == passing and not fb
    else:
        assert fb and len(acc) == 1
        i = acc[0]
        assert i in masked and all(conf[i] >= conf[t] for t in masked)
        assert all(conf[t] < conf[i] for t in masked if t < i)
    for t in acc:
        assert new[t] == choice[t]
    assert left == sum(1 for t in range(len(tok)) if new[t] == O.MASK)
    assert done == (left == 0)


def test_commit_brute_force_tiny_blocks():
    tau = 0.95
    levels = [0.3, 0.9499999, 0.95, 0.97, 0.3]
    for T in range(1, 5):
        for mask_bits in range(1 << T):
            tok = [O.MASK if (mask_bits >> t) & 1 else 100 + t for t in range(T)]
            for confs in itertools.product(levels[:4], repeat=T):
                _check_commit_properties(tok, np.array(confs), np.arange(T) + 7, tau)


def test_commit_threshold_is_inclusive():
    new, acc, fb, _, _ = O.commit([O.MASK, O.MASK], np.array([0.95, 0.2]), np.array([5, 6]), 0.95)
    assert acc == [0] and not fb and new[0] == 5


def test_commit_fallback_tie_lowest_position():
    new, acc, fb, _, _ = O.commit([7, O.MASK, O.MASK, O.MASK], np.array([0.99, 0.4, 0.6, 0.6]),
                                  np.array([1, 2, 3, 4]), 0.95)
    # position 0 is already written: its 0.99 neither commits nor blocks the fallback
    assert fb and acc == [2] and new.tolist() == [7, O.MASK, 3, O.MASK]


def test_block_size_one_is_autoregressive():
    # one position: the first round commits its argmax whatever its confidence
    for c in (0.01, 0.5, 0.99):
        tok, rounds = O.resolve_block(lambda r, tok: (np.array([c]), np.array([42])), 1)
        assert tok.tolist() == [42] and len(rounds) == 1


def test_resolve_at_most_block_size_rounds():
    T = 32
    r = np.random.default_rng(7)
    for _ in range(20):
        tok, rounds = O.resolve_block(lambda k, tok: (r.uniform(0, 0.94, T), np.arange(T)), T)
        assert len(rounds) == T and all(x["fallback"] for x in rounds) and np.all(tok != O.MASK)


# ---------------------------------------------------------------------------
# toy fallback model ([P1] section 三)
# ---------------------------------------------------------------------------

def _indep_forward(p, r, T):
    def fwd(k, tok):
        passed = r.uniform(size=T) < p
        conf = np.where(passed, 0.99, r.uniform(0.05, 0.9, size=T))
        return conf, np.arange(T)
    return fwd


def test_fallback_table_matches_page_formula():
    gold = json.load(open(os.path.join(GOLD, "fallback_toy_model.json")))
    T = gold["block_size"]
    r = np.random.default_rng(11)
    for p, want in zip(gold["p"], gold["p_no_pass"]):
        if want < 1e-3:
            assert p >= 0.2                       # "rare for p >= 0.2"
            continue
        n = 20000
        fb = 0
        for _ in range(n):
            conf, choice = _indep_forward(p, r, T)(0, None)
            _, _, f, _, _ = O.commit(np.full(T, O.MASK), conf, choice)
            fb += f
        se = math.sqrt(want * (1 - want) / n)
        assert abs(fb / n - want) < 5 * se + 1e-4, (p, fb / n, want)


def _markov_expectations(T, p):
    """Expected rounds and fallback rounds to resolve T positions when each
    masked position passes independently with probability p: from m masked,
    k ~ Bin(m, p) pass; k = 0 forces one commit."""
    ER = [0.0] * (T + 1)
    EF = [0.0] * (T + 1)
    for m in range(1, T + 1):
        pk = [math.comb(m, k) * p ** k * (1 - p) ** (m - k) for k in range(m + 1)]
        ER[m] = 1 + pk[0] * ER[m - 1] + sum(pk[k] * ER[m - k] for k in range(1, m + 1))
        EF[m] = pk[0] * (1 + EF[m - 1]) + sum(pk[k] * EF[m - k] for k in range(1, m + 1))
    return ER[T], EF[T]


@pytest.mark.parametrize("p", [0.05, 0.2, 0.5])
def test_resolve_rounds_match_markov_chain(p):
    T = 32
    r = np.random.default_rng(int(p * 1000))
    n = 3000
    rounds, fbs = [], []
    for _ in range(n):
        tok, rec = O.resolve_block(_indep_forward(p, r, T), T)
        assert np.all(tok != O.MASK)
        rounds.append(len(rec)); fbs.append(sum(x["fallback"] for x in rec))
    er, ef = _markov_expectations(T, p)
    assert abs(np.mean(rounds) - er) < 5 * np.std(rounds) / math.sqrt(n) + 1e-9, (np.mean(rounds), er)
    assert abs(np.mean(fbs) - ef) < 5 * np.std(fbs) / math.sqrt(n) + 1e-3, (np.mean(fbs), ef)


def test_page_constants_fixture():
    c = json.load(open(os.path.join(GOLD, "page_constants.json")))
    assert c["block_size"]["value"] == 32 and c["threshold"]["value"] == 0.95
    assert c["routed_experts"]["value"] == 256 and c["top_k"]["value"] == 8
    assert c["max_steps"]["value"] == 32


# ---------------------------------------------------------------------------
# 4-bit LM-head weights: two codes per byte, low nibble first, n - 8, one
# scale per row and 128-column group (the reading taken for the INT4 format)
# ---------------------------------------------------------------------------

def test_int4_dequantize_hand_example():
    # 0x8F: column 0 = 15 -> +7, column 1 = 8 -> 0; 0x10: column 2 = 0 -> -8, column 3 = 1 -> -7
    w = O.int4_dequantize(np.array([[0x8F, 0x10]], np.uint8), np.array([[0.5]]), group=4)
    assert w.tolist() == [[3.5, 0.0, -4.0, -3.5]]


def test_int4_dequantize_matches_per_element_loop():
    rng = np.random.default_rng(5)
    R, H, G = 3, 256, 128
    codes = rng.integers(0, 256, size=(R, H // 2), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.2, size=(R, H // G))
    w = O.int4_dequantize(codes, scales)
    for r in range(R):
        for c in range(H):
            byte = int(codes[r][c // 2])
            nib = byte & 15 if c % 2 == 0 else byte >> 4
            assert w[r][c] == (nib - 8) * scales[r][c // G], (r, c)


def test_int4_dequantize_group_boundary_and_extremes():
    codes = np.full((2, 128), 0x99, np.uint8)      # every nibble 9 -> +1
    codes[1, :] = 0xF0                               # even columns -8, odd columns +7
    scales = np.array([[1.0, 2.0], [0.25, 4.0]])
    w = O.int4_dequantize(codes, scales)
    assert (w[0, :128] == 1.0).all() and (w[0, 128:] == 2.0).all()
    assert (w[1, 0:128:2] == -2.0).all() and (w[1, 1:128:2] == 1.75).all()
    assert (w[1, 128::2] == -32.0).all() and (w[1, 129::2] == 28.0).all()


def test_int4_lm_head_zero_codes_give_uniform_confidence():
    # every code 8 stands for 0: all logits 0, conf = 1/V, choice = token 0
    V, H = 300, 256
    w = O.int4_dequantize(np.full((V, H // 2), 0x88, np.uint8), np.full((V, H // 128), 0.37))
    h = np.random.default_rng(1).standard_normal((3, H))
    conf, choice, _ = O.lm_head_confidence(h, w)
    assert np.allclose(conf, 1.0 / V, rtol=0, atol=1e-15) and (choice == 0).all()


# ---------------------------------------------------------------------------
# generation: blocks after blocks (aitujian.cn 三 block_decode; goremy.ai
# decoding step 6 and "What generation controls ship by default?")
# ---------------------------------------------------------------------------

def _scripted(script):
    """forward(block, round, tokens, prefix) from a table
    {(block, round): (conf list, choice list)}; records what it was given."""
    seen = []

    def forward(b, r, tok, prefix):
        seen.append((b, r, tuple(int(v) for v in tok), prefix))
        c, ch = script[(b, r)]
        return np.array(c, np.float64), np.array(ch)
    return forward, seen


def test_generate_stops_after_a_block_ending_in_eos_only():
    EOS = 7
    script = {
        # block 0: EOS at position 1 (not last): generation goes on
        (0, 0): ([0.99, 0.99, 0.99, 0.99], [5, 7, 9, 11]),
        # block 1: two rounds (positions 0, 3 pass; then a fallback on 2, then 1)
        (1, 0): ([0.97, 0.5, 0.6, 0.96], [1, 2, 3, 7]),
        (1, 1): ([0.1, 0.3, 0.8, 0.2], [0, 2, 3, 0]),
        (1, 2): ([0.0, 0.2, 0.0, 0.0], [0, 2, 0, 0]),
        # block 2 must never run
    }
    fwd, seen = _scripted(script)
    out, blocks, stop = O.generate(fwd, 4, 100, EOS, prompt=(40, 41))
    assert stop == "eos"
    assert out == [5, 7, 9, 11, 1, 2, 3, 7]
    assert [b["rounds"] for b in blocks] == [1, 3]
    assert [b["fallbacks"] for b in blocks] == [0, 2]
    # the prefix grows by whole resolved blocks; each round of a block sees
    # that block's own tokens so far
    assert [s[3] for s in seen] == [(40, 41), (40, 41, 5, 7, 9, 11), (40, 41, 5, 7, 9, 11),
                                    (40, 41, 5, 7, 9, 11)]
    assert [s[2] for s in seen[1:]] == [(-1, -1, -1, -1), (1, -1, -1, 7), (1, -1, 3, 7)]


def test_generate_max_new_tokens_cuts_but_resolves_the_final_block():
    script = {(0, 0): ([0.99] * 4, [1, 2, 3, 4]),
              (1, 0): ([0.99, 0.2, 0.99, 0.3], [5, 6, 7, 8]),
              (1, 1): ([0.0, 0.99, 0.0, 0.99], [0, 6, 0, 8])}
    fwd, seen = _scripted(script)
    out, blocks, stop = O.generate(fwd, 4, 6, eos_token=99)
    assert stop == "length" and out == [1, 2, 3, 4, 5, 6]
    assert blocks[1]["tokens"].tolist() == [5, 6, 7, 8] and blocks[1]["rounds"] == 2
    # exactly a multiple of the block: no extra block
    fwd, seen = _scripted(script)
    out, blocks, stop = O.generate(fwd, 4, 4, eos_token=99)
    assert stop == "length" and out == [1, 2, 3, 4] and len(blocks) == 1


def test_generate_unresolved_block_after_max_steps():
    script = {(0, 0): ([0.99] * 3, [1, 2, 3]),
              (1, 0): ([0.5, 0.4, 0.3], [4, 5, 6]),
              (1, 1): ([0.0, 0.4, 0.3], [4, 5, 6])}
    fwd, _ = _scripted(script)
    out, blocks, stop = O.generate(fwd, 3, 9, eos_token=99, max_steps=2)
    assert stop == "unresolved" and out == [1, 2, 3]
    assert blocks[1]["tokens"].tolist() == [4, 5, -1] and blocks[1]["rounds"] == 2


def test_generate_threshold_decides_the_commits():
    script = {(0, 0): ([0.85, 0.97, 0.5], [1, 2, 3]),
              (0, 1): ([0.0, 0.0, 0.9], [1, 2, 3]),
              (0, 2): ([0.0, 0.0, 0.9], [1, 2, 3])}
    fwd, _ = _scripted(script)
    _, blocks, _ = O.generate(fwd, 3, 3, eos_token=99, threshold=0.8)
    assert blocks[0]["rounds"] == 2 and blocks[0]["fallbacks"] == 0
    fwd, _ = _scripted(script)
    _, blocks, _ = O.generate(fwd, 3, 3, eos_token=99, threshold=0.95)
    assert blocks[0]["rounds"] == 3 and blocks[0]["fallbacks"] == 2


def test_request_bound_counts_the_whole_final_block():
    # 131072 tokens including room to resolve the final block
    assert O.request_fits(131072 - 32, 32, 32) and O.request_fits(131072 - 32, 1, 32)
    assert not O.request_fits(131072 - 31, 1, 32)      # the final block needs 32 positions
    assert not O.request_fits(131040, 33, 32)          # 33 new tokens take two blocks
    assert O.request_fits(0, 131072, 32) and not O.request_fits(1, 131072, 32)
    assert O.request_fits(131068, 4, 4) and not O.request_fits(131068, 5, 4)
    with pytest.raises(ValueError):
        O.generate(lambda *a: None, 4, 5, 0, prompt=range(131068))
