"""Shared helpers of the GPU parity tests: oracle views of GPU-resident
weights, tolerance and margin-band rules."""

import numpy as np
import torch

import block_diffusion_decode_amd as bdd
import oracle as O
import workloads as W

# Floating-point outputs: |gpu - ref| <= ABS + REL * |ref| (bf16 weights, fp32 accumulate).
ABS, REL = 1e-3, 1e-2
# Decisions taken from floating point are compared bit-exactly outside this band.
BAND = 1e-3
TAU = 0.95


def close(gpu, ref, abs_=ABS, rel=REL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(gpu - ref) <= abs_ + rel * np.abs(ref)


def assert_close(gpu, ref, what, abs_=ABS, rel=REL):
    ok = close(gpu, ref, abs_, rel)
    if not ok.all():
        i = np.unravel_index(np.argmax(~ok), ok.shape)
        err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
        raise AssertionError(f"{what}: {int((~ok).sum())}/{ok.size} outside tolerance; first at {i}: "
                             f"gpu={np.asarray(gpu)[i]} ref={np.asarray(ref)[i]}; max err {err.max():.3g}")


def dims_of(d: W.Dims) -> bdd.MoEDims:
    return bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, bdd.BDD_BF16 if d.wdtype == "bf16" else bdd.BDD_F32)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


class LazyExperts:
    """e -> (w_gate_up[e], w_down[e]) as float64, copied from the GPU on first use."""

    def __init__(self, gu: torch.Tensor, dn: torch.Tensor, ids=None):
        self.gu, self.dn = gu, dn
        self.pos = {e: j for j, e in enumerate(ids)} if ids is not None else None
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            j = e if self.pos is None else self.pos[e]
            self.cache[e] = (f64(self.gu[j]), f64(self.dn[j]))
        return self.cache[e]


def oracle_layer(layer: dict) -> dict:
    return {
        "w_router": f64(layer["w_router"]),
        "router_bias": f64(layer["router_bias"]),
        "ws_gate_up": f64(layer["ws_gate_up"]),
        "ws_down": f64(layer["ws_down"]),
        "experts": LazyExperts(layer["w_gate_up"], layer["w_down"], layer.get("experts")),
    }


def topk_gap(logits: np.ndarray, K: int) -> np.ndarray:
    """Per position: K-th largest minus (K+1)-th largest logit (inf if K = E)."""
    s = -np.sort(-logits, axis=1)
    if K >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    return s[:, K - 1] - s[:, K]


def coreset_in_band(p, idx, top_p) -> bool:
    """The coreset cut lies within BAND of a decision boundary."""
    if top_p >= 1.0:
        return False
    members, mass, order = O.coreset_select(p, idx, top_p)
    M = mass.sum()
    cum = np.cumsum(mass[order]) / M
    k = len(members)
    near = abs(cum[k - 1] - top_p) < BAND or (k >= 2 and abs(cum[k - 2] - top_p) < BAND)
    gap = np.inf
    if k < len(order) and mass[order[k]] > 0:
        gap = (mass[order[k - 1]] - mass[order[k]]) / M
    return bool(near or gap < BAND)


def top2_gap(z: np.ndarray) -> np.ndarray:
    s = -np.sort(-z, axis=1)
    return s[:, 0] - s[:, 1]


def commit_in_band(tokens, conf, tau=TAU) -> bool:
    """The commit decision is within BAND of a threshold or a fallback tie."""
    masked = np.nonzero(np.asarray(tokens) == O.MASK)[0]
    if masked.size == 0:
        return False
    c = np.asarray(conf)[masked]
    if np.any(np.abs(c - tau) < BAND):
        return True
    if not np.any(c >= tau) and masked.size >= 2:
        s = np.sort(c)[::-1]
        return bool(s[0] - s[1] < BAND)
    return False


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 1e-38)))
    return np.ldexp(1.0, (e - 7).astype(int))


def commit_check(tok_before, c_ref, ch_ref, excl, c_gpu, ch_gpu, tok_after_gpu, ri_gpu, tau=TAU):
    """Compare one GPU commit with the oracle's.  ``excl`` marks positions whose
    GPU inputs legitimately differ (an upstream decision inside the margin
    band).  Returns (tok_ref_after, exact): exact means the whole round was
    compared and both token states agree; otherwise only the uniquely
    determined part was compared and the caller must stop comparing rounds.
    Raises AssertionError on a mismatch."""
    tok_before = np.asarray(tok_before)
    tok_after_gpu = np.asarray(tok_after_gpu)
    masked = tok_before == O.MASK
    # written tokens never change, and a round with masked positions writes one
    assert np.array_equal(tok_after_gpu[~masked], tok_before[~masked])
    if masked.any():
        assert (tok_after_gpu[masked] != O.MASK).sum() >= 1
    amb = np.asarray(excl) | (np.abs(np.asarray(c_ref) - tau) < BAND)
    if not (masked & amb).any() and not commit_in_band(tok_before, c_ref, tau):
        tok_ref, acc, fb, left, done = O.commit(tok_before, c_ref, ch_ref, tau)
        assert np.array_equal(tok_after_gpu, tok_ref), (tok_after_gpu, tok_ref)
        assert list(ri_gpu) == [len(acc), int(fb), left, int(done)]
        return tok_ref, True
    # some masked position is ambiguous: if a clear position passes there is no
    # fallback, and every clear position's decision is unique
    clear_pass = masked & ~amb & (np.asarray(c_ref) >= tau)
    if clear_pass.any():
        for t in np.nonzero(masked & ~amb)[0]:
            wrote = tok_after_gpu[t] != O.MASK
            assert wrote == (c_ref[t] >= tau), t
            if wrote:
                assert tok_after_gpu[t] == ch_ref[t], t
        for t in np.nonzero(masked & amb)[0]:   # GPU consistent with its own confidence
            wrote = tok_after_gpu[t] != O.MASK
            assert wrote == (c_gpu[t] >= tau), t
            if wrote:
                assert tok_after_gpu[t] == ch_gpu[t], t
        assert ri_gpu[1] == 0
    return None, False


class Int4Rows:
    """Rows of a dequantised 4-bit matrix (codes uint8 [R][C/2], bf16 scales
    [R][C/128]), built slice by slice in float64 (the oracle's LM head reads
    its weight in row blocks)."""

    def __init__(self, codes, scales):
        self.codes = codes.cpu().numpy()
        self.scales = scales.float().cpu().numpy().astype(np.float64)
        self.shape = (self.codes.shape[0], 2 * self.codes.shape[1])

    def __getitem__(self, sl):
        return O.int4_dequantize(self.codes[sl], self.scales[sl])


class Int4Experts:
    """e -> (dequantised gate/up [2I][H], down [H][I]) in float64, on first use."""

    def __init__(self, w):
        self.w, self.cache = w, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            w = self.w
            self.cache[e] = (O.int4_dequantize(w["gu_codes"][e].cpu().numpy(), f64(w["gu_scales"][e])),
                             O.int4_dequantize(w["dn_codes"][e].cpu().numpy(), f64(w["dn_scales"][e])))
        return self.cache[e]


def oracle_layer_int4(w: dict) -> dict:
    """The oracle's view of a 4-bit layer from workloads.layer_weights_int4:
    the router as is, every expert matrix dequantised."""
    return {"w_router": f64(w["w_router"]), "router_bias": f64(w["router_bias"]),
            "ws_gate_up": O.int4_dequantize(w["sgu_codes"].cpu().numpy(), f64(w["sgu_scales"])),
            "ws_down": O.int4_dequantize(w["sdn_codes"].cpu().numpy(), f64(w["sdn_scales"])),
            "experts": Int4Experts(w)}


def packed_layer_int4(w: dict, device) -> dict:
    """The library's 4-bit layer: the router as is, the expert matrices packed
    by bdd_pack_int4."""
    def pk(c, s):
        return bdd.pack_int4(w[c].to(device), w[s].to(device))
    return {"w_router": w["w_router"].to(device), "router_bias": w["router_bias"].to(device),
            "w_gate_up": pk("gu_codes", "gu_scales"), "w_down": pk("dn_codes", "dn_scales"),
            "ws_gate_up": pk("sgu_codes", "sgu_scales"), "ws_down": pk("sdn_codes", "sdn_scales")}
