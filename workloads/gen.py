"""Counter-keyed synthetic tensors for the block-diffusion decode round.

Pages referred to below:
  [P1] aitujian.cn article on Clover-35B-A3B-Preview (Chinese), sections
       一 (decode accounting), 三 (decoding loop, toy fallback model),
       四 (backbone: 40 layers, 256 routed experts top-8, one shared expert),
       五 (MoE account for a 32-position block).
  [P2] goremy.ai, "What Is Clover-35B-A3B? Block Diffusion on a Qwen3.6 MoE",
       sections "How does confidence-threshold block decoding work?" and
       "What is the MoE coreset and why does it matter?".
  [P3] 10100.com article on Clover-35B-A3B-Preview, part 01 (structure).

Every value is a pure function of (seed, tensor name, element index): a
32-bit counter is hashed twice with the "lowbias32" integer mixer (Chris
Wellons, 2018: xor-shift 16, multiply 0x7feb352d, xor-shift 15, multiply
0x846ca68b, xor-shift 16).  Normal variates use the Irwin-Hall sum of four
16-bit uniforms scaled to unit variance (support +-2*sqrt(3)).  All steps
are integer operations, one exactly rounded float64 multiply, a float64 ->
float32 conversion and torch's float32 -> bfloat16 conversion (round to
nearest even), so the same call yields identical bits on the CPU and on a
GPU, and any sub-range of a tensor can be regenerated alone.

The workload shapes are the ones the task's benchmark configurations name
(hidden 2048, 256 experts top-8, intermediate 512, vocab 248320, block 32;
the tiny fp32 case uses hidden 256, 16 experts top-4, intermediate 128,
vocab 1024, block 8).
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np
import torch

_M32 = 0xFFFFFFFF
_CHUNK = 1 << 23


@dataclass(frozen=True)
class Dims:
    """Shapes of one workload.  T block positions, H hidden, E routed experts,
    K experts per token, I routed-expert intermediate, I_s shared-expert
    intermediate, V vocabulary; wdtype is the stored weight type."""

    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    I_s: int
    V: int
    wdtype: str  # "f32" or "bf16"
    w_std: float  # expert / router / shared weights
    lm_std: float  # LM-head rows

    @property
    def torch_wdtype(self):
        return torch.float32 if self.wdtype == "f32" else torch.bfloat16

    @property
    def expert_bytes(self) -> int:
        """Bytes of one routed expert's gate, up and down matrices."""
        return 3 * self.H * self.I * (4 if self.wdtype == "f32" else 2)


# Tiny fp32 step: every weight N(0, 0.02).
C0 = Dims("tiny_fp32", T=8, H=256, E=16, K=4, I=128, I_s=128, V=1024,
          wdtype="f32", w_std=0.02, lm_std=0.02)
# Clover-shaped MoE layer ([P1] 四, [P2] architecture): bf16 weights N(0, 0.02).
C1 = Dims("clover_layer", T=32, H=2048, E=256, K=8, I=512, I_s=512, V=248320,
          wdtype="bf16", w_std=0.02, lm_std=2048 ** -0.5)
# LM head alone: rows N(0, 1/H) so that unit-RMS inputs give N(0,1) logits.
LMHEAD_C3 = C1


# --------------------------------------------------------------------------
# counter-based random numbers
# --------------------------------------------------------------------------

def key_of(*parts) -> tuple[int, int]:
    """Two 32-bit keys derived from an arbitrary tuple of names and ints."""
    d = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(d[:4], "little"), int.from_bytes(d[4:], "little")


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2^32 for 0 <= x < 2^32 without int64 overflow.
    return (x * (c & 0xFFFF) + ((x * (c >> 16)) & 0xFFFF) * 65536) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def counter_words(key: tuple[int, int], ctr: torch.Tensor) -> torch.Tensor:
    """32-bit words (as int64) for counters 0 <= ctr < 2^32."""
    k0, k1 = key
    return _mix32((_mix32(ctr ^ k0) + k1) & _M32)


def _ranges(start: int, n: int):
    s = start
    while s < start + n:
        e = min(s + _CHUNK, start + n)
        yield s, e
        s = e


def counter_uniform(key, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """float64 uniforms in (0, 1) with 24-bit resolution, elements start..start+n."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s, e in _ranges(start, n):
        ctr = torch.arange(s, e, dtype=torch.int64, device=device)
        w = counter_words(key, ctr)
        out[s - start:e - start] = ((w >> 8).to(torch.float64) + 0.5) * (2.0 ** -24)
    return out


def counter_normal(key, n: int, std: float = 1.0, device="cpu", start: int = 0,
                   dtype=torch.float32) -> torch.Tensor:
    """Approximately normal variates (Irwin-Hall of four 16-bit uniforms)."""
    assert 2 * (start + n) <= (1 << 32)
    scale = math.sqrt(3.0) / 65536.0 * std
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s, e in _ranges(start, n):
        i = torch.arange(s, e, dtype=torch.int64, device=device)
        w0 = counter_words(key, 2 * i)
        w1 = counter_words(key, 2 * i + 1)
        tot = (w0 & 0xFFFF) + (w0 >> 16) + (w1 & 0xFFFF) + (w1 >> 16) - 131070
        out[s - start:e - start] = (tot.to(torch.float64) * scale).to(torch.float32)
    return out.to(dtype)


# --------------------------------------------------------------------------
# model tensors
# --------------------------------------------------------------------------

def _normal_tensor(key, shape, std, dtype, device):
    n = int(np.prod(shape))
    return counter_normal(key, n, std, device).to(dtype).reshape(shape)


def zipf_router_bias(seed: int, layer: int, E: int, s: float = 1.1,
                     gamma: float = 1.0) -> torch.Tensor:
    """Router bias b_e = -s * gamma * ln(rank_e) with rank a seeded permutation
    of 1..E, so that expert popularity falls off like a Zipf(s) law.  Built on
    the CPU in float64 and stored as float32."""
    u = counter_uniform(key_of(seed, "zipf_rank", layer), E).numpy()
    order = np.argsort(u, kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    b = -s * gamma * np.log(rank.astype(np.float64))
    return torch.from_numpy(b.astype(np.float32))


def router_weights(seed: int, layer: int, d: Dims, dtype, device="cpu", bias: str = "flat",
                   gamma: float = 1.0) -> dict:
    """A layer's router weight w_router [E][H] (N(0, w_std), stored as dtype)
    and router_bias [E] float32 (zeros, or the Zipf bias)."""
    out = {"w_router": _normal_tensor(key_of(seed, "router", layer), (d.E, d.H), d.w_std, dtype, device)}
    if bias == "flat":
        out["router_bias"] = torch.zeros(d.E, dtype=torch.float32, device=device)
    elif bias == "zipf":
        out["router_bias"] = zipf_router_bias(seed, layer, d.E, 1.1, gamma).to(device)
    else:
        raise ValueError(bias)
    return out


def layer_weights(seed: int, layer: int, d: Dims, device="cpu",
                  bias: str = "flat", gamma: float = 1.0,
                  experts=None) -> dict:
    """One MoE layer.  Layouts are [out][in] (input dimension contiguous):
      w_router  [E][H]        router_bias [E] float32
      w_gate_up [E][2I][H]    rows 0..I-1 gate, rows I..2I-1 up
      w_down    [E][H][I]
      ws_gate_up [2I_s][H]    ws_down [H][I_s]   (the shared expert)
    With ``experts`` given, w_gate_up / w_down hold only those experts (in
    that order) and 'experts' lists them."""
    dt = d.torch_wdtype
    out = router_weights(seed, layer, d, dt, device, bias, gamma)
    ex = list(range(d.E)) if experts is None else list(experts)
    gu = torch.empty((len(ex), 2 * d.I, d.H), dtype=dt, device=device)
    dn = torch.empty((len(ex), d.H, d.I), dtype=dt, device=device)
    for j, e in enumerate(ex):
        gu[j] = _normal_tensor(key_of(seed, "gate_up", layer, e), (2 * d.I, d.H), d.w_std, dt, device)
        dn[j] = _normal_tensor(key_of(seed, "down", layer, e), (d.H, d.I), d.w_std, dt, device)
    out["w_gate_up"] = gu
    out["w_down"] = dn
    out["experts"] = ex
    out["ws_gate_up"] = _normal_tensor(key_of(seed, "shared_gate_up", layer), (2 * d.I_s, d.H), d.w_std, dt, device)
    out["ws_down"] = _normal_tensor(key_of(seed, "shared_down", layer), (d.H, d.I_s), d.w_std, dt, device)
    return out


def int4_matrix(key: tuple, rows: int, cols: int, std: float, device="cpu", group: int = 128):
    """Synthetic 4-bit weight matrix [rows][cols]: (codes uint8 [rows][cols/2],
    scales bf16 [rows][cols/group]).  Byte j of a row holds columns 2j (low
    nibble) and 2j + 1 (high nibble).  Codes are a rounded normal, n =
    clamp(round(2.5 z), -8, 7) + 8; scales are std / 2.5 * U(0.8, 1.2), so the
    weights (n - 8) * scale have about the given spread.  ``key`` is a tuple
    of names and ints naming the matrix."""
    assert cols % group == 0
    k_codes, k_scales = key_of(*key, "codes"), key_of(*key, "scales")
    n = torch.empty(rows * cols, dtype=torch.uint8, device=device)
    for s_, e_ in _ranges(0, rows * cols):
        z = counter_normal(k_codes, e_ - s_, 1.0, device, start=s_)
        n[s_:e_] = (torch.round(z * 2.5).clamp_(-8, 7) + 8).to(torch.uint8)
    n = n.reshape(rows, cols // 2, 2)
    codes = (n[..., 0] | (n[..., 1] << 4)).contiguous()
    u = counter_uniform(k_scales, rows * (cols // group), device)
    scales = (std / 2.5 * (0.8 + 0.4 * u)).to(torch.bfloat16).reshape(rows, cols // group)
    return codes, scales


def layer_weights_int4(seed: int, layer: int, d: Dims, device="cpu", bias: str = "flat",
                       gamma: float = 1.0) -> dict:
    """One MoE layer with 4-bit expert weights (the format int4_matrix
    describes): the router (bf16, the same tensor layer_weights draws) and
    bias, and per expert matrix its codes and scales:
      gu_codes [E][2I][H/2], gu_scales [E][2I][H/128]   (rows 0..I-1 gate)
      dn_codes [E][H][I/2],  dn_scales [E][H][I/128]
      sgu_codes / sgu_scales, sdn_codes / sdn_scales    (the shared expert)
    The routed experts' matrices are drawn as one stacked matrix each (expert
    e = rows e*R .. (e+1)*R - 1)."""
    out = router_weights(seed, layer, d, torch.bfloat16, device, bias, gamma)
    c, sc = int4_matrix((seed, "i4_gate_up", layer), d.E * 2 * d.I, d.H, d.w_std, device)
    out["gu_codes"], out["gu_scales"] = c.reshape(d.E, 2 * d.I, d.H // 2), sc.reshape(d.E, 2 * d.I, d.H // 128)
    c, sc = int4_matrix((seed, "i4_down", layer), d.E * d.H, d.I, d.w_std, device)
    out["dn_codes"], out["dn_scales"] = c.reshape(d.E, d.H, d.I // 2), sc.reshape(d.E, d.H, d.I // 128)
    out["sgu_codes"], out["sgu_scales"] = int4_matrix((seed, "i4_shared_gate_up", layer), 2 * d.I_s, d.H,
                                                      d.w_std, device)
    out["sdn_codes"], out["sdn_scales"] = int4_matrix((seed, "i4_shared_down", layer), d.H, d.I_s, d.w_std, device)
    return out


def lm_head_rows(seed: int, d: Dims, rows, device="cpu", unit_rows=()) -> torch.Tensor:
    """Selected rows of the LM-head weight [V][H], regenerated alone.  Rows in
    ``unit_rows`` are rescaled to unit Euclidean norm (planted rows)."""
    key = key_of(seed, "lm_head")
    rows = list(rows)
    out = torch.empty((len(rows), d.H), dtype=torch.float32, device=device)
    for j, v in enumerate(rows):
        out[j] = counter_normal(key, d.H, d.lm_std, device, start=v * d.H)
    unit = set(unit_rows)
    for j, v in enumerate(rows):
        if v in unit:
            r = out[j].double()
            out[j] = (r / torch.linalg.vector_norm(r)).float()
    return out.to(d.torch_wdtype)


def lm_head_weight(seed: int, d: Dims, device="cpu", unit_rows=()) -> torch.Tensor:
    """LM-head weight [V][H] (row v = token v's output embedding)."""
    key = key_of(seed, "lm_head")
    w = counter_normal(key, d.V * d.H, d.lm_std, device).reshape(d.V, d.H)
    if len(unit_rows):
        idx = torch.tensor(sorted(set(unit_rows)), dtype=torch.int64)
        rows = lm_head_rows(seed, d, idx.tolist(), device, unit_rows=idx.tolist()).float()
        w[idx.to(device)] = rows
    return w.to(d.torch_wdtype)


def lm_head_int4(seed: int, d: Dims, device="cpu", group: int = 128, unit_rows=()):
    """Synthetic 4-bit LM head of shape [V][H]: (codes uint8 [V][H/2], scales
    bf16 [V][H/group]).  Byte j of a row holds columns 2j (low nibble) and
    2j + 1 (high nibble).  Codes are a rounded normal, n = clamp(round(2.5 z),
    -8, 7) + 8, the histogram of quantised weights; scales are
    lm_std / 2.5 * U(0.8, 1.2), so the weights the codes stand for have
    about the bf16 head's spread.  Rows in ``unit_rows`` hold instead the
    4-bit rounding (quantize_int4) of the bf16 head's planted unit rows, so
    inputs planted along those rows peak on the same tokens."""
    assert d.H % group == 0
    n = torch.empty(d.V * d.H, dtype=torch.uint8, device=device)
    key = key_of(seed, "lm_int4_codes")
    for s, e in _ranges(0, d.V * d.H):
        z = counter_normal(key, e - s, 1.0, device, start=s)
        n[s:e] = (torch.round(z * 2.5).clamp_(-8, 7) + 8).to(torch.uint8)
    n = n.reshape(d.V, d.H // 2, 2)
    codes = (n[..., 0] | (n[..., 1] << 4)).contiguous()
    u = counter_uniform(key_of(seed, "lm_int4_scales"), d.V * (d.H // group), device)
    scales = (d.lm_std / 2.5 * (0.8 + 0.4 * u)).to(torch.bfloat16).reshape(d.V, d.H // group)
    if len(unit_rows):
        idx = sorted(set(int(v) for v in unit_rows))
        rows = lm_head_rows(seed, d, idx, "cpu", unit_rows=idx).float()
        qc, qs = quantize_int4(rows, group)
        it = torch.tensor(idx, dtype=torch.int64, device=device)
        codes[it] = qc.to(device)
        scales[it] = qs.to(device)
    return codes, scales


def quantize_int4(w: torch.Tensor, group: int = 128):
    """Round rows w [R][C] to the 4-bit format of int4_matrix: per row and
    group, scale s = bf16(max |w| / 7) and code n = clamp(round(w / s), -8, 7)
    + 8 (an input-preparation step; the method only reads the codes)."""
    R, C = w.shape
    g = w.double().reshape(R, C // group, group)
    s = (g.abs().amax(dim=2) / 7.0).to(torch.bfloat16)
    sd = s.double().clamp_min(1e-30).unsqueeze(2)
    n = (torch.round(g / sd).clamp_(-8, 7) + 8).to(torch.uint8).reshape(R, C // 2, 2)
    return (n[..., 0] | (n[..., 1] << 4)).contiguous(), s


def block_hidden(seed: int, d: Dims, device="cpu", tag="h") -> torch.Tensor:
    """Block hidden states h [T][H] float32, N(0, 1)."""
    return counter_normal(key_of(seed, "hidden", tag), d.T * d.H, 1.0, device).reshape(d.T, d.H)


# --------------------------------------------------------------------------
# MASK re-embedding stubs (the mixer that would produce these is not built)
# --------------------------------------------------------------------------

def _round_plan(seed: int, tag: str, d: Dims, rounds: int, p: float):
    """Per (round, position): planted vocab id, pass flag, and the position's
    rank inside its round (used to space the failing peaks apart)."""
    n = rounds * d.T
    u_v = counter_uniform(key_of(seed, tag, "vocab"), n).numpy()
    u_p = counter_uniform(key_of(seed, tag, "pass"), n).numpy()
    u_r = counter_uniform(key_of(seed, tag, "rank"), n).numpy().reshape(rounds, d.T)
    v = np.minimum((u_v * d.V).astype(np.int64), d.V - 1).reshape(rounds, d.T)
    passed = (u_p < p).reshape(rounds, d.T)
    rank = np.argsort(np.argsort(u_r, axis=1, kind="stable"), axis=1, kind="stable")
    return v, passed, rank


def lmhead_stub_inputs(seed: int, d: Dims, rounds: int, p: float, device="cpu",
                       pass_logit=(18.5, 20.5), fail_logit=(12.0, 14.0)):
    """LM-head inputs for a multi-round resolve, [rounds][T][H] bf16.

    Position t in round r gets g + c * w_v, with g ~ N(0,1), w_v the LM-head
    row of a seeded token v, and c chosen (float64, on the CPU) so that the
    planted logit g'w_v equals a target: with probability p a passing level
    drawn from ``pass_logit``, otherwise a failing level in ``fail_logit``
    spaced by position rank so that failing confidences stay apart.  The
    other logits are N(0,1)-like.  Returns (h [R][T][H], info dict)."""
    v, passed, rank = _round_plan(seed, "lmstub", d, rounds, p)
    u_l = counter_uniform(key_of(seed, "lmstub", "level"), rounds * d.T).numpy().reshape(rounds, d.T)
    rows = lm_head_rows(seed, d, sorted(set(v.ravel().tolist())), "cpu").double()
    row_of = {int(x): j for j, x in enumerate(sorted(set(v.ravel().tolist())))}
    g = counter_normal(key_of(seed, "lmstub", "g"), rounds * d.T * d.H, 1.0).double()
    g = g.reshape(rounds, d.T, d.H)
    target = np.where(
        passed,
        pass_logit[0] + (pass_logit[1] - pass_logit[0]) * u_l,
        fail_logit[0] + (fail_logit[1] - fail_logit[0]) * (rank + 0.5 * u_l + 0.25) / d.T,
    )
    h = torch.empty_like(g)
    for r in range(rounds):
        for t in range(d.T):
            w = rows[row_of[int(v[r, t])]]
            c = (target[r, t] - float(g[r, t] @ w)) / float(w @ w)
            h[r, t] = g[r, t] + c * w
    info = {"vocab": v, "passed": passed, "target_logit": target}
    return h.to(torch.float32).to(torch.bfloat16).to(device), info


def planted_round_inputs(seed: int, d: Dims, rounds: int, p: float,
                         amp_pass: float, amp_fail: tuple[float, float],
                         device="cpu", tag="xstub"):
    """Hidden states entering the first layer, [rounds][T][H] float32.

    Position t in round r gets g + a * w_v / |w_v| with g ~ N(0,1) and w_v the
    LM-head row of a seeded token v: amplitude ``amp_pass`` with probability
    p, otherwise an amplitude in ``amp_fail`` spaced by position rank.  The
    amplitudes are input-recipe constants; which positions pass is decided by
    the model itself.  Returns (x [R][T][H], info dict)."""
    v, passed, rank = _round_plan(seed, tag, d, rounds, p)
    uniq = sorted(set(v.ravel().tolist()))
    rows = lm_head_rows(seed, d, uniq, "cpu", unit_rows=uniq).double()
    row_of = {int(x): j for j, x in enumerate(uniq)}
    g = counter_normal(key_of(seed, tag, "g"), rounds * d.T * d.H, 1.0).double()
    g = g.reshape(rounds, d.T, d.H)
    amp = np.where(passed, amp_pass,
                   amp_fail[0] + (amp_fail[1] - amp_fail[0]) * (rank + 0.5) / d.T)
    x = torch.empty_like(g)
    for r in range(rounds):
        for t in range(d.T):
            w = rows[row_of[int(v[r, t])]]
            x[r, t] = g[r, t] + amp[r, t] * w / torch.linalg.vector_norm(w)
    info = {"vocab": v, "passed": passed, "amplitude": amp, "unit_rows": uniq}
    return x.to(torch.float32).to(device), info
