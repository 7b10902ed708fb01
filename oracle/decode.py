"""Plain float64 definitions of each step of the denoising round.

TEST INFRASTRUCTURE ONLY (see the package docstring for the pages [P1]-[P3],
the readings taken, and who may import this module).

Arrays are NumPy; weights arrive as float64 copies of the stored (bf16 or
fp32) values.  Shapes follow the pages' notation: T block positions, H
hidden, E routed experts, K experts per token, I expert intermediate, V
vocabulary.  Weight layouts are [out][in].
"""

from __future__ import annotations

import numpy as np

MASK = -1


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits,
    ties to even), returned as float64.  bf16 is the model's storage type
    ([P2] "How do you run Clover-35B-A3B?": the model runs in BF16)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])          # x = m * 2^e with 0.5 <= |m| < 1
    q = np.ldexp(m, 8)              # 128 <= |q| < 256: 8 significant bits
    out[nz] = np.ldexp(np.rint(q), e - 8)   # np.rint rounds half to even
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


# ---------------------------------------------------------------------------
# normalisation and experts
# ---------------------------------------------------------------------------

def rmsnorm(h, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm with unit gain: h / sqrt(mean(h^2) + eps), per row.  The pages
    name no norm; this is the pre-norm reading of the layer."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_expert(x, w_gate_up, w_down) -> np.ndarray:
    """One SwiGLU expert on rows x [n][H]: gate g = x W_g^T, up u = x W_u^T
    (W_g = rows 0..I-1 of w_gate_up, W_u = rows I..2I-1), a = silu(g) * u,
    output a W_d^T with w_down [H][I]."""
    x = np.asarray(x, dtype=np.float64)
    I = w_gate_up.shape[0] // 2
    g = x @ w_gate_up[:I].T
    u = x @ w_gate_up[I:].T
    return (silu(g) * u) @ w_down.T


# ---------------------------------------------------------------------------
# routing and coreset ([P1] 四; [P2] MoE coreset section)
# ---------------------------------------------------------------------------

def route(xhat, w_router, bias, K: int):
    """Top-K token routing.  logits l = xhat W_r^T + b; p = softmax over all E
    experts; S_t = the K largest logits (ties -> lower expert id); weights
    w = p restricted to S_t and renormalised.  Returns (l, p, idx, w) with
    idx [T][K] in descending-logit order."""
    x = np.asarray(xhat, dtype=np.float64)
    l = x @ np.asarray(w_router, np.float64).T + np.asarray(bias, np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    idx = np.argsort(-l, axis=1, kind="stable")[:, :K]
    pk = np.take_along_axis(p, idx, axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return l, p, idx, w


def coreset_select(p, idx, top_p: float):
    """Block coreset ([P2] "What is the MoE coreset"): sum each token's top-K
    routing scores per expert over the block, rank experts by that mass
    (descending; ties -> lower id), keep the shortest ranked prefix whose
    mass reaches top_p of the total.  top_p >= 1 keeps every expert with
    positive mass.  Returns (members sorted ascending, mass [E], order)."""
    p = np.asarray(p, dtype=np.float64)
    T, E = p.shape
    mass = np.zeros(E)
    for t in range(T):
        for e in idx[t]:
            mass[e] += p[t, e]
    order = np.lexsort((np.arange(E), -mass))     # primary -mass, then id
    n_pos = int(np.count_nonzero(mass > 0))
    if top_p >= 1.0:
        k = n_pos
    else:
        cum = np.cumsum(mass[order])
        k = int(np.searchsorted(cum, top_p * mass.sum(), side="left")) + 1
        k = min(max(k, 1), n_pos)
    return np.sort(order[:k]), mass, order


def reroute(l, p, members, K: int):
    """Routing restricted to the coreset: each token re-takes the
    min(K, |C|) largest logits among the members (ties -> lower id) and
    renormalises its softmax scores over them."""
    l = np.asarray(l, dtype=np.float64)
    members = np.sort(np.asarray(members))
    k = min(K, len(members))
    sub = l[:, members]
    pick = np.argsort(-sub, axis=1, kind="stable")[:, :k]
    idx = members[pick]
    pk = np.take_along_axis(p, idx, axis=1)
    return idx, pk / pk.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# one MoE layer and the layer stack
# ---------------------------------------------------------------------------

def moe_layer(xhat, layer: dict, K: int, top_p: float = 1.0):
    """MoE FFN of one layer on the normalised block xhat [T][H] ([P1] 四:
    256 routed experts, top-8, one shared expert).  ``layer`` holds float64
    arrays w_router [E][H], router_bias [E], ws_gate_up, ws_down, and a
    mapping ``experts`` e -> (w_gate_up[e], w_down[e]) (only the experts the
    block uses need to be present).

    y_t = sum_{e in S_t} w_te * SwiGLU_e(xhat_t) + SwiGLU_shared(xhat_t).
    Returns y and a dict with the routing (logits, p, idx, w), the coreset
    members (None without coreset) and the union of experts read."""
    l, p, idx, w = route(xhat, layer["w_router"], layer["router_bias"], K)
    members = None
    if top_p < 1.0:
        members, _, _ = coreset_select(p, idx, top_p)
        idx, w = reroute(l, p, members, K)
    y, union = moe_given_routing(xhat, layer, idx, w)
    info = {"logits": l, "p": p, "idx": idx, "w": w, "coreset": members, "union": union}
    return y, info


def moe_given_routing(xhat, layer: dict, idx, w):
    """The expert part of moe_layer for a routing already taken: idx [T][K]
    expert ids (-1 = unused slot) and their weights w [T][K].
    y_t = sum_k w[t,k] * SwiGLU_{idx[t,k]}(xhat_t) + SwiGLU_shared(xhat_t)
    ([P1] 四).  Returns (y, sorted union of experts)."""
    x = np.asarray(xhat, dtype=np.float64)
    idx = np.asarray(idx)
    T = x.shape[0]
    y = swiglu_expert(x, layer["ws_gate_up"], layer["ws_down"])
    union = sorted(set(int(e) for e in idx.ravel() if e >= 0))
    for e in union:
        gu, dn = layer["experts"][e]
        rows = [t for t in range(T) if e in idx[t]]
        out = swiglu_expert(x[rows], gu, dn)
        for j, t in enumerate(rows):
            k = int(np.nonzero(idx[t] == e)[0][0])
            y[t] += w[t, k] * out[j]
    return y, union


def moe_stack(x_in, layers, K: int, top_p: float = 1.0, round_bf16: bool = True,
              eps: float = 1e-6):
    """Layer stack with the mixer replaced by identity: h <- h + MoE(RMSNorm(h))
    per layer, then the final RMSNorm feeding the LM head.  With round_bf16
    the normalised activations are rounded to bf16 where they are stored.
    ``layers`` may be a list of dicts or a callable layer_index -> dict (so a
    long stack can regenerate one layer at a time).  Returns (hhat, infos)."""
    h = np.asarray(x_in, dtype=np.float64).copy()
    n = len(layers) if not callable(layers) else None
    infos = []
    l = 0
    while n is None or l < n:
        layer = layers(l) if callable(layers) else layers[l]
        if layer is None:
            break
        xh = rmsnorm(h, eps)
        if round_bf16:
            xh = bf16_round(xh)
        y, info = moe_layer(xh, layer, K, top_p)
        info["xhat"] = xh
        infos.append(info)
        h = h + y
        l += 1
    hh = rmsnorm(h, eps)
    return (bf16_round(hh) if round_bf16 else hh), infos


# ---------------------------------------------------------------------------
# LM head, confidence, commit ([P1] 三; [P2] decoding loop)
# ---------------------------------------------------------------------------

def lm_head_confidence(hhat, w_lm, chunk: int = 16384):
    """z = hhat W_lm^T; prob = softmax(z); conf = max prob; choice = argmax
    (lowest id on ties).  The logits are formed in row blocks of W_lm only
    to bound memory; each logit is the same dot product.  Returns
    (conf [T], choice [T], logits [T][V]); conf = 1 / sum_v exp(z_v - max z)."""
    h = np.asarray(hhat, dtype=np.float64)
    V = w_lm.shape[0]
    z = np.empty((h.shape[0], V))
    for s in range(0, V, chunk):
        z[:, s:s + chunk] = h @ np.asarray(w_lm[s:s + chunk], np.float64).T
    m = z.max(axis=1)
    choice = np.argmax(z, axis=1)        # first occurrence of the maximum
    conf = 1.0 / np.exp(z - m[:, None]).sum(axis=1)
    return conf, choice, z


INT4_GROUP = 128


def int4_dequantize(codes, scales, group: int = INT4_GROUP) -> np.ndarray:
    """Dequantised weight [R][H] of a 4-bit weight-only format ([P3] 10100.com
    article on Clover-35B-A3B-Preview, part 03, memory and quantisation: the
    model is deployed in INT4 on a 16 GB card; the pages give no format).

    Reading taken: codes[r][j] is a byte holding columns 2j (low nibble) and
    2j + 1 (high nibble); a nibble n in 0..15 stands for the integer n - 8;
    scales[r][c // group] (bf16 values, here as float64) multiplies every
    column c of its row-group.  w[r][c] = (n - 8) * s."""
    b = np.asarray(codes, dtype=np.uint8)
    R, half = b.shape
    n = np.empty((R, 2 * half), dtype=np.int64)
    n[:, 0::2] = b & 0x0F
    n[:, 1::2] = b >> 4
    s = np.asarray(scales, dtype=np.float64)
    assert s.shape == (R, (2 * half) // group)
    return (n - 8).astype(np.float64) * np.repeat(s, group, axis=1)


def commit(tokens, conf, choice, threshold: float = 0.95):
    """One LowConfidence commit.  Among still-masked positions, every one with
    conf >= threshold is written; if none qualifies, the single most
    confident masked position (lowest index on ties) is written instead.
    Written tokens never change afterwards.  Returns (new tokens, accepted
    position list, fallback flag, masked count after, resolved flag)."""
    tok = np.array(tokens, dtype=np.int64).copy()
    masked = np.nonzero(tok == MASK)[0]
    if masked.size == 0:
        return tok, [], False, 0, True
    acc = [int(t) for t in masked if conf[t] >= threshold]
    fallback = False
    if not acc:
        best = max(conf[t] for t in masked)
        acc = [int(min(t for t in masked if conf[t] == best))]
        fallback = True
    for t in acc:
        tok[t] = int(choice[t])
    n_left = int(np.count_nonzero(tok == MASK))
    return tok, acc, fallback, n_left, n_left == 0


def resolve_block(forward, T: int, threshold: float = 0.95, max_steps: int = 32):
    """Resolve one block ([P1] 三 pseudocode inner loop): start all MASK, then
    per round run ``forward(round, tokens) -> (conf, choice)`` and commit,
    until every position is written or max_steps rounds ran.  Returns
    (tokens, per-round records)."""
    tok = np.full(T, MASK, dtype=np.int64)
    rounds = []
    for r in range(max_steps):
        conf, choice = forward(r, tok.copy())
        tok, acc, fb, left, done = commit(tok, conf, choice, threshold)
        rounds.append({"accepted": acc, "fallback": fb, "masked_after": left,
                       "conf": np.asarray(conf), "choice": np.asarray(choice)})
        if done:
            break
    return tok, rounds


# ---------------------------------------------------------------------------
# generation: blocks after blocks ([P1] 三 block_decode pseudocode, outer
# loop; [P2] decoding step 6 and "What generation controls ship by default?")
# ---------------------------------------------------------------------------

MAX_REQUEST_TOKENS = 131072


def request_fits(prompt_len: int, max_new_tokens: int, T: int,
                 limit: int = MAX_REQUEST_TOKENS) -> bool:
    """[P2] generation controls: a request longer than 131072 tokens,
    counting the room needed to resolve the final block, is rejected.  The
    final block is resolved whole, so the new tokens occupy whole blocks:
    prompt_len + ceil(max_new_tokens / T) * T must not exceed the limit."""
    if prompt_len < 0 or max_new_tokens < 1 or T < 1:
        return False
    blocks = -(-max_new_tokens // T)
    return prompt_len + blocks * T <= limit


def generate(forward, T: int, max_new_tokens: int, eos_token: int, prompt=(),
             threshold: float = 0.95, max_steps: int = 32):
    """Blocks of T positions after the prompt ([P1] 三 block_decode): each
    block starts all MASK and is resolved by rounds (resolve_block) of
    ``forward(block, round, tokens, prefix) -> (conf, choice)``; the resolved
    block is appended to the prefix and to the output; generation stops after
    a block whose last token is eos_token, or once max_new_tokens tokens have
    been produced (the final block is still resolved whole; the output is cut
    to max_new_tokens).  A block still masked after max_steps rounds ends the
    generation unresolved.  Requests failing request_fits are rejected
    (ValueError).  Returns (output tokens, per-block records, stop reason in
    'eos', 'length', 'unresolved')."""
    if not request_fits(len(prompt), max_new_tokens, T):
        raise ValueError("request exceeds the token limit")
    prefix = list(prompt)
    out, blocks = [], []
    while True:
        b = len(blocks)
        tok, rounds = resolve_block(lambda r, t: forward(b, r, t, tuple(prefix)), T, threshold, max_steps)
        blocks.append({"tokens": tok.copy(), "rounds": len(rounds),
                       "fallbacks": sum(int(x["fallback"]) for x in rounds)})
        if np.any(tok == MASK):
            return out, blocks, "unresolved"
        out.extend(int(v) for v in tok)
        prefix.extend(int(v) for v in tok)
        if tok[-1] == eos_token:
            return out[:max_new_tokens], blocks, "eos"
        if len(out) >= max_new_tokens:
            return out[:max_new_tokens], blocks, "length"
