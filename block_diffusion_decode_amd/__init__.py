"""Python binding of libbdd (the block-diffusion decode round on MI355X).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed
to the C ABI declared in include/bdd.h, and every step runs in the library's
HIP kernels.  The binding fails loudly if libbdd.so is missing; there is no
fallback path.

Entry points (same names as the C ABI, without the bdd_ prefix):
  moe_block_forward, coreset_select, lmhead_confidence_commit,
  block_denoise_round, pack_lm_head (bdd_lmhead_pack), and the
  *_workspace_bytes queries.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdd.so")

MASK = -1
BDD_F32, BDD_BF16, BDD_INT4 = 0, 1, 2
_STATUS = {1: "BDD_UNRESOLVED", 0: "BDD_OK", -1: "BDD_ERR_INVALID_ARG", -2: "BDD_ERR_UNSUPPORTED",
           -3: "BDD_ERR_WORKSPACE", -4: "BDD_ERR_HIP"}
BDD_UNRESOLVED = 1


class BddError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("wdtype", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("ws_gate_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p)]


EXPORTS = [
    "bdd_moe_workspace_bytes", "bdd_moe_block_forward", "bdd_coreset_select",
    "bdd_lmhead_workspace_bytes", "bdd_lmhead_confidence_commit",
    "bdd_round_workspace_bytes", "bdd_block_denoise_round",
    "bdd_status_string", "bdd_last_error", "bdd_device_cus",
    "bdd_timing_enable", "bdd_timing_read", "bdd_lmhead_packed_bytes", "bdd_lmhead_pack",
    "bdd_lmhead_pack_int4",
    "bdd_round_graph_create", "bdd_round_graph_launch", "bdd_round_graph_destroy",
    "bdd_generate_fits", "bdd_generate_workspace_bytes", "bdd_generate",
    "bdd_block_denoise_round_noalloc", "bdd_int4_packed_bytes", "bdd_pack_int4",
]

# Scratch bytes of bdd_block_denoise_round_noalloc (BDD_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


def lib() -> ctypes.CDLL:
    """Load libbdd.so (built by block_diffusion_decode_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_diffusion_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dims_p, w_p = ctypes.POINTER(_Dims), ctypes.POINTER(_Weights)
    L.bdd_moe_workspace_bytes.argtypes = [dims_p]
    L.bdd_moe_workspace_bytes.restype = sz
    L.bdd_moe_block_forward.argtypes = [dims_p, w_p, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.bdd_moe_block_forward.restype = i32
    L.bdd_coreset_select.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp, vp, vp]
    L.bdd_coreset_select.restype = i32
    L.bdd_lmhead_workspace_bytes.argtypes = [i32, i32, i32]
    L.bdd_lmhead_workspace_bytes.restype = sz
    L.bdd_lmhead_confidence_commit.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.bdd_lmhead_confidence_commit.restype = i32
    L.bdd_round_workspace_bytes.argtypes = [dims_p, i32]
    L.bdd_round_workspace_bytes.restype = sz
    L.bdd_block_denoise_round.argtypes = [dims_p, i32, w_p, f32, vp, i32, f32, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, sz, vp]
    L.bdd_block_denoise_round.restype = i32
    L.bdd_block_denoise_round_noalloc.argtypes = [dims_p, i32, w_p, f32, vp, i32, f32, vp, vp, vp, vp, vp,
                                                  vp, vp, vp, vp, vp]
    L.bdd_block_denoise_round_noalloc.restype = i32
    L.bdd_status_string.argtypes = [i32]
    L.bdd_status_string.restype = ctypes.c_char_p
    L.bdd_last_error.argtypes = []
    L.bdd_last_error.restype = ctypes.c_char_p
    L.bdd_device_cus.argtypes = []
    L.bdd_device_cus.restype = i32
    L.bdd_lmhead_packed_bytes.argtypes = [i32, i32, i32]
    L.bdd_lmhead_packed_bytes.restype = sz
    L.bdd_lmhead_pack.argtypes = [vp, i32, i32, i32, vp, vp]
    L.bdd_lmhead_pack.restype = i32
    L.bdd_lmhead_pack_int4.argtypes = [vp, vp, i32, i32, vp, vp]
    L.bdd_lmhead_pack_int4.restype = i32
    L.bdd_int4_packed_bytes.argtypes = [i32, i32, i32]
    L.bdd_int4_packed_bytes.restype = sz
    L.bdd_pack_int4.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.bdd_pack_int4.restype = i32
    L.bdd_round_graph_create.argtypes = [dims_p, i32, w_p, f32, vp, i32, f32, vp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, sz, ctypes.POINTER(vp)]
    L.bdd_round_graph_create.restype = i32
    L.bdd_round_graph_launch.argtypes = [vp, vp]
    L.bdd_round_graph_launch.restype = i32
    L.bdd_round_graph_destroy.argtypes = [vp]
    L.bdd_round_graph_destroy.restype = None
    L.bdd_generate_fits.argtypes = [i32, i32, i32]
    L.bdd_generate_fits.restype = i32
    L.bdd_generate_workspace_bytes.argtypes = [dims_p, i32]
    L.bdd_generate_workspace_bytes.restype = sz
    L.bdd_generate.argtypes = [dims_p, i32, w_p, f32, vp, i32, f32, i32, i32, i32, i32, i32, vp, i32, vp,
                               ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                               ctypes.POINTER(ctypes.c_int32), vp, sz, vp]
    L.bdd_generate.restype = i32
    L.bdd_timing_enable.argtypes = [i32, ctypes.c_char_p]
    L.bdd_timing_enable.restype = i32
    L.bdd_timing_read.argtypes = [i32, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_int32)]
    L.bdd_timing_read.restype = i32
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise BddError(status, lib().bdd_last_error().decode())


# --------------------------------------------------------------------------- marshalling

@dataclass(frozen=True)
class MoEDims:
    T: int
    H: int
    E: int
    K: int
    I: int
    I_shared: int
    wdtype: int  # BDD_F32, BDD_BF16 or BDD_INT4 (4-bit experts, bf16 router and activations)

    @property
    def torch_dtype(self):
        """dtype of the router and the normalised activations"""
        return torch.float32 if self.wdtype == BDD_F32 else torch.bfloat16

    def c(self) -> _Dims:
        return _Dims(self.T, self.H, self.E, self.K, self.I, self.I_shared, self.wdtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def int4_packed_bytes(n_mats: int, rows: int, cols: int) -> int:
    return int(lib().bdd_int4_packed_bytes(n_mats, rows, cols))


def _weights(d: MoEDims, w: dict, dev) -> _Weights:
    dt = d.torch_dtype
    _need(w["w_router"], "w_router", dt, (d.E, d.H), dev)
    if d.wdtype == BDD_INT4:
        # packed by pack_int4: E matrices of 2I x H and of H x I, the shared expert's one each
        _need(w["w_gate_up"], "w_gate_up", torch.uint8, (int4_packed_bytes(d.E, 2 * d.I, d.H),), dev)
        _need(w["w_down"], "w_down", torch.uint8, (int4_packed_bytes(d.E, d.H, d.I),), dev)
    else:
        _need(w["w_gate_up"], "w_gate_up", dt, (d.E, 2 * d.I, d.H), dev)
        _need(w["w_down"], "w_down", dt, (d.E, d.H, d.I), dev)
    bias = w.get("router_bias")
    if bias is not None:
        _need(bias, "router_bias", torch.float32, (d.E,), dev)
    if d.I_shared > 0:
        if d.wdtype == BDD_INT4:
            _need(w["ws_gate_up"], "ws_gate_up", torch.uint8, (int4_packed_bytes(1, 2 * d.I_shared, d.H),), dev)
            _need(w["ws_down"], "ws_down", torch.uint8, (int4_packed_bytes(1, d.H, d.I_shared),), dev)
        else:
            _need(w["ws_gate_up"], "ws_gate_up", dt, (2 * d.I_shared, d.H), dev)
            _need(w["ws_down"], "ws_down", dt, (d.H, d.I_shared), dev)
    return _Weights(w["w_router"].data_ptr(), None if bias is None else bias.data_ptr(),
                    w["w_gate_up"].data_ptr(), w["w_down"].data_ptr(),
                    w["ws_gate_up"].data_ptr() if d.I_shared > 0 else None,
                    w["ws_down"].data_ptr() if d.I_shared > 0 else None)


def _workspace(nbytes: int, dev, ws):
    if ws is not None:
        if ws.dtype != torch.uint8 or ws.numel() < nbytes or not ws.is_cuda:
            raise ValueError(f"workspace must be a uint8 GPU tensor of >= {nbytes} bytes")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


# --------------------------------------------------------------------------- entry points

def moe_workspace_bytes(d: MoEDims) -> int:
    return int(lib().bdd_moe_workspace_bytes(ctypes.byref(d.c())))


def lmhead_workspace_bytes(T: int, H: int, V: int) -> int:
    return int(lib().bdd_lmhead_workspace_bytes(T, H, V))


def round_workspace_bytes(d: MoEDims, V: int) -> int:
    return int(lib().bdd_round_workspace_bytes(ctypes.byref(d.c()), V))


def device_cus() -> int:
    return int(lib().bdd_device_cus())


def timing_enable(on: bool, filter: str | None = None):
    """Bracket the library's kernel launches with hipEvents (see bdd_timing_enable)."""
    _check(lib().bdd_timing_enable(1 if on else 0, None if filter is None else filter.encode()))


def timing_read(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} recorded since the last read."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    tot = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = lib().bdd_timing_read(max_kernels, names, tot, cnt)
    if n < 0:
        _check(n)
    out = {}
    for k in range(min(n, max_kernels)):
        nm = names.raw[64 * k:64 * (k + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (float(tot[k]), int(cnt[k]))
    return out


def moe_block_forward(d: MoEDims, weights: dict, h: torch.Tensor, coreset_top_p: float = 1.0,
                      ws: torch.Tensor | None = None, out: dict | None = None, stream=None) -> dict:
    """One MoE layer on the block (see bdd_moe_block_forward).  Returns a dict
    with y, xhat, topk_idx, topk_w, n_distinct, coreset_bits, coreset_size."""
    dev = h.device
    _need(h, "h", torch.float32, (d.T, d.H))
    cw = _weights(d, weights, dev)
    o = out if out is not None else {
        "y": torch.empty((d.T, d.H), dtype=torch.float32, device=dev),
        "xhat": torch.empty((d.T, d.H), dtype=d.torch_dtype, device=dev),
        "topk_idx": torch.empty((d.T, d.K), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((d.T, d.K), dtype=torch.float32, device=dev),
        "n_distinct": torch.empty(1, dtype=torch.int32, device=dev),
        "coreset_bits": torch.empty((d.E + 31) // 32, dtype=torch.int32, device=dev),
        "coreset_size": torch.empty(1, dtype=torch.int32, device=dev),
    }
    nb = moe_workspace_bytes(d)
    ws = _workspace(nb, dev, ws)
    _check(lib().bdd_moe_block_forward(
        ctypes.byref(d.c()), ctypes.byref(cw), _ptr(h), float(coreset_top_p), _ptr(o["y"]),
        _ptr(o["xhat"]), _ptr(o["topk_idx"]), _ptr(o["topk_w"]), _ptr(o["n_distinct"]),
        _ptr(o["coreset_bits"]), _ptr(o["coreset_size"]), _ptr(ws), ws.numel(), _stream(stream)))
    return o


def coreset_select(router_prob: torch.Tensor, topk_idx: torch.Tensor, top_p: float,
                   stream=None):
    """Block coreset of a routing (see bdd_coreset_select).  Returns
    (coreset_bits int32 [ceil(E/32)], coreset_size int32 [1], expert_mass fp32 [E])."""
    T, E = router_prob.shape
    K = topk_idx.shape[1]
    dev = router_prob.device
    _need(router_prob, "router_prob", torch.float32, (T, E))
    _need(topk_idx, "topk_idx", torch.int32, (T, K), dev)
    bits = torch.empty((E + 31) // 32, dtype=torch.int32, device=dev)
    size = torch.empty(1, dtype=torch.int32, device=dev)
    mass = torch.empty(E, dtype=torch.float32, device=dev)
    _check(lib().bdd_coreset_select(_ptr(router_prob), _ptr(topk_idx), T, E, K, float(top_p),
                                    _ptr(bits), _ptr(size), _ptr(mass), _stream(stream)))
    return bits, size, mass


@dataclass
class LMHead:
    """LM-head weight [V][H] in the packed tile layout (see bdd_lmhead_pack and
    bdd_lmhead_pack_int4).  ``dtype`` is the type of the hidden states it
    takes; ``int4`` marks 4-bit weights (hidden states bf16)."""
    packed: torch.Tensor  # uint8, bdd_lmhead_packed_bytes(V, H, cdtype) bytes
    V: int
    H: int
    dtype: torch.dtype
    int4: bool = False

    @property
    def cdtype(self) -> int:
        if self.int4:
            return BDD_INT4
        return BDD_BF16 if self.dtype == torch.bfloat16 else BDD_F32


def pack_lm_head(w_lm: torch.Tensor, stream=None) -> LMHead:
    """Pack w_lm [V][H] (bf16 or fp32, on the GPU) for the LM head."""
    V, H = w_lm.shape
    dt = w_lm.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("w_lm must be float32 or bfloat16")
    _need(w_lm, "w_lm", dt, (V, H))
    cdt = BDD_BF16 if dt == torch.bfloat16 else BDD_F32
    nb = int(lib().bdd_lmhead_packed_bytes(V, H, cdt))
    if nb == 0:
        raise BddError(-1, f"cannot pack an LM head of shape {(V, H)}")
    packed = torch.empty(nb, dtype=torch.uint8, device=w_lm.device)
    _check(lib().bdd_lmhead_pack(_ptr(w_lm), V, H, cdt, _ptr(packed), _stream(stream)))
    return LMHead(packed, V, H, dt)


def pack_int4(codes: torch.Tensor, scales: torch.Tensor, stream=None) -> torch.Tensor:
    """Pack 4-bit weight matrices for the 4-bit expert kernels (bdd_pack_int4):
    codes uint8 [n][rows][cols/2] or [rows][cols/2] (column 2j in the low
    nibble of byte j, nibble n standing for n - 8), scales bf16 [n][rows][cols/128]
    or [rows][cols/128], on the GPU.  Returns the packed uint8 tensor."""
    if codes.dim() == 2:
        codes, scales = codes.unsqueeze(0), scales.unsqueeze(0)
    n, rows, half = codes.shape
    cols = 2 * half
    _need(codes, "codes", torch.uint8, (n, rows, half))
    _need(scales, "scales", torch.bfloat16, (n, rows, cols // 128), codes.device)
    nb = int4_packed_bytes(n, rows, cols)
    if nb == 0:
        raise BddError(-2, f"cannot pack 4-bit matrices of shape {(n, rows, cols)}")
    packed = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    _check(lib().bdd_pack_int4(_ptr(codes), _ptr(scales), n, rows, cols, _ptr(packed), _stream(stream)))
    return packed


def pack_lm_head_int4(codes: torch.Tensor, scales: torch.Tensor, stream=None) -> LMHead:
    """Pack a 4-bit LM head (see bdd_lmhead_pack_int4): codes uint8 [V][H/2]
    (column 2j in the low nibble of byte j, nibble n standing for n - 8) and
    scales bf16 [V][H/128], both on the GPU."""
    V, half = codes.shape
    H = 2 * half
    _need(codes, "codes", torch.uint8, (V, half))
    _need(scales, "scales", torch.bfloat16, (V, H // 128), codes.device)
    nb = int(lib().bdd_lmhead_packed_bytes(V, H, BDD_INT4))
    if nb == 0:
        raise BddError(-1, f"cannot pack a 4-bit LM head of shape {(V, H)}")
    packed = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    _check(lib().bdd_lmhead_pack_int4(_ptr(codes), _ptr(scales), V, H, _ptr(packed), _stream(stream)))
    return LMHead(packed, V, H, torch.bfloat16, int4=True)


def lmhead_confidence_commit(hhat: torch.Tensor, lm: LMHead, tokens: torch.Tensor,
                             threshold: float = 0.95, ws: torch.Tensor | None = None,
                             conf=None, choice=None, round_info=None, stream=None):
    """LM head + confidence + LowConfidence commit (see
    bdd_lmhead_confidence_commit).  ``tokens`` (int32 [T], MASK = -1) is
    updated in place.  Returns (conf, choice, round_info)."""
    T, H = hhat.shape
    V = lm.V
    dev = hhat.device
    dt = hhat.dtype
    if dt != lm.dtype or H != lm.H:
        raise ValueError(f"hhat {tuple(hhat.shape)} {dt} does not match the LM head (H={lm.H}, {lm.dtype})")
    _need(hhat, "hhat", dt, (T, H))
    if lm.packed.device != dev:
        raise ValueError("LM head and hhat are on different devices")
    _need(tokens, "tokens", torch.int32, (T,), dev)
    conf = torch.empty(T, dtype=torch.float32, device=dev) if conf is None else conf
    choice = torch.empty(T, dtype=torch.int32, device=dev) if choice is None else choice
    round_info = torch.empty(4, dtype=torch.int32, device=dev) if round_info is None else round_info
    nb = lmhead_workspace_bytes(T, H, V)
    ws = _workspace(nb, dev, ws)
    _check(lib().bdd_lmhead_confidence_commit(
        _ptr(hhat), _ptr(lm.packed), T, H, V, lm.cdtype,
        float(threshold), _ptr(tokens), _ptr(conf), _ptr(choice), _ptr(round_info), _ptr(ws),
        ws.numel(), _stream(stream)))
    return conf, choice, round_info


class RoundPlan:
    """Marshalled arguments of bdd_block_denoise_round for a fixed set of
    layers and LM head, so repeated rounds only pass pointers."""

    def __init__(self, d: MoEDims, layers: list, lm: LMHead, coreset_top_p: float = 1.0,
                 threshold: float = 0.95):
        dev = lm.packed.device
        self.d, self.dev = d, dev
        self.V = lm.V
        if lm.H != d.H or lm.dtype != d.torch_dtype or lm.int4 != (d.wdtype == BDD_INT4):
            raise ValueError("LM head does not match the layer dims (a round's head has the layers' weight type: "
                             "bf16, fp32, or 4-bit with 4-bit experts)")
        self.lm = lm
        self.layers = layers  # keep the tensors alive
        arr = (_Weights * max(1, len(layers)))()
        for i, w in enumerate(layers):
            arr[i] = _weights(d, w, dev)
        self.c_layers = arr
        self.c_dims = d.c()
        self.top_p = float(coreset_top_p)
        self.threshold = float(threshold)
        self.ws = _workspace(round_workspace_bytes(d, self.V), dev, None)

    def __call__(self, x_in, tokens, conf, choice, round_info, layer_topk_idx=None,
                 layer_n_distinct=None, hhat_out=None, stream=None, layer_xhat=None):
        d = self.d
        _need(x_in, "x_in", torch.float32, (d.T, d.H), self.dev)
        _need(tokens, "tokens", torch.int32, (d.T,), self.dev)
        _need(conf, "conf", torch.float32, (d.T,), self.dev)
        _need(choice, "choice", torch.int32, (d.T,), self.dev)
        _need(round_info, "round_info", torch.int32, (4,), self.dev)
        L = len(self.layers)
        if layer_topk_idx is not None:
            _need(layer_topk_idx, "layer_topk_idx", torch.int32, (L, d.T, d.K), self.dev)
        if layer_n_distinct is not None:
            _need(layer_n_distinct, "layer_n_distinct", torch.int32, (L,), self.dev)
        if hhat_out is not None:
            _need(hhat_out, "hhat_out", d.torch_dtype, (d.T, d.H), self.dev)
        if layer_xhat is not None:
            _need(layer_xhat, "layer_xhat", d.torch_dtype, (L, d.T, d.H), self.dev)
        _check(lib().bdd_block_denoise_round(
            ctypes.byref(self.c_dims), L, self.c_layers, self.top_p, _ptr(self.lm.packed), self.V,
            self.threshold, _ptr(x_in), _ptr(tokens), _ptr(conf), _ptr(choice), _ptr(round_info),
            _ptr(layer_topk_idx), _ptr(layer_n_distinct), _ptr(layer_xhat), _ptr(hhat_out), _ptr(self.ws),
            self.ws.numel(), _stream(stream)))


def block_denoise_round_noalloc(plan: "RoundPlan", x_in, tokens, conf, choice, round_info,
                                layer_topk_idx=None, layer_n_distinct=None, hhat_out=None, stream=None):
    """The round of ``plan`` through bdd_block_denoise_round_noalloc: the
    library's static per-GPU scratch instead of the plan's workspace (no
    device allocation in the call).  Same outputs as plan(...)."""
    d = plan.d
    _need(x_in, "x_in", torch.float32, (d.T, d.H), plan.dev)
    _need(tokens, "tokens", torch.int32, (d.T,), plan.dev)
    _need(conf, "conf", torch.float32, (d.T,), plan.dev)
    _need(choice, "choice", torch.int32, (d.T,), plan.dev)
    _need(round_info, "round_info", torch.int32, (4,), plan.dev)
    L = len(plan.layers)
    if layer_topk_idx is not None:
        _need(layer_topk_idx, "layer_topk_idx", torch.int32, (L, d.T, d.K), plan.dev)
    if layer_n_distinct is not None:
        _need(layer_n_distinct, "layer_n_distinct", torch.int32, (L,), plan.dev)
    if hhat_out is not None:
        _need(hhat_out, "hhat_out", d.torch_dtype, (d.T, d.H), plan.dev)
    _check(lib().bdd_block_denoise_round_noalloc(
        ctypes.byref(plan.c_dims), L, plan.c_layers, plan.top_p, _ptr(plan.lm.packed), plan.V, plan.threshold,
        _ptr(x_in), _ptr(tokens), _ptr(conf), _ptr(choice), _ptr(round_info), _ptr(layer_topk_idx),
        _ptr(layer_n_distinct), None, _ptr(hhat_out), _stream(stream)))


def generate_fits(prompt_len: int, max_new_tokens: int, block_size: int) -> bool:
    """Whether a request fits the 131072-token bound (see bdd_generate_fits)."""
    return bool(lib().bdd_generate_fits(prompt_len, max_new_tokens, block_size))


def generate(plan: "RoundPlan", x_rounds: torch.Tensor, max_new_tokens: int, max_steps: int,
             eos_token: int, prompt_len: int = 0, out_tokens: torch.Tensor | None = None, stream=None,
             rounds_per_read: int = 0, with_fallbacks: bool = False):
    """Multi-block generation (bdd_generate) with the plan's layers, LM head,
    coreset and threshold.  x_rounds [n_blocks][max_steps][T][H] fp32 on the
    device.  rounds_per_read 0: one host read per block.  Returns (tokens
    int32 [n_blocks][T], block_rounds list, n_returned, stop) where stop is
    "eos", "length" or "unresolved"; with_fallbacks adds the per-block
    fallback counts as a fifth element."""
    d = plan.d
    if x_rounds.dim() != 4 or x_rounds.shape[1] != max_steps or tuple(x_rounds.shape[2:]) != (d.T, d.H):
        raise ValueError(f"x_rounds must be [n_blocks][{max_steps}][{d.T}][{d.H}]")
    _need(x_rounds, "x_rounds", torch.float32, tuple(x_rounds.shape), plan.dev)
    nb = x_rounds.shape[0]
    if out_tokens is None:
        out_tokens = torch.empty((nb, d.T), dtype=torch.int32, device=plan.dev)
    _need(out_tokens, "out_tokens", torch.int32, (nb, d.T), plan.dev)
    wsb = int(lib().bdd_generate_workspace_bytes(ctypes.byref(plan.c_dims), plan.V))
    if getattr(plan, "gen_ws", None) is None or plan.gen_ws.numel() < wsb:
        plan.gen_ws = _workspace(wsb, plan.dev, None)
    rounds = (ctypes.c_int32 * nb)()
    fallbacks = (ctypes.c_int32 * nb)()
    result = (ctypes.c_int32 * 3)()
    st = lib().bdd_generate(ctypes.byref(plan.c_dims), len(plan.layers), plan.c_layers, plan.top_p,
                            _ptr(plan.lm.packed), plan.V, plan.threshold, max_steps, rounds_per_read, prompt_len,
                            max_new_tokens, eos_token, _ptr(x_rounds), nb, _ptr(out_tokens), rounds, fallbacks,
                            result, _ptr(plan.gen_ws), plan.gen_ws.numel(), _stream(stream))
    if st not in (0, BDD_UNRESOLVED):
        _check(st)
    stop = "unresolved" if st == BDD_UNRESOLVED else ("eos" if result[2] == 1 else "length")
    n = int(result[1])
    out = (out_tokens, [int(rounds[i]) for i in range(n)], int(result[0]), stop)
    return out + ([int(fallbacks[i]) for i in range(n)],) if with_fallbacks else out


class RoundGraph:
    """A round bound to fixed buffers and captured as a HIP graph
    (bdd_round_graph_create); call launch() to enqueue one round."""

    def __init__(self, plan: RoundPlan, x_in, tokens, conf, choice, round_info, layer_topk_idx=None,
                 layer_n_distinct=None, hhat_out=None):
        d = plan.d
        _need(x_in, "x_in", torch.float32, (d.T, d.H), plan.dev)
        _need(tokens, "tokens", torch.int32, (d.T,), plan.dev)
        _need(conf, "conf", torch.float32, (d.T,), plan.dev)
        _need(choice, "choice", torch.int32, (d.T,), plan.dev)
        _need(round_info, "round_info", torch.int32, (4,), plan.dev)
        self.keep = (plan, x_in, tokens, conf, choice, round_info, layer_topk_idx, layer_n_distinct, hhat_out)
        h = ctypes.c_void_p()
        _check(lib().bdd_round_graph_create(
            ctypes.byref(plan.c_dims), len(plan.layers), plan.c_layers, plan.top_p, _ptr(plan.lm.packed),
            plan.V, plan.threshold, _ptr(x_in), _ptr(tokens), _ptr(conf), _ptr(choice), _ptr(round_info),
            _ptr(layer_topk_idx), _ptr(layer_n_distinct), None, _ptr(hhat_out), _ptr(plan.ws), plan.ws.numel(),
            ctypes.byref(h)))
        self.handle = h
        # bound now: at interpreter exit the module's globals may be gone before __del__ runs
        self._destroy = lib().bdd_round_graph_destroy

    def launch(self, stream=None):
        _check(lib().bdd_round_graph_launch(self.handle, _stream(stream)))

    def __del__(self):
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self.handle = None


def block_denoise_round(d: MoEDims, layers: list, lm: LMHead, x_in: torch.Tensor,
                        tokens: torch.Tensor, threshold: float = 0.95, coreset_top_p: float = 1.0,
                        layer_topk_idx=None, layer_n_distinct=None, hhat_out=None, stream=None):
    """One full denoising round (see bdd_block_denoise_round).  ``tokens`` is
    updated in place.  Returns (conf, choice, round_info)."""
    plan = RoundPlan(d, layers, lm, coreset_top_p, threshold)
    dev = lm.packed.device
    conf = torch.empty(d.T, dtype=torch.float32, device=dev)
    choice = torch.empty(d.T, dtype=torch.int32, device=dev)
    ri = torch.empty(4, dtype=torch.int32, device=dev)
    plan(x_in, tokens, conf, choice, ri, layer_topk_idx, layer_n_distinct, hhat_out, stream)
    return conf, choice, ri
