"""CPU checks of the C ABI: the library loads, exports every function that
include/bdd.h declares, sizes workspaces, and rejects bad arguments on the
host before touching a GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import block_diffusion_decode_amd as bdd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bdd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bdd.LIB_PATH),
                                reason="libbdd.so not built (run __graft_entry__.build())")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bdd_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("bdd_moe_block_forward", "bdd_coreset_select", "bdd_lmhead_confidence_commit",
              "bdd_block_denoise_round"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bdd.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert sorted(bdd.EXPORTS) == sorted(_declared())


def test_status_strings():
    L = bdd.lib()
    assert L.bdd_status_string(0) == b"BDD_OK"
    assert L.bdd_status_string(-1) == b"BDD_ERR_INVALID_ARG"
    assert L.bdd_status_string(-3) == b"BDD_ERR_WORKSPACE"


def test_workspace_queries():
    d = bdd.MoEDims(32, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    m = bdd.moe_workspace_bytes(d)
    # at least the per-pick activations and outputs: T*K*(I + H) fp32
    assert m >= 32 * 8 * (512 + 2048) * 4
    assert bdd.round_workspace_bytes(d, 248320) > m
    assert bdd.lmhead_workspace_bytes(32, 2048, 248320) > 0
    assert bdd.moe_workspace_bytes(bdd.MoEDims(64, 2048, 256, 8, 512, 512, bdd.BDD_BF16)) > m
    bad = bdd.MoEDims(65, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    assert bdd.moe_workspace_bytes(bad) == 0
    assert bdd.lmhead_workspace_bytes(0, 2048, 10) == 0
    assert bdd.lmhead_workspace_bytes(65, 2048, 10) == 0


def _call_moe(d):
    L = bdd.lib()
    w = bdd._Weights(1, None, 1, 1, 1, 1)
    return L.bdd_moe_block_forward(ctypes.byref(d.c()), ctypes.byref(w), ctypes.c_void_p(1), 1.0,
                                   ctypes.c_void_p(1), None, ctypes.c_void_p(1), ctypes.c_void_p(1),
                                   ctypes.c_void_p(1), None, None, None, 0, None)


@pytest.mark.parametrize("dims,status", [
    ((0, 256, 16, 4, 128, 128, 0), -1),       # T < 1
    ((65, 256, 16, 4, 128, 128, 0), -2),      # T > 64
    ((8, 256, 16, 17, 128, 128, 0), -1),      # K > E
    ((8, 250, 16, 4, 128, 128, 0), -2),       # H not a multiple of 128
    ((8, 288, 16, 4, 128, 128, 0), -2),       # H multiple of 32, not of 128
    ((8, 256, 300, 4, 128, 128, 0), -2),      # E > 256
    ((8, 256, 16, 4, 128, 128, 7), -1),       # bad dtype
    ((8, 256, 16, 4, 128, 128, 0), -3),       # valid dims, missing workspace
])
def test_moe_forward_rejects_on_host(dims, status):
    assert _call_moe(bdd.MoEDims(*dims)) == status
    assert bdd.lib().bdd_last_error()


def test_lmhead_rejects_bad_threshold_and_shapes():
    L = bdd.lib()
    p = ctypes.c_void_p(1)
    args = lambda T, H, V, dt, thr: (p, p, T, H, V, dt, thr, p, p, p, p, None, 0, None)
    assert L.bdd_lmhead_confidence_commit(*args(32, 2048, 1000, 1, 0.0)) == -1
    assert L.bdd_lmhead_confidence_commit(*args(32, 2048, 1000, 1, 1.5)) == -1
    assert L.bdd_lmhead_confidence_commit(*args(32, 4096, 1000, 1, 0.95)) == -2   # LDS budget
    assert L.bdd_lmhead_confidence_commit(*args(32, 2048, 1000, 1, 0.95)) == -3   # no workspace
    assert L.bdd_lmhead_confidence_commit(None, p, 32, 2048, 10, 1, 0.95, p, p, p, p, p, 1 << 30, None) == -1


def test_int4_lm_head_sizes_and_host_checks():
    L = bdd.lib()
    # 16-row tiles: 8 H bytes of codes and H / 128 * 32 bytes of scales each
    for V, H in [(16, 128), (5003, 256), (248320, 2048)]:
        tiles = (V + 15) // 16
        assert L.bdd_lmhead_packed_bytes(V, H, bdd.BDD_INT4) == tiles * 8 * H + tiles * (H // 128) * 32
    assert L.bdd_lmhead_packed_bytes(100, 192, bdd.BDD_INT4) == 0
    assert L.bdd_lmhead_packed_bytes(100, 192, bdd.BDD_BF16) == 7 * 16 * 192 * 2
    p = ctypes.c_void_p(1)
    assert L.bdd_lmhead_pack_int4(None, p, 10, 256, p, None) == -1
    assert L.bdd_lmhead_pack_int4(p, p, 0, 256, p, None) == -1
    assert L.bdd_lmhead_pack_int4(p, p, 10, 192, p, None) == -2
    # the float pack does not take the 4-bit type, and INT4 heads need H % 128 == 0
    assert L.bdd_lmhead_pack(p, 10, 256, bdd.BDD_INT4, p, None) == -1
    args = lambda H, dt: (p, p, 32, H, 1000, dt, 0.95, p, p, p, p, None, 0, None)
    assert L.bdd_lmhead_confidence_commit(*args(192, bdd.BDD_INT4)) == -2
    assert L.bdd_lmhead_confidence_commit(*args(2048, bdd.BDD_INT4)) == -3   # no workspace
    assert L.bdd_lmhead_confidence_commit(*args(2048, 3)) == -1


def test_coreset_rejects_on_host():
    L = bdd.lib()
    p = ctypes.c_void_p(1)
    assert L.bdd_coreset_select(p, p, 4, 16, 4, 0.0, p, p, None, None) == -1
    assert L.bdd_coreset_select(p, p, 4, 16, 20, 0.9, p, p, None, None) == -1
    assert L.bdd_coreset_select(None, p, 4, 16, 4, 0.9, p, p, None, None) == -1


def test_round_rejects_null_layers():
    L = bdd.lib()
    d = bdd.MoEDims(8, 256, 16, 4, 128, 128, 0)
    p = ctypes.c_void_p(1)
    st = L.bdd_block_denoise_round(ctypes.byref(d.c()), 2, None, 1.0, p, 1024, 0.95, p, p, p, p, p,
                                   None, None, None, None, None, 0, None)
    assert st == -1


def test_generate_request_bound():
    # prompt + new tokens, rounded up to whole blocks, at most 131072
    # (goremy.ai page, "What generation controls ship by default?")
    fits = bdd.generate_fits
    assert fits(0, 1, 32) and fits(131072 - 32, 32, 32) and fits(131072 - 32, 1, 32)
    assert not fits(131072 - 31, 1, 32)        # the final block needs 32 positions
    assert not fits(131040, 33, 32)            # two blocks past 131040
    assert fits(131072 - 64, 33, 32)
    assert not fits(-1, 1, 32) and not fits(0, 0, 32)
    d = bdd.MoEDims(32, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    assert bdd.lib().bdd_generate_workspace_bytes(ctypes.byref(d.c()), 248320) > bdd.round_workspace_bytes(d, 248320)


def test_generate_rejects_on_the_host():
    # rejected before any pointer is used or anything is enqueued
    L = bdd.lib()
    d = bdd.MoEDims(32, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    rounds = (ctypes.c_int32 * 4)()
    result = (ctypes.c_int32 * 3)()
    st = L.bdd_generate(ctypes.byref(d.c()), 1, None, 1.0, None, 248320, 0.95, 32, 0, 131072 - 31, 1, 0, None, 4,
                        None, rounds, None, result, None, 0, None)
    assert st == -1 and b"131072" in L.bdd_last_error()
    st = L.bdd_generate(ctypes.byref(d.c()), 1, None, 1.0, None, 248320, 0.95, 0, 0, 0, 32, 0, None, 4,
                        None, rounds, None, result, None, 0, None)
    assert st == -1   # max_steps < 1
    st = L.bdd_generate(ctypes.byref(d.c()), 1, None, 1.0, None, 248320, 0.95, 32, -1, 0, 32, 0, None, 4,
                        None, rounds, None, result, None, 0, None)
    assert st == -1   # rounds_per_read < 0
    st = L.bdd_generate(ctypes.byref(d.c()), 1, None, 1.0, None, 248320, 0.95, 32, 0, 0, 65, 0, None, 2,
                        None, rounds, None, result, None, 0, None)
    assert st == -1   # three blocks needed, two given


def test_generate_bound_matches_the_oracle():
    # the library's host check of the request bound against the oracle's reading
    import oracle as O
    for T in (1, 4, 8, 32):
        for prompt in (0, 1, 1000, 131072 - 64, 131072 - 33, 131072 - 32, 131072 - 31, 131072 - 1, 131072):
            for new in (1, 2, 31, 32, 33, 64, 65, 131072):
                assert bool(bdd.generate_fits(prompt, new, T)) == O.request_fits(prompt, new, T), (T, prompt, new)


def test_noalloc_round_rejects_dims_beyond_its_scratch():
    # checked on the host before any device call: dims whose round workspace
    # exceeds the static scratch are refused, invalid dims get the round's error
    L = bdd.lib()
    p = ctypes.c_void_p(1)
    w = bdd._Weights(1, None, 1, 1, 1, 1)
    args = lambda d, V: (ctypes.byref(d.c()), 1, ctypes.byref(w), 1.0, p, V, 0.95, p, p, p, p, p,
                         None, None, None, None, None)
    big = bdd.MoEDims(32, 8192, 256, 8, 8192, 8192, bdd.BDD_F32)
    assert bdd.round_workspace_bytes(big, 1000) > bdd.NOALLOC_SCRATCH_BYTES
    assert L.bdd_block_denoise_round_noalloc(*args(big, 1000)) == -2
    assert b"static scratch" in L.bdd_last_error()
    bad = bdd.MoEDims(65, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    assert L.bdd_block_denoise_round_noalloc(*args(bad, 1000)) == -2
    clover = bdd.MoEDims(32, 2048, 256, 8, 512, 512, bdd.BDD_BF16)
    assert 0 < bdd.round_workspace_bytes(clover, 248320) <= bdd.NOALLOC_SCRATCH_BYTES
