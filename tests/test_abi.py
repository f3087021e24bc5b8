"""The C ABI without a GPU: every declared symbol is exported, argument checks
return their codes before any launch, and the layout arithmetic matches the
documented layout."""
import ctypes
import os
import re

import pytest

from learnable_kv_cache_amd import lte

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lte.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lte_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = lte.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    # and the binding declares a signature for each
    assert set(names) == set(lte.SIGNATURES)


def test_status_strings_and_version():
    L = lte.lib()
    assert L.lte_version() == 1
    for code in range(7):
        assert L.lte_status_string(code)
    assert L.lte_status_string(99) == b"unknown status"


BASE = dict(batch=2, q_heads=8, kv_heads=2, head_dim=128, sink=4, window=32, capacity=16,
            hidden=32)


@pytest.mark.parametrize("change,code", [
    ({}, 0),
    ({"q_heads": 6, "kv_heads": 4}, 1),      # Hq % Hkv != 0
    ({"head_dim": 96}, 2),
    ({"head_dim": 0}, 1),
    ({"window": 4}, 2),                       # receptive field needs w >= 5
    ({"sink": -1}, 1),
    ({"capacity": -3}, 1),
    ({"capacity": 5000}, 2),
    ({"sink": 300}, 2),
    ({"q_heads": 6, "kv_heads": 2}, 2),       # G = 3
    ({"q_heads": 64, "kv_heads": 2}, 2),      # G = 32
    ({"hidden": 16}, 2),
    ({"batch": 0}, 1),
    ({"q_heads": 256, "kv_heads": 256}, 2),   # 32-bit row offsets
])
def test_config_checks(change, code):
    c = lte.Config(**{**BASE, **change})
    assert lte.lib().lte_check_config(ctypes.byref(c.c())) == code


def _layer():
    return lte.Layer(lte.Config(**BASE))


def test_calls_fail_before_launch_on_bad_arguments():
    L = lte.lib()
    layer = _layer()
    cfg = ctypes.byref(layer._c)
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    T = 64
    ws = layer.workspace_bytes(T)
    # null tensors
    assert L.lte_prefill(cfg, T, None, fake, fake, None, fake, None, fake, ws, fake, None) == 1
    # T out of range
    assert L.lte_prefill(cfg, 0, fake, fake, fake, None, fake, None, fake, ws, fake, None) == 1
    assert L.lte_prefill(cfg, 40000, fake, fake, fake, None, fake, None, fake, ws, fake, None) == 2
    # no CNN and no override
    assert L.lte_prefill(cfg, T, fake, fake, fake, None, None, None, fake, ws, fake, None) == 1
    # workspace too small
    assert L.lte_prefill(cfg, T, fake, fake, fake, None, fake, None, fake, ws - 1, fake, None) == 5
    # ragged prefill: null lengths, then the same checks as the equal-length call
    VL = L.lte_prefill_varlen
    assert VL(cfg, T, None, fake, fake, fake, None, fake, None, fake, ws, fake, None) == 1
    assert VL(cfg, T, fake, None, fake, fake, None, fake, None, fake, ws, fake, None) == 1
    assert VL(cfg, 40000, fake, fake, fake, fake, None, fake, None, fake, ws, fake, None) == 2
    assert VL(cfg, T, fake, fake, fake, fake, None, None, None, fake, ws, fake, None) == 1
    assert VL(cfg, T, fake, fake, fake, fake, None, fake, None, fake, ws - 1, fake, None) == 5
    # chunked prefill: bad n, null cache, small workspace, n past the row limit
    good_cnn = lte._CNN(0x1000, 0x1000, 0x1000, 0x1000)
    cw = L.lte_chunk_workspace_bytes(cfg, 8)
    assert cw > 0 and L.lte_chunk_workspace_bytes(cfg, 0) == 0
    assert L.lte_chunk_workspace_bytes(cfg, 40000) == 0
    CH = L.lte_prefill_chunk
    assert CH(cfg, 0, fake, fake, fake, ctypes.byref(good_cnn), fake, fake, cw, fake, None) == 1
    assert CH(cfg, 8, fake, fake, fake, ctypes.byref(good_cnn), None, fake, cw, fake, None) == 1
    assert CH(cfg, 8, fake, fake, fake, None, fake, fake, cw, fake, None) == 1
    assert CH(cfg, 8, fake, fake, fake, ctypes.byref(good_cnn), fake, fake, cw - 1, fake,
              None) == 5
    assert CH(cfg, 40000, fake, fake, fake, ctypes.byref(good_cnn), fake, fake, cw, fake,
              None) == 2
    # decode: null cache, small workspace, CNN with a null member
    assert L.lte_decode_attend(cfg, fake, None, fake, 1 << 30, fake, None) == 1
    assert L.lte_decode_attend(cfg, fake, fake, fake, 16, fake, None) == 5
    bad_cnn = lte._CNN(0x1000, 0, 0x1000, 0x1000)
    assert L.lte_score_evict(cfg, ctypes.byref(bad_cnn), fake, fake, fake, None) == 1
    assert L.lte_cache_init(cfg, None, None) == 1
    # the decode step without a workspace: the same argument checks
    SD = L.lte_decode_step_static
    assert SD(cfg, fake, fake, fake, ctypes.byref(good_cnn), None, fake, None) == 1
    assert SD(cfg, fake, fake, fake, ctypes.byref(bad_cnn), fake, fake, None) == 1
    assert SD(cfg, fake, None, fake, ctypes.byref(good_cnn), fake, fake, None) == 1
    assert L.lte_cache_get_layout(cfg, None) == 1


def test_cache_layout_matches_the_documented_sections():
    layer = _layer()
    c = layer.cfg
    L = layer.cache_layout()
    S = c.sink + c.capacity + c.window
    bg = c.batch * c.kv_heads
    sizes = [("k", bg * S * c.head_dim * 2), ("v", bg * S * c.head_dim * 2),
             ("ret_idx", bg * c.capacity * 4), ("ret_score", bg * c.capacity * 4),
             ("ring_score", bg * c.window * 4), ("count", bg * 4), ("pos", bg * 8),
             ("next_unscored", bg * 8), ("flags", bg * 4), ("weak", bg * 4),
             ("nx_slot", bg * 4), ("nx_score", bg * 4), ("arrive", bg * 4)]
    off = 0
    for name, n in sizes:
        assert L[name] == off, name
        assert L[name] % 256 == 0
        off = (off + n + 255) // 256 * 256
    assert L["total"] == off == layer.cache_bytes()
    # the cache holds exactly s + C + w slots per (b, g)
    assert L["v"] - L["k"] >= bg * S * c.head_dim * 2


def test_workspace_layout():
    layer = _layer()
    c = layer.cfg
    for T in (1, 100, 4096, 32768):
        W = layer.workspace_layout(T)
        bg = c.batch * c.kv_heads
        assert W["rank"] >= W["scores"] + bg * T * 4 and W["thr"] >= W["rank"] + bg * T * 4
        assert W["scores"] > 0            # decode partials sit before the prefill views
        assert W["total"] == layer.workspace_bytes(T)
        assert layer.workspace_bytes(0) <= W["total"]
