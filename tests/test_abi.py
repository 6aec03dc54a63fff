"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/dflash.h declares, and rejects bad arguments before
touching the device."""

import ctypes
import os
import re

import pytest

from block_diffusion_drafting_ctx_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libdflash.so not built (python -m block_diffusion_drafting_ctx_amd.build)")
    return _abi.lib()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dflash_fuse_ctx", "dflash_draft_block", "dflash_verify", "dflash_create", "dflash_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(_abi.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert set(_abi.EXPORTED) == set(declared_functions())


def test_version(lib):
    assert "gfx950" in _abi.dflash_version()


def _cfg(**kw):
    base = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=5, ffn=12288, vocab=151936,
                block=16, n_target_layers=5, max_batch=1, max_ctx=4160, max_fuse_rows=17)
    base.update(kw)
    return _abi.make_config(**base)


def test_workspace_bytes_valid_and_invalid(lib):
    assert _abi.dflash_workspace_bytes(_cfg()) > 0
    assert _abi.dflash_workspace_bytes(_cfg(max_batch=32)) > _abi.dflash_workspace_bytes(_cfg())
    for bad in (dict(hidden=100), dict(head_dim=96), dict(n_q_heads=30), dict(vocab=1000), dict(block=0),
                dict(conv_width=2), dict(conv_width=3, block=12), dict(n_layers=9), dict(n_target_layers=0)):
        assert _abi.dflash_workspace_bytes(_cfg(**bad)) == 0, bad


def test_create_rejects_null_arguments_without_a_device(lib):
    cfg = _cfg()
    out = ctypes.c_void_p()
    st = lib.dflash_create(ctypes.byref(cfg), None, None, None, None, None, 0, ctypes.byref(out))
    assert st == _abi.DFLASH_EINVAL
    assert out.value is None
    assert "null" in lib.dflash_last_error().decode()
    bad = _cfg(head_dim=96)
    st = lib.dflash_create(ctypes.byref(bad), None, None, None, None, None, 0, ctypes.byref(out))
    assert st == _abi.DFLASH_EUNSUPPORTED


def test_calls_reject_null_context(lib):
    assert lib.dflash_fuse_ctx(None, 1, None, 1, 0, None, None) == _abi.DFLASH_EINVAL
    assert lib.dflash_verify(None, 1, None, None, 1, 1, None, None, None, None) == _abi.DFLASH_EINVAL
    assert lib.dflash_draft_block(None, 1, None, None, None, None, None) == _abi.DFLASH_EINVAL
    assert lib.dflash_reload_weights(None, None) == _abi.DFLASH_EINVAL
    # the context-free verify checks its sizes on the host before any device call:
    # beyond the static scratch (2000 x 17 x 19 keys), a bad vocabulary, bad n_d
    assert lib.dflash_verify_static(2000, 151936, None, None, 16, 16, None, 100, None, None, None, None, None,
                                    None) == _abi.DFLASH_EINVAL
    assert "static scratch" in lib.dflash_last_error().decode()
    assert lib.dflash_verify_static(1, 1000, None, None, 1, 1, None, 100, None, None, None, None, None,
                                    None) == _abi.DFLASH_EINVAL
    assert lib.dflash_verify_static(1, 1024, None, None, 1, 65, None, 100, None, None, None, None, None,
                                    None) == _abi.DFLASH_EINVAL
    assert lib.dflash_verify_static(0, 1024, None, None, 1, 1, None, 100, None, None, None, None, None,
                                    None) == _abi.DFLASH_OK
    lib.dflash_destroy(None)


def test_workspace_holds_the_tiled_weight_copy(lib):
    # the bf16 copy of every projection matrix lives in the workspace: at the
    # 8B shape that is W_fc + every layer's Q/K/V/O/gate/up/down + W_lm
    H, F, V, L, T = 4096, 12288, 151936, 5, 5
    Nq, Nk = 32 * 128, 8 * 128
    weights = 2 * (H * T * H + V * H + L * ((Nq + 2 * Nk) * H + H * Nq + 2 * F * H + H * F) + L * 2 * Nk * H)
    assert _abi.dflash_workspace_bytes(_cfg()) >= weights


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(ImportError):
        _abi.lib()
