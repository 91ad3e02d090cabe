"""The C-ABI library loads and exports every entry point include/kpage.h declares (CPU only, no compute)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_11_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kpage.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kpage_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_bound_entry_points():
    assert set(_declared_functions()) == set(K.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(K.LIB_PATH):
        pytest.fail(f"{K.LIB_PATH} not built")
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(K, "_lib_handle", None)
    with pytest.raises(K.KpageError):
        K.lib()
