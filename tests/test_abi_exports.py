"""The C-ABI library loads and exports every function include/echo.h declares (no GPU calls)."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "echo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(echo_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_matches_binding_table():
    from dsa_indexer_top_amd import binding
    assert _declared() == binding.EXPORTED


def test_library_exports_all_symbols():
    from dsa_indexer_top_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    L = binding.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert "gfx950" in binding.version()
    assert binding.pool_metadata_bytes(2_000_000, 200_000) == 4 * 2_000_000 + 13 * 200_000


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from dsa_indexer_top_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        binding.lib()
