"""The C-ABI library loads and exports every entry point include/ja.h
declares; the ctypes binding binds exactly those names.  No GPU needed."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ja.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ja_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    from tensor_relational_join_amd import binding as B

    declared = _declared()
    assert len(declared) >= 30
    lib = B.raw()
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (ja_[a-z0-9_]+)$", out, flags=re.M)))
    assert exported == declared


def test_binding_covers_the_header_exactly():
    from tensor_relational_join_amd import binding as B

    assert B.EXPORTED == _declared()
    for name in B.EXPORTED:
        assert callable(getattr(B, name)), name


def test_version_and_status_strings():
    from tensor_relational_join_amd import binding as B

    assert B.ja_abi_version() == 1
    for code, name in B.STATUS.items():
        assert B.ja_status_str(code) == name
    assert B.ja_status_str(-99) == "JA_ERR_UNKNOWN"
