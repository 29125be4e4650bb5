"""The product path and the oracle stay apart (CPU only): nothing under
paged_kv_offload_amd/ imports, includes, loads or names the oracle, the
oracle includes no kvx header and imports neither the package nor the
input generators, and the built library links no oracle code."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_offload_amd")
ORACLE = os.path.join(ROOT, "oracle")


def sources(top, exts):
    for d, _, files in os.walk(top):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_product_never_names_the_oracle():
    for path in sources(PKG, (".py", ".cpp", ".h", ".hip", ".c")):
        with open(path) as f:
            text = f.read()
        assert not re.search(r"\boracle\b|kvx_oracle|kvxo_", text), path


def test_oracle_shares_nothing_with_the_product():
    for path in sources(ORACLE, (".py", ".c", ".h")):
        with open(path) as f:
            text = f.read()
        assert not re.search(r'#include\s+"kvx', text), path
        assert not re.search(r"^\s*(import|from)\s+(paged_kv_offload_amd|synth)\b", text, re.M), path


def test_built_library_links_no_oracle():
    lib = os.path.join(PKG, "libkvx.so")
    if not os.path.exists(lib):
        pytest.skip("libkvx.so is not built")
    out = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    needed = re.findall(r"\(NEEDED\).*\[(.*)\]", out)
    assert needed and not any("oracle" in n for n in needed), needed
    syms = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    assert "kvxo_" not in syms
