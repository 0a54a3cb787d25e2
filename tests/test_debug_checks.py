"""The kept-block and tree-mask checks of the library's debug build, compiled
for the host with the system C++ compiler and run on crafted rows (no GPU)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))

EXPECTED = {
    "good": 0, "range": 1, "order": 2, "duplicate": 2, "padding": 3, "forced_init": 4,
    "forced_local": 4, "count": 5, "negative": 1, "few_good": 0, "few_short": 4,
    "mask_good": 0, "mask_no_self": 0, "mask_high": 6, "mask_later": 7, "mask_bit63": 0,
}


def test_debug_checks_on_the_host(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "debug_checks_host"
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-o", str(exe),
                    os.path.join(HERE, "debug_checks_host.cpp")], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {ln.split()[0]: int(ln.split()[1]) for ln in out.splitlines()}
    assert got == EXPECTED
