"""The boundary as a C ABI: a plain C99 program that includes only include/relbias_attn.h is
compiled with gcc (-Wall -Wextra -Werror -pedantic), linked against the built library and run.
It checks argument errors, empty problems, workspace sizes and the version string, none of which
needs a device (CPU tier)."""

import os
import shutil
import subprocess

import pytest

import transformer_attention_learned_amd as rba

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_c_client_builds_links_and_runs(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = rba.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    exe = str(tmp_path / "client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_client.c"),
           lib, "-Wl,-rpath," + os.path.dirname(lib), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)
