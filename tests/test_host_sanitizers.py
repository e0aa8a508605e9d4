"""The host tile-map code (builder, transpose, chooser, time model) built
with AddressSanitizer and UndefinedBehaviorSanitizer by the host compiler
alone (no device code) and run on random geometries: every map must be
internally consistent and the sanitizers must stay silent."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_tile_amd", "csrc")


def test_tile_map_builder_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "tilemap_fuzz")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", CSRC, os.path.join(ROOT, "tests", "c", "tilemap_fuzz.cpp"),
           os.path.join(CSRC, "tilemap.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("host compiler lacks the sanitizer runtimes")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok 300 geometries" in run.stdout
