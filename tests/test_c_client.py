"""The C ABI from a plain C99 program (no Python, no GPU): include/na.h must
compile as C with warnings as errors, libna.so must link and run, and the
host entry points must agree with the oracle's tile map."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_attention_tile_amd")


@pytest.fixture(scope="module")
def c_output(tmp_path_factory, na):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("c") / "abi_host")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, "-L", LIBDIR, "-lna",
           "-Wl,-rpath," + LIBDIR]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, *vals = line.split()
        out[key] = vals
    return out


def test_c_client_matches_the_oracle(na, c_output):
    grid, window, stride = (30, 48, 80), (18, 24, 24), (16, 8, 8)
    tiles = [int(x) for x in c_output["tiles"]]
    tq, tk = tuple(tiles[:3]), tuple(tiles[3:])
    assert (tq, tk) == tuple(tuple(t) for t in na.na_choose_tiles(grid, window, stride, 128, na.NA_BF16))
    o = oracle.tile_map_stats(grid, window, stride, tq, tk)
    nq, nnz, nfull, nbnd, comp, eff = (int(x) for x in c_output["map"])
    assert (nq, nnz, nfull, nbnd, comp, eff) == (o["n_q_tiles"], o["nnz"], o["n_full"], o["n_boundary"],
                                                o["computed_slots"], o["effective_slots"])
    qptr, kv, nf = oracle.tile_map(grid, window, stride, tq, tk)
    assert int(c_output["kvsum"][0]) == int(np.asarray(kv, dtype=np.int64).sum())
    assert int(c_output["kvsum"][2]) == int(qptr[-1]) == nnz
    assert c_output["sim"][0] == "1" and float(c_output["sim"][1]) == pytest.approx(o["efficiency"], rel=1e-6)
    assert int(c_output["workspace"][0]) == na.na_workspace_bytes(1, 24, 128, grid, window, stride, na.NA_BF16)
    assert int(c_output["bad"][0]) == na.NA_ERR_INVALID_ARG
