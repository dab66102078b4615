"""The XCD-aware tile schedule (host C++), compiled with g++ and checked on the
CPU for the GPT-2 Large, Llama-3-8B-share, 32B-share and ragged matrix sets."""
import os
import shutil
import subprocess

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpp", "schedule_check.cpp")
INC = os.path.join(ROOT, "matrix_optimizer_step_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", INC, SRC, "-o", exe], check=True)
    return exe


def _grid(shape, tile=256):
    r, c = shape
    m, n = min(r, c), max(r, c)
    mp, np_ = -(-m // tile) * tile, -(-n // tile) * tile
    return mp // tile, np_ // tile, np_, mp


@pytest.mark.parametrize("diag16,pairs", [(16, 0), (9, 1)])
@pytest.mark.parametrize("name", ["gpt2_large_144", "llama3_8b_share_28", "qwen32b_share_14",
                                  "ragged_illcond_64"])
def test_schedule_covers_every_tile_once_and_balances(checker, name, diag16, pairs):
    # bf16 (9, 1): diagonal tiles cost 9/16 (36 of their 64 blocks) and go in
    # pairs of block rows 2p, 2p+1 (one table entry covers both)
    wl = workloads.get(name)
    lines = "\n".join("%d %d %d %d" % _grid(s) for s in wl.shapes)
    r = subprocess.run([checker, str(diag16), str(pairs)], input=lines, capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_mixed_batch_has_stage_tables_of_different_lengths(checker):
    # the GPU parity case for per-stage launch sizes relies on this
    from tests.test_parity_gpu import MIXED_SHAPES
    lines = "\n".join("%d %d %d %d" % _grid(s) for s in MIXED_SHAPES)
    r = subprocess.run([checker], input=lines, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    _, gram, poly, _ = r.stdout.split()
    assert (int(gram), int(poly)) == (72, 48)
