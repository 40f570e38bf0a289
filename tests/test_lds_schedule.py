"""The LDS staging of the bf16 kernels is race-free (host model, no GPU).

tests/lds_schedule_model.cpp replays every wave's program of the pipelined dense
kernel (8 and 4 waves, head_dim 96, with and without the RoPE angle table of its
prologue) and of the phased kernel (head_dim 64, 96 and
128) for every key count 1..1100 and several long ones, using the schedule functions
the kernels call (vit_perception_encoder_amd/csrc/schedule.hpp), and checks that no
LDS region is read before its DMA is waited for and published by a barrier, none is
overwritten before its last read or while a DMA into it may still land, and every DMA
is waited for.  Planted schedule mistakes must each be reported."""
import shutil
import subprocess
from pathlib import Path

import pytest

pytestmark = pytest.mark.cpu
ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path_factory.mktemp("lds") / "lds_schedule_model"
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-o", str(exe),
                    str(ROOT / "tests" / "lds_schedule_model.cpp")], check=True)
    return exe


def test_kernel_schedules_are_race_free(model):
    r = subprocess.run([str(model)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")


@pytest.mark.parametrize("mutation", [
    "pipe_issue_early",            # the tile after next issued at a sync: one tile never arrives
    "pipe_issue_before_barrier",   # a DMA into a stage other waves may still read
    "pipe_sync_even",              # barriers on even iterations instead of odd
    "pipe_no_final_barrier",       # output staging over K/V another wave still reads
    "pipe_prologue_short",         # the prologue waits for one DMA too few
    "pipe_prologue_old_count",     # tile 1 issued after the first barrier, the wait still leaving its DMA out
    "phased_issue_early",          # a stage refilled two phases early
    "phased_wait_late",            # a tile waited for two phases late
    "split_k_early",               # key-split: K of tile j+3 into the slot of K of tile j+1
    "split_leave_k",               # key-split: K of tile j+1 left in flight at its barrier
    "split_merge_no_barrier",      # key-split: group 0 reads group 1's partials before they are stored
])
def test_planted_schedule_mistakes_are_caught(model, mutation):
    r = subprocess.run([str(model), mutation], capture_output=True, text=True)
    assert r.returncode == 1 and r.stdout.startswith("violation"), r.stdout
