"""Properties of the generated gfx950 code that the sources rely on (host only:
hipcc cross-compiles the device code to assembly, no GPU needed).

The LDS DMA is written as inline asm that sets M0 and issues global_load_lds_dwordx4.
LLVM reserves M0 and ignores a clobber of it, so the asm is only correct if the
compiler itself keeps no value in M0: every M0 write in the library's device code
must be the one inside those asm statements, immediately followed by its DMA."""
import re
import shutil
import subprocess
from pathlib import Path

import pytest

pytestmark = pytest.mark.cpu
ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not Path("/opt/rocm/bin/hipcc").exists():
        pytest.skip("hipcc not available")
    from vit_perception_encoder_amd import build as b

    out = tmp_path_factory.mktemp("asm")
    subprocess.run([b.hipcc(), *b.COMMON, *b.DEVICE_FLAGS, "--cuda-device-only", "-S", "-o", str(out / "k.s"),
                    *map(str, b.SOURCES)], check=True, capture_output=True)
    return (out / "k.s").read_text().splitlines()


def test_m0_is_only_written_by_the_dma_asm(asm):
    code = [l.strip() for l in asm if l.strip() and not l.strip().startswith(";") and not l.strip().startswith(".")]
    n_dma = 0
    for i, line in enumerate(code):
        if not re.search(r"\bm0\b", line):
            continue
        assert line.startswith("s_mov_b32 m0,"), f"compiler use of M0: {line}"
        assert code[i + 1].startswith("global_load_lds_dwordx4"), f"M0 write not followed by its DMA: {line}"
        n_dma += 1
    assert n_dma > 100  # every kernel's DMA sites were seen
