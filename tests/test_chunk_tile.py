"""The chunk boundaries (ssm::chunk_tile, compiled for the host from the kernels' header)
against exact integer arithmetic: chunk c of nc starts at tile g * floor(c * nu / nc),
nu = ceil(nf / g), capped at nf.  The cases include sequences near the size limit cut
into very many chunks, where the plain product c * nu would pass 2^63."""
import os
import random
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def chunk_tile(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available to build the chunk_tile dump")
    exe = str(tmp_path_factory.mktemp("chunktile") / "dump")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "chunk_tile_dump.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(cases):
        text = "".join(f"{c} {nf} {nc} {g}\n" for c, nf, nc, g in cases)
        out = subprocess.run([exe], input=text, check=True, capture_output=True, text=True)
        return [int(v) for v in out.stdout.split()]
    return run


def exact(c, nf, nc, g):
    nu = -(-nf // g)
    return min(g * (c * nu // nc), nf)


def test_chunk_tile_is_exact(chunk_tile):
    rnd = random.Random(3)
    cases = []
    # the 2.8B plans, every chunk
    cases += [(c, 1024, 54, 1) for c in range(55)] + [(c, 1024, 32, 1) for c in range(33)]
    # sparse intervals (units of g tiles) with a ragged last unit
    cases += [(c, 1001, nc, g) for g in (2, 4, 32) for nc in (1, 3, 7) for c in range(nc + 1)]
    # near the size limit: nf up to 2^42 tiles, up to 10^8 chunks
    for _ in range(300):
        g = rnd.choice([1, 2, 4, 32])
        nf = rnd.randrange(1, 1 << 42)
        nu = -(-nf // g)
        nc = rnd.randrange(1, min(nu, 10 ** 8) + 1)
        c = rnd.randrange(0, nc + 1)
        cases.append((c, nf, nc, g))
    cases.append((10 ** 8 - 1, (1 << 42) - 1, 10 ** 8, 1))
    got = chunk_tile(cases)
    for case, v in zip(cases, got):
        assert v == exact(*case), case
    # boundaries are non-decreasing and end at nf
    for nf, nc, g in ((1 << 40, 99999, 1), (12345, 617, 2)):
        b = chunk_tile([(c, nf, nc, g) for c in range(nc + 1)])
        assert b[0] == 0 and b[-1] == nf and all(x <= y for x, y in zip(b, b[1:]))
