"""CPU check of the lane addresses of every direct-to-LDS tile load.

The step kernels compute the global address of each 16-byte tile load from
a wave-uniform base and a 32-bit lane offset (csrc/rba_addr.h).  A lane
offset that goes negative wraps to about 4 GiB past the base and faults the
GPU; one did, in the last, ragged key tile, before the offset of a ragged
load was taken from the tile's first row.  tests/addr_check.cpp calls the
kernels' own address functions on the host for every tile, wave, lane,
load and ragged chunk length (d = 64 and 128; the K / V tiles of the
forward and dQ passes, the K, Q, dO, LSE and delta loads of the dK / dV
pass) and counts reads that leave their tensor or head, or fetch a row or
chunk other than the one their LDS slot holds.  The same program built
with the earlier ragged offset must find out-of-range reads, which shows
that the enumeration reaches the case that faulted."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_sequence_parallelism_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "addr_check.cpp")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def _run(tmp_path, *defines):
    exe = str(tmp_path / ("addr_check" + "".join(d.lower() for d in defines)))
    cmd = [_hipcc(), "--offload-host-only", "-x", "hip", "-O2", "-std=c++17", f"-I{CSRC}",
           *[f"-D{d}" for d in defines], SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    res = {}
    for line in out.stdout.splitlines():
        m = re.match(r"(\S+) checked=(\d+) bad=(\d+) misplaced=(\d+)", line)
        assert m, line
        res[m.group(1)] = tuple(int(x) for x in m.groups()[1:])
    return res


def test_tile_load_addresses_stay_in_bounds(tmp_path):
    res = _run(tmp_path)
    assert set(res) == {"kv_tiles_d64", "kv_tiles_d128", "dkdv_k_d64", "dkdv_q_do_d64", "dkdv_lse_d64",
                        "dkdv_k_d128", "dkdv_q_do_d128", "dkdv_lse_d128"}
    for name, (checked, bad, misplaced) in res.items():
        assert checked > 0, name
        assert bad == 0, f"{name}: {bad} of {checked} reads leave their tensor or head"
        assert misplaced == 0, f"{name}: {misplaced} reads fetch the wrong row or chunk"


def test_earlier_ragged_offset_is_caught(tmp_path):
    res = _run(tmp_path, "PLANT_OLD_RAGGED")
    assert res["kv_tiles_d64"][1] > 0 and res["kv_tiles_d128"][1] > 0
