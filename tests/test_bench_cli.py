"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard, the
source hash that ties stored counter readings to the kernel code, the
lookup of stored traffic, the bound rule and the count of the receiver slots
that kernels with per-tile receiver lists sweep."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }\n"
    strip = lambda t: " ".join(bench._COMMENT.sub(" ", t).split())
    assert strip(a) == strip(b)
    assert strip("return x + 2;") != strip("return x + 1;")
    h = bench.kernel_source_hash("das_bi_rows_kernel")
    assert len(h) == 16 and h == bench.kernel_source_hash("das_bi_rows_kernel")
    # each kernel's readings depend on its own source: the hashes differ
    hashes = {bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert len(hashes) == len(bench.KERNEL_SOURCES)


def test_stored_traffic_is_none_for_an_unmeasured_workload():
    assert bench.stored_traffic("das_bi_staged_kernel", "no-such-workload") is None
    assert bench.stored_traffic("no_such_kernel", "main") is None


def test_pick_bound():
    import bench
    # algorithmic bytes slower than the flops: HBM
    assert bench.pick_bound(2.0, 1.0, None, None) == "hbm"
    # counted bytes keep HBM at 48% while the VALU is 83% busy: ALU
    assert bench.pick_bound(0.3, 2.0, 0.48, 0.83) == "alu"
    # counted bytes keep HBM busier than the VALU: HBM
    assert bench.pick_bound(0.3, 2.0, 0.9, 0.6) == "hbm"
    # no counters on these sources: the algorithmic rule alone
    assert bench.pick_bound(0.3, 2.0, 0.9, None) == "alu"
    assert bench.pick_bound(0.3, 2.0, None, 0.6) == "alu"


@pytest.mark.parametrize("tile,block", [((16, 16, 1), 8), ((8, 8, 2), 16), ((16, 16, 1), 4)])
def test_listed_slots_against_every_voxel(tile, block):
    """The executed-fraction helper takes each tile's cone test at one voxel
    (nearest the receiver laterally, on the deepest plane).  On a ragged grid
    (tiles cut at every edge) it must count the same live (tile, receiver)
    pairs as the same test evaluated at every voxel of every tile."""
    import numpy as np
    import das_synth
    cfg = das_synth.custom_config("tiny", name="slots", array=(12, 5), grid=(37, 21, 5), voxel=0.4e-3, z0=1e-3,
                                  f_number=1.5)
    rx = das_synth.array_positions(cfg).astype(np.float64)
    (ox, oy, oz), (sx, sy, sz), (nx, ny, nz) = das_synth.voxel_grid(cfg)
    ct = np.cos(np.arctan(1.0 / (2.0 * cfg.f_number)))
    a_, b_ = (1.0 - ct * ct) * 1.001, ct * ct
    px, py, pz = tile
    slots = 0
    for z0 in range(0, nz, pz):
        for y0 in range(0, ny, py):
            for x0 in range(0, nx, px):
                xs = ox + np.arange(x0, min(x0 + px, nx)) * sx
                ys = oy + np.arange(y0, min(y0 + py, ny)) * sy
                zs = oz + np.arange(z0, min(z0 + pz, nz)) * sz
                v = np.stack(np.meshgrid(xs, ys, zs, indexing="ij"), -1).reshape(-1, 3)
                d = v[:, None, :] - rx[None, :, :]
                rho2 = d[..., 0] ** 2 + d[..., 1] ** 2
                live = ((d[..., 2] > 0) & (b_ * rho2 < a_ * d[..., 2] ** 2)).any(0)
                slots += int(np.ceil(live.sum() / block)) * block * px * py * pz
    assert 0 < slots < -(-nx // px) * -(-ny // py) * -(-nz // pz) * px * py * pz * cfg.M
    assert bench.listed_slots(cfg, tile, block) == slots
