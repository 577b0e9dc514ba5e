"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Bar: max|err| <= 1e-4 max|oracle| and relative L2 <= 1e-5,
complex data per component.

Small ragged shapes are compared element by element over every voxel and
frame; the named full-size configurations are compared on a seeded voxel
sample (all scatterer voxels, the grid corners, random voxels) in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, oracle_ref, run_gpu, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu

ALGS = [("baseline", "kqmb"), ("batch_inner", "kqmb"), ("batch_inner", "qmkb")]


def _ragged(iq=False, B=12, array=(37, 1), grid=(13, 7, 3), K=300, sources=None, **kw):
    sources = sources or ((0.0, 0.0), (1.5e-3, -0.5e-3), (-1e-3, 1e-3))
    return das_synth.custom_config("tiny", name="ragged", seed=17, array=array, grid=grid, K=K, B=B,
                                   tx="diverging", sources=sources, iq=iq, n_scatterers=0, **kw)


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("alg,layout", ALGS)
@pytest.mark.parametrize("B", [12, 16, 32, 40, 48, 64])
def test_ragged_full_compare(gpu, iq, alg, layout, B):
    cfg = _ragged(iq=iq, B=B)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), iq)
    ref = oracle_ref(inp)
    assert_parity(y, ref, f"{alg}/{layout} B={B} iq={iq}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_tiny_full_compare(gpu, alg, layout):
    cfg = das_synth.get_config("tiny")
    inp = Inputs(cfg)
    y = to_numpy(run_gpu(inp, alg, layout), False)
    assert_parity(y, oracle_ref(inp), f"tiny {alg}/{layout}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_tiny_iq_full_compare(gpu, alg, layout):
    cfg = das_synth.custom_config("tiny", iq=True, seed=8)
    inp = Inputs(cfg)
    y = to_numpy(run_gpu(inp, alg, layout), True)
    assert_parity(y, oracle_ref(inp), f"tiny-iq {alg}/{layout}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_degenerate_shapes(gpu, alg, layout):
    # one voxel, one receiver, one event, one frame, K = 2
    cfg = das_synth.custom_config("tiny", name="deg", array=(1, 1), grid=(1, 1, 1), K=2, B=1, n_scatterers=0,
                                  z0=1e-3, f_number=0.0, fs=1e6)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), False)
    ref = oracle_ref(inp)
    # s = 2 * 1e-3 / 1540 * 1e6 = 1.3 > K-2: the only term is dropped, the result is exactly 0
    assert np.all(ref == 0.0) and np.all(y == 0.0)


@pytest.mark.parametrize("f_number", [0.3, 0.45, 0.7, 1.0, 3.0, 0.0])
@pytest.mark.parametrize("alg,layout", [("baseline", "kqmb"), ("batch_inner", "qmkb")])
def test_receive_apodization_f_numbers(gpu, f_number, alg, layout):
    """Receive Hann at several f-numbers.  The kernels evaluate it as the plan's
    polynomial in (1 - cos theta) / (1 - cos theta_max), fitted once per plan;
    the oracle keeps the definition (fp64 atan2 and cos).  0 switches
    apodization off.  A 37 x 3 array over a 13 x 7 x 3 grid
    puts many receivers on both sides of the aperture edge."""
    cfg = _ragged(B=32, array=(37, 3), f_number=f_number)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), False)
    assert_parity(y, oracle_ref(inp), f"f# {f_number} {alg}/{layout}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_terms_off_the_record_end(gpu, alg, layout):
    # K short enough that deep voxels lose part of their (q, m) terms
    cfg = _ragged(K=140, B=16)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), False)
    ref = oracle_ref(inp)
    assert_parity(y, ref, f"short record {alg}/{layout}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_accumulate_adds_into_out(gpu, alg, layout):
    import torch
    cfg = _ragged(B=16)
    inp = Inputs(cfg, w_tx="uniform")
    ref = oracle_ref(inp)
    start = torch.linspace(-3.0, 3.0, cfg.B * cfg.N, device="cuda").reshape(cfg.B, cfg.N)
    out = run_gpu(inp, alg, layout, out=start.clone(), accumulate_into=True)
    y = out.cpu().numpy().astype(np.float64) - start.cpu().numpy()
    assert_parity(y, ref, f"accumulate {alg}/{layout}")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_q_chunks_sum_to_the_whole(gpu, alg, layout):
    cfg = _ragged(B=32)
    inp = Inputs(cfg)
    y = to_numpy(run_gpu(inp, alg, layout, q_chunk=1), False)
    assert_parity(y, oracle_ref(inp), f"q chunks {alg}/{layout}")


@pytest.mark.parametrize("kernel", ["default", "dpp_rows"])
@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("voxel", [0.25e-3, 0.6e-3, 1.5e-3], ids=["fine", "mixed", "coarse"])
@pytest.mark.parametrize("B", [16, 32, 64])
def test_staged_windows_and_fallback(gpu, monkeypatch, layout, voxel, iq, B, kernel):
    """The LDS-staged kernels.  Default: whole-row lanes (all 32 or 16 fp32
    or 16 complex frames of a frame tile per lane, 16 or 8 receivers a step);
    "dpp_rows" forces the DPP-row
    kernel: fp32 B = 32, 2 frames per lane, one 32-frame tile of 16 receivers
    a step; fp32 B = 64 and complex64 B = 32 and 64: split rows (two voxels
    per DPP row, 16 bytes per lane, 8 receivers a step, 256-byte rows).
    Coarse voxels give k-windows wider than the LDS capacity, which must fall
    back to direct loads; fine voxels stay in LDS; the mixed pitch exercises
    both within one launch."""
    if kernel == "dpp_rows":
        monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    cfg = das_synth.custom_config("tiny", name="staged", seed=23, array=(19, 3), grid=(11, 10, 3), K=700, B=B,
                                  tx="diverging", sources=((0.0, 0.0), (2e-3, 1e-3)), voxel=voxel,
                                  z0=3e-3, n_scatterers=0, iq=iq)
    inp = Inputs(cfg, w_tx="uniform")
    plan_info = __import__("volumetric_delay_sum_amd").plan_from_fields(inp.fields, "batch_inner", layout).info
    assert plan_info["staged"] == 1
    y = to_numpy(run_gpu(inp, "batch_inner", layout), iq)
    assert_parity(y, oracle_ref(inp), f"staged {layout} voxel {voxel} iq={iq}")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_split_and_whole_rows_agree(gpu, monkeypatch, iq):
    """B = 64: the DPP-row staged kernel with split rows (its default there)
    and with whole rows (two frame tiles) both meet the bar."""
    cfg = _ragged(B=64, grid=(17, 9, 4), iq=iq, array=(23, 2))
    inp = Inputs(cfg, w_tx="uniform")
    monkeypatch.setenv("DAS_STAGED_ROWS", "0")              # the DPP-row kernel
    split = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), iq)
    monkeypatch.setenv("DAS_STAGED_SPLIT", "1")
    whole = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), iq)
    ref = oracle_ref(inp)
    assert_parity(split, ref, "split rows")
    assert_parity(whole, ref, "whole rows")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_staged_and_direct_kernels_agree(gpu, monkeypatch, iq):
    cfg = _ragged(B=32, grid=(17, 9, 2), iq=iq)
    inp = Inputs(cfg, w_tx="uniform")
    staged = to_numpy(run_gpu(inp, "batch_inner", "kqmb"), iq)
    monkeypatch.setenv("DAS_BI_KERNEL", "direct")
    import volumetric_delay_sum_amd as das
    assert das.plan_from_fields(inp.fields, "batch_inner", "kqmb").info["staged"] == 0
    direct = to_numpy(run_gpu(inp, "batch_inner", "kqmb"), iq)
    ref = oracle_ref(inp)
    assert_parity(staged, ref, "staged")
    assert_parity(direct, ref, "direct")


def test_baseline_and_batch_inner_agree(gpu):
    cfg = das_synth.get_config("tiny")
    inp = Inputs(cfg)
    a = to_numpy(run_gpu(inp, "baseline"), False)
    b = to_numpy(run_gpu(inp, "batch_inner", "kqmb"), False)
    c = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), False)
    assert_parity(a, b.astype(np.float64), "BL vs BI")
    # the two batch-inner layouts run the same arithmetic in the same order
    assert np.array_equal(b, c)


# --------------------------------------------------------------------------
# Named configurations at full size, sampled voxels
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def mid_inputs(gpu):
    return Inputs(das_synth.get_config("mid"))


@pytest.mark.parametrize("alg,layout", ALGS)
def test_mid_sampled(mid_inputs, alg, layout):
    inp = mid_inputs
    vox = sample_voxels(inp.cfg, 400)
    out = run_gpu(inp, alg, layout)
    assert_all_written(out, f"mid {alg}/{layout}")
    y = to_numpy(out, False)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox), f"mid {alg}/{layout}")


@pytest.fixture(scope="module")
def main_inputs(gpu):
    return Inputs(das_synth.get_config("main"))


@pytest.mark.parametrize("alg,layout", ALGS)
def test_main_sampled(main_inputs, alg, layout):
    inp = main_inputs
    vox = sample_voxels(inp.cfg, 192)
    out = run_gpu(inp, alg, layout)
    assert_all_written(out, f"main {alg}/{layout}")
    y = to_numpy(out, False)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox), f"main {alg}/{layout}")


def test_main_scatterer_neighbourhoods_dense(main_inputs):
    """Every voxel of the 5^3 neighbourhoods of six central scatterers against the
    oracle, and the GPU's brightest voxel of each neighbourhood is the oracle's."""
    inp = main_inputs
    cfg = inp.cfg
    nx, ny, nz = cfg.grid
    sv = das_synth.scatterer_voxels(cfg)
    idx = np.stack([sv % nx, (sv // nx) % ny, sv // (nx * ny)], axis=-1)
    centre = np.abs(idx[:, :2] - np.array([nx / 2, ny / 2])).max(axis=1)
    chosen = idx[np.argsort(centre, kind="stable")[:6]]
    y = to_numpy(run_gpu(inp, "batch_inner", "kqmb"), False)
    for ix, iy, iz in chosen:
        nb = [((z * ny + yy) * nx + x) for z in range(iz - 2, iz + 3) for yy in range(iy - 2, iy + 3)
              for x in range(ix - 2, ix + 3)]
        ref = oracle_ref(inp, voxels=nb, frames=[0, 17])
        got = y[[0, 17]][:, nb]
        assert_parity(got, ref, f"neighbourhood of ({ix},{iy},{iz})")
        for j in range(2):
            assert np.argmax(np.abs(got[j])) == np.argmax(np.abs(ref[j]))


def test_main_noise_only(gpu):
    """Worst case for relative error: no scatterer energy to dilute it."""
    inp = Inputs(das_synth.get_config("main"), scatterers=False)
    vox = sample_voxels(inp.cfg, 128, seed=3)
    out = run_gpu(inp, "batch_inner", "kqmb")
    assert_all_written(out, "main noise-only")
    y = to_numpy(out, False)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox), "main noise-only")


@pytest.mark.parametrize("alg,layout", ALGS)
def test_main_c64_sampled(gpu, alg, layout):
    inp = Inputs(das_synth.get_config("main-c64"))
    vox = sample_voxels(inp.cfg, 128)
    out = run_gpu(inp, alg, layout)
    assert_all_written(out, f"main-c64 {alg}/{layout}")
    y = to_numpy(out, True)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox), f"main-c64 {alg}/{layout}")
