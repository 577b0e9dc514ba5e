"""GPU: binary16 sample storage (the FP16 variant of "ffdas: volumetric
ultrasound reconstruction at warp speed", Section 3; ffdas docs,
mixed-precision API).  The permute rounds float32 samples to binary16 and the
batch-inner kernels widen them back before the interpolation, so the result
must match the fp64 oracle of the rounded samples to the usual bar (max|err|
<= 1e-4 max|oracle|, relative L2 <= 1e-5, complex per component), and the
permuted halves must match the oracle's rounding bit for bit."""
import json
import os

import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, oracle_ref, run_gpu, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu

GOLDEN16 = os.path.join(os.path.dirname(__file__), "golden", "binary16_cases.json")


def _special_values():
    cases = json.load(open(GOLDEN16))["cases"]
    v = np.array([int(c["f32"], 16) for c in cases], dtype=np.uint32).view(np.float32)
    return np.concatenate([v, -v, np.array([np.nan, -np.nan], dtype=np.float32)])


@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("iq,B,K", [(False, 32, 64), (False, 16, 68), (False, 12, 70), (False, 64, 66),
                                    (True, 8, 64), (True, 32, 67)])
def test_permute_rounds_to_binary16_bit_for_bit(gpu, layout, iq, B, K):
    import torch
    import oracle
    import volumetric_delay_sum_amd as das
    Q, M = 3, 5
    rng = np.random.default_rng([B, K, int(iq)])
    shape = (B, Q, M, K, 2) if iq else (B, Q, M, K)
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-20, 12, shape))).astype(np.float32)
    flat = x.reshape(-1)
    sp = _special_values()
    pos = rng.choice(flat.size, size=sp.size, replace=False)
    flat[pos] = sp
    plan = das.Plan(B=B, Q=Q, M=M, K=K, nx=2, ny=2, nz=2, origin=(0, 0, 5e-3), spacing=(2e-4,) * 3,
                    fs=20e6, c=1540.0, f_demod=5e6 if iq else 0.0, dtype="c64" if iq else "f32",
                    layout=layout, storage="f16")
    xd = torch.from_numpy(x).cuda()
    for q0, qn in ((0, Q), (1, 2)):
        out = torch.full(plan.permuted_shape(qn), float("nan"), dtype=torch.float16, device="cuda")
        plan.permute(xd, out, q0, qn)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        sub = oracle.to_binary16(x[:, q0:q0 + qn])
        want = (oracle.permute_kqmb if layout == "kqmb" else oracle.permute_qmkb)(sub).astype(np.float16)
        nan = np.isnan(want)
        np.testing.assert_array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan].view(np.uint16), want[~nan].view(np.uint16))


def _ragged(iq=False, B=12, **kw):
    return das_synth.custom_config("tiny", name="ragged16", seed=23, array=(37, 1), grid=(13, 7, 3), K=300, B=B,
                                   tx="diverging", sources=((0.0, 0.0), (1.5e-3, -0.5e-3), (-1e-3, 1e-3)),
                                   iq=iq, n_scatterers=0, **kw)


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("B", [7, 12, 16, 32, 40, 64, 96])
def test_binary16_ragged_full_compare(gpu, iq, layout, B):
    cfg = _ragged(iq=iq, B=B)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "batch_inner", layout, storage="f16"), iq)
    assert_parity(y, oracle_ref(inp, storage="f16"), f"f16 {layout} B={B} iq={iq}")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_binary16_direct_kernel(gpu, monkeypatch, iq):
    monkeypatch.setenv("DAS_BI_KERNEL", "direct")
    cfg = _ragged(iq=iq, B=32)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "batch_inner", "kqmb", storage="f16"), iq)
    assert_parity(y, oracle_ref(inp, storage="f16"), f"f16 direct iq={iq}")


# frames per lane of the binary16 staged instances.  Whole-row lanes (the
# default where B is a multiple of 16): 32 fp32 frames (B a multiple of 32),
# else 16 fp32 or complex frames.  DPP rows (DAS_STAGED_ROWS=0): B a multiple of 32
# takes two (complex: one pair of halves per frame, two frames), a multiple of
# 16 only takes one, and fp32 data with B a multiple of 64 takes four
FPL16_ROWS = {(False, 16): 16, (False, 32): 32, (False, 48): 16, (False, 64): 32,
              (True, 16): 16, (True, 32): 16, (True, 48): 16, (True, 64): 16}
FPL16_DPP = {(False, 16): 1, (False, 32): 2, (False, 48): 1, (False, 64): 4,
             (True, 16): 1, (True, 32): 2, (True, 48): 1, (True, 64): 2}


@pytest.mark.parametrize("kernel", ["default", "dpp_rows"])
@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("voxel", [0.2e-3, 1.2e-3])
@pytest.mark.parametrize("B", [16, 32, 48, 64])
def test_binary16_staged_windows_and_fallback(gpu, monkeypatch, iq, voxel, B, kernel):
    # coarse voxels make windows too wide for LDS: the direct-load fallback inside the staged kernel
    import volumetric_delay_sum_amd as das
    if kernel == "dpp_rows":
        monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    cfg = das_synth.custom_config("tiny", name="win16", seed=29, array=(19, 3), grid=(11, 10, 3), K=700, B=B,
                                  tx="diverging", sources=((0.0, 0.0), (2e-3, 1e-3)), iq=iq, n_scatterers=0,
                                  voxel=voxel, z0=3e-3)
    inp = Inputs(cfg, w_tx="uniform")
    info = das.plan_from_fields(inp.fields, "batch_inner", "qmkb", storage="f16").info
    assert info["staged"] == 1
    rows = kernel == "default" and (iq, B) in FPL16_ROWS
    assert info["whole_rows"] == (1 if rows else 0), info
    assert info["frames_per_lane"] == (FPL16_ROWS if rows else FPL16_DPP)[(iq, B)], info
    y = to_numpy(run_gpu(inp, "batch_inner", "qmkb", storage="f16", q_chunk=1), iq)
    assert_parity(y, oracle_ref(inp, storage="f16"), f"f16 windows voxel={voxel} iq={iq}")


def test_binary16_differs_from_float32_by_the_rounding_only(gpu):
    # the same inputs through both storages: the difference is the beamform of
    # the rounding error, which the oracle gives independently
    import oracle
    cfg = _ragged(B=32)
    inp = Inputs(cfg, w_tx="uniform")
    y16 = to_numpy(run_gpu(inp, "batch_inner", "kqmb", storage="f16"), False)
    y32 = to_numpy(run_gpu(inp, "batch_inner", "kqmb"), False)
    d = (oracle.to_binary16(inp.rf_host) - inp.rf_host).astype(np.float32)
    yd = oracle.das_sum(inp.fields, d, inp.rx, inp.tau, inp.w)
    assert np.abs(yd).max() > 0
    err = (y16 - y32) - yd
    assert np.abs(err).max() <= 1e-4 * np.abs(y32).max()


@pytest.fixture(scope="module")
def main_inputs(gpu):
    return Inputs(das_synth.get_config("main"))


@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
def test_binary16_main_sampled(main_inputs, layout):
    """Main (32 x 32 array, 9 events, 2048 samples, 32 frames, 64^3 voxels) with
    binary16 storage, in the launch configuration the benchmark times."""
    inp = main_inputs
    vox = sample_voxels(inp.cfg, 192)
    out = run_gpu(inp, "batch_inner", layout, storage="f16")
    assert_all_written(out, f"main f16 {layout}")
    y = to_numpy(out, False)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox, storage="f16"), f"main f16 {layout}")


def test_binary16_main_c64_sampled(gpu):
    cfg = das_synth.get_config("main-c64")
    inp = Inputs(cfg)
    vox = sample_voxels(cfg, 96)
    out = run_gpu(inp, "batch_inner", "qmkb", storage="f16")
    assert_all_written(out, "main-c64 f16")
    y = to_numpy(out, True)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox, storage="f16"), "main-c64 f16")


def test_binary16_streamed(gpu):
    import torch
    import volumetric_delay_sum_amd as das
    cfg = das_synth.custom_config("tiny", name="stream16", seed=31, array=(16, 8), grid=(16, 16, 6), K=512, B=32,
                                  tx="diverging", n_scatterers=0,
                                  sources=((0.0, 0.0), (2e-3, 0.0), (-2e-3, 0.0), (0.0, 2e-3), (0.0, -2e-3)))
    inp = Inputs(cfg, w_tx="uniform")
    plan = das.plan_from_fields(inp.fields, algorithm="batch_inner", layout="kqmb", storage="f16")
    out = torch.full(plan.output_shape(), float("nan"), dtype=torch.float32, device="cuda")
    pa = torch.empty(plan.permuted_shape(2), dtype=torch.float16, device="cuda")
    pb = torch.empty_like(pa)
    sp, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    plan.beamform_streamed(inp.rf_d, inp.rx_d, inp.tau_d, inp.w_d, out, pa, pb, 2,
                           stream_permute=sp, stream_beamform=sb)
    sp.synchronize()
    torch.cuda.synchronize()
    assert_parity(to_numpy(out, False), oracle_ref(inp, storage="f16"), "f16 streamed")


def test_binary16_plan_takes_half_buffers_only(gpu):
    import torch
    import volumetric_delay_sum_amd as das
    plan = das.Plan(B=32, Q=2, M=4, K=64, nx=2, ny=2, nz=2, origin=(0, 0, 5e-3), spacing=(2e-4,) * 3,
                    fs=20e6, c=1540.0, storage="f16")
    rf = torch.zeros((32, 2, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        plan.permute(rf, torch.empty(plan.permuted_shape(), dtype=torch.float32, device="cuda"))
    perm = torch.empty(plan.permuted_shape(), dtype=torch.float16, device="cuda")
    plan.permute(rf, perm)
    out = torch.empty(plan.output_shape(), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        plan.beamform(perm.float(), torch.zeros((4, 3), device="cuda"), torch.zeros((2, 8), device="cuda"),
                      torch.zeros((2, 8), device="cuda"), out)
    plan.beamform(perm, torch.zeros((4, 3), device="cuda"), torch.zeros((2, 8), device="cuda"),
                  torch.ones((2, 8), device="cuda"), out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_binary16_large_sampled(gpu):
    """Large (128 x 128 x 96 voxels, 64 frames, 16 events of 1024 x 4096
    samples) with binary16 storage in one QMKB chunk, as the benchmark runs it;
    three frames on a seeded voxel sample against the oracle of the rounded
    samples."""
    import torch
    import oracle
    cfg = das_synth.get_config("large")
    inp = Inputs(cfg)
    out = run_gpu(inp, "batch_inner", "qmkb", storage="f16")
    assert_all_written(out, "large f16")
    frames = [0, 31, 63]
    vox = sample_voxels(cfg, 768, seed=7)
    y = to_numpy(out, cfg.iq)[frames][:, vox]
    fields = dict(inp.fields, B=len(frames))
    rf_sub = oracle.to_binary16(inp.rf_d[frames].cpu().numpy())
    del inp, out
    torch.cuda.empty_cache()
    ref = oracle.das_sum(fields, rf_sub, das_synth.array_positions(cfg), *das_synth.tx_tables(cfg), voxels=vox)
    assert_parity(y, ref, "large f16")
