"""float64 and complex128 baseline (the docs' ALG1 data types) against the
oracle, through the C ABI.

Both sides evaluate every term in fp64 with the same operations in the same
order; they differ only in the math library's last bits (square root, atan2,
cos, sincos) and in the order of the sum over (q, m).  With some 1e4 terms per
voxel that is ~1e-14 relative, so the bar here is max|err| <= 1e-11 max|ref|
and relative L2 <= 1e-12 (complex compared per component): seven orders
tighter than the fp32 path's, and far above the rounding noise."""
import numpy as np
import pytest

import das_synth
import das_testing as T

pytestmark = pytest.mark.gpu

MAX_REL_F64 = 1e-11
L2_REL_F64 = 1e-12


def _assert_f64(y, ref, what):
    assert np.all(np.isfinite(np.asarray(y).real)) and np.all(np.isfinite(np.asarray(y).imag)), what
    for i, (mx, l2) in enumerate(T.parity_errors(y, ref)):
        assert mx <= MAX_REL_F64 and l2 <= L2_REL_F64, f"{what} component {i}: max {mx:.3e}, L2 {l2:.3e}"


def _wide_rf(inp, seed):
    """The config's RF widened to float64, plus a part float32 cannot hold."""
    x = inp.rf_host.astype(np.float64)
    x += np.random.default_rng([seed, 64]).standard_normal(x.shape) * 1e-6
    return x


def _run(inp, x64, q_chunk=None):
    import torch
    import volumetric_delay_sum_amd as das
    fields = dict(inp.fields)
    plan = das.plan_from_fields(fields, algorithm="baseline", wide=True)
    rf = torch.from_numpy(x64).cuda()
    out = torch.full(plan.output_shape(), float("nan"), dtype=torch.float64, device="cuda")
    Q = fields["Q"]
    qc = Q if q_chunk is None else q_chunk
    print(f"fp64 baseline {inp.cfg.name} iq={plan.iq} q_chunk={qc}", flush=True)
    for q0 in range(0, Q, qc):
        plan.beamform(rf, inp.rx_d, inp.tau_d, inp.w_d, out, q0, min(qc, Q - q0), accumulate=q0 > 0)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    return y[..., 0] + 1j * y[..., 1] if plan.iq else y


@pytest.mark.parametrize("iq", [False, True])
def test_tiny_full_volume(gpu, oracle_mod, iq):
    cfg = das_synth.custom_config("tiny", iq=True, seed=8) if iq else das_synth.get_config("tiny")
    inp = T.Inputs(cfg, w_tx="uniform")
    x = _wide_rf(inp, 1)
    ref = oracle_mod.das_sum(inp.fields, x, inp.rx, inp.tau, inp.w)
    _assert_f64(_run(inp, x), ref, f"tiny iq={iq}")


@pytest.mark.parametrize("iq", [False, True])
def test_mid_sampled_voxels(gpu, oracle_mod, iq):
    cfg = das_synth.custom_config("mid", iq=True, seed=12) if iq else das_synth.get_config("mid")
    name = cfg.name + (" iq" if iq else "")
    inp = T.Inputs(cfg)
    x = _wide_rf(inp, 2)
    y = _run(inp, x, q_chunk=2)                  # chunks after the first accumulate
    vox = T.sample_voxels(cfg, 1500)
    frames = [0, cfg.B - 1]
    ref = oracle_mod.das_sum(inp.fields, x, inp.rx, inp.tau, inp.w, voxels=vox, frames=frames)
    _assert_f64(y[frames][:, vox], ref, name)


def test_single_frame_no_batch(gpu, oracle_mod):
    # B = 1: ALG1 needs no batch dimension; t0 > 0, random transmit weights
    # and a ragged grid (13 x 11 x 9 voxels)
    cfg = das_synth.custom_config("tiny", name="one-frame", seed=23, B=1, grid=(13, 11, 9), t0=0.4e-6)
    inp = T.Inputs(cfg, w_tx="uniform")
    x = _wide_rf(inp, 3)
    ref = oracle_mod.das_sum(inp.fields, x, inp.rx, inp.tau, inp.w)
    _assert_f64(_run(inp, x), ref, "B=1")


def test_auto_plan_runs_the_chosen_kernel(gpu, oracle_mod):
    # AUTO on Mid (fp32, B = 16) resolves to batch-inner; the chunked run meets the fp32 bar
    cfg = das_synth.get_config("mid")
    inp = T.Inputs(cfg)
    import volumetric_delay_sum_amd as das
    assert das.plan_from_fields(inp.fields, algorithm="auto").batch_inner
    y = T.to_numpy(T.run_gpu(inp, "auto"), False)
    vox = T.sample_voxels(cfg, 1500)
    T.assert_parity(y[:, vox], T.oracle_ref(inp, voxels=vox), "mid auto")


@pytest.mark.parametrize("f_number", [0.3, 1.0, 3.0, 0.0, 1e-7])
@pytest.mark.parametrize("iq", [False, True])
def test_receive_aperture_f_numbers(gpu, oracle_mod, f_number, iq):
    # The kernel skips receivers outside a voxel's aperture, deciding most of
    # them by a tangent test with a margin before atan2; a 37 x 3 array over
    # a 13 x 7 x 3 grid puts many pairs on both sides of the aperture edge.
    # f# 0 switches apodization off (nothing skipped); at f# 1e-7 the
    # aperture is wider than atan(1e6) and only the exact test runs.
    cfg = das_synth.custom_config("tiny", name="f64-apod", seed=31, iq=iq, B=4, array=(37, 3),
                                  grid=(13, 7, 3), f_number=f_number, n_scatterers=0)
    inp = T.Inputs(cfg, w_tx="uniform")
    x = _wide_rf(inp, 4)
    ref = oracle_mod.das_sum(inp.fields, x, inp.rx, inp.tau, inp.w)
    _assert_f64(_run(inp, x), ref, f"f# {f_number} iq={iq}")
