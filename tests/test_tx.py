"""GPU transmit-table generator against the oracle's tables (through the C ABI).

Tolerance: the weight is copied, so it must be exact; the delay is the same
fp64 expression rounded once to float32 on both sides, so the two agree to
within one float32 ulp (a last-place difference in the fp64 square root can
move a value across a float32 rounding boundary)."""
import math

import numpy as np
import pytest

import das_synth

pytestmark = pytest.mark.gpu


def _events(cfg, oracle_mod):
    if cfg.tx == "plane":
        return [(oracle_mod.TX_PLANE, (0.0, 0.0, 1.0), 1.0)] * cfg.Q
    return [(oracle_mod.TX_DIVERGING, (vx, vy, -cfg.src_depth), 1.0) for vx, vy in cfg.sources]


def _run(das, fields, events, Q, q_begin=0):
    import torch
    plan = das.plan_from_fields(dict(fields, Q=Q), algorithm="baseline")
    tau = torch.full((Q, plan.N), float("nan"), dtype=torch.float32, device="cuda")
    w = torch.full((Q, plan.N), float("nan"), dtype=torch.float32, device="cuda")
    print(f"tx_tables N={plan.N} Q={Q} q_begin={q_begin} events={len(events)}", flush=True)
    plan.tx_tables(events, tau, w, q_begin=q_begin)
    torch.cuda.synchronize()
    return tau.cpu().numpy(), w.cpu().numpy()


def _compare(tau, w, tau_ref, w_ref, what):
    np.testing.assert_array_equal(w, w_ref, err_msg=what)
    assert np.all(np.isfinite(tau)), what
    ulp = np.abs(tau.view(np.int32).astype(np.int64) - tau_ref.view(np.int32))
    assert ulp.max() <= 1, f"{what}: {ulp.max()} ulp"
    return float((ulp == 0).mean())


@pytest.mark.parametrize("name", ["tiny", "mid", "main", "large"])
def test_named_configs(gpu, oracle_mod, name):
    cfg = das_synth.get_config(name)
    fields = das_synth.problem_fields(cfg)
    events = _events(cfg, oracle_mod)
    tau, w = _run(gpu, fields, events, cfg.Q)
    tau_ref, w_ref = oracle_mod.tx_tables(fields, events)
    exact = _compare(tau, w, tau_ref, w_ref, name)
    assert exact > 0.999, f"{name}: only {exact:.5f} of the delays are bit-identical"


def test_mixed_events_several_launches_and_untouched_rows(gpu, oracle_mod):
    # 20 events (two launches of the generator) written to rows 3..22 of 25,
    # on a ragged grid (105 voxels, not a multiple of the block)
    fields = dict(nx=7, ny=5, nz=3, origin=(-1e-3, -0.5e-3, 5e-3), spacing=(0.3e-3, 0.25e-3, 0.4e-3),
                  c=1540.0, B=1, M=4, K=16, fs=20e6, t0=0.0, f_number=1.0, f_demod=0.0, iq=False)
    events = []
    for i in range(20):
        if i % 2:
            a = -0.4 + 0.08 * i
            events.append((oracle_mod.TX_PLANE, (math.sin(a) * 0.6, math.sin(a) * 0.8, math.cos(a)), 0.1 * i))
        else:
            events.append((oracle_mod.TX_DIVERGING, (1e-3 * (i - 10) / 10, -0.5e-3, -(5e-3 + 1e-3 * i)), 1.5))
    tau, w = _run(gpu, fields, events, Q=25, q_begin=3)
    tau_ref, w_ref = oracle_mod.tx_tables(fields, events)
    _compare(tau[3:23], w[3:23], tau_ref, w_ref, "mixed")
    assert np.all(np.isnan(tau[:3])) and np.all(np.isnan(tau[23:]))
    assert np.all(np.isnan(w[:3])) and np.all(np.isnan(w[23:]))


def test_single_voxel(gpu, oracle_mod):
    fields = dict(nx=1, ny=1, nz=1, origin=(0.0, 0.0, 7e-3), spacing=(1e-4, 1e-4, 1e-4), c=1500.0,
                  B=1, M=1, K=2, fs=1e7, t0=0.0, f_number=0.0, f_demod=0.0, iq=False)
    events = [(oracle_mod.TX_DIVERGING, (0.0, 0.0, -1e-2), 1.0)]
    tau, w = _run(gpu, fields, events, Q=1)
    tau_ref, w_ref = oracle_mod.tx_tables(fields, events)
    _compare(tau, w, tau_ref, w_ref, "single voxel")


def test_generated_tables_drive_the_beamformer(gpu, oracle_mod):
    # the Mid volume beamformed from GPU-made tables equals the one from the
    # host-made tables wherever the tables agree bit for bit, and meets the
    # parity bar against the oracle everywhere
    import torch
    import das_testing as T
    cfg = das_synth.get_config("mid")
    inp = T.Inputs(cfg)
    tau, w = _run(gpu, inp.fields, _events(cfg, oracle_mod), cfg.Q)
    inp.tau, inp.w = tau, w
    inp.tau_d, inp.w_d = torch.from_numpy(tau).cuda(), torch.from_numpy(w).cuda()
    y = T.to_numpy(T.run_gpu(inp, "batch_inner"), False)
    vox = T.sample_voxels(cfg, 2000)
    T.assert_parity(y[:, vox], T.oracle_ref(inp, voxels=vox), "mid from GPU tables")
