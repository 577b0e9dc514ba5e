"""Pins for the fp64 CPU oracle: checks against facts other than the oracle itself.

Each test fixes a part of the definition of the delay-and-sum result ("ffdas:
volumetric ultrasound reconstruction at warp speed", Section 3: per-voxel
transmit tables, receive delay and weight from receiver geometry, two samples
k and k+1 per receiver; ffdas docs "How It Works": interpolate and sum aligned
samples over every receiver and transmit event):

* hand-derived golden cases (tests/golden/hand_cases.json),
* a brute-force precomputed delay table summed with numpy's own linear
  interpolation (the stored-table alternative the pages reject for size),
* closed forms: constant RF, a linear ramp (linear interpolation is exact on
  lines), a single impulse (the hat-function response),
* invariants: linearity, frame permutation, a t0 shift against a sample roll,
* special values of the Hann receive apodization,
* point scatterers that must peak at their voxel.
"""
import json
import math
import os

import numpy as np
import pytest

import das_synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ---------------------------------------------------------------------------
# Independent helpers: written from the geometry, not from the oracle's code.
# Distance by np.linalg.norm, angle by arccos(dz/d), Hann as cos^2 of half the
# phase, interpolation by np.interp.
# ---------------------------------------------------------------------------

def _fields(B, Q, M, K, grid, origin, spacing, fs=20e6, c=1540.0, t0=0.0, f_number=1.0,
            f_demod=0.0, iq=False):
    return dict(B=B, Q=Q, M=M, K=K, nx=grid[0], ny=grid[1], nz=grid[2], origin=origin,
                spacing=spacing, fs=fs, c=c, t0=t0, f_number=f_number, f_demod=f_demod, iq=iq)


def _centres(fields, voxels):
    nx, ny = fields["nx"], fields["ny"]
    v = np.asarray(voxels, dtype=np.int64)
    idx = np.stack([v % nx, (v // nx) % ny, v // (nx * ny)], axis=-1).astype(np.float64)
    return np.asarray(fields["origin"], dtype=np.float64) + idx * np.asarray(fields["spacing"], dtype=np.float64)


def _geometry(fields, rx, tau_tx, voxels):
    """Per (q, m, voxel): s, total time tau and w_rx, all fp64."""
    r = _centres(fields, voxels)                                  # V x 3
    p = rx.astype(np.float64)                                     # M x 3
    diff = r[None, :, :] - p[:, None, :]                          # M x V x 3
    d = np.linalg.norm(diff, axis=-1)                             # M x V
    dz = diff[..., 2]
    F = fields["f_number"]
    if F <= 0:
        w_rx = np.ones_like(d)
    else:
        theta = np.arccos(np.clip(dz / d, -1.0, 1.0))
        theta_max = math.atan(1.0 / (2.0 * F))
        w_rx = np.where((dz > 0) & (theta < theta_max),
                        np.cos(0.5 * np.pi * theta / theta_max) ** 2, 0.0)
    tt = tau_tx.astype(np.float64)[:, np.asarray(voxels)]         # Q x V
    tau = tt[:, None, :] + d[None, :, :] / fields["c"]            # Q x M x V
    s = (tau - fields["t0"]) * fields["fs"]
    return s, tau, w_rx


def _brute_force(fields, rf, rx, tau_tx, w_tx, voxels):
    """Build the full delay/weight table, then sum with np.interp per row."""
    s, tau, w_rx = _geometry(fields, rx, tau_tx, voxels)
    B, Q, M, K = fields["B"], fields["Q"], fields["M"], fields["K"]
    ks = np.arange(K, dtype=np.float64)
    wt = w_tx.astype(np.float64)[:, np.asarray(voxels)]
    valid = (np.floor(s) >= 0) & (np.floor(s) <= K - 2)
    out = np.zeros((B, len(voxels)), dtype=np.complex128 if fields["iq"] else np.float64)
    for b in range(B):
        for q in range(Q):
            for m in range(M):
                row = rf[b, q, m].astype(np.float64)
                if fields["iq"]:
                    v = np.interp(s[q, m], ks, row[:, 0]) + 1j * np.interp(s[q, m], ks, row[:, 1])
                    v = v * np.exp(2j * np.pi * fields["f_demod"] * tau[q, m])
                else:
                    v = np.interp(s[q, m], ks, row)
                out[b] += np.where(valid[q, m], wt[q] * w_rx[m] * v, 0.0)
    return out


def _random_problem(seed, iq=False, w_mode="uniform", t0=0.0, K=96, grid=(3, 2, 4), M=5, Q=2, B=3,
                    f_number=1.0):
    rng = np.random.default_rng(seed)
    spacing = (0.3e-3, 0.25e-3, 0.2e-3)
    origin = (-0.3e-3, -0.1e-3, 2.0e-3)
    f = _fields(B, Q, M, K, grid, origin, spacing, fs=20e6, c=1540.0, t0=t0, f_number=f_number,
                f_demod=(5e6 if iq else 0.0), iq=iq)
    rx = np.zeros((M, 3), dtype=np.float32)
    rx[:, :2] = rng.uniform(-1.5e-3, 1.5e-3, (M, 2))
    N = grid[0] * grid[1] * grid[2]
    tau = rng.uniform(0.5e-6, 2.0e-6, (Q, N)).astype(np.float32)
    w = (rng.random((Q, N)) if w_mode == "uniform" else np.ones((Q, N))).astype(np.float32)
    shape = (B, Q, M, K, 2) if iq else (B, Q, M, K)
    x = rng.standard_normal(shape).astype(np.float32)
    return f, x, rx, tau, w


# ---------------------------------------------------------------------------

def _golden_rf(rule, B, Q, M, K):
    k = np.arange(K, dtype=np.float64)
    b = np.arange(B, dtype=np.float64)[:, None, None, None]
    if rule == "k":
        x = np.broadcast_to(k, (B, Q, M, K))
    elif rule == "k2":
        x = np.broadcast_to(k * k, (B, Q, M, K))
    elif rule == "b_plus_k":
        x = np.broadcast_to(100.0 * b + k, (B, Q, M, K))
    elif rule == "k_plus_halfj":
        x = np.stack([np.broadcast_to(k, (B, Q, M, K)), np.full((B, Q, M, K), 0.5)], axis=-1)
    else:
        raise KeyError(rule)
    return np.ascontiguousarray(x, dtype=np.float32)


def test_golden_hand_cases(oracle_mod):
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 8
    for case in cases:
        g = case["grid"]
        M = len(case["rx_pos"])
        f = _fields(case["B"], case["Q"], M, case["K"], (g["nx"], g["ny"], g["nz"]), g["origin"],
                    g["spacing"], fs=case["fs"], c=case["c"], t0=case["t0"], f_number=case["f_number"],
                    f_demod=case["f_demod"], iq=case["iq"])
        x = _golden_rf(case["rf"], case["B"], case["Q"], M, case["K"])
        y = oracle_mod.das_sum(f, x, np.array(case["rx_pos"], dtype=np.float32),
                               np.array(case["tau_tx"], dtype=np.float32),
                               np.array(case["w_tx"], dtype=np.float32))
        exp = np.array(case["expected"], dtype=np.float64)
        if case["iq"]:
            exp = exp[..., 0] + 1j * exp[..., 1]
        np.testing.assert_allclose(y, exp, rtol=1e-12, atol=1e-12, err_msg=case["name"])


@pytest.mark.parametrize("iq", [False, True])
@pytest.mark.parametrize("seed", [11, 12, 13])
def test_brute_force_delay_table(oracle_mod, seed, iq):
    f, x, rx, tau, w = _random_problem(seed, iq=iq, t0=(0.1e-6 if seed == 12 else 0.0))
    N = f["nx"] * f["ny"] * f["nz"]
    vox = np.arange(N)
    ref = _brute_force(f, x, rx, tau, w, vox)
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    scale = np.abs(ref).max()
    assert scale > 0
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * scale)


def test_brute_force_tiny_config_subset(oracle_mod):
    cfg = das_synth.get_config("tiny")
    f = das_synth.problem_fields(cfg)
    rx = das_synth.array_positions(cfg)
    tau, w = das_synth.tx_tables(cfg, w_tx="uniform")
    x = das_synth.rf(cfg).numpy()
    vox = np.random.default_rng(5).choice(cfg.N, 40, replace=False)
    ref = _brute_force(f, x, rx, tau, w, vox)
    y = oracle_mod.das_sum(f, x, rx, tau, w, voxels=vox)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("iq", [False, True])
def test_constant_rf_closed_form(oracle_mod, iq):
    f, x, rx, tau, w = _random_problem(21, iq=iq, K=128)
    C = 1.75
    x[...] = 0
    if iq:
        x[..., 0] = C
        x[..., 1] = -0.5
    else:
        x[...] = C
    N = f["nx"] * f["ny"] * f["nz"]
    vox = np.arange(N)
    s, tautot, w_rx = _geometry(f, rx, tau, vox)
    valid = (np.floor(s) >= 0) & (np.floor(s) <= f["K"] - 2)
    wt = w.astype(np.float64)[:, None, :] * w_rx[None, :, :]
    if iq:
        expect = ((C - 0.5j) * np.where(valid, wt * np.exp(2j * np.pi * f["f_demod"] * tautot), 0)).sum((0, 1))
    else:
        expect = C * np.where(valid, wt, 0.0).sum((0, 1))
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    for b in range(f["B"]):
        np.testing.assert_allclose(y[b], expect, rtol=1e-12, atol=1e-12)


def test_constant_rf_some_terms_out_of_range(oracle_mod):
    """K small enough that part of the (q, m) terms fall off the end of the record."""
    f, x, rx, tau, w = _random_problem(22, K=48)
    x[...] = 1.0
    vox = np.arange(f["nx"] * f["ny"] * f["nz"])
    s, _, w_rx = _geometry(f, rx, tau, vox)
    valid = (np.floor(s) >= 0) & (np.floor(s) <= f["K"] - 2)
    assert 0 < valid.mean() < 1, "test geometry must straddle the range edge"
    expect = np.where(valid, w.astype(np.float64)[:, None, :] * w_rx[None], 0).sum((0, 1))
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    np.testing.assert_allclose(y[0], expect, rtol=1e-12, atol=1e-12)


def test_ramp_is_exact(oracle_mod):
    """Linear interpolation reproduces lines: x = alpha_b + beta*k gives sum w*(alpha_b + beta*s)."""
    f, x, rx, tau, w = _random_problem(31, K=160, t0=0.05e-6)
    alpha = np.array([0.5, -2.0, 3.25], dtype=np.float64)
    beta = 0.125
    k = np.arange(f["K"], dtype=np.float64)
    x[...] = (alpha[:, None, None, None] + beta * k).astype(np.float32)
    vox = np.arange(f["nx"] * f["ny"] * f["nz"])
    s, _, w_rx = _geometry(f, rx, tau, vox)
    valid = (np.floor(s) >= 0) & (np.floor(s) <= f["K"] - 2)
    wt = np.where(valid, w.astype(np.float64)[:, None, :] * w_rx[None], 0.0)
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    for b in range(f["B"]):
        expect = (wt * (alpha[b] + beta * s)).sum((0, 1))
        np.testing.assert_allclose(y[b], expect, rtol=1e-11, atol=1e-11)


def test_impulse_response_is_the_hat(oracle_mod):
    f, x, rx, tau, w = _random_problem(41, K=128)
    x[...] = 0
    bq, qq, mq = 1, 1, 3
    vox = np.arange(f["nx"] * f["ny"] * f["nz"])
    s, _, w_rx = _geometry(f, rx, tau, vox)
    kstar = int(np.round(np.median(s[qq, mq])))
    assert 1 <= kstar <= f["K"] - 2
    x[bq, qq, mq, kstar] = 1.0
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    hat = np.maximum(0.0, 1.0 - np.abs(s[qq, mq] - kstar))
    expect = w.astype(np.float64)[qq] * w_rx[mq] * hat
    assert np.count_nonzero(expect) > 0
    np.testing.assert_allclose(y[bq], expect, rtol=1e-12, atol=1e-14)
    others = [b for b in range(f["B"]) if b != bq]
    assert np.all(y[others] == 0.0)


def test_linearity(oracle_mod):
    f, x, rx, tau, w = _random_problem(51)
    rng = np.random.default_rng(52)
    x1 = rng.integers(-50, 50, x.shape).astype(np.float32)
    x2 = rng.integers(-50, 50, x.shape).astype(np.float32)
    comb = (2.0 * x1 - 3.0 * x2).astype(np.float32)        # exact in float32
    y1 = oracle_mod.das_sum(f, x1, rx, tau, w)
    y2 = oracle_mod.das_sum(f, x2, rx, tau, w)
    yc = oracle_mod.das_sum(f, comb, rx, tau, w)
    np.testing.assert_allclose(yc, 2.0 * y1 - 3.0 * y2, rtol=0, atol=1e-10 * np.abs(yc).max())


def test_frame_permutation_equivariance(oracle_mod):
    f, x, rx, tau, w = _random_problem(61, iq=True)
    perm = np.array([2, 0, 1])
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    yp = oracle_mod.das_sum(f, np.ascontiguousarray(x[perm]), rx, tau, w)
    assert np.array_equal(yp, y[perm])
    ys = oracle_mod.das_sum(f, x, rx, tau, w, frames=[1])
    assert np.array_equal(ys[0], y[1])


def test_t0_shift_matches_sample_roll(oracle_mod):
    f, x, rx, tau, w = _random_problem(71, K=200)
    j = 7
    vox = np.arange(f["nx"] * f["ny"] * f["nz"])
    s, _, _ = _geometry(f, rx, tau, vox)
    assert s.min() > j + 1 and s.max() < f["K"] - 3, "all terms must stay inside both records"
    f2 = dict(f, t0=f["t0"] + j / f["fs"])
    x2 = np.zeros_like(x)
    x2[..., : f["K"] - j] = x[..., j:]
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    y2 = oracle_mod.das_sum(f2, x2, rx, tau, w)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-9 * np.abs(y).max())


def test_range_boundary_rule(oracle_mod):
    """s in {-0.5, 0, K-1.5, K-1, K-0.5}: only k in [0, K-2] contributes."""
    K = 10
    f = _fields(1, 1, 1, K, (1, 1, 5), (0.0, 0.0, 1.0), (1.0, 1.0, 1.0), fs=1.0, c=1.0, f_number=0.0)
    targets = np.array([-0.5, 0.0, K - 1.5, K - 1.0, K - 0.5])
    z = 1.0 + np.arange(5)
    tau = (targets - z).astype(np.float32)[None, :]
    x = (np.arange(K, dtype=np.float32) + 1.0)[None, None, None, :]
    y = oracle_mod.das_sum(f, np.ascontiguousarray(x), np.zeros((1, 3), np.float32), tau,
                           np.ones((1, 5), np.float32))
    np.testing.assert_array_equal(y[0], [0.0, 1.0, (K - 1 + K) / 2.0, 0.0, 0.0])


def test_hann_special_values(oracle_mod):
    """theta = 0 -> 1, theta_max/2 -> 1/2, theta >= theta_max -> 0, behind -> 0, F <= 0 -> 1."""
    for F in (0.5, 1.0, 2.0):
        tmax = math.atan(1.0 / (2.0 * F))
        dz = 1.0e-2
        assert oracle_mod.rx_weight(0.0, dz, F) == 1.0
        assert abs(oracle_mod.rx_weight(dz * math.tan(tmax / 2), dz, F) - 0.5) < 1e-12
        assert oracle_mod.rx_weight(dz * math.tan(tmax) * 1.000001, dz, F) == 0.0
        assert oracle_mod.rx_weight(dz * math.tan(tmax) * 0.999999, dz, F) < 1e-9
        assert oracle_mod.rx_weight(0.0, -dz, F) == 0.0
        # radial, not separable: the same rho in any direction gives the same weight
        diag = oracle_mod.rx_weight(math.hypot(0.003 / math.sqrt(2), 0.003 / math.sqrt(2)), dz, F)
        assert abs(oracle_mod.rx_weight(0.003, dz, F) - diag) < 1e-12
    assert oracle_mod.rx_weight(5.0, 1.0, 0.0) == 1.0
    assert oracle_mod.rx_weight(5.0, -1.0, -1.0) == 1.0


def test_hann_through_the_sum(oracle_mod):
    """One voxel on the axis, receivers placed at chosen angles, one receiver lit per frame."""
    F = 1.0
    tmax = math.atan(1.0 / (2.0 * F))
    z = 4e-3
    angles = [0.0, tmax / 2, tmax * 1.01, -tmax / 2]
    M = len(angles)
    rx = np.zeros((M, 3), np.float32)
    rx[:, 0] = [z * math.tan(a) for a in angles]
    f = _fields(M, 1, M, 512, (1, 1, 1), (0.0, 0.0, z), (1e-4, 1e-4, 1e-4), f_number=F)
    x = np.zeros((M, 1, M, 512), np.float32)
    for b in range(M):
        x[b, 0, b, :] = 1.0
    y = oracle_mod.das_sum(f, x, rx, np.zeros((1, 1), np.float32), np.ones((1, 1), np.float32))
    np.testing.assert_allclose(y[:, 0], [1.0, 0.5, 0.0, 0.5], atol=1e-6)


@pytest.mark.parametrize("noise", [False, True])
def test_point_scatterers_peak_at_their_voxel(oracle_mod, noise):
    cfg = das_synth.get_config("tiny")
    f = das_synth.problem_fields(cfg)
    rx = das_synth.array_positions(cfg)
    tau, w = das_synth.tx_tables(cfg)
    x = das_synth.rf(cfg, noise=noise).numpy()
    y = oracle_mod.das_sum(f, x, rx, tau, w, frames=[0, 5])
    nx, ny, nz = cfg.grid
    sv = das_synth.scatterer_voxels(cfg)
    assert sv.size == cfg.n_scatterers
    for j in range(2):
        a = np.abs(y[j]).reshape(nz, ny, nx)
        for n in sv:
            ix, iy, iz = n % nx, (n // nx) % ny, n // (nx * ny)
            nb = a[max(iz - 2, 0): iz + 3, max(iy - 2, 0): iy + 3, max(ix - 2, 0): ix + 3]
            assert a[iz, iy, ix] == nb.max(), (n, j)


def test_iq_scatterer_is_coherent(oracle_mod):
    """With the right phase sign the echo adds up coherently at the scatterer."""
    cfg = das_synth.custom_config("tiny", iq=True, n_scatterers=3)
    f = das_synth.problem_fields(cfg)
    rx = das_synth.array_positions(cfg)
    tau, w = das_synth.tx_tables(cfg)
    x = das_synth.rf(cfg, noise=False, frames=range(cfg.B)).numpy()
    sv = das_synth.scatterer_voxels(cfg)
    y = oracle_mod.das_sum(f, x, rx, tau, w, voxels=sv, frames=[0])[0]
    # upper bound for a fully coherent sum: amplitude x sum of weights
    s, _, w_rx = _geometry(f, rx, tau, sv)
    bound = das_synth.ECHO_AMPLITUDE * w_rx.sum(0)
    assert np.all(np.abs(y) > 0.9 * bound), (np.abs(y), bound)
    # the conjugate phase would scatter the contributions
    x_conj = x.copy()
    x_conj[..., 1] *= -1
    yc = oracle_mod.das_sum(f, x_conj, rx, tau, w, voxels=sv, frames=[0])[0]
    assert np.all(np.abs(yc) < 0.5 * bound)


def test_voxel_and_frame_subsets_match_full(oracle_mod):
    f, x, rx, tau, w = _random_problem(81)
    y = oracle_mod.das_sum(f, x, rx, tau, w)
    vox = [5, 0, 17]
    ys = oracle_mod.das_sum(f, x, rx, tau, w, voxels=vox, frames=[2, 0])
    assert np.array_equal(ys, y[[2, 0]][:, vox])


def test_rejects_bad_arguments(oracle_mod):
    f, x, rx, tau, w = _random_problem(91)
    with pytest.raises(ValueError):
        oracle_mod.das_sum(f, x[:, :, :, :-1], rx, tau, w)
    with pytest.raises(ValueError):
        oracle_mod.das_sum(f, x, rx, tau, w, voxels=[10 ** 6])
    with pytest.raises(ValueError):
        oracle_mod.das_sum(f, x, rx, tau, w, frames=[f["B"]])
    with pytest.raises(TypeError):
        oracle_mod.das_sum(f, x.astype(np.float16), rx, tau, w)


def test_float64_input_reads_doubles(oracle_mod):
    # float64 RF (the fp64 / complex128 baseline's input): values that float32
    # holds exactly give the float32 result bit for bit; the part float32
    # drops is summed too (linearity), so the reader sees all 53 bits
    for iq in (False, True):
        f, x, rx, tau, w = _random_problem(93, iq=iq)
        y32 = oracle_mod.das_sum(f, x, rx, tau, w)
        np.testing.assert_array_equal(oracle_mod.das_sum(f, x.astype(np.float64), rx, tau, w), y32)
        fine = np.random.default_rng(5).standard_normal(x.shape) * 1e-9
        x64 = x.astype(np.float64) + fine
        assert np.any(x64.astype(np.float32).astype(np.float64) != x64)
        y64 = oracle_mod.das_sum(f, x64, rx, tau, w)
        y_fine = oracle_mod.das_sum(f, fine, rx, tau, w)
        assert np.abs(y_fine).max() > 0
        np.testing.assert_allclose(y64, y32 + y_fine, rtol=0, atol=1e-12 * np.abs(y32).max())


def test_permute_references():
    import oracle
    x = np.arange(2 * 3 * 4 * 5, dtype=np.float32).reshape(2, 3, 4, 5)
    y = oracle.permute_kqmb(x)
    assert y.shape == (5, 3, 4, 2) and y[4, 2, 3, 1] == x[1, 2, 3, 4]
    z = oracle.permute_qmkb(x)
    assert z.shape == (3, 4, 5, 2) and z[2, 3, 4, 1] == x[1, 2, 3, 4]
    xi = np.arange(2 * 3 * 4 * 5 * 2, dtype=np.float32).reshape(2, 3, 4, 5, 2)
    assert oracle.permute_kqmb(xi)[4, 2, 3, 1, 1] == xi[1, 2, 3, 4, 1]


# ---------------------------------------------------------------------------
# Binary16 storage (the FP16 variant): the rounding, pinned bit for bit to
# hand-derived cases, and the beamform of rounded samples.
# ---------------------------------------------------------------------------

GOLDEN16 = os.path.join(os.path.dirname(__file__), "golden", "binary16_cases.json")


def test_binary16_hand_cases():
    import oracle
    cases = json.load(open(GOLDEN16))["cases"]
    x = np.array([int(c["f32"], 16) for c in cases], dtype=np.uint32).view(np.float32)
    got = oracle.to_binary16(x).astype(np.float16).view(np.uint16)
    for c, g in zip(cases, got):
        assert int(g) == int(c["f16"], 16), f"{c['f32']} -> {int(g):#06x}, expected {c['f16']} ({c['why']})"


def test_binary16_keeps_representable_values_and_nan():
    import oracle
    # every finite binary16 value, as float32, comes back unchanged
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = h[np.isfinite(h)].astype(np.float32)
    np.testing.assert_array_equal(oracle.to_binary16(finite), finite)
    assert np.isnan(oracle.to_binary16(np.array([np.nan], dtype=np.float32)))[0]
    with pytest.raises(TypeError):
        oracle.to_binary16(np.zeros(3, dtype=np.float64))


def test_binary16_is_the_nearest_half():
    import oracle
    # brute force over random float32 values in the normal range: no finite
    # half is closer than the rounded one, and the error is at most 2^-11 |x|
    rng = np.random.default_rng(61)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-13, 15, 4000))).astype(np.float32)
    y = oracle.to_binary16(x).astype(np.float64)
    halves = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    grid = np.unique(halves[np.isfinite(halves)].astype(np.float64))
    xd = x.astype(np.float64)
    i = np.clip(np.searchsorted(grid, xd), 1, grid.size - 1)
    best = np.minimum(np.abs(grid[i] - xd), np.abs(grid[i - 1] - xd))
    np.testing.assert_array_equal(np.abs(y - xd), best)
    normal = (np.abs(xd) >= np.exp2(-14)) & (np.abs(xd) <= 65504.0)
    assert normal.sum() > 3000
    assert np.all(np.abs(y - xd)[normal] <= np.exp2(-11) * np.abs(xd)[normal])


def test_binary16_storage_beamform(oracle_mod):
    import oracle
    for iq in (False, True):
        f, x, rx, tau, w = _random_problem(71, iq=iq)
        # samples a half holds exactly: storage changes nothing
        xi = np.random.default_rng(72).integers(-2048, 2049, x.shape).astype(np.float32)
        np.testing.assert_array_equal(oracle_mod.das_sum(f, oracle.to_binary16(xi), rx, tau, w),
                                      oracle_mod.das_sum(f, xi, rx, tau, w))
        # general samples: the change is the beamform of the rounding error
        # (linearity; the error is exact in float32), bounded by the weight sum
        # times the largest error, itself at most 2^-11 max|x|
        x16 = oracle.to_binary16(x)
        d = (x16 - x).astype(np.float32)
        assert np.abs(d).max() > 0
        y32 = oracle_mod.das_sum(f, x, rx, tau, w)
        y16 = oracle_mod.das_sum(f, x16, rx, tau, w)
        yd = oracle_mod.das_sum(f, d, rx, tau, w)
        np.testing.assert_allclose(y16, y32 + yd, rtol=0, atol=1e-12 * np.abs(y32).max())
        ones = np.ones(x.shape, dtype=np.float32)
        if iq:
            ones[..., 1] = 0.0
        wsum = np.abs(oracle_mod.das_sum(f, ones, rx, tau, w))     # weights are >= 0 here
        bound = wsum * np.abs(d).max() * (2.0 if iq else 1.0)
        assert np.all(np.abs(y16 - y32) <= bound + 1e-12)
        assert np.abs(d).max() <= np.exp2(-11) * np.abs(x).max()


# --------------------------------------------------------------------------
# The binary16 pair of the matrix-core variant: x = hi + lo
# --------------------------------------------------------------------------

def _f32(v):
    return np.array(v, dtype=np.float32)


def test_split_binary16_hand_cases():
    import oracle
    # 1 + 2^-11 + 2^-20 lies just above the tie between 1 and 1 + 2^-10, so hi
    # rounds up; the remainder -2^-11 + 2^-20 needs 10 significant bits: exact
    x = _f32([1 + 2.0 ** -11 + 2.0 ** -20])
    hi, lo = oracle.split_binary16(x)
    assert hi[0] == 1 + 2.0 ** -10 and lo[0] == -2.0 ** -11 + 2.0 ** -20
    # exactly on the tie: ties to even keeps 1, the remainder 2^-11 is a half
    hi, lo = oracle.split_binary16(_f32([1 + 2.0 ** -11]))
    assert hi[0] == 1.0 and lo[0] == 2.0 ** -11
    # a half needs no remainder; zero stays zero; the sign is kept
    hi, lo = oracle.split_binary16(_f32([0.5, -3.75, 0.0, 65504.0]))
    np.testing.assert_array_equal(hi, _f32([0.5, -3.75, 0.0, 65504.0]))
    np.testing.assert_array_equal(lo, _f32([0.0, 0.0, 0.0, 0.0]))
    # 0.1: hi = 0x2e66 = 0.0999755859375, remainder 2.4414e-5 rounds to a half
    hi, lo = oracle.split_binary16(_f32([0.1]))
    assert hi[0] == np.float32(np.float16(0.1)) == 0.0999755859375
    assert lo[0] == np.float32(np.float16(np.float32(0.1) - np.float32(0.0999755859375)))
    # a remainder below the normal range is a subnormal half (absolute step 2^-24)
    hi, lo = oracle.split_binary16(_f32([2.0 ** -4 + 2.0 ** -20]))
    assert hi[0] == 2.0 ** -4 and lo[0] == 2.0 ** -20


def test_split_binary16_error_bound_and_halves():
    import oracle
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-2, 14, 20000))).astype(np.float32)
    x = x[np.abs(x) < 65000]
    hi, lo = oracle.split_binary16(x)
    # both parts are binary16 values
    np.testing.assert_array_equal(hi.astype(np.float16).astype(np.float32), hi)
    np.testing.assert_array_equal(lo.astype(np.float16).astype(np.float32), lo)
    # hi is the nearest half; the pair is within 2^-22 |x| in the normal range
    err = np.abs(x.astype(np.float64) - hi - lo)
    assert np.all(err <= 2.0 ** -22 * np.abs(x.astype(np.float64)) + 2.0 ** -25)
    assert np.all(np.abs(x.astype(np.float64) - hi) <= 2.0 ** -11 * np.abs(x.astype(np.float64)))
    # values of at most 22 significant bits split exactly while the remainder's
    # lowest bit is still a binary16 step (|x| >= 2^-3)
    m = rng.integers(2 ** 21, 2 ** 22, 5000)
    e = rng.integers(-3, 5, 5000)
    y = (m.astype(np.float64) * np.exp2(e - 21)).astype(np.float32)
    hy, ly = oracle.split_binary16(y)
    np.testing.assert_array_equal(hy.astype(np.float64) + ly.astype(np.float64), y.astype(np.float64))


def test_split_binary16_takes_float32_only():
    import oracle
    with pytest.raises(TypeError):
        oracle.split_binary16(np.zeros(3, dtype=np.float64))
