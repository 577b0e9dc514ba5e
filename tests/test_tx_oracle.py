"""Pins of the oracle's transmit-table generator (CPU only).

The tables hold the time a plane or diverging transmit front reaches each
voxel centre ("ffdas: volumetric ultrasound reconstruction at warp speed",
Section 3, baseline paragraph: per-voxel transmit tables).  Each test checks a
property that the wavefront geometry fixes, not the formula restated: on-axis
points, travel along and across the propagation direction, spherical
symmetry, the far-source limit, and an independent generator."""
import math

import numpy as np
import pytest

import das_synth

C = 1540.0


def _fields(nx=9, ny=7, nz=11, origin=(-1e-3, -0.8e-3, 4e-3), spacing=(0.25e-3, 0.25e-3, 0.3e-3)):
    return dict(nx=nx, ny=ny, nz=nz, origin=origin, spacing=spacing, c=C)


def _positions(f):
    n = np.arange(f["nx"] * f["ny"] * f["nz"])
    ix, iy, iz = n % f["nx"], (n // f["nx"]) % f["ny"], n // (f["nx"] * f["ny"])
    o, s = f["origin"], f["spacing"]
    return np.stack([o[0] + ix * s[0], o[1] + iy * s[1], o[2] + iz * s[2]], axis=-1)


def test_zero_degree_plane_is_depth_over_c(oracle_mod):
    f = _fields()
    tau, w = oracle_mod.tx_tables(f, [(oracle_mod.TX_PLANE, (0.0, 0.0, 1.0), 0.75)])
    z = _positions(f)[:, 2]
    np.testing.assert_array_equal(tau[0], (z / C).astype(np.float32))
    assert np.all(w == np.float32(0.75))


def test_diverging_on_axis_is_depth_over_c(oracle_mod):
    # voxels straight below the source: the front has travelled |v_z| + z
    f = _fields(nx=1, ny=1, nz=40, origin=(1e-3, -2e-3, 2e-3))
    tau, _ = oracle_mod.tx_tables(f, [(oracle_mod.TX_DIVERGING, (1e-3, -2e-3, -10e-3), 1.0)])
    z = _positions(f)[:, 2]
    np.testing.assert_allclose(tau[0].astype(np.float64), z / C, rtol=1.2e-7, atol=0)


@pytest.mark.parametrize("alpha", [-0.3, 0.0, 0.2, 0.5])
def test_plane_travel_along_and_across_the_direction(oracle_mod, alpha):
    u = (math.sin(alpha), 0.0, math.cos(alpha))
    tau, _ = oracle_mod.tx_tables(_fields(), [(oracle_mod.TX_PLANE, u, 1.0)])
    r = _positions(_fields())
    t = tau[0].astype(np.float64)
    # along u: the delay grows by distance / c; across u (here the y axis and
    # the in-plane normal): it does not change
    i, j = 3, 200
    along = float(np.dot(r[j] - r[i], u))
    assert abs((t[j] - t[i]) - along / C) <= 4 * np.spacing(np.float32(t[j]))
    same = [k for k in range(len(r)) if abs(np.dot(r[k] - r[i], u)) < 1e-15]
    assert len(same) >= 2 and np.ptp(t[same]) == 0.0


def test_diverging_spherical_symmetry_and_lipschitz(oracle_mod):
    f = _fields(nx=15, ny=15, nz=6, origin=(-1.75e-3, -1.75e-3, 3e-3))
    v = (0.0, 0.0, -8e-3)
    tau, _ = oracle_mod.tx_tables(f, [(oracle_mod.TX_DIVERGING, v, 1.0)])
    r = _positions(f)
    t = tau[0].astype(np.float64)
    # mirror images through the source axis are equidistant from the source
    mirror = (-r[:, 0], r[:, 1], r[:, 2])
    nxy = f["nx"]
    ix = np.arange(len(r)) % nxy
    j = np.arange(len(r)) - ix + (nxy - 1 - ix)
    np.testing.assert_array_equal(t, t[j])
    assert np.allclose(mirror[0], r[j, 0])
    # a front moves at c: delays differ by at most distance / c
    rng = np.random.default_rng(3)
    a, b = rng.integers(0, len(r), 500), rng.integers(0, len(r), 500)
    dist = np.linalg.norm(r[a] - r[b], axis=1)
    assert np.all(np.abs(t[a] - t[b]) <= dist / C + 2 * np.spacing(np.float32(t.max())))
    # and exactly at c along a ray from the source
    d = np.linalg.norm(r - np.array(v), axis=1)
    np.testing.assert_allclose(t, (d - 8e-3) / C, rtol=1.2e-7, atol=1e-13)


def test_far_source_tends_to_the_zero_degree_plane(oracle_mod):
    f = _fields()
    r = _positions(f)
    plane, _ = oracle_mod.tx_tables(f, [(oracle_mod.TX_PLANE, (0.0, 0.0, 1.0), 1.0)])
    prev = None
    for depth in (1e-1, 1e0, 1e1):
        div, _ = oracle_mod.tx_tables(f, [(oracle_mod.TX_DIVERGING, (0.0, 0.0, -depth), 1.0)])
        gap = np.abs(div[0].astype(np.float64) - plane[0]).max()
        # the front's sag over the lateral extent is about rho^2 / (2 depth)
        rho2 = (r[:, 0] ** 2 + r[:, 1] ** 2).max()
        assert gap <= rho2 / (2 * depth) / C * 1.01 + 1e-12
        if prev is not None:
            assert gap < prev
        prev = gap


def test_matches_the_input_generator_on_the_named_configs(oracle_mod):
    for name in ("tiny", "mid", "main"):
        cfg = das_synth.get_config(name)
        fields = das_synth.problem_fields(cfg)
        if cfg.tx == "plane":
            events = [(oracle_mod.TX_PLANE, (0.0, 0.0, 1.0), 1.0)] * cfg.Q
        else:
            events = [(oracle_mod.TX_DIVERGING, (vx, vy, -cfg.src_depth), 1.0) for vx, vy in cfg.sources]
        tau, w = oracle_mod.tx_tables(fields, events)
        tau_g, w_g = das_synth.tx_tables(cfg)
        ulp = np.abs(tau.view(np.int32).astype(np.int64) - tau_g.view(np.int32))
        assert ulp.max() <= 1, name
        np.testing.assert_array_equal(w, w_g)


def test_rejects_unknown_kind(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.tx_tables(_fields(), [(7, (0.0, 0.0, 1.0), 1.0)])
