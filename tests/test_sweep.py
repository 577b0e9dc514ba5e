"""GPU parity over seeded random shapes: frame counts that select every kernel
variant (baseline, direct loads, LDS-staged with 1, 2 or 4 frames per lane,
split rows, fallback to direct loads), both layouts, fp32 and complex64,
binary16 or native sample storage, several f-numbers and start times, plane
and diverging transmits, events in one call or one at a time.  Each case is compared element by element with the fp64 oracle
to the same bar as the other parity tests."""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_parity, oracle_ref, run_gpu, to_numpy

pytestmark = pytest.mark.gpu

N_CASES = 40


def _case(i):
    rng = np.random.default_rng([2024, i])
    iq = bool(rng.random() < 0.35)
    B = int(rng.choice([1, 5, 16, 24, 32, 48, 64, 96, 128]))
    nsrc = int(rng.integers(1, 4))
    sources = tuple((float(rng.uniform(-3e-3, 3e-3)), float(rng.uniform(-3e-3, 3e-3))) for _ in range(nsrc))
    cfg = das_synth.custom_config(
        "tiny", name=f"sweep{i}", seed=100 + i,
        array=(int(rng.integers(1, 24)), int(rng.integers(1, 4))),
        grid=(int(rng.integers(1, 14)), int(rng.integers(1, 10)), int(rng.integers(1, 6))),
        K=int(rng.integers(40, 700)), B=B, iq=iq, n_scatterers=0,
        tx="plane" if rng.random() < 0.25 else "diverging", sources=sources,
        voxel=float(rng.choice([0.15e-3, 0.25e-3, 0.5e-3, 1.2e-3])),
        z0=float(rng.uniform(1e-3, 6e-3)),
        f_number=float(rng.choice([0.0, 0.5, 1.0, 2.0])),
        # start time from a generator of its own, so the other draws stay as they were:
        # zero, a whole number of sample periods, or any fraction of a microsecond
        t0=float(np.random.default_rng([2025, i]).choice([0.0, 2.0 / 20e6, 0.37e-6, -0.61e-6])))
    r = rng.random()
    alg, layout = ("baseline", "kqmb") if r < 0.2 else ("batch_inner", "kqmb" if r < 0.6 else "qmkb")
    q_chunk = 1 if rng.random() < 0.3 else None
    storage = "f16" if alg == "batch_inner" and rng.random() < 0.3 else "native"
    return cfg, alg, layout, q_chunk, storage


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shapes(gpu, i):
    cfg, alg, layout, q_chunk, storage = _case(i)
    what = (f"case {i}: B={cfg.B} iq={cfg.iq} M={cfg.M} grid={cfg.grid} K={cfg.K} Q={cfg.Q} "
            f"voxel={cfg.voxel} f#={cfg.f_number} t0={cfg.t0} {cfg.tx} {alg}/{layout} q_chunk={q_chunk} "
            f"storage={storage}")
    print(what, flush=True)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout, q_chunk=q_chunk, storage=storage), cfg.iq)
    ref = oracle_ref(inp, storage=storage)
    if np.abs(ref).max() == 0.0:            # every term out of range: exact zeros
        assert np.all(np.asarray(y) == 0.0), what
    else:
        assert_parity(y, ref, what)
