"""GPU parity with a non-zero start time t0 (the time of sample k = 0).

Every named workload records from t0 = 0, so these cases are the only ones
that check the sign of t0 in the sample position s = (tau - t0) fs and that
the IQ phase exp(+j 2 pi f0 tau) is taken on the absolute time tau, not on
tau - t0.  Each kernel is compared element by element with the fp64 oracle on
a small ragged shape: the baseline, the batch-inner kernel with direct loads
and the LDS-staged one (one, two or four frames per lane, whole and split
rows), both permuted layouts, fp32 and complex64 samples, native and binary16
storage.  t0 takes a whole number of sample periods, a positive fraction of
one and a negative value.
"""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_parity, oracle_ref, run_gpu, to_numpy

pytestmark = pytest.mark.gpu

FS = 20e6
# 3 / fs exactly; +1.37 us = 27.4 sample periods; -0.83 us = -16.6 periods
T0S = [3.0 / FS, 1.37e-6, -0.83e-6]
T0_IDS = ["3_periods", "plus_1.37us", "minus_0.83us"]


def _cfg(t0, iq=False, B=32, K=320):
    # depth 5.0-5.4 mm, receivers within 5.4 mm laterally, sources within
    # 2 mm: s = (tau - t0) fs stays inside [0, K - 2] for every t0 above, so
    # a wrong sign moves every term by 2 t0 fs samples instead of dropping it
    return das_synth.custom_config("tiny", name="start_time", seed=41, array=(37, 1), grid=(13, 7, 3), K=K, B=B,
                                   tx="diverging", sources=((0.0, 0.0), (1.5e-3, -0.5e-3), (-1e-3, 1e-3)),
                                   iq=iq, n_scatterers=0, t0=t0)


KERNELS = [
    # (algorithm, layout, DAS_BI_KERNEL override)
    ("baseline", "kqmb", None),
    ("batch_inner", "kqmb", None),
    ("batch_inner", "qmkb", None),
    ("batch_inner", "kqmb", "direct"),
]
KERNEL_IDS = ["baseline", "staged-kqmb", "staged-qmkb", "direct"]


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("t0", T0S, ids=T0_IDS)
def test_start_time_native(gpu, monkeypatch, t0, kernel, iq):
    alg, layout, override = kernel
    if override:
        monkeypatch.setenv("DAS_BI_KERNEL", override)
    inp = Inputs(_cfg(t0, iq=iq), w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), iq)
    assert_parity(y, oracle_ref(inp), f"t0={t0} {alg}/{layout}/{override} iq={iq}")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("kernel", KERNELS[1:], ids=KERNEL_IDS[1:])
@pytest.mark.parametrize("t0", T0S, ids=T0_IDS)
def test_start_time_binary16(gpu, monkeypatch, t0, kernel, iq):
    alg, layout, override = kernel
    if override:
        monkeypatch.setenv("DAS_BI_KERNEL", override)
    inp = Inputs(_cfg(t0, iq=iq), w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout, storage="f16"), iq)
    assert_parity(y, oracle_ref(inp, storage="f16"), f"t0={t0} f16 {alg}/{layout}/{override} iq={iq}")


@pytest.mark.parametrize("kernel", ["default", "dpp_rows"])
@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("B", [16, 64], ids=["B16", "B64"])
@pytest.mark.parametrize("storage", ["native", "f16"])
def test_start_time_other_staged_shapes(gpu, monkeypatch, B, iq, storage, kernel):
    """B = 16 and B = 64 at a fractional negative t0.  Default: whole-row
    lanes with 16- and 32-frame tiles.  "dpp_rows" (DAS_STAGED_ROWS=0): the
    DPP-row kernel with one frame per lane (B = 16) and, for B = 64, split
    rows (two voxels per DPP row, 16 bytes per lane)."""
    import volumetric_delay_sum_amd as das
    if kernel == "dpp_rows":
        monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    inp = Inputs(_cfg(-0.83e-6, iq=iq, B=B), w_tx="uniform")
    info = das.plan_from_fields(inp.fields, "batch_inner", "qmkb", storage=storage).info
    assert info["staged"] == 1 and info["whole_rows"] == (1 if kernel == "default" else 0)
    y = to_numpy(run_gpu(inp, "batch_inner", "qmkb", storage=storage), iq)
    assert_parity(y, oracle_ref(inp, storage=storage), f"t0<0 B={B} {storage} iq={iq} {kernel}")


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
def test_iq_phase_on_absolute_time(gpu, monkeypatch, kernel):
    """With t0 = 1.37 us and f0 = 5 MHz, a phase taken on tau - t0 instead of tau
    would turn the whole volume by exp(-j 2 pi f0 t0) = exp(-j 2 pi 6.85): the
    result would then sit far outside the bar (the check on the wrong-phase
    volume below makes sure the case can tell the two apart)."""
    alg, layout, override = kernel
    if override:
        monkeypatch.setenv("DAS_BI_KERNEL", override)
    t0 = 1.37e-6
    inp = Inputs(_cfg(t0, iq=True), w_tx="uniform")
    y = to_numpy(run_gpu(inp, alg, layout), True)
    ref = oracle_ref(inp)
    assert_parity(y, ref, f"IQ phase {alg}/{layout}/{override}")
    f0 = inp.fields["f_demod"]
    wrong = ref * np.exp(-2j * np.pi * f0 * t0)
    err = np.abs(y - wrong).max() / np.abs(wrong).max()
    assert err > 0.5, f"the phase on tau - t0 would also pass ({err:.2e}): the case cannot tell them apart"
