"""GPU: das_beamform_noalloc, the entry point that allocates no device memory
(its whole-row tile order lives in the library's fixed device array), against
das_beamform on the same inputs: bit for bit (the same kernels on the same
tiles), and against the oracle bar (max|err| <= 1e-4 max|oracle|, relative
L2 <= 1e-5).  Two calls in a row, the second on a smaller volume, so the
second runs over what the first left in the shared array; then the Main
workload (2048 tiles, sorted by default) in fp32 and complex64.
"""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, oracle_ref, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu


def _run(inp, noalloc):
    import torch
    import volumetric_delay_sum_amd as das
    plan = das.plan_from_fields(inp.fields, "batch_inner", "qmkb")
    assert plan.info["whole_rows"] == 1
    Q = inp.cfg.Q
    perm = torch.empty(plan.permuted_shape(Q), dtype=plan.permuted_dtype(), device="cuda")
    out = torch.full(plan.output_shape(), float("nan"), dtype=torch.float32, device="cuda")
    plan.permute(inp.rf_d, perm, 0, Q)
    plan.beamform(perm, inp.rx_d, inp.tau_d, inp.w_d, out, 0, Q, noalloc=noalloc)
    torch.cuda.synchronize()
    assert_all_written(out, f"noalloc={noalloc}")
    return out.cpu().numpy()


def _case(grid, iq=False):
    return das_synth.custom_config("tiny", name="noalloc", seed=67, array=(24, 6), grid=grid, K=500, B=32,
                                   tx="diverging", sources=((0.0, 0.0), (1.2e-3, -0.4e-3)), n_scatterers=0,
                                   iq=iq, f_number=1.5)


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_noalloc_two_calls(gpu, monkeypatch, iq):
    import torch
    monkeypatch.setenv("DAS_ROWS_ORDER", "2")           # sort the tiles at any size
    for grid in ((40, 24, 8), (19, 13, 5)):              # 60 tiles, then 18
        inp = Inputs(_case(grid, iq), w_tx="uniform")
        a = _run(inp, noalloc=True)
        b = _run(inp, noalloc=False)
        assert np.array_equal(a, b), f"grid {grid} iq={iq}"
        assert_parity(to_numpy(torch.from_numpy(a), iq), oracle_ref(inp), f"noalloc grid {grid} iq={iq}")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_noalloc_main(gpu, iq):
    import torch
    inp = Inputs(das_synth.get_config("main-c64" if iq else "main"))
    a = _run(inp, noalloc=True)
    b = _run(inp, noalloc=False)
    assert np.array_equal(a, b), f"main iq={iq}"
    vox = sample_voxels(inp.cfg, 64, seed=8)
    assert_parity(to_numpy(torch.from_numpy(a), iq)[:, vox], oracle_ref(inp, voxels=vox), f"main noalloc iq={iq}")
