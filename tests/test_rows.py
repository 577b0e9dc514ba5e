"""GPU: the LDS-staged batch-inner kernel with whole-row lanes ("ffdas:
volumetric ultrasound reconstruction at warp speed", Section 3, batch-inner
tiling and spatial locality; FP16 paragraph for binary16 storage): 8 or 16
receivers a step (fp32), complex64 samples, native and binary16 storage.
The default (fp32, 16 receivers a step, native) also runs in every fp32
parity test with B a multiple of 32.

Each case meets the same bar as every other kernel against the fp64 oracle
(max|err| <= 1e-4 max|oracle|, relative L2 <= 1e-5): ragged grids and
receiver counts, 32, 64 and 96 frames (several frame tiles), start times of
both signs, coarse voxels whose windows exceed the staged rows (direct
loads), one event per call with accumulation, both layouts, and the Main
workload sampled at full size.
"""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, oracle_ref, run_gpu, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu

VARIANTS = [("1", False), ("2", False), ("1", True)]
IDS = ["f32-8rx", "f32-16rx", "c64-8rx"]


def _use(monkeypatch, rows):
    monkeypatch.setenv("DAS_STAGED_ROWS", rows)


def _ragged(iq, B=32, K=300, **kw):
    base = dict(name="rows", seed=61, array=(37, 2), grid=(19, 13, 5), K=K, B=B, tx="diverging",
                sources=((0.0, 0.0), (1.5e-3, -0.5e-3), (-1e-3, 1e-3)), n_scatterers=0, iq=iq)
    base.update(kw)
    return das_synth.custom_config("tiny", **base)


def _info(inp, storage="native"):
    import volumetric_delay_sum_amd as das
    return das.plan_from_fields(inp.fields, "batch_inner", "qmkb", storage=storage).info


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("B", [16, 32, 48, 64, 96])
@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_ragged(gpu, monkeypatch, rows, iq, B, layout, storage):
    _use(monkeypatch, rows)
    inp = Inputs(_ragged(iq, B=B), w_tx="uniform")
    info = _info(inp, storage)
    assert info["whole_rows"] == 1 and info["receivers_per_step"] == 8 * int(rows)
    y = to_numpy(run_gpu(inp, "batch_inner", layout, storage=storage), iq)
    assert_parity(y, oracle_ref(inp, storage=storage), f"rows={rows} iq={iq} B={B} {layout} {storage}")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("t0", [3.0 / 20e6, 1.37e-6, -0.83e-6], ids=["3_periods", "plus_1.37us", "minus_0.83us"])
@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_start_time(gpu, monkeypatch, rows, iq, t0, storage):
    _use(monkeypatch, rows)
    inp = Inputs(_ragged(iq, t0=t0, K=320), w_tx="uniform")
    y = to_numpy(run_gpu(inp, "batch_inner", "qmkb", storage=storage), iq)
    assert_parity(y, oracle_ref(inp, storage=storage), f"rows={rows} iq={iq} t0={t0} {storage}")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("voxel", [0.6e-3, 1.5e-3], ids=["mixed", "coarse"])
@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_windows_wider_than_the_regions(gpu, monkeypatch, rows, iq, voxel, storage):
    """Coarse voxels: some steps' windows exceed a region (38 positions with
    16 receivers a step, 78 with 8), and those steps read the permuted buffer."""
    _use(monkeypatch, rows)
    cfg = _ragged(iq, K=900, voxel=voxel, z0=3e-3, grid=(19, 10, 3), array=(19, 3), f_number=0.0,
                  sources=((0.0, 0.0), (2e-3, 1e-3)))
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "batch_inner", "kqmb", storage=storage), iq)
    assert_parity(y, oracle_ref(inp, storage=storage), f"rows={rows} iq={iq} voxel={voxel} {storage}")


@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_one_event_per_call_and_accumulate(gpu, monkeypatch, rows, iq):
    import torch
    _use(monkeypatch, rows)
    inp = Inputs(_ragged(iq, B=64), w_tx="uniform")
    ref = oracle_ref(inp)
    assert_parity(to_numpy(run_gpu(inp, "batch_inner", "qmkb", q_chunk=1), iq), ref, f"rows={rows} q chunks")
    shape = (inp.cfg.B, inp.cfg.N, 2) if iq else (inp.cfg.B, inp.cfg.N)
    start = torch.linspace(-3.0, 3.0, int(np.prod(shape)), device="cuda").reshape(shape)
    out = run_gpu(inp, "batch_inner", "kqmb", out=start.clone(), accumulate_into=True)
    got = to_numpy(out, iq) - to_numpy(start, iq)
    assert_parity(got, ref, f"rows={rows} accumulate")


@pytest.mark.parametrize("rows,iq", [("1", False), ("1", True)], ids=["f32-8rx", "c64-8rx"])
def test_main_sampled(gpu, monkeypatch, rows, iq):
    _use(monkeypatch, rows)
    inp = Inputs(das_synth.get_config("main-c64" if iq else "main"))
    vox = sample_voxels(inp.cfg, 128, seed=5)
    out = run_gpu(inp, "batch_inner", "qmkb")
    assert_all_written(out, f"main rows={rows} iq={iq}")
    assert_parity(to_numpy(out, iq)[:, vox], oracle_ref(inp, voxels=vox), f"main rows={rows} iq={iq}")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_tiles_outside_every_aperture(gpu, monkeypatch, rows, iq, storage):
    """A volume much wider than the array: the outer tiles (8 voxels wide
    along x) see no receiver inside their cones and skip every receiver
    block, the next ones keep a few blocks, the central ones all.  Every voxel whose receive weights
    are all zero comes out exactly 0 (and exactly unchanged when accumulating),
    the rest meet the usual bar."""
    import torch
    _use(monkeypatch, rows)
    cfg = _ragged(iq, B=32, K=400, array=(16, 4), grid=(40, 9, 4), voxel=0.5e-3, z0=2e-3, f_number=2.0,
                  sources=((0.0, 0.0), (1e-3, 0.0)))
    inp = Inputs(cfg, w_tx="uniform")
    ref = oracle_ref(inp, storage=storage)
    y = to_numpy(run_gpu(inp, "batch_inner", "qmkb", storage=storage), iq)
    zero = ref == 0.0
    assert 0.5 < zero.mean() < 0.99, zero.mean()
    assert np.array_equal(y == 0.0, zero)
    assert_parity(y, ref, f"rows={rows} iq={iq} apertures")
    shape = (cfg.B, cfg.N, 2) if iq else (cfg.B, cfg.N)
    start = torch.linspace(-3.0, 3.0, int(np.prod(shape)), device="cuda").reshape(shape)
    out = run_gpu(inp, "batch_inner", "qmkb", out=start.clone(), accumulate_into=True, storage=storage)
    got, base = to_numpy(out, iq), to_numpy(start, iq)
    assert np.array_equal(got[zero], base[zero])
    assert_parity(got - base, ref, f"rows={rows} iq={iq} apertures accumulate")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
def test_main_binary16_default(gpu, iq):
    """The default binary16 plans on Main (16 receivers a step fp32, 8
    complex), sampled, against the oracle of the rounded samples."""
    inp = Inputs(das_synth.get_config("main-c64" if iq else "main"))
    assert _info(inp, "f16")["whole_rows"] == 1
    vox = sample_voxels(inp.cfg, 128, seed=6)
    out = run_gpu(inp, "batch_inner", "qmkb", storage="f16")
    assert_all_written(out, f"main f16 iq={iq}")
    assert_parity(to_numpy(out, iq)[:, vox], oracle_ref(inp, voxels=vox, storage="f16"), f"main f16 iq={iq}")


@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("array", [(48, 48), (64, 64)], ids=["2304rx", "4096rx"])
def test_many_receivers(gpu, monkeypatch, array, iq):
    """A 48 x 48 array (2304 receivers: three rounds of the per-receiver
    test) and the largest array the kernel lists, 64 x 64 = 4096 receivers,
    without apodization so that every receiver is listed (the whole 8 KB
    list, 512 blocks), over a small grid."""
    f_number = 1.0 if array[0] < 64 else 0.0
    cfg = _ragged(iq, B=32 if not iq else 16, K=500, array=array, grid=(12, 9, 3),
                  sources=((0.0, 0.0), (1e-3, 1e-3)), f_number=f_number)
    inp = Inputs(cfg, w_tx="uniform")
    assert _info(inp)["whole_rows"] == 1
    y = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), iq)
    assert_parity(y, oracle_ref(inp), f"{array[0] * array[1]} receivers iq={iq}")


@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_grid_with_negative_spacing(gpu, monkeypatch, rows, iq):
    """The same voxels indexed from the far corner (negative pitch on every
    axis): the aperture test must take the plane farthest in front of each
    receiver from either end of the z axis.  The result is the ordinary one
    with the voxel index reversed."""
    import copy
    import torch
    _use(monkeypatch, rows)
    cfg = _ragged(iq, K=320, f_number=1.5)
    inp = Inputs(cfg, w_tx="uniform")
    nx, ny, nz = cfg.grid
    (ox, oy, oz), (sx, sy, sz) = inp.fields["origin"], inp.fields["spacing"]
    flip = copy.copy(inp)
    flip.fields = dict(inp.fields, origin=(ox + (nx - 1) * sx, oy + (ny - 1) * sy, oz + (nz - 1) * sz),
                       spacing=(-sx, -sy, -sz))
    rev = np.arange(cfg.N)[::-1].copy()                 # flipped voxel n is ordinary voxel N - 1 - n
    flip.tau, flip.w = inp.tau[:, rev].copy(), inp.w[:, rev].copy()
    flip.tau_d, flip.w_d = torch.from_numpy(flip.tau).cuda(), torch.from_numpy(flip.w).cuda()
    ref = oracle_ref(flip)
    y = to_numpy(run_gpu(flip, "batch_inner", "qmkb"), iq)
    assert_parity(y, ref, f"negative pitch rows={rows} iq={iq}")
    y0 = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), iq)
    assert_parity(y, y0[:, rev], f"negative pitch against ordinary rows={rows} iq={iq}")


ORDER_CASES = {
    # 4 x 2 lateral tiles (a multiple of 8: chunks of one tile shared out to
    # the dies by work), 3 depths
    "die_chunks": dict(grid=(32, 16, 6), array=(24, 6)),
    # 4 x 4 lateral tiles (chunks of two), 4 depths
    "die_chunks_2": dict(grid=(32, 32, 8), array=(20, 8)),
    # 3 x 2 lateral tiles, ragged on every axis
    "ragged": dict(grid=(19, 13, 5)),
    # outer tiles with no live block, inner ones with all
    "apertures": dict(array=(16, 4), grid=(40, 9, 4), voxel=0.5e-3, z0=2e-3, f_number=2.0),
    # no receive apodization: every tile has every block
    "no_apodization": dict(grid=(24, 17, 4), f_number=0.0),
}


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("B", [32, 48])
@pytest.mark.parametrize("case", list(ORDER_CASES))
@pytest.mark.parametrize("rows,iq", VARIANTS, ids=IDS)
def test_tile_order(gpu, monkeypatch, rows, iq, case, B, storage):
    """Tiles launched by decreasing live receiver count (DAS_ROWS_ORDER=2
    sorts at any size) give the sums of the sequence-order launch
    (DAS_ROWS_ORDER=0) bit for bit, and meet the oracle bar."""
    _use(monkeypatch, rows)
    inp = Inputs(_ragged(iq, B=B, K=400, **ORDER_CASES[case]), w_tx="uniform")
    got = {}
    for mode in ("0", "2"):
        monkeypatch.setenv("DAS_ROWS_ORDER", mode)
        out = run_gpu(inp, "batch_inner", "qmkb", storage=storage)
        assert_all_written(out, f"order {mode} {case}")
        got[mode] = out.cpu().numpy()
    assert np.array_equal(got["0"], got["2"]), f"rows={rows} iq={iq} {case} B={B} {storage}"
    import torch
    assert_parity(to_numpy(torch.from_numpy(got["2"]), iq), oracle_ref(inp, storage=storage),
                  f"ordered rows={rows} iq={iq} {case} B={B} {storage}")


def test_tile_order_two_streams(gpu, monkeypatch):
    """Calls in flight on two streams at once, with different receiver
    positions (so different tile orders), each take a work area of their
    own: every result equals the one computed alone, bit for bit."""
    import torch
    import volumetric_delay_sum_amd as das
    monkeypatch.setenv("DAS_ROWS_ORDER", "2")
    inp = Inputs(_ragged(False, B=32, K=500, array=(24, 6), grid=(40, 24, 8), f_number=1.5,
                         sources=((0.0, 0.0), (1e-3, 0.0))), w_tx="uniform")
    plan = das.plan_from_fields(inp.fields, "batch_inner", "qmkb")
    Q = inp.cfg.Q
    perm = torch.empty(plan.permuted_shape(Q), dtype=plan.permuted_dtype(), device="cuda")
    plan.permute(inp.rf_d, perm, 0, Q)
    rx_b = inp.rx_d.clone()
    rx_b[:, 0] += 2.5e-3                                  # the array moved along x: other live counts
    rxs = (inp.rx_d, rx_b)
    ref = []
    for rx in rxs:
        o = torch.empty(plan.output_shape(), dtype=torch.float32, device="cuda")
        plan.beamform(perm, rx, inp.tau_d, inp.w_d, o, 0, Q)
        torch.cuda.synchronize()
        ref.append(o.cpu().numpy())
    assert not np.array_equal(ref[0], ref[1])
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    outs = [[torch.full(plan.output_shape(), float("nan"), device="cuda") for _ in range(6)] for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(6):
        for j in (0, 1):
            plan.beamform(perm, rxs[j], inp.tau_d, inp.w_d, outs[j][i], 0, Q, stream=streams[j])
    torch.cuda.synchronize()
    for j in (0, 1):
        for i in range(6):
            assert np.array_equal(outs[j][i].cpu().numpy(), ref[j]), f"stream {j} call {i}"


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("q_chunk", [16, 17, 20])
def test_complex_transmit_phasors_many_events(gpu, layout, storage, q_chunk):
    # A complex launch of up to 16 events keeps each voxel's w_tx exp(+j 2 pi
    # f0 tau_tx) in LDS; a launch of more events forms the phasor per step.
    # 20 diverging events with random transmit weights, called in chunks of
    # 16 (the table: 16 + 4), 17 (17 events without it, then 3 with it) and
    # 20 (without it), against the oracle.
    src = tuple((x * 1e-3, y * 1e-3) for x in (-1.5, -0.5, 0.5, 1.5) for y in (-1.0, -0.5, 0.0, 0.5, 1.0))
    inp = Inputs(_ragged(True, B=32, sources=src), w_tx="uniform")
    assert inp.cfg.Q == 20
    y = to_numpy(run_gpu(inp, "batch_inner", layout, storage=storage, q_chunk=q_chunk), True)
    assert_parity(y, oracle_ref(inp, storage=storage), f"Q=20 chunks of {q_chunk} {layout} {storage}")
