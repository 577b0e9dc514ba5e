"""GPU: the matrix-core (repack) variant ("ffdas: volumetric ultrasound
reconstruction at warp speed", Section 3, tensor-core paragraphs and
Algorithm 3; ffdas docs, ALG4).

Its permute must write the binary16 pairs of the oracle's split bit for bit
(or the binary16 rounding with binary16 storage), and its beamform must meet
the same bar as every other kernel against the fp64 oracle (max|err| <= 1e-4
max|oracle|, relative L2 <= 1e-5): of the float32 samples with native
storage, of the rounded samples with binary16 storage.  Cases cover ragged
grids and receiver counts, 32, 64 and 96 frames, records that end inside the
window, start times of both signs, several f-numbers, coarse voxels (windows
wider than the staged rows: the direct-read path), one event per call,
accumulation, tiles whose receiver lists are empty or short, receiver counts
up to and past the listed maximum, and the named Main and Large workloads at
full size.
"""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, oracle_ref, run_gpu, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu


def _repack_layout(rf, q_begin, q_count, storage):
    """The permuted buffer as the oracle defines it: (q, M, 2, P, B, 8) halves,
    the hi then the lo parts of the samples in pieces of 8 positions (P =
    ceil(K/8), positions past K zero), each piece the B frames side by side
    (binary16 storage: (q, M, P, B, 8) rounded samples)."""
    import oracle
    B, Q, M, K = rf.shape
    npc = (K + 7) // 8
    pad = np.zeros((B, q_count, M, 8 * npc), dtype=np.float32)
    pad[..., :K] = rf[:, q_begin:q_begin + q_count]
    pieces = lambda a: np.ascontiguousarray(a.reshape(B, q_count, M, npc, 8).transpose(1, 2, 3, 0, 4))
    if storage == "f16":
        return pieces(oracle.to_binary16(pad)).astype(np.float16)
    hi, lo = oracle.split_binary16(pad)
    return np.stack([pieces(hi).astype(np.float16), pieces(lo).astype(np.float16)], axis=2)


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("B,K,q_begin,q_count", [(32, 64, 0, 3), (32, 67, 1, 2), (64, 130, 2, 1), (96, 5, 0, 3), (64, 333, 0, 3), (32, 16, 1, 1)])
def test_permute_writes_the_split_bit_for_bit(gpu, storage, B, K, q_begin, q_count):
    import torch
    import volumetric_delay_sum_amd as das
    Q, M = 3, 5
    rng = np.random.default_rng([B, K, q_begin])
    x = (rng.standard_normal((B, Q, M, K)) * np.exp2(rng.uniform(-12, 12, (B, Q, M, K)))).astype(np.float32)
    x[0, :, 0, :4] = [0.0, -0.0, 2.0 ** -24, 65504.0]         # zero, negative zero, smallest half, largest half
    x = np.clip(x, -60000.0, 60000.0)
    plan = das.Plan(B=B, Q=Q, M=M, K=K, nx=2, ny=2, nz=1, origin=(0, 0, 5e-3), spacing=(2e-4,) * 3, fs=20e6,
                    c=1540.0, algorithm="repack", storage=storage)
    perm = torch.empty(plan.permuted_shape(q_count), dtype=plan.permuted_dtype(), device="cuda")
    plan.permute(torch.from_numpy(x).cuda(), perm, q_begin, q_count)
    torch.cuda.synchronize()
    got = perm.cpu().numpy().view(np.uint16)
    want = _repack_layout(x, q_begin, q_count, storage).view(np.uint16)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{int((got != want).sum())} halves differ"


def _ragged(B=32, K=300, **kw):
    base = dict(name="repack", seed=53, array=(37, 2), grid=(21, 11, 3), K=K, B=B, tx="diverging",
                sources=((0.0, 0.0), (1.5e-3, -0.5e-3), (-1e-3, 1e-3)), n_scatterers=0)
    base.update(kw)
    return das_synth.custom_config("tiny", **base)


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("B", [32, 64, 96])
def test_ragged_full_compare(gpu, storage, B):
    inp = Inputs(_ragged(B=B), w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack", storage=storage), False)
    assert_parity(y, oracle_ref(inp, storage=storage), f"repack B={B} {storage}")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("t0", [3.0 / 20e6, 1.37e-6, -0.83e-6], ids=["3_periods", "plus_1.37us", "minus_0.83us"])
def test_start_time(gpu, storage, t0):
    inp = Inputs(_ragged(t0=t0, K=320), w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack", storage=storage), False)
    assert_parity(y, oracle_ref(inp, storage=storage), f"repack t0={t0} {storage}")


@pytest.mark.parametrize("f_number", [0.3, 1.0, 3.0, 0.0])
def test_f_numbers(gpu, f_number):
    inp = Inputs(_ragged(f_number=f_number, array=(37, 3)), w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack"), False)
    assert_parity(y, oracle_ref(inp), f"repack f#={f_number}")


def test_record_ends_inside_the_window(gpu):
    # deep voxels lose part of their terms off the end of a short record
    inp = Inputs(_ragged(K=140), w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack"), False)
    assert_parity(y, oracle_ref(inp), "repack short record")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("voxel", [0.15e-3, 0.6e-3, 1.5e-3], ids=["fine", "mixed", "coarse"])
def test_windows_staged_and_direct(gpu, storage, voxel):
    """Fine voxels keep every group's window in the staged rows; coarse ones
    give windows wider than a staged row, which the waves read straight from
    the permuted buffer (several 16-position blocks per receiver)."""
    cfg = _ragged(B=32, K=700, voxel=voxel, z0=3e-3, grid=(19, 10, 3), array=(19, 3),
                  sources=((0.0, 0.0), (2e-3, 1e-3)))
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack", storage=storage), False)
    assert_parity(y, oracle_ref(inp, storage=storage), f"repack voxel={voxel} {storage}")


def _max_group_window(cfg):
    """Widest sample window (positions, k over the group plus one) of any
    8 x 4 voxel group and (event, receiver) of the configuration, all voxels
    counted (no apodization)."""
    rx = das_synth.array_positions(cfg).astype(np.float64)
    tau, _ = das_synth.tx_tables(cfg)
    nx, ny, nz = cfg.grid
    widest = 0
    for iz in range(nz):
        for gy in range(0, ny, 4):
            for gx in range(0, nx, 8):
                vox = np.array([(iz * ny + y) * nx + x for y in range(gy, min(gy + 4, ny))
                                for x in range(gx, min(gx + 8, nx))])
                pos = das_synth.voxel_positions(cfg, vox)
                d = np.linalg.norm(pos[None] - rx[:, None], axis=-1) / cfg.c
                k = np.floor((tau[:, vox][:, None, :] + d[None] - cfg.t0) * cfg.fs)
                widest = max(widest, int((k.max(-1) - k.min(-1)).max()) + 2)
    return widest


@pytest.mark.parametrize("storage", ["native", "f16"])
def test_windows_wider_than_the_staged_rows(gpu, storage):
    """No apodization and 1.5 mm voxels: group windows span more positions than
    a staged row holds (72), so those groups read their sample tiles straight
    from the permuted buffer, several 16-position blocks each."""
    cfg = _ragged(B=32, K=1200, voxel=1.5e-3, z0=3e-3, grid=(19, 10, 2), array=(19, 3), f_number=0.0,
                  sources=((0.0, 0.0), (2e-3, 1e-3)))
    assert _max_group_window(cfg) > 72
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack", storage=storage), False)
    assert_parity(y, oracle_ref(inp, storage=storage), f"repack wide windows {storage}")


def test_one_event_per_call_and_accumulate(gpu):
    import torch
    inp = Inputs(_ragged(B=64), w_tx="uniform")
    ref = oracle_ref(inp)
    y = to_numpy(run_gpu(inp, "repack", q_chunk=1), False)
    assert_parity(y, ref, "repack q chunks")
    start = torch.linspace(-3.0, 3.0, inp.cfg.B * inp.cfg.N, device="cuda").reshape(inp.cfg.B, inp.cfg.N)
    out = run_gpu(inp, "repack", out=start.clone(), accumulate_into=True)
    assert_parity(out.cpu().numpy().astype(np.float64) - start.cpu().numpy(), ref, "repack accumulate")


def test_degenerate_single_voxel(gpu):
    cfg = das_synth.custom_config("tiny", name="deg", array=(1, 1), grid=(1, 1, 1), K=40, B=32, n_scatterers=0,
                                  z0=1e-3, f_number=0.0)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack"), False)
    assert_parity(y, oracle_ref(inp), "repack one voxel")


@pytest.mark.parametrize("storage", ["native", "f16"])
@pytest.mark.parametrize("B", [32, 64])
def test_tiles_outside_every_aperture(gpu, storage, B):
    """A volume much wider than the array: the outer 16 x 16 tiles see no
    receiver inside their cones (an empty receiver list, no step), the next
    ones list a few receivers, the central ones most.  Every voxel whose
    receive weights are all zero comes out exactly 0 (and exactly unchanged
    when accumulating), the rest meet the usual bar."""
    import torch
    cfg = _ragged(B=B, K=400, array=(16, 4), grid=(56, 9, 4), voxel=0.5e-3, z0=2e-3, f_number=2.0,
                  sources=((0.0, 0.0), (1e-3, 0.0)))
    inp = Inputs(cfg, w_tx="uniform")
    ref = oracle_ref(inp, storage=storage)
    y = to_numpy(run_gpu(inp, "repack", storage=storage), False)
    zero = ref == 0.0
    assert 0.5 < zero.mean() < 0.99, zero.mean()
    assert np.array_equal(y == 0.0, zero)
    assert_parity(y, ref, f"repack apertures B={B} {storage}")
    start = torch.linspace(-3.0, 3.0, cfg.B * cfg.N, device="cuda").reshape(cfg.B, cfg.N)
    out = run_gpu(inp, "repack", out=start.clone(), accumulate_into=True, storage=storage)
    got, base = to_numpy(out, False), to_numpy(start, False)
    assert np.array_equal(got[zero], base[zero])
    assert_parity(got - base, ref, f"repack apertures accumulate B={B} {storage}")


@pytest.mark.parametrize("array,f_number", [((48, 48), 1.0), ((64, 64), 0.0), ((65, 64), 1.0)],
                         ids=["2304rx", "4096rx_all", "4160rx_unlisted"])
def test_many_receivers(gpu, array, f_number):
    """2304 receivers (five rounds of the per-receiver test), 4096 without
    apodization (every receiver, one step per 8), and 4160 with apodization,
    past the 4096 entries a tile lists: then every receiver is swept, those
    outside a tile's apertures with zero weights."""
    cfg = _ragged(B=32, K=500, array=array, grid=(20, 9, 2), sources=((0.0, 0.0), (1e-3, 1e-3)),
                  f_number=f_number)
    inp = Inputs(cfg, w_tx="uniform")
    y = to_numpy(run_gpu(inp, "repack"), False)
    assert_parity(y, oracle_ref(inp), f"repack {array[0] * array[1]} receivers f#={f_number}")


def test_repack_and_batch_inner_agree(gpu):
    inp = Inputs(_ragged(B=32))
    a = to_numpy(run_gpu(inp, "repack"), False)
    b = to_numpy(run_gpu(inp, "batch_inner", "qmkb"), False)
    ref = oracle_ref(inp)
    assert_parity(a, ref, "repack")
    assert_parity(b, ref, "batch-inner")
    assert_parity(a, b, "repack vs batch-inner")


# --------------------------------------------------------------------------
# Named workloads at full size
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def main_inputs(gpu):
    return Inputs(das_synth.get_config("main"))


@pytest.mark.parametrize("storage", ["native", "f16"])
def test_main_sampled(main_inputs, storage):
    inp = main_inputs
    vox = sample_voxels(inp.cfg, 192)
    out = run_gpu(inp, "repack", storage=storage)
    assert_all_written(out, f"main repack {storage}")
    y = to_numpy(out, False)[:, vox]
    assert_parity(y, oracle_ref(inp, voxels=vox, storage=storage), f"main repack {storage}")


def test_main_noise_only(gpu):
    """The worst case for relative error: no scatterer energy to dilute it."""
    inp = Inputs(das_synth.get_config("main"), scatterers=False)
    vox = sample_voxels(inp.cfg, 128, seed=3)
    out = run_gpu(inp, "repack")
    assert_all_written(out, "main noise-only repack")
    assert_parity(to_numpy(out, False)[:, vox], oracle_ref(inp, voxels=vox), "main noise-only repack")


@pytest.mark.parametrize("storage", ["native", "f16"])
def test_large_sampled(gpu, storage):
    """Large (128 x 128 x 96 voxels, 64 frames, 16 events of 1024 x 4096 samples)
    in one chunk of all 16 events, as the benchmark runs it."""
    import torch
    import oracle
    cfg = das_synth.get_config("large")
    inp = Inputs(cfg)
    print(f"large repack {storage}", flush=True)
    out = run_gpu(inp, "repack", storage=storage)
    assert_all_written(out, f"large repack {storage}")
    frames = [0, 33, 63]
    vox = sample_voxels(cfg, 768, seed=8)
    y = to_numpy(out, cfg.iq)[frames][:, vox]
    fields = dict(inp.fields, B=len(frames))
    rf_sub = inp.rf_d[frames].cpu().numpy()
    if storage == "f16":
        rf_sub = oracle.to_binary16(rf_sub)
    del inp, out
    torch.cuda.empty_cache()
    ref = oracle.das_sum(fields, rf_sub, das_synth.array_positions(cfg), *das_synth.tx_tables(cfg), voxels=vox)
    assert_parity(y, ref, f"large repack {storage}")
