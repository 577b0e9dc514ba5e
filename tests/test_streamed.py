"""Streamed batch-inner pass (das_beamform_streamed): the permute of one chunk
of transmit events overlapped with the beamform of the previous one on a
second stream.  It must equal the plain chunked sequence bit for bit, and on
the Large workload (17 GB of RF, streamed in 3-event chunks) match the oracle
on a seeded sample of voxels and frames."""
import numpy as np
import pytest

import das_synth
from das_testing import Inputs, assert_all_written, assert_parity, run_gpu, sample_voxels, to_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def main_inputs(gpu):
    return Inputs(das_synth.get_config("main"))


def _streamed(inp, q_chunk, accumulate_into=None, same_stream=False):
    import torch
    import volumetric_delay_sum_amd as das
    plan = das.plan_from_fields(inp.fields, algorithm="batch_inner", layout="kqmb")
    dev = inp.rf_d.device
    if accumulate_into is None:
        out = torch.full(plan.output_shape(), float("nan"), dtype=torch.float32, device=dev)
    else:
        out = accumulate_into.clone()
    pa = torch.empty(plan.permuted_shape(q_chunk), dtype=torch.float32, device=dev)
    pb = torch.empty_like(pa)
    sp = torch.cuda.Stream(dev)
    sb = sp if same_stream else torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    plan.beamform_streamed(inp.rf_d, inp.rx_d, inp.tau_d, inp.w_d, out, pa, pb, q_chunk,
                           accumulate=accumulate_into is not None, stream_permute=sp, stream_beamform=sb)
    sp.synchronize()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("q_chunk", [1, 2, 4, 9])
def test_streamed_equals_chunked_sequence(main_inputs, q_chunk):
    ref = run_gpu(main_inputs, "batch_inner", "kqmb", q_chunk=q_chunk)
    got = _streamed(main_inputs, q_chunk)
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())


def test_streamed_on_one_stream_and_accumulating(main_inputs):
    import torch
    ref = run_gpu(main_inputs, "batch_inner", "kqmb", q_chunk=2)
    base = torch.full_like(ref, 0.5)
    got = _streamed(main_inputs, 2, accumulate_into=base, same_stream=True)
    # the first chunk adds onto 0.5, the rest accumulate as in the sequence
    ref2 = run_gpu(main_inputs, "batch_inner", "kqmb", q_chunk=2, out=base.clone(), accumulate_into=base)
    assert np.array_equal(got.cpu().numpy(), ref2.cpu().numpy())


def test_large_streamed_matches_oracle_on_a_sample(gpu):
    """Large: 128 x 128 x 96 voxels, 64 frames, 16 events of 1024 x 4096 samples."""
    import torch
    import oracle
    cfg = das_synth.get_config("large")
    inp = Inputs(cfg)
    import volumetric_delay_sum_amd as das
    plan = das.plan_from_fields(inp.fields, algorithm="batch_inner", layout="kqmb")
    qc = plan.max_q_chunk()
    assert qc == 3 and plan.info["staged"] == 1
    out = _streamed(inp, qc)
    assert_all_written(out, "large streamed")
    frames = [0, 31, 63]
    vox = sample_voxels(cfg, 1024, seed=5)
    y = to_numpy(out, cfg.iq)[frames][:, vox]
    fields = dict(inp.fields, B=len(frames))
    rf_sub = inp.rf_d[frames].cpu().numpy()
    del inp
    torch.cuda.empty_cache()
    ref = oracle.das_sum(fields, rf_sub, das_synth.array_positions(cfg), *das_synth.tx_tables(cfg), voxels=vox)
    assert_parity(y, ref, "large streamed")


def test_large_qmkb_one_chunk_past_4gib_matches_oracle(gpu):
    """Large in one QMKB chunk of all 16 events (17 GB): the staged kernel rebases
    its copies per (event, receiver block) plane past 4 GiB."""
    import torch
    import oracle
    cfg = das_synth.get_config("large")
    inp = Inputs(cfg)
    import volumetric_delay_sum_amd as das
    plan = das.plan_from_fields(inp.fields, algorithm="batch_inner", layout="qmkb")
    assert plan.max_q_chunk() == cfg.Q and plan.info["staged"] == 1
    assert plan.permuted_bytes(cfg.Q) > 4 * 2 ** 30
    print("large qmkb one chunk", flush=True)
    out = run_gpu(inp, "batch_inner", "qmkb", q_chunk=cfg.Q)
    assert_all_written(out, "large qmkb one chunk")
    frames = [0, 37, 63]
    vox = sample_voxels(cfg, 1024, seed=6)
    y = to_numpy(out, cfg.iq)[frames][:, vox]
    fields = dict(inp.fields, B=len(frames))
    rf_sub = inp.rf_d[frames].cpu().numpy()
    del inp, out
    torch.cuda.empty_cache()
    ref = oracle.das_sum(fields, rf_sub, das_synth.array_positions(cfg), *das_synth.tx_tables(cfg), voxels=vox)
    assert_parity(y, ref, "large qmkb one chunk")
