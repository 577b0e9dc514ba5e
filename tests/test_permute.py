"""GPU permute: bit-exact against the oracle's numpy transposes
(B x Q x M x K -> K x Q x M x B or Q x M x K x B), including q-range chunks,
IQ data and ragged shapes: both the register transpose (fp32, B a multiple of
16, K of 4; tails of the sample tile) and the LDS one (everything else)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _plan(B, Q, M, K, iq, layout):
    import volumetric_delay_sum_amd as das
    return das.Plan(B=B, Q=Q, M=M, K=K, nx=2, ny=2, nz=2, origin=(0, 0, 1e-3), spacing=(1e-4,) * 3, fs=20e6,
                    c=1540.0, f_demod=(5e6 if iq else 0.0), dtype=("c64" if iq else "f32"),
                    algorithm="batch_inner", layout=layout)


@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
@pytest.mark.parametrize("iq", [False, True], ids=["f32", "c64"])
@pytest.mark.parametrize("shape", [(8, 1, 64, 512), (12, 3, 37, 301), (33, 2, 5, 70), (1, 1, 1, 2), (64, 2, 16, 128),
                                   (32, 2, 7, 100), (16, 3, 5, 36), (48, 1, 3, 4), (32, 1, 3, 70)])
def test_permute_bit_exact(gpu, layout, iq, shape):
    import torch
    import oracle
    B, Q, M, K = shape
    plan = _plan(B, Q, M, K, iq, layout)
    g = torch.Generator(device="cuda").manual_seed(B * 1000 + K)
    x = torch.randn(shape + ((2,) if iq else ()), generator=g, device="cuda")
    out = torch.full(plan.permuted_shape(), float("nan"), device="cuda")
    plan.permute(x, out)
    torch.cuda.synchronize()
    ref = (oracle.permute_kqmb if layout == "kqmb" else oracle.permute_qmkb)(x.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("layout", ["kqmb", "qmkb"])
def test_permute_q_ranges(gpu, layout):
    import torch
    import oracle
    B, Q, M, K = 16, 5, 20, 200
    plan = _plan(B, Q, M, K, False, layout)
    x = torch.randn((B, Q, M, K), device="cuda")
    full = (oracle.permute_kqmb if layout == "kqmb" else oracle.permute_qmkb)
    for q0, qc in [(0, 1), (2, 2), (4, 1), (1, 4)]:
        out = torch.full(plan.permuted_shape(qc), float("nan"), device="cuda")
        plan.permute(x, out, q0, qc)
        torch.cuda.synchronize()
        ref = full(x[:, q0:q0 + qc].cpu().numpy())
        assert np.array_equal(out.cpu().numpy(), ref), (q0, qc)


def test_permute_main_size(gpu):
    """Main-sized input (32 x 9 x 1024 x 2048 fp32): checked on a seeded sample of rows."""
    import torch
    B, Q, M, K = 32, 9, 1024, 2048
    plan = _plan(B, Q, M, K, False, "kqmb")
    x = torch.randn((B, Q, M, K), device="cuda")
    out = torch.empty(plan.permuted_shape(), device="cuda")
    plan.permute(x, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for _ in range(64):
        q, m, k = int(rng.integers(Q)), int(rng.integers(M)), int(rng.integers(K))
        assert torch.equal(out[k, q, m, :], x[:, q, m, k])
