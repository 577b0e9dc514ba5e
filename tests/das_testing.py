"""Shared helpers of the GPU tests: run the HIP path through the C ABI, run the
oracle on the same seeded inputs, and compare to the stated tolerance."""
from __future__ import annotations

import numpy as np

import das_synth

# Parity bar for floating point: max|err| <= 1e-4 max|oracle| and relative
# L2 <= 1e-5, complex data compared per component.
MAX_REL = 1e-4
L2_REL = 1e-5


def parity_errors(y, ref):
    """[(max_err / max|ref|, ||err|| / ||ref||)] per component."""
    y = np.asarray(y)
    ref = np.asarray(ref)
    comps = [(y.real, ref.real), (y.imag, ref.imag)] if np.iscomplexobj(ref) else [(y, ref)]
    out = []
    for g, r in comps:
        g = g.astype(np.float64)
        err = g - r
        out.append((float(np.abs(err).max() / np.abs(r).max()),
                    float(np.linalg.norm(err) / np.linalg.norm(r))))
    return out


def assert_parity(y, ref, what=""):
    assert np.all(np.isfinite(np.asarray(y).real)) and np.all(np.isfinite(np.asarray(y).imag)), \
        f"{what}: non-finite output (unwritten element?)"
    for i, (mx, l2) in enumerate(parity_errors(y, ref)):
        assert mx <= MAX_REL and l2 <= L2_REL, f"{what} component {i}: max {mx:.3e}, L2 {l2:.3e}"


def assert_all_written(out, what=""):
    """Every element of a NaN-filled device output was written (and is finite):
    the whole volume, not only the voxels a sampled comparison looks at."""
    import torch
    bad = int((~torch.isfinite(out)).sum().item())
    assert bad == 0, f"{what}: {bad} of {out.numel()} output values unwritten or non-finite"


class Inputs:
    """Seeded inputs of one configuration, on the GPU and as host copies."""

    def __init__(self, cfg: das_synth.Config, w_tx: str = "ones", scatterers: bool = True,
                 noise: bool = True, device: str = "cuda"):
        import torch
        self.cfg = cfg
        self.fields = das_synth.problem_fields(cfg)
        self.rx = das_synth.array_positions(cfg)
        self.tau, self.w = das_synth.tx_tables(cfg, w_tx=w_tx)
        self.rf_d = das_synth.rf(cfg, device=device, scatterers=scatterers, noise=noise)
        self.rx_d = torch.from_numpy(self.rx).to(device)
        self.tau_d = torch.from_numpy(self.tau).to(device)
        self.w_d = torch.from_numpy(self.w).to(device)
        self._rf_host = None

    @property
    def rf_host(self) -> np.ndarray:
        if self._rf_host is None:
            self._rf_host = self.rf_d.cpu().numpy()
        return self._rf_host


def run_gpu(inp: Inputs, algorithm: str, layout: str = "kqmb", q_chunk: int | None = None,
            out=None, accumulate_into=None, storage: str = "native"):
    """Beamform all events through the C ABI; returns the device output tensor.

    Batch-inner runs permute + beamform per chunk of q_chunk events (all Q at
    once by default), accumulating chunks after the first.  storage "f16":
    binary16 samples in the permuted buffer.
    """
    import torch
    import volumetric_delay_sum_amd as das

    plan = das.plan_from_fields(inp.fields, algorithm=algorithm, layout=layout, storage=storage)
    if out is None:
        out = torch.full(plan.output_shape(), float("nan"), dtype=torch.float32, device=inp.rf_d.device)
    Q = inp.cfg.Q
    first_acc = accumulate_into is not None
    if plan.permuted_input:
        qc = min(Q if q_chunk is None else q_chunk, plan.max_q_chunk())
        assert qc >= 1
        perm = torch.empty(plan.permuted_shape(qc), dtype=plan.permuted_dtype(), device=inp.rf_d.device)
        for q0 in range(0, Q, qc):
            n = min(qc, Q - q0)
            view = perm.view(-1)[: perm.numel() // qc * n]
            plan.permute(inp.rf_d, view, q0, n)
            plan.beamform(view, inp.rx_d, inp.tau_d, inp.w_d, out, q0, n, accumulate=(q0 > 0 or first_acc))
    else:
        qc = Q if q_chunk is None else q_chunk
        for q0 in range(0, Q, qc):
            n = min(qc, Q - q0)
            plan.beamform(inp.rf_d, inp.rx_d, inp.tau_d, inp.w_d, out, q0, n, accumulate=(q0 > 0 or first_acc))
    torch.cuda.synchronize()
    return out


def to_numpy(out, iq: bool) -> np.ndarray:
    y = out.cpu().numpy().astype(np.float64)
    return y[..., 0] + 1j * y[..., 1] if iq else y


def oracle_ref(inp: Inputs, voxels=None, frames=None, storage: str = "native"):
    """The oracle on the same inputs; storage "f16": of the samples rounded to binary16."""
    import oracle
    rf = oracle.to_binary16(inp.rf_host) if storage == "f16" else inp.rf_host
    return oracle.das_sum(inp.fields, rf, inp.rx, inp.tau, inp.w, voxels=voxels, frames=frames)


def sample_voxels(cfg: das_synth.Config, count: int, seed: int = 0) -> np.ndarray:
    """Seeded voxel sample: every scatterer voxel, the grid corners, then random voxels."""
    nx, ny, nz = cfg.grid
    corners = [((iz * ny + iy) * nx + ix) for iz in (0, nz - 1) for iy in (0, ny - 1) for ix in (0, nx - 1)]
    base = list(das_synth.scatterer_voxels(cfg)) + corners
    rng = np.random.default_rng([seed, 99])
    extra = rng.choice(cfg.N, size=max(0, count - len(base)), replace=False)
    vox = np.unique(np.concatenate([np.array(base, dtype=np.int64), extra.astype(np.int64)]))
    return vox
