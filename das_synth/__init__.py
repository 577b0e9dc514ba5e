"""Seeded synthetic inputs for volumetric delay-and-sum (DAS).

This module makes the inputs that both the GPU library and the CPU oracle consume:
matrix-array receiver positions, the voxel grid, per-voxel transmit tables
(tau_tx, w_tx), and RF data of shape B x Q x M x K (frames, transmit events,
receivers, samples) made of seeded noise plus point-scatterer echoes.

It holds none of the beamformer's arithmetic: no receive delay, no apodization,
no interpolation and no accumulation.  What it does compute is the forward model
of the acquisition (when an echo from a scatterer reaches a receiver, and the
transmit delay table, which the method takes as a precomputed per-voxel input;
"ffdas: volumetric ultrasound reconstruction at warp speed", Section 3, the
paragraph on the baseline kernel).

Workloads follow the five named configurations (Tiny, Mid, Main, Main-c64,
Large).  The pages give no worked dataset, so these synthetic volumes are the
workload.  Noise for frame b comes from a Philox generator seeded with
(seed, b) on the device that holds the RF, so each frame can be regenerated on
its own; scatterer positions come from numpy's generator seeded [seed, 10**6].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "custom_config", "array_positions",
    "voxel_grid", "voxel_positions", "tx_tables", "scatterer_voxels",
    "echo_plane", "rf", "problem_fields", "accumulations",
]

SPEED_OF_SOUND = 1540.0      # m/s
ECHO_SIGMA = 0.1e-6          # s, Gaussian envelope of each echo
ECHO_AMPLITUDE = 10.0        # relative to unit-variance noise
ECHO_F0 = 5.0e6              # Hz, centre frequency of the echoes


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    array: tuple[int, int]          # elements along x, y (M = Mx * My)
    pitch: float                    # m
    tx: str                         # "plane" or "diverging"
    sources: tuple[tuple[float, float], ...]   # virtual-source (x, y) in m, z = -src_depth
    K: int
    fs: float
    B: int
    grid: tuple[int, int, int]      # nx, ny, nz
    voxel: float                    # voxel pitch, m
    z0: float                       # depth of the first voxel plane, m
    n_scatterers: int
    iq: bool = False                # complex64 IQ data demodulated at f0
    f0: float = ECHO_F0
    src_depth: float = 10e-3
    c: float = SPEED_OF_SOUND
    t0: float = 0.0
    f_number: float = 1.0

    @property
    def M(self) -> int:
        return self.array[0] * self.array[1]

    @property
    def Q(self) -> int:
        return len(self.sources)

    @property
    def N(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]


def _grid_sources(vals_mm: Sequence[float]) -> tuple[tuple[float, float], ...]:
    return tuple((x * 1e-3, y * 1e-3) for y in vals_mm for x in vals_mm)


CONFIGS = {
    "tiny": Config("tiny", 1, (8, 8), 0.3e-3, "plane", ((0.0, 0.0),), 512, 20e6, 8,
                   (16, 16, 16), 0.2e-3, 5e-3, 3),
    "mid": Config("mid", 2, (16, 16), 0.3e-3, "diverging",
                  ((0.0, 0.0), (2e-3, 0.0), (-2e-3, 0.0), (0.0, 2e-3), (0.0, -2e-3)),
                  1024, 20e6, 16, (64, 64, 64), 0.2e-3, 5e-3, 20),
    "main": Config("main", 3, (32, 32), 0.3e-3, "diverging", _grid_sources((-2, 0, 2)),
                   2048, 20e6, 32, (64, 64, 64), 0.25e-3, 5e-3, 50),
    "main-c64": Config("main-c64", 4, (32, 32), 0.3e-3, "diverging", _grid_sources((-2, 0, 2)),
                       2048, 20e6, 32, (64, 64, 64), 0.25e-3, 5e-3, 50, iq=True),
    "large": Config("large", 5, (32, 32), 0.3e-3, "diverging", _grid_sources((-3, -1, 1, 3)),
                    4096, 25e6, 64, (128, 128, 96), 0.2e-3, 5e-3, 100),
}


def get_config(name: str) -> Config:
    return CONFIGS[name.lower()]


def custom_config(base: str = "tiny", **changes) -> Config:
    """A named configuration with some fields replaced (small ragged test shapes)."""
    return dataclasses.replace(get_config(base), **changes)


def accumulations(cfg: Config) -> int:
    """Nominal voxel x receiver x transmit x frame count of one full call."""
    return cfg.N * cfg.M * cfg.Q * cfg.B


def array_positions(cfg: Config) -> np.ndarray:
    """Mx x My elements centred on the origin at z = 0, m = j*Mx + i (x fastest)."""
    mx, my = cfg.array
    xs = (np.arange(mx) - (mx - 1) / 2.0) * cfg.pitch
    ys = (np.arange(my) - (my - 1) / 2.0) * cfg.pitch
    pos = np.zeros((my, mx, 3), dtype=np.float64)
    pos[:, :, 0] = xs[None, :]
    pos[:, :, 1] = ys[:, None]
    return pos.reshape(-1, 3).astype(np.float32)


def voxel_grid(cfg: Config) -> tuple[tuple[float, float, float], tuple[float, float, float], tuple[int, int, int]]:
    """(origin, spacing, (nx, ny, nz)); laterally centred on x = y = 0, first plane at z0."""
    nx, ny, nz = cfg.grid
    d = cfg.voxel
    origin = (-(nx - 1) / 2.0 * d, -(ny - 1) / 2.0 * d, cfg.z0)
    return origin, (d, d, d), (nx, ny, nz)


def voxel_positions(cfg: Config, idx: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 voxel centres for linear indices n = (iz*ny + iy)*nx + ix."""
    origin, spacing, (nx, ny, nz) = voxel_grid(cfg)
    if idx is None:
        idx = np.arange(nx * ny * nz, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    ix = idx % nx
    iy = (idx // nx) % ny
    iz = idx // (nx * ny)
    return np.stack([origin[0] + ix * spacing[0], origin[1] + iy * spacing[1],
                     origin[2] + iz * spacing[2]], axis=-1)


def _tx_delay(cfg: Config, pos: np.ndarray, q: int) -> np.ndarray:
    """Transmit delay of event q at positions pos (fp64, seconds).

    Plane wave at 0 degrees: z / c.  Diverging wave from a virtual source at
    (vx, vy, -src_depth): (|r - v| - src_depth) / c, i.e. time zero when the
    wavefront crosses z = 0 right under the source.
    """
    if cfg.tx == "plane":
        return pos[..., 2] / cfg.c
    vx, vy = cfg.sources[q]
    v = np.array([vx, vy, -cfg.src_depth])
    return (np.linalg.norm(pos - v, axis=-1) - cfg.src_depth) / cfg.c


def tx_tables(cfg: Config, w_tx: str = "ones", seed: Optional[int] = None) -> tuple[np.ndarray, np.ndarray]:
    """Per-voxel transmit delay and weight tables, each Q x N float32.

    w_tx = "ones" (the named configs) or "uniform" (seeded U[0,1], to exercise
    the weight table in tests).
    """
    pos = voxel_positions(cfg)
    tau = np.empty((cfg.Q, cfg.N), dtype=np.float32)
    for q in range(cfg.Q):
        tau[q] = _tx_delay(cfg, pos, q).astype(np.float32)
    if w_tx == "ones":
        w = np.ones((cfg.Q, cfg.N), dtype=np.float32)
    elif w_tx == "uniform":
        rng = np.random.default_rng([cfg.seed if seed is None else seed, 7])
        w = rng.random((cfg.Q, cfg.N)).astype(np.float32)
    else:
        raise ValueError(f"unknown w_tx mode {w_tx!r}")
    return tau, w


def scatterer_voxels(cfg: Config) -> np.ndarray:
    """Distinct voxel indices at least 3 voxels from every face (sorted)."""
    nx, ny, nz = cfg.grid
    rng = np.random.default_rng([cfg.seed, 10 ** 6])
    if min(nx, ny, nz) < 7 or cfg.n_scatterers == 0:
        return np.zeros(0, dtype=np.int64)
    chosen: set[int] = set()
    while len(chosen) < cfg.n_scatterers:
        ix = int(rng.integers(3, nx - 3))
        iy = int(rng.integers(3, ny - 3))
        iz = int(rng.integers(3, nz - 3))
        chosen.add((iz * ny + iy) * nx + ix)
    return np.array(sorted(chosen), dtype=np.int64)


def echo_plane(cfg: Config) -> np.ndarray:
    """Noise-free echoes of all scatterers, Q x M x K (float32, or complex64 for IQ).

    An echo arriving at time ts has the Gaussian-windowed form
    A exp(-(t-ts)^2 / (2 sigma^2)) cos(2 pi f0 (t-ts)); as demodulated IQ it is
    A exp(-(t-ts)^2 / (2 sigma^2)) exp(-j 2 pi f0 ts).  The echoes are static
    across frames.
    """
    dtype = np.complex64 if cfg.iq else np.float32
    plane = np.zeros((cfg.Q, cfg.M, cfg.K), dtype=np.complex128 if cfg.iq else np.float64)
    sv = scatterer_voxels(cfg)
    if sv.size == 0:
        return plane.astype(dtype)
    rx = array_positions(cfg).astype(np.float64)
    spos = voxel_positions(cfg, sv)                       # S x 3
    half = int(math.ceil(6 * ECHO_SIGMA * cfg.fs)) + 1
    offs = np.arange(-half, half + 1)
    t_rx = np.linalg.norm(spos[:, None, :] - rx[None, :, :], axis=-1) / cfg.c   # S x M
    for q in range(cfg.Q):
        ts = _tx_delay(cfg, spos, q)[:, None] + t_rx                          # S x M
        centre = np.floor((ts - cfg.t0) * cfg.fs).astype(np.int64)           # S x M
        k = centre[..., None] + offs                                           # S x M x W
        t = cfg.t0 + k / cfg.fs
        dt = t - ts[..., None]
        env = ECHO_AMPLITUDE * np.exp(-dt * dt / (2 * ECHO_SIGMA ** 2))
        if cfg.iq:
            val = env * np.exp(-2j * np.pi * cfg.f0 * ts[..., None])
        else:
            val = env * np.cos(2 * np.pi * cfg.f0 * dt)
        ok = (k >= 0) & (k < cfg.K)
        m_idx = np.broadcast_to(np.arange(cfg.M)[None, :, None], k.shape)
        np.add.at(plane[q], (m_idx[ok], k[ok]), val[ok])
    return plane.astype(dtype)


def _frame_noise(cfg: Config, b: int, device, torch):
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1_000_003 + b)
    shape = (cfg.Q, cfg.M, cfg.K, 2) if cfg.iq else (cfg.Q, cfg.M, cfg.K)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def rf(cfg: Config, device="cpu", frames: Optional[Sequence[int]] = None,
       scatterers: bool = True, noise: bool = True):
    """RF data as a torch float32 tensor.

    Shape (len(frames), Q, M, K) for real data, (len(frames), Q, M, K, 2) for IQ
    (re/im interleaved, i.e. complex64 storage).  Frames default to all B.
    """
    import torch

    frames = list(range(cfg.B)) if frames is None else list(frames)
    shape = (len(frames), cfg.Q, cfg.M, cfg.K) + ((2,) if cfg.iq else ())
    out = torch.zeros(shape, dtype=torch.float32, device=device)
    echo = None
    if scatterers:
        e = echo_plane(cfg)
        if cfg.iq:
            e = np.stack([e.real, e.imag], axis=-1).astype(np.float32)
        echo = torch.from_numpy(np.ascontiguousarray(e)).to(device)
    for i, b in enumerate(frames):
        if noise:
            out[i] = _frame_noise(cfg, b, device, torch)
        if echo is not None:
            out[i] += echo
    return out


def problem_fields(cfg: Config) -> dict:
    """Scalar description of the problem (grid, rates, sizes) as plain numbers."""
    origin, spacing, (nx, ny, nz) = voxel_grid(cfg)
    return dict(B=cfg.B, Q=cfg.Q, M=cfg.M, K=cfg.K, nx=nx, ny=ny, nz=nz,
                origin=origin, spacing=spacing, fs=cfg.fs, c=cfg.c, t0=cfg.t0,
                f_number=cfg.f_number, f_demod=(cfg.f0 if cfg.iq else 0.0),
                iq=cfg.iq)
