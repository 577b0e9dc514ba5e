"""fp64 CPU oracle for volumetric delay-and-sum (DAS).

TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check and the
benchmark's CPU-baseline leg are the only users; the GPU library never imports,
links or runs anything here, and this package imports nothing from it.

``das_sum`` wraps the plain C implementation in ``das_oracle.c`` (single
threaded, fp64, compiled -O2 without fast-math).  The permute references are
numpy transposes: the permute is a pure relayout, so the library primitive is
its definition ("ffdas: volumetric ultrasound reconstruction at warp speed",
Section 3, batch-inner tiling: B x Q x M x K becomes K x Q x M x B; ffdas docs,
"How It Works", ALG2: the batch index moves to the innermost position).
``to_binary16`` is the rounding of the binary16 storage variant (numpy's
float16 conversion, pinned against hand-derived bit patterns);
``split_binary16`` writes a float32 sample as a sum of two such halves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "das_oracle.c")
_LIB = os.path.join(_HERE, "libdas_oracle.so")
_lib = None


class _Geometry(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Q", ctypes.c_int32), ("M", ctypes.c_int32), ("K", ctypes.c_int32),
        ("nx", ctypes.c_int32), ("ny", ctypes.c_int32), ("nz", ctypes.c_int32),
        ("complex_iq", ctypes.c_int32), ("rf_f64", ctypes.c_int32),
        ("origin", ctypes.c_double * 3), ("spacing", ctypes.c_double * 3),
        ("fs", ctypes.c_double), ("c", ctypes.c_double), ("t0", ctypes.c_double),
        ("f_number", ctypes.c_double), ("f_demod", ctypes.c_double),
    ]


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/libdas_oracle.so`` with gcc -O2."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.das_oracle_sum.restype = ctypes.c_int
        lib.das_oracle_sum.argtypes = [
            ctypes.POINTER(_Geometry), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p]
        lib.das_oracle_rx_weight.restype = ctypes.c_double
        lib.das_oracle_rx_weight.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
        _lib = lib
    return _lib


def _as_f32(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"{name} must be float32, got {a.dtype}")
    return a


def das_sum(fields: dict, rf, rx_pos, tau_tx, w_tx,
            voxels: Optional[Sequence[int]] = None,
            frames: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 DAS of the given voxels and frames.

    fields: B, Q, M, K, nx, ny, nz, origin, spacing, fs, c, t0, f_number,
            f_demod, iq (as made by ``das_synth.problem_fields``).
    rf: float32 or float64 B x Q x M x K (IQ: B x Q x M x K x 2).  The frame axis of rf
        must hold all B frames (frame indices address it directly).
    Returns float64 (n_frames, n_voxels), or complex128 for IQ.
    """
    lib = _load()
    g = _Geometry()
    for key in ("B", "Q", "M", "K", "nx", "ny", "nz"):
        setattr(g, key, int(fields[key]))
    g.complex_iq = 1 if fields.get("iq") else 0
    g.origin[:] = [float(v) for v in fields["origin"]]
    g.spacing[:] = [float(v) for v in fields["spacing"]]
    g.fs, g.c, g.t0 = float(fields["fs"]), float(fields["c"]), float(fields["t0"])
    g.f_number, g.f_demod = float(fields["f_number"]), float(fields.get("f_demod", 0.0))

    rf = np.ascontiguousarray(rf)
    if rf.dtype not in (np.float32, np.float64):
        raise TypeError(f"rf must be float32 or float64, got {rf.dtype}")
    g.rf_f64 = 1 if rf.dtype == np.float64 else 0
    rx_pos = _as_f32(rx_pos, "rx_pos")
    tau_tx = _as_f32(tau_tx, "tau_tx")
    w_tx = _as_f32(w_tx, "w_tx")
    n_total = g.nx * g.ny * g.nz
    expect_rf = g.B * g.Q * g.M * g.K * (2 if g.complex_iq else 1)
    if rf.size != expect_rf:
        raise ValueError(f"rf has {rf.size} values, expected {expect_rf}")
    if rx_pos.size != 3 * g.M or tau_tx.size != g.Q * n_total or w_tx.size != g.Q * n_total:
        raise ValueError("rx_pos / tau_tx / w_tx sizes do not match the problem")
    vox = np.arange(n_total, dtype=np.int64) if voxels is None else np.ascontiguousarray(voxels, dtype=np.int64)
    frm = np.arange(g.B, dtype=np.int32) if frames is None else np.ascontiguousarray(frames, dtype=np.int32)
    comps = 2 if g.complex_iq else 1
    out = np.zeros((frm.size, vox.size, comps), dtype=np.float64)
    rc = lib.das_oracle_sum(ctypes.byref(g), rf.ctypes.data, rx_pos.ctypes.data, tau_tx.ctypes.data,
                            w_tx.ctypes.data, vox.ctypes.data, vox.size, frm.ctypes.data, frm.size,
                            out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    if g.complex_iq:
        return out[..., 0] + 1j * out[..., 1]
    return out[..., 0]


def rx_weight(rho: float, dz: float, f_number: float) -> float:
    """The oracle's receive apodization for one (rho, dz) offset."""
    return _load().das_oracle_rx_weight(float(rho), float(dz), float(f_number))


def permute_kqmb(x: np.ndarray) -> np.ndarray:
    """B x Q x M x K (x 2 for IQ) -> K x Q x M x B (x 2): y[k,q,m,b] = x[b,q,m,k]."""
    axes = (3, 1, 2, 0) + ((4,) if x.ndim == 5 else ())
    return np.ascontiguousarray(np.transpose(x, axes))


def permute_qmkb(x: np.ndarray) -> np.ndarray:
    """B x Q x M x K (x 2 for IQ) -> Q x M x K x B (x 2): batch moved innermost."""
    axes = (1, 2, 3, 0) + ((4,) if x.ndim == 5 else ())
    return np.ascontiguousarray(np.transpose(x, axes))


def to_binary16(x: np.ndarray) -> np.ndarray:
    """Samples as they are held with binary16 storage, widened back to float32.

    "ffdas: volumetric ultrasound reconstruction at warp speed", Section 3, FP16
    variant: the samples are kept in half precision and converted to fp32
    before the interpolation; ffdas docs, mixed-precision API: half for real
    data, half2 (a pair of halves) for complex data.  Each float32 value is
    rounded to the nearest IEEE binary16 value, ties to even, with subnormal
    halves kept, overflow to infinity and NaN kept NaN (numpy's float16
    conversion); the widening back is exact.  Complex data (a trailing re/im
    axis) is rounded per component.  The beamform of binary16 storage is then
    ``das_sum`` of these samples.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError(f"binary16 storage rounds float32 samples, got {x.dtype}")
    with np.errstate(over="ignore"):
        return x.astype(np.float16).astype(np.float32)


def split_binary16(x: np.ndarray) -> tuple:
    """A float32 sample as the sum of two binary16 values, hi + lo.

    The matrix-core (repack) variant multiplies binary16 operands ("ffdas:
    volumetric ultrasound reconstruction at warp speed", Section 3,
    tensor-core paragraphs: the products run on mixed-precision matrix
    units), so float32 samples are held as a pair: hi is the sample rounded
    to the nearest binary16 value (ties to even, ``to_binary16``), lo the
    remainder x - hi (exact in float32) rounded the same way.  For samples in
    the binary16 normal range, x - hi - lo is at most 2^-22 |x|.  Returns the
    two arrays as float32 values.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError(f"the split takes float32 samples, got {x.dtype}")
    hi = to_binary16(x)
    with np.errstate(invalid="ignore"):
        rest = (x.astype(np.float64) - hi.astype(np.float64)).astype(np.float32)
    return hi, to_binary16(rest)


# Transmit-event kinds (the values of the library's enum, restated).
TX_PLANE, TX_DIVERGING = 0, 1


def tx_tables(fields: dict, events) -> tuple:
    """Per-voxel transmit delays and weights of plane and diverging events.

    "ffdas: volumetric ultrasound reconstruction at warp speed", Section 3,
    baseline paragraph: the transmit delays and weights are tables computed
    ahead per voxel.  A plane event with unit propagation direction u reaches
    voxel centre r at (u . r) / c (time zero as the front crosses the origin);
    a diverging event from a virtual source v (v_z < 0) at (|r - v| - |v_z|) / c
    (time zero as the front crosses z = 0 under the source).  The weight is the
    event's constant.  Plain fp64 numpy, every operation rounded on its own in
    the order written, then one rounding to float32.

    fields: nx, ny, nz, origin, spacing, c.  events: (kind, (vx, vy, vz), weight).
    Returns (tau, w), each len(events) x N float32.
    """
    nx, ny, nz = int(fields["nx"]), int(fields["ny"]), int(fields["nz"])
    origin = [float(v) for v in fields["origin"]]
    spacing = [float(v) for v in fields["spacing"]]
    c = float(fields["c"])
    n = np.arange(nx * ny * nz, dtype=np.int64)
    ix, iy, iz = n % nx, (n // nx) % ny, n // (nx * ny)
    x = origin[0] + ix.astype(np.float64) * spacing[0]
    y = origin[1] + iy.astype(np.float64) * spacing[1]
    z = origin[2] + iz.astype(np.float64) * spacing[2]
    tau = np.empty((len(events), n.size), dtype=np.float32)
    w = np.empty((len(events), n.size), dtype=np.float32)
    for e, (kind, v, weight) in enumerate(events):
        vx, vy, vz = (float(a) for a in v)
        if kind == TX_PLANE:
            t = (vx * x + vy * y + vz * z) / c
        elif kind == TX_DIVERGING:
            dx, dy, dz = x - vx, y - vy, z - vz
            t = (np.sqrt(dx * dx + dy * dy + dz * dz) - abs(vz)) / c
        else:
            raise ValueError(f"unknown transmit kind {kind}")
        tau[e] = t.astype(np.float32)
        w[e] = np.float32(weight)
    return tau, w

