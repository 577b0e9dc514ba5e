"""Volumetric delay-and-sum (DAS) beamforming on AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libdas.so`` (declared in ``include/das.h``).  It
only marshals arguments: every step of the beamformer runs in the library's
HIP kernels.  Tensors are PyTorch device tensors; the library enqueues work on
the current PyTorch stream unless a stream is given, and returns without
synchronizing.

The operation ("ffdas: volumetric ultrasound reconstruction at warp speed",
Section 3; ffdas docs "How It Works"): for each voxel n and frame b, sum over
transmit events q and receivers m of w_tx[q,n] * w_rx[m,n] times the RF sample
linearly interpolated at the delay tau_tx[q,n] + |r_n - p_m| / c.

``Plan(..., storage="f16")`` keeps the permuted samples in binary16 (the
paper's FP16 variant; the docs' ``half`` / ``half2``): permuted buffers are then
torch.float16 tensors, rounded by ``permute`` and widened to fp32 by
``beamform``.

``Plan(..., algorithm="repack")`` runs the matrix-core variant (the paper's
tensor-core repackaging; the docs' ALG4).  Its permuted buffer is a
torch.float16 tensor of shape (q, M, 2, P, B, 8): the hi and lo halves of the
float32 samples in pieces of 8 positions, P = ceil(K / 8), each piece the B
frames side by side; (q, M, P, B, 8) with ``storage="f16"``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "F32", "C64", "F64", "C128", "ALG_DEFAULT", "ALG_BASELINE", "ALG_BATCH_INNER", "ALG_AUTO", "ALG_REPACK",
    "LAYOUT_KQMB", "LAYOUT_QMKB", "LAYOUT_QMPB", "STORE_NATIVE", "STORE_F16",
    "TX_PLANE", "TX_DIVERGING", "DasError", "Plan", "load_library", "library_path", "plan_from_fields",
]

F32, C64, F64, C128 = 0, 1, 2, 3
ALG_DEFAULT, ALG_BASELINE, ALG_BATCH_INNER, ALG_AUTO, ALG_REPACK = 0, 1, 2, 3, 4
LAYOUT_KQMB, LAYOUT_QMKB, LAYOUT_QMPB = 0, 1, 2
STORE_NATIVE, STORE_F16 = 0, 1
TX_PLANE, TX_DIVERGING = 0, 1

_ALG = {"default": ALG_DEFAULT, "baseline": ALG_BASELINE, "batch_inner": ALG_BATCH_INNER,
        "bl": ALG_BASELINE, "bi": ALG_BATCH_INNER, "auto": ALG_AUTO, "repack": ALG_REPACK, "tc": ALG_REPACK}
_LAYOUT = {"kqmb": LAYOUT_KQMB, "qmkb": LAYOUT_QMKB, "qmpb": LAYOUT_QMPB}
_DTYPE = {"f32": F32, "c64": C64, "f64": F64, "c128": C128}
_STORAGE = {"native": STORE_NATIVE, "f16": STORE_F16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdas.so")
_lib = None


class DasError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {_error_string(code)} (status {code})")


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Q", ctypes.c_int32), ("M", ctypes.c_int32), ("K", ctypes.c_int32),
        ("nx", ctypes.c_int32), ("ny", ctypes.c_int32), ("nz", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("algorithm", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("storage", ctypes.c_int32),
        ("origin", ctypes.c_double * 3), ("spacing", ctypes.c_double * 3),
        ("fs", ctypes.c_double), ("c", ctypes.c_double), ("t0", ctypes.c_double),
        ("f_number", ctypes.c_double), ("f_demod", ctypes.c_double),
    ]


class _PlanInfo(ctypes.Structure):
    _fields_ = [
        ("algorithm", ctypes.c_int32), ("layout", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
        ("frames_per_lane", ctypes.c_int32), ("lanes_per_voxel", ctypes.c_int32),
        ("voxels_per_group", ctypes.c_int32), ("N", ctypes.c_int64), ("staged", ctypes.c_int32),
        ("store_bytes", ctypes.c_int32), ("whole_rows", ctypes.c_int32), ("receivers_per_step", ctypes.c_int32),
    ]


class _TxEvent(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32), ("v", ctypes.c_double * 3),
                ("weight", ctypes.c_double)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdas.so; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libdas.so is not built at {_LIB_PATH}; run "
                          "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.das_plan.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(vp)]
    lib.das_plan.restype = ctypes.c_int
    lib.das_plan_destroy.argtypes = [vp]
    lib.das_plan_destroy.restype = None
    lib.das_plan_get_info.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    lib.das_plan_get_info.restype = ctypes.c_int
    lib.das_permuted_bytes.argtypes = [vp, i32]
    lib.das_permuted_bytes.restype = ctypes.c_size_t
    lib.das_permute.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.das_permute.restype = ctypes.c_int
    lib.das_beamform.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.das_beamform.restype = ctypes.c_int
    lib.das_beamform_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.das_beamform_noalloc.restype = ctypes.c_int
    lib.das_beamform_streamed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp]
    lib.das_beamform_streamed.restype = ctypes.c_int
    lib.das_tx_tables.argtypes = [vp, ctypes.POINTER(_TxEvent), i32, i32, vp, vp, vp]
    lib.das_tx_tables.restype = ctypes.c_int
    lib.das_max_q_chunk.argtypes = [vp]
    lib.das_max_q_chunk.restype = i32
    lib.das_error_string.argtypes = [ctypes.c_int]
    lib.das_error_string.restype = ctypes.c_char_p
    lib.das_abi_version.argtypes = []
    lib.das_abi_version.restype = i32
    _lib = lib
    return lib


def _error_string(code: int) -> str:
    return load_library().das_error_string(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise DasError(code, what)


def _stream_handle(stream, device) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """A validated problem.  Holds no device memory."""

    def __init__(self, *, B: int, Q: int, M: int, K: int, nx: int, ny: int, nz: int,
                 origin: Sequence[float], spacing: Sequence[float], fs: float, c: float,
                 t0: float = 0.0, f_number: float = 1.0, f_demod: float = 0.0,
                 dtype: str = "f32", algorithm: str = "batch_inner", layout: str = "kqmb",
                 storage: str = "native"):
        lib = load_library()
        p = _Problem()
        p.B, p.Q, p.M, p.K = int(B), int(Q), int(M), int(K)
        p.nx, p.ny, p.nz = int(nx), int(ny), int(nz)
        p.dtype = _DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
        p.algorithm = _ALG[algorithm] if isinstance(algorithm, str) else int(algorithm)
        p.layout = _LAYOUT[layout] if isinstance(layout, str) else int(layout)
        p.storage = _STORAGE[storage] if isinstance(storage, str) else int(storage)
        p.origin[:] = [float(v) for v in origin]
        p.spacing[:] = [float(v) for v in spacing]
        p.fs, p.c, p.t0 = float(fs), float(c), float(t0)
        p.f_number, p.f_demod = float(f_number), float(f_demod)
        h = ctypes.c_void_p()
        _check(lib.das_plan(ctypes.byref(p), ctypes.byref(h)), "das_plan")
        self._lib = lib
        self._h = h
        self.problem = p
        info = _PlanInfo()
        _check(lib.das_plan_get_info(h, ctypes.byref(info)), "das_plan_get_info")
        self.info = {f: getattr(info, f) for f, _ in _PlanInfo._fields_}

    # -- sizes --------------------------------------------------------------
    @property
    def N(self) -> int:
        return self.problem.nx * self.problem.ny * self.problem.nz

    @property
    def iq(self) -> bool:
        return self.problem.dtype in (C64, C128)

    @property
    def wide(self) -> bool:
        """Samples (RF and output) are float64."""
        return self.problem.dtype in (F64, C128)

    @property
    def store_f16(self) -> bool:
        """The permuted buffer holds binary16 samples (torch.float16 tensors)."""
        return self.problem.storage == STORE_F16

    @property
    def batch_inner(self) -> bool:
        return self.info["algorithm"] == ALG_BATCH_INNER

    @property
    def repack(self) -> bool:
        return self.info["algorithm"] == ALG_REPACK

    @property
    def permuted_input(self) -> bool:
        """beamform reads the buffer made by permute (batch-inner and repack)."""
        return self.batch_inner or self.repack

    def permuted_dtype(self):
        """torch dtype of the permuted buffer."""
        import torch
        return torch.float16 if (self.store_f16 or self.repack) else torch.float32

    def permuted_bytes(self, q_count: Optional[int] = None) -> int:
        return int(self._lib.das_permuted_bytes(self._h, self.problem.Q if q_count is None else int(q_count)))

    def max_q_chunk(self) -> int:
        """Most transmit events one beamform call accepts (see das_max_q_chunk)."""
        return int(self._lib.das_max_q_chunk(self._h))

    def permuted_shape(self, q_count: Optional[int] = None) -> tuple:
        p = self.problem
        qc = p.Q if q_count is None else int(q_count)
        if self.repack:
            npc = (p.K + 7) // 8
            return (qc, p.M, npc, p.B, 8) if self.store_f16 else (qc, p.M, 2, npc, p.B, 8)
        shape = (p.K, qc, p.M, p.B) if p.layout == LAYOUT_KQMB else (qc, p.M, p.K, p.B)
        return shape + ((2,) if self.iq else ())

    def _permuted_numel(self, q_count: int) -> int:
        """Elements of the permuted tensor of q_count events (halves for repack)."""
        n = 1
        for d in self.permuted_shape(max(q_count, 1)):
            n *= d
        return n if q_count >= 1 else 0

    def output_shape(self) -> tuple:
        return (self.problem.B, self.N) + ((2,) if self.iq else ())

    # -- argument checks (sizes are unknown to the C ABI) --------------------
    def _tensor(self, t, numel: int, name: str, samples: bool = False, permuted: bool = False):
        """samples: RF or output, float64 for F64 / C128 plans; permuted: a permuted
        buffer, float16 for STORE_F16 plans; everything else float32."""
        import torch
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor")
        if t.dtype in (torch.complex64, torch.complex128, torch.complex32):
            t = torch.view_as_real(t)
        if permuted and (self.store_f16 or self.repack):
            want = torch.float16
        else:
            want = torch.float64 if (samples and self.wide) else torch.float32
        if t.dtype != want:
            raise TypeError(f"{name} must be {want} (or its complex type for IQ), got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() != numel:
            raise ValueError(f"{name} has {t.numel()} floats, expected {numel}")
        return t

    def _q_range(self, q_begin, q_count):
        q_count = self.problem.Q - int(q_begin) if q_count is None else int(q_count)
        return int(q_begin), q_count

    # -- entry points ---------------------------------------------------------
    def permute(self, rf, out, q_begin: int = 0, q_count: Optional[int] = None, stream=None):
        """B x Q x M x K -> the plan's frames-innermost layout, events [q_begin, q_begin+q_count)."""
        p = self.problem
        q_begin, q_count = self._q_range(q_begin, q_count)
        c = 2 if self.iq else 1
        rf = self._tensor(rf, p.B * p.Q * p.M * p.K * c, "rf", samples=True)
        out = self._tensor(out, self._permuted_numel(q_count), "out", samples=True, permuted=True)
        _check(self._lib.das_permute(self._h, rf.data_ptr(), out.data_ptr(), q_begin, q_count,
                                     _stream_handle(stream, rf.device)), "das_permute")
        return out

    def beamform(self, rf, rx_pos, tau_tx, w_tx, out, q_begin: int = 0, q_count: Optional[int] = None,
                 accumulate: bool = False, stream=None, noalloc: bool = False):
        """Sum events [q_begin, q_begin+q_count) into out (B x N, or B x N x 2 for IQ).

        noalloc: call das_beamform_noalloc (no device allocation; the library's
        fixed work area, shared by every such call on the device).
        """
        p = self.problem
        q_begin, q_count = self._q_range(q_begin, q_count)
        c = 2 if self.iq else 1
        rf_numel = self._permuted_numel(q_count) if self.permuted_input else p.B * p.Q * p.M * p.K * c
        rf = self._tensor(rf, rf_numel, "rf", samples=True, permuted=self.permuted_input)
        rx_pos = self._tensor(rx_pos, 3 * p.M, "rx_pos")
        tau_tx = self._tensor(tau_tx, p.Q * self.N, "tau_tx")
        w_tx = self._tensor(w_tx, p.Q * self.N, "w_tx")
        out = self._tensor(out, p.B * self.N * c, "out", samples=True)
        fn, name = ((self._lib.das_beamform_noalloc, "das_beamform_noalloc") if noalloc
                    else (self._lib.das_beamform, "das_beamform"))
        _check(fn(self._h, rf.data_ptr(), rx_pos.data_ptr(), tau_tx.data_ptr(), w_tx.data_ptr(), out.data_ptr(),
                  q_begin, q_count, 1 if accumulate else 0, _stream_handle(stream, rf.device)), name)
        return out

    def beamform_streamed(self, rf, rx_pos, tau_tx, w_tx, out, perm_a, perm_b, q_chunk: int,
                          accumulate: bool = False, stream_permute=None, stream_beamform=None):
        """All Q events in chunks of q_chunk: permute of chunk c+1 (stream_permute) overlaps
        the beamform of chunk c (stream_beamform); perm_a / perm_b hold das_permuted_bytes(q_chunk)."""
        p = self.problem
        c = 2 if self.iq else 1
        q_chunk = int(q_chunk)
        rf = self._tensor(rf, p.B * p.Q * p.M * p.K * c, "rf", samples=True)
        rx_pos = self._tensor(rx_pos, 3 * p.M, "rx_pos")
        tau_tx = self._tensor(tau_tx, p.Q * self.N, "tau_tx")
        w_tx = self._tensor(w_tx, p.Q * self.N, "w_tx")
        out = self._tensor(out, p.B * self.N * c, "out", samples=True)
        chunk = self._permuted_numel(q_chunk)
        perm_a = self._tensor(perm_a, chunk, "perm_a", samples=True, permuted=True)
        perm_b = self._tensor(perm_b, chunk, "perm_b", samples=True, permuted=True)
        _check(self._lib.das_beamform_streamed(self._h, rf.data_ptr(), rx_pos.data_ptr(), tau_tx.data_ptr(),
                                               w_tx.data_ptr(), out.data_ptr(), perm_a.data_ptr(),
                                               perm_b.data_ptr(), q_chunk, 1 if accumulate else 0,
                                               _stream_handle(stream_permute, rf.device),
                                               _stream_handle(stream_beamform, rf.device)),
               "das_beamform_streamed")
        return out

    def tx_tables(self, events, tau_tx, w_tx, q_begin: int = 0, stream=None):
        """Fill rows [q_begin, q_begin + len(events)) of the Q x N transmit tables.

        events: sequence of (kind, (vx, vy, vz), weight) with kind TX_PLANE
        (unit propagation direction, vz > 0) or TX_DIVERGING (virtual source
        position in metres, vz < 0)."""
        p = self.problem
        arr = (_TxEvent * max(len(events), 1))()
        for i, (kind, v, weight) in enumerate(events):
            arr[i].kind = int(kind)
            arr[i].reserved = 0
            arr[i].v[:] = [float(x) for x in v]
            arr[i].weight = float(weight)
        tau_tx = self._tensor(tau_tx, p.Q * self.N, "tau_tx")
        w_tx = self._tensor(w_tx, p.Q * self.N, "w_tx")
        _check(self._lib.das_tx_tables(self._h, arr, int(q_begin), len(events), tau_tx.data_ptr(),
                                       w_tx.data_ptr(), _stream_handle(stream, tau_tx.device)),
               "das_tx_tables")
        return tau_tx, w_tx

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.das_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_from_fields(fields: dict, algorithm: str = "batch_inner", layout: str = "kqmb",
                     wide: bool = False, storage: str = "native") -> Plan:
    """Plan from a plain description (B, Q, M, K, nx, ny, nz, origin, spacing, fs, c, t0,
    f_number, f_demod, iq); wide: float64 samples (F64 / C128); storage: "native" or
    "f16" (binary16 samples in the permuted buffer)."""
    iq = bool(fields.get("iq"))
    dtype = ("c128" if iq else "f64") if wide else ("c64" if iq else "f32")
    return Plan(B=fields["B"], Q=fields["Q"], M=fields["M"], K=fields["K"], nx=fields["nx"],
                ny=fields["ny"], nz=fields["nz"], origin=fields["origin"], spacing=fields["spacing"],
                fs=fields["fs"], c=fields["c"], t0=fields.get("t0", 0.0),
                f_number=fields.get("f_number", 1.0), f_demod=fields.get("f_demod", 0.0),
                dtype=dtype, algorithm=algorithm, layout=layout, storage=storage)
