"""C-ABI contract of libdas.so on the host: it loads, exports every declared
symbol, and rejects bad arguments with the documented status before touching
a device.  No kernel runs here."""
import ctypes
import os
import re
import subprocess

import pytest

import volumetric_delay_sum_amd as das

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "das.h")

OK, INVALID, UNSUPPORTED, ALIGNMENT, NO_DEVICE, LAUNCH, WORK_AREA = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def lib():
    return das.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(das_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("das_plan", "das_permute", "das_beamform", "das_plan_destroy", "das_error_string",
                     "das_permuted_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"libdas.so does not export {name}"


def test_abi_version(lib):
    text = open(HEADER).read()
    v = int(re.search(r"#define DAS_ABI_VERSION (\d+)", text).group(1))
    assert lib.das_abi_version() == v


def _c_layout(struct, fields, tmp_path):
    """sizeof and field offsets of a header struct, as the C compiler lays it out."""
    src = tmp_path / "layout.c"
    body = "".join(f'printf("%zu ", offsetof({struct}, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "das.h"\n'
                   f'int main(void){{printf("%zu ", sizeof({struct}));{body}return 0;}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    return [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]


@pytest.mark.parametrize("cls,struct", [(das._Problem, "das_problem"), (das._PlanInfo, "das_plan_info"),
                                        (das._TxEvent, "das_tx_event")])
def test_ctypes_mirrors_match_the_header(cls, struct, tmp_path):
    fields = [f for f, _ in cls._fields_]
    got = _c_layout(struct, fields, tmp_path)
    assert got[0] == ctypes.sizeof(cls)
    assert got[1:] == [getattr(cls, f).offset for f in fields]


def _problem(**kw):
    base = dict(B=4, Q=2, M=8, K=64, nx=4, ny=4, nz=2, origin=(0.0, 0.0, 5e-3), spacing=(2e-4,) * 3,
                fs=20e6, c=1540.0, t0=0.0, f_number=1.0, f_demod=0.0, dtype="f32", algorithm="batch_inner",
                layout="kqmb")
    base.update(kw)
    return base


def _status(**kw):
    try:
        das.Plan(**_problem(**kw))
        return OK
    except das.DasError as e:
        return e.code


@pytest.mark.parametrize("field,value", [("B", 0), ("Q", 0), ("M", 0), ("K", 1), ("nx", 0), ("ny", -1),
                                         ("nz", 0), ("fs", 0.0), ("c", -1.0), ("fs", float("nan")),
                                         ("t0", float("inf")), ("algorithm", 7), ("layout", 3), ("dtype", 5)])
def test_plan_rejects_invalid_problems(field, value):
    assert _status(**{field: value}) == INVALID


def test_plan_rejects_nonfinite_geometry():
    assert _status(origin=(0.0, float("nan"), 0.0)) == INVALID
    assert _status(spacing=(1e-4, float("inf"), 1e-4)) == INVALID


def test_plan_dtype_demod_mismatch_is_unsupported():
    assert _status(dtype="f32", f_demod=5e6) == UNSUPPORTED
    assert _status(dtype="c64", f_demod=0.0) == UNSUPPORTED
    assert _status(dtype="c64", f_demod=5e6) == OK


def test_plan_rejects_sizes_beyond_addressing():
    assert _status(nx=2048, ny=2048, nz=1024) == UNSUPPORTED          # N > 2^31
    assert _status(K=1 << 20, B=512) == UNSUPPORTED                   # 16 K B elem > 4 GiB


def test_plan_null_pointers(lib):
    h = ctypes.c_void_p()
    assert lib.das_plan(None, ctypes.byref(h)) == INVALID
    p = das._Problem()
    assert lib.das_plan(ctypes.byref(p), None) == INVALID


def test_plan_info_and_sizes():
    pl = das.Plan(**_problem(B=32, dtype="c64", f_demod=5e6))
    assert pl.info["algorithm"] == das.ALG_BATCH_INNER
    assert pl.info["elem_bytes"] == 8
    assert pl.info["frames_per_lane"] == 16                 # IQ, B % 16 == 0: whole-row lanes, 16 complex frames a lane
    assert pl.info["lanes_per_voxel"] == 8
    assert pl.info["whole_rows"] == 1 and pl.info["receivers_per_step"] == 8
    assert pl.info["N"] == 32
    assert pl.permuted_bytes(1) == 64 * 1 * 8 * 32 * 8
    assert pl.permuted_bytes(2) == 2 * pl.permuted_bytes(1)
    assert pl.permuted_bytes(3) == 0
    assert pl.permuted_bytes(0) == 0
    assert pl.permuted_shape(1) == (64, 1, 8, 32, 2)
    pl2 = das.Plan(**_problem(algorithm="default"))
    assert pl2.info["algorithm"] == das.ALG_BASELINE       # DEFAULT dispatches to the baseline
    assert pl.info["staged"] == 1
    assert das.Plan(**_problem(B=40, dtype="c64", f_demod=5e6)).info["staged"] == 0   # IQ, B % 16 != 0
    assert das.Plan(**_problem(B=32)).info["staged"] == 1      # fp32, B % 32 == 0: LDS-staged
    assert das.Plan(**_problem(B=16)).info["staged"] == 1      # fp32, B % 16 == 0: LDS-staged, 1 frame per lane
    assert das.Plan(**_problem(B=24)).info["staged"] == 0
    assert das.Plan(**_problem(B=32, algorithm="baseline")).info["staged"] == 0
    pl3 = das.Plan(**_problem(layout="qmkb"))
    assert pl3.permuted_shape(2) == (2, 8, 64, 4)


def test_float64_dtypes_are_baseline_only():
    f64 = das.Plan(**_problem(dtype="f64", algorithm="baseline"))
    assert f64.info["elem_bytes"] == 8 and f64.info["algorithm"] == das.ALG_BASELINE and f64.wide
    c128 = das.Plan(**_problem(dtype="c128", f_demod=5e6, algorithm="default"))
    assert c128.info["elem_bytes"] == 16 and c128.info["algorithm"] == das.ALG_BASELINE and c128.iq
    assert _status(dtype="f64", algorithm="batch_inner") == UNSUPPORTED
    assert _status(dtype="c128", f_demod=5e6, algorithm="batch_inner") == UNSUPPORTED
    assert _status(dtype="c128", f_demod=0.0, algorithm="baseline") == UNSUPPORTED    # complex needs f_demod
    assert _status(dtype="f64", f_demod=5e6, algorithm="baseline") == UNSUPPORTED     # real needs none
    assert _status(dtype=7, algorithm="baseline") == INVALID
    # one frame (no batch dimension) is a valid fp64 problem
    assert das.Plan(**_problem(B=1, dtype="f64", algorithm="baseline")).info["frames_per_lane"] == 8


def test_float64_plans_do_not_permute(lib):
    pl = das.Plan(**_problem(dtype="f64", algorithm="baseline"))
    g = _fake(0x10000)
    assert lib.das_permute(pl._h, g, g, 0, 1, None) == UNSUPPORTED


@pytest.mark.parametrize("dtype,B,alg", [("f32", 32, das.ALG_BATCH_INNER), ("f32", 16, das.ALG_BATCH_INNER),
                                         ("f32", 8, das.ALG_BASELINE), ("f32", 1, das.ALG_BASELINE),
                                         ("c64", 16, das.ALG_BATCH_INNER), ("c64", 4, das.ALG_BASELINE),
                                         ("f64", 64, das.ALG_BASELINE), ("c128", 64, das.ALG_BASELINE)])
def test_auto_selection(dtype, B, alg):
    pl = das.Plan(**_problem(B=B, dtype=dtype, f_demod=5e6 if dtype in ("c64", "c128") else 0.0,
                             algorithm="auto"))
    assert pl.info["algorithm"] == alg
    # DEFAULT stays the baseline, as the docs dispatch it
    assert das.Plan(**_problem(B=B, dtype=dtype, f_demod=5e6 if dtype in ("c64", "c128") else 0.0,
                               algorithm="default")).info["algorithm"] == das.ALG_BASELINE


@pytest.mark.parametrize("B,fl", [(1, 1), (8, 1), (16, 16), (24, 1), (32, 32), (48, 16), (64, 32), (96, 32), (66, 1),
                                  (160, 32), (192, 32), (68, 4)])
def test_frames_per_lane_choice(B, fl):
    # fp32 batch-inner: the LDS-staged whole-row kernel wherever B % 16 == 0
    # (all 32 frames of a frame tile per lane when B % 32 == 0, else 16),
    # direct loads otherwise
    pl = das.Plan(**_problem(B=B))
    assert pl.info["frames_per_lane"] == fl
    assert pl.info["staged"] == (1 if B % 16 == 0 else 0)
    assert pl.info["whole_rows"] == (1 if B % 16 == 0 else 0)
    assert pl.info["receivers_per_step"] == (16 if B % 16 == 0 else 0)


@pytest.mark.parametrize("B,fl", [(32, 2), (64, 4), (96, 2), (160, 2), (192, 4)])
def test_frames_per_lane_choice_dpp_rows(B, fl, monkeypatch):
    # DAS_STAGED_ROWS=0 keeps the DPP-row staged kernel (4 frames per lane in
    # split rows when B % 64 == 0, else 2), for comparisons
    monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    pl = das.Plan(**_problem(B=B))
    assert pl.info["frames_per_lane"] == fl and pl.info["whole_rows"] == 0 and pl.info["staged"] == 1
    assert pl.info["receivers_per_step"] == (8 if B % 64 == 0 else 16)


@pytest.mark.parametrize("rows,iq,per_step", [("1", False, 8), ("2", False, 16), ("1", True, 8), ("2", True, 8)])
def test_whole_row_receivers_per_step(rows, iq, per_step, monkeypatch):
    # DAS_STAGED_ROWS picks 8 or 16 receivers a step; complex items keep 8
    monkeypatch.setenv("DAS_STAGED_ROWS", rows)
    pl = das.Plan(**_problem(B=32, dtype="c64" if iq else "f32", f_demod=5e6 if iq else 0.0))
    assert pl.info["whole_rows"] == 1 and pl.info["receivers_per_step"] == per_step
    assert pl.info["lanes_per_voxel"] == 8 and pl.info["frames_per_lane"] == (16 if iq else 32)


def test_whole_rows_limits():
    # both storages; records of at most 65535 samples; at most 4096 receivers
    # (the kernel's receive-aperture mask)
    assert das.Plan(**_problem(B=32, storage="f16")).info["whole_rows"] == 1
    assert das.Plan(**_problem(B=32, K=65535)).info["whole_rows"] == 1
    assert das.Plan(**_problem(B=32, K=65536)).info["whole_rows"] == 0
    assert das.Plan(**_problem(B=32, M=4096)).info["whole_rows"] == 1
    assert das.Plan(**_problem(B=32, M=4097)).info["whole_rows"] == 0


@pytest.mark.parametrize("B,fl", [(32, 2), (64, 4), (96, 4), (160, 4)])
def test_frames_per_lane_choice_direct(B, fl, monkeypatch):
    monkeypatch.setenv("DAS_BI_KERNEL", "direct")
    pl = das.Plan(**_problem(B=B))
    assert pl.info["frames_per_lane"] == fl
    assert pl.info["staged"] == 0


@pytest.mark.parametrize("B,fl", [(1, 1), (8, 1), (16, 16), (31, 1), (32, 16), (40, 2), (48, 16), (64, 16), (34, 2)])
def test_frames_per_lane_choice_iq(B, fl):
    # complex64 batch-inner: the LDS-staged whole-row kernel wherever B % 16
    # == 0 (16 complex frames a lane), direct loads otherwise
    pl = das.Plan(**_problem(B=B, dtype="c64", f_demod=5e6))
    assert pl.info["frames_per_lane"] == fl
    assert pl.info["staged"] == (1 if B % 16 == 0 else 0)
    assert pl.info["whole_rows"] == (1 if B % 16 == 0 else 0)


@pytest.mark.parametrize("B,fl", [(16, 1), (32, 2), (48, 1), (64, 2)])
def test_frames_per_lane_choice_iq_dpp_rows(B, fl, monkeypatch):
    # DAS_STAGED_ROWS=0: the DPP-row kernel, 2 complex frames a lane in split
    # rows when B % 32 == 0, else 1
    monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    pl = das.Plan(**_problem(B=B, dtype="c64", f_demod=5e6))
    assert pl.info["frames_per_lane"] == fl and pl.info["staged"] == 1 and pl.info["whole_rows"] == 0


def test_error_strings(lib):
    for code in range(0, 8):
        s = lib.das_error_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.das_error_string(-3) == b"unknown status"


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_permute_argument_errors(lib):
    pl = das.Plan(**_problem())
    h = pl._h
    good = _fake(0x10000)
    assert lib.das_permute(None, good, good, 0, 1, None) == INVALID
    assert lib.das_permute(h, None, good, 0, 1, None) == INVALID
    assert lib.das_permute(h, good, None, 0, 1, None) == INVALID
    assert lib.das_permute(h, good, good, -1, 1, None) == INVALID
    assert lib.das_permute(h, good, good, 0, 0, None) == INVALID
    assert lib.das_permute(h, good, good, 1, 2, None) == INVALID          # past Q
    assert lib.das_permute(h, _fake(0x10004), good, 0, 1, None) == ALIGNMENT
    assert lib.das_permute(h, good, _fake(0x10008), 0, 1, None) == ALIGNMENT


def test_beamform_argument_errors(lib):
    pl = das.Plan(**_problem())
    h = pl._h
    g = _fake(0x10000)
    bad = _fake(0x10004)
    assert lib.das_beamform(None, g, g, g, g, g, 0, 1, 0, None) == INVALID
    for i in range(5):
        args = [g] * 5
        args[i] = None
        assert lib.das_beamform(h, *args, 0, 1, 0, None) == INVALID
    assert lib.das_beamform(h, g, g, g, g, g, 0, 3, 0, None) == INVALID
    assert lib.das_beamform(h, g, g, g, g, g, 2, 1, 0, None) == INVALID
    assert lib.das_beamform(h, g, g, g, g, g, 0, 1, 2, None) == INVALID       # accumulate not 0/1
    for i in range(5):
        args = [g] * 5
        args[i] = bad
        assert lib.das_beamform(h, *args, 0, 1, 0, None) == ALIGNMENT


def test_noalloc_work_area_limit(lib):
    """das_beamform_noalloc rejects a whole-row plan that sorts more voxel
    tiles than its fixed work area holds (65536 of 8 x 8 x 2) with its own
    status, before any HIP call (so fake pointers are safe here), and checks
    its arguments as das_beamform does."""
    g, bad = _fake(0x10000), _fake(0x10004)
    big = _problem(B=32, Q=1, M=64, K=64, nx=1024, ny=1024, nz=18, layout="qmkb")   # 128 x 128 x 9 tiles
    pl = das.Plan(**big)
    assert pl.info["whole_rows"] == 1
    assert lib.das_beamform_noalloc(pl._h, g, g, g, g, g, 0, 1, 0, None) == WORK_AREA
    assert b"65536" in lib.das_error_string(WORK_AREA)
    assert lib.das_beamform_noalloc(None, g, g, g, g, g, 0, 1, 0, None) == INVALID
    assert lib.das_beamform_noalloc(pl._h, g, g, g, g, g, 0, 2, 0, None) == INVALID       # past Q
    assert lib.das_beamform_noalloc(pl._h, g, bad, g, g, g, 0, 1, 0, None) == ALIGNMENT


def test_streamed_argument_errors(lib):
    pl = das.Plan(**_problem())
    h = pl._h
    g, g2, bad = _fake(0x10000), _fake(0x20000), _fake(0x10004)
    ok = [g, g, g, g, g, g, g2]                 # rf, rx, tau, w, out, perm_a, perm_b
    assert lib.das_beamform_streamed(None, *ok, 1, 0, None, None) == INVALID
    for i in range(7):
        args = list(ok)
        args[i] = None
        assert lib.das_beamform_streamed(h, *args, 1, 0, None, None) == INVALID
    assert lib.das_beamform_streamed(h, g, g, g, g, g, g, g, 1, 0, None, None) == INVALID   # perm_a == perm_b
    assert lib.das_beamform_streamed(h, *ok, 0, 0, None, None) == INVALID                 # q_chunk 0
    assert lib.das_beamform_streamed(h, *ok, 1, 2, None, None) == INVALID                 # accumulate not 0/1
    assert lib.das_beamform_streamed(h, *ok, 3, 0, None, None) == UNSUPPORTED             # above max_q_chunk (Q)
    base = das.Plan(**_problem(algorithm="baseline"))
    assert lib.das_beamform_streamed(base._h, *ok, 1, 0, None, None) == UNSUPPORTED       # nothing to permute
    for i in range(7):
        args = list(ok)
        args[i] = bad
        assert lib.das_beamform_streamed(h, *args, 1, 0, None, None) == ALIGNMENT
    if not _gpu():
        assert lib.das_beamform_streamed(h, *ok, 1, 0, None, None) == NO_DEVICE


def _tx_events(*specs):
    arr = (das._TxEvent * len(specs))()
    for i, (kind, v, weight) in enumerate(specs):
        arr[i].kind, arr[i].reserved = kind, 0
        arr[i].v[:] = v
        arr[i].weight = weight
    return arr


def test_tx_tables_argument_errors(lib):
    pl = das.Plan(**_problem())                  # Q = 2
    h = pl._h
    g, bad = _fake(0x10000), _fake(0x10004)
    plane = (das.TX_PLANE, (0.0, 0.0, 1.0), 1.0)
    div = (das.TX_DIVERGING, (1e-3, 0.0, -1e-2), 0.5)
    ev = _tx_events(plane, div)
    assert lib.das_tx_tables(None, ev, 0, 2, g, g, None) == INVALID
    assert lib.das_tx_tables(h, None, 0, 2, g, g, None) == INVALID
    assert lib.das_tx_tables(h, ev, 0, 2, None, g, None) == INVALID
    assert lib.das_tx_tables(h, ev, 0, 2, g, None, None) == INVALID
    assert lib.das_tx_tables(h, ev, 0, 0, g, g, None) == INVALID          # empty
    assert lib.das_tx_tables(h, ev, 1, 2, g, g, None) == INVALID          # past Q
    assert lib.das_tx_tables(h, ev, -1, 1, g, g, None) == INVALID
    for spec in [(5, (0.0, 0.0, 1.0), 1.0),                               # unknown kind
                 (das.TX_PLANE, (0.0, 0.0, 1.1), 1.0),                    # not a unit vector
                 (das.TX_PLANE, (1.0, 0.0, 0.0), 1.0),                    # not towards +z
                 (das.TX_DIVERGING, (0.0, 0.0, 1e-3), 1.0),               # source not behind the array
                 (das.TX_DIVERGING, (0.0, 0.0, -1e-2), float("nan")),     # weight
                 (das.TX_DIVERGING, (float("inf"), 0.0, -1e-2), 1.0)]:
        assert lib.das_tx_tables(h, _tx_events(spec), 0, 1, g, g, None) == INVALID, spec
    r = _tx_events(plane)
    r[0].reserved = 1
    assert lib.das_tx_tables(h, r, 0, 1, g, g, None) == INVALID
    assert lib.das_tx_tables(h, ev, 0, 2, bad, g, None) == ALIGNMENT
    assert lib.das_tx_tables(h, ev, 0, 2, g, bad, None) == ALIGNMENT
    if not _gpu():
        assert lib.das_tx_tables(h, ev, 0, 2, g, g, None) == NO_DEVICE


def test_batch_inner_kqmb_chunk_limit(lib):
    # K * q_count * M * B * 4 > 4 GiB: the KQMB batch-inner kernel needs a smaller chunk
    pl = das.Plan(**_problem(B=64, Q=16, M=1024, K=4096))
    g = _fake(0x10000)
    assert lib.das_beamform(pl._h, g, g, g, g, g, 0, 16, 0, None) == UNSUPPORTED
    assert lib.das_beamform(pl._h, g, g, g, g, g, 0, 4, 0, None) == UNSUPPORTED
    assert lib.das_max_q_chunk(pl._h) == 3
    assert pl.max_q_chunk() == 3
    assert das.Plan(**_problem(B=64, Q=16, M=1024, K=4096, layout="qmkb")).max_q_chunk() == 16
    assert das.Plan(**_problem(B=64, Q=16, M=1024, K=4096, algorithm="baseline")).max_q_chunk() == 16
    assert lib.das_max_q_chunk(None) == 0
    # Main-c64: 8 events of 2048 x 1024 x 32 complex samples are exactly 4 GiB, 7 fit
    assert das.Plan(**_problem(B=32, Q=9, M=1024, K=2048, dtype="c64", f_demod=5e6)).max_q_chunk() == 7
    # a 1-event chunk passes validation (and then needs a device)
    rc = lib.das_beamform(pl._h, g, g, g, g, g, 0, 1, 0, None) if not _gpu() else NO_DEVICE
    assert rc == NO_DEVICE


def _gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu(), reason="checks the no-device path")
def test_no_device_is_reported(lib):
    pl = das.Plan(**_problem())
    g = _fake(0x10000)
    assert lib.das_permute(pl._h, g, g, 0, 1, None) == NO_DEVICE
    assert lib.das_beamform(pl._h, g, g, g, g, g, 0, 1, 0, None) == NO_DEVICE


def test_binding_checks_tensor_sizes_before_the_call():
    torch = pytest.importorskip("torch")
    pl = das.Plan(**_problem())
    cpu = torch.zeros(10)
    with pytest.raises(TypeError):
        pl.beamform(cpu, cpu, cpu, cpu, cpu)


@pytest.mark.parametrize("B,dtype", [(64, "f32"), (32, "c64")])
def test_split_rows_can_be_switched_off(B, dtype, monkeypatch):
    # DPP-row kernel: DAS_STAGED_SPLIT=1 keeps whole rows (8 bytes per lane), for comparisons
    monkeypatch.setenv("DAS_STAGED_ROWS", "0")
    kw = dict(B=B, dtype=dtype, f_demod=5e6 if dtype == "c64" else 0.0)
    assert das.Plan(**_problem(**kw)).info["frames_per_lane"] == (4 if dtype == "f32" else 2)
    monkeypatch.setenv("DAS_STAGED_SPLIT", "1")
    pl = das.Plan(**_problem(**kw))
    assert pl.info["staged"] == 1
    assert pl.info["frames_per_lane"] == (2 if dtype == "f32" else 1)


# ---- binary16 storage of the permuted buffer -------------------------------

def test_storage_enum_is_validated():
    assert _status(storage=2) == INVALID
    assert _status(storage=-1) == INVALID
    assert _status(storage="native") == OK and _status(storage="f16") == OK


def test_binary16_storage_needs_batch_inner():
    assert _status(storage="f16", algorithm="baseline") == UNSUPPORTED
    assert _status(storage="f16", algorithm="default") == UNSUPPORTED
    assert _status(storage="f16", algorithm="auto", B=8) == UNSUPPORTED        # auto resolves to the baseline
    assert _status(storage="f16", algorithm="auto", B=32) == OK
    assert _status(storage="f16", dtype="f64", algorithm="baseline") == UNSUPPORTED
    assert _status(storage="f16", dtype="c128", f_demod=5e6, algorithm="baseline") == UNSUPPORTED


@pytest.mark.parametrize("dtype,B,store,fl,staged,rows", [
    ("f32", 32, 2, 32, 1, 1), ("f32", 64, 2, 32, 1, 1), ("f32", 128, 2, 32, 1, 1), ("f32", 96, 2, 32, 1, 1),
    ("f32", 16, 2, 16, 1, 1), ("f32", 48, 2, 16, 1, 1),
    ("f32", 24, 2, 2, 0, 0), ("f32", 68, 2, 4, 0, 0), ("f32", 7, 2, 1, 0, 0), ("c64", 32, 4, 16, 1, 1),
    ("c64", 64, 4, 16, 1, 1), ("c64", 16, 4, 16, 1, 1), ("c64", 48, 4, 16, 1, 1), ("c64", 34, 4, 2, 0, 0)])
def test_binary16_plan_info(dtype, B, store, fl, staged, rows):
    # binary16 rows run the whole-row kernel where its frame tiles fit (32 or
    # 16 fp32 or 16 complex frames: B a multiple of 16)
    iq = dtype == "c64"
    pl = das.Plan(**_problem(B=B, dtype=dtype, f_demod=5e6 if iq else 0.0, storage="f16"))
    assert pl.store_f16
    assert pl.info["elem_bytes"] == (8 if iq else 4)
    assert pl.info["store_bytes"] == store
    assert pl.info["frames_per_lane"] == fl
    assert pl.info["staged"] == staged
    assert pl.info["whole_rows"] == rows
    native = das.Plan(**_problem(B=B, dtype=dtype, f_demod=5e6 if iq else 0.0))
    assert native.info["store_bytes"] == native.info["elem_bytes"]
    assert pl.permuted_bytes(1) * 2 == native.permuted_bytes(1)
    assert pl.permuted_shape(2) == native.permuted_shape(2)


def test_binary16_direct_frames_per_lane(monkeypatch):
    monkeypatch.setenv("DAS_BI_KERNEL", "direct")
    pl = das.Plan(**_problem(B=32, storage="f16"))
    assert pl.info["staged"] == 0 and pl.info["frames_per_lane"] == 2
    assert das.Plan(**_problem(B=64, storage="f16")).info["frames_per_lane"] == 4


def test_binary16_kqmb_chunk_limit_counts_half_bytes():
    # a KQMB chunk must stay below 4 GiB: with 2-byte samples twice the events fit
    kw = dict(B=64, Q=64, M=1024, K=4096)
    native = das.Plan(**_problem(**kw))
    half = das.Plan(**_problem(storage="f16", **kw))
    assert native.max_q_chunk() == 3
    assert half.max_q_chunk() == 7


# --------------------------------------------------------------------------
# Repack (matrix-core) plans
# --------------------------------------------------------------------------

def test_repack_plan_limits():
    assert _status(algorithm="repack", B=32) == OK
    assert _status(algorithm="repack", B=64, storage="f16") == OK
    assert _status(algorithm="repack", B=16) == UNSUPPORTED                  # 32-frame tiles
    assert _status(algorithm="repack", B=40) == UNSUPPORTED
    assert _status(algorithm="repack", B=32, dtype="c64", f_demod=5e6) == UNSUPPORTED
    assert _status(algorithm="repack", B=32, dtype="f64") == UNSUPPORTED
    assert _status(algorithm="repack", B=32, K=65535) == OK
    assert _status(algorithm="repack", B=32, K=65536) == UNSUPPORTED          # 16-bit window indices
    assert _status(algorithm="repack", B=32, Q=2, nx=2048, ny=1024, nz=1024) == UNSUPPORTED   # Q N >= 2^32
    # its layout belongs to it alone
    assert _status(algorithm="batch_inner", B=32, layout="qmpb") == INVALID
    assert _status(algorithm="repack", B=32, layout="qmkb") == OK             # ignored: the plan picks QMPB


@pytest.mark.parametrize("storage,B,K,planes", [("native", 32, 64, 2), ("native", 64, 66, 2),
                                                ("f16", 32, 64, 1), ("f16", 96, 70, 1)])
def test_repack_plan_info_and_sizes(storage, B, K, planes):
    pl = das.Plan(**_problem(algorithm="repack", B=B, K=K, storage=storage))
    assert pl.repack and pl.permuted_input and not pl.batch_inner
    assert pl.info["algorithm"] == das.ALG_REPACK
    assert pl.info["layout"] == das.LAYOUT_QMPB
    assert pl.info["lanes_per_voxel"] == 2
    assert pl.info["frames_per_lane"] == (32 if B % 64 == 0 else 16)
    assert pl.info["staged"] == 1
    npc = (K + 7) // 8
    assert pl.permuted_bytes(1) == 8 * planes * npc * B * 16                 # M = 8
    assert pl.permuted_bytes(2) == 2 * pl.permuted_bytes(1)
    assert pl.permuted_shape(2) == ((2, 8, npc, B, 8) if storage == "f16" else (2, 8, 2, npc, B, 8))
    assert pl.max_q_chunk() == 2
    import torch
    assert pl.permuted_dtype() == torch.float16
