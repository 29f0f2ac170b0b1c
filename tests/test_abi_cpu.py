"""CPU-side checks of the C ABI library: it loads, exports every declared symbol, and validates
requests before touching a device.  No compute call is made here."""
import ctypes
import glob
import os
import re

import pytest

import block_scaled_precision_gemm_amd as bsg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(bsg_[a-z_0-9]+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = bsg.load_library()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"libbsg.so does not export {n}"


def test_abi_version_and_status_strings():
    lib = bsg.load_library()
    assert lib.bsg_abi_version() == 3
    for code, name in bsg.STATUS.items():
        assert lib.bsg_status_string(code).decode() == name


def _create(**kw):
    prob = bsg.Problem(ctypes.sizeof(bsg.Problem), 1, 1, 0, 256, 256, 256, -1)
    for k, v in kw.items():
        setattr(prob, k, v)
    h = ctypes.c_void_p()
    st = bsg.load_library().bsg_plan_create(ctypes.byref(prob), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, 8), ("format", 3, 8), ("out_dtype", 0, 8), ("flags", 8, 8),
    ("M", 0, 2), ("N", 0, 2), ("K", 0, 2), ("N", 250, 2), ("K", 48, 2), ("M", 1 << 31, 2),
])
def test_plan_create_validation(field, value, status):
    st, h = _create(**{field: value})
    assert st == status, bsg.load_library().bsg_last_error()
    assert not h.value


@pytest.mark.parametrize("fields,status", [
    (dict(batch=-1), 2), (dict(batch=65536), 3),
    (dict(batch=2, stride_a=-16), 2), (dict(batch=2, stride_d=-32), 2),
    (dict(batch=2, stride_a=8), 4), (dict(batch=2, stride_b=24), 4), (dict(batch=2, stride_d=100), 4),
    (dict(batch=2, stride_sa=2), 4), (dict(batch=2, stride_bias=6), 4),
])
def test_batched_plan_validation(fields, status):
    st, h = _create(**fields)
    assert st == status, bsg.load_library().bsg_last_error()
    assert not h.value


@pytest.mark.parametrize("fields,status", [
    (dict(lda=128), 2), (dict(ldb=240), 2), (dict(ldd=128), 2),         # below the packed value
    (dict(lda=264), 4), (dict(ldb=280), 4), (dict(ldd=260), 4),         # rows not 16-byte aligned
    (dict(format=2, lda=272), 4),                                       # NVFP4: 136 bytes per row
    (dict(lda=1 << 31), 2), (dict(M=1 << 16, lda=1 << 15), 3),          # too large, spans >= 2^31
])
def test_leading_dimension_validation(fields, status):
    st, h = _create(**fields)
    assert st == status, bsg.load_library().bsg_last_error()
    assert not h.value


def test_abi1_problem_size_is_accepted():
    """An ABI-1 caller (48-byte bsg_problem, no batch fields) still passes validation: without a GPU
    it reaches the device check; any other size is an ABI error."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, _ = _create(struct_size=bsg.PROBLEM_V1_SIZE, batch=7, stride_a=3)  # bytes past 48 are not read
    assert st == 5, bsg.load_library().bsg_last_error()
    st, _ = _create(struct_size=bsg.PROBLEM_V1_SIZE + 8)
    assert st == 8
    # ABI 2 (96 bytes, no leading dimensions): the fields past it are not read (here invalid ones)
    st, _ = _create(struct_size=bsg.PROBLEM_V2_SIZE, lda=8, ldb=8, ldd=8)
    assert st == 5, bsg.load_library().bsg_last_error()
    st, _ = _create(lda=512, ldb=288, ldd=272)  # valid leading dimensions reach the device check
    assert st == 5, bsg.load_library().bsg_last_error()


def test_struct_layout_matches_header(tmp_path):
    """The ctypes mirrors of bsg_problem / bsg_plan_info have the C layout (compiled with gcc)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "bsg.h"\n'
        "int main(void) { printf(\"%zu %zu %zu %zu %zu %zu %u %zu %zu %u\\n\", sizeof(bsg_problem),"
        " offsetof(bsg_problem, device), offsetof(bsg_problem, batch), offsetof(bsg_problem, stride_a),"
        " offsetof(bsg_problem, stride_d), sizeof(bsg_plan_info), BSG_PROBLEM_V1_SIZE,"
        " offsetof(bsg_problem, lda), offsetof(bsg_problem, ldd), BSG_PROBLEM_V2_SIZE); return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    P = bsg.Problem
    want = [ctypes.sizeof(P), P.device.offset, P.batch.offset, P.stride_a.offset, P.stride_d.offset,
            ctypes.sizeof(bsg.PlanInfo), bsg.PROBLEM_V1_SIZE, P.lda.offset, P.ldd.offset, bsg.PROBLEM_V2_SIZE]
    assert got == want


def test_scale_layout_flag_passes_validation():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    for fmt in (1, 2):
        st, h = _create(format=fmt, flags=4 | 3)  # K-tile-major scales with bias + SiLU: valid, no device
        assert st == 5 and not h.value, bsg.load_library().bsg_last_error()


@pytest.mark.parametrize("rows,codes", [(1, 1), (1, 4), (3, 5), (257, 128), (130, 66), (0, 4), (4, 0), (-1, 8)])
def test_scales_ktile_bytes(rows, codes):
    want = 0 if rows < 1 or codes < 1 else 4 * rows * -(-codes // 4)  # G = ceil(codes / 4) dwords per row
    assert bsg.load_library().bsg_scales_ktile_bytes(rows, codes) == want == bsg.scales_ktile_bytes(rows, codes)


def test_pack_scales_argument_errors():
    lib = bsg.load_library()
    assert lib.bsg_pack_scales(None, 16, 4, 4, None) == 1
    assert lib.bsg_pack_scales(16, None, 4, 4, None) == 1
    assert lib.bsg_pack_scales(16, 32, 0, 4, None) == 2
    assert lib.bsg_pack_scales(16, 32, 4, 0, None) == 2
    assert lib.bsg_pack_scales(16, 32, 1 << 20, 1 << 13, None) == 2  # 2^33 bytes
    assert lib.bsg_pack_scales(16, 34, 4, 4, None) == 4  # dst not 4-byte aligned


def test_packed_strides_for_ktile_scales():
    st = bsg.packed_strides("nvfp4", 3, 16, 96, "ktile")  # 6 codes per row: 2 groups of 4
    assert st["sa"] == 2 * 3 * 4 and st["sb"] == 2 * 16 * 4
    st = bsg.packed_strides("mxfp8", 100, 32, 4096, "ktile")
    assert st["sa"] == 100 * 128 and st["sb"] == 32 * 128  # a multiple of 4 codes: same bytes as row-major


def test_nvfp4_k_rules():
    st, _ = _create(format=2, K=40)
    assert st == 2  # not a multiple of the 16-element block
    st, _ = _create(format=2, K=48)
    assert st == 3  # a valid NVFP4 K that no compiled kernel covers


def test_valid_problem_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = _create()
    assert st == 5 and not h.value
    assert b"device" in bsg.load_library().bsg_last_error().lower()


def test_forced_architecture_is_refused(monkeypatch):
    """BSG_FORCE_ARCH=<not gfx950> fails plan creation with BSG_ERR_DEVICE before any device query."""
    monkeypatch.setenv("BSG_FORCE_ARCH", "gfx942")
    st, h = _create()
    assert st == 5 and not h.value
    assert b"BSG_FORCE_ARCH=gfx942" in bsg.load_library().bsg_last_error()
    st, _ = _create(K=48)  # validation still comes first
    assert st == 2


def test_null_arguments():
    lib = bsg.load_library()
    assert lib.bsg_plan_create(None, None) == 1
    assert lib.bsg_run(None, 1, 1, 1, 1, None, 1.0, 1, None) == 1
    assert lib.bsg_plan_destroy(None) == 0
    assert lib.bsg_plan_query(None, None) == 1
    assert lib.bsg_test_decode_nvfp4_f16(None, None, None, 0, None) == 0
    assert lib.bsg_test_decode_nvfp4_f16(None, None, None, -32, None) == 2
    assert lib.bsg_test_decode_nvfp4_f16(None, None, None, 48, None) == 2
    assert lib.bsg_test_decode_nvfp4_f16(None, None, None, 32, None) == 1


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(bsg.LibraryNotBuilt):
        import importlib
        mod = importlib.import_module("block_scaled_precision_gemm_amd")
        saved = mod._lib
        try:
            mod._lib = None
            mod.load_library(str(tmp_path / "nope.so"))
        finally:
            mod._lib = saved
