"""The C ABI library: it loads, exports every entry point include/hkv.h
declares, and rejects bad arguments before touching a GPU. No kernels run."""

import ctypes
import pathlib
import re
import subprocess

import pytest

from conftest import ROOT, gpu_available

HEADER = pathlib.Path(ROOT) / "include" / "hkv.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(hkv_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted([
        "hkv_create", "hkv_destroy", "hkv_get_options", "hkv_find", "hkv_find_ptr", "hkv_contains",
        "hkv_insert_or_assign", "hkv_insert_or_assign_noalloc", "hkv_insert_and_evict", "hkv_find_or_insert", "hkv_assign", "hkv_size",
        "hkv_export_batch", "hkv_set_outcome_counters", "hkv_profile_start", "hkv_profile_stop",
        "hkv_last_error"])


def test_library_exports_every_declared_symbol():
    from hash_table_cache_amd import _native

    out = subprocess.run(["nm", "-D", "--defined-only", str(_native.LIB_PATH)], check=True,
                         capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(_native.load(), name) is not None
    assert set(_native.EXPORTS) == set(declared_functions())
    # nothing but the ABI is exported from the library's own code
    assert {n for n in exported if n.startswith("hkv")} == set(declared_functions())


def test_mixed_driver_library_exports_its_entry_point():
    from hash_table_cache_amd import build as hb

    out = subprocess.run(["nm", "-D", "--defined-only", str(hb.MIXED_LIB_PATH)], check=True,
                         capture_output=True, text=True).stdout
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == {"hkv_mixed_run"}


def test_oracle_library_exports():
    import oracle

    L = oracle.lib()
    for name in ["oracle_create", "oracle_find", "oracle_insert_or_assign", "oracle_assign",
                 "oracle_size", "oracle_export", "oracle_route"]:
        assert getattr(L, name) is not None


def _create(**kw):
    from hash_table_cache_amd import _native

    o = dict(capacity=1024, dim=8, bucket_slots=128, dual_bucket=0, values_on_host=0, device=0, flags=0)
    o.update(kw)
    opt = _native.HkvOptions(o["capacity"], o["dim"], o["bucket_slots"], o["dual_bucket"],
                             o["values_on_host"], o["device"], o["flags"])
    h = ctypes.c_void_p()
    st = _native.load().hkv_create(ctypes.byref(opt), ctypes.byref(h))
    return st, h, _native.load().hkv_last_error().decode()


@pytest.mark.parametrize("kw,needle", [
    (dict(capacity=0), "multiple of 128"),
    (dict(capacity=1000), "multiple of 128"),
    (dict(dim=0), "dim"),
    (dict(dim=(1 << 20) + 1), "dim"),  # rows of at most 2^20 floats
    (dict(capacity=128 << 31), "2^31 - 1 buckets"),
    (dict(bucket_slots=64), "128-slot"),
    (dict(dual_bucket=2), "0 or 1"),
    (dict(flags=0x80), "flags"),
])
def test_create_rejects_bad_options(kw, needle):
    from hash_table_cache_amd import _native

    st, h, msg = _create(**kw)
    assert st == _native.HKV_EINVAL
    assert h.value is None
    assert needle in msg


def test_null_arguments():
    from hash_table_cache_amd import _native

    L = _native.load()
    assert L.hkv_create(None, None) == _native.HKV_EINVAL
    assert L.hkv_find(None, 1, None, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_insert_or_assign(None, 1, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_insert_or_assign_noalloc(None, 1, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_assign(None, 1, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_export_batch(None, 0, 1, None, None, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_find_ptr(None, 1, None, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_contains(None, 1, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_insert_and_evict(None, 1, None, None, None, None, None, None, None, None) == _native.HKV_EINVAL
    assert L.hkv_find_or_insert(None, 1, None, None, None, None, None) == _native.HKV_EINVAL
    out = ctypes.c_uint64()
    assert L.hkv_size(None, ctypes.byref(out), None) == _native.HKV_EINVAL
    assert L.hkv_set_outcome_counters(None, None) == _native.HKV_EINVAL
    assert L.hkv_profile_start(None) == _native.HKV_EINVAL
    cnt = ctypes.c_uint32()
    assert L.hkv_profile_stop(None, None, 0, ctypes.byref(cnt)) == _native.HKV_EINVAL
    assert L.hkv_destroy(None) == _native.HKV_OK
    assert "NULL" in L.hkv_last_error().decode()


@pytest.mark.skipif(gpu_available(), reason="checks the no-device error path")
def test_create_without_device_reports_hip_error():
    from hash_table_cache_amd import _native

    st, h, msg = _create()
    assert st == _native.HKV_EHIP
    assert "no HIP device" in msg


def test_mixed_driver_rejects_null_arguments():
    from hash_table_cache_amd import _native
    from hash_table_cache_amd import build as hb

    L = ctypes.CDLL(str(hb.MIXED_LIB_PATH))
    P = ctypes.c_void_p
    L.hkv_mixed_run.argtypes = [P, ctypes.c_uint32, P, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32,
                                P, P, P, P, P, ctypes.POINTER(ctypes.c_double)]
    L.hkv_mixed_run.restype = ctypes.c_int32
    secs = ctypes.c_double(0)
    roles = (ctypes.c_int32 * 1)(0)
    # no table, no roles, no threads, no pool: rejected before any HIP call
    assert L.hkv_mixed_run(None, 1, roles, 1, 1, 1, None, None, None, None, None, ctypes.byref(secs)) == \
        _native.HKV_EINVAL
    assert L.hkv_mixed_run(None, 0, None, 1, 1, 1, None, None, None, None, None, None) == _native.HKV_EINVAL


def test_every_hip_build_targets_gfx950_without_packed_fp32():
    """Every hipcc compile of the package (library, mixed-workload driver,
    access-pattern program) targets gfx950 and turns packed fp32 instructions
    off; and the built code object holds none of them."""
    from hash_table_cache_amd import build as hb

    flags = hb.compile_flags()
    assert "--offload-arch=gfx950" in flags
    i = flags.index("-packed-fp32-ops")
    assert flags[i - 3:i + 1] == ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    # the kernels' own assembly, built here from source
    out = subprocess.run([hb.hipcc(), *flags, "--offload-device-only", "-S", "-x", "hip",
                          str(hb.CSRC / "hkv_kernels.hip"), "-o", "-"], capture_output=True, text=True, check=True)
    for op in ("add", "mul", "fma"):
        assert "v_pk_" + op + "_f32" not in out.stdout
