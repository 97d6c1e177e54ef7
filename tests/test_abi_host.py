"""Host-only checks of the C-ABI library (CPU, no GPU needed).

Every call here returns before the library touches the HIP runtime: symbol
exports, configuration checks, workspace sizing and the schedule table.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_kv_state_amd as K
from compressed_kv_state_amd import kvm as B
from kvm_inputs import WORKLOADS
from oracle.kvm_oracle import Params, schedule as oracle_schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvm_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = K.library()
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def base(**kw):
    d = dict(batch=2, heads=3, chunk=64, window=128, n_sinks=4, sched="sqrt", alpha=8, max_tokens=4096)
    d.update(kw)
    return K.KvmConfig(**d)


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(heads=0), dict(head_dim=128), dict(rope_dims=16), dict(chunk=48), dict(chunk=512),
    dict(window=100), dict(window=0), dict(n_sinks=-1), dict(n_sinks=65), dict(alpha=0),
    dict(sched="fixed", max_slots=0), dict(sched="saturating", alpha=8, max_slots=0), dict(max_tokens=0),
    dict(rope_theta=0.0), dict(ln_eps=-1.0), dict(softmax_scale=-1.0),
    dict(sched="fixed", max_slots=4, n_sinks=4),   # no non-sink row for merged tokens
    dict(sched="power", alpha=2, exponent=0.0), dict(sched="power", alpha=2, exponent=1.5),
    dict(sched="power", alpha=0, exponent=0.5),
])
def test_invalid_configs_are_rejected(bad):
    with pytest.raises(K.KvmError) as e:
        K.workspace_bytes(base(**bad))
    assert e.value.status == K.KVM_E_INVALID_ARG


def test_all_sinks_first_chunk_needs_room_in_second():
    # n_sinks == chunk: the second chunk is the first with merge candidates
    K.workspace_bytes(base(n_sinks=64, sched="fixed", max_slots=65))
    with pytest.raises(K.KvmError):
        K.workspace_bytes(base(n_sinks=64, sched="fixed", max_slots=64))


def test_unknown_flags_and_dtype_rejected():
    lib = K.library()
    c = base().to_c()
    c.flags = 32
    n = ctypes.c_size_t()
    assert lib.kvm_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == K.KVM_E_INVALID_ARG
    c.flags = B.KVM_FLAG_SERIAL_PREFILL | B.KVM_FLAG_TRACE   # known bits pass
    assert lib.kvm_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == K.KVM_OK
    c = base().to_c()
    c.dtype = 7
    assert lib.kvm_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == K.KVM_E_INVALID_ARG
    assert b"dtype" in lib.kvm_last_error()


def test_null_arguments():
    lib = K.library()
    c = base().to_c()
    assert lib.kvm_workspace_bytes(None, None) == K.KVM_E_INVALID_ARG
    assert lib.kvm_workspace_bytes(ctypes.byref(c), None) == K.KVM_E_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.kvm_state_create(ctypes.byref(c), None, 1 << 30, None, ctypes.byref(h)) == K.KVM_E_INVALID_ARG
    assert lib.kvm_prefill(None, None, None, None, None, None, 1, None) == K.KVM_E_INVALID_ARG
    assert lib.kvm_decode_step(None, None, None, None, None, None, None) == K.KVM_E_INVALID_ARG
    assert lib.kvm_state_destroy(None) == K.KVM_OK
    assert lib.kvm_status_str(3) == b"KVM_E_CAPACITY"


def test_workspace_too_small_or_misaligned():
    lib = K.library()
    c = base().to_c()
    need = K.workspace_bytes(base())
    h = ctypes.c_void_p()
    # a fake, never-dereferenced address: the size check happens before any HIP call
    assert lib.kvm_state_create(ctypes.byref(c), 1 << 20, need - 1, None, ctypes.byref(h)) == K.KVM_E_WORKSPACE
    assert lib.kvm_state_create(ctypes.byref(c), (1 << 20) + 8, need, None, ctypes.byref(h)) == K.KVM_E_WORKSPACE
    assert not h.value


def test_workspace_grows_with_tokens_and_trace():
    a = K.workspace_bytes(base(max_tokens=4096))
    b = K.workspace_bytes(base(max_tokens=8192))
    c = K.workspace_bytes(base(max_tokens=8192, trace=True))
    assert 0 < a < b < c


@pytest.mark.parametrize("wi", range(len(WORKLOADS)))
def test_schedule_table_matches_oracle(wi):
    w = WORKLOADS[wi]
    n = 600
    cfg = K.KvmConfig.of(w, max_tokens=w.n_tokens + w.decode_steps)
    sk, app, rows = K.schedule(cfg, n)
    want = oracle_schedule(n, Params.of(w))
    np.testing.assert_array_equal(sk.numpy(), [x[0] for x in want])
    np.testing.assert_array_equal(app.numpy(), [x[1] for x in want])
    np.testing.assert_array_equal(rows.numpy(), [x[2] for x in want])


def test_workload_workspace_sizes_fit_one_gpu():
    for w in WORKLOADS:
        cfg = K.KvmConfig.of(w, max_tokens=w.n_tokens + w.decode_steps)
        assert K.workspace_bytes(cfg) < 64 * 2**30


@pytest.mark.parametrize("alpha,ex", [(2, 0.6), (8, 0.5), (16, 0.33), (3, 1.0)])
def test_power_schedule_matches_oracle(alpha, ex):
    cfg = base(sched="power", alpha=alpha, exponent=ex, max_tokens=64 * 700)
    n = 600
    sk, app, rows = K.schedule(cfg, n)
    want = oracle_schedule(n, Params(chunk=64, window=128, n_sinks=4, sched="power", alpha=alpha, exponent=ex))
    np.testing.assert_array_equal(app.numpy(), [x[1] for x in want])
    np.testing.assert_array_equal(rows.numpy(), [x[2] for x in want])


def test_unprotected_sinks_can_be_the_only_merge_targets():
    # with protection a fixed state of n_sinks rows leaves merged tokens no row; unprotected sinks take them
    with pytest.raises(K.KvmError):
        K.workspace_bytes(base(sched="fixed", max_slots=4, n_sinks=4))
    K.workspace_bytes(base(sched="fixed", max_slots=4, n_sinks=4, sink_protect=False))


def test_profile_mask_bits_are_checked():
    lib = K.library()
    assert lib.kvm_profile_enable(None, 1) == K.KVM_E_INVALID_ARG
    # every defined phase bit is named in the header and the mask covers exactly them
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "kvm.h")).read()
    bits = [int(v) for v in re.findall(r"#define KVM_PROFILE_(?!ALL)\w+ (\d+)", hdr)]
    assert sorted(bits) == [1, 2, 4, 8, 16, 32]
    assert int(re.search(r"#define KVM_PROFILE_ALL (\d+)", hdr).group(1)) == sum(bits)


def test_host_library_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """kvm_api.cpp built for the host only with g++ -fsanitize=address,undefined (the kernel
    launchers replaced by do-nothing stand-ins, tests/sanitize/stub_launch.cpp), driven through
    every host-side path that needs no GPU (tests/sanitize/driver.cpp), with leak detection."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "kvm_sanitized"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "compressed_kv_state_amd", "csrc"),
           os.path.join(ROOT, "compressed_kv_state_amd", "csrc", "kvm_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "sanitized host checks: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
