"""The C ABI on the CPU: the library loads, exports every entry point that
include/kvscore.h declares, and rejects bad arguments on the host before any
HIP call (no device is touched by these tests)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvscore.h")


def _lib():
    import kv_cache_eviction_amd as kv
    if not os.path.exists(kv.LIB_PATH):
        from kv_cache_eviction_amd import build
        build.build()
    return kv, kv.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:kvs_status|size_t|int32_t|void|const char\s*\*)\s*(\w+)\s*\(",
                                 src, flags=re.M)))


def test_exports_match_header():
    kv, lib = _lib()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kv.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == names
    assert sorted(kv.EXPORTS) == names


def _desc(kv, **kw):
    base = dict(batch=1, n=1024, h_q=8, h_kv=2, d=128, d_model=1024)
    base.update(kw)
    return kv.lore_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=6, h_kv=4), 1),          # h_q not a multiple of h_kv
    (dict(h_q=34, h_kv=2), 2),         # group of 17
    (dict(d=96), 2),                   # head dim
    (dict(w=40, m=4, t=8), 2),         # 72 scoring rows
    (dict(n=20), 1),                   # n < n_sink + w
    (dict(chunk=0), 1),
    (dict(eps=float("nan")), 1),
    (dict(lambda_l=-0.5), 1),         # the lookahead weight is nonnegative
    (dict(budget=-1), 1),
    (dict(batch=32768, h_q=8, h_kv=2), 2),   # 65536 (sequence, KV head) rows
    (dict(batch=1, h_q=65536, h_kv=4096), 2),  # 65536 query heads
])
def test_bad_descriptor_rejected_before_launch(kw, status):
    kv, lib = _lib()
    d = _desc(kv, **kw)
    assert lib.kvs_lore_workspace_bytes(ctypes.byref(d)) == 0
    rc = lib.kvscore_probs(ctypes.byref(d), 1, None, None, None, None, None, None, None, None, 0, None)
    assert rc == status, kv.last_error()
    assert kv.last_error()


def test_null_pointers_and_workspace():
    kv, lib = _lib()
    d = _desc(kv)
    need = lib.kvs_lore_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.kvscore_probs(ctypes.byref(d), 1, None, None, None, None, None, None, None, None,
                             0, None) == 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    rc = lib.kvscore_probs(ctypes.byref(d), 1, fake, fake, fake, fake, fake, fake, fake, None, 16, None)
    assert rc == 3 and "workspace" in kv.last_error()
    rc = lib.kvscore_deletion(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, fake,
                              fake, fake, 16, None)
    assert rc == 1 and "omega" in kv.last_error()
    rc = lib.kvscore_topb_select(ctypes.byref(d), fake, fake, None, fake, 16, None)
    assert rc == 3
    assert lib.kv_compact(1, 1, 10, 11, 11, 128, 1, fake, fake, fake, fake, fake, None, None,
                          None, None) == 1
    assert lib.kv_compact(1, 1, 10, 5, 5, 96, 1, fake, fake, fake, fake, fake, None, None,
                          None, None) == 2
    assert lib.kv_compact(1, 1, 10, 5, 5, 128, 1, fake, fake, fake, fake, fake, None, fake,
                          None, None) == 1


def test_reliability_weights_host_checks():
    kv, lib = _lib()
    d = _desc(kv)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    f = ctypes.c_float
    big = 1 << 30
    rc = lib.kvscore_reliability_weights(ctypes.byref(d), fake, None, fake, f(1), f(1), f(0.3),
                                         fake, None, fake, big, None)
    assert rc == 1 and "NULL" in kv.last_error()
    rc = lib.kvscore_reliability_weights(ctypes.byref(d), fake, fake, fake, f(float("nan")), f(1),
                                         f(0.3), fake, None, fake, big, None)
    assert rc == 1 and "finite" in kv.last_error()
    rc = lib.kvscore_reliability_weights(ctypes.byref(d), fake, fake, fake, f(1), f(1), f(0.3),
                                         fake, None, fake, 16, None)
    assert rc == 3 and "workspace" in kv.last_error()
    odd = ctypes.c_void_p(0x1008)  # 8-byte aligned only
    rc = lib.kvscore_reliability_weights(ctypes.byref(d), odd, fake, fake, f(1), f(1), f(0.3),
                                         fake, None, fake, big, None)
    assert rc == 1 and "aligned" in kv.last_error()
    rc = lib.kvscore_probs(ctypes.byref(d), 1, fake, odd, fake, fake, fake, fake, fake, None, big, None)
    assert rc == 1 and "aligned" in kv.last_error()
    assert lib.kv_compact(1, 1, 10, 5, 5, 128, 1, fake, fake, fake, odd, fake, None, None,
                          None, None) == 1
    # no trajectories: nothing to weight, no pointer is read
    d0 = _desc(kv, m=0, t=0)
    assert lib.kvscore_reliability_weights(ctypes.byref(d0), None, None, None, f(1), f(1), f(0),
                                           None, None, None, 0, None) == 0


def test_output_fidelity_host_checks():
    kv, lib = _lib()
    d = _desc(kv)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    odd = ctypes.c_void_p(0x1008)
    assert lib.kvs_fidelity_workspace_bytes(ctypes.byref(d), 0, 10) == 0      # no queries
    assert lib.kvs_fidelity_workspace_bytes(ctypes.byref(d), 65, 10) == 0     # above 64 rows
    assert lib.kvs_fidelity_workspace_bytes(ctypes.byref(d), 8, 1025) == 0    # n_keep > n
    need = lib.kvs_fidelity_workspace_bytes(ctypes.byref(d), 8, 200)
    assert need > 0
    f = lib.kvscore_output_fidelity
    assert f(ctypes.byref(d), 8, 0, *([fake] * 7), fake, need, None) == 1
    assert f(ctypes.byref(d), 8, 200, fake, fake, fake, None, fake, fake, fake, fake, need,
             None) == 1
    assert f(ctypes.byref(d), 8, 200, fake, fake, fake, fake, odd, fake, fake, fake, need,
             None) == 1 and "aligned" in kv.last_error()
    rc = f(ctypes.byref(d), 8, 200, *([fake] * 7), fake, need - 1, None)
    assert rc == 3 and "workspace" in kv.last_error()


def test_counter_causal_and_refresh_host_checks():
    kv, lib = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    d = _desc(kv, n=5120, h_q=28, h_kv=4)
    cc = lib.kvscore_counter_causal
    assert cc(ctypes.byref(d), fake, fake, None, fake, fake, fake, None) == 1   # V missing
    assert cc(ctypes.byref(d), fake, fake, fake, fake, fake, ctypes.c_void_p(0x1008),
              None) == 1 and "aligned" in kv.last_error()
    big = _desc(kv, n=1 << 21, h_q=64, h_kv=8)  # one launch's grid would be too tall
    assert cc(ctypes.byref(big), *([fake] * 6), None) == 2
    r = lib.kvscore_refresh
    ws = lib.kvs_refresh_workspace_bytes(2, 640)
    assert ws > 0 and lib.kvs_refresh_workspace_bytes(0, 640) == 0
    args = (fake, fake, fake, None, fake, fake, fake, None, fake, ws, None)
    # J = 0 enqueues nothing and reads no pointer
    assert r(2, 4, 640, 128, 1, 16, 0, *([None] * 9), 0, None) == 0
    assert r(2, 4, 640, 128, 1, 16, 16, *args) == 1       # no room for the last token
    assert r(2, 4, 640, 96, 1, 16, 64, *args) == 2        # head dim
    assert r(2, 4, 640, 128, 1, 16, 64, *([fake] * 7), None, fake, ws,
             None) == 1                                   # ids without ids_out
    assert r(2, 4, 640, 128, 1, 16, 64, *args[:-2], ws - 1, None) == 3


def test_selection_descriptor_needs_only_selection_fields():
    kv, lib = _lib()
    d = kv.lore_desc(batch=2, n=1024, h_q=3, h_kv=3, d=128, d_model=1, w=102, m=0, t=0,
                     n_sink=0, chunk=1, budget=102)
    assert lib.kvs_lore_workspace_bytes(ctypes.byref(d)) == 0     # not a scoring descriptor
    # chunk keys + per-segment candidate lists (one int per chunk each) + one
    # count per 1024-chunk segment, each region 256-byte aligned
    rows, nchunks = 2 * 3, 1024
    assert lib.kvs_topb_workspace_bytes(ctypes.byref(d)) == 2 * rows * nchunks * 4 + 256


def test_h2o_descriptor_checks():
    kv, lib = _lib()
    d = kv.h2o_desc(batch=2, heads=3, d=128, cap=16385)      # prompt above 16384
    assert lib.kvs_h2o_workspace_bytes(ctypes.byref(d), kv.KVS_H2O_PREFILL) == 0
    d = kv.h2o_desc(batch=1, heads=1100, d=128, cap=16384)   # grid: 1100 * 64 workgroups
    assert lib.kvs_h2o_workspace_bytes(ctypes.byref(d), kv.KVS_H2O_PREFILL) == 0
    d = kv.h2o_desc(batch=2, heads=3, d=128, cap=16384)
    assert lib.kvs_h2o_workspace_bytes(ctypes.byref(d), kv.KVS_H2O_PREFILL) > 0
    d = kv.h2o_desc(batch=2, heads=3, d=128, cap=1024)
    assert lib.kvs_h2o_workspace_bytes(ctypes.byref(d), kv.KVS_H2O_PREFILL) > 0
    rc = lib.kvscore_h2o_accumulate(ctypes.byref(d), 7, None, None, None, None, None, None,
                                    None, None, None, None, None, 0, None)
    assert rc == 1
    d = kv.h2o_desc(batch=2, heads=3, d=128, cap=300, cur_len=0)
    rc = lib.kvscore_h2o_accumulate(ctypes.byref(d), kv.KVS_H2O_DECODE, None, None, None, None,
                                    None, None, None, None, None, None, None, 0, None)
    assert rc == 1


def test_binding_checks_shapes_before_calling():
    kv, _ = _lib()
    import torch
    d = _desc(kv)
    with pytest.raises(kv.KvsError):
        kv.kvscore_probs(d, torch.zeros(1), None, None, None, None, None, None)


def test_retention_shift_and_noalloc_host_checks():
    """Bad sizes and NULL pointers are refused on the host (no device touched)."""
    kv, lib = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    assert lib.kvscore_retention_shift(0, 5, 10, 1, 2, fake, fake, fake, None) == 1
    assert lib.kvscore_retention_shift(2, 11, 10, 1, 2, fake, fake, fake, None) == 1   # n_keep > n
    assert lib.kvscore_retention_shift(2, 5, 10, 6, 5, fake, fake, fake, None) == 1    # n_sink + w > n
    assert lib.kvscore_retention_shift(2, 5, 10, 1, 2, None, fake, fake, None) == 1
    d = kv.lore_desc(batch=64, n=1 << 20, h_q=8, h_kv=8, d=128, d_model=1, w=32, m=0, t=0,
                     n_sink=1, chunk=1, budget=128)
    assert lib.kvscore_topb_select_noalloc(ctypes.byref(d), fake, fake, None, None) == 2
    assert "maximum" in kv.last_error()


def test_probs_mask_checks():
    """kvscore_probs takes the window-causal or no mask; the causal and slot
    masks belong to kvscore_h2o_accumulate (unsupported here), others are invalid."""
    kv, lib = _lib()
    d = _desc(kv)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the mask check fails first
    for mask, status in ((kv.KVS_MASK_CAUSAL, 2), (kv.KVS_MASK_SLOTS, 2), (9, 1), (-1, 1)):
        rc = lib.kvscore_probs(ctypes.byref(d), mask, fake, fake, fake, fake, fake, fake, fake, None,
                               0, None)
        assert rc == status, (mask, kv.last_error())


def test_row_limits_of_one_launch():
    """Sequences x heads index one grid dimension (at most 65535 workgroups):
    every entry point refuses more before enqueueing anything, and accepts
    the largest count."""
    kv, lib = _lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: a host check fails first
    over = kv.lore_desc(batch=16384, n=1024, h_q=4, h_kv=4, d=128, d_model=1)   # 65536 rows
    edge = kv.lore_desc(batch=16383, n=1024, h_q=4, h_kv=4, d=128, d_model=1)   # 65532 rows
    assert lib.kvs_topb_workspace_bytes(ctypes.byref(over)) == 0
    assert "65535" in kv.last_error()
    assert lib.kvs_topb_workspace_bytes(ctypes.byref(edge)) > 0
    assert lib.kvscore_topb_select(ctypes.byref(over), fake, fake, None, fake, 1 << 40, None) == 2
    assert lib.kvs_fidelity_workspace_bytes(ctypes.byref(over), 8, 100) == 0
    assert lib.kvscore_counter_causal(ctypes.byref(over), *([fake] * 6), None) == 2
    assert lib.kv_compact(256, 256, 10, 5, 5, 128, 1, fake, fake, fake, fake, fake, None, None,
                          None, None) == 2
    assert lib.kvscore_refresh(256, 256, 640, 128, 1, 16, 64, fake, fake, fake, None, fake, fake,
                               fake, None, fake, 1 << 40, None) == 2
    h = kv.h2o_desc(batch=256, heads=256, d=128, cap=300, cur_len=10)
    assert lib.kvs_h2o_workspace_bytes(ctypes.byref(h), kv.KVS_H2O_PREFILL) == 0
    rc = lib.kvscore_h2o_accumulate(ctypes.byref(h), kv.KVS_H2O_DECODE, *([fake] * 10), None, 0,
                                    None)
    assert rc == 2 and "65535" in kv.last_error()


def test_header_is_plain_c(tmp_path):
    """include/kvscore.h is a C header: it compiles as C11 and as C++17 with
    every warning an error, and each declared entry point can be named from
    C (compile only; nothing is linked)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc = os.path.join(root, "include")
    hdr = open(os.path.join(inc, "kvscore.h")).read()
    names = sorted(set(re.findall(r"\b(kvs_\w+|kvscore_\w+|kv_compact)\(", hdr)))
    assert "kvscore_deletion" in names and "kv_compact" in names
    body = "\n".join("  (void)&%s;" % n for n in names)
    src = tmp_path / "use.c"
    src.write_text('#include "kvscore.h"\nint main(void) {\n%s\n  return 0;\n}\n' % body)
    for cmd in (["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only"],
                ["g++", "-x", "c++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsyntax-only"]):
        r = subprocess.run(cmd + ["-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
