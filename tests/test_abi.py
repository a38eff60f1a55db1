"""The C-ABI library: it loads without a GPU, exports every symbol the
header declares, and its host-side validation returns the documented typed
errors before touching the device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import causal_gqa_flashattention_amd as fa
    if not os.path.exists(fa.lib_path()):
        pytest.skip("library not built (run __graft_entry__.build())")
    return fa.load_library()


@pytest.fixture(scope="module")
def vlib(lib):
    """The library for validation tests that pass fake device pointers (P
    below).  Every such call must fail on the host before any launch; in a
    process that sees a GPU a regressed check would launch a kernel on an
    unmapped address instead, so these tests run only where no device is
    visible (the unmarked CPU suite)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-pointer validation tests run only without a visible GPU")
    return lib


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("fa_fwd", "fa_bwd_delta", "fa_bwd", "fa_bwd_dq", "fa_bwd_dkv", "fa_status_str", "fa_version",
              "fa_fwd_block_sparse", "fa_bwd_block_sparse", "fa_bwd_dq_block_sparse",
              "fa_bwd_dkv_block_sparse"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(12):
        assert lib.fa_status_str(s)
    assert b"Lq <= Lk" in lib.fa_status_str(6)


P = 4096  # a fake, 16-byte aligned pointer value: validation never dereferences


@pytest.mark.parametrize("args,status", [
    # q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal
    ((P, P, P, P, P, 1, 2, 1, 8, 8, 48, 0.1, 1), 4),     # head dim
    ((P, P, P, P, P, 1, 3, 2, 8, 8, 64, 0.1, 1), 5),     # Hq % Hkv
    ((P, P, P, P, P, 1, 2, 0, 8, 8, 64, 0.1, 1), 5),     # Hkv == 0
    ((P, P, P, P, P, 1, 2, 1, 9, 8, 64, 0.1, 1), 6),     # causal Lq > Lk
    ((P, P, P, P, P, 1, 2, 1, 8, 0, 64, 0.1, 0), 3),     # no keys
    ((P, P, P, P, P, -1, 2, 1, 8, 8, 64, 0.1, 0), 3),    # negative size
    ((P, P, P, P, P, 1, 2, 1, 8, 8, 64, float("nan"), 0), 7),
    ((P, P, P, P, P, 1, 2, 1, 8, 8, 64, -1.0, 0), 7),
    ((0, P, P, P, P, 1, 2, 1, 8, 8, 64, 0.1, 1), 1),     # null q
    ((P, P, P + 2, P, P, 1, 2, 1, 8, 8, 64, 0.1, 1), 2), # misaligned v
    ((P, P, P, P, P, 65536, 65536, 1, 65536, 65536, 256, 0.1, 0), 3),  # int64 overflow
])
def test_fwd_validation(vlib, args, status):
    assert vlib.fa_fwd(*args, None) == status


def test_empty_forward_is_ok_without_pointers(vlib):
    assert vlib.fa_fwd(0, 0, 0, 0, 0, 0, 2, 1, 8, 8, 64, 0.1, 1, None) == 0
    assert vlib.fa_fwd(0, 0, 0, 0, 0, 1, 2, 1, 0, 8, 64, 0.1, 1, None) == 0


def test_bwd_validation(vlib):
    a = [P] * 10
    assert vlib.fa_bwd(*a, 1, 2, 1, 8, 8, 80, 0.1, 1, None) == 4    # unsupported head dim
    assert vlib.fa_bwd(*a, 1, 4, 3, 8, 8, 64, 0.1, 1, None) == 5
    assert vlib.fa_bwd(*a, 1, 2, 1, 9, 8, 64, 0.1, 1, None) == 6
    bad = list(a)
    bad[7] = 0  # dq NULL
    assert vlib.fa_bwd(*bad, 1, 2, 1, 8, 8, 64, 0.1, 1, None) == 1
    # the dK/dV half does not need dq
    assert vlib.fa_bwd_dq(P, P, P, P, P, P, 0, 1, 2, 1, 8, 8, 64, 0.1, 1, None) == 1
    assert vlib.fa_bwd_dkv(P, P, P, P, P, P, 0, P, 1, 2, 1, 8, 8, 64, 0.1, 1, None) == 1
    assert vlib.fa_bwd_delta(P, P, P, 1, 2, 8, 80, None) == 4
    assert vlib.fa_bwd_delta(P, 0, P, 1, 2, 8, 64, None) == 1
    assert vlib.fa_bwd_delta(0, 0, 0, 1, 2, 0, 64, None) == 0


@pytest.mark.parametrize("args,status", [
    ((P, P, P, P, P, 1, 2, 1, 8, 8, 48, 0.1, 1), 4),
    ((P, P, P, P, P, 1, 3, 2, 8, 8, 64, 0.1, 1), 5),
    ((P, P, P, P, P, 1, 2, 1, 9, 8, 64, 0.1, 1), 6),
    ((0, P, P, P, P, 1, 2, 1, 8, 8, 64, 0.1, 1), 1),
    ((P, P, P + 2, P, P, 1, 2, 1, 8, 8, 64, 0.1, 1), 2),
])
def test_block_sparse_validation_matches_dense(vlib, args, status):
    # the mask pointer (here a fake one, or NULL) changes none of the checks
    for m in (None, P + 1):
        assert vlib.fa_fwd_block_sparse(*args, m, None) == status
    a = list(args[:3]) + [P] * 7
    if args[0] == 0:
        a[0] = 0
    if args[2] == P + 2:
        a[2] = P + 2
    tail = list(args[5:])
    assert vlib.fa_bwd_block_sparse(*a, *tail, P + 1, None) == status
    assert vlib.fa_bwd_dq_block_sparse(*a[:7], *tail, P + 1, None) == status
    assert vlib.fa_bwd_dkv_block_sparse(*a[:8], *tail, P + 1, None) == status


def test_block_sparse_empty_is_ok(vlib):
    assert vlib.fa_fwd_block_sparse(0, 0, 0, 0, 0, 0, 2, 1, 8, 8, 64, 0.1, 1, 0, None) == 0
    assert vlib.fa_bwd_block_sparse(*([0] * 10), 0, 2, 1, 8, 8, 64, 0.1, 1, 0, None) == 0


def test_block_sparse_length_limit(vlib):
    # tile lists live in LDS: Lq, Lk <= FA_MASK_MAX_LEN under a mask (plain calls are not limited)
    big = 262144 + 64
    assert vlib.fa_fwd_block_sparse(P, P, P, P, P, 1, 1, 1, big, big, 128, 0.1, 1, P, None) == 3
    assert vlib.fa_bwd_block_sparse(*([P] * 10), 1, 1, 1, 64, big, 128, 0.1, 1, P, None) == 3


# ---------------------------------------------------------------- general calls

def _t(lib, data, sb, sh, sl):
    import causal_gqa_flashattention_amd as fa
    return fa.FaTensor(data, sb, sh, sl)


def _dense(lib, H, L, D, data=P):
    return _t(lib, data, H * L * D, L * D, D)


def test_ex_symbols_and_status_strings(lib):
    assert b"stride" in lib.fa_status_str(9)
    assert b"element type" in lib.fa_status_str(10)


@pytest.mark.parametrize("q_strides,o_strides,status", [
    ((2 * 128 * 64, 128 * 64, 60), (2 * 128 * 64, 128 * 64, 64), 9),    # row stride not a multiple of 8
    ((2 * 128 * 64, -128 * 64, 64), (2 * 128 * 64, 128 * 64, 64), 9),   # negative head stride
    ((2 * 128 * 64, 128 * 64, 1 << 24), (2 * 128 * 64, 128 * 64, 64), 9),  # row stride too large
    ((2 * 128 * 64, 128 * 64, 64), (2 * 128 * 64, 128 * 64, 32), 9),    # output rows overlap
    ((2 * 128 * 64, 128 * 64, 64), (2 * 128 * 64, 8, 128), 9),          # output heads overlap
    ((2 * 128 * 64, 128 * 64, 64), (2 * 128 * 64, 64, 64), 9),          # heads and rows collide
    ((2 * 128 * 64, 128 * 64, 64), (128 * 64, 128 * 64, 64), 9),       # batches overlap heads
])
def test_fwd_ex_stride_validation(vlib, q_strides, o_strides, status):
    # B=2, Hq=2, Hkv=1, Lq=Lk=128, D=64
    q = _t(vlib, P, *q_strides)
    kv = _dense(vlib, 1, 128, 64)
    o = _t(vlib, P, *o_strides)
    assert vlib.fa_fwd_ex(q, kv, kv, o, P, 2, 2, 1, 128, 128, 64, 0.1, 1, 0, None, None) == status


def test_ex_dtype_and_empty(vlib):
    q = _dense(vlib, 2, 128, 64)
    kv = _dense(vlib, 1, 128, 64)
    assert vlib.fa_fwd_ex(q, kv, kv, q, P, 1, 2, 1, 128, 128, 64, 0.1, 1, 2, None, None) == 10
    assert vlib.fa_bwd_delta_ex(q, q, P, 1, 2, 128, 64, 7, None) == 10
    z = _t(vlib, None, 0, 0, 0)
    assert vlib.fa_fwd_ex(z, z, z, z, None, 0, 2, 1, 128, 128, 64, 0.1, 1, 1, None, None) == 0
    assert vlib.fa_bwd_ex(z, z, z, None, None, z, z, z, z, 0, 2, 1, 8, 8, 64, 0.1, 1, 1, None, 3, None) == 0
    # no gradient asked for: nothing to do
    assert vlib.fa_bwd_ex(z, z, z, None, None, z, z, z, z, 1, 2, 1, 8, 8, 64, 0.1, 1, 0, None, 0, None) == 0


def test_bwd_ex_validation(vlib):
    q = _dense(vlib, 2, 128, 64)
    kv = _dense(vlib, 1, 128, 64)
    z = _t(vlib, None, 0, 0, 0)
    bad = _t(vlib, P, 2 * 128 * 64, 128 * 64, 32)  # rows overlap
    # dq only: the dK/dV tensors may be NULL; an overlapping dq is refused
    assert vlib.fa_bwd_ex(q, kv, kv, P, P, q, bad, z, z, 1, 2, 1, 128, 128, 64, 0.1, 1, 0, None, 1, None) == 9
    # dK/dV only: dq may be NULL, dk must be given
    assert vlib.fa_bwd_ex(q, kv, kv, P, P, q, z, z, kv, 1, 2, 1, 128, 128, 64, 0.1, 1, 0, None, 2, None) == 1
    # an overlapping dv (stride 0 rows) is refused, a stride-0 input is not looked at as an output
    zero_rows = _t(vlib, P, 128 * 64, 128 * 64, 0)
    assert vlib.fa_bwd_ex(q, kv, kv, P, P, q, z, kv, zero_rows, 1, 2, 1, 128, 128, 64, 0.1, 1, 0, None, 2,
                         None) == 9
    # misaligned data pointer in a strided view
    mis = _t(vlib, P + 8, 2 * 128 * 64, 128 * 64, 64)
    assert vlib.fa_bwd_ex(mis, kv, kv, P, P, q, q, kv, kv, 1, 2, 1, 128, 128, 64, 0.1, 1, 0, None, 3, None) == 2


# ---------------------------------------------------------------- short queries

def test_short_workspace_bytes(lib):
    f = lib.fa_short_workspace_bytes
    f.restype = ctypes.c_size_t
    assert f(1, 32, 8, 9, 1000, 128) == 0          # Lq above the short limit
    assert f(1, 32, 8, 1, 1000, 80) == 0           # head dim
    assert f(1, 6, 4, 1, 1000, 128) == 0           # Hq % Hkv
    assert f(0, 32, 8, 1, 1000, 128) == 0          # empty
    a = f(1, 32, 8, 1, 32768, 128)
    assert a > 0 and a % 16 == 0
    assert f(1, 32, 8, 8, 32768, 128) >= a          # more rows, more partials
    assert f(1, 32, 8, 1, 32768, 256) >= a


def test_short_validation(vlib):
    q = _dense(vlib, 4, 1, 64)
    kv = _dense(vlib, 1, 256, 64)
    ws_bytes = vlib.fa_short_workspace_bytes(1, 4, 1, 1, 256, 64)
    assert vlib.fa_fwd_short(q, kv, kv, q, P, 1, 4, 1, 9, 256, 64, 0.1, 1, 0, P, 1 << 30, None) == 3
    assert vlib.fa_fwd_short(q, kv, kv, q, P, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, None, 1 << 30, None) == 1
    assert vlib.fa_fwd_short(q, kv, kv, q, P, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, P + 4, 1 << 30, None) == 2
    assert vlib.fa_fwd_short(q, kv, kv, q, P, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, P, ws_bytes - 16, None) == 11
    assert vlib.fa_fwd_short(q, kv, kv, q, P, 1, 4, 1, 1, 256, 64, 0.1, 1, 3, P, 1 << 30, None) == 10
    z = _t(vlib, None, 0, 0, 0)
    assert vlib.fa_fwd_short(z, z, z, z, None, 0, 4, 1, 1, 256, 64, 0.1, 1, 0, None, 0, None) == 0
    # dq needs the workspace; dK/dV alone does not (the misaligned dk is what fails)
    mis = _t(vlib, P + 8, 256 * 64, 256 * 64, 64)
    assert vlib.fa_bwd_short(q, kv, kv, P, P, q, q, z, z, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, 1, None, 0, None) == 1
    assert vlib.fa_bwd_short(q, kv, kv, P, P, q, q, z, z, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, 1, P, 64, None) == 11
    assert vlib.fa_bwd_short(q, kv, kv, P, P, q, z, mis, kv, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, 2, None, 0,
                            None) == 2
    # a failing dq check launches nothing, not even the dK/dV half
    assert vlib.fa_bwd_short(q, kv, kv, P, P, q, q, kv, kv, 1, 4, 1, 1, 256, 64, 0.1, 1, 0, 3, None, 0,
                            None) == 1


def test_short_noalloc_validation(vlib):
    q = _dense(vlib, 4, 1, 64)
    kv = _dense(vlib, 1, 4096, 64)
    f = vlib.fa_fwd_short_noalloc
    # the checks of fa_fwd_short
    assert f(q, kv, kv, q, P, 1, 4, 1, 1, 4096, 80, 0.1, 1, 0, None) == 4   # head dim
    assert f(q, kv, kv, q, P, 1, 4, 1, 9, 4096, 64, 0.1, 1, 0, None) == 3   # Lq above the short limit
    assert f(q, kv, kv, q, 0, 1, 4, 1, 1, 4096, 64, 0.1, 1, 0, None) == 1   # lse NULL
    assert f(q, kv, kv, q, P, 1, 4, 1, 1, 4096, 64, 0.1, 1, 3, None) == 10  # element type
    # a shape whose partials exceed the static scratch: refused before launch
    big_q = _dense(vlib, 32, 8, 256)
    big_kv = _dense(vlib, 8, 4096, 256)
    ws = vlib.fa_short_workspace_bytes
    ws.restype = ctypes.c_size_t
    assert ws(128, 32, 8, 8, 4096, 256) > (64 << 20)
    assert f(big_q, big_kv, big_kv, big_q, P, 128, 32, 8, 8, 4096, 256, 0.1, 1, 0, None) == 11


def test_bwd_workspace_plan(lib):
    f = lib.fa_bwd_workspace_bytes
    f.restype = ctypes.c_size_t
    assert f(1, 32, 8, 8192, 8192, 128, 0) == 0        # two rounds of key-tile workgroups: no split
    assert f(1, 32, 8, 8192, 8192, 128, 1) > 0         # a mask may hold a sink column
    assert f(1, 16, 2, 8192, 8192, 256, 0) > 0         # one round at head dim 256: split
    assert f(1, 16, 2, 8192, 8192, 256, 0) % 16 == 0
    assert f(1, 4, 1, 60, 60, 128, 0) == 0             # one query tile: nothing to split
    assert f(1, 6, 4, 100, 100, 128, 0) == 0           # Hq % Hkv


def test_bwd_ws_validation(vlib):
    q = _dense(vlib, 16, 8192, 256)
    kv = _dense(vlib, 2, 8192, 256)
    f = vlib.fa_bwd_ws
    args = (q, kv, kv, P, P, q, q, kv, kv, 1, 16, 2, 8192, 8192, 256, 0.1, 1, 0, None, 3)
    assert f(*args, None, 0, None) == 1                 # split planned, no workspace
    assert f(*args, P, 1024, None) == 11                # too small
    assert f(*args, P + 8, 1 << 30, None) == 2          # misaligned
