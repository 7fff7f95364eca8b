"""The C ABI on the CPU: exports, struct layout, and every error path.

Sessions here use validate_only, in which the library makes no HIP call: each
collective runs the full argument checks and returns without launching.
Pointers are fake addresses that are never dereferenced.
"""

import ctypes
import re
import subprocess
from pathlib import Path

import pytest

import rank_reductions_amd as rr

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "rc.h"

OK = rr.RC_OK
NR = rr.RC_ERR_NOT_REGISTERED
DUP = rr.RC_ERR_DUPLICATE_REGISTRATION
SHAPE = rr.RC_ERR_SHAPE_MISMATCH
OPM = rr.RC_ERR_OP_MISMATCH
ROOT_M = rr.RC_ERR_ROOT_MISMATCH
SENDERS = rr.RC_ERR_BROADCAST_SENDERS
DTYPE = rr.RC_ERR_DTYPE_MISMATCH
INVAL = rr.RC_ERR_INVALID_ARGUMENT

MiB = 1 << 20


@pytest.fixture
def lib():
    lib = rr.library()
    lib.rc_reset()
    yield lib
    lib.rc_reset()


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rc_\w+)\s*\(", text, re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    for want in ("rc_register", "rc_all_reduce", "rc_reduce", "rc_broadcast", "rc_reduce_scatter",
                 "rc_all_gather", "rc_all_reduce_many", "rc_finish", "rc_reset", "rc_last_error",
                 "rc_status_name", "rc_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in rc.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", str(rr.library_path())], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (rc_\w+)", out))
    assert set(declared_functions()) <= exported
    header = re.search(r"#define RC_ABI_VERSION (\d+)", (ROOT / "include" / "rc.h").read_text())
    assert lib.rc_abi_version() == int(header.group(1)) == rr.RC_ABI_VERSION == 3


def test_struct_layout_matches_a_c_compiler(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "rc.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\","
        "sizeof(rc_buf), offsetof(rc_buf, recv), offsetof(rc_buf, dtype), offsetof(rc_buf, root),"
        "offsetof(rc_buf, dims), sizeof(rc_config), offsetof(rc_config, algo),"
        "offsetof(rc_config, tile_elems), offsetof(rc_config, max_workgroups),"
        "offsetof(rc_config, waves_per_cu), sizeof(rc_param), offsetof(rc_param, acc),"
        "offsetof(rc_param, buf));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(rr.RcBuf), rr.RcBuf.recv.offset, rr.RcBuf.dtype.offset, rr.RcBuf.root.offset,
            rr.RcBuf.dims.offset, ctypes.sizeof(rr.RcConfig), rr.RcConfig.algo.offset,
            rr.RcConfig.tile_elems.offset, rr.RcConfig.max_workgroups.offset, rr.RcConfig.waves_per_cu.offset,
            ctypes.sizeof(rr.RcParam), rr.RcParam.acc.offset, rr.RcParam.buf.offset]
    assert got == want


def test_status_names(lib):
    names = {c: lib.rc_status_name(c).decode() for c in range(11)}
    assert names[0] == "RC_OK"
    assert names[3] == "RC_ERR_SHAPE_MISMATCH"
    assert names[6] == "RC_ERR_BROADCAST_SENDERS"
    assert names[10] == "RC_ERR_PARAM_MISMATCH"
    assert lib.rc_status_name(99).decode() == "RC_UNKNOWN_STATUS"


# ------------------------------------------------------------------ helpers

def reg(lib, R, **kw):
    cfg = rr.make_config(validate_only=True, **kw)
    return lib.rc_register(R, ctypes.byref(cfg))


def bufs(sends, recvs, shape=(257,), dtype=rr.RC_F32, op=rr.RC_SUM, root=0):
    return rr.make_bufs(sends, recvs, shape, dtype, op, root)


def call(lib, name, b):
    return getattr(lib, name)(ctypes.cast(b, ctypes.c_void_p), None)


def addrs(R, base=0x10000000, stride=4 * MiB):
    return [base + r * stride for r in range(R)]


def ar_bufs(R=4, n=257, **kw):
    return bufs(addrs(R), addrs(R, base=0x80000000), (n,), **kw)


# ------------------------------------------------------------------ lifecycle

def test_not_registered(lib):
    for name in ("rc_all_reduce", "rc_reduce", "rc_broadcast", "rc_reduce_scatter", "rc_all_gather"):
        assert call(lib, name, ar_bufs()) == NR
        assert lib.rc_last_error()
    assert lib.rc_all_reduce_many(1, ctypes.cast(ar_bufs(), ctypes.c_void_p), None) == NR
    assert lib.rc_finish() == NR


def test_register_finish_reset_cycle(lib):
    assert reg(lib, 4) == OK
    assert lib.rc_last_error() == b""
    assert reg(lib, 4) == DUP
    assert b"already open" in lib.rc_last_error()
    assert call(lib, "rc_all_reduce", ar_bufs()) == OK
    assert lib.rc_finish() == OK
    assert lib.rc_finish() == NR
    assert call(lib, "rc_all_reduce", ar_bufs()) == NR
    assert reg(lib, 2) == OK
    assert lib.rc_reset() == OK
    assert lib.rc_reset() == OK  # from any state
    assert call(lib, "rc_all_reduce", ar_bufs(2)) == NR
    assert reg(lib, 2) == OK


def test_register_arguments(lib):
    assert lib.rc_register(0, None) == INVAL
    assert lib.rc_register(17, None) == INVAL
    cfg = rr.make_config(validate_only=True)
    cfg.struct_size = 8
    assert lib.rc_register(4, ctypes.byref(cfg)) == INVAL
    for field, bad in (("algo", 3), ("cache_hint", 7), ("tile_elems", 1000), ("tile_elems", 131072),
                       ("max_workgroups", -1), ("device", -2), ("waves_per_cu", 33), ("waves_per_cu", -1),
                       ("reserved", 1)):
        cfg = rr.make_config(validate_only=True)
        setattr(cfg, field, bad)
        assert lib.rc_register(4, ctypes.byref(cfg)) == INVAL, field
    assert reg(lib, 16, algo="ring", tile_elems=8192, max_workgroups=3, cache_hint="normal", waves_per_cu=6) == OK


def test_failed_call_leaves_session_usable(lib):
    assert reg(lib, 4) == OK
    assert call(lib, "rc_all_reduce", bufs(addrs(4), addrs(4, 0x80000000), [(257,), (257,), (256,), (257,)])) == SHAPE
    assert b"rank 2" in lib.rc_last_error()
    assert call(lib, "rc_all_reduce", ar_bufs()) == OK
    assert lib.rc_last_error() == b""


# ------------------------------------------------------------------ CollectiveError cases

def test_shape_mismatch(lib):
    reg(lib, 4)
    assert call(lib, "rc_all_reduce", bufs(addrs(4), addrs(4, 0x80000000), [(16, 16)] * 3 + [(256,)])) == SHAPE
    assert call(lib, "rc_reduce", bufs(addrs(4), addrs(4, 0x80000000), [(8,)] * 3 + [(9,)])) == SHAPE
    # reduce_scatter: count not divisible by R
    assert call(lib, "rc_reduce_scatter", bufs(addrs(4), addrs(4, 0x80000000), (258,))) == SHAPE
    assert call(lib, "rc_reduce_scatter", bufs(addrs(4), addrs(4, 0x80000000), (256,))) == OK


def test_op_mismatch_and_i32_mean(lib):
    reg(lib, 3)
    assert call(lib, "rc_all_reduce", bufs(addrs(3), addrs(3, 0x80000000), op=[0, 0, 1])) == OPM
    assert call(lib, "rc_reduce_scatter", bufs(addrs(3), addrs(3, 0x80000000), (9,), op=[2, 0, 2])) == OPM
    assert call(lib, "rc_all_reduce", bufs(addrs(3), addrs(3, 0x80000000), dtype=rr.RC_I32, op=rr.RC_MEAN)) == INVAL
    assert call(lib, "rc_all_reduce", bufs(addrs(3), addrs(3, 0x80000000), dtype=rr.RC_I32, op=rr.RC_MAX)) == OK
    # ops are ignored by broadcast and all_gather
    assert call(lib, "rc_all_gather", bufs(addrs(3), addrs(3, 0x80000000), op=[0, 1, 2])) == OK


def test_dtype_mismatch(lib):
    reg(lib, 2)
    assert call(lib, "rc_all_reduce", bufs(addrs(2), addrs(2, 0x80000000), dtype=[0, 1])) == DTYPE
    assert call(lib, "rc_all_reduce", bufs(addrs(2), addrs(2, 0x80000000), dtype=[0, 5])) == INVAL


def test_root_mismatch_and_range(lib):
    reg(lib, 4)
    s, r = addrs(4), addrs(4, 0x80000000)
    assert call(lib, "rc_reduce", bufs(s, r, root=[1, 1, 2, 1])) == ROOT_M
    assert call(lib, "rc_reduce", bufs(s, r, root=4)) == INVAL
    assert call(lib, "rc_reduce", bufs(s, r, root=-1)) == INVAL
    assert call(lib, "rc_reduce", bufs(s, [None, None, r[2], None], root=2)) == OK
    assert call(lib, "rc_reduce", bufs(s, [r[0], None, None, None], root=2)) == INVAL
    sends = [None, None, s[2], None]
    assert call(lib, "rc_broadcast", bufs(sends, r, root=[-1, -1, 2, -1])) == ROOT_M
    assert call(lib, "rc_broadcast", bufs(sends, r, root=1)) == ROOT_M   # not the sender
    assert call(lib, "rc_broadcast", bufs(sends, r, root=2)) == OK
    assert call(lib, "rc_broadcast", bufs(sends, r, root=-1)) == OK
    assert call(lib, "rc_broadcast", bufs(sends, r, root=5)) == INVAL


def test_broadcast_sender_count(lib):
    reg(lib, 4)
    r = addrs(4, 0x80000000)
    assert call(lib, "rc_broadcast", bufs([None] * 4, r, root=-1)) == SENDERS
    assert call(lib, "rc_broadcast", bufs([0x1000, None, 0x2000, None], r, root=-1)) == SENDERS
    assert call(lib, "rc_broadcast", bufs([0x1000, None, None, None], [None, r[1], r[2], r[3]], root=-1)) == OK
    assert call(lib, "rc_broadcast", bufs([0x1000, None, None, None], [None, None, r[2], r[3]], root=-1)) == INVAL


def test_check_order(lib):
    """dtype before shape before op before root (documented order)."""
    reg(lib, 2)
    s, r = addrs(2), addrs(2, 0x80000000)
    assert call(lib, "rc_reduce", bufs(s, r, [(4,), (5,)], dtype=[0, 1], op=[0, 1], root=[0, 1])) == DTYPE
    assert call(lib, "rc_reduce", bufs(s, r, [(4,), (5,)], op=[0, 1], root=[0, 1])) == SHAPE
    assert call(lib, "rc_reduce", bufs(s, r, (4,), op=[0, 1], root=[0, 1])) == OPM
    assert call(lib, "rc_reduce", bufs(s, r, (4,), root=[0, 1])) == ROOT_M
    # malformed fields come first of all
    assert call(lib, "rc_reduce", bufs([None, s[1]], r, [(4,), (5,)], dtype=[0, 1])) == INVAL


def test_invalid_fields(lib):
    reg(lib, 2)
    s, r = addrs(2), addrs(2, 0x80000000)
    assert lib.rc_all_reduce(None, None) == INVAL
    assert call(lib, "rc_all_reduce", bufs([s[0], None], r)) == INVAL
    assert call(lib, "rc_all_reduce", bufs(s, [r[0], None])) == INVAL
    assert call(lib, "rc_all_reduce", bufs([s[0] + 2, s[1]], r)) == INVAL   # not 4-byte aligned
    assert call(lib, "rc_all_reduce", bufs(s, r, op=7)) == INVAL
    b = bufs(s, r)
    b[1].ndim = 9
    assert call(lib, "rc_all_reduce", b) == INVAL
    b = bufs(s, r, (4, 4))
    b[0].dims[1] = -4
    assert call(lib, "rc_all_reduce", b) == INVAL
    b = bufs(s, r, (1 << 30, 1 << 30))
    assert call(lib, "rc_all_reduce", b) == INVAL   # count too large


def test_zero_elements_accept_null(lib):
    reg(lib, 3)
    assert call(lib, "rc_all_reduce", bufs([None] * 3, [None] * 3, (0,))) == OK
    assert call(lib, "rc_all_reduce", bufs([None] * 3, [None] * 3, (4, 0, 2))) == OK
    assert call(lib, "rc_reduce_scatter", bufs([None] * 3, [None] * 3, (0,))) == OK
    assert call(lib, "rc_broadcast", bufs([None, 256, None], [None] * 3, (0,), root=-1)) == OK


def test_scalar_shape(lib):
    reg(lib, 2)
    assert call(lib, "rc_all_reduce", bufs(addrs(2), addrs(2, 0x80000000), ())) == OK


# ------------------------------------------------------------------ in place and overlap

def test_in_place_forms_allowed(lib):
    R, n = 4, 1024
    reg(lib, R)
    s = addrs(R)
    assert call(lib, "rc_all_reduce", bufs(s, s, (n,))) == OK
    assert call(lib, "rc_reduce", bufs(s, [None, s[1], None, None], (n,), root=1)) == OK
    sends = [None, None, s[2], None]
    assert call(lib, "rc_broadcast", bufs(sends, [s[0], s[1], s[2], s[3]], (n,), root=-1)) == OK
    m = n // R
    assert call(lib, "rc_reduce_scatter", bufs(s, [s[r] + r * m * 4 for r in range(R)], (n,))) == OK
    assert call(lib, "rc_all_gather", bufs([s[r] + r * m * 4 for r in range(R)], s, (m,))) == OK


def test_overlaps_rejected(lib):
    R, n = 4, 1024
    reg(lib, R)
    s = addrs(R)
    r = addrs(R, 0x80000000)
    # an output overlapping another rank's input
    bad = list(r)
    bad[0] = s[1] + 64
    assert call(lib, "rc_all_reduce", bufs(s, bad, (n,))) == INVAL
    # two outputs overlapping
    bad = list(r)
    bad[2] = r[1] + 8
    assert call(lib, "rc_all_reduce", bufs(s, bad, (n,))) == INVAL
    # in place shifted by one element
    assert call(lib, "rc_all_reduce", bufs(s, [x + 4 for x in s], (n,))) == INVAL
    # reduce_scatter: output inside the input, but not at the rank's own shard
    m = n // R
    assert call(lib, "rc_reduce_scatter", bufs(s, [s[r] + ((r + 1) % R) * m * 4 for r in range(R)], (n,))) == INVAL
    # all_gather: shard inside the output at another rank's place
    assert call(lib, "rc_all_gather", bufs([s[r] + ((r + 1) % R) * m * 4 for r in range(R)], s, (m,))) == INVAL
    # inputs may overlap each other freely
    assert call(lib, "rc_all_reduce", bufs([s[0]] * R, r, (n,))) == OK


# ------------------------------------------------------------------ batched

def many(lib, rows, R):
    flat = (rr.RcBuf * (len(rows) * R))()
    k = 0
    for row in rows:
        for b in row:
            flat[k] = b
            k += 1
    return lib.rc_all_reduce_many(len(rows), ctypes.cast(flat, ctypes.c_void_p), None)


def test_batched_validation(lib):
    R = 4
    reg(lib, R)
    t0 = bufs(addrs(R, 0x10000000), addrs(R, 0x20000000), (100,), op=rr.RC_MEAN)
    t1 = bufs(addrs(R, 0x30000000), addrs(R, 0x40000000), (7, 3), op=rr.RC_MEAN)
    assert many(lib, [t0, t1], R) == OK
    assert lib.rc_all_reduce_many(0, None, None) == OK
    assert lib.rc_all_reduce_many(-1, None, None) == INVAL
    t1b = bufs(addrs(R, 0x30000000), addrs(R, 0x40000000), [(7, 3)] * 3 + [(21,)], op=rr.RC_MEAN)
    assert many(lib, [t0, t1b], R) == SHAPE
    assert b"tensor 1" in lib.rc_last_error()
    t1c = bufs(addrs(R, 0x30000000), addrs(R, 0x40000000), (7, 3), op=rr.RC_SUM)
    assert many(lib, [t0, t1c], R) == OPM
    t1d = bufs(addrs(R, 0x30000000), addrs(R, 0x40000000), (7, 3), dtype=rr.RC_I32, op=rr.RC_MEAN)
    assert many(lib, [t0, t1d], R) == INVAL
    # outputs of two tensors overlapping
    t1e = bufs(addrs(R, 0x30000000), [a + 16 for a in addrs(R, 0x20000000)], (7, 3), op=rr.RC_MEAN)
    assert many(lib, [t0, t1e], R) == INVAL
