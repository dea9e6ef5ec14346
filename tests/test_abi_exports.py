"""The C-ABI library loads and exports every function include/qspec.h declares;
host-side helpers and argument checks work without a GPU (no compute calls)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qspec.h")
LIB = os.path.join(ROOT, "quantized_speculative_decoding_int4_amd", "lib", "libqspec.so")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libqspec.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_six_calls():
    names = _declared_functions()
    for n in ("qs_pack_weights", "qs_linear_w4a16", "qs_linear_w4a4", "qs_lmhead",
              "qs_verify_greedy", "qs_verify_sample"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_status_strings(lib):
    f = lib.qs_status_string
    f.restype = ctypes.c_char_p
    f.argtypes = [ctypes.c_int]
    assert f(0) == b"ok"
    for code in (-1, -2, -3, -4, -5, -6):
        assert f(code) and f(code) != b"unknown status"
    assert f(12345) == b"unknown status"


def test_size_helpers(lib):
    wb = lib.qs_packed_weight_bytes
    sb = lib.qs_packed_scale_bytes
    for f in (wb, sb):
        f.restype = ctypes.c_size_t
        f.argtypes = [ctypes.c_int, ctypes.c_int]
    assert wb(4096, 4096) == 4096 * 4096 // 2
    assert sb(4096, 4096) == 4096 * 32 * 2
    assert wb(128256, 4096) == 262668288          # LM-head nibbles
    assert sb(128256, 4096) == 8208384            # LM-head scales
    assert wb(17, 128) == 32 * 128 // 2          # padded to whole 16-row blocks
    assert wb(16, 100) == 0 and wb(0, 128) == 0


def test_verify_workspace_helper(lib):
    f = lib.qs_verify_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int] * 3
    assert f(1, 3, 128256) > 0
    assert f(0, 3, 10) == 0 and f(1, -1, 10) == 0 and f(1, 64, 10) == 0
    # per-sequence arrival counters sit in a fixed area at the start, one 256-byte line per
    # sequence; larger batches run in blocks of 16384 sequences that reuse one block's workspace
    assert f(1, 0, 1) >= 16384 * 256
    assert f(16384, 3, 4096) > f(8192, 3, 4096) and f(10**6, 3, 4096) == f(16384, 3, 4096)


def test_argument_errors_before_any_device_work(lib):
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lin = lib.qs_linear_w4a16
    lin.argtypes = [p, p, p, p, i, i, i, p]
    lin.restype = i
    fake = 1 << 20  # never dereferenced: the checks fail first
    assert lin(None, fake, fake, fake, 4, 4096, 4096, None) == -1
    assert lin(fake, fake, fake, fake, 4, 4096, 4000, None) == -1     # K % 128 != 0
    assert lin(fake, fake, fake, fake, 0, 4096, 4096, None) == -1     # M < 1
    assert lin(fake, fake, fake, fake, 257, 4096, 4096, None) == -2   # M > 256
    assert lin(fake + 8, fake, fake, fake, 4, 4096, 4096, None) == -3  # misaligned x
    w4 = lib.qs_linear_w4a4
    w4.argtypes = [p, p, p, p, i, i, i, p, p, p, p, sz, p]
    w4.restype = i
    assert w4(fake, fake, fake, fake, 64, 4096, 4096, None, None, None, None, 0, None) == -4
    vg = lib.qs_verify_greedy
    vg.argtypes = [p, p, i, i, i, p, p, p, p, p, sz, p]
    vg.restype = i
    assert vg(fake, fake, 1, 64, 10, fake, None, fake, fake, fake, 1 << 20, None) == -2  # gamma > 63
    assert vg(fake, fake, 1, 3, 10, fake, None, fake, fake, None, 0, None) == -4
    assert vg(fake, None, 1, 3, 10, fake, None, fake, fake, fake, 1 << 24, None) == -1   # draft ids
    # chain descriptors are read on the host: a chain whose K does not follow the previous N
    desc = (ctypes.c_char * 48)()
    ctypes.memmove(desc, (ctypes.c_uint64 * 6)(fake, fake, (4096 << 32) | 4096, fake, fake,
                                               (8192 << 32) | 4096), 48)
    pl = lib.qs_chain_pass_launches
    pl.argtypes = [i, i, p, i]
    pl.restype = i
    assert pl(0, 4, ctypes.addressof(desc), 2) == -1                  # 8192 > 4096 columns
    assert pl(0, 4, ctypes.addressof(desc), 1) in (-6, 0, 1)          # one linear: valid
    assert pl(3, 4, ctypes.addressof(desc), 1) == -1                  # bad mode (0, 1, 2 are modes)
    assert pl(0, 300, ctypes.addressof(desc), 1) == -2                # M > 256
    to = lib.qs_set_barrier_timeout_us
    to.argtypes = [i]
    to.restype = i
    assert to(-1) == -1
    stf = lib.qs_chain_pass_status
    stf.argtypes = [i, i, p, i, p, sz, p, p]
    stf.restype = i
    assert stf(0, 4, ctypes.addressof(desc), 1, fake, 1 << 30, None, None) == -1   # no result pointer
    flag = ctypes.c_int(7)
    assert stf(0, 4, ctypes.addressof(desc), 1, None, 0, ctypes.addressof(flag), None) == -4  # no workspace


def test_no_gpu_means_device_error(lib):
    """Valid arguments on a machine without a gfx950 device report QS_ERR_DEVICE
    (the library never falls back to another device or to the host)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p, i = ctypes.c_void_p, ctypes.c_int
    lin = lib.qs_linear_w4a16
    lin.argtypes = [p, p, p, p, i, i, i, p]
    lin.restype = i
    fake = 1 << 20
    assert lin(fake, fake, fake, fake, 4, 4096, 4096, None) == -6


def test_new_entry_points_argument_errors(lib):
    """W4A8 linear, LM-head with the fused Top-1 and tree verify: errors returned before any
    device work (fake pointers are never dereferenced)."""
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fake = 1 << 20
    w8 = lib.qs_linear_w4a8
    w8.argtypes = [p, p, p, p, i, i, i, p, p, p, p, sz, p]
    w8.restype = i
    assert w8(None, fake, fake, fake, 4, 4096, 4096, None, None, None, fake, 1 << 30, None) == -1
    assert w8(fake, fake, fake, fake, 4, 4096, 4000, None, None, None, fake, 1 << 30, None) == -1
    assert w8(fake, fake, fake, fake, 300, 4096, 4096, None, None, None, fake, 1 << 30, None) == -2
    assert w8(fake, fake, fake, fake, 1, 4096, 4096, None, None, None, None, 0, None) == -4  # always staged
    lw = lib.qs_linear_workspace_bytes
    lw.argtypes = [i, i, i, i]
    lw.restype = sz
    assert lw(2, 1, 4096, 4096) > 0 and lw(3, 1, 4096, 4096) == 0
    tw = lib.qs_lmhead_top1_workspace_bytes
    tw.argtypes = [i, i, i, i]
    tw.restype = sz
    assert tw(0, 4, 128256, 4096) >= 4 * 501 * 16 and tw(1, 1, 128256, 4096) > tw(0, 1, 128256, 4096)
    assert tw(3, 4, 128256, 4096) == 0 and tw(0, 0, 128256, 4096) == 0
    t1 = lib.qs_lmhead_top1
    t1.argtypes = [i, p, p, p, p, i, i, i, p, p, p, sz, p]
    t1.restype = i
    assert t1(3, fake, fake, fake, None, 4, 1000, 512, fake, None, fake, 1 << 30, None) == -1   # bad mode
    assert t1(0, fake, fake, fake, None, 4, 1000, 512, None, None, fake, 1 << 30, None) == -1   # top1 NULL
    assert t1(0, fake, fake, fake, None, 257, 1000, 512, fake, None, fake, 1 << 30, None) == -2
    assert t1(0, fake, fake, fake, None, 4, 1000, 512, fake, None, fake, 16, None) == -4        # short ws
    tg = lib.qs_verify_tree_greedy
    tg.argtypes = [p, p, p, i, i, i, p, p, p, p, p, sz, p]
    tg.restype = i
    assert tg(fake, fake, fake, 1, 0, 10, fake, fake, fake, None, fake, 1 << 30, None) == -1   # T < 1
    assert tg(fake, fake, fake, 1, 65, 10, fake, fake, fake, None, fake, 1 << 30, None) == -2  # T > 64
    assert tg(fake, None, fake, 1, 4, 10, fake, fake, fake, None, fake, 1 << 30, None) == -1   # tokens
    assert tg(fake, fake, fake, 1, 4, 10, fake, fake, fake, None, fake, 0, None) == -4


def test_chain_trace_argument_errors(lib):
    """The traced chain pass refuses a missing timestamp buffer, a bad mode and oversized rows before
    any device work, and its size helper returns 0 for invalid arguments."""
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fake = 1 << 20
    tr = lib.qs_chain_forward_trace
    tr.argtypes = [i, p, i, p, i, p, p, sz, p, sz, p]
    tr.restype = i
    assert tr(0, fake, 4, fake, 1, fake, fake, 1 << 30, None, 1 << 30, None) == -1   # no timestamp buffer
    assert tr(3, fake, 4, fake, 1, fake, fake, 1 << 30, fake, 1 << 30, None) == -1   # bad mode
    assert tr(0, fake, 4, None, 1, fake, fake, 1 << 30, fake, 1 << 30, None) == -1   # no chain
    tb = lib.qs_chain_trace_bytes
    tb.argtypes = [i, i, p, i]
    tb.restype = sz
    assert tb(0, 4, None, 1) == 0 and tb(3, 4, None, 1) == 0


def test_noalloc_greedy_refuses_before_any_device_work(lib):
    """The greedy verify without a workspace: argument errors and sizes beyond its fixed scratch are
    refused on the host (fake pointers are never dereferenced)."""
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fake = 1 << 20
    mx = lib.qs_verify_greedy_noalloc_max_bytes
    mx.argtypes = []
    mx.restype = sz
    assert mx() == 8 << 20
    vw = lib.qs_verify_workspace_bytes
    vw.argtypes = [i, i, i]
    vw.restype = sz
    f = lib.qs_verify_greedy_noalloc
    f.argtypes = [p, p, i, i, i, p, p, p, p, p]
    f.restype = i
    assert f(None, fake, 1, 3, 1000, fake, None, fake, fake, None) == -1            # logits NULL
    assert f(fake, None, 1, 3, 1000, fake, None, fake, fake, None) == -1            # draft ids NULL, gamma > 0
    assert f(fake, fake, 0, 3, 1000, fake, None, fake, fake, None) == -1            # B < 1
    assert vw(4096, 63, 1 << 20) > mx()
    assert f(fake, fake, 4096, 63, 1 << 20, fake, None, fake, fake, None) == -2     # beyond the scratch
    assert f(fake, fake, 1, 64, 1000, fake, None, fake, fake, None) == -2           # gamma out of range
