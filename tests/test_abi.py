"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/unweight.h, and rejects bad arguments and malformed UWF1
blobs on the host before any device work."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def uw():
    from decode_gemm_exp_amd import uw as _uw
    return _uw


def declared_symbols():
    with open(os.path.join(ROOT, "include", "unweight.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(uw_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(uw):
    syms = declared_symbols()
    assert len(syms) >= 19
    lib = ctypes.CDLL(uw.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), f"{s} declared but not exported"
    assert set(syms) == set(uw.EXPORTED)


def test_status_strings_and_version(uw):
    for st in range(-7, 1):
        assert uw._lib.uw_status_str(st)
    assert uw.version() >> 16 == 1
    assert uw.variant_count() >= 2


def test_invalid_arguments_rejected_without_device(uw):
    h = ctypes.c_void_p()
    opts = uw.uw_compress_opts(8, 0)
    assert uw._lib.uw_compress(None, 4, 64, 0, ctypes.byref(opts), None, ctypes.byref(h)) == -1
    assert uw._lib.uw_compress(16, -1, 64, 0, ctypes.byref(opts), None, ctypes.byref(h)) == -1
    assert uw._lib.uw_compress(16, 4, 100, 0, ctypes.byref(opts), None, ctypes.byref(h)) == -2
    assert uw._lib.uw_compress(16, 4, 64, 7, ctypes.byref(opts), None, ctypes.byref(h)) == -1
    bad = uw.uw_compress_opts(3, 0)
    assert uw._lib.uw_compress(16, 4, 64, 0, ctypes.byref(bad), None, ctypes.byref(h)) == -1
    assert uw._lib.uw_get_info(None, None) == -1
    assert uw._lib.uw_decode_full(None, None, None) == -1
    n = ctypes.c_size_t()
    assert uw._lib.uw_workspace_size(None, 0, 1, ctypes.byref(n)) == -1


def _blob(oracle, sg=2):
    from tests.test_oracle_pins import three_group_input
    return bytearray(oracle.compress(three_group_input(), seg_groups=sg).export())


@pytest.mark.parametrize("mutate", [
    "magic", "version", "layout", "seg_groups", "cols", "truncate", "extra", "palette", "code_len",
    "hist", "vflags_tail", "vrank", "seg_off_first", "seg_off_last", "V"])
def test_import_rejects_corrupt_blobs(uw, oracle, mutate):
    b = _blob(oracle)
    if mutate == "magic":
        b[0] = ord("X")
    elif mutate == "version":
        struct.pack_into("<I", b, 4, 2)
    elif mutate == "layout":
        struct.pack_into("<I", b, 8, 5)
    elif mutate == "seg_groups":
        struct.pack_into("<I", b, 12, 3)
    elif mutate == "cols":
        struct.pack_into("<Q", b, 24, 100)
    elif mutate == "truncate":
        b = b[:-10]
    elif mutate == "extra":
        b = b + bytes(256)
    elif mutate == "palette":
        b[40 + 15] = 200
    elif mutate == "code_len":
        b[56 + 13] = 2
    elif mutate == "hist":
        struct.pack_into("<Q", b, 88 + 8 * 126, 112)
    elif mutate == "vflags_tail":
        off = 2304 + 256
        struct.pack_into("<I", b, off, 4 | (1 << 7))      # a flag past the 3 groups
    elif mutate == "vrank":
        struct.pack_into("<I", b, 2304 + 512, 1)
    elif mutate == "seg_off_first":
        struct.pack_into("<I", b, 2304 + 1024, 1)
    elif mutate == "seg_off_last":
        struct.pack_into("<I", b, 2304 + 1024 + 8, 7)
    elif mutate == "V":
        struct.pack_into("<Q", b, 72, 2)
    assert uw.uw_import_status(bytes(b)) == -5


def test_import_rejects_empty_and_short(uw):
    assert uw.uw_import_status(b"") == -1          # NULL blob: invalid argument
    assert uw.uw_import_status(b"UWF1" + bytes(12)) == -5
