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
    assert uw.variant_count() == 24   # GEMV, nine LDS tiles, four register-fed kinds, six wide-step tiles, four eight-wave tiles


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


# ------------------------------------------------------ tuning table ------
# The table that UW_PIPE_AUTO and cfg == NULL consult is host state: its
# parsing, keying and nearest-batch rule are checked here without a GPU.

def _entry(uw, batch, pipeline, variant=0, split_k=0, n=28672, k=8192, layout=0, residency=3, group=0):
    return {"batch": batch, "projection": 0, "pipeline": pipeline, "variant": variant, "split_k": split_k,
            "decode_cus": 0, "layout": layout, "residency": residency, "n": n, "k": k, "sequence_us": 1.0,
            "group": group}


def test_tuning_table_nearest_batch(uw):
    uw.uw_clear_tuning()
    try:
        uw.uw_set_tuning([_entry(uw, 1, 3, 1), _entry(uw, 4, 3, 11), _entry(uw, 64, 3, 2),
                          _entry(uw, 1024, 1, 9, 2)])
        pick = lambda b: uw.uw_lookup_tuning(28672, 8192, 0, 3, b)["batch"]  # noqa: E731
        assert pick(1) == 1
        assert pick(2) == 1          # log2 distance 1 to both 1 and 4: the smaller
        assert pick(3) == 4
        assert pick(16) == 4         # distance 2 to both 4 and 64: the smaller
        assert pick(200) == 64
        assert pick(700) == 1024
        assert pick(1 << 20) == 1024
        e = uw.uw_lookup_tuning(28672, 8192, 0, 3, 1024)
        assert (e["pipeline"], e["variant"], e["split_k"]) == (1, 9, 2)
        # other keys are separate: residency, layout and shape
        assert uw.uw_lookup_tuning(28672, 8192, 0, 1, 64) is None
        assert uw.uw_lookup_tuning(28672, 8192, 1, 3, 64) is None
        assert uw.uw_lookup_tuning(8192, 28672, 0, 3, 64) is None
        # the same key and batch replaces
        uw.uw_set_tuning([_entry(uw, 64, 2, 3)])
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 64)["pipeline"] == 2
    finally:
        uw.uw_clear_tuning()
    assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 64) is None


def test_tuning_table_rejects_malformed_entries(uw):
    uw.uw_clear_tuning()
    bad = [_entry(uw, 1, 3), _entry(uw, 0, 3), _entry(uw, 8, 7), _entry(uw, 8, 3, residency=0),
           _entry(uw, 8, 3, variant=99), _entry(uw, 8, 3, layout=2)]
    for b in bad[1:]:
        with pytest.raises(uw.UwError) as ei:
            uw.uw_set_tuning([bad[0], b])
        assert ei.value.status == -1
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 1) is None   # none of the call's entries was added
    # register-fed variants (the first follows the GEMV and the nine LDS
    # tiles with 64-wide K steps) and 128-wide K steps (variant 21, the
    # eight-wave 128x128) are [N][K] only
    for v in (11, 21):
        with pytest.raises(uw.UwError):
            uw.uw_set_tuning([_entry(uw, 8, 3, variant=v, layout=1)])
    assert uw._lib.uw_lookup_tuning(1, 1, 0, 3, 0, None) == -1


def test_tuning_table_group_entries_are_separate(uw):
    """A grouped call's entry (gate+up of 8B: 2 matrices, total N 28672) is
    keyed apart from a single matrix of the same N, and apart from groups of
    another size; group 1, negative and beyond 64 are malformed."""
    uw.uw_clear_tuning()
    try:
        uw.uw_set_tuning([_entry(uw, 64, 3, 2), _entry(uw, 64, 1, 3, group=2), _entry(uw, 64, 2, 4, group=3)])
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 64)["pipeline"] == 3
        e2 = uw.uw_lookup_tuning_grouped(28672, 8192, 0, 3, 2, 64)
        assert (e2["pipeline"], e2["variant"], e2["group"]) == (1, 3, 2)
        assert uw.uw_lookup_tuning_grouped(28672, 8192, 0, 3, 3, 100)["pipeline"] == 2
        assert uw.uw_lookup_tuning_grouped(28672, 8192, 0, 3, 4, 64) is None
        assert uw.uw_lookup_tuning_grouped(28672, 8192, 1, 3, 2, 64) is None
        for g in (1, -1, 65):
            with pytest.raises(uw.UwError) as ei:
                uw.uw_set_tuning([_entry(uw, 8, 3, group=g)])
            assert ei.value.status == -1
        for g in (0, 1, 65):
            assert uw._lib.uw_lookup_tuning_grouped(28672, 8192, 0, 3, g, 64, ctypes.byref(uw.uw_tune_entry())) == -1
    finally:
        uw.uw_clear_tuning()


def test_load_tuning_json_group_field(uw, tmp_path):
    """uw_load_tuning reads "group" (as uw_autotune_grouped writes it) and
    takes a missing one as 0."""
    import json
    uw.uw_clear_tuning()
    single = {k: v for k, v in _entry(uw, 8, 3, 1).items() if k != "group"}
    grouped = _entry(uw, 8, 1, 4, split_k=2, n=6144, k=4096, group=3)
    path = tmp_path / "grouped.json"
    path.write_text(json.dumps({"entries": [single, grouped]}))
    try:
        uw.uw_load_tuning(str(path))
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 8)["group"] == 0
        e = uw.uw_lookup_tuning_grouped(6144, 4096, 0, 3, 3, 8)
        assert (e["pipeline"], e["variant"], e["split_k"]) == (1, 4, 2)
        assert uw.uw_lookup_tuning(6144, 4096, 0, 3, 8) is None
        uw.uw_clear_tuning()
        path.write_text(json.dumps({"entries": [dict(grouped, group=99)]}))
        with pytest.raises(uw.UwError) as ei:
            uw.uw_load_tuning(str(path))
        assert ei.value.status == -5
    finally:
        uw.uw_clear_tuning()


def test_autotune_grouped_host_checks(uw):
    """Argument checks that fail before any device work."""
    bs = (ctypes.c_int64 * 1)(8)
    assert uw._lib.uw_autotune_grouped(None, 2, 1, bs, 1, None, None, None) == -1
    arr = (ctypes.c_void_p * 2)(None, None)
    assert uw._lib.uw_autotune_grouped(arr, 1, 2, bs, 1, None, None, None) == -1   # group of one
    assert uw._lib.uw_autotune_grouped(arr, 2, 1, bs, 1, None, None, None) == -1   # NULL matrices
    assert uw._lib.uw_autotune_grouped(arr, 2, 0, bs, 1, None, None, None) == -1


def test_load_tuning_json(uw, tmp_path):
    import json
    uw.uw_clear_tuning()
    entries = [_entry(uw, 1, 3, 1), _entry(uw, 1, 3, 1, n=8192, k=28672, layout=1),
               _entry(uw, 1024, 1, 6, n=8192, k=28672, layout=1)]
    path = tmp_path / "tuned.json"
    path.write_text(json.dumps({"entries": entries}, indent=2))
    try:
        uw.uw_load_tuning(str(path))
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 1)["variant"] == 1
        e = uw.uw_lookup_tuning(8192, 28672, 1, 3, 512)
        assert (e["batch"], e["pipeline"], e["variant"]) == (1024, 1, 6)
        # an unreadable or malformed file adds nothing
        uw.uw_clear_tuning()
        for text in ("{}", '{"entries": [{"batch": 4}]}', '{"entries": [' + json.dumps(dict(entries[0], pipeline=9)) + "]}"):
            path.write_text(text)
            with pytest.raises(uw.UwError) as ei:
                uw.uw_load_tuning(str(path))
            assert ei.value.status == -5
        with pytest.raises(uw.UwError):
            uw.uw_load_tuning(str(tmp_path / "missing.json"))
        assert uw.uw_lookup_tuning(28672, 8192, 0, 3, 1) is None
    finally:
        uw.uw_clear_tuning()


def test_kernel_events_host_rules(uw):
    """uw_set_kernel_events: both NULL clears, one NULL alone is invalid."""
    assert uw._lib.uw_set_kernel_events(None, None) == 0
    assert uw._lib.uw_set_kernel_events(ctypes.c_void_p(16), None) == -1
    assert uw._lib.uw_set_kernel_events(None, ctypes.c_void_p(16)) == -1
    assert uw._lib.uw_set_kernel_events(None, None) == 0


def test_allocator_and_release_host_rules(uw):
    a = uw.uw_allocator()
    a.alloc = uw.ALLOC_FN(lambda n, c: None)
    assert uw._lib.uw_set_allocator(ctypes.byref(a)) == -1     # one hook without the other
    assert uw._lib.uw_set_allocator(None) == 0
    assert uw._lib.uw_release_resources() == 0                 # nothing was created
    n = ctypes.c_size_t()
    assert uw._lib.uw_workspace_size_cfg(None, 15, 1, None, ctypes.byref(n)) == -1
    assert uw._lib.uw_workspace_size_grouped(None, 1, 15, 1, None, ctypes.byref(n)) == -1
