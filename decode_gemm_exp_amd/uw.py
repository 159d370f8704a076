"""Thin ctypes binding of libunweight.so (include/unweight.h).

Argument marshalling only: every step of the codec and the GEMMs runs in the
library's HIP kernels.  torch tensors are accepted for device buffers and
their ``data_ptr()`` is passed through; streams default to torch's current
stream.  Importing this module fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libunweight.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() (hipcc for gfx950) first")

_lib = ctypes.CDLL(LIB_PATH)

UW_OK = 0
UW_ERR_UNSUPPORTED = -2
STATUS = {0: "ok", -1: "invalid", -2: "unsupported", -3: "nomem", -4: "device", -5: "corrupt",
          -6: "state", -7: "workspace"}
PIPE_FULL, PIPE_EXPONENT, PIPE_PALETTE_TRANSCODE, PIPE_PALETTE_DIRECT = 0, 1, 2, 3
PIPE_AUTO = 15
PIPELINES = {"full": 0, "exponent": 1, "transcode": 2, "direct": 3, "auto": 15}
LAYOUT_NK, LAYOUT_KN = 0, 1


class UwError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


class uw_compress_opts(ctypes.Structure):
    _fields_ = [("seg_groups", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


class uw_kernel_cfg(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("split_k", ctypes.c_int32), ("decode_cus", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class uw_info(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_uint32), ("seg_groups", ctypes.c_uint32),
                ("rows", ctypes.c_uint64), ("cols", ctypes.c_uint64), ("n", ctypes.c_uint64),
                ("k", ctypes.c_uint64), ("numel", ctypes.c_uint64), ("groups", ctypes.c_uint64),
                ("segments", ctypes.c_uint64), ("palette_size", ctypes.c_uint32), ("n_coded", ctypes.c_uint32),
                ("palette", ctypes.c_uint8 * 16), ("code_len", ctypes.c_uint8 * 16),
                ("code", ctypes.c_uint16 * 16), ("hist", ctypes.c_uint64 * 256),
                ("coded_count", ctypes.c_uint64 * 16), ("verbatim_groups", ctypes.c_uint64),
                ("stream_words", ctypes.c_uint64), ("code_bits", ctypes.c_uint64),
                ("compressed_bytes", ctypes.c_uint64), ("export_bytes", ctypes.c_uint64),
                ("bits_per_weight", ctypes.c_double), ("has_stream", ctypes.c_int32),
                ("has_palette_idx", ctypes.c_int32), ("element_bits", ctypes.c_int32)]


class uw_tune_entry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("projection", ctypes.c_int32), ("pipeline", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("split_k", ctypes.c_int32), ("decode_cus", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("residency", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n", ctypes.c_uint64), ("k", ctypes.c_uint64), ("sequence_us", ctypes.c_double)]


ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)


class uw_allocator(ctypes.Structure):
    _fields_ = [("alloc", ALLOC_FN), ("free", FREE_FN), ("ctx", ctypes.c_void_p)]


class uw_gemm_plan(ctypes.Structure):
    _fields_ = [("pipeline", ctypes.c_int32), ("variant", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("k_slices", ctypes.c_int32), ("reserved", ctypes.c_int32), ("kernel", ctypes.c_char * 64)]


class uw_job(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("pipeline", ctypes.c_int32), ("cfg", uw_kernel_cfg),
                ("x_dev", ctypes.c_void_p), ("y_dev", ctypes.c_void_p), ("batch", ctypes.c_int64)]


_vp, _i64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "uw_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "uw_version": (ctypes.c_uint32, []),
    "uw_compress": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.POINTER(uw_compress_opts), _vp,
                                   ctypes.POINTER(_vp)]),
    "uw_compress_fp8": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.POINTER(uw_compress_opts), _vp,
                                   ctypes.POINTER(_vp)]),
    "uw_get_info": (ctypes.c_int, [_vp, ctypes.POINTER(uw_info)]),
    "uw_export": (ctypes.c_int, [_vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "uw_import": (ctypes.c_int, [_vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "uw_free": (None, [_vp]),
    "uw_decode_full": (ctypes.c_int, [_vp, _vp, _vp]),
    "uw_decode_fp8": (ctypes.c_int, [_vp, _vp, _vp]),
    "uw_decode_exponent": (ctypes.c_int, [_vp, _vp, _vp]),
    "uw_transcode_palette": (ctypes.c_int, [_vp, _vp, _vp]),
    "uw_drop_stream": (ctypes.c_int, [_vp, _vp]),
    "uw_workspace_size": (ctypes.c_int, [_vp, ctypes.c_int, _i64, ctypes.POINTER(_sz)]),
    "uw_matmul_reconstruct": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _vp, _vp, _sz,
                                             ctypes.POINTER(uw_kernel_cfg), _vp]),
    "uw_matmul_stage": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _i64, _vp, _vp, _sz,
                                       ctypes.POINTER(uw_kernel_cfg), _vp]),
    "uw_matmul_reconstruct_grouped": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int, ctypes.c_int, _vp, _i64,
                                                     _vp, _vp, _sz, ctypes.POINTER(uw_kernel_cfg), _vp]),
    "uw_gemm_bf16": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _i64, _vp,
                                    ctypes.POINTER(uw_kernel_cfg), _vp]),
    "uw_variant_count": (ctypes.c_int32, []),
    "uw_sequence_workspace_size": (ctypes.c_int, [ctypes.POINTER(uw_job), ctypes.c_int, ctypes.POINTER(_sz)]),
    "uw_run_sequence": (ctypes.c_int, [ctypes.POINTER(uw_job), ctypes.c_int, ctypes.c_int32, _vp, _sz, _vp]),
    "uw_sync_status": (ctypes.c_int, [_vp, _vp]),
    "uw_autotune": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int, ctypes.c_char_p,
                                   ctypes.POINTER(uw_tune_entry), _vp]),
    "uw_autotune_grouped": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_char_p,
                                           ctypes.POINTER(uw_tune_entry), _vp]),
    "uw_drop_palette": (ctypes.c_int, [_vp, _vp]),
    "uw_workspace_size_cfg": (ctypes.c_int, [_vp, ctypes.c_int, _i64, ctypes.POINTER(uw_kernel_cfg),
                                             ctypes.POINTER(_sz)]),
    "uw_workspace_size_grouped": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.c_int, ctypes.c_int, _i64,
                                                 ctypes.POINTER(uw_kernel_cfg), ctypes.POINTER(_sz)]),
    "uw_matmul_stage_static": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _i64, _vp,
                                              ctypes.POINTER(uw_kernel_cfg), _vp]),
    "uw_plan_gemm": (ctypes.c_int, [_vp, ctypes.c_int, _i64, ctypes.POINTER(uw_kernel_cfg),
                                    ctypes.POINTER(uw_gemm_plan)]),
    "uw_yardstick": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _sz, _i64, _vp, ctypes.POINTER(ctypes.c_double)]),
    "uw_set_allocator": (ctypes.c_int, [ctypes.POINTER(uw_allocator)]),
    "uw_release_resources": (ctypes.c_int, []),
    "uw_set_kernel_events": (ctypes.c_int, [_vp, _vp]),
    "uw_set_tuning": (ctypes.c_int, [ctypes.POINTER(uw_tune_entry), ctypes.c_int]),
    "uw_load_tuning": (ctypes.c_int, [ctypes.c_char_p]),
    "uw_clear_tuning": (ctypes.c_int, []),
    "uw_lookup_tuning": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, _i64,
                                        ctypes.POINTER(uw_tune_entry)]),
    "uw_lookup_tuning_grouped": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, _i64, ctypes.POINTER(uw_tune_entry)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(st: int, what: str) -> None:
    if st != UW_OK:
        raise UwError(st, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    return int(t)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _cfg(cfg) -> ctypes.POINTER(uw_kernel_cfg) | None:
    if cfg is None:
        return None
    if isinstance(cfg, dict):
        c = uw_kernel_cfg(cfg.get("variant", 0), cfg.get("split_k", 0), cfg.get("decode_cus", 0), 0)
    else:
        c = cfg
    return ctypes.pointer(c)


def version() -> int:
    return _lib.uw_version()


def variant_count() -> int:
    return _lib.uw_variant_count()


class Matrix:
    """Owns one uw_matrix handle."""

    def __init__(self, handle: int):
        self.handle = ctypes.c_void_p(handle)

    def info(self) -> uw_info:
        inf = uw_info()
        _check(_lib.uw_get_info(self.handle, ctypes.byref(inf)), "uw_get_info")
        return inf

    def free(self) -> None:
        if self.handle and self.handle.value:
            _lib.uw_free(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def uw_compress(w_dev: torch.Tensor, n: int, k: int, layout: int = LAYOUT_NK, seg_groups: int = 4,
                stream=None) -> Matrix:
    opts = uw_compress_opts(seg_groups, 0)
    h = ctypes.c_void_p()
    _check(_lib.uw_compress(_ptr(w_dev), n, k, layout, ctypes.byref(opts), _stream(stream), ctypes.byref(h)),
           "uw_compress")
    return Matrix(h.value)


def uw_get_info(m: Matrix) -> uw_info:
    return m.info()


def uw_export(m: Matrix) -> bytes:
    n = ctypes.c_size_t()
    _check(_lib.uw_export(m.handle, None, 0, ctypes.byref(n)), "uw_export(size)")
    buf = np.zeros(n.value, dtype=np.uint8)
    _check(_lib.uw_export(m.handle, buf.ctypes.data, n.value, ctypes.byref(n)), "uw_export")
    return buf.tobytes()


def uw_import(blob: bytes, stream=None) -> Matrix:
    arr = np.frombuffer(blob, dtype=np.uint8)
    h = ctypes.c_void_p()
    _check(_lib.uw_import(arr.ctypes.data, len(blob), _stream(stream), ctypes.byref(h)), "uw_import")
    return Matrix(h.value)


def uw_import_status(blob: bytes) -> int:
    """Status of uw_import without keeping the handle (validation tests)."""
    arr = np.frombuffer(blob, dtype=np.uint8)
    h = ctypes.c_void_p()
    st = _lib.uw_import(arr.ctypes.data if len(blob) else None, len(blob), None, ctypes.byref(h))
    if h.value:
        _lib.uw_free(h)
    return st


def uw_free(m: Matrix) -> None:
    m.free()


def uw_compress_fp8(w_dev: torch.Tensor, n: int, k: int, layout: int = LAYOUT_NK, seg_groups: int = 4,
                    stream=None) -> Matrix:
    """FP8 E4M3 weights given as a uint8 device tensor of the stored shape."""
    opts = uw_compress_opts(seg_groups, 0)
    h = ctypes.c_void_p()
    _check(_lib.uw_compress_fp8(_ptr(w_dev), n, k, layout, ctypes.byref(opts), _stream(stream), ctypes.byref(h)),
           "uw_compress_fp8")
    return Matrix(h.value)


def uw_decode_fp8(m: Matrix, out: torch.Tensor, stream=None) -> None:
    _check(_lib.uw_decode_fp8(m.handle, _ptr(out), _stream(stream)), "uw_decode_fp8")


def uw_decode_full(m: Matrix, out: torch.Tensor, stream=None) -> None:
    _check(_lib.uw_decode_full(m.handle, _ptr(out), _stream(stream)), "uw_decode_full")


def uw_decode_exponent(m: Matrix, out: torch.Tensor, stream=None) -> None:
    _check(_lib.uw_decode_exponent(m.handle, _ptr(out), _stream(stream)), "uw_decode_exponent")


def uw_transcode_palette(m: Matrix, out: torch.Tensor | None, stream=None) -> None:
    _check(_lib.uw_transcode_palette(m.handle, _ptr(out), _stream(stream)), "uw_transcode_palette")


def uw_drop_stream(m: Matrix, stream=None) -> None:
    _check(_lib.uw_drop_stream(m.handle, _stream(stream)), "uw_drop_stream")


def uw_workspace_size(m: Matrix, pipeline: int, batch: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.uw_workspace_size(m.handle, pipeline, batch, ctypes.byref(n)), "uw_workspace_size")
    return n.value


def uw_workspace_size_cfg(m: Matrix, pipeline: int, batch: int, cfg=None) -> int:
    n = ctypes.c_size_t()
    _check(_lib.uw_workspace_size_cfg(m.handle, pipeline, batch, _cfg(cfg), ctypes.byref(n)),
           "uw_workspace_size_cfg")
    return n.value


def uw_workspace_size_grouped(ms, pipeline: int, batch: int, cfg=None) -> int:
    arr = (ctypes.c_void_p * len(ms))(*[m.handle.value for m in ms])
    n = ctypes.c_size_t()
    _check(_lib.uw_workspace_size_grouped(arr, len(ms), pipeline, batch, _cfg(cfg), ctypes.byref(n)),
           "uw_workspace_size_grouped")
    return n.value


def uw_matmul_reconstruct(m: Matrix, pipeline: int, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor | None,
                          cfg=None, stream=None) -> None:
    batch = x.shape[0]
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.uw_matmul_reconstruct(m.handle, pipeline, _ptr(x), batch, _ptr(y), _ptr(ws), nbytes, _cfg(cfg),
                                      _stream(stream)), "uw_matmul_reconstruct")


def uw_matmul_stage(m: Matrix, pipeline: int, prep: torch.Tensor | None, x: torch.Tensor, y: torch.Tensor,
                    ws: torch.Tensor | None, cfg=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.uw_matmul_stage(m.handle, pipeline, _ptr(prep), _ptr(x), x.shape[0], _ptr(y), _ptr(ws), nbytes,
                                _cfg(cfg), _stream(stream)), "uw_matmul_stage")


STATIC_SCRATCH_BYTES = 64 << 20


def uw_matmul_stage_static(m: Matrix, pipeline: int, prep: torch.Tensor | None, x: torch.Tensor, y: torch.Tensor,
                           cfg=None, stream=None) -> None:
    _check(_lib.uw_matmul_stage_static(m.handle, pipeline, _ptr(prep), _ptr(x), x.shape[0], _ptr(y), _cfg(cfg),
                                       _stream(stream)), "uw_matmul_stage_static")


def uw_matmul_reconstruct_grouped(ms, pipeline: int, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor | None,
                                  cfg=None, stream=None) -> None:
    arr = (ctypes.c_void_p * len(ms))(*[m.handle.value for m in ms])
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.uw_matmul_reconstruct_grouped(arr, len(ms), pipeline, _ptr(x), x.shape[0], _ptr(y), _ptr(ws),
                                              nbytes, _cfg(cfg), _stream(stream)), "uw_matmul_reconstruct_grouped")


def uw_gemm_bf16(w: torch.Tensor, n: int, k: int, layout: int, x: torch.Tensor, y: torch.Tensor, cfg=None,
                 stream=None) -> None:
    _check(_lib.uw_gemm_bf16(_ptr(w), n, k, layout, _ptr(x), x.shape[0], _ptr(y), _cfg(cfg), _stream(stream)),
           "uw_gemm_bf16")


@dataclass
class Job:
    m: Matrix
    pipeline: int
    x: torch.Tensor
    y: torch.Tensor
    cfg: dict | None = None


def _jobs(jobs) -> ctypes.Array:
    arr = (uw_job * len(jobs))()
    for i, j in enumerate(jobs):
        c = j.cfg or {}
        arr[i] = uw_job(j.m.handle.value, j.pipeline,
                        uw_kernel_cfg(c.get("variant", 0), c.get("split_k", 0), c.get("decode_cus", 0), 0),
                        _ptr(j.x), _ptr(j.y), j.x.shape[0])
    return arr


def uw_sequence_workspace_size(jobs) -> int:
    n = ctypes.c_size_t()
    _check(_lib.uw_sequence_workspace_size(_jobs(jobs), len(jobs), ctypes.byref(n)), "uw_sequence_workspace_size")
    return n.value


def uw_run_sequence(jobs, decode_cus: int, ws: torch.Tensor | None, stream=None, _arr=None) -> None:
    arr = _arr if _arr is not None else _jobs(jobs)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.uw_run_sequence(arr, len(jobs), decode_cus, _ptr(ws), nbytes, _stream(stream)),
           "uw_run_sequence")


def uw_drop_palette(m: Matrix, stream=None) -> None:
    _check(_lib.uw_drop_palette(m.handle, _stream(stream)), "uw_drop_palette")


def uw_autotune(ms, proj, batches, max_passes: int = 3, json_path: str | None = None, stream=None):
    """Returns a list of dicts, one per (batch, projection)."""
    nproj = max(proj) + 1
    arr = (ctypes.c_void_p * len(ms))(*[m.handle.value for m in ms])
    pj = (ctypes.c_int32 * len(proj))(*proj)
    bs = (ctypes.c_int64 * len(batches))(*batches)
    out = (uw_tune_entry * (len(batches) * nproj))()
    _check(_lib.uw_autotune(arr, pj, len(ms), nproj, bs, len(batches), max_passes,
                            json_path.encode() if json_path else None, out, _stream(stream)), "uw_autotune")
    return [_entry_dict(e) for e in out]


def uw_autotune_grouped(groups, batches, json_path: str | None = None, stream=None):
    """groups: a list of equal-shaped groups (lists of Matrix), e.g. the gate
    and up matrices of successive layers.  Returns one dict per batch."""
    size = len(groups[0])
    flat = [m for g in groups for m in g]
    if any(len(g) != size for g in groups):
        raise ValueError("uw_autotune_grouped: groups of different sizes")
    arr = (ctypes.c_void_p * len(flat))(*[m.handle.value for m in flat])
    bs = (ctypes.c_int64 * len(batches))(*batches)
    out = (uw_tune_entry * len(batches))()
    _check(_lib.uw_autotune_grouped(arr, size, len(groups), bs, len(batches),
                                    json_path.encode() if json_path else None, out, _stream(stream)),
           "uw_autotune_grouped")
    return [_entry_dict(e) for e in out]


def uw_plan_gemm(m: Matrix, pipeline: int, batch: int, cfg=None) -> dict:
    pl = uw_gemm_plan()
    _check(_lib.uw_plan_gemm(m.handle, pipeline, batch, _cfg(cfg), ctypes.byref(pl)), "uw_plan_gemm")
    d = {f: getattr(pl, f) for f, _ in uw_gemm_plan._fields_ if f != "reserved"}
    d["kernel"] = pl.kernel.decode()
    return d


YARDSTICK_SINK_BYTES = 4 << 20


def uw_yardstick(kind: int, src, dst, nbytes: int = 0, iters: int = 0, stream=None) -> float:
    """kind 0 copy, 1 read, 2 MFMA loop; returns the work (bytes or flops)."""
    w = ctypes.c_double()
    _check(_lib.uw_yardstick(kind, _ptr(src), _ptr(dst), nbytes, iters, _stream(stream), ctypes.byref(w)),
           "uw_yardstick")
    return w.value


def uw_sync_status(m: Matrix, stream=None) -> int:
    return _lib.uw_sync_status(m.handle, _stream(stream))


_TUNE_FIELDS = [f for f, _ in uw_tune_entry._fields_ if f != "reserved"]


def _entry_dict(e: uw_tune_entry) -> dict:
    return {f: getattr(e, f) for f in _TUNE_FIELDS}


def uw_set_tuning(entries) -> None:
    """entries: dicts with the uw_tune_entry fields (as uw_autotune returns)."""
    arr = (uw_tune_entry * max(1, len(entries)))()
    for i, d in enumerate(entries):
        for f in _TUNE_FIELDS:
            if f in d:
                setattr(arr[i], f, d[f])
    _check(_lib.uw_set_tuning(arr, len(entries)), "uw_set_tuning")


def uw_load_tuning(json_path: str) -> None:
    _check(_lib.uw_load_tuning(json_path.encode()), "uw_load_tuning")


def uw_clear_tuning() -> None:
    _check(_lib.uw_clear_tuning(), "uw_clear_tuning")


def uw_lookup_tuning(n: int, k: int, layout: int, residency: int, batch: int) -> dict | None:
    e = uw_tune_entry()
    st = _lib.uw_lookup_tuning(n, k, layout, residency, batch, ctypes.byref(e))
    if st == -6:
        return None
    _check(st, "uw_lookup_tuning")
    return _entry_dict(e)


def uw_lookup_tuning_grouped(n: int, k: int, layout: int, residency: int, group: int, batch: int) -> dict | None:
    e = uw_tune_entry()
    st = _lib.uw_lookup_tuning_grouped(n, k, layout, residency, group, batch, ctypes.byref(e))
    if st == -6:
        return None
    _check(st, "uw_lookup_tuning_grouped")
    return _entry_dict(e)


def uw_set_kernel_events(before, after) -> None:
    """before, after: torch.cuda.Event objects already recorded once (so that
    they exist), or None for both to clear."""
    b = ctypes.c_void_p(before.cuda_event) if before is not None else None
    a = ctypes.c_void_p(after.cuda_event) if after is not None else None
    _check(_lib.uw_set_kernel_events(b, a), "uw_set_kernel_events")


def uw_release_resources() -> None:
    _check(_lib.uw_release_resources(), "uw_release_resources")


# The hooks given to uw_set_allocator must outlive every handle made under
# them; the binding keeps the last ones alive for the life of the process.
_ALLOCATORS: list = []


def uw_set_allocator(alloc=None, free=None, ctx: int | None = None) -> None:
    """alloc(bytes) -> device pointer (int, 0 for failure); free(ptr).  Both
    None restores hipMalloc / hipFree."""
    if alloc is None and free is None:
        _check(_lib.uw_set_allocator(None), "uw_set_allocator")
        return
    a = uw_allocator(ALLOC_FN(lambda n, c: alloc(n) or None), FREE_FN(lambda p, c: free(p)), ctx)
    _ALLOCATORS.append(a)
    _check(_lib.uw_set_allocator(ctypes.byref(a)), "uw_set_allocator")


class TorchAllocator:
    """Device memory from torch's caching allocator for uw_set_allocator:
    each block is a uint8 tensor kept alive until the library frees it."""

    def __init__(self, device="cuda:0"):
        self.device = device
        self.live: dict[int, torch.Tensor] = {}
        self.allocs = 0
        self.frees = 0

    def alloc(self, nbytes: int) -> int:
        t = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        p = (t.data_ptr() + 255) // 256 * 256
        self.live[p] = t
        self.allocs += 1
        return p

    def free(self, p: int) -> None:
        self.live.pop(p, None)
        self.frees += 1
