"""Python face of the CPU oracle.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module; the product library never does.  It wraps ``uwo.cpp`` (the codec,
written one element / one bit at a time) and adds the fp64 GEMM reference.

Sources: [EVC] "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
(easyvibecoding.app/curated/736), cited by section heading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uwo.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

SECTION_NAMES = ("sm", "vflags", "vrank", "vexp", "seg_off", "stream")
UWO_OK = 0
UWO_ERR_CORRUPT = -5


def build(force: bool = False) -> str:
    """Compile uwo.cpp with the host compiler (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall",
                               "-Wextra", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB if os.path.exists(_LIB) else build()
        L = ctypes.CDLL(path)
        vp, u64, u32, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        L.uwo_compress.restype = vp
        L.uwo_compress.argtypes = [vp, u64, u64, u32, u32, ctypes.POINTER(i32)]
        L.uwo_compress_fp8.restype = vp
        L.uwo_compress_fp8.argtypes = [vp, u64, u64, u32, u32, ctypes.POINTER(i32)]
        L.uwo_decode_fp8.argtypes = [vp, vp]
        L.uwo_free.argtypes = [vp]
        L.uwo_scalars.argtypes = [vp, vp]
        L.uwo_tables.argtypes = [vp, vp, vp, vp, vp, vp]
        L.uwo_section.argtypes = [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(u64)]
        L.uwo_poke_u32.argtypes = [vp, i32, u64, u32]
        for name in ("uwo_decode_exponent", "uwo_decode_full", "uwo_transcode"):
            getattr(L, name).argtypes = [vp, vp]
        L.uwo_export.restype = u64
        L.uwo_export.argtypes = [vp, vp, u64]
        L.uwo_package_merge.argtypes = [vp, i32, i32, vp]
        L.uwo_canonical.argtypes = [vp, i32, vp]
        L.uwo_gemm_ref.argtypes = [vp, u64, u64, vp, u64, u32, vp, u64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


@dataclass
class Compressed:
    """One matrix compressed by the oracle; owns the C++ object."""
    handle: int
    rows: int
    cols: int
    numel: int
    groups: int
    segments: int
    flag_words: int
    seg_groups: int
    layout: int
    palette_size: int
    n_coded: int
    V: int
    W: int
    code_bits: int
    palette: np.ndarray
    code_len: np.ndarray
    code: np.ndarray
    hist: np.ndarray
    coded_count: np.ndarray
    fp8: bool = False

    def section(self, name: str) -> np.ndarray:
        ptr, nbytes = ctypes.c_void_p(), ctypes.c_uint64()
        st = lib().uwo_section(self.handle, SECTION_NAMES.index(name), ctypes.byref(ptr),
                               ctypes.byref(nbytes))
        assert st == UWO_OK
        buf = (ctypes.c_uint8 * nbytes.value).from_address(ptr.value) if nbytes.value else b""
        raw = np.frombuffer(bytes(buf), dtype=np.uint8)
        return raw if name in ("sm", "vexp") else raw.view(np.uint32)

    def poke(self, name: str, index: int, value: int) -> None:
        assert lib().uwo_poke_u32(self.handle, SECTION_NAMES.index(name), index, value) == UWO_OK

    def decode_exponent(self) -> tuple[int, np.ndarray]:
        out = np.zeros(self.numel, dtype=np.uint8)
        st = lib().uwo_decode_exponent(self.handle, _ptr(out))
        return st, out

    def decode_full(self) -> tuple[int, np.ndarray]:
        out = np.zeros(self.numel, dtype=np.uint16)
        st = lib().uwo_decode_full(self.handle, _ptr(out))
        return st, out

    def decode_fp8(self) -> tuple[int, np.ndarray]:
        """UWF8 handles: the original E4M3 bytes."""
        out = np.zeros(self.numel, dtype=np.uint8)
        st = lib().uwo_decode_fp8(self.handle, _ptr(out))
        return st, out

    def transcode(self) -> tuple[int, np.ndarray]:
        out = np.zeros(self.numel // 2, dtype=np.uint8)
        st = lib().uwo_transcode(self.handle, _ptr(out))
        return st, out

    def export(self) -> bytes:
        n = lib().uwo_export(self.handle, None, 0)
        buf = np.zeros(n, dtype=np.uint8)
        lib().uwo_export(self.handle, _ptr(buf), n)
        return buf.tobytes()

    def total_bytes(self, header: int = 2304) -> int:
        """Compressed size: header plus the six sections, unpadded (the kept
        section is one byte per weight for BF16, half a byte for FP8)."""
        kept = self.numel // 2 if self.fp8 else self.numel
        return (header + kept + 8 * self.flag_words + 64 * self.V
                + 4 * (self.segments + 1) + 4 * (self.W + 2))

    def free(self) -> None:
        if self.handle:
            lib().uwo_free(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def compress(w_stored: np.ndarray, seg_groups: int = 4, layout: int = 0) -> Compressed:
    """Compress the stored 2-D uint16 array (bf16 bit patterns)."""
    w = np.ascontiguousarray(w_stored, dtype=np.uint16)
    assert w.ndim == 2
    st = ctypes.c_int(0)
    h = lib().uwo_compress(_ptr(w), w.shape[0], w.shape[1], seg_groups, layout, ctypes.byref(st))
    if not h:
        raise ValueError(f"oracle compress failed with status {st.value}")
    return _wrap(h)


def compress_fp8(w_stored: np.ndarray, seg_groups: int = 4, layout: int = 0) -> Compressed:
    """Compress the stored 2-D uint8 array of FP8 E4M3 bytes (UWF8 reading:
    the exponent field coded as the BF16 exponent byte is, sign+mantissa
    nibbles kept)."""
    w = np.ascontiguousarray(w_stored, dtype=np.uint8)
    assert w.ndim == 2
    st = ctypes.c_int(0)
    h = lib().uwo_compress_fp8(_ptr(w), w.shape[0], w.shape[1], seg_groups, layout, ctypes.byref(st))
    if not h:
        raise ValueError(f"oracle FP8 compress failed with status {st.value}")
    c = _wrap(h)
    c.fp8 = True
    return c


def _wrap(h) -> Compressed:
    sc = np.zeros(14, dtype=np.uint64)
    lib().uwo_scalars(h, _ptr(sc))
    pal = np.zeros(16, np.uint8)
    ln = np.zeros(16, np.uint8)
    cd = np.zeros(16, np.uint16)
    hist = np.zeros(256, np.uint64)
    cc = np.zeros(16, np.uint64)
    lib().uwo_tables(h, _ptr(pal), _ptr(ln), _ptr(cd), _ptr(hist), _ptr(cc))
    s = [int(v) for v in sc]
    return Compressed(h, s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], s[8], s[9], s[10],
                      s[11], s[12], pal, ln, cd, hist, cc)


def package_merge(weights, lmax: int = 12) -> np.ndarray:
    w = np.ascontiguousarray(weights, dtype=np.uint64)
    out = np.zeros(len(w), np.uint8)
    st = lib().uwo_package_merge(_ptr(w), len(w), lmax, _ptr(out))
    if st != UWO_OK:
        raise ValueError("package-merge needs 2 <= n <= 2**lmax")
    return out


def canonical(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(len(ln), np.uint16)
    lib().uwo_canonical(_ptr(ln), len(ln), _ptr(out))
    return out


# ---- GEMM reference ---------------------------------------------------------
# y[b][n] = sum_k x[b][k] * W[n][k] on the ORIGINAL weights, accumulated in
# fp64, with the magnitude sum A[b][n] = sum_k |x[b][k] * W[n][k]| used by the
# per-element bound |y_gpu - y| <= 2^-10 * A.  ([EVC] "重建矩陣乘法核心運作":
# the reconstructive matmul computes the same product as a matmul on the
# uncompressed weights; the bound is the stated acceptance rule.)  The sums are
# uwo.cpp's ``gemm_ref`` (k ascending, one column at a time); this wrapper only
# hands disjoint column ranges to worker threads.

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    return f32.astype(np.float64)


def logical_weight(w_stored: np.ndarray, layout: int) -> np.ndarray:
    """W as [N][K] whatever the stored layout (0: stored W, 1: stored W^T)."""
    return w_stored if layout == 0 else w_stored.T


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gemm_ref(x_bits: np.ndarray, w_stored: np.ndarray, layout: int,
             cols: np.ndarray | None = None, threads: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(y, A) in fp64 for y = x . W^T; ``cols`` restricts to output columns n."""
    import concurrent.futures as cf
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_stored, dtype=np.uint16)
    assert x.ndim == 2 and w.ndim == 2
    batch, K = x.shape
    N = w.shape[0] if layout == 0 else w.shape[1]
    assert (w.shape[1] if layout == 0 else w.shape[0]) == K
    sel = np.arange(N, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nc = len(sel)
    y = np.zeros((batch, nc), np.float64)
    A = np.zeros((batch, nc), np.float64)
    nt = max(1, min(threads or default_threads(), nc))
    bounds = [nc * t // nt for t in range(nt + 1)]

    def run(t: int) -> int:
        c0, c1 = bounds[t], bounds[t + 1]
        if c1 <= c0:
            return UWO_OK
        yp = np.zeros((batch, c1 - c0), np.float64)
        ap = np.zeros((batch, c1 - c0), np.float64)
        part = np.ascontiguousarray(sel[c0:c1])
        st = lib().uwo_gemm_ref(_ptr(x), batch, K, _ptr(w), N, layout, _ptr(part), c1 - c0,
                                _ptr(yp), _ptr(ap))
        y[:, c0:c1] = yp
        A[:, c0:c1] = ap
        return st

    if nt == 1:
        sts = [run(0)]
    else:
        with cf.ThreadPoolExecutor(max_workers=nt) as ex:
            sts = list(ex.map(run, range(nt)))
    assert all(st == UWO_OK for st in sts), "oracle gemm_ref rejected its arguments"
    return y, A


def gemm_check(y_gpu: np.ndarray, y_ref: np.ndarray, A: np.ndarray) -> tuple[bool, float]:
    """Pass iff |y_gpu - y_ref| <= 2^-10 * A element-wise (exact where A == 0).

    Returns (ok, worst ratio err / (2^-10 A)).
    """
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = np.ldexp(A, -10)
    ok = bool(np.all(err <= bound))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return ok, float(ratio.max()) if ratio.size else 0.0
