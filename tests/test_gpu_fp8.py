"""GPU parity of the FP8 E4M3 codec (UWF8) through the C ABI against the oracle.

The handle's code tables, counts and sizes must equal the oracle's, and the
decoded E4M3 bytes, exponent fields and palette slots must match bit for bit.
With a prefix code, equal tables, equal symbols and equal stream word counts
fix the stream itself up to its zero padding.  Inputs are seeded synthetic
FP8 weights (N(0, 0.02) scaled per tensor to the E4M3 maximum) plus tiles of
every byte value, NaN included.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def uw():
    from decode_gemm_exp_amd import uw as _uw
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return _uw


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_fp8(uw, oracle, w_np, layout=0, sg=4):
    rows, cols = w_np.shape
    n, k = (rows, cols) if layout == 0 else (cols, rows)
    say(f"fp8 case rows={rows} cols={cols} layout={layout} sg={sg}")
    w_dev = torch.from_numpy(np.ascontiguousarray(w_np)).to(DEV)
    m = uw.uw_compress_fp8(w_dev, n, k, layout, seg_groups=sg)
    torch.cuda.synchronize()
    om = oracle.compress_fp8(w_np, seg_groups=sg, layout=layout)
    info = m.info()
    assert info.element_bits == 8
    assert info.palette_size == om.palette_size and info.verbatim_groups == om.V == 0
    assert bytes(info.palette) == om.palette.tobytes()
    assert bytes(info.code_len) == om.code_len.tobytes()
    assert list(info.code) == [int(c) for c in om.code]
    assert list(info.hist) == [int(h) for h in om.hist]
    assert list(info.coded_count) == [int(c) for c in om.coded_count]
    assert info.stream_words == om.W and info.code_bits == om.code_bits
    assert info.compressed_bytes == om.total_bytes()
    numel = w_np.size
    out = torch.empty(numel, dtype=torch.uint8, device=DEV)
    uw.uw_decode_fp8(m, out)
    e = torch.empty(numel, dtype=torch.uint8, device=DEV)
    uw.uw_decode_exponent(m, e)
    p = torch.empty(numel // 2, dtype=torch.uint8, device=DEV)
    uw.uw_transcode_palette(m, p)
    assert uw.uw_sync_status(m) == 0
    assert np.array_equal(out.cpu().numpy(), w_np.ravel())
    st, oe = om.decode_exponent()
    assert st == 0 and np.array_equal(e.cpu().numpy(), oe)
    st, op = om.transcode()
    assert st == 0 and np.array_equal(p.cpu().numpy(), op)
    return m, om


@pytest.mark.parametrize("shape,layout,sg", [
    ((37, 1024), 0, 4), ((1000, 256), 1, 2), ((96, 4096), 0, 1), ((64, 512), 0, 8),
    ((129, 192), 0, 4), ((1, 64), 0, 1), ((300, 320), 1, 64)])
def test_fp8_codec_matches_oracle(uw, oracle, shape, layout, sg):
    from decode_gemm_exp_amd import synth
    w = synth.fp8_weights(*shape, seed=21 + sg, stream=layout).numpy()
    check_fp8(uw, oracle, w, layout, sg)


def test_fp8_every_byte_value(uw, oracle):
    rng = np.random.default_rng(8)
    w = np.stack([rng.permutation(256).astype(np.uint8) for _ in range(48)])   # 48 x 256, NaN included
    check_fp8(uw, oracle, w, 0, 4)
    check_fp8(uw, oracle, w, 1, 2)   # the same stored array read as W^T[K][N]


@pytest.mark.parametrize("value", [0x00, 0x38, 0xFF])
def test_fp8_single_exponent_value(uw, oracle, value):
    # one exponent value only: a one-symbol code (every window but one invalid)
    w = np.full((64, 128), value, np.uint8)
    w[::3] ^= 0x81 & (0x87 if value != 0xFF else 0x80)   # vary sign/mantissa, keep the exponent field
    check_fp8(uw, oracle, w, 0, 4)


def test_fp8_fallback_decoder_matches(uw, oracle, monkeypatch):
    from decode_gemm_exp_amd import synth
    w = synth.fp8_weights(256, 512, seed=4).numpy()
    monkeypatch.setenv("UW_DECODE_DIRECT", "1")
    check_fp8(uw, oracle, w, 0, 4)


def test_fp8_and_bf16_calls_refuse_each_other(uw):
    from decode_gemm_exp_amd import synth
    w8 = synth.fp8_weights(64, 256, seed=2).to(DEV)
    m8 = uw.uw_compress_fp8(w8, 64, 256, 0)
    w16 = synth.weights(64, 256, seed=2).to(DEV)
    m16 = uw.uw_compress(w16, 64, 256, 0)
    torch.cuda.synchronize()
    out16 = torch.empty(64 * 256, dtype=torch.int16, device=DEV)
    out8 = torch.empty(64 * 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(Exception):
        uw.uw_decode_full(m8, out16)
    with pytest.raises(Exception):
        uw.uw_decode_fp8(m16, out8)
    with pytest.raises(Exception):
        uw.uw_export(m8)
    with pytest.raises(Exception):
        uw.uw_workspace_size(m8, 0, 1)
    assert m16.info().element_bits == 16


@pytest.mark.timeout(600)
def test_fp8_gate_shape_full_size(uw, oracle):
    """The 8B gate shape (14336 x 4096) in FP8: lossless round trip on the GPU
    and the same code tables and stream size as the oracle."""
    from decode_gemm_exp_amd import synth
    w = synth.fp8_weights(14336, 4096, seed=9).numpy()
    m, om = check_fp8(uw, oracle, w, 0, 4)
    info = m.info()
    say(f"fp8 gate: {info.bits_per_weight:.3f} bits/weight")
    assert info.bits_per_weight < 8.0
