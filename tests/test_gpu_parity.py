"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Compressed streams and decoded weights must match bit for bit; GEMM outputs
must satisfy |y - y_ref| <= 2^-10 * sum_k |x_k w_k| per element against the
fp64 oracle on the original weights; one-hot probes must reproduce weights
exactly.  Every workload is seeded synthetic data (decode_gemm_exp_amd.synth).
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


@pytest.fixture(scope="module")
def synth():
    from decode_gemm_exp_amd import synth as _s
    return _s


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.astype(np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def gpu_compress(uw, w_dev, n, k, layout, sg=4):
    m = uw.uw_compress(w_dev, n, k, layout, seg_groups=sg)
    torch.cuda.synchronize()
    return m


def check_codec(uw, oracle, w_dev, n, k, layout, sg=4, check_transcode=True):
    """Compress on the GPU, compare the UWF1 blob with the oracle's, decode."""
    w_np = bits(w_dev)
    m = gpu_compress(uw, w_dev, n, k, layout, sg)
    om = oracle.compress(w_np, seg_groups=sg, layout=layout)
    blob = uw.uw_export(m)
    oblob = om.export()
    assert len(blob) == len(oblob)
    if blob != oblob:
        a = np.frombuffer(blob, np.uint8)
        b = np.frombuffer(oblob, np.uint8)
        bad = np.nonzero(a != b)[0]
        pytest.fail(f"UWF1 blob differs at {len(bad)} bytes, first at {bad[:8]}")
    numel = w_np.size
    out = torch.empty(numel, dtype=torch.int16, device=DEV)
    uw.uw_decode_full(m, out)
    e = torch.empty(numel, dtype=torch.uint8, device=DEV)
    uw.uw_decode_exponent(m, e)
    assert uw.uw_sync_status(m) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w_np.ravel())
    assert np.array_equal(e.cpu().numpy(), ((w_np.ravel() >> 7) & 0xFF).astype(np.uint8))
    if check_transcode:
        p = torch.empty(numel // 2, dtype=torch.uint8, device=DEV)
        uw.uw_transcode_palette(m, p)
        st, op = om.transcode()
        assert st == 0
        assert np.array_equal(p.cpu().numpy(), op)
    return m, om


def run_pipeline(uw, m, pipeline, x, cfg=None):
    info = m.info()
    y = torch.full((x.shape[0], info.n), float("nan"), dtype=torch.float32, device=DEV)
    ws_bytes = uw.uw_workspace_size_cfg(m, pipeline, x.shape[0], cfg) if cfg else uw.uw_workspace_size(
        m, pipeline, x.shape[0])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    uw.uw_matmul_reconstruct(m, pipeline, x, y, ws, cfg=cfg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_gemm(oracle, y, x_np, w_np, layout, cols=None, what=""):
    y_ref, A = oracle.gemm_ref(x_np, w_np, layout, cols=cols)
    yy = y if cols is None else y[:, cols]
    assert np.all(np.isfinite(yy)), what
    ok, worst = oracle.gemm_check(yy, y_ref, A)
    assert ok, f"{what}: worst err/bound = {worst:.3g}"
    return worst


# ----------------------------------------------------------------- small edge cases

@pytest.mark.parametrize("shape,layout,sg", [
    ((256, 512), 0, 8), ((1, 64), 0, 1), ((3, 192), 0, 2), ((200, 192), 0, 64), ((257, 320), 0, 4),
    ((72, 128), 1, 8), ((200, 64), 1, 1)])
def test_codec_small_shapes(uw, synth, oracle, shape, layout, sg):
    r, c = shape
    say(f"codec small shape={shape} layout={layout} sg={sg}")
    w = synth.weights(r, c, 0.02, 0.01, 12, seed=31 + r + c).to(DEV)
    n, k = (r, c) if layout == 0 else (c, r)
    check_codec(uw, oracle, w, n, k, layout, sg)


@pytest.mark.parametrize("shape,sg", [((512, 1024), 4), ((300, 192), 1)])
def test_codec_run_palette(uw, synth, oracle, shape, sg):
    """Weights without outliers: the palette is a run of consecutive
    exponents, which the decoders look up with a bytewise add."""
    r, c = shape
    say(f"codec run palette shape={shape} sg={sg}")
    w = run_palette_weights(synth, r, c, 5 + r).to(DEV)
    m, _ = check_codec(uw, oracle, w, r, c, 0, sg)
    assert _palette_is_run(m)


def test_codec_all_bf16_patterns(uw, oracle):
    say("codec all 65536 bf16 patterns")
    rng = np.random.default_rng(1)
    w_np = rng.permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16).reshape(1024, 64)
    for sg in (1, 8, 64):
        check_codec(uw, oracle, to_dev_bits(w_np), 1024, 64, 0, sg)


def test_codec_degenerate(uw, oracle):
    say("codec degenerate: single exponent, all verbatim, none verbatim")
    one = np.full((4, 128), 0x3F80, np.uint16)
    one[1, 5] = 0xBF80
    check_codec(uw, oracle, to_dev_bits(one), 4, 128, 0, 2)
    base = np.array([(e << 7) for e in range(10, 28)] + [0x3C00] * 46, np.uint16)
    allv = np.tile(base, 8).reshape(4, 128)
    m, om = check_codec(uw, oracle, to_dev_bits(allv), 4, 128, 0, 8)
    assert m.info().verbatim_groups == 8 and m.info().stream_words == 0
    nov = ((np.arange(512, dtype=np.uint16) % 16 + 100) << 7).reshape(2, 256)
    check_codec(uw, oracle, to_dev_bits(nov), 2, 256, 0, 8)


def test_import_oracle_blob_and_decode(uw, synth, oracle):
    """The decoder on streams written by the oracle (independent of GPU compress)."""
    say("import oracle blob")
    w_np = synth.bits_numpy(synth.weights(128, 512, 0.02, 0.003, 11, seed=5))
    om = oracle.compress(w_np, seg_groups=4)
    m = uw.uw_import(om.export())
    out = torch.empty(w_np.size, dtype=torch.int16, device=DEV)
    uw.uw_decode_full(m, out)
    assert uw.uw_sync_status(m) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w_np.ravel())


def test_decoder_flags_invalid_code(uw, oracle):
    """A '1' bit where the only codeword is '0', planted in the oracle's blob on the host."""
    say("decoder corruption flag")
    w_np = np.full((2, 128), 0x3F80, np.uint16)
    om = oracle.compress(w_np, seg_groups=1)
    om.poke("stream", 0, 0x80000000)
    m = uw.uw_import(om.export())
    e = torch.empty(w_np.size, dtype=torch.uint8, device=DEV)
    uw.uw_decode_exponent(m, e)
    assert uw.uw_sync_status(m) == -5
    # the flag clears after being reported; a clean decode reports ok
    m2 = uw.uw_import(oracle.compress(w_np, seg_groups=1).export())
    uw.uw_decode_exponent(m2, e)
    assert uw.uw_sync_status(m2) == 0


# ----------------------------------------------------------------- GEMM edge cases

@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("batch", [1, 3, 8, 17, 100])
def test_gemm_ragged_all_pipelines(uw, synth, oracle, layout, batch):
    n, k = 200, 192 if layout == 0 else 200
    if layout == 1:
        n, k = 192, 200      # stored [K=200][N=192]: K tail not a multiple of 64
    r, c = (n, k) if layout == 0 else (k, n)
    say(f"gemm ragged layout={layout} batch={batch}")
    w = synth.weights(r, c, 0.02, 0.01, 10, seed=77 + batch).to(DEV)
    x = synth.activations(batch, k, seed=3 + batch).to(DEV)
    m = gpu_compress(uw, w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    w_np, x_np = bits(w), bits(x)
    for p in range(4):
        y = run_pipeline(uw, m, p, x)
        check_gemm(oracle, y, x_np, w_np, layout, what=f"pipeline {p}")
    # every variant, forced (the register-fed ones, last, take stored [N][K] only)
    nk_only = set(rf_variants(uw)) | set(wide_variants(uw))
    for v in range(1, uw.variant_count() + 1):
        if layout == 1 and v in nk_only:
            with pytest.raises(uw.UwError) as ei:
                run_pipeline(uw, m, 3, x, cfg={"variant": v})
            assert ei.value.status == uw.UW_ERR_UNSUPPORTED
            continue
        y = run_pipeline(uw, m, 3, x, cfg={"variant": v})
        check_gemm(oracle, y, x_np, w_np, layout, what=f"variant {v}")


def RF_FIRST(uw):
    """The first register-fed variant (they follow the GEMV and the LDS tiles)."""
    return min(rf_variants(uw))


def rf_variants(uw):
    """The register-fed variants, found from the kernel each one plans."""
    w = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    m = uw.uw_compress(w, 64, 128, 0)
    return [v for v in range(1, uw.variant_count() + 1)
            if uw.uw_plan_gemm(m, 0, 16, {"variant": v})["kernel"].startswith("k_mfma_rf")]


def wide_variants(uw):
    """The LDS tiles with 128-wide K steps (stored [N][K]): the last template
    argument of the kernel each variant plans is the K step in units of 64."""
    w = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    m = uw.uw_compress(w, 64, 128, 0)
    out = []
    for v in range(1, uw.variant_count() + 1):
        kern = uw.uw_plan_gemm(m, 0, 16, {"variant": v})["kernel"]
        if kern.startswith("k_mfma2<") and kern.endswith(", 2>"):
            out.append(v)
    assert len(out) == 8, out
    return out


def eight_wave_variants(uw):
    """The eight-wave 128x256 and 64x128 tiles with 64-wide K steps (either
    layout), found from the kernel each variant plans."""
    w = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    m = uw.uw_compress(w, 64, 128, 0)
    out = [v for v in range(1, uw.variant_count() + 1)
           if any(uw.uw_plan_gemm(m, 0, 16, {"variant": v})["kernel"].endswith(t)
                  for t in (", 128, 256, 2, 8, false, 1>", ", 64, 128, 2, 8, false, 1>"))]
    assert len(out) == 2, out
    return out


# the small tiles (64x128, 32x128, 32x256, and the eight-wave 128x256 and
# 64x128) over K slices of 1, 2, 5 and an
# odd or even number of steps, forced K splits that leave uneven slices,
# both layouts, a ragged batch (and a ragged N where the layout allows it:
# stored [K][N] keeps N a multiple of 64); for stored [N][K] also the tiles
# with 128-wide K steps, where K = 64, 320 and 2112 end half way through a
# step and the forced splits of 2112 (17 steps) leave a half-step slice end
# and, at 7 slices, an empty last slice
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("k", [64, 128, 320, 2112])
def test_gemm_small_tiles_step_counts(uw, synth, oracle, layout, k):
    n, batch = (328 if layout == 0 else 320), 45
    r, c = (n, k) if layout == 0 else (k, n)
    say(f"gemm small tiles layout={layout} k={k}")
    w = synth.weights(r, c, 0.02, 0.01, 10, seed=501 + k + layout).to(DEV)
    x = synth.activations(batch, k, seed=502 + k).to(DEV)
    m = gpu_compress(uw, w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    w_np, x_np = bits(w), bits(x)
    splits = (1, 3, 7) if k == 2112 else (1,)
    for v in (2 + 0, 2 + 5, 2 + 6) + tuple(eight_wave_variants(uw)) + (tuple(wide_variants(uw)) if layout == 0 else ()):
        for sk in splits:
            for p in (0, 1, 3):
                y = run_pipeline(uw, m, p, x, cfg={"variant": v, "split_k": sk})
                check_gemm(oracle, y, x_np, w_np, layout, what=f"pipeline {p} variant {v} split {sk}")


# mid batch: the default 256x256 tiles with K split across blocks (33 K
# steps, so slices are uneven), ragged N and batch tiles, both layouts, all
# pipelines; then the four- and eight-wave tiles with forced odd splits
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("batch", [200, 300])
def test_gemm_mid_batch_split(uw, synth, oracle, layout, batch):
    n, k = (600, 2112) if layout == 0 else (576, 2112)
    r, c = (n, k) if layout == 0 else (k, n)
    say(f"gemm mid batch layout={layout} batch={batch}")
    w = synth.weights(r, c, 0.02, 0.005, 10, seed=91 + batch + layout).to(DEV)
    x = synth.activations(batch, k, seed=5 + batch).to(DEV)
    m = gpu_compress(uw, w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    w_np, x_np = bits(w), bits(x)
    for p in range(4):
        y = run_pipeline(uw, m, p, x)
        check_gemm(oracle, y, x_np, w_np, layout, what=f"pipeline {p}")
    # ... and the single-rebuild 512x128 tile (x in registers), split and not,
    # and ([N][K]) the 128x128 and both single-rebuild tiles with 128-wide K
    # steps
    cases = ((2 + 7, 3), (2 + 4, 5), (2 + 8, 3), (2 + 8, 1))
    if layout == 0:
        wide = wide_variants(uw)
        cases += tuple((v, sk) for v in (wide[1], wide[4], wide[5]) for sk in (1, 3))
    for v, sk in cases:
        for p in (0, 3):
            y = run_pipeline(uw, m, p, x, cfg={"variant": v, "split_k": sk})
            check_gemm(oracle, y, x_np, w_np, layout, what=f"pipeline {p} variant {v} split {sk}")


# a palette grid whose last round of resident blocks is short: 72 N tiles x 8
# M tiles of 128x128 on 256 CUs holding two blocks each leaves 64 blocks for a
# second round, so the default splits K in two; the BF16 pipeline keeps one
# slice; a ragged batch (1000 rows)
def test_gemm_palette_tail_split(uw, synth, oracle):
    n, k, batch = 9216, 1024, 1000
    say(f"gemm palette tail split n={n} k={k} batch={batch}")
    w = synth.weights(n, k, 0.02, 0.005, 10, seed=417).to(DEV)
    x = synth.activations(batch, k, seed=418).to(DEV)
    m = gpu_compress(uw, w, n, k, 0)
    uw.uw_transcode_palette(m, None)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert uw.uw_workspace_size(m, 3, batch) >= 2 * batch * n * 4, "expected a two-slice K split"
    w_np, x_np = bits(w), bits(x)
    for p in range(4):
        y = run_pipeline(uw, m, p, x)
        check_gemm(oracle, y, x_np, w_np, 0, what=f"pipeline {p}")


# register-fed MFMA kernels (stored [N][K]), x per wave and x shared through
# LDS: row counts that leave partial 32-, 64- and 128-row blocks (waves with
# no rows left still stage x), K with a partial 128-wide window (K % 128 ==
# 64), a K whose windows split unevenly over the four waves, batches across
# the 16-row groups and past the 64-row launch limit, K slices, verbatim-rich
# and run palettes
@pytest.mark.parametrize("n,k,outliers", [(200, 1088, 0.01), (70, 4096, 0.0), (96, 320, 0.02)])
def test_register_fed_mfma(uw, synth, oracle, n, k, outliers):
    say(f"register-fed mfma n={n} k={k} outliers={outliers}")
    w = synth.weights(n, k, 0.02, outliers, 10, seed=n * 7 + k).to(DEV)
    m = gpu_compress(uw, w, n, k, 0)
    uw.uw_transcode_palette(m, None)
    w_np = bits(w)
    for batch in (1, 5, 16, 17, 40, 64, 65, 130):
        x = synth.activations(batch, k, seed=batch + 11).to(DEV)
        x_np = bits(x)
        for v in rf_variants(uw):
            for p in range(4):
                y = run_pipeline(uw, m, p, x, cfg={"variant": v})
                check_gemm(oracle, y, x_np, w_np, 0, what=f"batch {batch} variant {v} pipeline {p}")
            for split in (2, 3):
                y = run_pipeline(uw, m, 3, x, cfg={"variant": v, "split_k": split})
                check_gemm(oracle, y, x_np, w_np, 0, what=f"batch {batch} variant {v} split {split}")


def _palette_is_run(m):
    info = m.info()
    pal = list(info.palette)[:info.palette_size]
    return pal[-1] - pal[0] == info.palette_size - 1


def run_palette_weights(synth, r, c, seed):
    """N(0, 0.02) weights with magnitudes below 2^-12 raised to it: every
    exponent lies in one window narrower than the palette, so the palette is
    a run by construction (drawn values alone leave a few rare small
    exponents whose sampled counts can put a gap into the top 16)."""
    f = synth.weights(r, c, 0.02, 0.0, 0, seed=seed).float()
    small = f.abs() < 2.0 ** -12
    f = torch.where(small, torch.where(f < 0, -(2.0 ** -12), 2.0 ** -12), f)
    return f.to(torch.bfloat16)


# stored shapes for the vector (small-batch) kernels: NK rows with K a multiple
# of 4096 / 2048 / 1024 (the pipelined kernel, U = 4 / 2 / 1), an NK shape it
# does not cover, and KN shapes with several K slices, odd row-pair counts and
# a partial last column block (1024 columns: whole blocks, the flag words
# are wave-uniform scalar loads); 7173 rows spread over 256 CUs take 15
# waves per block with a partly filled last round.  outlier_frac picks verbatim-rich weights (a
# palette with a gap) or none (a palette that is a run of exponents).
@pytest.mark.parametrize("n,k,layout,outliers", [
    (300, 4096, 0, 0.01), (70, 2048, 0, 0.0), (33, 1024, 0, 0.01), (200, 3072, 0, 0.0), (40, 1088, 0, 0.01),
    (7173, 1024, 0, 0.01),
    (192, 2008, 1, 0.01), (1088, 1032, 1, 0.0), (64, 520, 1, 0.01), (1024, 2056, 1, 0.01),
])
def test_gemv_shapes(uw, synth, oracle, n, k, layout, outliers):
    r, c = (n, k) if layout == 0 else (k, n)
    say(f"gemv shapes n={n} k={k} layout={layout} outliers={outliers}")
    w = (run_palette_weights(synth, r, c, n + k) if outliers == 0.0
         else synth.weights(r, c, 0.02, outliers, 10, seed=n + k)).to(DEV)
    m = gpu_compress(uw, w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    assert _palette_is_run(m) == (outliers == 0.0)
    w_np = bits(w)
    for batch in (1, 2, 3, 8, 9):
        x = synth.activations(batch, k, seed=batch).to(DEV)
        x_np = bits(x)
        for p in range(4):
            y = run_pipeline(uw, m, p, x, cfg={"variant": 1})
            check_gemm(oracle, y, x_np, w_np, layout, what=f"batch {batch} pipeline {p}")
        if layout == 1:
            for split in (1, 7):
                y = run_pipeline(uw, m, 3, x, cfg={"variant": 1, "split_k": split})
                check_gemm(oracle, y, x_np, w_np, layout, what=f"batch {batch} split {split}")


def test_grouped_matmul(uw, synth, oracle):
    """uw_matmul_reconstruct_grouped: matrices that all take the GEMV share
    one launch (a run palette next to a palette with gaps runs with the
    general lookup; more than eight rows go in chunks); a group of five, a
    group holding a [K][N] matrix and batches that resolve to MFMA kernels
    are launched one matrix at a time; at 5 to 7 rows a group of small
    matrices takes the grouped GEMV by default, at 8 to 32 rows one launch of
    32-row tiles; where the group's kernel is an LDS tile (80 and 300 rows,
    a forced odd split, a [K][N]-only group) the whole group is one launch.  Every column block is checked against
    the fp64 reference."""
    say("grouped matmul")
    k = 2048
    specs = [(700, 0, 0.0), (300, 0, 0.002), (1100, 0, 0.0), (64, 0, 0.002), (520, 0, 0.0), (384, 1, 0.002),
             (320, 1, 0.0)]
    ms, wnps = [], []
    for i, (n, layout, out) in enumerate(specs):
        r, c = (n, k) if layout == 0 else (k, n)
        w = (run_palette_weights(synth, r, c, 300 + i) if out == 0.0
             else synth.weights(r, c, 0.02, out, 10, seed=300 + i)).to(DEV)
        m = gpu_compress(uw, w, n, k, layout)
        uw.uw_transcode_palette(m, None)
        ms.append(m)
        wnps.append(bits(w))
    assert _palette_is_run(ms[0]) and not _palette_is_run(ms[1])
    groups = [(0, 1), (0, 1, 2, 3), (1, 3), (0, 1, 2, 3, 4), (0, 5, 1), (5, 6)]
    for idx in groups:
        sub = [ms[i] for i in idx]
        N = sum(ms[i].info().n for i in idx)
        for batch, cfg in ((1, None), (3, None), (7, None), (9, {"variant": 1}), (24, None), (80, None),
                           (300, None), (100, {"variant": 2 + 7, "split_k": 3})):
            x = synth.activations(batch, k, seed=batch + 7).to(DEV)
            x_np = bits(x)
            for p in (0, 1, 3):
                y = torch.full((batch, N), float("nan"), dtype=torch.float32, device=DEV)
                ws_bytes = uw.uw_workspace_size_grouped(sub, p, batch, cfg)
                ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
                uw.uw_matmul_reconstruct_grouped(sub, p, x, y, ws, cfg=cfg)
                torch.cuda.synchronize()
                yn = y.cpu().numpy()
                col = 0
                for i in idx:
                    n = ms[i].info().n
                    check_gemm(oracle, yn[:, col:col + n], x_np, wnps[i], specs[i][1],
                               what=f"group {idx} batch {batch} pipeline {p} matrix {i}")
                    col += n


@pytest.mark.parametrize("layout", [0, 1])
def test_gemm_one_hot_exact(uw, synth, oracle, layout):
    """x row j one-hot at k_j: y[j][n] must equal W[n][k_j] exactly."""
    n, k = 256, 320
    r, c = (n, k) if layout == 0 else (k, n)
    say(f"one-hot layout={layout}")
    w = synth.weights(r, c, 0.02, 0.02, 12, seed=9).to(DEV)
    w_np = bits(w)
    W = w_np if layout == 0 else w_np.T
    m = gpu_compress(uw, w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    for batch in (1, 5, 40, 130):
        ks = (np.arange(batch) * 37) % k
        x_np = np.zeros((batch, k), np.uint16)
        x_np[np.arange(batch), ks] = 0x3F80    # 1.0
        x = to_dev_bits(x_np)
        expect = oracle.bf16_to_f64(W[:, ks].T).astype(np.float32)
        for p in range(4):
            y = run_pipeline(uw, m, p, x)
            assert np.array_equal(y, expect), f"batch {batch} pipeline {p}"
        if layout == 0:   # output placement of the register-fed kernels
            for v in rf_variants(uw):
                y = run_pipeline(uw, m, 2, x, cfg={"variant": v})
                assert np.array_equal(y, expect), f"batch {batch} variant {v}"


def test_gemm_identity_exact(uw, synth):
    k = 128
    w_np = np.zeros((k, k), np.uint16)
    w_np[np.arange(k), np.arange(k)] = 0x3F80
    x = synth.activations(20, k, seed=4).to(DEV)
    m = gpu_compress(uw, to_dev_bits(w_np), k, k, 0)
    uw.uw_transcode_palette(m, None)
    xf = x.float().cpu().numpy()
    for p in range(4):
        assert np.array_equal(run_pipeline(uw, m, p, x), xf)


def test_determinism(uw, synth):
    w = synth.weights(512, 1024, 0.02, 0.001, 10, seed=12).to(DEV)
    a = uw.uw_export(gpu_compress(uw, w, 512, 1024, 0))
    b = uw.uw_export(gpu_compress(uw, w, 512, 1024, 0))
    assert a == b


def test_sequence_runner_matches_single_calls(uw, synth, oracle):
    say("sequence runner")
    mats, jobs, ref = [], [], []
    x = synth.activations(4, 512, seed=8).to(DEV)
    for i, (n, k, layout) in enumerate([(384, 512, 0), (256, 512, 0), (512, 384, 1)]):
        r, c = (n, k) if layout == 0 else (k, n)
        w = synth.weights(r, c, 0.02, 0.002, 10, seed=50 + i).to(DEV)
        m = gpu_compress(uw, w, n, k, layout)
        uw.uw_transcode_palette(m, None)
        xi = x if k == 512 else synth.activations(4, k, seed=9).to(DEV)
        for p in range(4):
            y = torch.zeros((4, n), dtype=torch.float32, device=DEV)
            jobs.append(uw.Job(m, p, xi, y))
            ref.append((bits(w), bits(xi), layout))
        mats.append(m)
    ws = torch.empty(uw.uw_sequence_workspace_size(jobs), dtype=torch.uint8, device=DEV)
    for dcus in (0, 64):
        for j in jobs:
            j.y.fill_(float("nan"))
        uw.uw_run_sequence(jobs, dcus, ws)
        torch.cuda.synchronize()
        for j, (w_np, x_np, layout) in zip(jobs, ref):
            check_gemm(oracle, j.y.cpu().numpy(), x_np, w_np, layout, what=f"seq cus={dcus}")


def test_alternating_residency_sequence(uw, synth, oracle):
    """Hard/easy layers: easy matrices keep only their palette indices
    (Huffman stream dropped, direct palette), hard ones only the Huffman
    stream (decoded at run time).  A sequence alternating them, with each
    hard matrix's decode running beside the previous GEMM on every CU or on
    a CU share, matches the fp64 reference; sections that were dropped are
    refused."""
    say("alternating residency")
    k = 1024
    x = synth.activations(3, k, seed=12).to(DEV)
    jobs, ref = [], []
    for layer in range(4):
        for i, (n, layout) in enumerate([(640, 0), (320, 0), (512, 1)]):
            r, c = (n, k) if layout == 0 else (k, n)
            w = synth.weights(r, c, 0.02, 0.002, 9, seed=200 + 10 * layer + i).to(DEV)
            m = gpu_compress(uw, w, n, k, layout)
            if layer % 2 == 0:
                uw.uw_transcode_palette(m, None)
                uw.uw_drop_stream(m)
                info = m.info()
                assert info.has_palette_idx and not info.has_stream
                with pytest.raises(uw.UwError):
                    uw.uw_decode_exponent(m, torch.empty(r * c, dtype=torch.uint8, device=DEV))
                pipe = 3
            else:
                assert not m.info().has_palette_idx
                pipe = 1 if i != 1 else 2
            y = torch.full((3, n), float("nan"), dtype=torch.float32, device=DEV)
            jobs.append(uw.Job(m, pipe, x, y))
            ref.append((bits(w), layout))
    ws = torch.empty(uw.uw_sequence_workspace_size(jobs), dtype=torch.uint8, device=DEV)
    x_np = bits(x)
    for dcus in (0, 96, 100000):
        for j in jobs:
            j.y.fill_(float("nan"))
        uw.uw_run_sequence(jobs, dcus, ws)
        torch.cuda.synchronize()
        for j, (w_np, layout) in zip(jobs, ref):
            check_gemm(oracle, j.y.cpu().numpy(), x_np, w_np, layout, what=f"alternating cus={dcus}")


@pytest.mark.parametrize("sg", [1, 8, 64])
def test_fallback_decoder_matches(uw, synth, oracle, monkeypatch, sg):
    """The direct-from-HBM decoder (used when a wave's stream does not fit in
    LDS) gives the same bytes as the oracle."""
    say(f"fallback decoder sg={sg}")
    monkeypatch.setenv("UW_DECODE_DIRECT", "1")
    w = synth.weights(1024, 1024, 0.02, 0.002, 11, seed=40 + sg).to(DEV)
    check_codec(uw, oracle, w, 1024, 1024, 0, sg)


def test_sequence_per_job_split_and_autotune(uw, synth, oracle):
    """Per-job CU splits in one sequence, and the autotuner's choices, keep
    results within tolerance."""
    say("sequence per-job split + autotune")
    specs = [(384, 512, 0), (384, 512, 0), (512, 384, 1)]
    mats, wnps = [], []
    for i, (n, k, layout) in enumerate(specs):
        r, c = (n, k) if layout == 0 else (k, n)
        w = synth.weights(r, c, 0.02, 0.002, 10, seed=60 + i).to(DEV)
        m = gpu_compress(uw, w, n, k, layout)
        uw.uw_transcode_palette(m, None)
        mats.append(m)
        wnps.append(bits(w))
    tuned = uw.uw_autotune(mats, [0, 1, 2], [2, 24], max_passes=1)
    assert len(tuned) == 6
    for e in tuned:
        assert 0 <= e["pipeline"] <= 3 and 0 <= e["variant"] <= uw.variant_count() and e["sequence_us"] > 0
    for batch in (2, 24):
        choice = {e["projection"]: e for e in tuned if e["batch"] == batch}
        jobs, refs = [], []
        for i, (m, (n, k, layout)) in enumerate(zip(mats, specs)):
            x = synth.activations(batch, k, seed=70 + i).to(DEV)
            y = torch.full((batch, n), float("nan"), dtype=torch.float32, device=DEV)
            c = choice[i]
            # CU splits: none, masked, and (a count past the device's CUs)
            # both kernels on every CU on two unmasked streams
            splits = [100000, 32, 128] if batch == 2 else [0, 100000, 32]
            cfg = {"variant": c["variant"], "decode_cus": splits[i]}
            jobs.append(uw.Job(m, [1, 2, c["pipeline"]][i], x, y, cfg))
            refs.append((bits(x), wnps[i], layout))
        ws = torch.empty(uw.uw_sequence_workspace_size(jobs), dtype=torch.uint8, device=DEV)
        uw.uw_run_sequence(jobs, 16, ws)
        torch.cuda.synchronize()
        for j, (x_np, w_np, layout) in zip(jobs, refs):
            check_gemm(oracle, j.y.cpu().numpy(), x_np, w_np, layout, what=f"tuned batch {batch}")
