"""uw_matmul_stage_static (scratch in a static device array, no allocation)
against uw_matmul_stage (caller workspace): bit-identical outputs on two
calls in a row, the second with a smaller input, for kernels that use the
scratch (split-K partial sums of the LDS-tiled and register-fed MFMA kernels,
the [K][N] GEMV's slices); within the fp64 bound of the oracle; and a call
that would need more scratch than the array holds is refused."""
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


def prep_for(uw, m, p):
    info = m.info()
    if p == 0:
        buf = torch.empty(info.numel, dtype=torch.int16, device=DEV)
        uw.uw_decode_full(m, buf)
    elif p == 1:
        buf = torch.empty(info.numel, dtype=torch.uint8, device=DEV)
        uw.uw_decode_exponent(m, buf)
    elif p == 2:
        buf = torch.empty(info.numel // 2, dtype=torch.uint8, device=DEV)
        uw.uw_transcode_palette(m, buf)
    else:
        buf = None
    return buf


def both(uw, m, p, prep, x, cfg):
    info = m.info()
    b = x.shape[0]
    y_ws = torch.full((b, info.n), float("nan"), dtype=torch.float32, device=DEV)
    y_st = torch.full((b, info.n), float("nan"), dtype=torch.float32, device=DEV)
    nbytes = uw.uw_workspace_size_cfg(m, p, b, cfg) if cfg else uw.uw_workspace_size(m, p, b)
    ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=DEV)
    uw.uw_matmul_stage(m, p, prep, x, y_ws, ws, cfg=cfg)
    uw.uw_matmul_stage_static(m, p, prep, x, y_st, cfg=cfg)
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_st.cpu().numpy()


# (stored shape, layout, pipeline, [(batch, cfg) for two calls in a row])
CASES = [
    ((2048, 4096), 0, 3, [(200, None), (48, None)]),                               # LDS tiles, split K
    ((2048, 4096), 0, 1, [(96, {"variant": 3, "split_k": 4}), (40, {"variant": 3, "split_k": 2})]),
    ((2048, 4096), 0, 3, [(32, None), (9, None)]),                                 # register-fed, packed x
    ((4096, 1536), 1, 2, [(3, {"variant": 1}), (1, None)]),                       # [K][N] GEMV slices
    ((4096, 1536), 1, 3, [(300, None), (70, None)]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_static_scratch_matches_workspace(uw, synth, oracle, case):
    (r, c), layout, p, calls = CASES[case]
    n, k = (r, c) if layout == 0 else (c, r)
    say(f"no-alloc stage: stored {r}x{c} layout {layout} pipeline {p} calls {calls}")
    w = synth.weights(r, c, 0.02, 0.001, 10, seed=600 + case).to(DEV)
    m = uw.uw_compress(w, n, k, layout)
    uw.uw_transcode_palette(m, None)
    prep = prep_for(uw, m, p)
    w_np = bits(w)
    for batch, cfg in calls:
        x = synth.activations(batch, k, seed=700 + batch).to(DEV)
        y_ws, y_st = both(uw, m, p, prep, x, cfg)
        assert np.all(np.isfinite(y_st))
        assert np.array_equal(y_ws, y_st), f"batch {batch}: static scratch differs from the workspace call"
        cols = np.arange(0, n, max(1, n // 256))
        y_ref, A = oracle.gemm_ref(bits(x), w_np, layout, cols=cols)
        ok, worst = oracle.gemm_check(y_st[:, cols], y_ref, A)
        assert ok, f"batch {batch}: worst err/bound {worst:.3g}"


def test_static_scratch_refuses_oversize(uw, synth):
    n, k, batch = 16384, 1024, 1024
    say("no-alloc stage: oversize request refused")
    w = synth.weights(n, k, 0.02, 0.0, 0, seed=650).to(DEV)
    m = uw.uw_compress(w, n, k, 0)
    uw.uw_transcode_palette(m, None)
    x = synth.activations(batch, k, seed=651).to(DEV)
    y = torch.zeros((batch, n), dtype=torch.float32, device=DEV)
    cfg = {"variant": 3, "split_k": 8}   # 8 slices x 1024 x 16384 floats = 512 MiB of partials
    assert uw.uw_workspace_size_cfg(m, 3, batch, cfg) > uw.STATIC_SCRATCH_BYTES
    with pytest.raises(uw.UwError) as ei:
        uw.uw_matmul_stage_static(m, 3, None, x, y, cfg=cfg)
    assert ei.value.status == -7
    torch.cuda.synchronize()
    assert float(y.abs().sum()) == 0.0      # nothing was enqueued
    # the same call without a split needs no scratch at all
    uw.uw_matmul_stage_static(m, 3, None, x, y, cfg={"variant": 3, "split_k": 1})
    torch.cuda.synchronize()
    assert np.all(np.isfinite(y.cpu().numpy()))
