"""The no-allocation sampler entry point (dg_sampler_step_noalloc), for
callers that cannot allocate device memory: through the C ABI, two calls in
a row (the second on a smaller input, so the static scratch holds the first
call's contents) give bit-for-bit what dg_sampler_step gives on a workspace
of its own, and sizes beyond the static scratch are refused."""
import ctypes as C

import pytest
import torch

from synth import workloads as wl

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def _step(B, noalloc, logits, n, V, t, canvas, stats, scfg, bias=None):
    if noalloc:
        B.sampler_step_noalloc(scfg, logits, V - 1, canvas, t, SEED, stats)
    else:
        ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device="cuda")
        B.sampler_step(scfg, logits, V - 1, canvas, t, SEED, stats, ws)


@pytest.mark.parametrize("draw_mode", [0, 1])
def test_noalloc_matches_the_workspace_entry_point(B, draw_mode):
    scfg = B.sampler_default()
    scfg.draw_mode = draw_mode
    # first call: the full-vocabulary workload's shape; second: a smaller one
    for (n, V, t) in (((256, 262144, 3)), (64, 4096, 0)):
        logits = wl.sampler_logits(t, shape=(n, V), device="cuda")
        bt, bv = wl.canvas_boost(wl.TINY.replace(canvas=n, vocab=V), 3)
        outs = []
        for noalloc in (False, True):
            canvas = B.Canvas(n, V - 1, 2, "cuda", bt.cuda(), bv.cuda())
            stats = B.StepStats(n, "cuda")
            for step in range(t, t + 2):
                _step(B, noalloc, logits, n, V, step, canvas, stats, scfg)
            torch.cuda.synchronize()
            outs.append([canvas.tokens.clone(), canvas.committed.clone(), canvas.state.clone(),
                         canvas.prev_argmax.clone(), stats.entropy.clone(), stats.lse.clone(),
                         stats.argmax.clone(), stats.selected.clone(), stats.mean_entropy.clone()])
        for a, b in zip(*outs):
            assert torch.equal(a, b), (n, V)
        assert int(outs[1][2][B.ST_COMMITTED]) >= 2


def test_noalloc_refuses_sizes_beyond_the_static_scratch(B):
    cap = B.sampler_static_scratch_bytes()
    assert cap == 2 << 20
    n, V = 1024, 1 << 20
    assert B.sampler_workspace_bytes(n, V) > cap
    logits = torch.empty((1, 8), dtype=torch.bfloat16, device="cuda")   # never read: refused first
    canvas = B.Canvas(n, V - 1, 0, "cuda")
    stats = B.StepStats(n, "cuda")
    c, s = canvas.struct(), stats.struct()
    code = B.lib.dg_sampler_step_noalloc(C.byref(B.sampler_default()), logits.data_ptr(), B.DG_BF16, n, V, V,
                                         V - 1, C.byref(c), 0, SEED, C.byref(s), None)
    assert code == -3 and b"static" in B.lib.dg_last_error()
