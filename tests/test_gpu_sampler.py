"""Parity of the HIP EB sampler (dg_sampler_step) with the oracle, through the
C ABI, on seeded synthetic logits: small ragged shapes, the full 256 x 262144
bf16 workload, float32 logits with a per-row boost, scripted stop sequences,
edge sizes and determinism."""
import numpy as np
import pytest
import torch

from oracle import sampler as S
from synth import workloads as wl

from parity import check_sampler_step

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def _biased(L, bias):
    L = np.asarray(L, np.float64).copy()
    if bias is not None:
        tok, mag = bias
        L[np.arange(L.shape[0]), tok] += mag.astype(np.float64)
    return L


def run_and_compare(B, logits_fn, n, V, steps, bias=None, seed=SEED, canvas_idx=0,
                    bound_mode=0, step_ids=None, commit_mode=0, draw_mode=0):
    """Run the GPU sampler step by step and check every step against the oracle.

    Returns (gpu tokens, number of steps run, list of per-step records)."""
    dev = torch.device("cuda")
    mask = V - 1
    btok = bval = None
    if bias is not None:
        btok = torch.tensor(bias[0], dtype=torch.int32, device=dev)
        bval = torch.tensor(bias[1], dtype=torch.float32, device=dev)
    canvas = B.Canvas(n, mask, canvas_idx, dev, btok, bval)
    stats = B.StepStats(n, dev)
    ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    cfg = B.sampler_default()
    cfg.bound_mode = bound_mode
    cfg.commit_mode = commit_mode
    cfg.draw_mode = draw_mode
    ocfg = S.SamplerConfig(mask_id=mask, bound_mode=["sum", "sum_minus_max"][bound_mode],
                           commit_mode=["keep", "reselect_all"][commit_mode],
                           draw_mode=["inverse_cdf", "gumbel_max"][draw_mode])
    st = S.CanvasState.fresh(n, mask, canvas_idx)
    recs = []
    ids = step_ids if step_ids is not None else range(steps)
    for t in ids:
        Ld = logits_fn(t)
        B.sampler_step(cfg, Ld, mask, canvas, t, seed, stats, ws)
        torch.cuda.synchronize()
        L = _biased(Ld.float().cpu().numpy(), bias)
        if step_ids is not None:
            st.steps = t
        recs.append(check_sampler_step(B, st, ocfg, L, t, seed, canvas_idx, stats, canvas))
        if st.done:
            break
    assert np.array_equal(canvas.tokens.cpu().numpy(), st.tokens)
    return canvas.tokens.cpu().numpy(), len(recs), recs


def test_small_bf16_trajectory(B):
    n, V = 64, 4096
    toks, steps, recs = run_and_compare(
        B, lambda t: wl.sampler_logits(t, shape=(n, V), device="cuda"), n, V, 48)
    assert sum(r.selected.sum() for r in recs) >= 1
    assert not np.any(toks == V - 1)


@pytest.mark.parametrize("V", [5000, 2056, 8])
def test_ragged_vocab_f32_with_boost(B, V):
    n = 32
    g = torch.Generator().manual_seed(V)
    tok = torch.randint(0, V - 1, (n,), generator=g).numpy()
    mag = (torch.rand(n, generator=g) * 12).numpy().astype(np.float32)

    def logits(t):
        gg = torch.Generator().manual_seed(1000 * V + t)
        return torch.randn(n, V, generator=gg).to("cuda")
    run_and_compare(B, logits, n, V, 48, bias=(tok, mag), canvas_idx=3)


@pytest.mark.parametrize("draw_mode", [0, 1])
def test_bias_tokens_on_chunk_edges_bf16(B, draw_mode):
    """bf16 logits over 40008 columns (three chunks of 16384 columns, the last
    ragged) with the bias token at chunk and vector edges, on MASK, boosted
    past the row's maximum, and banned with a -inf bias: the statistics pass
    takes MASK and the bias token out of its per-chunk reduction and adds the
    biased value once, which must give the oracle's statistics and draws."""
    n, V = 32, 40008
    edges = [0, 7, 8, 2047, 2048, 16383, 16384, 16385, 32767, 32768, 40000, V - 2, V - 1]
    g = torch.Generator().manual_seed(77)
    tok = torch.randint(0, V - 1, (n,), generator=g).numpy()
    tok[:len(edges)] = edges
    mag = (torch.rand(n, generator=g) * 12).numpy().astype(np.float32)
    mag[1::3] = 40.0    # the bias token becomes the argmax
    mag[5] = -np.inf    # token 16383 banned in row 5
    mag[20] = -5.0

    def logits(t):
        return wl.sampler_logits(t + 11, shape=(n, V), device="cuda")
    run_and_compare(B, logits, n, V, 48, bias=(tok, mag), canvas_idx=2, draw_mode=draw_mode)


def test_peak_far_above_the_first_chunk(B):
    """A row's maximum sits in its last chunk, 20 to 80 logits above the
    rest: the statistics pass sums each chunk against a running reference
    taken from the first chunk, and must sum such a chunk again against its
    own maximum instead of overflowing 2^d."""
    n, V = 16, 65536
    g = torch.Generator().manual_seed(5)
    cols = torch.randint(3 * 16384, V - 1, (n,), generator=g)
    peaks = torch.linspace(20.0, 80.0, n)

    def logits(t):
        L = wl.sampler_logits(t + 21, shape=(n, V), max_peak=1.0, device="cuda")
        L[torch.arange(n), cols.cuda()] = peaks.cuda().to(torch.bfloat16)
        return L
    run_and_compare(B, logits, n, V, None, step_ids=[0, 23, 47])


def test_sum_minus_max_mode(B):
    n, V = 48, 1024
    run_and_compare(B, lambda t: wl.sampler_logits(t + 7, shape=(n, V), max_peak=30.0, device="cuda"),
                    n, V, 48, bound_mode=1)


@pytest.mark.parametrize("bound_mode", [0, 1])
def test_reselect_all_commit_mode(B, bound_mode):
    n, V = 48, 1024
    toks, steps, recs = run_and_compare(
        B, lambda t: wl.sampler_logits(t + 7, shape=(n, V), max_peak=30.0, device="cuda"),
        n, V, 48, bound_mode=bound_mode, commit_mode=B.DG_COMMIT_RESELECT_ALL)
    # earlier commits were taken back on the device, not just never made
    taken_back = sum(int((recs[k].selected & ~recs[k + 1].selected).sum())
                     for k in range(len(recs) - 2))
    assert taken_back > 0
    assert not np.any(toks == V - 1)


def test_reselect_all_on_the_full_vocabulary(B):
    n, V = wl.SAMPLER_ONLY_SHAPE
    buf = torch.empty((n, V), dtype=torch.bfloat16, device="cuda")

    def logits(t):
        return wl.sampler_logits(t, device="cuda", out=buf)
    run_and_compare(B, logits, n, V, 4, commit_mode=B.DG_COMMIT_RESELECT_ALL)


def test_gumbel_max_draws_small_bf16(B):
    n, V = 64, 4096
    toks, steps, recs = run_and_compare(
        B, lambda t: wl.sampler_logits(t + 3, shape=(n, V), device="cuda"), n, V, 48,
        draw_mode=B.DG_DRAW_GUMBEL_MAX)
    assert sum(r.selected.sum() for r in recs) >= 1 and not np.any(toks == V - 1)


@pytest.mark.parametrize("V", [5000, 8])
def test_gumbel_max_draws_f32_with_boost(B, V):
    n = 32
    g = torch.Generator().manual_seed(V + 1)
    tok = torch.randint(0, V - 1, (n,), generator=g).numpy()
    mag = (torch.rand(n, generator=g) * 12).numpy().astype(np.float32)

    def logits(t):
        gg = torch.Generator().manual_seed(2000 * V + t)
        return torch.randn(n, V, generator=gg).to("cuda")
    run_and_compare(B, logits, n, V, 48, bias=(tok, mag), canvas_idx=5, draw_mode=B.DG_DRAW_GUMBEL_MAX)


def test_gumbel_max_draws_full_vocabulary(B):
    n, V = wl.SAMPLER_ONLY_SHAPE
    buf = torch.empty((n, V), dtype=torch.bfloat16, device="cuda")

    def logits(t):
        return wl.sampler_logits(t, device="cuda", out=buf)
    run_and_compare(B, logits, n, V, None, step_ids=[0, 1, 47], draw_mode=B.DG_DRAW_GUMBEL_MAX)


def test_full_vocab_256_rows_selected_steps(B):
    n, V = wl.SAMPLER_ONLY_SHAPE
    buf = torch.empty((n, V), dtype=torch.bfloat16, device="cuda")

    def logits(t):
        return wl.sampler_logits(t, device="cuda", out=buf)
    run_and_compare(B, logits, n, V, None, step_ids=[0, 1, 2, 47])


def test_stop_rule_fires_on_device(B):
    """Confident, stable rows: the canvas stops at t = 1 and is filled by argmax."""
    n, V = 256, 64
    import math
    import scipy.optimize
    h = 0.0049

    def logits(t):
        tau = S.temperature(t, S.SamplerConfig())
        p = scipy.optimize.brentq(lambda q: -(q * math.log(q) + (1 - q) * math.log(1 - q)) - h,
                                  0.5, 1 - 1e-15)
        L = torch.full((n, V), -1e4, dtype=torch.float32)
        ids = torch.arange(n) % 50
        L[torch.arange(n), ids] = 0.0
        L[torch.arange(n), ids + 1] = tau * (math.log(1 - p) - math.log(p))
        return L.cuda()
    toks, steps, recs = run_and_compare(B, logits, n, V, 48)
    assert steps == 2 and recs[-1].stop
    assert np.array_equal(toks[~(recs[0].selected | recs[1].selected)],
                          (np.arange(n) % 50)[~(recs[0].selected | recs[1].selected)])


@pytest.mark.parametrize("n", [1, 1024])
def test_edge_row_counts(B, n):
    V = 256
    run_and_compare(B, lambda t: wl.sampler_logits(t, shape=(n, V), device="cuda"), n, V, 48)


def test_deterministic_and_done_is_sticky(B):
    n, V = 128, 8192
    dev = torch.device("cuda")
    outs = []
    for rep in range(2):
        canvas = B.Canvas(n, V - 1, 0, dev)
        stats = B.StepStats(n, dev)
        ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
        ents = []
        for t in range(48):
            B.sampler_step(B.sampler_default(), wl.sampler_logits(t, shape=(n, V), device="cuda"),
                           V - 1, canvas, t, SEED, stats, ws)
            ents.append(stats.entropy.clone())
            if canvas.state[0].item():
                break
        outs.append((canvas.tokens.clone(), torch.stack(ents), canvas.state.clone()))
        # further calls on a finished canvas change nothing
        before = canvas.tokens.clone()
        B.sampler_step(B.sampler_default(), wl.sampler_logits(0, shape=(n, V), device="cuda"),
                       V - 1, canvas, -1, SEED, stats, ws)
        torch.cuda.synchronize()
        assert torch.equal(before, canvas.tokens)
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2])


def test_nan_logits_still_give_tokens_inside_the_vocabulary(B):
    # rows whose logits are NaN (all or some) have no meaningful distribution;
    # whatever is committed must still be a valid id, since the next step
    # embeds it
    n, V = 64, 4096
    dev = torch.device("cuda")
    canvas = B.Canvas(n, V - 1, 0, dev)
    stats = B.StepStats(n, dev)
    ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    for t in range(48):
        L = wl.sampler_logits(t, shape=(n, V), device="cuda")
        L[3] = float("nan")
        L[10, 100:200] = float("nan")
        B.sampler_step(B.sampler_default(), L, V - 1, canvas, t, SEED, stats, ws)
        torch.cuda.synchronize()
        tok = canvas.tokens
        assert int(tok.min()) >= 0 and int(tok.max()) < V
        if canvas.state[0].item():
            break
    assert bool(canvas.committed.all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["nan_row", "inf_logit"])
def test_row_without_finite_mass_commits_its_argmax(B, dtype, kind):
    """Row 0 has no finite positive probability mass: all NaN (argmax id 0),
    or one +inf logit (exp(z - M) is NaN there, 0 elsewhere; the argmax is
    the +inf column). Its entropy clamps to 0, so it is selected first, and
    the draw commits the argmax without scanning any chunk of the row (a
    scan would start before row 0, outside the logits)."""
    n, V = 64, 8192
    dev = torch.device("cuda")
    L = wl.sampler_logits(0, shape=(n, V), device="cuda").to(dtype)
    want = 0 if kind == "nan_row" else 1234
    if kind == "nan_row":
        L[0] = float("nan")
    else:
        L[0, 1234] = float("inf")
    canvas = B.Canvas(n, V - 1, 0, dev)
    stats = B.StepStats(n, dev)
    ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    B.sampler_step(B.sampler_default(), L, V - 1, canvas, 0, SEED, stats, ws)
    torch.cuda.synchronize()
    assert int(stats.selected[0]) == 1
    assert int(stats.argmax[0]) == want
    assert int(canvas.committed[0]) == 1 and int(canvas.tokens[0]) == want
    tok = canvas.tokens.cpu().numpy()
    assert tok.min() >= 0 and tok.max() < V


def test_full_vocabulary_f32_logits_with_bias_on_chunk_edges(B):
    """f32 logits over the full 262144-column vocabulary (two splits of eight
    16384-column chunks each, the f32 register layout of the statistics
    pass), bias tokens on chunk and split edges, a peak 60 logits above the
    rest in the last chunk of some rows."""
    n, V = 32, 262144
    edges = [0, 16383, 16384, 131071, 131072, 131073, 147456, V - 2, V - 1]
    g = torch.Generator().manual_seed(31)
    tok = torch.randint(0, V - 1, (n,), generator=g).numpy()
    tok[:len(edges)] = edges
    mag = (torch.rand(n, generator=g) * 12).numpy().astype(np.float32)
    mag[2::5] = 40.0
    peak_rows = torch.arange(16, 24)

    def logits(t):
        gg = torch.Generator().manual_seed(7000 + t)
        L = torch.randn(n, V, generator=gg)
        L[peak_rows, V - 3] = 60.0
        return L.to("cuda")
    run_and_compare(B, logits, n, V, None, step_ids=[0, 23, 47], bias=(tok, mag), canvas_idx=4)
