"""Parity of the HIP model path with the oracle, through the C ABI: the embed,
one decoder layer (windowed and global, f32 and bf16), the LM head with its
fused statistics, the encoder prefill/append, and full canvas trajectories
on the tiny f32 workload (per step, decomposed, and as whole trajectories)."""
import numpy as np
import scipy.special
import pytest
import torch

from oracle import generate as G
from oracle import model as M
from oracle import sampler as S
from synth import workloads as wl

from model_fixtures import (SMALL_BF16, check_logit_rows, device_model, device_v, fill_synthetic_kv,
                            oracle_kv_from_device, oracle_weights, rel_l2, rel_l2_rows, route_margins,
                            routing_near_tie_ok)
from parity import ENT_TOL_NORTH, check_sampler_step, check_statistics

pytestmark = pytest.mark.gpu

SEED = 0x5EED
# e4m3 projection and expert weights with bf16 per-row scales: both sides
# decode the same codes exactly, so the error budget is the bf16 one
SMALL_FP8 = SMALL_BF16.replace(name="small_fp8", weight_dtype="fp8")
CFGS = {"tiny_f32": wl.TINY, "small_bf16": SMALL_BF16, "small_fp8": SMALL_FP8}
# 320 canvas rows: expert groups of more than 64 rows take the LDS-staged
# grouped GEMM, the shared expert spans two 256-row blocks (the second with
# one live wave), and smaller groups stay on the streaming GEMM
WIDE_BF16 = SMALL_BF16.replace(name="wide_bf16", canvas=320)
LAYER_CFGS = dict(CFGS, wide_bf16=WIDE_BF16)
# per-row relative L2 bounds against the float64 oracle: f32 path vs bf16 path
LAYER_TOL = {"tiny_f32": 1e-4, "small_bf16": 1.5e-2, "small_fp8": 1.5e-2, "wide_bf16": 1.5e-2}
DELTA_TOL = {"tiny_f32": 1e-4, "small_bf16": 3e-2, "small_fp8": 3e-2, "wide_bf16": 3e-2}
LOGIT_TOL = {"tiny_f32": 1e-5, "small_bf16": 1e-2, "small_fp8": 1e-2}
KV_TOL = {"tiny_f32": 1e-4, "small_bf16": 3e-2, "small_fp8": 3e-2}


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def _canvas_tokens(cfg, n_committed):
    toks, _ = wl.committed_canvas(cfg, n_committed)
    return toks.cuda()


def test_embed_is_exact_row_copy(B):
    cfg = SMALL_BF16
    model = device_model(B, cfg)
    tok = _canvas_tokens(cfg, 20)
    X = torch.empty(cfg.canvas, cfg.d_model, dtype=torch.float32, device="cuda")
    B.embed(model, tok, X)
    torch.cuda.synchronize()
    assert torch.equal(X, model.embed[tok.long()].float())


def test_embed_ids_outside_the_vocabulary_give_zero_rows(B):
    cfg = SMALL_BF16
    model = device_model(B, cfg)
    tok = _canvas_tokens(cfg, 20)
    bad = torch.tensor([-1, cfg.vocab, 2**31 - 1, -(2**31)], dtype=torch.int32, device="cuda")
    tok[5:9] = bad
    X = torch.full((cfg.canvas, cfg.d_model), 7.0, dtype=torch.float32, device="cuda")
    B.embed(model, tok, X)
    torch.cuda.synchronize()
    good = torch.ones(cfg.canvas, dtype=torch.bool, device="cuda")
    good[5:9] = False
    assert torch.equal(X[good], model.embed[tok[good].long()].float())
    assert torch.count_nonzero(X[~good]) == 0


def test_router_ids_stay_valid_and_distinct_on_nan_activations(B):
    # a NaN activation must not turn into an expert id outside [0, E) (the
    # permutation and the expert GEMMs index with them)
    cfg = SMALL_BF16
    model = device_model(B, cfg)
    n = cfg.canvas
    kv = B.KVCache(model, 300 + n)
    fill_synthetic_kv(kv, cfg, 300)
    X = torch.randn(n, cfg.d_model, dtype=torch.float32, device="cuda")
    X[3] = float("nan")
    X[17, :5] = float("nan")
    ids = torch.zeros(n, cfg.top_k, dtype=torch.int32, device="cuda")
    gates = torch.zeros(n, cfg.top_k, dtype=torch.float32, device="cuda")
    B.decoder_layer(model, 0, X, kv, model.workspace(n), ids, gates)
    torch.cuda.synchronize()
    g = ids.cpu().numpy()
    assert g.min() >= 0 and g.max() < cfg.n_experts
    assert all(len(set(r.tolist())) == cfg.top_k for r in g)


def test_stale_values_beyond_the_visible_rows_never_reach_the_output(B):
    """Cache rows at or past len hold NaN (a reused cache), and the canvas
    K/V rows past a 40-row canvas in the workspace hold NaN left by an
    earlier 64-row call: the decoder layers (windowed and global) and the
    encoder give bit-for-bit the results of zero-filled buffers, since
    attention masks those keys' scores and reads their values as zero."""
    cfg = SMALL_BF16
    model = device_model(B, cfg)
    P, n = 300, 40                      # 40 canvas rows: a partial 64-row key block
    tok = _canvas_tokens(cfg, 20)[:n].contiguous()
    outs = []
    for poison in (False, True):
        kv = B.KVCache(model, P + 200)
        fill_synthetic_kv(kv, cfg, P)
        ws = torch.zeros_like(model.workspace(cfg.canvas))
        if poison:
            # an earlier call over 64 rows whose last 24 are NaN leaves NaN
            # canvas K/V rows 40..63 in the workspace
            X64 = torch.randn(64, cfg.d_model, dtype=torch.float32, device="cuda")
            X64[n:] = float("nan")
            for l in range(cfg.n_layers):
                B.decoder_layer(model, l, X64, kv, ws)
            for l in range(cfg.n_layers):
                kv.k[l][:, P:] = float("nan")
                kv.v[l][:, :, P:] = float("nan")
        X = torch.empty(n, cfg.d_model, dtype=torch.float32, device="cuda")
        B.embed(model, tok, X)
        for l in range(cfg.n_layers):
            B.decoder_layer(model, l, X, kv, ws)
        B.prefill_append(model, kv, tok, ws)
        torch.cuda.synchronize()
        outs.append((X.clone(), [kv.k[l][:, :P + n].clone() for l in range(cfg.n_layers)],
                     [kv.v[l][:, :, :P + n].clone() for l in range(cfg.n_layers)]))
    assert torch.isfinite(outs[1][0]).all()
    assert torch.equal(outs[0][0], outs[1][0])
    for l in range(cfg.n_layers):
        assert torch.equal(outs[0][1][l], outs[1][1][l]) and torch.equal(outs[0][2][l], outs[1][2][l]), l


@pytest.mark.parametrize("name", list(LAYER_CFGS))
@pytest.mark.parametrize("layer", [0, 1])
def test_decoder_layer(B, name, layer):
    cfg = LAYER_CFGS[name]
    model = device_model(B, cfg)
    P = 300 if name != "tiny_f32" else wl.TINY_PREFIX
    n = cfg.canvas
    kv = B.KVCache(model, P + n)
    fill_synthetic_kv(kv, cfg, P)
    tok = _canvas_tokens(cfg, n // 2)
    X = torch.empty(n, cfg.d_model, dtype=torch.float32, device="cuda")
    B.embed(model, tok, X)
    X0 = X.cpu().numpy().astype(np.float64)
    ids = torch.zeros(n, cfg.top_k, dtype=torch.int32, device="cuda")
    gates = torch.zeros(n, cfg.top_k, dtype=torch.float32, device="cuda")
    ws = model.workspace(n)
    B.decoder_layer(model, layer, X, kv, ws, ids, gates)
    torch.cuda.synchronize()
    Xg = X.cpu().numpy()
    W = oracle_weights(model)
    okv = oracle_kv_from_device(kv, cfg, P)
    tr = {}
    M.decoder_layer(X0, W.layer(layer), okv.K[layer], okv.V[layer], layer, cfg, trace=tr)
    ids_g = ids.cpu().numpy()
    bad = routing_near_tie_ok(tr["router"], ids_g, tr["ids"], 5e-3 if name != "tiny_f32" else 1e-5)
    assert not bad, bad[:5]
    Xo = M.decoder_layer(X0, W.layer(layer), okv.K[layer], okv.V[layer], layer, cfg, ids_override=ids_g)
    assert rel_l2_rows(Xg, Xo).max() < LAYER_TOL[name], rel_l2_rows(Xg, Xo).max()
    assert rel_l2(Xg - X0, Xo - X0) < DELTA_TOL[name], rel_l2(Xg - X0, Xo - X0)
    same = np.all(np.sort(ids_g, 1) == np.sort(tr["ids"], 1), axis=1)
    g_o = np.take_along_axis(tr["gates"], np.argsort(tr["ids"], 1), 1)
    g_g = np.take_along_axis(gates.cpu().numpy(), np.argsort(ids_g, 1), 1)
    assert np.abs(g_o[same] - g_g[same]).max() < (2e-2 if name != "tiny_f32" else 1e-5)


@pytest.mark.parametrize("name", ["small_bf16", "full_width"])
def test_e4m3_lm_head_logits_and_statistics(B, name):
    """The LM head reading an e4m3 copy of the tied matrix (bf16 scale per
    vocabulary row) and the bf16 head, on random activations with per-row
    logit boosts U(0, 12), at the first, middle and last temperatures of the
    schedule: logits within the bf16 / e4m3 bars of the oracle on the same
    (dequantised) matrix, the statistics against the logits each stored, and
    every row's entropy within the stated 1e-2 nats of the oracle's own
    float64 logits."""
    cfg = SMALL_BF16 if name == "small_bf16" else wl.FULL_LAYER
    embed = wl.embedding(cfg, device="cuda")
    codes, scale = wl.lm_head_e4m3(cfg, device="cuda")
    fnorm = wl.final_norm(cfg, device="cuda")
    layers = [wl.layer_weights(cfg, l, device="cuda") for l in range(cfg.n_layers)]
    m8 = B.Model(cfg, embed, fnorm, layers, lm_head_e4m3=codes, lm_head_scale=scale)
    mb = B.Model(cfg, embed, fnorm, layers)
    n = cfg.canvas
    g = torch.Generator().manual_seed(6)
    X = torch.randn(n, cfg.d_model, generator=g).cuda()
    bt, bv = wl.canvas_boost(cfg, 1)
    bt, bv = bt.cuda(), bv.cuda()
    ws = m8.workspace(n)
    scfg = B.sampler_default()
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    Xn = X.cpu().numpy().astype(np.float64)
    W8 = M.Weights(cfg, embed.cpu(), fnorm.cpu(), lambda l: {}, lm_head=(codes.cpu(), scale.cpu()))
    btn, bvn = bt.cpu().numpy(), bv.cpu().numpy().astype(np.float64)
    for key, model in (("e4m3", m8), ("bf16", mb)):
        Lo = M.lm_logits(Xn, W8.final_norm, W8.LM if key == "e4m3" else W8.E, cfg.norm_eps)
        Lo_b = Lo.copy()
        Lo_b[np.arange(n), btn] += bvn
        for t in (0, 23, 47):
            tau = S.temperature(t, ocfg)
            stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=model.act_dtype)
            B.lm_head(model, X, scfg, t, stats, ws, bt, bv)
            torch.cuda.synchronize()
            Lg = stats.logits.float().cpu().numpy().astype(np.float64)
            assert rel_l2_rows(Lg, Lo).max() < (5e-2 if key == "e4m3" else 1e-2), (key, rel_l2_rows(Lg, Lo).max())
            Lb = Lg.copy()
            Lb[np.arange(n), btn] += bvn
            check_statistics(stats, ocfg, Lb, t, rounded_from_f32=True)
            Ho, ao, _, _ = S.row_stats(Lo_b, tau, cfg.mask_id)
            dH = np.abs(stats.entropy.cpu().numpy() - Ho)
            assert dH.max() < ENT_TOL_NORTH, (key, t, float(dH.max()))
            del Lg, Lb
        del Lo, Lo_b


@pytest.mark.parametrize("name", list(CFGS))
def test_lm_head_logits_and_statistics(B, name):
    cfg = CFGS[name]
    model = device_model(B, cfg)
    n = cfg.canvas
    g = torch.Generator().manual_seed(5)
    X = torch.randn(n, cfg.d_model, generator=g).cuda()
    bt, bv = wl.canvas_boost(cfg, 0)
    bt, bv = bt.cuda(), bv.cuda()
    ws = model.workspace(n)
    scfg = B.sampler_default()
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    for t in (0, 23, 47):
        stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=model.act_dtype)
        B.lm_head(model, X, scfg, t, stats, ws, bt, bv)
        torch.cuda.synchronize()
        Lg = stats.logits.float().cpu().numpy()
        Lo = M.lm_logits(X.cpu().numpy().astype(np.float64), model.final_norm.cpu().numpy().astype(np.float64),
                         model.embed.float().cpu().numpy().astype(np.float64), cfg.norm_eps)
        assert rel_l2_rows(Lg, Lo).max() < LOGIT_TOL[name], rel_l2_rows(Lg, Lo).max()
        Lb = Lg.astype(np.float64)
        Lb[np.arange(n), bt.cpu().numpy()] += bv.cpu().numpy().astype(np.float64)
        # the reduction against the logits it stored (their f32 originals:
        # within the first-order effect of the bf16 rounding)
        check_statistics(stats, ocfg, Lb, t, rounded_from_f32=name != "tiny_f32")
        # and against the oracle's own logits of the same activations
        Lob = Lo.copy()
        Lob[np.arange(n), bt.cpu().numpy()] += bv.cpu().numpy().astype(np.float64)
        Ho, _, _, _ = S.row_stats(Lob, S.temperature(t, ocfg), cfg.mask_id)
        assert np.abs(stats.entropy.cpu().numpy() - Ho).max() < ENT_TOL_NORTH


def test_lm_head_outside_the_tiled_kernel(B):
    """A bf16 model whose width is not a multiple of 64 (d_model 96): the LM
    head takes the generic LDS GEMM with the same statistics epilogue."""
    cfg = SMALL_BF16.replace(name="odd_bf16", n_layers=1, d_model=96, n_q_heads=2, n_kv_heads=1, head_dim=64,
                             vocab=1000)
    model = device_model(B, cfg)
    n = cfg.canvas
    g = torch.Generator().manual_seed(7)
    X = torch.randn(n, cfg.d_model, generator=g).cuda()
    ws = model.workspace(n)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    for t in (0, 47):
        stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=torch.bfloat16)
        B.lm_head(model, X, B.sampler_default(), t, stats, ws)
        torch.cuda.synchronize()
        Lg = stats.logits.float().cpu().numpy().astype(np.float64)
        Lo = M.lm_logits(X.cpu().numpy().astype(np.float64), model.final_norm.cpu().numpy().astype(np.float64),
                         model.embed.float().cpu().numpy().astype(np.float64), cfg.norm_eps)
        assert rel_l2_rows(Lg, Lo).max() < 1e-2, rel_l2_rows(Lg, Lo).max()
        check_statistics(stats, ocfg, Lg, t, rounded_from_f32=True)
        Ho, _, _, _ = S.row_stats(Lo, S.temperature(t, ocfg), cfg.mask_id)
        assert np.abs(stats.entropy.cpu().numpy() - Ho).max() < ENT_TOL_NORTH


@pytest.mark.parametrize("name", list(CFGS))
def test_prefill_append_matches_oracle_encoder(B, name):
    cfg = CFGS[name]
    model = device_model(B, cfg)
    n_tok = 200
    toks = wl.prefix_tokens(cfg, n_tok).cuda()
    kv = B.KVCache(model, 256)
    ws = model.workspace(64)                     # chunks of 64 rows
    B.prefill_append(model, kv, toks[:150], ws)
    B.prefill_append(model, kv, toks[150:], ws)
    torch.cuda.synchronize()
    assert kv.length == n_tok
    W = oracle_weights(model)
    okv = M.KVCache.empty(cfg)
    M.encoder_append(W, okv, toks.cpu().numpy())
    for l in range(cfg.n_layers):
        kg = kv.k[l][:, :n_tok].float().cpu().numpy()
        vg = device_v(kv, l, n_tok).numpy()
        assert rel_l2(kg, okv.K[l]) < KV_TOL[name], (l, rel_l2(kg, okv.K[l]))
        assert rel_l2(vg, okv.V[l]) < KV_TOL[name], (l, rel_l2(vg, okv.V[l]))
    # one pass with a large workspace gives the same cache
    kv2 = B.KVCache(model, 256)
    B.prefill_append(model, kv2, toks, model.workspace(256))
    torch.cuda.synchronize()
    for l in range(cfg.n_layers):
        d = rel_l2(kv2.k[l][:, :n_tok].float().cpu().numpy(), kv.k[l][:, :n_tok].float().cpu().numpy())
        assert d < (1e-6 if name == "tiny_f32" else 1e-2), (l, d)


def test_prefill_capacity_is_checked(B):
    cfg = wl.TINY
    model = device_model(B, cfg)
    kv = B.KVCache(model, 64)
    with pytest.raises(B.DgError) as e:
        B.prefill_append(model, kv, wl.prefix_tokens(cfg, 65).cuda(), model.workspace(32))
    assert e.value.code == -3 and kv.length == 0


def _tiny_setup(B):
    cfg = wl.TINY
    model = device_model(B, cfg)
    prompt = wl.prefix_tokens(cfg, wl.TINY_PREFIX)
    kv = B.KVCache(model, wl.TINY_PREFIX + 2 * cfg.canvas)
    ws = model.workspace(cfg.canvas * 4)
    B.prefill_append(model, kv, prompt.cuda(), ws)
    W = oracle_weights(model)
    okv = M.KVCache.empty(cfg)
    M.encoder_append(W, okv, prompt.numpy())
    return cfg, model, kv, ws, W, okv


@pytest.mark.parametrize("commit_mode", [0, 1])
def test_tiny_canvas_steps_decomposed(B, commit_mode):
    """Every step of a tiny f32 canvas: logits against the oracle's decoder on
    the same input state, then the sampler's decisions on the same logits
    (commits final, or every position re-selected at every step)."""
    cfg, model, kv, ws, W, okv = _tiny_setup(B)
    n = cfg.canvas
    bt, bv = wl.canvas_boost(cfg, 0)
    canvas = B.Canvas(n, cfg.mask_id, 0, "cuda", bt.cuda(), bv.cuda())
    stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=torch.float32)
    scfg = B.sampler_default()
    scfg.commit_mode = commit_mode
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id, commit_mode=["keep", "reselect_all"][commit_mode])
    st = S.CanvasState.fresh(n, cfg.mask_id, 0)
    for t in range(48):
        before = canvas.tokens.cpu().numpy()
        assert np.array_equal(before, st.tokens)
        B.canvas_step(model, canvas, kv, t, SEED, scfg, stats, ws)
        torch.cuda.synchronize()
        Lo = M.canvas_logits(W, before, okv, (bt.numpy(), bv.numpy()))
        Lg = stats.logits.cpu().numpy().astype(np.float64)
        Lg[np.arange(n), bt.numpy()] += bv.numpy().astype(np.float64)
        assert rel_l2_rows(Lg, Lo).max() < 1e-4, (t, rel_l2_rows(Lg, Lo).max())
        check_sampler_step(B, st, ocfg, Lg, t, SEED, 0, stats, canvas)
        if st.done:
            break
    assert st.done and not np.any(canvas.tokens.cpu().numpy() == cfg.mask_id)
    # the finished canvas goes through the encoder and onto the cache
    B.prefill_append(model, kv, canvas.tokens, ws)
    M.encoder_append(W, okv, st.tokens)
    torch.cuda.synchronize()
    assert kv.length == okv.length == wl.TINY_PREFIX + n
    for l in range(cfg.n_layers):
        assert rel_l2(kv.k[l][:, :kv.length].cpu().numpy(), okv.K[l]) < 1e-4


def test_small_bf16_canvas_steps_with_gumbel_max_draws(B):
    """Canvas steps whose draws are the Gumbel-max candidates kept by the LM
    head epilogue: the sampler's decisions on the logits the step wrote
    against the oracle's Gumbel-max draws (near ties of the perturbed values
    excused), and the logits themselves against the oracle decoder."""
    cfg = SMALL_BF16
    model = device_model(B, cfg)
    P, n = 160, cfg.canvas
    prompt = wl.prefix_tokens(cfg, P)
    kv = B.KVCache(model, P + n)
    ws = model.workspace(n)
    B.prefill_append(model, kv, prompt.cuda(), ws)
    W = oracle_weights(model)
    okv = M.KVCache.empty(cfg)
    M.encoder_append(W, okv, prompt.numpy())
    bt, bv = wl.canvas_boost(cfg, 0)
    canvas = B.Canvas(n, cfg.mask_id, 4, "cuda", bt.cuda(), bv.cuda())
    stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=torch.bfloat16)
    scfg = B.sampler_default()
    scfg.draw_mode = B.DG_DRAW_GUMBEL_MAX
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id, draw_mode="gumbel_max")
    st = S.CanvasState.fresh(n, cfg.mask_id, 4)
    drawn = 0
    for t in range(10):
        before = canvas.tokens.cpu().numpy()
        assert np.array_equal(before, st.tokens)
        B.canvas_step(model, canvas, kv, t, SEED, scfg, stats, ws)
        torch.cuda.synchronize()
        Lo = M.canvas_logits(W, before, okv, (bt.numpy(), bv.numpy()))
        Lg = stats.logits.float().cpu().numpy().astype(np.float64)
        Lg[np.arange(n), bt.numpy()] += bv.numpy().astype(np.float64)
        check_logit_rows(rel_l2_rows(Lg, Lo), 2e-2, lambda: route_margins(W, before, okv), 3e-2)
        rec = check_sampler_step(B, st, ocfg, Lg, t, SEED, 4, stats, canvas, rounded_from_f32=True)
        drawn += int(rec.selected.sum())
        if st.done:
            break
    assert drawn >= 2


def test_tiny_generation_matches_the_oracle_trajectory(B):
    """Two canvases generated end to end on the GPU (dg_generate_canvas with
    the append) against the oracle's own independent generation."""
    cfg, model, kv, ws, W, okv = _tiny_setup(B)
    n = cfg.canvas
    scfg = B.sampler_default()
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=torch.float32)
    for c in range(2):
        bt, bv = wl.canvas_boost(cfg, c)
        canvas = B.Canvas(n, cfg.mask_id, c, "cuda", bt.cuda(), bv.cuda())
        steps = B.generate_canvas(model, canvas, kv, scfg, SEED, True, stats, ws, poll_every=3)
        ost, recs = G.denoise_canvas(G.model_provider(W, okv, (bt.numpy(), bv.numpy())), n, ocfg, SEED, c)
        M.encoder_append(W, okv, ost.tokens)
        toks = canvas.tokens.cpu().numpy()
        if not np.array_equal(toks, ost.tokens):
            # only allowed when the oracle's own run met a near tie somewhere
            gaps = []
            for r in recs:
                h = np.sort(r.H_dec[~np.isnan(r.H_dec)])
                gaps.append(np.min(np.diff(h)) if h.size > 1 else 1.0)
            assert min(gaps) < 1e-3, (c, toks, ost.tokens)
        else:
            assert steps == ost.steps
    torch.cuda.synchronize()
    assert kv.length == wl.TINY_PREFIX + 2 * n


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_experts_hit_counts_the_routed_experts(B, name):
    """The per-layer hit count a step reports equals the number of distinct
    routed experts of that layer, taken layer by layer from the same state."""
    cfg = CFGS[name]
    model = device_model(B, cfg)
    P = 300 if name != "tiny_f32" else wl.TINY_PREFIX
    n = cfg.canvas
    kv = B.KVCache(model, P + n)
    fill_synthetic_kv(kv, cfg, P)
    ws = model.workspace(n)
    canvas = B.Canvas(n, cfg.mask_id, 0, "cuda")
    canvas.tokens.copy_(_canvas_tokens(cfg, n // 2))
    stats = B.StepStats(n, vocab=cfg.vocab, logits_dtype=model.act_dtype, n_layers=cfg.n_layers)
    B.canvas_step(model, canvas, kv, 0, SEED, B.sampler_default(), stats, ws)
    X = torch.empty(n, cfg.d_model, dtype=torch.float32, device="cuda")
    B.embed(model, _canvas_tokens(cfg, n // 2), X)
    ids = torch.zeros(n, cfg.top_k, dtype=torch.int32, device="cuda")
    want = []
    for l in range(cfg.n_layers):
        B.decoder_layer(model, l, X, kv, ws, ids)
        want.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    assert stats.experts_hit.cpu().tolist() == want


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "small_bf16_gumbel"])
def test_step_graph_replays_match_eager_steps(B, name):
    """A captured step replayed with eager work and synchronisation between the
    replays gives, at every step, bit-for-bit the eager step's canvas, state,
    statistics and logits (inverse-CDF draws, and Gumbel-max draws whose
    step index the replay reads from the canvas state)."""
    gumbel = name.endswith("_gumbel")
    name = name.replace("_gumbel", "")
    cfg = CFGS[name]
    model = device_model(B, cfg)
    P = 300 if name != "tiny_f32" else wl.TINY_PREFIX
    n = cfg.canvas
    kv = B.KVCache(model, P + n)
    fill_synthetic_kv(kv, cfg, P)
    bt, bv = wl.canvas_boost(cfg, 0)
    bt, bv = bt.cuda(), bv.cuda()
    dt = model.act_dtype
    ca, cb = B.Canvas(n, cfg.mask_id, 0, "cuda", bt, bv), B.Canvas(n, cfg.mask_id, 0, "cuda", bt, bv)
    sa = B.StepStats(n, vocab=cfg.vocab, logits_dtype=dt)
    sb = B.StepStats(n, vocab=cfg.vocab, logits_dtype=dt)
    ws_a, ws_b = model.workspace(n), model.workspace(n)
    scfg = B.sampler_default()
    if gumbel:
        scfg.draw_mode = B.DG_DRAW_GUMBEL_MAX
    graph = B.StepGraph(model, cb, kv, scfg, SEED, sb, ws_b)
    for t in range(6):
        B.canvas_step(model, ca, kv, t, SEED, scfg, sa, ws_a)
        graph.launch()
        torch.cuda.synchronize()
        assert torch.equal(ca.tokens, cb.tokens), t
        assert torch.equal(ca.committed, cb.committed), t
        assert torch.equal(ca.state, cb.state), t
        assert torch.equal(sa.entropy, sb.entropy), t
        assert torch.equal(sa.argmax, sb.argmax), t
        assert torch.equal(sa.logits, sb.logits), t
        # eager work of the program between replays
        _ = (sb.entropy * 2).sum().item()


@pytest.mark.parametrize("head", ["bf16", "e4m3"])
def test_lm_head_bias_tokens_on_tile_edges(B, head):
    """The LM head's epilogue takes each 128-column half tile with or without
    per-column tests (bias token, MASK, vocabulary end): bias tokens placed on
    half-tile and tile edges (0, 127, 128, 255, 256, MASK, V - 2, ...), some
    boosted past the row's maximum, one banned with -inf. Statistics against
    the oracle on the stored logits, and every row's entropy within 1e-2 nats
    of the oracle's own float64 logits, at tau 0.8 and 0.4."""
    cfg = SMALL_BF16
    n, V = cfg.canvas, cfg.vocab
    embed = wl.embedding(cfg, device="cuda")
    fnorm = wl.final_norm(cfg, device="cuda")
    layers = [wl.layer_weights(cfg, l, device="cuda") for l in range(cfg.n_layers)]
    if head == "e4m3":
        codes, scale = wl.lm_head_e4m3(cfg, device="cuda")
        model = B.Model(cfg, embed, fnorm, layers, lm_head_e4m3=codes, lm_head_scale=scale)
        W = M.Weights(cfg, embed.cpu(), fnorm.cpu(), lambda l: {}, lm_head=(codes.cpu(), scale.cpu()))
        E = W.LM
    else:
        model = B.Model(cfg, embed, fnorm, layers)
        W = M.Weights(cfg, embed.cpu(), fnorm.cpu(), lambda l: {})
        E = W.E
    edges = [0, 127, 128, 255, 256, 383, 384, 511, 512, V - 129, V - 128, V - 2, cfg.mask_id]
    g = torch.Generator().manual_seed(21)
    bt = torch.randint(0, V - 1, (n,), generator=g, dtype=torch.int32)
    bt[:len(edges)] = torch.tensor(edges, dtype=torch.int32)
    bv = torch.rand(n, generator=g) * 12
    bv[1::4] = 30.0
    bv[3] = float("-inf")
    X = torch.randn(n, cfg.d_model, generator=g).cuda()
    ws = model.workspace(n)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    Lo = M.lm_logits(X.cpu().numpy().astype(np.float64), W.final_norm, E, cfg.norm_eps)
    btn, bvn = bt.numpy().astype(np.int64), bv.numpy().astype(np.float64)
    Lo_b = Lo.copy()
    Lo_b[np.arange(n), btn] += bvn
    for t in (0, 47):
        stats = B.StepStats(n, vocab=V, logits_dtype=torch.bfloat16)
        B.lm_head(model, X, B.sampler_default(), t, stats, ws, bt.cuda(), bv.cuda())
        torch.cuda.synchronize()
        Lg = stats.logits.float().cpu().numpy().astype(np.float64)
        assert rel_l2_rows(Lg, Lo).max() < (5e-2 if head == "e4m3" else 1e-2)
        Lb = Lg.copy()
        Lb[np.arange(n), btn] += bvn
        check_statistics(stats, ocfg, Lb, t, rounded_from_f32=True)
        Ho, _, _, _ = S.row_stats(Lo_b, S.temperature(t, ocfg), cfg.mask_id)
        assert np.abs(stats.entropy.cpu().numpy() - Ho).max() < ENT_TOL_NORTH, (head, t)
