"""Parity of lockstep batches of canvases (dg_canvas_step_batch,
dg_generate_batch): several users' canvases, each with its own prompt, KV
cache length, logit boost and canvas index, go through one decoder pass and
one LM head; every canvas is checked against the oracle run on that canvas
alone (its logits, statistics and sampler decisions), so batching must leave
each canvas exactly as if it had run by itself."""
import types

import numpy as np
import pytest
import torch

from oracle import generate as G
from oracle import model as M
from oracle import sampler as S
from synth import workloads as wl

from model_fixtures import SMALL_BF16, check_logit_rows, oracle_weights, rel_l2_rows, route_margins
from parity import ENT_TOL_NORTH, check_sampler_step

pytestmark = pytest.mark.gpu

SEED = 0x5EED
# router logit gaps under which the two sides may pick different experts:
# float32 activations (noise ~1e-6), bf16 activations (noise ~5e-3, from the
# rounding of the normalised activations and of the attention output)
ROUTE_TIE = 1e-3
ROUTE_TIE_BF16 = 3e-2


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def _model(B, cfg, max_canvas):
    embed = wl.embedding(cfg, device="cuda")
    fnorm = wl.final_norm(cfg, device="cuda")
    layers = [wl.layer_weights(cfg, l, device="cuda") for l in range(cfg.n_layers)]
    return B.Model(cfg, embed, fnorm, layers, max_canvas=max_canvas)


def _users(B, cfg, model, prompt_lens, ws, boost=True):
    """Per user: a cache prefilled with its own prompt, the oracle's cache of
    the same prompt, and a fresh canvas (own boost and canvas index)."""
    W = oracle_weights(model)
    users = []
    for b, P in enumerate(prompt_lens):
        prompt = wl.prefix_tokens(cfg, P, stream=b)
        kv = B.KVCache(model, P + cfg.canvas)
        B.prefill_append(model, kv, prompt.cuda(), ws)
        okv = M.KVCache.empty(cfg)
        M.encoder_append(W, okv, prompt.numpy())
        bt = bv = None
        if boost:
            bt, bv = wl.canvas_boost(cfg, b)
        canvas = B.Canvas(cfg.canvas, cfg.mask_id, b + 1, "cuda",
                          bt.cuda() if boost else None, bv.cuda() if boost else None)
        users.append(types.SimpleNamespace(kv=kv, okv=okv, canvas=canvas, bt=bt, bv=bv,
                                           st=S.CanvasState.fresh(cfg.canvas, cfg.mask_id, b + 1)))
    torch.cuda.synchronize()
    return W, users


def _rows(stats, r0, n, b):
    """Canvas b's view of the batch statistics."""
    return types.SimpleNamespace(entropy=stats.entropy[r0:r0 + n], lse=stats.lse[r0:r0 + n],
                                 argmax=stats.argmax[r0:r0 + n], selected=stats.selected[r0:r0 + n],
                                 mean_entropy=stats.mean_entropy[b:b + 1])


def _run_decomposed(B, cfg, model, W, users, ws, logit_tol, max_steps=48, route_tie=ROUTE_TIE, commit_mode=0):
    n = cfg.canvas
    nb = len(users)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id, commit_mode=["keep", "reselect_all"][commit_mode])
    stats = B.StepStats(n * nb, vocab=cfg.vocab, logits_dtype=model.act_dtype, n_canvases=nb)
    scfg = B.sampler_default()
    scfg.commit_mode = commit_mode
    finished_at = [None] * nb
    for t in range(max_steps):
        before = [u.canvas.tokens.cpu().numpy() for u in users]
        for u, tb in zip(users, before):
            assert np.array_equal(tb, u.st.tokens)
        B.canvas_step_batch(model, [u.canvas for u in users], [u.kv for u in users], t, SEED, scfg, stats, ws)
        torch.cuda.synchronize()
        Lall = stats.logits.float().cpu().numpy().astype(np.float64)
        for b, u in enumerate(users):
            if u.st.done:
                # a finished canvas rides along unchanged
                assert np.array_equal(u.canvas.tokens.cpu().numpy(), u.st.tokens)
                assert u.canvas.state[B.ST_STEP].item() == finished_at[b] + 1
                continue
            r0 = b * n
            boost = (u.bt.numpy(), u.bv.numpy()) if u.bt is not None else None
            Lo = M.canvas_logits(W, before[b], u.okv, boost)
            Lg = Lall[r0:r0 + n].copy()
            if boost is not None:
                Lg[np.arange(n), boost[0]] += boost[1].astype(np.float64)
            check_logit_rows(rel_l2_rows(Lg, Lo), logit_tol, lambda: route_margins(W, before[b], u.okv), route_tie)
            check_sampler_step(B, u.st, ocfg, Lg, t, SEED, b + 1, _rows(stats, r0, n, b), u.canvas,
                               rounded_from_f32=model.act_dtype == torch.bfloat16)
            if u.st.done:
                finished_at[b] = t
        if all(u.st.done for u in users):
            break
    if max_steps == 48:
        assert all(u.st.done for u in users)
    return finished_at


@pytest.mark.parametrize("commit_mode", [0, 1])
def test_tiny_f32_batch_of_three_users(B, commit_mode):
    cfg = wl.TINY.replace(canvas=64)
    model = _model(B, cfg, 3 * 64)
    ws = model.workspace(3 * 64)
    W, users = _users(B, cfg, model, [128, 200, 64], ws)
    _run_decomposed(B, cfg, model, W, users, ws, 1e-4, commit_mode=commit_mode)


def test_small_bf16_batch_with_an_e4m3_lm_head(B):
    """Two users' canvases through the e4m3 LM head over two 128-row canvases:
    logits against the oracle decoder with the dequantised head."""
    cfg = SMALL_BF16.replace(canvas=128)
    codes, scale = wl.lm_head_e4m3(cfg, device="cuda")
    embed = wl.embedding(cfg, device="cuda")
    fnorm = wl.final_norm(cfg, device="cuda")
    layers = [wl.layer_weights(cfg, l, device="cuda") for l in range(cfg.n_layers)]
    model = B.Model(cfg, embed, fnorm, layers, max_canvas=256, lm_head_e4m3=codes, lm_head_scale=scale)
    ws = model.workspace(256)
    _, users = _users(B, cfg, model, [150, 300], ws)
    host = [{k: v.cpu() for k, v in L.items()} for L in layers]
    W8 = M.Weights(cfg, embed.cpu(), fnorm.cpu(), lambda l: host[l], lm_head=(codes.cpu(), scale.cpu()))
    _run_decomposed(B, cfg, model, W8, users, ws, 2e-2, max_steps=3, route_tie=ROUTE_TIE_BF16)


def test_small_bf16_batch_of_two_users(B):
    cfg = SMALL_BF16.replace(canvas=128)
    model = _model(B, cfg, 256)
    ws = model.workspace(256)
    W, users = _users(B, cfg, model, [150, 300], ws)
    _run_decomposed(B, cfg, model, W, users, ws, 2e-2, max_steps=6, route_tie=ROUTE_TIE_BF16)


def test_generate_batch_matches_each_users_oracle_generation(B):
    cfg = wl.TINY.replace(canvas=64)
    model = _model(B, cfg, 128)
    ws = model.workspace(128)
    W, users = _users(B, cfg, model, [128, 96], ws)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    stats = B.StepStats(128, vocab=cfg.vocab, logits_dtype=torch.float32, n_canvases=2)
    steps = B.generate_batch(model, [u.canvas for u in users], [u.kv for u in users], B.sampler_default(), SEED,
                             True, stats, ws, poll_every=2)
    torch.cuda.synchronize()
    for b, u in enumerate(users):
        boost = (u.bt.numpy(), u.bv.numpy())
        ost, recs = G.denoise_canvas(G.model_provider(W, u.okv, boost), cfg.canvas, ocfg, SEED, b + 1)
        toks = u.canvas.tokens.cpu().numpy()
        if np.array_equal(toks, ost.tokens):
            assert steps[b] == ost.steps, (b, steps[b], ost.steps)
        else:
            # only allowed when the oracle's own run met a near tie somewhere
            gaps = []
            for r in recs:
                h = np.sort(r.H_dec)
                gaps.append(np.min(np.diff(h)) if h.size > 1 else 1.0)
            assert min(gaps) < 1e-3, (b, toks, ost.tokens)
        assert u.kv.length == u.okv.length + cfg.canvas


def test_full_width_batch_of_four_canvases(B):
    """One lockstep step of 4 x 256 canvas rows at the full widths (one layer,
    the 262144-way LM head over 1024 rows in four 256-row blocks), each canvas
    on its own cache; logits of every row against the oracle, rows whose
    oracle routing is a near tie excused."""
    cfg = wl.FULL_LAYER
    nb, n = 4, cfg.canvas
    model = _model(B, cfg, nb * n)
    ws = model.workspace(nb * n)
    W = oracle_weights(model)
    canvases, kvs, okvs, states = [], [], [], []
    for b, (P, nc) in enumerate([(1024, 0), (1500, 64), (2048, 128), (3001, 200)]):
        prompt = wl.prefix_tokens(cfg, P, stream=b)
        kv = B.KVCache(model, P + n)
        B.prefill_append(model, kv, prompt.cuda(), ws)
        okv = M.KVCache.empty(cfg)
        M.encoder_append(W, okv, prompt.numpy())
        toks, com = wl.committed_canvas(cfg, nc)
        c = B.Canvas(n, cfg.mask_id, b, "cuda")
        c.tokens.copy_(toks.cuda())
        c.committed.copy_(com.cuda())
        canvases.append(c)
        kvs.append(kv)
        okvs.append(okv)
        st = S.CanvasState(tokens=toks.numpy().astype(np.int64), committed=com.numpy().astype(bool),
                           prev_argmax=np.full(n, -1, np.int64), canvas_idx=b)
        st.steps = 5
        states.append(st)
    stats = B.StepStats(nb * n, vocab=cfg.vocab, logits_dtype=torch.bfloat16, n_canvases=nb)
    B.canvas_step_batch(model, canvases, kvs, 5, SEED, B.sampler_default(), stats, ws)
    torch.cuda.synchronize()
    Lall = stats.logits.float().cpu().numpy().astype(np.float64)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    for b in range(nb):
        r0 = b * n
        X0 = W.E[states[b].tokens].copy()
        tr = {}
        Xo = M.decoder_layer(X0, W.layer(0), okvs[b].K[0], okvs[b].V[0], 0, cfg, trace=tr)
        srt = -np.sort(-tr["router"], axis=1)
        gap = srt[:, cfg.top_k - 1] - srt[:, cfg.top_k]
        Lo = M.lm_logits(Xo, W.final_norm, W.E, cfg.norm_eps)
        Lg = Lall[r0:r0 + n]
        err = rel_l2_rows(Lg, Lo)
        bad = np.nonzero(err >= 2e-2)[0]
        assert np.all(gap[bad] < ROUTE_TIE_BF16) and bad.size <= n // 32, (b, bad, err[bad], gap[bad])
        ok = err < 2e-2
        Ho, _, _, _ = S.row_stats(Lo, S.temperature(5, ocfg), cfg.mask_id)
        assert np.abs(stats.entropy[r0:r0 + n].cpu().numpy() - Ho)[ok].max() < ENT_TOL_NORTH
        rec = check_sampler_step(B, states[b], ocfg, Lg, 5, SEED, b, _rows(stats, r0, n, b), canvases[b],
                                 rounded_from_f32=True)
        assert rec.selected.sum() >= 1
        del Lo
