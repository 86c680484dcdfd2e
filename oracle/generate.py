"""Oracle for block-autoregressive multi-canvas generation. TEST INFRASTRUCTURE ONLY.

[MC-zh] "模型總覽" (overview) and [AIT] "기술적 특징": the encoder prefills
the prompt into the KV cache; a canvas starts as placeholders ([GATE], how the
model generates) and is denoised by the diffusion sampler until it is fully
denoised; it is then run through the encoder and appended to the KV cache,
and the next canvas starts.

The logits of each step come from a provider: the decoder over the canvas and
the cache (``model_provider``) or a scripted list of logit tensors
(``scripted_provider``), so that schedule, selection, re-masking and the stop
rule can be exercised with no transformer at all.
"""
from __future__ import annotations

import numpy as np

from . import model as M
from . import sampler as S


def model_provider(W: M.Weights, kv: M.KVCache, boost=None):
    def provide(state: S.CanvasState, t: int):
        return M.canvas_logits(W, state.tokens, kv, boost)
    return provide


def scripted_provider(seq):
    """Logits for step t are seq[t] (any [N][V] array)."""
    def provide(state: S.CanvasState, t: int):
        return np.asarray(seq[t], dtype=np.float64)
    return provide


def denoise_canvas(provider, n: int, scfg: S.SamplerConfig, seed: int, canvas_idx: int = 0,
                   on_step=None):
    """Run the EB sampler from an all-MASK canvas until it finishes.

    Returns (final state, list of StepRecord).
    """
    state = S.CanvasState.fresh(n, scfg.mask_id, canvas_idx)
    records = []
    for t in range(scfg.max_steps):
        logits = provider(state, t)
        rec = S.sampler_step(state, logits, t, scfg, seed)
        records.append(rec)
        if on_step is not None:
            on_step(state, rec, logits)
        if state.done:
            break
    return state, records


def generate(W: M.Weights, prompt, n_canvases: int, scfg: S.SamplerConfig, seed: int,
             boost_fn=None, append_last: bool = True):
    """Prefill the prompt, then denoise and append ``n_canvases`` canvases.

    ``boost_fn(canvas_idx)`` may return a per-row one-hot logit boost.
    Returns (list of canvas token arrays, list of step counts, KV cache).
    """
    cfg = W.cfg
    kv = M.KVCache.empty(cfg)
    M.encoder_append(W, kv, prompt)
    canvases, steps = [], []
    for c in range(n_canvases):
        boost = boost_fn(c) if boost_fn is not None else None
        state, recs = denoise_canvas(model_provider(W, kv, boost), cfg.canvas, scfg, seed, c)
        canvases.append(state.tokens.copy())
        steps.append(state.steps)
        if append_last or c < n_canvases - 1:
            M.encoder_append(W, kv, state.tokens)
    return canvases, steps, kv
