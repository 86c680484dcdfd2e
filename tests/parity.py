"""Comparison rules between the HIP path and the oracle (test helpers).

Integer decisions are compared exactly; a mismatch is excused only when the
oracle itself finds the decision within a stated distance of a tie:
* argmax: the oracle's top two tempered logits are within ARGMAX_TIE (relative);
* selection: given identical float32 entropies both sides must agree exactly;
* draw: u*S lies within DRAW_TIE * S of a CDF boundary (float64 on both sides);
* stop: the canvas-mean entropy lies within STOP_TIE of the threshold.
Floating outputs: entropies within ENT_TOL (nats) of the oracle's float64 on
the same logits; logits within a relative L2 bound per row.
"""
from __future__ import annotations

import numpy as np

from oracle import sampler as S

ARGMAX_TIE = 1e-6
DRAW_TIE = 1e-12
STOP_TIE = 1e-3
ENT_TOL = 2e-4          # same logits: float32 accumulation vs float64
ENT_TOL_NORTH = 1e-2    # the stated end-to-end entropy tolerance


def argmax_ok(z_row: np.ndarray, got: int, want: int) -> bool:
    if got == want:
        return True
    zs = np.sort(z_row[np.isfinite(z_row)])[::-1]
    if zs.size < 2:
        return False
    return abs(zs[0] - zs[1]) <= ARGMAX_TIE * max(1.0, abs(zs[0])) and z_row[got] >= zs[1]


GUMBEL_TIE = 1e-5       # relative gap of the two largest z - log(-log u) (float32 vs float64)


def gumbel_is_near_tie(logits_row, tau, mask_id, seed, pos, step, canvas_idx) -> bool:
    vals = S.gumbel_perturbed(logits_row, tau, mask_id, seed, pos, step, canvas_idx)
    top = np.sort(vals[np.isfinite(vals)])[::-1]
    return top.size >= 2 and top[0] - top[1] <= GUMBEL_TIE * max(1.0, abs(top[0]))


def token_mismatch_excused(ocfg, logits_row, tau, seed, pos, step, canvas_idx) -> bool:
    """A drawn token may differ only where the draw is within rounding of a tie."""
    if ocfg.draw_mode == "gumbel_max":
        return gumbel_is_near_tie(logits_row, tau, ocfg.mask_id, seed, pos, step, canvas_idx)
    u = S.draw_uniform(seed, pos, step, canvas_idx)
    return draw_is_near_tie(logits_row, tau, ocfg.mask_id, u)


def draw_is_near_tie(logits_row, tau, mask_id, u) -> bool:
    z = S.tempered(logits_row, tau, mask_id)
    w = np.exp(z - z.max())
    cdf = np.cumsum(w)
    tgt = u * cdf[-1]
    return bool(np.min(np.abs(cdf - tgt)) <= DRAW_TIE * cdf[-1])


def rel_l2_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def check_sampler_step(B, st, ocfg, L, t, seed, canvas_idx, stats, canvas, ent_tol=ENT_TOL):
    """Compare one GPU sampler step with the oracle fed the same (biased) logits.

    ``st`` is the oracle CanvasState before the step; it is advanced in place
    (adopting the GPU's tokens only where a draw is an excused near-tie).
    Returns the oracle's StepRecord."""
    tau = S.temperature(t, ocfg)
    H, a, M, Ssum = S.row_stats(L, tau, ocfg.mask_id)
    Hg = stats.entropy.cpu().numpy()
    ag = stats.argmax.cpu().numpy().astype(np.int64)
    assert np.max(np.abs(Hg - H)) < ent_tol, (t, np.max(np.abs(Hg - H)))
    lse = stats.lse.cpu().numpy()
    assert np.max(np.abs(lse - (M + np.log(Ssum)))) < 1e-4 * max(1.0, float(np.abs(M).max()))
    z = S.tempered(L, tau, ocfg.mask_id)
    for i in np.nonzero(ag != a)[0]:
        assert argmax_ok(z[i], int(ag[i]), int(a[i])), (t, i, ag[i], a[i])
    rec = S.sampler_step(st, L, t, ocfg, seed, H32_override=Hg, argmax_override=ag)
    sel_g = stats.selected.cpu().numpy().astype(bool)
    assert np.array_equal(sel_g, rec.selected), t
    tok_g = canvas.tokens.cpu().numpy().astype(np.int64)
    for i in np.nonzero(tok_g != st.tokens)[0]:
        assert rec.selected[i], (t, i)
        assert token_mismatch_excused(ocfg, L[i], tau, seed, int(i), t, canvas_idx), (t, i, tok_g[i], st.tokens[i])
        st.tokens[i] = tok_g[i]
    assert np.array_equal(canvas.committed.cpu().numpy().astype(bool), st.committed)
    state = canvas.state.cpu().numpy()
    assert state[B.ST_DONE] == int(st.done)
    assert state[B.ST_STEP] == t + 1
    assert state[B.ST_STABLE] == st.stable
    assert state[B.ST_STOP] == int(rec.stop)
    assert state[B.ST_FINISHED] == int(rec.finished)
    assert state[B.ST_SELECTED] == int(rec.selected.sum())
    assert stats.mean_entropy.item() == rec.mean_H
    assert np.array_equal(canvas.prev_argmax.cpu().numpy(), ag)
    assert np.array_equal(tok_g, st.tokens)
    return rec
