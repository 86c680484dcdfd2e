"""Comparison rules between the HIP path and the oracle (test helpers).

Integer decisions are compared exactly; a mismatch is excused only when the
oracle itself finds the decision within a stated distance of a tie:
* argmax: the GPU's pick is within the rounding of the oracle's maximum
  (ARGMAX_TIE relative on the same logits; the logit error of the row when
  the oracle's logits are its own);
* selection (fed the GPU's entropies): the oracle's float64 prefix sum at
  the cut lies within SEL_TIE of the bound, or every position on which the
  two disagree has an entropy within SEL_TIE of the entropy at the cut;
* draw: u*S lies within DRAW_TIE * S of a CDF boundary (float64 on both sides);
* stop: the canvas-mean entropy lies within STOP_TIE of the threshold.
Where a selection or stop is excused, the oracle adopts the GPU's decision
and the rest of the step (draws, re-mask, fill, state) is still compared.
Floating outputs: entropies within ENT_TOL (nats) of the oracle's float64 on
the same logits, and within ENT_TOL_NORTH of the oracle's own logits;
logits within a relative L2 bound per row.
"""
from __future__ import annotations

import numpy as np

from oracle import sampler as S

ARGMAX_TIE = 1e-6
DRAW_TIE = 1e-12
SEL_TIE = 1e-3
STOP_TIE = 1e-3
ENT_TOL = 2e-4          # same logits: float32 accumulation vs float64
ENT_TOL_NORTH = 1e-2    # the stated end-to-end entropy tolerance
MEAN_REL = 1e-12        # canvas mean: float64 position-order sum vs math.fsum


def argmax_ok(z_row: np.ndarray, got: int, want: int, slack: float = 0.0) -> bool:
    """``got`` is an acceptable argmax of z_row: equal to the first maximum,
    or within ARGMAX_TIE (relative) plus ``slack`` of it."""
    if got == want:
        return True
    zs = np.sort(z_row[np.isfinite(z_row)])[::-1]
    if zs.size < 2:
        return False
    return bool(z_row[got] >= zs[0] - ARGMAX_TIE * max(1.0, abs(zs[0])) - slack)


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


def selection_mismatch_excused(H, committed, bound, mode, sel_gpu, sel_ora) -> bool:
    """The GPU's selection may differ from the oracle's (both fed the same
    entropies) only at a near-tie: the oracle's prefix sums around the cut
    lie within SEL_TIE of the bound, or every disputed position's entropy is
    within SEL_TIE of the entropy at the cut."""
    diff = np.nonzero(np.asarray(sel_gpu, bool) != np.asarray(sel_ora, bool))[0]
    if diff.size == 0:
        return True
    s_in, s_out = S.selection_cut(H, committed, bound, mode)
    if abs(s_in - bound) < SEL_TIE or abs(s_out - bound) < SEL_TIE:
        return True
    H = np.asarray(H, np.float64)
    chosen = np.nonzero(np.asarray(sel_ora, bool))[0]
    h_cut = H[chosen].max() if chosen.size else 0.0
    return bool(np.all(np.abs(H[diff] - h_cut) < SEL_TIE))


def rel_l2_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of each value (the most its
    round-to-nearest rounding can move it): 2^(floor(log2|x|) - 8)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, np.exp2(e - 8), 0.0)


def entropy_rounding_bound(Lrec, tau, mask_id):
    """Per row, the most the entropy of softmax(L / tau) can move to first
    order when every logit moves by at most half a bf16 ulp of its rounded
    value Lrec: |dH| <= sum_v p_v |log p_v + H| |dz_v| (dH/dz_v = -p_v
    (log p_v + H)). Used where the GPU's statistics come from the unrounded
    f32 logits and only their bf16 rounding is stored."""
    z = S.tempered(Lrec, tau, mask_id)
    H, _, M, Ssum = S.row_stats(Lrec, tau, mask_id)
    lp = z - (M + np.log(Ssum))[:, None]
    p = np.exp(lp)
    dz = bf16_half_ulp(Lrec) / tau
    with np.errstate(invalid="ignore"):
        w = np.where(p > 0, p * np.abs(lp + H[:, None]) * dz, 0.0)
    return w.sum(axis=1)


def check_statistics(stats, ocfg, L, t, *, rounded_from_f32=False, ent_tol=ENT_TOL):
    """The GPU's entropy, LSE and argmax of one step against the oracle on the
    logits the step drew from (L: logits of record plus bias, float64).
    rounded_from_f32: the GPU took the statistics from f32 values whose bf16
    rounding L holds, so entropies may differ by the first-order effect of
    that rounding (1.5x, plus ent_tol) and the argmax by a tie within it."""
    tau = S.temperature(t, ocfg)
    H, a, M, Ssum = S.row_stats(L, tau, ocfg.mask_id)
    Hg = stats.entropy.cpu().numpy().astype(np.float64)
    ag = stats.argmax.cpu().numpy().astype(np.int64)
    lse = stats.lse.cpu().numpy().astype(np.float64)
    z = S.tempered(L, tau, ocfg.mask_id)
    if rounded_from_f32:
        bound = 1.5 * entropy_rounding_bound(L, tau, ocfg.mask_id) + ent_tol
        # the rounding of the row's largest finite logit (a -inf from a
        # banning bias is no rounding)
        slack = 2.0 * bf16_half_ulp(np.max(np.where(np.isfinite(L), np.abs(L), 0.0), axis=1)) / tau
    else:
        bound = np.full(L.shape[0], ent_tol)
        slack = np.zeros(L.shape[0])
    err = np.abs(Hg - H)
    assert np.all(err <= bound), (t, int(np.argmax(err - bound)), float(err.max()))
    lse_tol = 1e-4 * max(1.0, float(np.abs(M).max())) + slack
    assert np.all(np.abs(lse - (M + np.log(Ssum))) <= lse_tol), t
    for i in np.nonzero(ag != a)[0]:
        assert argmax_ok(z[i], int(ag[i]), int(a[i]), float(slack[i])), (t, i, ag[i], a[i])
    return Hg, ag


def check_sampler_step(B, st, ocfg, L, t, seed, canvas_idx, stats, canvas, ent_tol=ENT_TOL,
                       rounded_from_f32=False):
    """Compare one GPU sampler step with the oracle fed the same (biased)
    logits L, the logits the GPU drew from.

    ``st`` is the oracle CanvasState before the step; it is advanced in place
    (adopting the GPU's selection or stop only where excused as a near-tie,
    and its tokens only where a draw is an excused near-tie). Returns the
    oracle's StepRecord."""
    tau = S.temperature(t, ocfg)
    Hg, ag = check_statistics(stats, ocfg, L, t, rounded_from_f32=rounded_from_f32, ent_tol=ent_tol)
    sel_g = stats.selected.cpu().numpy().astype(bool)
    state = canvas.state.cpu().numpy()
    st0 = st.copy()
    rec = S.sampler_step(st, L, t, ocfg, seed, H_override=Hg, argmax_override=ag)
    overrides = {}
    if not np.array_equal(sel_g, rec.selected):
        cand_com = st0.committed if ocfg.commit_mode == "keep" else np.zeros_like(st0.committed)
        assert selection_mismatch_excused(Hg, cand_com, ocfg.bound, ocfg.bound_mode, sel_g, rec.selected), t
        overrides["selected_override"] = sel_g
    if int(state[B.ST_STOP]) != int(rec.stop):
        assert abs(rec.mean_H - ocfg.stop_entropy) < STOP_TIE, (t, rec.mean_H)
        overrides["stop_override"] = bool(state[B.ST_STOP])
    if overrides:
        st.__dict__.update(st0.copy().__dict__)
        rec = S.sampler_step(st, L, t, ocfg, seed, H_override=Hg, argmax_override=ag, **overrides)
    assert np.array_equal(sel_g, rec.selected), t
    tok_g = canvas.tokens.cpu().numpy().astype(np.int64)
    for i in np.nonzero(tok_g != st.tokens)[0]:
        assert rec.selected[i], (t, i)
        assert token_mismatch_excused(ocfg, L[i], tau, seed, int(i), t, canvas_idx), (t, i, tok_g[i], st.tokens[i])
        st.tokens[i] = tok_g[i]
    assert np.array_equal(canvas.committed.cpu().numpy().astype(bool), st.committed)
    assert state[B.ST_DONE] == int(st.done)
    assert state[B.ST_STEP] == t + 1
    assert state[B.ST_STABLE] == st.stable
    assert state[B.ST_STOP] == int(rec.stop)
    assert state[B.ST_FINISHED] == int(rec.finished)
    assert state[B.ST_SELECTED] == int(rec.selected.sum())
    mg = stats.mean_entropy.item()
    assert abs(mg - rec.mean_H) <= MEAN_REL * max(1.0, abs(rec.mean_H)), (mg, rec.mean_H)
    assert np.array_equal(canvas.prev_argmax.cpu().numpy(), ag)
    assert np.array_equal(tok_g, st.tokens)
    return rec
