"""Oracle for the Entropy-Bounded (EB) sampler: schedule, statistics, selection,
Philox draw, re-masking, adaptive stop. TEST INFRASTRUCTURE ONLY.

Follows [MC-zh] best practice 1 ("擴散取樣設定", diffusion sampling
settings) and its Korean twin [MC-ko] recommendation 1: at most 48 denoising
steps; a temperature that falls linearly from 0.8 to 0.4 and shapes the
logits; at each step the lowest-entropy tokens are chosen so that their
mutual-information upper bound stays at or under an entropy bound of 0.1;
unselected tokens are fully re-noised; sampling stops early only when the
canvas-mean entropy is under 0.005 and the most probable prediction has not
changed over two consecutive steps. [AIT] "알아두면 좋은 것" repeats the same
numbers.

Readings taken where the pages are silent:
* bound: the sum of the selected positions' entropies (nats) is <= bound;
  at least one position is selected while candidates remain;
* candidates are the uncommitted positions; commits are final (commit mode
  "keep"). [BLOG]'s self-correction remark is read as commit mode
  "reselect_all": every position is a candidate at every step, a selected
  position takes a fresh draw, and every unselected position (committed
  before or not) is re-masked and loses its commit;
* entropy, argmax and draws use the tempered distribution softmax(L / tau_t)
  with the MASK id excluded;
* tau_t = tau0 + (tau1 - tau0) * t / (max_steps - 1), indexed by step;
* a committed token is a categorical draw by inverse CDF in vocabulary order
  with one Philox4x32-10 uniform per (position, step, canvas); the optional
  "gumbel_max" draw takes instead the argmax over v of z_v - log(-log u_v)
  (the Gumbel-max identity: an exact draw from softmax(z)), one Philox
  uniform per (position, step, canvas, vocabulary id);
* ties: argmax -> lowest id; selection order -> lower position first;
* stop is tested after the commit; on stop, at the last step, or when every
  position is committed, the remaining positions take their argmax.

Sums that decide an integer outcome are taken by their plain definition in
float64: the selection's prefix sums and the canvas-mean entropy with
``math.fsum`` (the correctly rounded sum, independent of the order), the draw
CDF with numpy's cumulative sum.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ---------------------------------------------------------------------------
# Sampler constants stated on the pages ([MC-zh] best practice 1; [MC-ko]
# recommendation 1; [AIT] good-to-know list).
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class SamplerConfig:
    max_steps: int = 48
    temp_start: float = 0.8
    temp_end: float = 0.4
    bound: float = 0.1
    stop_entropy: float = 0.005
    stable_steps: int = 2
    bound_mode: str = "sum"           # "sum" | "sum_minus_max"
    commit_mode: str = "keep"         # "keep" | "reselect_all"
    draw_mode: str = "inverse_cdf"    # "inverse_cdf" | "gumbel_max"
    mask_id: int = -1                 # excluded vocabulary id (-1: none)


def temperature(t: int, cfg: SamplerConfig) -> float:
    """Linear schedule tau0 -> tau1 over steps 0 .. max_steps-1 ([MC-zh] BP1)."""
    if not 0 <= t < cfg.max_steps:
        raise ValueError("step index out of range")
    if cfg.max_steps == 1:
        return cfg.temp_start
    return cfg.temp_start + (cfg.temp_end - cfg.temp_start) * t / (cfg.max_steps - 1)


# ---------------------------------------------------------------------------
# Per-position statistics of the tempered distribution.
# ---------------------------------------------------------------------------


def tempered(logits_row, tau: float, mask_id: int) -> np.ndarray:
    """z = L / tau in float64 with the MASK column set to -inf."""
    z = np.asarray(logits_row, dtype=np.float64) / tau
    if mask_id >= 0:
        z = z.copy()
        z[..., mask_id] = -np.inf
    return z


def row_stats(logits, tau: float, mask_id: int):
    """Entropy (nats), argmax, max and partition sum of softmax(L/tau) per row.

    H = -sum p log p computed as log S - T / S with M = max z,
    S = sum exp(z - M), T = sum exp(z - M) (z - M); clamped at 0. Argmax takes
    the lowest id among equal maxima (numpy.argmax returns the first).
    Returns float64 H [rows], int64 argmax [rows], float64 M, float64 S.
    """
    z = tempered(np.atleast_2d(logits), tau, mask_id)
    M = z.max(axis=1)
    d = z - M[:, None]
    e = np.exp(d)
    S = e.sum(axis=1)
    with np.errstate(invalid="ignore"):
        ed = np.where(e > 0, e * d, 0.0)    # 0 * -inf contributes 0
    T = ed.sum(axis=1)
    H = np.maximum(0.0, np.log(S) - T / S)
    a = np.argmax(z, axis=1)
    return H, a, M, S


# ---------------------------------------------------------------------------
# EB selection.
# ---------------------------------------------------------------------------


def eb_select(H, committed, bound: float, mode: str = "sum") -> np.ndarray:
    """Positions committed this step ([MC-zh] BP1 token selection).

    Candidates are uncommitted positions, ordered by (entropy, position)
    ascending. With S_k the sum of the first k sorted entropies (float64,
    ``math.fsum``), the step commits the first k* candidates where
      mode "sum":           k* = max{k >= 1 : S_k <= bound}, or 1 if none;
      mode "sum_minus_max": k* = max{k >= 1 : S_{k-1} <= bound}
                            (the bound on the k-1 smallest, S_0 = 0).
    The entropies are non-negative, so S_k grows with k and the first k whose
    sum breaks the bound ends the prefix. Returns a bool mask over all
    positions.
    """
    H = np.asarray(H, dtype=np.float64)
    committed = np.asarray(committed).astype(bool)
    n = H.shape[0]
    sel = np.zeros(n, dtype=bool)
    cand = [i for i in range(n) if not committed[i]]
    if not cand:
        return sel
    order = sorted(cand, key=lambda i: (float(H[i]), i))
    k_star = 0
    for k in range(1, len(order) + 1):
        s_k = math.fsum(float(H[i]) for i in order[:k])
        s_prev = math.fsum(float(H[i]) for i in order[:k - 1])
        ok = (s_k <= bound) if mode == "sum" else (s_prev <= bound)
        if not ok:
            break
        k_star = k
    k_star = max(k_star, 1)
    for i in order[:k_star]:
        sel[i] = True
    return sel


def selection_cut(H, committed, bound: float, mode: str = "sum"):
    """The two sums the selection compared with the bound around its cut, for
    judging near-ties: (the sum at the last accepted k*, the sum at k* + 1),
    i.e. (S_{k*}, S_{k*+1}) in mode "sum" and (S_{k*-1}, S_{k*}) in mode
    "sum_minus_max" (float64, math.fsum; inf past the last candidate)."""
    H = np.asarray(H, dtype=np.float64)
    committed = np.asarray(committed).astype(bool)
    sel = eb_select(H, committed, bound, mode)
    cand = [i for i in range(H.shape[0]) if not committed[i]]
    order = sorted(cand, key=lambda i: (float(H[i]), i))
    k = int(sel.sum()) - (1 if mode == "sum_minus_max" else 0)

    def prefix(j):
        return math.fsum(float(H[i]) for i in order[:j]) if j <= len(order) else math.inf
    return prefix(k), prefix(k + 1)


# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC'11): a counter-based generator; ten rounds of a bijection
# on four 32-bit words, each round multiplying two words by fixed odd
# constants and mixing the high halves with the other words and a round key
# that advances by two Weyl constants.
# ---------------------------------------------------------------------------

_PHILOX_M0 = 0xD2511F53
_PHILOX_M1 = 0xCD9E8D57
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_U32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds on Python ints; returns a tuple of 4 words."""
    c0, c1, c2, c3 = (int(c) & _U32 for c in ctr)
    k0, k1 = (int(k) & _U32 for k in key)
    for r in range(10):
        if r:
            k0 = (k0 + _PHILOX_W0) & _U32
            k1 = (k1 + _PHILOX_W1) & _U32
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> 32, p0 & _U32
        hi1, lo1 = p1 >> 32, p1 & _U32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def draw_uniform(seed: int, pos: int, step: int, canvas_idx: int) -> float:
    """u in [0,1): key = (seed lo, seed hi), counter = (pos, step, canvas, 0),
    first output word, top 24 bits scaled by 2**-24."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    x0 = philox4x32_10((pos, step, canvas_idx, 0), (seed & _U32, seed >> 32))[0]
    return (x0 >> 8) * 2.0 ** -24


def philox4x32_10_many(c0, c1, c2, c3, key):
    """Philox4x32-10 over numpy arrays of counters (uint64 holding 32-bit
    words), the same rounds as philox4x32_10; returns 4 arrays of words."""
    c = [np.asarray(x, dtype=np.uint64) & _U32 for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = (int(k) & _U32 for k in key)
    m = np.uint64(_U32)
    for r in range(10):
        if r:
            k0 = (k0 + _PHILOX_W0) & _U32
            k1 = (k1 + _PHILOX_W1) & _U32
        p0 = np.uint64(_PHILOX_M0) * c[0]
        p1 = np.uint64(_PHILOX_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return c


def gumbel_uniforms(seed: int, pos: int, step: int, canvas_idx: int, V: int) -> np.ndarray:
    """u_v in (0,1) for v < V: counter = (pos, step, canvas, 1 + v // 4),
    output word v % 4, (top 23 bits + 1/2) * 2**-23: never 0 or 1, and every
    value exact in float32, so both precisions take the same u."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    blocks = np.arange((V + 3) // 4, dtype=np.uint64) + np.uint64(1)
    w = philox4x32_10_many(pos, step, canvas_idx, blocks, (seed & _U32, seed >> 32))
    words = np.stack(w, axis=1).reshape(-1)[:V]
    return ((words >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_perturbed(logits_row, tau: float, mask_id: int, seed: int, pos: int, step: int,
                     canvas_idx: int) -> np.ndarray:
    """z_v - log(-log u_v) with z = softmax's argument (MASK at -inf)."""
    z = tempered(logits_row, tau, mask_id)
    u = gumbel_uniforms(seed, pos, step, canvas_idx, z.shape[0])
    return z - np.log(-np.log(u))


def draw_token_gumbel(logits_row, tau: float, mask_id: int, seed: int, pos: int, step: int,
                      canvas_idx: int) -> int:
    """Gumbel-max draw: the lowest v maximising z_v - log(-log u_v)."""
    return int(np.argmax(gumbel_perturbed(logits_row, tau, mask_id, seed, pos, step, canvas_idx)))


def draw_token(logits_row, tau: float, mask_id: int, u: float) -> int:
    """Inverse-CDF categorical draw from softmax(L/tau) in vocabulary order.

    Returns the smallest v with sum_{w<=v} exp(z_w - M) > u * S (float64).
    """
    z = tempered(logits_row, tau, mask_id)
    M = z.max()
    w = np.exp(z - M)
    cdf = np.cumsum(w)
    S = cdf[-1]
    v = int(np.searchsorted(cdf, u * S, side="right"))
    return min(v, z.shape[0] - 1)


# ---------------------------------------------------------------------------
# One sampler step on given logits (O5..O10).
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class CanvasState:
    tokens: np.ndarray            # int64 [N]
    committed: np.ndarray         # bool [N]
    prev_argmax: np.ndarray       # int64 [N]
    stable: int = 0               # consecutive steps with an unchanged argmax vector
    done: bool = False
    steps: int = 0
    canvas_idx: int = 0

    @classmethod
    def fresh(cls, n: int, mask_id: int, canvas_idx: int = 0) -> "CanvasState":
        return cls(tokens=np.full(n, mask_id, dtype=np.int64),
                   committed=np.zeros(n, dtype=bool),
                   prev_argmax=np.full(n, -1, dtype=np.int64),
                   canvas_idx=canvas_idx)

    def copy(self) -> "CanvasState":
        return dataclasses.replace(self, tokens=self.tokens.copy(),
                                   committed=self.committed.copy(),
                                   prev_argmax=self.prev_argmax.copy())


@dataclasses.dataclass
class StepRecord:
    t: int
    tau: float
    H: np.ndarray          # float64 [N]
    H_dec: np.ndarray      # float64 [N]: the entropies the decisions use (H, or those fed in)
    argmax: np.ndarray     # int64 [N]
    selected: np.ndarray   # bool [N]
    drawn: dict            # pos -> token
    mean_H: float
    stop: bool
    finished: bool


def mean_entropy(H) -> float:
    """Canvas-mean entropy over all N positions ([MC-zh] BP1: the mean model
    entropy of the whole canvas): math.fsum of the entropies over N."""
    H = np.asarray(H, dtype=np.float64)
    return math.fsum(float(h) for h in H) / len(H)


def sampler_step(state: CanvasState, logits, t: int, cfg: SamplerConfig, seed: int,
                 H_override=None, argmax_override=None, selected_override=None,
                 stop_override=None) -> StepRecord:
    """Advance ``state`` by one denoising step on logits [N][V] (in place).

    ``H_override`` / ``argmax_override`` let a parity test feed the
    entropies and argmaxes another implementation computed (after checking
    them against this oracle's), so that selection, draws, stop and fill are
    compared on identical inputs. ``selected_override`` / ``stop_override``
    let it adopt the other implementation's selection or stop decision where
    it has judged the two within a stated distance of a tie.
    """
    if state.done:
        raise ValueError("canvas already finished")
    if cfg.mask_id < 0:
        raise ValueError("a canvas needs a MASK id")
    tau = temperature(t, cfg)
    L = np.asarray(logits, dtype=np.float64)
    H, a, _, _ = row_stats(L, tau, cfg.mask_id)
    H_dec = H if H_override is None else np.asarray(H_override, np.float64)
    if argmax_override is not None:
        a = np.asarray(argmax_override, dtype=np.int64)
    if cfg.commit_mode == "keep":
        cand = ~state.committed
    elif cfg.commit_mode == "reselect_all":
        cand = np.ones_like(state.committed)
    else:
        raise ValueError("unknown commit mode")
    sel = eb_select(H_dec, ~cand, cfg.bound, cfg.bound_mode)
    if selected_override is not None:
        sel = np.asarray(selected_override).astype(bool) & cand
    drawn = {}
    for i in np.nonzero(sel)[0]:
        if cfg.draw_mode == "gumbel_max":
            tok = draw_token_gumbel(L[i], tau, cfg.mask_id, seed, int(i), t, state.canvas_idx)
        elif cfg.draw_mode == "inverse_cdf":
            u = draw_uniform(seed, int(i), t, state.canvas_idx)
            tok = draw_token(L[i], tau, cfg.mask_id, u)
        else:
            raise ValueError("unknown draw mode")
        state.tokens[i] = tok
        state.committed[i] = True
        drawn[int(i)] = tok
    # full re-noise of the unselected candidates ([MC-zh] BP1); under
    # "reselect_all" this also takes back earlier commits left unselected
    state.tokens[cand & ~sel] = cfg.mask_id
    state.committed[cand & ~sel] = False
    mH = mean_entropy(H_dec)
    same = bool(np.array_equal(a, state.prev_argmax))
    state.stable = state.stable + 1 if (t > 0 and same) else 1
    stop = (state.stable >= cfg.stable_steps) and (mH < cfg.stop_entropy)
    if stop_override is not None:
        stop = bool(stop_override)
    state.prev_argmax = a.astype(np.int64).copy()
    finished = stop or t == cfg.max_steps - 1 or bool(state.committed.all())
    if finished:
        rest = ~state.committed
        state.tokens[rest] = a[rest]
        state.committed[:] = True
        state.done = True
    state.steps = t + 1
    return StepRecord(t=t, tau=tau, H=H, H_dec=H_dec, argmax=a.astype(np.int64), selected=sel,
                      drawn=drawn, mean_H=mH, stop=stop, finished=finished)
