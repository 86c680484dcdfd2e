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
