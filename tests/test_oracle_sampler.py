"""Pins of the sampler oracle against the pages' constants, closed forms,
brute force, a library routine run independently (rocRAND's Philox) and
statistics. CPU only."""
import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import scipy.stats

from oracle import sampler as S

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "sampler_constants.json")))


# --------------------------------------------------------------- constants ---

def test_defaults_are_the_pages_constants():
    c = S.SamplerConfig()
    assert c.max_steps == GOLD["max_steps"]
    assert c.temp_start == GOLD["temp_start"] and c.temp_end == GOLD["temp_end"]
    assert c.bound == GOLD["entropy_bound"]
    assert c.stop_entropy == GOLD["stop_entropy"]
    assert c.stable_steps == GOLD["stable_steps"]


def test_schedule_endpoints_and_linearity():
    c = S.SamplerConfig()
    taus = [S.temperature(t, c) for t in range(c.max_steps)]
    assert taus[0] == 0.8
    assert abs(taus[-1] - 0.4) < 1e-15
    d = np.diff(taus)
    assert np.allclose(d, -0.4 / 47, rtol=0, atol=1e-15)
    assert abs(taus[1] - 0.7914893617021276) < 1e-15
    with pytest.raises(ValueError):
        S.temperature(48, c)
    with pytest.raises(ValueError):
        S.temperature(-1, c)


# -------------------------------------------------------------- statistics ---

@pytest.mark.parametrize("V", [4096, 262144])
def test_entropy_uniform_row_is_log_V(V):
    L = np.zeros((1, V))
    H, a, M, Ssum = S.row_stats(L, 0.8, -1)
    assert abs(H[0] - math.log(V)) < 1e-9
    assert a[0] == 0                          # ties -> lowest id
    assert Ssum[0] == V
    H, a, _, _ = S.row_stats(L, 0.8, V - 1)   # MASK excluded
    assert abs(H[0] - math.log(V - 1)) < 1e-9
    assert abs(math.log(262144) - 12.476649250079) < 1e-9 or V != 262144


def test_entropy_one_hot_is_zero():
    V = 1000
    L = np.full((3, V), -np.inf)
    L[0, 7] = 3.0
    L[1, 0] = -50.0
    L[2, V - 1] = 1e4
    H, a, _, _ = S.row_stats(L, 0.5, -1)
    assert np.all(H == 0.0)
    assert list(a) == [7, 0, V - 1]
    # a finite but overwhelming peak is also (numerically) zero entropy
    L2 = np.zeros((1, V))
    L2[0, 3] = 200.0
    H2, _, _, _ = S.row_stats(L2, 0.4, -1)
    assert H2[0] < 1e-100


def test_entropy_two_point_is_binary_entropy():
    for p in (0.5, 0.1, 1e-3, 0.9999):
        tau = 0.6
        L = np.full((1, 50), -np.inf)
        L[0, 10] = tau * math.log(p)
        L[0, 40] = tau * math.log(1 - p)
        H, a, _, _ = S.row_stats(L, tau, -1)
        hb = -(p * math.log(p) + (1 - p) * math.log(1 - p))
        assert abs(H[0] - hb) < 1e-12
        assert a[0] == (10 if p > 0.5 else 40 if p < 0.5 else 10)


def test_entropy_matches_scipy_and_is_shift_invariant():
    rng = np.random.default_rng(0)
    L = rng.normal(size=(6, 3000)) * rng.uniform(0.1, 5, size=(6, 1))
    tau = 0.55
    H, a, M, Ssum = S.row_stats(L, tau, 2999)
    for i in range(6):
        z = L[i, :2999] / tau
        p = scipy.special.softmax(z)
        assert abs(H[i] - scipy.stats.entropy(p)) < 1e-10
        assert abs((M[i] + math.log(Ssum[i])) - scipy.special.logsumexp(z)) < 1e-10
        assert a[i] == int(np.argmax(z))
    H2, a2, _, _ = S.row_stats(L + 123.25, tau, 2999)
    assert np.allclose(H, H2, atol=1e-10) and np.array_equal(a, a2)


def test_temperature_lowers_entropy():
    rng = np.random.default_rng(1)
    L = rng.normal(size=(4, 500))
    H_hot, _, _, _ = S.row_stats(L, 0.8, -1)
    H_cold, _, _, _ = S.row_stats(L, 0.4, -1)
    assert np.all(H_cold < H_hot)


# ------------------------------------------------------------- EB select ---

def _brute_force(H, committed, bound, mode):
    """The largest subset of candidates whose summed entropies (minus the
    largest, in sum_minus_max mode) stay within the bound, then the smallest
    sum, then the lexicographically smallest positions; one argmin position
    when no non-empty subset qualifies. Sums are exact (math.fsum)."""
    n = len(H)
    cand = [i for i in range(n) if not committed[i]]
    if not cand:
        return set()
    best = None
    for r in range(len(cand), 0, -1):
        for U in itertools.combinations(cand, r):
            hs = sorted(float(H[i]) for i in U)
            tot = math.fsum(hs)
            lim = math.fsum(hs[:-1]) if mode == "sum_minus_max" else tot
            if lim <= bound:
                key = (tot, sorted(U))
                if best is None or key < best:
                    best = key
        if best is not None:
            return set(best[1])
    i = min(cand, key=lambda i: (float(H[i]), i))
    return {i}


@pytest.mark.parametrize("mode", ["sum", "sum_minus_max"])
def test_eb_select_equals_brute_force(mode):
    rng = np.random.default_rng(42)
    checked = 0
    for trial in range(400):
        n = int(rng.integers(1, 11))
        scale = float(rng.choice([0.005, 0.02, 0.05, 0.2]))
        H = rng.exponential(scale, size=n)
        if trial % 5 == 0:                     # exact ties
            H[rng.integers(0, n, size=n // 2)] = H[0]
        com = rng.random(n) < 0.3
        got = set(np.nonzero(S.eb_select(H, com, 0.1, mode))[0].tolist())
        assert got == _brute_force(H, com, 0.1, mode), (H, com)
        checked += 1
    assert checked == 400


def test_selection_and_mean_use_exact_sums():
    """Prefix sums and the canvas mean are the correctly rounded float64 sums
    (math.fsum), so neither the summation order nor cancellation moves a
    decision: a cut that lands exactly on the bound is inclusive, and many
    tiny entropies after a large one still count in the mean."""
    H = np.array([0.05, 0.05, 0.3])
    assert 0.05 + 0.05 == 0.1
    sel = S.eb_select(H, np.zeros(3, bool), 0.1)
    assert sel.tolist() == [True, True, False]
    s_k, s_next = S.selection_cut(H, np.zeros(3, bool), 0.1)
    assert s_k == 0.1 and s_next == math.fsum(H)
    Hm = np.array([1.0] + [1e-16] * 10)
    naive = 0.0
    for h in Hm:
        naive += h
    assert naive == 1.0 and math.fsum(Hm) > 1.0
    assert S.mean_entropy(Hm) == math.fsum(Hm) / len(Hm) != naive / len(Hm)


def test_eb_select_special_cases():
    n = 16
    H = np.zeros(n)
    com = np.zeros(n, bool)
    com[3] = True
    sel = S.eb_select(H, com, 0.1)
    assert sel.sum() == n - 1 and not sel[3]             # all-zero -> all candidates
    H = np.linspace(0.5, 2.0, n).astype(np.float32)[::-1].copy()
    sel = S.eb_select(H, np.zeros(n, bool), 0.1)
    assert sel.sum() == 1 and sel[n - 1]                  # all > bound -> exactly one (min H)
    sel = S.eb_select(H, np.ones(n, bool), 0.1)
    assert sel.sum() == 0                                 # no candidates
    H = np.full(n, 0.04)
    assert S.eb_select(H, np.zeros(n, bool), 0.1).sum() == 2          # 0.08 <= 0.1 < 0.12
    assert S.eb_select(H, np.zeros(n, bool), 0.1, "sum_minus_max").sum() == 3
    # tie at the cut: lower position first
    H = np.array([0.06, 0.05, 0.05, 0.05])
    sel = S.eb_select(H, np.zeros(4, bool), 0.1)
    assert list(np.nonzero(sel)[0]) == [1, 2]


# ------------------------------------------------------------------ Philox ---

def _rocrand_probe():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("rocRAND headers or hipcc not available")
    out = os.path.join(os.environ.get("TMPDIR", "/tmp"), "dg_rocrand_philox_probe")
    src = os.path.join(HERE, "golden", "rocrand_philox_probe.cpp")
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", "-o", out, src],
                       check=True, capture_output=True)
    return out


def test_philox_matches_rocrand_engine():
    probe = _rocrand_probe()
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 2, 3, 4, 5, 6)]
    for _ in range(200):
        cases.append(tuple(int(x) for x in rng.integers(0, 2 ** 32, size=6, dtype=np.uint64)))
    for pos in (0, 17, 255):
        for step in (0, 47):
            cases.append((pos, step, 3, 0, 0x5EED, 0))
    inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    res = subprocess.run([probe], input=inp, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(cases)
    for c, line in zip(cases, lines):
        want = tuple(int(x) for x in line.split())
        assert S.philox4x32_10(c[:4], c[4:]) == want, c


def test_draw_uniform_is_uniform():
    n = 100_000
    u = np.array([S.draw_uniform(0x5EED, i % 256, (i // 256) % 48, i // (256 * 48)) for i in range(n)])
    assert u.min() >= 0.0 and u.max() < 1.0
    hist, _ = np.histogram(u, bins=50, range=(0, 1))
    chi2 = ((hist - n / 50) ** 2 / (n / 50)).sum()
    assert chi2 < scipy.stats.chi2.ppf(0.999, 49)
    # distinct counters give distinct words; the seed's high half matters
    assert S.draw_uniform(1, 0, 0, 0) != S.draw_uniform(1 + (1 << 32), 0, 0, 0)


# -------------------------------------------------------------------- draw ---

def test_draw_boundaries_on_a_uniform_row():
    L = np.zeros(5)                       # MASK = 4 excluded -> p = 1/4 each
    tau = 0.7
    assert S.draw_token(L, tau, 4, 0.0) == 0
    assert S.draw_token(L, tau, 4, 0.25 - 2 ** -24) == 0
    assert S.draw_token(L, tau, 4, 0.25) == 1      # cdf_0 = 0.25 is not > 0.25
    assert S.draw_token(L, tau, 4, 0.75) == 3
    assert S.draw_token(L, tau, 4, 1 - 2 ** -24) == 3


def test_draw_one_hot_and_never_mask():
    L = np.full(64, -np.inf)
    L[9] = 60.0
    for u in (0.0, 0.5, 1 - 2 ** -24):
        assert S.draw_token(L, 0.4, 63, u) == 9
    L = np.zeros(8)
    L[7] = 100.0                                   # MASK has the largest logit
    toks = {S.draw_token(L, 0.8, 7, u) for u in np.linspace(0, 1 - 1e-9, 50)}
    assert 7 not in toks


def test_draw_frequencies_follow_softmax():
    rng = np.random.default_rng(3)
    V = 12
    L = rng.normal(size=V) * 1.5
    tau = 0.8
    p = scipy.special.softmax(np.where(np.arange(V) == V - 1, -np.inf, L / tau))
    n = 20000
    counts = np.zeros(V)
    for i in range(n):
        counts[S.draw_token(L, tau, V - 1, S.draw_uniform(99, i, 0, 0))] += 1
    assert counts[V - 1] == 0
    se = np.sqrt(n * p * (1 - p)) + 1e-9
    assert np.all(np.abs(counts - n * p) < 5 * se + 1)


# -------------------------------------------------------------- stop rule ---

def _rows_with_entropy(n, V, h, tau, argmax_ids):
    """Rows whose tempered distribution is two-point with binary entropy h."""
    if h <= 0:
        p = 1.0
    else:
        p = scipy.optimize.brentq(lambda q: -(q * math.log(q) + (1 - q) * math.log(1 - q)) - h,
                                  0.5, 1 - 1e-15)
    L = np.full((n, V), -1e30)
    for i in range(n):
        a = int(argmax_ids[i])
        b = (a + 1) % (V - 1)
        L[i, a] = 0.0
        L[i, b] = tau * (math.log(1 - p) - math.log(p)) if p < 1 else -1e30
    return L


def _run(seq_fn, n=256, V=64, seed=5):
    cfg = S.SamplerConfig(mask_id=V - 1)
    st = S.CanvasState.fresh(n, cfg.mask_id)
    recs = []
    for t in range(cfg.max_steps):
        rec = S.sampler_step(st, seq_fn(t, S.temperature(t, cfg)), t, cfg, seed)
        recs.append(rec)
        _check_invariants(st, recs, V - 1)
        if st.done:
            break
    return st, recs


_prev_tokens = {}


def _check_invariants(st, recs, mask):
    for i in range(len(st.tokens)):
        if st.committed[i]:
            assert st.tokens[i] != mask
        else:
            assert st.tokens[i] == mask
    rec = recs[-1]
    if len(recs) > 1 and not rec.finished:
        assert rec.selected.sum() >= 1


def test_stop_fires_when_confident_and_stable():
    ids = np.arange(256) % 50
    st, recs = _run(lambda t, tau: _rows_with_entropy(256, 64, 0.0049, tau, ids))
    assert [r.stop for r in recs] == [False, True]        # never at t = 0
    assert st.steps == 2 and st.done
    assert recs[0].selected.sum() == 20                    # 20 * 0.0049 <= 0.1 < 21 * 0.0049
    assert np.array_equal(st.tokens[~recs[0].selected & ~recs[1].selected],
                          ids[~recs[0].selected & ~recs[1].selected])   # argmax fill


def test_no_stop_when_argmax_flips():
    st, recs = _run(lambda t, tau: _rows_with_entropy(256, 64, 0.0049, tau,
                                                      (np.arange(256) + t) % 50))
    assert not any(r.stop for r in recs)
    assert recs[-1].finished and st.committed.all()
    assert st.steps == 13                                  # 256 / 20 per step


def test_no_stop_when_entropy_too_high():
    ids = np.arange(256) % 50
    st, recs = _run(lambda t, tau: _rows_with_entropy(256, 64, 0.006, tau, ids))
    assert not any(r.stop for r in recs)
    assert st.steps == 16                                  # 16 per step


def test_stop_threshold_is_strict():
    cfg = S.SamplerConfig(mask_id=63)
    L = _rows_with_entropy(256, 64, 0.3, 0.8, np.arange(256) % 50)
    for h, want in ((np.float32(0.005), True),
                    (np.nextafter(np.float32(0.005), np.float32(1)), False)):
        assert (float(h) < 0.005) == want
        st = S.CanvasState.fresh(256, 63)
        Hs = np.full(256, h, np.float32)
        S.sampler_step(st, L, 0, cfg, 1, H_override=Hs)
        rec = S.sampler_step(st, L, 1, cfg, 1, H_override=Hs)
        assert rec.stop == want


def test_never_confident_runs_all_48_steps_then_fills_argmax():
    rng = np.random.default_rng(11)
    n, V = 64, 300
    seq = [rng.normal(size=(n, V)) for _ in range(48)]
    st, recs = _run(lambda t, tau: seq[t], n=n, V=V)
    assert st.steps == 48 and len(recs) == 48
    assert all(r.selected.sum() == 1 for r in recs)
    last = recs[-1]
    filled = np.ones(n, bool)
    for r in recs:
        filled &= ~r.selected
    assert filled.sum() == n - 48
    assert np.array_equal(st.tokens[filled], last.argmax[filled])
    assert not np.any(st.tokens == V - 1)


def test_everything_committed_at_step_zero():
    L = np.full((32, 16), -1e30)
    L[np.arange(32), np.arange(32) % 15] = 0.0             # one-hot rows, H = 0
    st, recs = _run(lambda t, tau: L, n=32, V=16)
    assert len(recs) == 1 and recs[0].finished and not recs[0].stop
    assert np.array_equal(st.tokens, np.arange(32) % 15)


def test_committed_tokens_never_change():
    rng = np.random.default_rng(12)
    n, V = 48, 200
    cfg = S.SamplerConfig(mask_id=V - 1)
    st = S.CanvasState.fresh(n, V - 1)
    seen = {}
    for t in range(48):
        L = rng.normal(size=(n, V)) * rng.uniform(0.5, 30, size=(n, 1))
        rec = S.sampler_step(st, L, t, cfg, 77)
        for i, tok in seen.items():
            assert st.tokens[i] == tok
        for i in np.nonzero(rec.selected)[0]:
            seen[int(i)] = int(st.tokens[i])
        if st.done:
            break
    assert st.done and st.committed.all()


# ---------------------------------------------------- reselect-all commits ---

def _one_hot_or_flat(n, V, confident):
    """Rows that are one-hot (entropy 0) where ``confident``, flat otherwise
    (entropy log(V - 1), far above the bound), MASK = V - 1 excluded."""
    L = np.zeros((n, V))
    for i in np.nonzero(confident)[0]:
        L[i, :] = -1e30
        L[i, i % (V - 1)] = 0.0
    return L


@pytest.mark.parametrize("mode", ["sum", "sum_minus_max"])
def test_reselect_all_step_equals_brute_force_over_every_position(mode):
    """Under reselect_all the selected set is the brute-force optimum over all
    positions, whatever was committed before; after the step the committed
    set is exactly the selected set, selected rows hold this step's draw and
    all other rows hold MASK."""
    rng = np.random.default_rng(21)
    V, mask, seed = 7, 6, 4242
    checked = 0
    for trial in range(300):
        n = int(rng.integers(1, 10))
        cfg = S.SamplerConfig(mask_id=mask, bound_mode=mode, commit_mode="reselect_all")
        H = rng.exponential(float(rng.choice([0.01, 0.03, 0.1])), size=n).astype(np.float32)
        order = sorted(range(n), key=lambda i: (H[i], i))
        if any(abs(s - 0.1) < 1e-6 for s in np.cumsum([float(H[i]) for i in order])):
            continue
        st = S.CanvasState.fresh(n, mask)
        st.committed[:] = rng.random(n) < 0.5
        st.tokens[st.committed] = rng.integers(0, mask, size=int(st.committed.sum()))
        L = rng.normal(size=(n, V)) * 3.0
        t = int(rng.integers(0, 47))
        rec = S.sampler_step(st, L, t, cfg, seed, H_override=H)
        want = _brute_force(H, np.zeros(n, bool), 0.1, mode)
        assert set(np.nonzero(rec.selected)[0].tolist()) == want
        tau = S.temperature(t, cfg)
        for i in range(n):
            if rec.selected[i]:
                u = S.draw_uniform(seed, i, t, 0)
                assert st.tokens[i] == S.draw_token(L[i], tau, mask, u)
            elif not rec.finished:
                assert st.tokens[i] == mask
        if not rec.finished:
            assert np.array_equal(st.committed, rec.selected)
        checked += 1
    assert checked > 250


def test_reselect_all_takes_back_a_commit_that_keep_retains():
    n, V = 8, 12
    first = np.zeros(n, bool)
    first[0] = True
    second = np.zeros(n, bool)
    second[5] = True
    runs = {}
    for mode in ("keep", "reselect_all"):
        cfg = S.SamplerConfig(mask_id=V - 1, commit_mode=mode)
        st = S.CanvasState.fresh(n, V - 1)
        r0 = S.sampler_step(st, _one_hot_or_flat(n, V, first), 0, cfg, 9)
        assert np.array_equal(r0.selected, first) and st.tokens[0] == 0
        r1 = S.sampler_step(st, _one_hot_or_flat(n, V, second), 1, cfg, 9)
        assert np.array_equal(r1.selected, second) and st.tokens[5] == 5
        runs[mode] = st
    assert runs["keep"].committed[0] and runs["keep"].tokens[0] == 0
    assert not runs["reselect_all"].committed[0] and runs["reselect_all"].tokens[0] == V - 1
    assert runs["reselect_all"].committed.sum() == 1


def test_reselect_all_can_select_a_committed_position_again():
    """A committed row that stays confident is selected again and redrawn
    (one-hot rows redraw the same token); a committed row that is not yet
    confident competes with the rest on entropy."""
    n, V = 6, 10
    cfg = S.SamplerConfig(mask_id=V - 1, commit_mode="reselect_all")
    st = S.CanvasState.fresh(n, V - 1)
    conf = np.array([1, 0, 0, 0, 0, 0], bool)
    S.sampler_step(st, _one_hot_or_flat(n, V, conf), 0, cfg, 3)
    conf2 = np.array([1, 0, 1, 0, 0, 0], bool)
    rec = S.sampler_step(st, _one_hot_or_flat(n, V, conf2), 1, cfg, 3)
    assert np.array_equal(rec.selected, conf2)
    assert st.tokens[0] == 0 and st.tokens[2] == 2
    assert np.array_equal(st.committed, conf2)


def test_reselect_all_finishes_only_when_one_step_selects_everything():
    n, V = 16, 9
    cfg = S.SamplerConfig(mask_id=V - 1, commit_mode="reselect_all")
    st = S.CanvasState.fresh(n, V - 1)
    half = np.arange(n) < n // 2
    for t in range(3):       # the same half is confident: never all selected
        rec = S.sampler_step(st, _one_hot_or_flat(n, V, half), t, cfg, 1)
        assert not rec.finished and st.committed.sum() == n // 2
    rec = S.sampler_step(st, _one_hot_or_flat(n, V, np.ones(n, bool)), 3, cfg, 1)
    assert rec.finished and not rec.stop and st.committed.all()
    assert np.array_equal(st.tokens, np.arange(n) % (V - 1))


def test_first_step_is_the_same_in_both_commit_modes():
    rng = np.random.default_rng(5)
    n, V = 40, 64
    L = rng.normal(size=(n, V)) * rng.uniform(1, 40, size=(n, 1))
    out = []
    for mode in ("keep", "reselect_all"):
        st = S.CanvasState.fresh(n, V - 1)
        rec = S.sampler_step(st, L, 0, S.SamplerConfig(mask_id=V - 1, commit_mode=mode), 8)
        out.append((rec.selected.copy(), st.tokens.copy(), st.committed.copy()))
    for a, b in zip(out[0], out[1]):
        assert np.array_equal(a, b)


def test_unknown_commit_mode_is_rejected():
    with pytest.raises(ValueError):
        S.sampler_step(S.CanvasState.fresh(4, 3), np.zeros((4, 4)), 0,
                       S.SamplerConfig(mask_id=3, commit_mode="nope"), 1)


# ------------------------------------------------------------- Gumbel-max ---

def test_vector_philox_equals_the_scalar_engine():
    rng = np.random.default_rng(17)
    ctr = rng.integers(0, 2 ** 32, size=(4, 300), dtype=np.uint64)
    key = (int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 32)))
    got = S.philox4x32_10_many(*ctr, key)
    for j in range(300):
        want = S.philox4x32_10([int(c[j]) for c in ctr], key)
        assert tuple(int(w[j]) for w in got) == want


def test_gumbel_draw_by_brute_force():
    """Token = lowest argmax of z_v - log(-log u_v), u_v from the scalar
    engine at counter (pos, step, canvas, 1 + v // 4), word v % 4."""
    rng = np.random.default_rng(18)
    seed = 0x1234_5678_9ABC_DEF0
    for trial in range(20):
        V = int(rng.integers(2, 40))
        L = rng.normal(size=V) * 2
        mask = int(rng.integers(0, V))
        tau, pos, step, cv = 0.7, int(rng.integers(0, 256)), int(rng.integers(0, 48)), trial
        best, tok = -math.inf, -1
        for v in range(V):
            if v == mask:
                continue
            w = S.philox4x32_10((pos, step, cv, 1 + v // 4), (seed & 0xFFFFFFFF, seed >> 32))[v % 4]
            u = ((w >> 9) + 0.5) * 2.0 ** -23
            val = L[v] / tau - math.log(-math.log(u))
            if val > best:
                best, tok = val, v
        assert S.draw_token_gumbel(L, tau, mask, seed, pos, step, cv) == tok


def test_gumbel_draw_special_rows():
    L = np.full(64, -np.inf)
    L[9] = 3.0
    for pos in range(20):
        assert S.draw_token_gumbel(L, 0.4, 63, 5, pos, 0, 0) == 9       # one finite logit
    L = np.zeros(8)
    L[7] = 100.0                                                          # MASK largest
    toks = {S.draw_token_gumbel(L, 0.8, 7, 5, pos, 1, 0) for pos in range(200)}
    assert 7 not in toks and len(toks) > 3
    u = S.gumbel_uniforms(3, 0, 0, 0, 4096)
    assert u.min() > 0 and u.max() < 1


def test_gumbel_draw_frequencies_follow_softmax():
    rng = np.random.default_rng(19)
    V = 10
    L = rng.normal(size=V) * 1.5
    tau = 0.8
    p = scipy.special.softmax(np.where(np.arange(V) == V - 1, -np.inf, L / tau))
    n = 20000
    counts = np.zeros(V)
    for i in range(n):
        counts[S.draw_token_gumbel(L, tau, V - 1, 99, i % 256, (i // 256) % 48, i // (256 * 48))] += 1
    assert counts[V - 1] == 0
    expected = n * p[:V - 1]
    chi2 = ((counts[:V - 1] - expected) ** 2 / expected).sum()
    assert chi2 < scipy.stats.chi2.ppf(0.999, V - 2)


def test_sampler_step_in_gumbel_mode_draws_the_gumbel_token():
    rng = np.random.default_rng(20)
    n, V = 24, 300
    cfg = S.SamplerConfig(mask_id=V - 1, draw_mode="gumbel_max")
    st = S.CanvasState.fresh(n, V - 1, canvas_idx=2)
    L = rng.normal(size=(n, V)) * rng.uniform(1, 40, size=(n, 1))
    rec = S.sampler_step(st, L, 3, cfg, 77, )
    tau = S.temperature(3, cfg)
    for i in np.nonzero(rec.selected)[0]:
        assert st.tokens[i] == S.draw_token_gumbel(L[i], tau, V - 1, 77, int(i), 3, 2)
    with pytest.raises(ValueError):
        S.sampler_step(S.CanvasState.fresh(n, V - 1), L, 0, S.SamplerConfig(mask_id=V - 1, draw_mode="x"), 1)
