"""Pins of the transformer oracle: closed forms, reductions to textbook
special cases, invariances and the encoder prefill/append invariant. CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import model as M
from synth import workloads as wl


# -------------------------------------------------------------------- fp8 ---

def test_e4m3_known_codes():
    assert fp8.e4m3_value(0x00) == 0.0
    assert fp8.e4m3_value(0x38) == 1.0            # exponent field 7 = bias
    assert fp8.e4m3_value(0xB8) == -1.0
    assert fp8.e4m3_value(0x7E) == 448.0          # largest finite
    assert math.isnan(fp8.e4m3_value(0x7F))
    assert fp8.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert fp8.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert fp8.e4m3_value(0x07) == 7 / 8 * 2.0 ** -6
    assert fp8.e4m3_value(0x3C) == 1.5


def test_e4m3_table_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = fp8.decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


# ---------------------------------------------------------------- rmsnorm ---

def test_rmsnorm_closed_form():
    x = np.array([[3.0, -4.0]])                  # mean square 12.5
    y = M.rmsnorm(x, np.array([1.0, 2.0]), 0.0)
    assert np.allclose(y, [[3 / math.sqrt(12.5), -8 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    c = np.full((1, 7), -2.5)
    assert np.allclose(M.rmsnorm(c, np.ones(7), 0.0), -1.0)
    z = np.zeros((1, 4))
    assert np.array_equal(M.rmsnorm(z, np.ones(4), 1e-6), z)


# ------------------------------------------------------------------- rope ---

def test_rope_position_zero_is_identity_and_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 3, 64))
    assert np.allclose(M.rope(x, np.zeros(5), 10000.0), x, atol=0)
    y = M.rope(x, np.arange(5) * 1000, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)


def test_rope_two_dims_is_a_plane_rotation():
    x = np.array([[[1.0, 0.0]]])
    for p in (0.0, 1.0, 2.5, 100.0):
        y = M.rope(x, np.array([p]), 10000.0)[0, 0]     # hd = 2 -> inv_freq = 1
        assert np.allclose(y, [math.cos(p), math.sin(p)], atol=1e-15)


def test_rope_score_depends_only_on_relative_position():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(1, 1, 128))
    k = rng.normal(size=(1, 1, 128))
    def score(pq, pk):
        return float((M.rope(q, np.array([pq]), 10000.0) * M.rope(k, np.array([pk]), 10000.0)).sum())
    s0 = score(10, 3)
    for shift in (1, 77, 5000):
        assert abs(score(10 + shift, 3 + shift) - s0) < 1e-10
    assert abs(score(11, 3) - s0) > 1e-6


# -------------------------------------------------------------- attention ---

def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(6, 4, 16))
    k = rng.normal(size=(1, 2, 16))
    v = rng.normal(size=(1, 2, 16))
    o = M.attend(q, k, v)
    for h in range(4):
        assert np.allclose(o[:, h, :], v[0, h // 2, :], atol=1e-15)


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(3, 2, 8))
    k = np.repeat(rng.normal(size=(1, 2, 8)), 5, axis=0)
    v = rng.normal(size=(5, 2, 8))
    o = M.attend(q, k, v)
    assert np.allclose(o, v.mean(axis=0)[None], atol=1e-14)


def test_attention_peaked_score_selects_a_value_and_grouping():
    hd = 16
    k = np.zeros((3, 2, hd))
    v = np.zeros((3, 2, hd))
    for j in range(3):
        k[j, :, j] = 1.0
        v[j, 0, :] = j + 1.0
        v[j, 1, :] = -(j + 1.0)
    q = np.zeros((1, 4, hd))
    q[0, 0, 2] = 400.0       # head 0 (KV group 0) looks at key 2
    q[0, 3, 0] = 400.0       # head 3 (KV group 1) looks at key 0
    o = M.attend(q, k, v)
    assert np.allclose(o[0, 0], 3.0) and np.allclose(o[0, 3], -1.0)
    assert np.allclose(o[0, 1], 2.0) and np.allclose(o[0, 2], -2.0)   # q = 0 -> mean


def test_attention_mask_hides_keys():
    rng = np.random.default_rng(4)
    q = rng.normal(size=(2, 2, 8))
    k = rng.normal(size=(4, 2, 8))
    v = rng.normal(size=(4, 2, 8))
    vis = np.array([[True, True, False, False], [True, True, True, True]])
    o = M.attend(q, k, v, vis)
    o2 = M.attend(q[:1], k[:2], v[:2])
    assert np.allclose(o[0], o2[0], atol=1e-15)


# -------------------------------------------------------------------- MoE ---

def _tiny_layer(E, k, d=16, F=24, seed=0):
    rng = np.random.default_rng(seed)
    return {
        "router": rng.normal(size=(E, d)) * 0.3,
        "router_bias": np.zeros(E),
        "w_gate": rng.normal(size=(E + 1, F, d)) * 0.2,
        "w_up": rng.normal(size=(E + 1, F, d)) * 0.2,
        "w_down": rng.normal(size=(E + 1, d, F)) * 0.2,
    }


def test_silu_and_swiglu_closed_forms():
    assert M.silu(np.array([0.0]))[0] == 0.0
    assert abs(M.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-16
    x = np.array([[2.0]])
    y = M.swiglu(x, np.array([[1.0]]), np.array([[3.0]]), np.array([[0.5]]))
    assert abs(y[0, 0] - (2 / (1 + math.exp(-2))) * 6 * 0.5) < 1e-14


def test_moe_all_experts_is_dense_softmax_mixture():
    E, d = 4, 16
    W = _tiny_layer(E, E)
    b = np.random.default_rng(5).normal(size=(7, d))
    y, ids, gates, r = M.moe(b, W, E)
    p = np.exp(r - r.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = M.swiglu(b, W["w_gate"][E], W["w_up"][E], W["w_down"][E])
    for e in range(E):
        want = want + p[:, e:e + 1] * M.swiglu(b, W["w_gate"][e], W["w_up"][e], W["w_down"][e])
    assert np.allclose(y, want, atol=1e-13)


def test_moe_single_expert_is_plain_ffn_plus_shared():
    W = _tiny_layer(1, 1)
    b = np.random.default_rng(6).normal(size=(5, 16))
    y, ids, gates, _ = M.moe(b, W, 1)
    assert np.all(ids == 0) and np.allclose(gates, 1.0)
    want = sum(M.swiglu(b, W["w_gate"][e], W["w_up"][e], W["w_down"][e]) for e in (0, 1))
    assert np.allclose(y, want, atol=1e-14)


def test_moe_topk_order_ties_and_permutation():
    E = 8
    W = _tiny_layer(E, 2)
    W["router"] = np.zeros((E, 16))
    W["router_bias"] = np.array([0.0, 1.0, 1.0, 0.5, 1.0, 0.0, 0.0, 0.0])
    b = np.random.default_rng(7).normal(size=(3, 16))
    _, ids, gates, _ = M.moe(b, W, 2)
    assert ids.tolist() == [[1, 2]] * 3                 # equal logits -> lower id
    assert np.allclose(gates, 0.5)
    W = _tiny_layer(E, 2, seed=8)
    b = np.random.default_rng(9).normal(size=(10, 16))
    perm = np.random.default_rng(10).permutation(10)
    y, ids, _, r = M.moe(b, W, 2)
    yp, idsp, _, _ = M.moe(b[perm], W, 2)
    assert np.allclose(yp, y[perm], atol=1e-14) and np.array_equal(idsp, ids[perm])
    assert np.array_equal(ids, np.argsort(-r, axis=1, kind="stable")[:, :2])


# ------------------------------------------------- decoder / encoder stack ---

def _tiny_model(cfg):
    def layer_fn(l):
        return wl.layer_weights(cfg, l)
    return M.Weights(cfg, wl.embedding(cfg), wl.final_norm(cfg), layer_fn)


SMALL = wl.TINY.replace(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                        n_experts=4, top_k=2, ffn_hidden=32, vocab=128, canvas=8, window=6)


def test_encoder_prefill_then_append_equals_one_prefill():
    W = _tiny_model(SMALL)
    toks = wl.prefix_tokens(SMALL, 20).numpy()
    kv1 = M.KVCache.empty(SMALL)
    M.encoder_append(W, kv1, toks)
    kv2 = M.KVCache.empty(SMALL)
    M.encoder_append(W, kv2, toks[:13])
    M.encoder_append(W, kv2, toks[13:17])
    M.encoder_append(W, kv2, toks[17:])
    for l in range(SMALL.n_layers):
        assert kv1.K[l].shape == (2, 20, 16)
        assert np.allclose(kv1.K[l], kv2.K[l], rtol=0, atol=1e-12)
        assert np.allclose(kv1.V[l], kv2.V[l], rtol=0, atol=1e-12)


def test_encoder_is_causal_and_windowed():
    W = _tiny_model(SMALL.replace(global_every=0))       # all layers local, window 6
    toks = wl.prefix_tokens(SMALL, 16).numpy()
    kv1 = M.KVCache.empty(W.cfg)
    M.encoder_append(W, kv1, toks)
    t2 = toks.copy()
    t2[8] = (t2[8] + 1) % 127                            # change a later token
    kv2 = M.KVCache.empty(W.cfg)
    M.encoder_append(W, kv2, t2)
    for l in range(2):
        assert np.array_equal(kv1.K[l][:, :8], kv2.K[l][:, :8])
        assert not np.allclose(kv1.K[l][:, 8], kv2.K[l][:, 8])
    # layer 0's keys depend on the token only; layer 1's keys at p depend on
    # the tokens q with p - q < 6
    assert np.array_equal(kv1.K[0][:, 9:], kv2.K[0][:, 9:])
    assert np.array_equal(kv1.K[1][:, 14:], kv2.K[1][:, 14:])        # 14 - 8 >= 6
    assert not np.allclose(kv1.K[1][:, 13], kv2.K[1][:, 13])         # 13 - 8 < 6


@pytest.mark.parametrize("global_every,n_layers", [(0, 3), (2, 4), (3, 4), (1, 2)])
def test_encoder_rows_equal_the_full_prefill(global_every, n_layers):
    """K/V at chosen rows from the dependency-restricted encoder equal the
    full causal prefill's cache at those rows, on every layer: local and
    global layers, rows at the start, inside, across window edges and last."""
    cfg = SMALL.replace(n_layers=n_layers, global_every=global_every, window=5)
    W = _tiny_model(cfg)
    n = 61
    toks = wl.prefix_tokens(cfg, n).numpy()
    kv = M.KVCache.empty(cfg)
    M.encoder_append(W, kv, toks)
    rng = np.random.default_rng(global_every * 10 + n_layers)
    for rows in ([0], [n - 1], [4, 5, 6], sorted(rng.choice(n, 7, replace=False).tolist()),
                 list(range(n))):
        tr = {}
        K, V = M.encoder_kv_rows(W, toks, rows, block=8, trace=tr)
        assert len(K) == n_layers and len(tr["router"]) == n_layers - 1
        for l in range(n_layers):
            assert K[l].shape == (cfg.n_kv_heads, len(rows), cfg.head_dim)
            assert np.allclose(K[l], kv.K[l][:, rows], rtol=0, atol=1e-12), (rows, l)
            assert np.allclose(V[l], kv.V[l][:, rows], rtol=0, atol=1e-12), (rows, l)
    # a prefix of the layers gives the same values for those layers
    K2, _ = M.encoder_kv_rows(W, toks, [30, 60], n_layers=2)
    assert np.allclose(K2[1], kv.K[1][:, [30, 60]], rtol=0, atol=1e-12)


def test_encoder_rows_reject_rows_outside_the_tokens():
    W = _tiny_model(SMALL)
    toks = wl.prefix_tokens(SMALL, 10).numpy()
    for rows in ([], [10], [-1]):
        with pytest.raises(ValueError):
            M.encoder_kv_rows(W, toks, rows)


def test_decoder_is_bidirectional_and_local_window_hides_old_prefix():
    cfg = SMALL.replace(global_every=0)
    W = _tiny_model(cfg)
    kv = M.KVCache.empty(cfg)
    M.encoder_append(W, kv, wl.prefix_tokens(cfg, 12).numpy())
    canvas = np.full(cfg.canvas, cfg.mask_id)
    canvas[5] = 17
    L1 = M.canvas_logits(W, canvas, kv)
    c2 = canvas.copy()
    c2[7] = 33
    L2 = M.canvas_logits(W, c2, kv)
    assert not np.allclose(L1[0], L2[0])                  # an earlier position sees a later one
    # perturb a prefix row older than the window: local layers cannot see it
    kv2 = kv.copy()
    for l in range(cfg.n_layers):
        kv2.K[l][:, 0] += 5.0
        kv2.V[l][:, 0] -= 5.0
    assert np.array_equal(M.canvas_logits(W, canvas, kv2), L1)
    # ... but a global layer can
    Wg = _tiny_model(SMALL.replace(global_every=1))
    assert not np.allclose(M.canvas_logits(Wg, canvas, kv2), M.canvas_logits(Wg, canvas, kv))


def test_window_covering_the_prefix_makes_local_equal_global():
    cfg_l = SMALL.replace(window=1024, global_every=0)
    cfg_g = SMALL.replace(window=1024, global_every=1)
    Wl, Wg = _tiny_model(cfg_l), _tiny_model(cfg_g)
    kv = M.KVCache.empty(cfg_l)
    M.encoder_append(Wl, kv, wl.prefix_tokens(cfg_l, 12).numpy())
    kvg = M.KVCache.empty(cfg_g)
    M.encoder_append(Wg, kvg, wl.prefix_tokens(cfg_g, 12).numpy())
    canvas = np.full(8, cfg_l.mask_id)
    assert np.allclose(M.canvas_logits(Wl, canvas, kv), M.canvas_logits(Wg, canvas, kvg), atol=1e-12)


def test_decoder_attention_is_one_joint_softmax():
    """With every projection the identity-like map and no MoE, a canvas query
    attends over [prefix || canvas] jointly: check against a direct build."""
    cfg = SMALL.replace(n_layers=1, global_every=1)
    W = _tiny_model(cfg)
    kv = M.KVCache.empty(cfg)
    M.encoder_append(W, kv, wl.prefix_tokens(cfg, 5).numpy())
    canvas = np.arange(8) + 3
    tr = {}
    Wl = W.layer(0)
    X = W.E[canvas]
    M.decoder_layer(X, Wl, kv.K[0], kv.V[0], 0, cfg, trace=tr)
    q, k, v = tr["q"], tr["k"], tr["v"]
    for h in range(cfg.n_q_heads):
        g = h // 2
        keys = np.concatenate([kv.K[0][g], k[:, g]], 0)
        vals = np.concatenate([kv.V[0][g], v[:, g]], 0)
        s = q[:, h] @ keys.T / 4.0
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.allclose(tr["attn"][:, h], p @ vals, atol=1e-13)


# ------------------------------------------------------ e4m3 LM head -------

def test_e4m3_lm_head_logits_by_brute_force():
    """The LM head on an e4m3 copy of the tied matrix: each logit is the sum
    over d of the normalised activation times the code's value (the scalar
    e4m3 decoder) times its vocabulary row's scale; the embedding lookup is
    untouched."""
    from oracle import fp8
    cfg = SMALL.replace(vocab=24, d_model=32)
    codes, scale = wl.lm_head_e4m3(cfg)
    W8 = M.Weights(cfg, wl.embedding(cfg), wl.final_norm(cfg), lambda l: wl.layer_weights(cfg, l),
                   lm_head=(codes, scale))
    Wb = _tiny_model(cfg)
    assert np.array_equal(W8.E, Wb.E)
    rng = np.random.default_rng(4)
    X = rng.normal(size=(3, cfg.d_model))
    L8 = M.lm_logits(X, W8.final_norm, W8.LM, cfg.norm_eps)
    a = M.rmsnorm(X, W8.final_norm, cfg.norm_eps)
    c = codes.numpy()
    s = scale.float().numpy()
    for i in range(3):
        for v in range(cfg.vocab):
            want = sum(a[i, k] * fp8.e4m3_value(int(c[v, k])) for k in range(cfg.d_model)) * float(s[v])
            assert abs(L8[i, v] - want) <= 1e-12 * max(1.0, abs(want))
    # close to, but not the same as, the bf16 head
    Lb = M.lm_logits(X, Wb.final_norm, Wb.LM, cfg.norm_eps)
    r = np.linalg.norm(L8 - Lb) / np.linalg.norm(Lb)
    assert 1e-4 < r < 0.1, r


def test_canvas_logits_read_the_e4m3_head():
    cfg = SMALL
    codes, scale = wl.lm_head_e4m3(cfg)
    W8 = M.Weights(cfg, wl.embedding(cfg), wl.final_norm(cfg), lambda l: wl.layer_weights(cfg, l),
                   lm_head=(codes, scale))
    Wb = _tiny_model(cfg)
    kv = M.KVCache.empty(cfg)
    M.encoder_append(Wb, kv, wl.prefix_tokens(cfg, 10).numpy())
    toks = np.full(cfg.canvas, cfg.mask_id)
    L8 = M.canvas_logits(W8, toks, kv)
    Lb = M.canvas_logits(Wb, toks, kv)
    assert not np.allclose(L8, Lb)
    X = W8.E[toks].copy()
    for l in range(cfg.n_layers):
        X = M.decoder_layer(X, W8.layer(l), kv.K[l], kv.V[l], l, cfg)
    assert np.allclose(L8, M.lm_logits(X, W8.final_norm, W8.LM, cfg.norm_eps), rtol=0, atol=1e-12)
