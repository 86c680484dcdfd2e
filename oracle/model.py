"""Oracle for the encoder-decoder MoE transformer around the canvas.
TEST INFRASTRUCTURE ONLY.

What the pages fix ([MC-zh] intro list, "模型總覽" overview and spec table;
[MC-ko] "모델 개요"; [AIT] "기술적 특징"):
* an autoregressive (causal) encoder prefills the prompt into a KV cache;
* a decoder processes the 256-token canvas with bidirectional attention and
  reaches the cached context through cross-attention;
* a fully denoised canvas is run through the encoder and appended to the KV
  cache before the next canvas;
* 30 layers, a 1024-token sliding window, a sparse MoE with 8 of 128 experts
  active plus 1 shared expert, a 262K vocabulary.

Readings taken where the pages are silent (the workload geometry is an input):
* one weight stack serves as encoder (run causally) and decoder (run
  bidirectionally over the canvas);
* decoder attention is one joint softmax per head over [cached prefix rows
  in the layer's window || all canvas rows], with the layer's own projections;
  canvas K/V are not cached while denoising;
* local layers show a canvas query the last ``window`` prefix rows; global
  layers (l % global_every == global_every - 1) show all of them; the encoder
  uses a per-query causal window (key q visible to query p iff q <= p and,
  on a local layer, p - q < window);
* pre-norm RMSNorm (weight given, eps from the config) before attention and
  before the MoE, a final RMSNorm before the tied LM head; attention scale
  1/sqrt(head_dim); no soft-capping;
* rotary position embedding, rotate-half form, inv_freq_j = base**(-2j/hd),
  applied to Q and K; prefix rows sit at positions 0..P-1 and the canvas at
  P..P+N-1; K is cached after rotation;
* router: r = b W_r^T + bias; top-k by value (ties -> lower expert id);
  gates = softmax of the k selected logits; expert FFN is SwiGLU
  (silu(x W_g^T) * (x W_u^T)) W_d^T; the shared expert has gate 1.

Everything is float64 numpy. Weights arrive as torch tensors in their storage
type (f32, bf16, or E4M3 codes with bf16 per-output-row scales) and are
widened here.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import fp8


# ---------------------------------------------------------------------------
# Weight widening.
# ---------------------------------------------------------------------------


def widen(t) -> np.ndarray:
    """torch tensor (f32/bf16/f16) or numpy array -> float64 numpy."""
    if hasattr(t, "detach"):
        return t.detach().to("cpu").float().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def widen_layer(L: dict) -> dict:
    """One layer's weights as float64 arrays; E4M3 matrices are dequantised
    with their per-output-row scales."""
    out = {}
    for name in ("attn_norm", "moe_norm", "router", "router_bias"):
        out[name] = widen(L[name])
    for name in ("wqkv", "wo", "w_gate", "w_up", "w_down"):
        if name + "_scale" in L:
            codes = L[name].detach().to("cpu").numpy()
            out[name] = fp8.dequantize(codes, widen(L[name + "_scale"]))
        else:
            out[name] = widen(L[name])
    return out


# ---------------------------------------------------------------------------
# Building blocks.
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x**2) + eps) * w over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [n][heads][hd] at positions pos [n]."""
    hd = x.shape[-1]
    half = hd // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [n][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible=None) -> np.ndarray:
    """Grouped-query softmax attention.

    q [n][Hq][hd], k/v [m][Hkv][hd]; query head h reads KV head h // (Hq/Hkv).
    visible [n][m] bool (None = all keys). Returns [n][Hq][hd].
    """
    n, Hq, hd = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.empty_like(q)
    for h in range(Hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        s = q[:, h, :] @ kh.T / np.sqrt(hd)
        if visible is not None:
            s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu(x, wg, wu, wd) -> np.ndarray:
    """(silu(x W_g^T) * (x W_u^T)) W_d^T."""
    return (silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def route(b: np.ndarray, W: dict, top_k: int):
    """Router logits, the top-k expert ids (value desc, id asc) and gates."""
    r = b @ W["router"].T + W["router_bias"][None, :]
    ids = np.argsort(-r, axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(r, ids, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = e / e.sum(axis=1, keepdims=True)
    return r, ids, gates


def moe(b: np.ndarray, W: dict, top_k: int, ids_override=None):
    """Shared expert plus the gated sum of the routed experts' SwiGLU outputs.

    ``ids_override`` [n][k] replaces the router's choice (the gates are then
    the softmax of those experts' logits); parity tests use it where another
    implementation's router broke a near-tie the other way.
    """
    E = W["router"].shape[0]
    r, ids, gates = route(b, W, top_k)
    if ids_override is not None:
        ids = np.asarray(ids_override, dtype=np.int64)
        sel = np.take_along_axis(r, ids, axis=1)
        e = np.exp(sel - sel.max(axis=1, keepdims=True))
        gates = e / e.sum(axis=1, keepdims=True)
    y = swiglu(b, W["w_gate"][E], W["w_up"][E], W["w_down"][E])
    for e_id in range(E):
        rows, slot = np.nonzero(ids == e_id)
        if rows.size == 0:
            continue
        ye = swiglu(b[rows], W["w_gate"][e_id], W["w_up"][e_id], W["w_down"][e_id])
        y[rows] += gates[rows, slot][:, None] * ye
    return y, ids, gates, r


def is_global_layer(layer: int, global_every: int) -> bool:
    """5:1 local:global reading: layer l is global iff l % g == g - 1."""
    return global_every > 0 and layer % global_every == global_every - 1


def qkv(a: np.ndarray, W: dict, cfg, pos: np.ndarray):
    """Projections for n rows: Q, K rotated at ``pos``; V unrotated."""
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    y = a @ W["wqkv"].T
    n = a.shape[0]
    q = y[:, : Hq * hd].reshape(n, Hq, hd)
    k = y[:, Hq * hd: (Hq + Hkv) * hd].reshape(n, Hkv, hd)
    v = y[:, (Hq + Hkv) * hd:].reshape(n, Hkv, hd)
    return rope(q, pos, cfg.rope_base), rope(k, pos, cfg.rope_base), v


# ---------------------------------------------------------------------------
# KV cache.
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class KVCache:
    """Per-layer post-RoPE keys and values, [Hkv][len][hd] float64."""
    K: list
    V: list

    @classmethod
    def empty(cls, cfg) -> "KVCache":
        z = np.zeros((cfg.n_kv_heads, 0, cfg.head_dim))
        return cls([z.copy() for _ in range(cfg.n_layers)], [z.copy() for _ in range(cfg.n_layers)])

    @property
    def length(self) -> int:
        return self.K[0].shape[1]

    def copy(self) -> "KVCache":
        return KVCache([k.copy() for k in self.K], [v.copy() for v in self.V])


# ---------------------------------------------------------------------------
# Decoder layer over the canvas (bidirectional + cross into the cache).
# ---------------------------------------------------------------------------


def decoder_layer(X: np.ndarray, W: dict, Kc: np.ndarray, Vc: np.ndarray, layer: int, cfg,
                  ids_override=None, trace: dict | None = None) -> np.ndarray:
    """One decoder layer on canvas rows X [N][d] at positions P..P+N-1.

    Kc/Vc: this layer's cache [Hkv][P][hd]. Keys: cache rows [s, P) with
    s = max(0, P - window) on a local layer and 0 on a global one, then all
    N canvas rows; no mask (bidirectional inside the canvas).
    """
    N = X.shape[0]
    P = Kc.shape[1]
    pos = np.arange(P, P + N)
    a = rmsnorm(X, W["attn_norm"], cfg.norm_eps)
    q, k, v = qkv(a, W, cfg, pos)
    s = 0 if is_global_layer(layer, cfg.global_every) else max(0, P - cfg.window)
    keys = np.concatenate([Kc[:, s:P, :].transpose(1, 0, 2), k], axis=0)
    vals = np.concatenate([Vc[:, s:P, :].transpose(1, 0, 2), v], axis=0)
    o = attend(q, keys, vals)
    X = X + o.reshape(N, -1) @ W["wo"].T
    b = rmsnorm(X, W["moe_norm"], cfg.norm_eps)
    y, ids, gates, r = moe(b, W, cfg.top_k, ids_override)
    if trace is not None:
        trace.update(a=a, q=q, k=k, v=v, attn=o, x_mid=X.copy(), b=b, router=r, ids=ids,
                     gates=gates, moe=y)
    return X + y


def lm_logits(X: np.ndarray, final_norm: np.ndarray, E: np.ndarray, eps: float,
              boost=None) -> np.ndarray:
    """L = rmsnorm(X) E^T over the tied embedding E [V][d]; an optional
    per-row one-hot boost (tok [N], mag [N]) is added before the sampler."""
    L = rmsnorm(X, final_norm, eps) @ E.T
    if boost is not None:
        tok, mag = boost
        L[np.arange(L.shape[0]), np.asarray(tok, dtype=np.int64)] += np.asarray(mag, np.float64)
    return L


class Weights:
    """Float64 view of a model: embedding, final norm and lazily widened layers.

    ``layer_fn(l)`` returns layer l's weights as torch tensors; layers are
    widened on first use and can be dropped with ``release``. ``lm_head``
    (optional): (e4m3 codes [V][d], per-row scales [V]) of an e4m3 copy of the
    tied matrix that the LM head reads instead of the embedding; ``LM`` is the
    matrix the LM head uses.
    """

    def __init__(self, cfg, embed, final_norm, layer_fn, lm_head=None):
        self.cfg = cfg
        self.E = widen(embed)
        if lm_head is None:
            self.LM = self.E
        else:
            codes, scale = lm_head
            codes = codes.detach().to("cpu").numpy() if hasattr(codes, "detach") else np.asarray(codes)
            self.LM = fp8.dequantize(codes, widen(scale))
        self.final_norm = widen(final_norm)
        self._fn = layer_fn
        self._cache: dict[int, dict] = {}

    def layer(self, l: int) -> dict:
        if l not in self._cache:
            self._cache[l] = widen_layer(self._fn(l))
        return self._cache[l]

    def release(self, l: int) -> None:
        self._cache.pop(l, None)


def canvas_logits(W: Weights, tokens, kv: KVCache, boost=None, keep_layers=True) -> np.ndarray:
    """Decoder forward over the canvas, then the LM head: logits [N][V]."""
    cfg = W.cfg
    X = W.E[np.asarray(tokens, dtype=np.int64)].copy()
    for l in range(cfg.n_layers):
        X = decoder_layer(X, W.layer(l), kv.K[l], kv.V[l], l, cfg)
        if not keep_layers:
            W.release(l)
    return lm_logits(X, W.final_norm, W.LM, cfg.norm_eps, boost)


# ---------------------------------------------------------------------------
# Encoder: causal prefill / append.
# ---------------------------------------------------------------------------


def encoder_append(W: Weights, kv: KVCache, tokens, keep_layers=True) -> None:
    """Run n tokens (positions P..P+n-1) through the causal encoder and append
    every layer's rotated K and V to the cache (in place).

    Query p sees cache and new keys q <= p, and on a local layer only those
    with p - q < window. The last layer's attention output and MoE are not
    computed: no cache entry depends on them.
    """
    cfg = W.cfg
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    if n == 0:
        return
    P = kv.length
    pos = np.arange(P, P + n)
    X = W.E[tokens].copy()
    for l in range(cfg.n_layers):
        Wl = W.layer(l)
        a = rmsnorm(X, Wl["attn_norm"], cfg.norm_eps)
        q, k, v = qkv(a, Wl, cfg, pos)
        kv.K[l] = np.concatenate([kv.K[l], k.transpose(1, 0, 2)], axis=1)
        kv.V[l] = np.concatenate([kv.V[l], v.transpose(1, 0, 2)], axis=1)
        if l == cfg.n_layers - 1:
            if not keep_layers:
                W.release(l)
            break
        kpos = np.arange(P + n)
        vis = kpos[None, :] <= pos[:, None]
        if not is_global_layer(l, cfg.global_every):
            vis &= (pos[:, None] - kpos[None, :]) < cfg.window
        keys = kv.K[l].transpose(1, 0, 2)
        vals = kv.V[l].transpose(1, 0, 2)
        o = attend(q, keys, vals, vis)
        X = X + o.reshape(n, -1) @ Wl["wo"].T
        b = rmsnorm(X, Wl["moe_norm"], cfg.norm_eps)
        y, _, _, _ = moe(b, Wl, cfg.top_k)
        X = X + y
        if not keep_layers:
            W.release(l)


def _visible_rows(out: np.ndarray, n: int, layer: int, cfg) -> np.ndarray:
    """Mask over rows 0..n-1 of the keys that queries ``out`` see on ``layer``
    of the causal encoder: every q <= r on a global layer, r - q < window on
    a local one."""
    mask = np.zeros(n, dtype=bool)
    if out.size == 0:
        return mask
    if is_global_layer(layer, cfg.global_every):
        mask[: int(out.max()) + 1] = True
        return mask
    edge = np.zeros(n + 1, dtype=np.int64)
    np.add.at(edge, np.maximum(out - cfg.window + 1, 0), 1)
    np.add.at(edge, out + 1, -1)
    return np.cumsum(edge[:n]) > 0


def encoder_kv_rows(W: Weights, tokens, rows, n_layers: int | None = None, block: int = 256,
                    trace: dict | None = None):
    """Keys and values that ``encoder_append`` of all of ``tokens`` into an
    empty cache writes at cache rows ``rows``, for layers 0 .. n_layers-1,
    computed over only the rows they depend on ([MC-zh] overview: the
    encoder's cache of the prompt; causal, windowed on local layers).

    Row r's input to layer l+1 is its input to layer l plus layer l's
    attention output and MoE at r; the attention at r reads layer l's keys
    and values at the rows r sees, which depend on those rows' inputs to
    layer l. Going from the top layer down gives the rows whose input each
    layer needs; going back up computes them with encoder_append's steps.
    Queries are taken in blocks of ``block`` rows; each query still sees
    exactly its own visible keys. Returns (K, V), lists over layers of
    [Hkv][len(rows)][hd] for the sorted distinct rows. ``trace`` (optional)
    receives "router": per layer below the last, the router logits at the
    sorted rows.
    """
    cfg = W.cfg
    L = cfg.n_layers if n_layers is None else n_layers
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    if rows.size == 0 or rows[0] < 0 or rows[-1] >= n:
        raise ValueError("rows must be non-empty and inside the token range")
    need = [None] * L
    need[L - 1] = rows
    for l in range(L - 2, -1, -1):
        mask = _visible_rows(need[l + 1], n, l, cfg)
        mask[need[l + 1]] = True
        mask[rows] = True
        need[l] = np.nonzero(mask)[0]
    Hq, hd = cfg.n_q_heads, cfg.head_dim
    cur = need[0]
    X = W.E[tokens[cur]].copy()
    K_out, V_out, routers = [], [], []
    for l in range(L):
        Wl = W.layer(l)
        a = rmsnorm(X, Wl["attn_norm"], cfg.norm_eps)
        q, k, v = qkv(a, Wl, cfg, cur)
        at = np.searchsorted(cur, rows)
        K_out.append(k[at].transpose(1, 0, 2).copy())
        V_out.append(v[at].transpose(1, 0, 2).copy())
        if l == L - 1:
            break
        nxt = need[l + 1]
        qi = np.searchsorted(cur, nxt)
        local = not is_global_layer(l, cfg.global_every)
        o = np.empty((nxt.size, Hq, hd))
        for b0 in range(0, nxt.size, block):
            r = nxt[b0: b0 + block]
            lo = int(r.min()) - cfg.window + 1 if local else 0
            kidx = np.nonzero((cur >= lo) & (cur <= int(r.max())))[0]
            kp = cur[kidx]
            vis = kp[None, :] <= r[:, None]
            if local:
                vis &= (r[:, None] - kp[None, :]) < cfg.window
            o[b0: b0 + block] = attend(q[qi[b0: b0 + block]], k[kidx], v[kidx], vis)
        Xn = X[qi] + o.reshape(nxt.size, -1) @ Wl["wo"].T
        b = rmsnorm(Xn, Wl["moe_norm"], cfg.norm_eps)
        y, _, _, rl = moe(b, Wl, cfg.top_k)
        routers.append(rl[np.searchsorted(nxt, rows)])
        X = Xn + y
        cur = nxt
    if trace is not None:
        trace["router"] = routers
    return K_out, V_out
