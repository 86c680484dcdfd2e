"""Parity of the encoder prefill at long context (the model cards' 256K
context; the cache a 131072-token prompt leaves behind), through
dg_prefill_append in 4096-row chunks:

* the 30-layer fp8 stack at full width (d=2816, 16/8 heads of 256, 128
  experts top-8 plus the shared one, F=704, 25 local + 5 global layers)
  prefilled with 131072 and with 262144 tokens; layers 0 and 1 checked row by
  row at sampled rows against the float64 oracle restricted to the rows they
  depend on, every layer's whole cache checked finite;
* a narrow bf16 stack [local, global, local] prefilled with 131072 tokens
  in two calls (130000 + 1072, so both calls end on a ragged chunk and the
  second starts off a chunk boundary); all three layers checked at sampled
  rows, the last one through the global layer's attention over every
  earlier row;
* 5000 tokens of a small bf16 geometry in 4096 + 904-row chunks, every
  cache row against the full oracle prefill.

Rows whose oracle routing is a near tie (k-th and (k+1)-th router logits
within ROUTE_TIE) at a layer below are held only to being finite, since the
two sides may then route them differently."""
import numpy as np
import pytest
import torch

from oracle import model as M
from synth import workloads as wl

from model_fixtures import SMALL_BF16, device_model, device_v, oracle_weights, rel_l2, rel_l2_rows

pytestmark = pytest.mark.gpu

KV_TOL = 3e-2          # per-row relative L2 of K and V against the float64 oracle (bf16 cache)
ROUTE_TIE = 1e-2
CHUNK = 4096

NARROW = wl.FULL_LAYER.replace(
    name="narrow_longctx_bf16", n_layers=3, d_model=256, n_q_heads=2, n_kv_heads=1, head_dim=256,
    n_experts=8, top_k=2, ffn_hidden=128, vocab=4096, canvas=64, window=1024, global_every=2)


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def _sample_rows(n):
    rows = {0, 1, 1023, 1024, 1025, CHUNK - 1, CHUNK, 70001, 131071, n - 1}
    if n > 131072:
        rows |= {131072, 200003}
    return np.array(sorted(r for r in rows if r < n), dtype=np.int64)


def _device_rows(kv, l, rows):
    idx = torch.as_tensor(rows, device=kv.k[l].device)
    k = kv.k[l].index_select(1, idx).float().cpu().numpy()                    # [Hkv][R][hd]
    v = kv.v[l].index_select(2, idx).transpose(1, 2).float().cpu().numpy()   # [Hkv][R][hd]
    return k, v


def _near_tie_rows(router_logits, top_k):
    """Per row: True if the k-th and (k+1)-th largest logits are within ROUTE_TIE."""
    if router_logits.shape[1] <= top_k:
        return np.zeros(router_logits.shape[0], dtype=bool)
    s = -np.sort(-router_logits, axis=1)
    return (s[:, top_k - 1] - s[:, top_k]) < ROUTE_TIE


def _compare(cfg, kv, rows, Ko, Vo, trace, n_layers):
    tie = np.zeros(rows.size, dtype=bool)
    report = []
    for l in range(n_layers):
        if l > 0:
            tie |= _near_tie_rows(trace["router"][l - 1], cfg.top_k)
        kg, vg = _device_rows(kv, l, rows)
        assert np.isfinite(kg).all() and np.isfinite(vg).all(), l
        ek = rel_l2_rows(kg.transpose(1, 0, 2).reshape(rows.size, -1), Ko[l].transpose(1, 0, 2).reshape(rows.size, -1))
        ev = rel_l2_rows(vg.transpose(1, 0, 2).reshape(rows.size, -1), Vo[l].transpose(1, 0, 2).reshape(rows.size, -1))
        report.append((l, float(ek[~tie].max(initial=0)), float(ev[~tie].max(initial=0)), int(tie.sum())))
        assert (ek[~tie] < KV_TOL).all(), (l, rows[~tie][ek[~tie] >= KV_TOL], ek)
        assert (ev[~tie] < KV_TOL).all(), (l, rows[~tie][ev[~tie] >= KV_TOL], ev)
    assert (~tie).sum() >= rows.size // 2, tie
    print("per layer: (layer, max K err, max V err, near-tie rows)", report, flush=True)


@pytest.fixture(scope="module")
def full_fp8(B):
    cfg = wl.STACK30_FP8
    model = device_model(B, cfg)
    cfg2 = cfg.replace(n_layers=2)
    host = {}

    def layer_fn(l):
        if l not in host:
            host[l] = {k: v.cpu() for k, v in model.layers[l].items()}
        return host[l]
    W = M.Weights(cfg2, model.embed.cpu(), model.final_norm.cpu(), layer_fn)
    return cfg, model, W


@pytest.mark.parametrize("n", [131072, 262144])
def test_full_width_fp8_prefill_long_context(B, full_fp8, n):
    cfg, model, W = full_fp8
    toks = wl.prefix_tokens(cfg, n)
    kv = B.KVCache(model, n)
    ws = model.workspace(CHUNK)
    print(f"prefill {n} tokens, full-width fp8 stack", flush=True)
    B.prefill_append(model, kv, toks.cuda(), ws)
    torch.cuda.synchronize()
    assert kv.length == n
    for l in range(cfg.n_layers):
        assert bool(torch.isfinite(kv.k[l][:, :n]).all()), l
        assert bool(torch.isfinite(kv.v[l][:, :, :n]).all()), l
    rows = _sample_rows(n)
    tr = {}
    Ko, Vo = M.encoder_kv_rows(W, toks.numpy(), rows, n_layers=2, trace=tr)
    _compare(cfg, kv, rows, Ko, Vo, tr, 2)
    del kv, ws
    torch.cuda.empty_cache()


def test_narrow_prefill_131072_rows_through_a_global_layer(B):
    cfg = NARROW
    n = 131072
    model = device_model(B, cfg)
    toks = wl.prefix_tokens(cfg, n)
    kv = B.KVCache(model, n)
    ws = model.workspace(CHUNK)
    dt = toks.cuda()
    B.prefill_append(model, kv, dt[:130000], ws)
    B.prefill_append(model, kv, dt[130000:], ws)
    torch.cuda.synchronize()
    assert kv.length == n
    layers = [{k: v.cpu() for k, v in L.items()} for L in model.layers]
    W = M.Weights(cfg, model.embed.cpu(), model.final_norm.cpu(), lambda l: layers[l])
    rows = _sample_rows(n)
    tr = {}
    Ko, Vo = M.encoder_kv_rows(W, toks.numpy(), rows, trace=tr)
    _compare(cfg, kv, rows, Ko, Vo, tr, cfg.n_layers)


def test_large_chunks_match_the_full_oracle_prefill(B):
    """5000 tokens of the small bf16 geometry (16 experts, top-4) in one call:
    chunks of 4096 and 904 rows (the permutation's bound allows 4096 here),
    every cache row of both layers against the oracle's full prefill."""
    cfg = SMALL_BF16
    n = 5000
    model = device_model(B, cfg)
    toks = wl.prefix_tokens(cfg, n)
    kv = B.KVCache(model, n)
    B.prefill_append(model, kv, toks.cuda(), model.workspace(CHUNK))
    torch.cuda.synchronize()
    okv = M.KVCache.empty(cfg)
    M.encoder_append(oracle_weights(model), okv, toks.numpy())
    for l in range(cfg.n_layers):
        kg = kv.k[l][:, :n].float().cpu().numpy()
        vg = device_v(kv, l, n).numpy()
        assert rel_l2(kg, okv.K[l]) < KV_TOL, (l, rel_l2(kg, okv.K[l]))
        assert rel_l2(vg, okv.V[l]) < KV_TOL, (l, rel_l2(vg, okv.V[l]))
