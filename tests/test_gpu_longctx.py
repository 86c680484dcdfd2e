"""Parity at the long-context, fp8 widths: one decoder layer of d=2816, 16/8
heads of 256, 128 experts (top-8) plus the shared one, F=704, with the expert
and attention-projection weights in OCP e4m3 and bf16 per-row scales, run as a
global layer: the canvas attends a 131072-row prefix KV (synthetic N(0,1)
bf16 rows, seeded per layer) plus its own 256 rows. The float64 oracle runs
the same layer on every canvas row (routing checked with the near-tie rule,
then the layer output and its residual delta per row)."""
import numpy as np
import pytest
import torch

from oracle import model as M
from synth import workloads as wl

from model_fixtures import device_model, device_v, fill_synthetic_kv, oracle_weights, rel_l2, rel_l2_rows, \
    routing_near_tie_ok

pytestmark = pytest.mark.gpu

PREFIX = 131072
CFG = wl.FULL_LAYER.replace(name="one_layer_fp8_longctx", weight_dtype="fp8", global_every=1)


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from discrete_text_diffusion_canvas_amd import binding
    return binding


def test_global_layer_over_a_131072_row_prefix_fp8_weights(B):
    cfg = CFG
    model = device_model(B, cfg)
    n = cfg.canvas
    kv = B.KVCache(model, PREFIX + n)
    fill_synthetic_kv(kv, cfg, PREFIX)
    ws = model.workspace(n)
    toks, _ = wl.committed_canvas(cfg, 128)
    X = torch.empty(n, cfg.d_model, dtype=torch.float32, device="cuda")
    B.embed(model, toks.cuda(), X)
    X0 = X.cpu().numpy().astype(np.float64)
    ids = torch.zeros(n, cfg.top_k, dtype=torch.int32, device="cuda")
    B.decoder_layer(model, 0, X, kv, ws, ids)
    torch.cuda.synchronize()
    Xg = X.cpu().numpy()
    ids_g = ids.cpu().numpy()
    K0 = kv.k[0][:, :PREFIX].float().cpu().numpy().astype(np.float64)
    V0 = device_v(kv, 0, PREFIX).numpy().astype(np.float64)
    del kv
    W = oracle_weights(model)
    tr = {}
    M.decoder_layer(X0, W.layer(0), K0, V0, 0, cfg, trace=tr)
    bad = routing_near_tie_ok(tr["router"], ids_g, tr["ids"], 1e-2)
    assert not bad, bad[:5]
    Xo = M.decoder_layer(X0, W.layer(0), K0, V0, 0, cfg, ids_override=ids_g)
    assert rel_l2_rows(Xg, Xo).max() < 2e-2, rel_l2_rows(Xg, Xo).max()
    assert rel_l2(Xg - X0, Xo - X0) < 3e-2, rel_l2(Xg - X0, Xo - X0)
