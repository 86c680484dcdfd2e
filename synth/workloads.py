"""Seeded synthetic workloads: model geometry, random-init weights and inputs.

Nothing here computes any step of the denoising method. The geometries are
the five benchmark workloads (tiny fp32 stack; sampler-only at full
vocabulary; one full-width layer plus LM head; the 30-layer stack; the
long-context fp8 stack). All tensors come from ``synth.hashgen`` and are a
pure function of their stream ids, so they are bit-identical whether they are
made on the CPU (for the oracle) or on the GPU (for the HIP path).

Stream ids: weights (0, layer, tensor); prefix tokens (1, n); per-canvas
logit boosts (2, canvas); sampler-only logits (3, t); router rank
permutation (4, layer); committed-canvas tokens (5, i); synthetic KV rows
(6, layer, kind).
"""
from __future__ import annotations

import dataclasses
import math

import torch

from . import hashgen as hg

WEIGHT_STD = 0.02

# tensor ids inside a layer's weight stream
_T_WQKV, _T_WO, _T_ROUTER, _T_GATE, _T_UP, _T_DOWN = 1, 2, 3, 4, 5, 6
_T_EMBED = 0


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    ffn_hidden: int
    vocab: int
    canvas: int
    window: int = 1024
    global_every: int = 6          # layer l is global iff l % global_every == global_every - 1
    weight_dtype: str = "bf16"     # "f32" | "bf16" | "fp8"
    act_dtype: str = "bf16"        # "f32" | "bf16"
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    zipf_s: float = 0.0            # router bias exponent (0 = no bias)

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def is_global(self, layer: int) -> bool:
        return self.global_every > 0 and layer % self.global_every == self.global_every - 1

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


TINY = ModelConfig(
    name="tiny_fp32", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
    n_experts=8, top_k=2, ffn_hidden=512, vocab=4096, canvas=32,
    weight_dtype="f32", act_dtype="f32", zipf_s=0.0,
)
FULL_LAYER = ModelConfig(
    name="one_layer_bf16", n_layers=1, d_model=2816, n_q_heads=16, n_kv_heads=8, head_dim=256,
    n_experts=128, top_k=8, ffn_hidden=704, vocab=262144, canvas=256,
    weight_dtype="bf16", act_dtype="bf16", zipf_s=1.1,
)
STACK30 = FULL_LAYER.replace(name="stack30_bf16", n_layers=30)
STACK30_FP8 = STACK30.replace(name="stack30_fp8_longctx", weight_dtype="fp8")

TINY_PREFIX = 128
SAMPLER_ONLY_SHAPE = (256, 262144)


def _store_dtype(cfg: ModelConfig):
    return torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16


def _dense(cfg, shape, key, device):
    """A weight in the config's dense dtype (f32 or bf16) ~N(0, 0.02)."""
    dt = torch.float32 if cfg.weight_dtype == "f32" else torch.bfloat16
    return hg.normal(key, shape, WEIGHT_STD, dtype=dt, device=device)


def quantize_e4m3(w: torch.Tensor):
    """OCP e4m3fn bytes with a bf16 scale per output row (the last dim is K).

    scale = bf16(absmax / 448); q = e4m3fn(clamp(w / scale, +-448)), round to
    nearest even. Returns (uint8 codes with w's shape, bf16 scales w.shape[:-1]).
    """
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    scale = (amax / 448.0).to(torch.bfloat16)
    scale = torch.where(scale.float() > 0, scale, torch.ones_like(scale))
    q = (wf / scale.float().unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def layer_weights(cfg: ModelConfig, layer: int, device="cpu") -> dict:
    """One layer's weights. Matrices are [out][in] (in = reduction dim, contiguous).

    Keys: attn_norm, wqkv, wo, moe_norm, router, router_bias, w_gate, w_up,
    w_down; with fp8 also *_scale for wqkv, wo, w_gate, w_up, w_down. Expert
    index n_experts is the shared expert.
    """
    d, E, F = cfg.d_model, cfg.n_experts, cfg.ffn_hidden
    dense = _store_dtype(cfg) if cfg.weight_dtype != "f32" else torch.float32
    L = {
        "attn_norm": torch.ones(d, dtype=torch.float32, device=device),
        "moe_norm": torch.ones(d, dtype=torch.float32, device=device),
    }
    wqkv = _dense(cfg, (cfg.qkv_rows, d), hg.stream_key(0, layer, _T_WQKV), device)
    wo = _dense(cfg, (d, cfg.n_q_heads * cfg.head_dim), hg.stream_key(0, layer, _T_WO), device)
    wg = _dense(cfg, (E + 1, F, d), hg.stream_key(0, layer, _T_GATE), device)
    wu = _dense(cfg, (E + 1, F, d), hg.stream_key(0, layer, _T_UP), device)
    wd = _dense(cfg, (E + 1, d, F), hg.stream_key(0, layer, _T_DOWN), device)
    L["router"] = hg.normal(hg.stream_key(0, layer, _T_ROUTER), (E, d), WEIGHT_STD,
                            dtype=dense, device=device)
    L["router_bias"] = router_bias(cfg, layer).to(device)
    if cfg.weight_dtype == "fp8":
        for name, w in (("wqkv", wqkv), ("wo", wo), ("w_gate", wg), ("w_up", wu), ("w_down", wd)):
            q, s = quantize_e4m3(w)
            L[name] = q
            L[name + "_scale"] = s
            del w
    else:
        L.update(wqkv=wqkv, wo=wo, w_gate=wg, w_up=wu, w_down=wd)
    return L


def embedding(cfg: ModelConfig, device="cpu") -> torch.Tensor:
    """Tied token embedding / LM-head matrix [vocab][d_model]."""
    dt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    return hg.normal(hg.stream_key(0, 1 << 20, _T_EMBED), (cfg.vocab, cfg.d_model),
                     WEIGHT_STD, dtype=dt, device=device)


def lm_head_e4m3(cfg: ModelConfig, device="cpu"):
    """An e4m3 copy of the tied embedding for the LM head: (codes, scales)."""
    return quantize_e4m3(embedding(cfg, device=device))


def final_norm(cfg: ModelConfig, device="cpu") -> torch.Tensor:
    return torch.ones(cfg.d_model, dtype=torch.float32, device=device)


def router_bias(cfg: ModelConfig, layer: int) -> torch.Tensor:
    """Zipf(s) per-expert bias: b_e = -s * ln(rank_e), ranks a seeded permutation.

    softmax(b) is then proportional to rank**-s. fp32, CPU.
    """
    E = cfg.n_experts
    if cfg.zipf_s == 0.0:
        return torch.zeros(E, dtype=torch.float32)
    perm = hg.permutation(hg.stream_key(4, layer), E)
    rank = torch.empty(E, dtype=torch.int64)
    rank[perm] = torch.arange(1, E + 1)
    return torch.tensor([-cfg.zipf_s * math.log(int(r)) for r in rank], dtype=torch.float32)


def prefix_tokens(cfg: ModelConfig, n: int, device="cpu", stream: int = 0) -> torch.Tensor:
    """n prompt tokens uniform over the non-MASK ids (int32)."""
    return hg.randint(hg.stream_key(1, n, stream), n, 0, cfg.vocab - 1, device).to(torch.int32)


def canvas_boost(cfg: ModelConfig, canvas_idx: int, max_boost: float = 12.0, device="cpu"):
    """Per-position one-hot logit boost: (token ids int32 [N], magnitudes f32 [N]).

    Token ids uniform over non-MASK ids, magnitudes U(0, max_boost); drawn
    once per canvas and fixed across its steps.
    """
    N = cfg.canvas
    key = hg.stream_key(2, canvas_idx)
    tok = hg.randint(key, N, 0, cfg.vocab - 1, device, lane=0).to(torch.int32)
    mag = (hg.uniform(key, N, device, lane=1) * max_boost).to(torch.float32)
    return tok, mag


def sampler_logits(t: int, shape=SAMPLER_ONLY_SHAPE, max_peak: float = 16.0,
                   device="cpu", out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 logits N(0,1) plus a per-row peak U(0, max_peak) at a random id.

    The peak id is uniform over [0, vocab-1) (never the last id, which the
    workloads reserve as MASK). Returns a [rows][vocab] bf16 tensor.
    """
    n, V = shape
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    key = hg.stream_key(3, t)
    hg.normal_(out, key, 1.0)
    pk = hg.stream_key(3, t, 1)
    tok = hg.randint(pk, n, 0, V - 1, out.device, lane=0)
    mag = (hg.uniform(pk, n, out.device, lane=1) * max_peak).to(torch.float32)
    rows = torch.arange(n, device=out.device)
    base = out[rows, tok].float()
    out[rows, tok] = (base + mag).to(torch.bfloat16)
    return out


def committed_canvas(cfg: ModelConfig, n_committed: int, device="cpu"):
    """Canvas state with n_committed positions holding uniform non-MASK ids.

    Returns (tokens int32 [N], committed uint8 [N]); the committed positions
    are a seeded random subset, the rest hold MASK.
    """
    N = cfg.canvas
    perm = hg.permutation(hg.stream_key(5, 0), N)
    pos = perm[:n_committed]
    toks = torch.full((N,), cfg.mask_id, dtype=torch.int32)
    ids = hg.randint(hg.stream_key(5, 1), N, 0, cfg.vocab - 1, "cpu").to(torch.int32)
    toks[pos] = ids[pos]
    com = torch.zeros(N, dtype=torch.uint8)
    com[pos] = 1
    return toks.to(device), com.to(device)


def synthetic_kv(cfg: ModelConfig, layer: int, n: int, device="cpu"):
    """Synthetic K and V rows ~N(0,1) in the activation dtype, [Hkv][n][hd]."""
    dt = _store_dtype(cfg)
    shape = (cfg.n_kv_heads, n, cfg.head_dim)
    k = hg.normal(hg.stream_key(6, layer, 0), shape, 1.0, dtype=dt, device=device)
    v = hg.normal(hg.stream_key(6, layer, 1), shape, 1.0, dtype=dt, device=device)
    return k, v
