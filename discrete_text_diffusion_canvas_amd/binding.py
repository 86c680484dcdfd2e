"""ctypes binding of libdg.so (include/dg.h). Argument marshalling only.

Every step of the denoising path runs in the library's HIP kernels; this
module only turns torch tensors into device pointers and structs. PyTorch is
used for device memory and streams. If the library has not been built the
import of the binding fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK = 0
DG_F32, DG_BF16, DG_FP8_E4M3 = 0, 1, 2
DG_BOUND_SUM, DG_BOUND_SUM_MINUS_MAX = 0, 1
DG_COMMIT_KEEP, DG_COMMIT_RESELECT_ALL = 0, 1
DG_DRAW_INVERSE_CDF, DG_DRAW_GUMBEL_MAX = 0, 1
STATE_WORDS = 8
ST_DONE, ST_STEP, ST_COMMITTED, ST_STABLE, ST_SELECTED, ST_STOP, ST_FINISHED = range(7)


class DgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dg error {code}: {msg}")
        self.code = code


class SamplerCfg(C.Structure):
    _fields_ = [("max_steps", C.c_int32), ("temp_start", C.c_float), ("temp_end", C.c_float),
                ("bound", C.c_float), ("stop_entropy", C.c_float), ("stable_steps", C.c_int32),
                ("bound_mode", C.c_int32), ("commit_mode", C.c_int32), ("draw_mode", C.c_int32)]


class CanvasStruct(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("committed", C.c_void_p), ("prev_argmax", C.c_void_p),
                ("state", C.c_void_p), ("bias_tok", C.c_void_p), ("bias_val", C.c_void_p),
                ("n", C.c_int32), ("canvas_idx", C.c_int32)]


class StepStatsStruct(C.Structure):
    _fields_ = [("entropy", C.c_void_p), ("lse", C.c_void_p), ("argmax", C.c_void_p),
                ("selected", C.c_void_p), ("mean_entropy", C.c_void_p), ("logits", C.c_void_p),
                ("logits_ld", C.c_int64), ("experts_hit", C.c_void_p)]


class ConfigStruct(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "ffn_hidden", "vocab", "mask_id", "max_canvas", "window", "global_every", "weight_dtype",
        "act_dtype")] + [("rope_base", C.c_float), ("norm_eps", C.c_float)]


class LayerStruct(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "attn_norm", "moe_norm", "wqkv", "wo", "router", "router_bias", "w_gate", "w_up", "w_down",
        "wqkv_scale", "wo_scale", "gate_scale", "up_scale", "down_scale")]


class WeightsStruct(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("layers", C.POINTER(LayerStruct)),
                ("lm_head_e4m3", C.c_void_p), ("lm_head_scale", C.c_void_p)]


class KVStruct(C.Structure):
    _fields_ = [("k", C.POINTER(C.c_void_p)), ("v", C.POINTER(C.c_void_p)), ("capacity", C.c_int64),
                ("len", C.c_int64)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no CPU fallback)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, u64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_size_t
    lib.dg_version.restype = C.c_char_p
    lib.dg_last_error.restype = C.c_char_p
    lib.dg_sampler_default.restype = SamplerCfg
    lib.dg_canvas_reset.argtypes = [C.POINTER(CanvasStruct), i32, vp]
    lib.dg_sampler_workspace_bytes.argtypes = [i32, i32]
    lib.dg_sampler_workspace_bytes.restype = sz
    lib.dg_sampler_step.argtypes = [C.POINTER(SamplerCfg), vp, i32, i32, i32, i64, i32,
                                    C.POINTER(CanvasStruct), i32, u64, C.POINTER(StepStatsStruct),
                                    vp, sz, vp]
    lib.dg_sampler_step_noalloc.argtypes = [C.POINTER(SamplerCfg), vp, i32, i32, i32, i64, i32,
                                            C.POINTER(CanvasStruct), i32, u64, C.POINTER(StepStatsStruct), vp]
    lib.dg_sampler_static_scratch_bytes.argtypes = []
    lib.dg_sampler_static_scratch_bytes.restype = sz
    P = C.POINTER
    lib.dg_model_create.argtypes = [P(ConfigStruct), P(WeightsStruct), P(C.c_void_p)]
    lib.dg_model_destroy.argtypes = [vp]
    lib.dg_model_destroy.restype = None
    lib.dg_workspace_bytes.argtypes = [vp, i32]
    lib.dg_workspace_bytes.restype = sz
    lib.dg_prefill_append.argtypes = [vp, P(KVStruct), vp, i32, vp, sz, vp]
    lib.dg_canvas_step.argtypes = [vp, P(CanvasStruct), P(KVStruct), i32, u64, P(SamplerCfg),
                                   P(StepStatsStruct), vp, sz, vp]
    lib.dg_generate_canvas.argtypes = [vp, P(CanvasStruct), P(KVStruct), P(SamplerCfg), u64, i32, i32,
                                       P(StepStatsStruct), P(C.c_int32), vp, sz, vp]
    lib.dg_canvas_step_batch.argtypes = [vp, P(CanvasStruct), P(KVStruct), i32, i32, u64, P(SamplerCfg),
                                         P(StepStatsStruct), vp, sz, vp]
    lib.dg_generate_batch.argtypes = [vp, P(CanvasStruct), P(KVStruct), i32, P(SamplerCfg), u64, i32, i32,
                                      P(StepStatsStruct), P(C.c_int32), vp, sz, vp]
    lib.dg_embed.argtypes = [vp, vp, i32, vp, vp]
    lib.dg_decoder_layer.argtypes = [vp, i32, vp, i32, P(KVStruct), vp, vp, vp, sz, vp]
    lib.dg_lm_head.argtypes = [vp, vp, i32, P(SamplerCfg), i32, vp, vp, P(StepStatsStruct), vp, sz, vp]
    lib.dg_step_graph_create.argtypes = [vp, P(CanvasStruct), P(KVStruct), P(SamplerCfg), u64, P(StepStatsStruct),
                                         vp, sz, P(C.c_void_p)]
    lib.dg_step_graph_launch.argtypes = [vp, vp]
    lib.dg_step_graph_destroy.argtypes = [vp]
    lib.dg_step_graph_destroy.restype = None
    for name in ("dg_canvas_reset", "dg_sampler_step", "dg_sampler_step_noalloc", "dg_model_create", "dg_prefill_append",
                 "dg_canvas_step", "dg_generate_canvas", "dg_canvas_step_batch", "dg_generate_batch",
                 "dg_embed", "dg_decoder_layer", "dg_lm_head",
                 "dg_step_graph_create", "dg_step_graph_launch"):
        getattr(lib, name).restype = i32
    return lib


lib = _load()


def check(code: int) -> None:
    if code != DG_OK:
        raise DgError(code, lib.dg_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DG_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DG_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def sampler_default() -> SamplerCfg:
    return lib.dg_sampler_default()


class Canvas:
    """Device buffers of one canvas (tokens, committed, prev_argmax, state)."""

    def __init__(self, n: int, mask_id: int, canvas_idx: int = 0, device="cuda",
                 bias_tok=None, bias_val=None):
        self.n = n
        self.mask_id = mask_id
        self.canvas_idx = canvas_idx
        self.tokens = torch.full((n,), mask_id, dtype=torch.int32, device=device)
        self.committed = torch.zeros(n, dtype=torch.uint8, device=device)
        self.prev_argmax = torch.full((n,), -1, dtype=torch.int32, device=device)
        self.state = torch.zeros(STATE_WORDS, dtype=torch.int32, device=device)
        self.bias_tok = bias_tok
        self.bias_val = bias_val

    def struct(self) -> CanvasStruct:
        return CanvasStruct(_ptr(self.tokens), _ptr(self.committed), _ptr(self.prev_argmax),
                            _ptr(self.state), _ptr(self.bias_tok), _ptr(self.bias_val),
                            self.n, self.canvas_idx)

    def reset(self, stream=None) -> None:
        s = self.struct()
        check(lib.dg_canvas_reset(C.byref(s), self.mask_id, _stream(stream)))


class StepStats:
    """Per-step outputs; ``logits`` ([n][vocab], act dtype) only for model steps;
    ``experts_hit`` ([n_layers] int32, routed experts hit per layer) only when
    ``n_layers`` is given."""

    def __init__(self, n: int, device="cuda", vocab: int = 0, logits_dtype=torch.bfloat16, n_layers: int = 0,
                 n_canvases: int = 1):
        self.entropy = torch.zeros(n, dtype=torch.float32, device=device)
        self.lse = torch.zeros(n, dtype=torch.float32, device=device)
        self.argmax = torch.zeros(n, dtype=torch.int32, device=device)
        self.selected = torch.zeros(n, dtype=torch.uint8, device=device)
        self.mean_entropy = torch.zeros(n_canvases, dtype=torch.float64, device=device)
        self.logits = torch.empty((n, vocab), dtype=logits_dtype, device=device) if vocab else None
        self.experts_hit = torch.zeros(n_layers, dtype=torch.int32, device=device) if n_layers else None

    def struct(self) -> StepStatsStruct:
        ld = self.logits.stride(0) if self.logits is not None else 0
        return StepStatsStruct(_ptr(self.entropy), _ptr(self.lse), _ptr(self.argmax),
                               _ptr(self.selected), _ptr(self.mean_entropy), _ptr(self.logits), ld,
                               _ptr(self.experts_hit))


def sampler_workspace_bytes(n: int, vocab: int) -> int:
    return int(lib.dg_sampler_workspace_bytes(n, vocab))


def sampler_step(scfg: SamplerCfg, logits: torch.Tensor, mask_id: int, canvas: Canvas, step_idx: int,
                 seed: int, stats: StepStats, ws: torch.Tensor, stream=None) -> None:
    n, V = logits.shape
    c = canvas.struct()
    s = stats.struct()
    check(lib.dg_sampler_step(C.byref(scfg), _ptr(logits), dtype_code(logits), n, V, logits.stride(0),
                              mask_id, C.byref(c), step_idx, seed, C.byref(s), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))


def sampler_step_noalloc(scfg: SamplerCfg, logits: torch.Tensor, mask_id: int, canvas: Canvas, step_idx: int,
                         seed: int, stats: StepStats, stream=None) -> None:
    """dg_sampler_step_noalloc: the sampler step on the library's static
    per-GPU scratch (no workspace argument, no device allocation)."""
    n, V = logits.shape
    c = canvas.struct()
    s = stats.struct()
    check(lib.dg_sampler_step_noalloc(C.byref(scfg), _ptr(logits), dtype_code(logits), n, V, logits.stride(0),
                                      mask_id, C.byref(c), step_idx, seed, C.byref(s), _stream(stream)))


def sampler_static_scratch_bytes() -> int:
    return int(lib.dg_sampler_static_scratch_bytes())


lib.dg_timing_enable.argtypes = [C.c_int32]
lib.dg_timing_enable.restype = C.c_int32
lib.dg_timing_read.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int32)]
lib.dg_timing_read.restype = C.c_int32


TIME_OFF, TIME_LM_HEAD, TIME_EXPERT_GATE_UP, TIME_EXPERT_DOWN, TIME_QKV, TIME_ATTENTION, TIME_O_PROJ = range(7)


def timing_enable(target: int) -> None:
    """Record HIP events around every launch of kernel ``target`` (TIME_*)."""
    check(lib.dg_timing_enable(int(target)))


def timing_read():
    """(summed milliseconds, launches) of the timed kernel since enable/read."""
    ms = C.c_double()
    n = C.c_int32()
    check(lib.dg_timing_read(C.byref(ms), C.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------------------
# Model, KV cache, workspace
# ---------------------------------------------------------------------------

_DT = {"f32": DG_F32, "bf16": DG_BF16, "fp8": DG_FP8_E4M3}


class Model:
    """Borrowed device weights plus the library's model handle.

    ``cfg`` is a geometry object with the fields of synth.workloads.ModelConfig;
    ``layers`` a list of dicts of device tensors (names as in dg_layer_weights);
    ``max_canvas`` the most canvas rows of one step (default cfg.canvas; a
    batch needs their sum); ``lm_head_e4m3``/``lm_head_scale`` an optional
    e4m3 copy of the tied matrix (uint8 [vocab][d], bf16 [vocab]) that the
    LM head then reads.
    """

    def __init__(self, cfg, embed, final_norm, layers, max_canvas: int | None = None, lm_head_e4m3=None,
                 lm_head_scale=None):
        self.cfg = cfg
        self.lm_head_e4m3, self.lm_head_scale = lm_head_e4m3, lm_head_scale
        self.embed, self.final_norm, self.layers = embed, final_norm, layers
        self._cs = ConfigStruct(
            n_layers=cfg.n_layers, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
            n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, n_experts=cfg.n_experts,
            top_k=cfg.top_k, ffn_hidden=cfg.ffn_hidden, vocab=cfg.vocab, mask_id=cfg.mask_id,
            max_canvas=max_canvas or cfg.canvas, window=cfg.window, global_every=cfg.global_every,
            weight_dtype=_DT[cfg.weight_dtype], act_dtype=_DT[cfg.act_dtype],
            rope_base=cfg.rope_base, norm_eps=cfg.norm_eps)
        arr = (LayerStruct * cfg.n_layers)()
        for i, L in enumerate(layers):
            for f, _ in LayerStruct._fields_:
                setattr(arr[i], f, _ptr(L.get(f.replace("gate_scale", "w_gate_scale")
                                           .replace("up_scale", "w_up_scale")
                                           .replace("down_scale", "w_down_scale"))))
        self._layers = arr
        self._ws = WeightsStruct(_ptr(embed), _ptr(final_norm), arr, _ptr(lm_head_e4m3), _ptr(lm_head_scale))
        h = C.c_void_p()
        check(lib.dg_model_create(C.byref(self._cs), C.byref(self._ws), C.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and lib is not None:
            lib.dg_model_destroy(h)
            self.handle = None

    @property
    def act_dtype(self):
        return torch.float32 if self.cfg.act_dtype == "f32" else torch.bfloat16

    def workspace(self, max_rows: int, device="cuda") -> torch.Tensor:
        nb = int(lib.dg_workspace_bytes(self.handle, max_rows))
        if nb == 0:
            raise ValueError("bad max_rows")
        return torch.empty(nb, dtype=torch.uint8, device=device)


class KVCache:
    """Per-layer K [Hkv][capacity][hd] and transposed V [Hkv][hd][capacity]
    (activation dtype, zero-filled); capacity is rounded up to a multiple of 64."""

    def __init__(self, model: Model, capacity: int, device="cuda"):
        c = model.cfg
        capacity = (capacity + 63) // 64 * 64
        kshape = (c.n_kv_heads, capacity, c.head_dim)
        vshape = (c.n_kv_heads, c.head_dim, capacity)
        self.k = [torch.zeros(kshape, dtype=model.act_dtype, device=device) for _ in range(c.n_layers)]
        self.v = [torch.zeros(vshape, dtype=model.act_dtype, device=device) for _ in range(c.n_layers)]
        self.capacity = capacity
        self._kp = (C.c_void_p * c.n_layers)(*[t.data_ptr() for t in self.k])
        self._vp = (C.c_void_p * c.n_layers)(*[t.data_ptr() for t in self.v])
        self.struct_ = KVStruct(self._kp, self._vp, capacity, 0)

    @property
    def length(self) -> int:
        return int(self.struct_.len)

    @length.setter
    def length(self, v: int) -> None:
        self.struct_.len = int(v)


def prefill_append(model: Model, kv: KVCache, tokens: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    check(lib.dg_prefill_append(model.handle, C.byref(kv.struct_), _ptr(tokens), tokens.numel(),
                                _ptr(ws), ws.numel(), _stream(stream)))


def canvas_step(model: Model, canvas: Canvas, kv: KVCache, step_idx: int, seed: int, scfg: SamplerCfg,
                stats: StepStats, ws: torch.Tensor, stream=None) -> None:
    c = canvas.struct()
    s = stats.struct()
    check(lib.dg_canvas_step(model.handle, C.byref(c), C.byref(kv.struct_), step_idx, seed, C.byref(scfg),
                             C.byref(s), _ptr(ws), ws.numel(), _stream(stream)))


def _batch_structs(canvases, kvs):
    cs = (CanvasStruct * len(canvases))(*[c.struct() for c in canvases])
    ks = (KVStruct * len(kvs))(*[k.struct_ for k in kvs])
    return cs, ks


def canvas_step_batch(model: Model, canvases, kvs, step_idx: int, seed: int, scfg: SamplerCfg,
                      stats: StepStats, ws: torch.Tensor, stream=None) -> None:
    """One lockstep step of several canvases, each on its own cache; ``stats``
    covers all their rows in order (mean_entropy one entry per canvas)."""
    if len(canvases) != len(kvs):
        raise ValueError("one KV cache per canvas")
    cs, ks = _batch_structs(canvases, kvs)
    s = stats.struct()
    check(lib.dg_canvas_step_batch(model.handle, cs, ks, len(canvases), step_idx, seed, C.byref(scfg),
                                   C.byref(s), _ptr(ws), ws.numel(), _stream(stream)))


def generate_batch(model: Model, canvases, kvs, scfg: SamplerCfg, seed: int, append_after: bool,
                   stats: StepStats, ws: torch.Tensor, poll_every: int = 4, stream=None) -> list:
    if len(canvases) != len(kvs):
        raise ValueError("one KV cache per canvas")
    cs, ks = _batch_structs(canvases, kvs)
    s = stats.struct()
    steps = (C.c_int32 * len(canvases))()
    check(lib.dg_generate_batch(model.handle, cs, ks, len(canvases), C.byref(scfg), seed,
                                int(bool(append_after)), poll_every, C.byref(s), steps, _ptr(ws), ws.numel(),
                                _stream(stream)))
    for kv, k in zip(kvs, ks):      # the appended lengths
        kv.struct_.len = k.len
    return list(steps)


class StepGraph:
    """One dg_canvas_step captured as a HIP graph, the step index read from the
    canvas state; valid until the next prefill_append on ``kv``. Holds the
    buffers it was captured with."""

    def __init__(self, model: Model, canvas: Canvas, kv: KVCache, scfg: SamplerCfg, seed: int, stats: StepStats,
                 ws: torch.Tensor):
        c = canvas.struct()
        s = stats.struct()
        h = C.c_void_p()
        check(lib.dg_step_graph_create(model.handle, C.byref(c), C.byref(kv.struct_), C.byref(scfg), seed,
                                       C.byref(s), _ptr(ws), ws.numel(), C.byref(h)))
        self.handle = h
        self._keep = (model, canvas, kv, stats, ws)

    def launch(self, stream=None) -> None:
        check(lib.dg_step_graph_launch(self.handle, _stream(stream)))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and lib is not None:
            lib.dg_step_graph_destroy(h)
            self.handle = None


def generate_canvas(model: Model, canvas: Canvas, kv: KVCache, scfg: SamplerCfg, seed: int,
                    append_after: bool, stats: StepStats, ws: torch.Tensor, poll_every: int = 4,
                    stream=None) -> int:
    c = canvas.struct()
    s = stats.struct()
    steps = C.c_int32()
    check(lib.dg_generate_canvas(model.handle, C.byref(c), C.byref(kv.struct_), C.byref(scfg), seed,
                                 int(bool(append_after)), poll_every, C.byref(s), C.byref(steps),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return steps.value


def embed(model: Model, tokens: torch.Tensor, X: torch.Tensor, stream=None) -> None:
    check(lib.dg_embed(model.handle, _ptr(tokens), tokens.numel(), _ptr(X), _stream(stream)))


def decoder_layer(model: Model, layer: int, X: torch.Tensor, kv: KVCache, ws: torch.Tensor,
                  route_ids=None, route_gates=None, stream=None) -> None:
    check(lib.dg_decoder_layer(model.handle, layer, _ptr(X), X.shape[0], C.byref(kv.struct_),
                               _ptr(route_ids), _ptr(route_gates), _ptr(ws), ws.numel(), _stream(stream)))


def lm_head(model: Model, X: torch.Tensor, scfg: SamplerCfg, step_idx: int, stats: StepStats,
            ws: torch.Tensor, bias_tok=None, bias_val=None, stream=None) -> None:
    s = stats.struct()
    check(lib.dg_lm_head(model.handle, _ptr(X), X.shape[0], C.byref(scfg), step_idx, _ptr(bias_tok),
                         _ptr(bias_val), C.byref(s), _ptr(ws), ws.numel(), _stream(stream)))
