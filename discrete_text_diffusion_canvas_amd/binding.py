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
STATE_WORDS = 8
ST_DONE, ST_STEP, ST_COMMITTED, ST_STABLE, ST_SELECTED, ST_STOP, ST_FINISHED = range(7)


class DgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dg error {code}: {msg}")
        self.code = code


class SamplerCfg(C.Structure):
    _fields_ = [("max_steps", C.c_int32), ("temp_start", C.c_float), ("temp_end", C.c_float),
                ("bound", C.c_float), ("stop_entropy", C.c_float), ("stable_steps", C.c_int32),
                ("bound_mode", C.c_int32)]


class CanvasStruct(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("committed", C.c_void_p), ("prev_argmax", C.c_void_p),
                ("state", C.c_void_p), ("bias_tok", C.c_void_p), ("bias_val", C.c_void_p),
                ("n", C.c_int32), ("canvas_idx", C.c_int32)]


class StepStatsStruct(C.Structure):
    _fields_ = [("entropy", C.c_void_p), ("lse", C.c_void_p), ("argmax", C.c_void_p),
                ("selected", C.c_void_p), ("mean_entropy", C.c_void_p)]


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
    for name in ("dg_canvas_reset", "dg_sampler_step"):
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
    def __init__(self, n: int, device="cuda"):
        self.entropy = torch.zeros(n, dtype=torch.float32, device=device)
        self.lse = torch.zeros(n, dtype=torch.float32, device=device)
        self.argmax = torch.zeros(n, dtype=torch.int32, device=device)
        self.selected = torch.zeros(n, dtype=torch.uint8, device=device)
        self.mean_entropy = torch.zeros(1, dtype=torch.float64, device=device)

    def struct(self) -> StepStatsStruct:
        return StepStatsStruct(_ptr(self.entropy), _ptr(self.lse), _ptr(self.argmax),
                               _ptr(self.selected), _ptr(self.mean_entropy))


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


lib.dg_timing_enable.argtypes = [C.c_int32]
lib.dg_timing_enable.restype = C.c_int32
lib.dg_timing_read.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int32)]
lib.dg_timing_read.restype = C.c_int32


def timing_enable(on: int) -> None:
    check(lib.dg_timing_enable(int(on)))


def timing_read():
    """(summed milliseconds, launches) of the dominant kernel since enable/read."""
    ms = C.c_double()
    n = C.c_int32()
    check(lib.dg_timing_read(C.byref(ms), C.byref(n)))
    return ms.value, n.value
