"""The C ABI library loads, exports every function include/dg.h declares, and
rejects bad arguments on the host before touching the GPU. CPU only."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
LIB = os.path.join(ROOT, "discrete_text_diffusion_canvas_amd", "libdg.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(dg_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdg.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("dg_sampler_step", "dg_last_error", "dg_canvas_reset"):
        assert must in names
    assert len(names) >= 6


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_defaults_are_the_model_cards_values(lib):
    from discrete_text_diffusion_canvas_amd import binding as B
    c = B.sampler_default()
    assert (c.max_steps, c.stable_steps, c.bound_mode, c.commit_mode) == (48, 2, 0, 0)
    assert abs(c.temp_start - 0.8) < 1e-7 and abs(c.temp_end - 0.4) < 1e-7
    assert abs(c.bound - 0.1) < 1e-8 and abs(c.stop_entropy - 0.005) < 1e-9


def test_sampler_step_validates_before_launch(lib):
    from discrete_text_diffusion_canvas_amd import binding as B
    L = B.lib
    cfg = B.sampler_default()
    fake = C.c_void_p(0x1000)            # never dereferenced: validation fails first
    canvas = B.CanvasStruct(0x1000, 0x1000, 0x1000, 0x1000, None, None, 16, 0)
    stats = B.StepStatsStruct(0x1000, 0x1000, 0x1000, 0x1000, None)

    def call(**kw):
        a = dict(cfg=cfg, logits=fake, dtype=B.DG_BF16, n=16, V=64, ld=64, mask=63, canvas=canvas,
                 step=0, stats=stats, ws=fake, wsb=1 << 20)
        a.update(kw)
        return L.dg_sampler_step(C.byref(a["cfg"]), a["logits"], a["dtype"], a["n"], a["V"], a["ld"],
                                 a["mask"], C.byref(a["canvas"]), a["step"], 1, C.byref(a["stats"]),
                                 a["ws"], a["wsb"], None)

    assert call(logits=None) == -1
    assert call(dtype=7) == -5
    assert call(V=60, ld=64) == -2                 # not a multiple of 8
    assert call(ld=32) == -2
    assert call(mask=64) == -1
    assert call(n=17) == -2                        # canvas n mismatch
    assert call(step=48) == -1
    assert call(step=-2) == -1
    assert call(wsb=0) == -3
    bad = B.sampler_default()
    bad.temp_end = 0.0
    assert call(cfg=bad) == -1
    bad = B.sampler_default()
    bad.temp_start = 1e-13       # its tempered excluded-column value would overflow
    assert call(cfg=bad) == -1
    assert b"temperatures" in L.dg_last_error()
    bad = B.sampler_default()
    bad.bound_mode = 9
    assert call(cfg=bad) == -1
    assert b"bound_mode" in L.dg_last_error()
    bad = B.sampler_default()
    bad.commit_mode = 2
    assert call(cfg=bad) == -1
    assert b"commit_mode" in L.dg_last_error()
    half = B.CanvasStruct(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 16, 0)
    assert call(canvas=half) == -1


def test_model_create_rejects_routing_beyond_the_permutation(lib):
    """128 experts top-8 fit a 1024-row canvas; 512 experts top-16 do not
    (the one-workgroup expert permutation's LDS bound). Validation runs on
    the host before any weight is read, so aligned placeholder pointers do."""
    from discrete_text_diffusion_canvas_amd import binding as B
    L = B.lib
    fake = 0x1000
    layer = B.LayerStruct(*([fake] * 9 + [None] * 5))
    arr = (B.LayerStruct * 1)(layer)
    w = B.WeightsStruct(fake, fake, arr)

    def create(E, k, canvas):
        cs = B.ConfigStruct(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, n_experts=E,
                            top_k=k, ffn_hidden=64, vocab=4096, mask_id=4095, max_canvas=canvas, window=128,
                            global_every=0, weight_dtype=B.DG_BF16, act_dtype=B.DG_BF16, rope_base=1e4,
                            norm_eps=1e-6)
        h = C.c_void_p()
        code = L.dg_model_create(C.byref(cs), C.byref(w), C.byref(h))
        if code == 0:
            L.dg_model_destroy(h)
        return code

    assert create(128, 8, 1024) == 0
    assert create(512, 16, 1024) == -5
    assert b"permutation" in L.dg_last_error()
    assert create(512, 16, 64) == 0


def test_batch_step_validates_before_launch(lib):
    """Batch limits are checked on the host before any device work:
    placeholder pointers are never dereferenced."""
    from discrete_text_diffusion_canvas_amd import binding as B
    L = B.lib
    fake = 0x1000
    layer = B.LayerStruct(*([fake] * 9 + [None] * 5))
    arr = (B.LayerStruct * 1)(layer)
    w = B.WeightsStruct(fake, fake, arr)
    cs = B.ConfigStruct(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, n_experts=8,
                        top_k=2, ffn_hidden=64, vocab=4096, mask_id=4095, max_canvas=256, window=128,
                        global_every=0, weight_dtype=B.DG_BF16, act_dtype=B.DG_BF16, rope_base=1e4, norm_eps=1e-6)
    h = C.c_void_p()
    assert L.dg_model_create(C.byref(cs), C.byref(w), C.byref(h)) == 0
    kp = (C.c_void_p * 1)(fake)
    kvs = (B.KVStruct * 3)(*[B.KVStruct(kp, kp, 1024, 0) for _ in range(3)])
    stats = B.StepStatsStruct(fake, fake, fake, fake, fake, fake, 4096, None)
    cfg = B.sampler_default()

    def call(ns, nb=None, step=0):
        cv = (B.CanvasStruct * len(ns))(*[B.CanvasStruct(fake, fake, fake, fake, None, None, n, 0) for n in ns])
        return L.dg_canvas_step_batch(h, cv, kvs, len(ns) if nb is None else nb, step, 1, C.byref(cfg),
                                      C.byref(stats), C.c_void_p(fake), 1 << 40, None)
    try:
        assert call([64, 64], nb=0) == -2
        assert call([64, 96]) == -2                     # not a multiple of 64
        assert b"multiple of 64" in L.dg_last_error()
        assert call([128, 128, 64]) == -2               # 320 rows > max_canvas 256
        assert b"max_canvas" in L.dg_last_error()
        assert call([64, 64], step=48) == -1
    finally:
        L.dg_model_destroy(h)


def test_draw_mode_is_validated(lib):
    from discrete_text_diffusion_canvas_amd import binding as B
    L = B.lib
    assert B.sampler_default().draw_mode == B.DG_DRAW_INVERSE_CDF
    fake = C.c_void_p(0x1000)
    canvas = B.CanvasStruct(0x1000, 0x1000, 0x1000, 0x1000, None, None, 16, 0)
    stats = B.StepStatsStruct(0x1000, 0x1000, 0x1000, 0x1000, None)
    bad = B.sampler_default()
    bad.draw_mode = 3
    code = L.dg_sampler_step(C.byref(bad), fake, B.DG_BF16, 16, 64, 64, 63, C.byref(canvas), 0, 1,
                             C.byref(stats), fake, 1 << 20, None)
    assert code == -1 and b"draw_mode" in L.dg_last_error()
