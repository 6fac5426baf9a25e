"""The C-ABI library loads without a GPU, exports every entry point declared in
include/mok.h, and rejects bad host-checkable arguments synchronously."""
import ctypes
import os
import re

import pytest
import torch

import mixture_experts_layer_table_amd as mok

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mok.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mok_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(mok.EXPORTS)
    lib = ctypes.CDLL(mok._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_config_default():
    c = mok.mok_config()
    assert mok.mok_config_default(c) == mok.MOK_OK
    assert (c.minibatch_rows, c.macrobatch_tokens, c.ring_bytes, c.capacity_multiplier, c.precision,
            c.persistent_workgroups) == (512, 0, 256 << 20, 1.0, mok.MOK_BF16, 0)
    assert ctypes.sizeof(mok.mok_config) == 40


BAD_SHAPES = [dict(T=-1), dict(H=100), dict(I=96), dict(E=0), dict(k=0), dict(k=9), dict(T=1 << 31),
              dict(T=1 << 17, H=8192),              # x [T,H] bf16 reaches 2 GiB
              dict(T=1 << 18, I=1024, k=2),         # h [R,2I] bf16 reaches 2 GiB
              dict(H=32768, I=32704),               # one expert's weight gradient [H,I] bf16 near 2 GiB
              dict(E=4097)]                         # past the expert limit


@pytest.mark.parametrize("bad", BAD_SHAPES)
def test_bad_shapes_rejected(bad):
    s = dict(T=64, H=128, I=64, E=8, k=2)
    s.update(bad)
    with pytest.raises(mok.MokError) as e:
        mok.query_sizes(mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 20), **s)
    assert e.value.status == mok.MOK_ERROR_INVALID_VALUE


# the largest shapes under each 2 GiB byte bound stay accepted
EDGE_SHAPES = [dict(T=(1 << 17) - 1, H=8192),         # x [T,H] one row short of 2 GiB
               dict(T=(1 << 18) - 1, I=1024, k=2),    # h [R,2I] one token short of 2 GiB
               dict(H=32768, I=32448),                # (H + 256) * I * 2 just under 2 GiB
               dict(E=4096, k=8)]


@pytest.mark.parametrize("edge", EDGE_SHAPES)
def test_shapes_at_the_bounds_accepted(edge):
    s = dict(T=64, H=128, I=64, E=8, k=2)
    s.update(edge)
    sizes = mok.query_sizes(mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 26), **s)
    assert all(v > 0 for v in sizes)


BAD_CONFIGS = [dict(minibatch_rows=8), dict(minibatch_rows=40), dict(capacity_multiplier=0.0),
               dict(capacity_multiplier=4.5), dict(precision=7), dict(ring_bytes=32 * 256),
               dict(macrobatch_tokens=-1), dict(debug_flags=16), dict(persistent_workgroups=-1),
               dict(persistent_workgroups=65536)]


@pytest.mark.parametrize("bad", BAD_CONFIGS)
def test_bad_configs_rejected(bad):
    c = dict(minibatch_rows=32, ring_bytes=1 << 20)
    c.update(bad)
    with pytest.raises(mok.MokError) as e:
        mok.query_sizes(mok.MoKConfig(**c), 64, 128, 64, 8, 2)
    assert e.value.status == mok.MOK_ERROR_INVALID_VALUE


def test_schedule_layout_matches_oracle_sizes():
    from oracle import schedule as S
    import synth
    for name in ("tiny", "full_layer", "ep64_share", "stream"):
        cfg = synth.CONFIGS[name]
        c = mok.MoKConfig(minibatch_rows=cfg.minibatch_rows, macrobatch_tokens=cfg.macrobatch_tokens,
                          ring_bytes=cfg.ring_bytes)
        lay = mok.schedule_layout(c, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
        assert lay.R == cfg.R
        assert lay.cap == S.capacity(cfg.T, cfg.k, cfg.E, cfg.minibatch_rows, cfg.macrobatch_tokens, 1.0)
        ids, _, _ = synth.make_routing(cfg)
        s = S.build(ids, cfg.E, cfg.minibatch_rows, cfg.macrobatch_tokens)
        assert (lay.NM, lay.G) == (s.NM, s.G)
        ws, sc, cx = mok.query_sizes(c, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
        assert sc == lay.total_bytes and cx >= cfg.R * 2 * cfg.I * 2


def test_canonical_row_copies_follow_k_and_mode():
    """fwd_ctx holds h [R][2I] bf16 and g * a [R][I] bf16 (the down weight
    gradient's operand, written by the forward), plus the x rows in canonical
    order [R][H] bf16 exactly when every routed row is its own token (k = 1)
    and the weight gradients run in BF16; the dy copy lives in the workspace, except when one
    macro-batch fits the ring (the ring then holds the dy rows in canonical
    order). With k > 1 the weight gradients read x and dy through the token
    index, and neither copy exists: a kernel reading a copy the plan did not
    make would read through a null pointer."""
    def align(n):
        return (n + 255) // 256 * 256
    T, H, I, E = 256, 256, 128, 4
    small_ring = 2 * 64 * 2 * H            # two 64-row slots: 4 mini-batches do not fit
    for k, prec, canon in ((1, mok.MOK_BF16, True), (2, mok.MOK_BF16, False), (1, mok.MOK_MXFP8, True),
                           (1, mok.MOK_MXFP8_WGRAD, False), (4, mok.MOK_MXFP8, False)):
        R = T * k
        big = mok.MoKConfig(minibatch_rows=64, ring_bytes=64 << 20, precision=prec)
        small = mok.MoKConfig(minibatch_rows=64, ring_bytes=small_ring, precision=prec)
        ws_big, _, cx = mok.query_sizes(big, T, H, I, E, k)
        ws_small, _, cx_small = mok.query_sizes(small, T, H, I, E, k)
        h_bytes, ga_bytes = align(R * 2 * I * 2), align(R * I * 2)
        assert cx == cx_small == h_bytes + ga_bytes + (align(R * H * 2) if canon else 0), (k, prec)
        if prec == mok.MOK_BF16 and canon:
            # one macro-batch in a ring that holds it: the dy rows stay in the
            # ring; two macro-batches (same ring): a dy copy in the workspace
            two_macro = mok.MoKConfig(minibatch_rows=64, ring_bytes=64 << 20, precision=prec,
                                      macrobatch_tokens=T // 2)
            ws_two, _, _ = mok.query_sizes(two_macro, T, H, I, E, k)
            assert ws_two - ws_big == align(R * H * 2)


def test_ring_slot_count_rule():
    from oracle import schedule as S
    # fewer than two mini-batches in the ring is rejected; exactly two is accepted
    H, MB = 128, 32
    two = 2 * MB * 2 * H
    mok.query_sizes(mok.MoKConfig(minibatch_rows=MB, ring_bytes=two), 64, H, 64, 8, 2)
    assert S.ring_slots(two, MB, 2 * H) == 2
    with pytest.raises(mok.MokError):
        mok.query_sizes(mok.MoKConfig(minibatch_rows=MB, ring_bytes=two - 1), 64, H, 64, 8, 2)


def test_null_and_misaligned_pointers_rejected_without_device_work():
    c = mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 20).c()
    sh = mok.mok_shape(64, 128, 64, 8, 2)
    assert mok.mok_build_schedule(c, sh, None, None, 1 << 20, None) == mok.MOK_ERROR_INVALID_VALUE
    assert mok.mok_build_schedule(c, sh, ctypes.c_void_p(0x1003), ctypes.c_void_p(0x2000), 1 << 20, None) \
        == mok.MOK_ERROR_INVALID_VALUE
    assert mok.mok_build_schedule(c, sh, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 16, None) \
        == mok.MOK_ERROR_BUFFER_TOO_SMALL
    w = mok.mok_weights()
    assert mok.mok_forward(c, sh, None, 0, None, 0, None, None, w, None, None, 0, None) == \
        mok.MOK_ERROR_INVALID_VALUE
    assert mok.mok_mxfp8_quantize(None, 1, 1, 33, 0, None, None, None) == mok.MOK_ERROR_INVALID_VALUE
    assert mok.mok_mxfp8_quantize(None, 1, 1, 32, 2, None, None, None) == mok.MOK_ERROR_INVALID_VALUE


def test_single_hip_runtime_in_process():
    # the binding shares torch's HIP runtime: only one libamdhip64 is mapped
    maps = open(f"/proc/{os.getpid()}/maps").read()
    hip = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_mxfp8_needs_128_multiples():
    # the block-scaled GEMMs load four scale bytes (128 values of K) as one aligned dword
    for H, I in ((128, 64), (192, 128)):
        with pytest.raises(mok.MokError) as e:
            mok.query_sizes(mok.MoKConfig(precision=mok.MOK_MXFP8), 64, H, I, 8, 2)
        assert e.value.status == mok.MOK_ERROR_INVALID_VALUE
    mok.query_sizes(mok.MoKConfig(precision=mok.MOK_MXFP8), 64, 256, 128, 8, 2)


def test_route_argument_checks():
    # validation happens before any device call
    bad = [(-1, 8, 2), (4, 0, 1), (4, 1025, 2), (4, 8, 0), (4, 8, 9), (4, 100, 65)]
    for T, E, k in bad:
        assert mok.mok_route(None, T, E, k, None, None, None) == mok.MOK_ERROR_INVALID_VALUE, (T, E, k)
        assert mok.mok_route_backward(None, None, None, T, E, k, None, None) == mok.MOK_ERROR_INVALID_VALUE
    assert mok.mok_route(None, 0, 8, 2, None, None, None) == mok.MOK_OK          # empty call
    assert mok.mok_route(None, 3, 8, 2, None, None, None) == mok.MOK_ERROR_INVALID_VALUE   # null pointers
    assert mok.mok_route_backward(None, None, None, 0, 8, 2, None, None) == mok.MOK_OK


def _tile_rows(cfg):
    # the kernels' documented m-tile: 128 rows for BF16 layers averaging at most 128 rows per expert
    return 128 if cfg.precision == "bf16" and cfg.T * cfg.k <= 128 * cfg.E else 256


@pytest.mark.parametrize("name", ["tiny", "full_layer", "ep64_share", "ep64_share_mxfp8", "stream"])
@pytest.mark.parametrize("n_cu", [0, 8, 256, 304])
def test_autosize_matches_the_two_wave_rule(name, n_cu):
    from oracle import schedule as S
    import synth
    cfg = synth.CONFIGS[name]
    prec = mok.MOK_MXFP8 if cfg.precision == "mxfp8" else mok.MOK_BF16
    base = mok.MoKConfig(macrobatch_tokens=cfg.macrobatch_tokens, ring_bytes=cfg.ring_bytes, precision=prec,
                         capacity_multiplier=1.5)
    out = mok.autosize_config(base, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, n_cu)
    units = n_cu if n_cu > 0 else 256
    want = S.autosize_minibatch(cfg.T, cfg.k, cfg.I, cfg.macrobatch_tokens, units, _tile_rows(cfg), 256)
    assert out.minibatch_rows == want
    row_bytes = 2 * cfg.H if prec == mok.MOK_BF16 else cfg.H + cfg.H // 32
    assert out.ring_bytes == max(cfg.ring_bytes, 2 * want * row_bytes)
    assert (out.macrobatch_tokens, out.precision, out.capacity_multiplier) == \
        (base.macrobatch_tokens, base.precision, base.capacity_multiplier)
    mok.query_sizes(out, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)   # the result is a valid config


def test_autosize_rejects_bad_arguments():
    c = mok.mok_config()
    mok.mok_config_default(c)
    before = (c.minibatch_rows, c.ring_bytes)
    assert mok.mok_config_autosize(c, mok.mok_shape(64, 100, 64, 8, 2), 0) == mok.MOK_ERROR_INVALID_VALUE
    assert (c.minibatch_rows, c.ring_bytes) == before           # untouched on error
    c.capacity_multiplier = 0.0
    assert mok.mok_config_autosize(c, mok.mok_shape(64, 128, 64, 8, 2), 0) == mok.MOK_ERROR_INVALID_VALUE
    lib = ctypes.CDLL(mok._LIB_PATH)
    lib.mok_config_autosize.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    assert lib.mok_config_autosize(None, None, 0) == mok.MOK_ERROR_INVALID_VALUE


def test_weight_structs_keep_their_tensors_alive():
    # the structs hold raw pointers; the binding keeps the tensors referenced so
    # that temporaries passed in are not freed (and their memory reused) before the call
    import gc
    import weakref
    import torch
    t = torch.ones(8)
    r = weakref.ref(t)
    w = mok.weights_bf16(t, torch.ones(2), torch.ones(2))
    del t
    gc.collect()
    assert r() is not None
    pair = (torch.ones(4, dtype=torch.uint8), torch.ones(1, dtype=torch.uint8))
    r2 = weakref.ref(pair[0])
    w8 = mok.weights_mxfp8(pair, pair, pair)
    del pair
    gc.collect()
    assert r2() is not None
    del w, w8
    gc.collect()
    assert r() is None and r2() is None


def test_whole_pass_mode_is_switched_off():
    # every entry point that takes a config rejects the flag before any device work
    for prec in (mok.MOK_BF16, mok.MOK_MXFP8):
        cfg = mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 20, precision=prec,
                            debug_flags=mok.MOK_DEBUG_WHOLE_PASS)
        with pytest.raises(mok.MokError) as e:
            mok.query_sizes(cfg, 64, 256, 128, 8, 1)
        assert e.value.status == mok.MOK_ERROR_UNSUPPORTED
    c = mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 20, debug_flags=mok.MOK_DEBUG_WHOLE_PASS).c()
    sh = mok.mok_shape(64, 128, 64, 8, 1)
    p = ctypes.c_void_p(0x1000)
    assert mok.mok_build_schedule(c, sh, p, p, 1 << 20, None) == mok.MOK_ERROR_UNSUPPORTED
    w = mok.mok_weights(0x1000, 0x1000, 0x1000)
    assert mok.mok_forward(c, sh, p, 1 << 30, p, 1 << 30, p, p, w, p, p, 1 << 30, None) == \
        mok.MOK_ERROR_UNSUPPORTED
    assert mok.mok_backward(c, sh, p, 1 << 30, p, 1 << 30, p, p, w, p, 1 << 30, p, p, p, p, p, p, None) == \
        mok.MOK_ERROR_UNSUPPORTED


def _cpu_workspace(I=64, **over):
    # a workspace on the host: enough for the binding's checks, which run
    # before any call into the library
    c = mok.MoKConfig(minibatch_rows=32, ring_bytes=1 << 20, **over)
    return mok.get_workspace(c, device="cpu", num_local_tokens=64, hidden_size=128, intermediate_size=I,
                             num_experts=8, topk=2)


def test_binding_rejects_int64_ids():
    # int64 ids read as int32 would put every id in range and route silently wrong
    ws = _cpu_workspace()
    with pytest.raises(ValueError, match="dtype"):
        mok.build_schedule(ws, torch.zeros((64, 2), dtype=torch.int64))
    with pytest.raises(ValueError, match="shape"):
        mok.build_schedule(ws, torch.zeros((64, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="contiguous"):
        mok.build_schedule(ws, torch.zeros((2, 64), dtype=torch.int32).t())


def test_binding_rejects_wrong_outputs_and_inputs():
    ws = _cpu_workspace()
    sched = torch.zeros(ws.schedule_bytes, dtype=torch.uint8)
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    tw = torch.zeros((64, 2), dtype=torch.float32)
    w = mok.weights_bf16(torch.zeros((8, 128, 64), dtype=torch.bfloat16),
                         torch.zeros((8, 128, 64), dtype=torch.bfloat16),
                         torch.zeros((8, 64, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out: shape"):
        mok.forward(ws, sched, x, tw, w, out=torch.zeros((63, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x: dtype"):
        mok.forward(ws, sched, x.float(), tw, w)
    with pytest.raises(ValueError, match="schedule"):
        mok.forward(ws, sched[:16], x, tw, w)
    bad_w = mok.weights_bf16(torch.zeros((8, 64, 128), dtype=torch.bfloat16),
                             torch.zeros((8, 128, 64), dtype=torch.bfloat16),
                             torch.zeros((8, 64, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="w_gate: shape"):
        mok.forward(ws, sched, x, tw, bad_w)
    ctx = torch.zeros(ws.fwd_ctx_bytes, dtype=torch.uint8)
    grads = dict(dx=torch.zeros((64, 128), dtype=torch.bfloat16),
                 dw_gate=torch.zeros((8, 128, 64), dtype=torch.bfloat16),
                 dw_up=torch.zeros((8, 128, 64), dtype=torch.bfloat16),
                 dw_down=torch.zeros((8, 128, 64), dtype=torch.bfloat16),       # transposed: wrong
                 dtopk_w=torch.zeros((64, 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="dw_down: shape"):
        mok.backward(ws, sched, ctx, x, tw, w, x, grads=grads)


def test_binding_rejects_weights_of_the_wrong_mode():
    ws = _cpu_workspace(I=128, precision=mok.MOK_MXFP8)
    sched = torch.zeros(ws.schedule_bytes, dtype=torch.uint8)
    w = mok.weights_bf16(torch.zeros((8, 128, 128), dtype=torch.bfloat16),
                         torch.zeros((8, 128, 128), dtype=torch.bfloat16),
                         torch.zeros((8, 128, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="MXFP8 mode"):
        mok.forward(ws, sched, torch.zeros((64, 128), dtype=torch.bfloat16), torch.zeros((64, 2)), w)


def test_noalloc_forward_rejects_oversized_scratch_without_device_work():
    # the EP-64 share's default 256 MiB ring needs more than the static scratch;
    # the size check comes before any device call
    c = mok.MoKConfig(minibatch_rows=512, ring_bytes=256 << 20).c()
    sh = mok.mok_shape(16384, 7168, 2048, 4, 1)
    p = ctypes.c_void_p(0x1000)
    w = mok.mok_weights(0x1000, 0x1000, 0x1000)
    assert mok.mok_forward_noalloc(c, sh, p, 1 << 40, p, p, w, p, p, 1 << 40, None) == \
        mok.MOK_ERROR_BUFFER_TOO_SMALL
    assert "scratch" in mok.mok_last_error()
