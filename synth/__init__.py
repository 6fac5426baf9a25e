"""Seeded synthetic inputs for the MoE layer.

This module is shared by the tests, the benchmark and the CPU oracle harness.
It holds random draws only: the router that turns logits into top-k ids and
gate weights (a step the layer takes as input, not one it computes), the
expert-load recipes, and rounding of fp32 draws to bf16 bit patterns. None of
the layer's own arithmetic (schedule, expert FFN, combine, gradients, MXFP8
codec) lives here.

Every tensor is drawn from ``numpy.random.SeedSequence(seed, spawn_key=(stream,
chunk))``: ``stream`` is fixed per tensor (routing, gates, x, W_gate, W_up,
W_down, dy, in that order) and ``chunk`` is the expert index for weights or a
block of rows for activations. Chunked streams let large tensors be drawn in
parallel threads and let a checker regenerate one expert's weights alone.

bf16 tensors are returned as ``uint16`` bit patterns (round to nearest even
from the fp32 draw); fp32 tensors as ``float32``; ids as ``int32``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_ROUTING, STREAM_GATES, STREAM_X, STREAM_WG, STREAM_WU, STREAM_WD, STREAM_DY = range(7)
ROW_BLOCK = 2048  # rows per seeded chunk of x / dy


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One synthetic workload: layer shape, routing recipe and knobs."""
    name: str
    T: int            # rows handed to the layer (tokens, or received rows for an EP share)
    H: int
    I: int
    E: int
    k: int
    routing: str      # "softmax_topk" | "zipf" | "uniform" | "dirichlet"
    zipf_s: float = 1.2
    dirichlet_alpha: float = 0.3
    minibatch_rows: int = 512
    macrobatch_tokens: int = 0      # 0 = one macro-batch
    ring_bytes: int = 256 << 20
    precision: str = "bf16"         # "bf16" | "mxfp8"
    tokens_per_step: int = 0        # pre-routing tokens this call stands for (throughput unit)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k


# The five workloads. "tokens_per_step" is the pre-routing token count that one
# call represents: the EP-64 share stands for 2,048 tokens held by one GPU.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, H=128, I=64, E=8, k=2, routing="softmax_topk",
                        minibatch_rows=32, ring_bytes=64 * 1024, tokens_per_step=64),
    "full_layer": LayerConfig("full_layer", T=2048, H=7168, I=2048, E=256, k=8,
                              routing="softmax_topk", tokens_per_step=2048),
    "ep64_share": LayerConfig("ep64_share", T=16384, H=7168, I=2048, E=4, k=1, routing="zipf",
                              ring_bytes=256 << 20, tokens_per_step=2048),
    "ep64_share_mxfp8": LayerConfig("ep64_share_mxfp8", T=16384, H=7168, I=2048, E=4, k=1,
                                    routing="zipf", precision="mxfp8", ring_bytes=256 << 20,
                                    tokens_per_step=2048),
    "ep64_share_mxfp8_uniform": LayerConfig("ep64_share_mxfp8_uniform", T=16384, H=7168, I=2048,
                                            E=4, k=1, routing="uniform", precision="mxfp8",
                                            ring_bytes=256 << 20, tokens_per_step=2048),
    "stream": LayerConfig("stream", T=163840, H=4096, I=1024, E=8, k=1, routing="dirichlet",
                          macrobatch_tokens=20480, ring_bytes=128 << 20, tokens_per_step=8 * 2048),
}


def seq(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, chunk)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------- routing

def largest_remainder(total: int, p: np.ndarray) -> np.ndarray:
    """Integer counts summing to ``total`` closest to ``total * p`` (largest remainder,
    ties to the lower index)."""
    q = total * np.asarray(p, dtype=np.float64)
    base = np.floor(q).astype(np.int64)
    rest = total - int(base.sum())
    frac = q - base
    order = sorted(range(len(p)), key=lambda i: (-frac[i], i))
    for i in order[:rest]:
        base[i] += 1
    return base


def softmax_topk_router(logits: np.ndarray, k: int):
    """Top-k on fp32 logits (descending, lower index first on ties), softmax in
    fp64 over all experts, renormalised over the chosen k, rounded to fp32."""
    T, E = logits.shape
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids, axis=1)
    w = (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def draw_logits(rng: np.random.Generator, T: int, E: int) -> np.ndarray:
    """N(0,1) fp32 logits; any row holding two exactly equal values is redrawn."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    while True:
        s = np.sort(logits, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            return logits
        logits[bad] = rng.standard_normal((bad.size, E), dtype=np.float32)


def draw_gates(rng: np.random.Generator, n: int) -> np.ndarray:
    """U(0,1) fp32 with exact zeros redrawn."""
    g = rng.random(n, dtype=np.float32)
    while True:
        z = np.nonzero(g == 0)[0]
        if z.size == 0:
            return g
        g[z] = rng.random(z.size, dtype=np.float32)


def make_routing(cfg: LayerConfig):
    """Returns (topk_ids int32 [T,k], topk_w float32 [T,k], logits or None)."""
    rng = seq(cfg.seed, STREAM_ROUTING)
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.routing == "softmax_topk":
        logits = draw_logits(rng, T, E)
        ids, w = softmax_topk_router(logits, k)
        return ids, w, logits
    assert k == 1, "load-recipe routing is defined for one routed row per token"
    if cfg.routing in ("zipf", "uniform"):
        if cfg.routing == "zipf":
            p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** cfg.zipf_s
        else:
            p = np.ones(E, dtype=np.float64)
        counts = largest_remainder(T, p / p.sum())
        ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts))
    elif cfg.routing == "dirichlet":
        MT = cfg.macrobatch_tokens or T
        parts = []
        for m0 in range(0, T, MT):
            n = min(MT, T - m0)
            p = rng.dirichlet(np.full(E, cfg.dirichlet_alpha))
            counts = largest_remainder(n, p)
            parts.append(rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts)))
        ids = np.concatenate(parts)
    else:
        raise ValueError(cfg.routing)
    w = draw_gates(seq(cfg.seed, STREAM_GATES), T)
    return ids.reshape(T, 1).astype(np.int32), w.reshape(T, 1), None


# ----------------------------------------------------------------------------- tensors

def _normal_bf16(seed, stream, chunk, shape, scale):
    a = seq(seed, stream, chunk).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return f32_to_bf16_bits(a)


def expert_weight(cfg: LayerConfig, which: str, e: int) -> np.ndarray:
    """One expert's weight as bf16 bits: W_gate/W_up [H,I] (std 1/sqrt(H)),
    W_down [I,H] (std 1/sqrt(I))."""
    if which == "gate":
        return _normal_bf16(cfg.seed, STREAM_WG, e, (cfg.H, cfg.I), 1.0 / np.sqrt(cfg.H))
    if which == "up":
        return _normal_bf16(cfg.seed, STREAM_WU, e, (cfg.H, cfg.I), 1.0 / np.sqrt(cfg.H))
    if which == "down":
        return _normal_bf16(cfg.seed, STREAM_WD, e, (cfg.I, cfg.H), 1.0 / np.sqrt(cfg.I))
    raise ValueError(which)


def expert_weights(cfg: LayerConfig, which: str, experts=None) -> np.ndarray:
    experts = range(cfg.E) if experts is None else list(experts)
    experts = list(experts)
    shape = (cfg.H, cfg.I) if which in ("gate", "up") else (cfg.I, cfg.H)
    out = np.empty((len(experts),) + shape, dtype=np.uint16)

    def one(i):
        out[i] = expert_weight(cfg, which, experts[i])
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(experts))))
    return out


def activation_rows(cfg: LayerConfig, which: str, rows=None) -> np.ndarray:
    """x or dy as bf16 bits, N(0,1), drawn in blocks of ROW_BLOCK rows. ``rows``
    (optional, sorted or not) selects a subset without drawing the rest."""
    stream = STREAM_X if which == "x" else STREAM_DY
    T, H = cfg.T, cfg.H
    nblk = (T + ROW_BLOCK - 1) // ROW_BLOCK

    def block(b):
        n = min(ROW_BLOCK, T - b * ROW_BLOCK)
        return _normal_bf16(cfg.seed, stream, b, (n, H), 1.0)

    if rows is None:
        out = np.empty((T, H), dtype=np.uint16)

        def one(b):
            out[b * ROW_BLOCK: b * ROW_BLOCK + min(ROW_BLOCK, T - b * ROW_BLOCK)] = block(b)
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nblk)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H), dtype=np.uint16)
    for b in np.unique(rows // ROW_BLOCK):
        blk = block(int(b))
        sel = np.nonzero(rows // ROW_BLOCK == b)[0]
        out[sel] = blk[rows[sel] - b * ROW_BLOCK]
    return out


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    topk_ids: np.ndarray   # int32 [T,k]
    topk_w: np.ndarray     # float32 [T,k]
    x: np.ndarray          # uint16 bf16 bits [T,H]
    w_gate: np.ndarray     # uint16 [E,H,I]
    w_up: np.ndarray       # uint16 [E,H,I]
    w_down: np.ndarray     # uint16 [E,I,H]
    dy: np.ndarray         # uint16 [T,H]
    logits: np.ndarray | None = None


def make_inputs(cfg: LayerConfig | str) -> LayerInputs:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    ids, w, logits = make_routing(cfg)
    return LayerInputs(cfg, ids, w,
                       activation_rows(cfg, "x"),
                       expert_weights(cfg, "gate"), expert_weights(cfg, "up"),
                       expert_weights(cfg, "down"),
                       activation_rows(cfg, "dy"), logits)


def small_config(name="small", *, T, H, I, E, k, minibatch_rows=32, macrobatch_tokens=0,
                 ring_bytes=1 << 20, routing="softmax_topk", seed=0, precision="bf16") -> LayerConfig:
    """A custom small workload for parity cases beyond the five named ones."""
    return LayerConfig(name, T=T, H=H, I=I, E=E, k=k, routing=routing,
                       minibatch_rows=minibatch_rows, macrobatch_tokens=macrobatch_tokens,
                       ring_bytes=ring_bytes, precision=precision, tokens_per_step=T, seed=seed)


# ----------------------------------------------------------------------------- MXFP8-lossless inputs

def lossless_mxfp8_inputs(cfg: LayerConfig) -> LayerInputs:
    """Inputs on which every MXFP8 quantization point of the layer is exact.

    Every operand the MXFP8 mode quantizes (x, dy, the three weights, and the
    activations a and dh the layer derives from them) then holds values n * 2^p
    with an integer 1 <= n <= 14: four significant bits at most, and a block
    maximum whose leading digits are at most 1.75, so that scaling by the E8M0
    block exponent never saturates past 448. The construction:

      x[:, :H/2]  integers 1..14        x[:, H/2:]  +-2^(0..3)
      W_gate[e][pg(i), i] = 32          (pg into the first half of H)
      W_up[e][pu(i), i]   = +-2^(0..2)  (pu into the second half of H)
      W_down[e][i, pd(i)] = +-2^(-3..0) (pd injective: one entry per row and column)
      dy = +-2^(0..3);   gate weights 1/2 or 1

    so that h_gate = 32 n >= 32 (where silu is the identity to within
    exp(-32)), h_up and G = dy W_down^T are single terms, and a, dh, y and the
    combine are exact in fp32 and bf16. Requires k <= 2, I <= H/2, H even.
    Routing (ids) follows ``cfg.routing``; these are draws only, like every
    other input here.
    """
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    assert k <= 2 and H % 2 == 0 and I <= H // 2
    ids, _, logits = make_routing(cfg)
    rng = seq(cfg.seed, STREAM_X, 1 << 20)
    half = H // 2
    x = np.empty((T, H), dtype=np.float32)
    x[:, :half] = rng.integers(1, 15, size=(T, half))
    x[:, half:] = rng.choice([-1.0, 1.0], size=(T, H - half)) * 2.0 ** rng.integers(0, 4, size=(T, H - half))
    wg = np.zeros((E, H, I), dtype=np.float32)
    wu = np.zeros((E, H, I), dtype=np.float32)
    wd = np.zeros((E, I, H), dtype=np.float32)
    cols = np.arange(I)
    for e in range(E):
        wg[e, rng.integers(0, half, size=I), cols] = 32.0
        wu[e, rng.integers(half, H, size=I), cols] = rng.choice([-1.0, 1.0], size=I) * 2.0 ** rng.integers(0, 3, size=I)
        wd[e, cols, rng.permutation(H)[:I]] = rng.choice([-1.0, 1.0], size=I) * 2.0 ** -rng.integers(0, 4, size=I)
    dy = rng.choice([-1.0, 1.0], size=(T, H)) * 2.0 ** rng.integers(0, 4, size=(T, H))
    w = rng.choice([0.5, 1.0], size=(T, k)).astype(np.float32)
    b = f32_to_bf16_bits
    return LayerInputs(cfg, ids, w, b(x), b(wg), b(wu), b(wd), b(dy.astype(np.float32)), logits)
