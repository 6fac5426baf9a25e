"""O2/O3 — forward and backward of the MoE layer in fp64 (test infrastructure only).

The schedule, ring, mini-batches and macro-batches only decide evaluation
order; the layer's value is the plain sparse-MoE result ("Mixture-of-Kittens(MoK)란?"
explainer, section 1: each input activates a few experts). This module writes
that result out from its definition, per expert, in fp64.

Definitions followed:
* expert FFN = SwiGLU ("Cursor Open-Sources Mixture-of-Kittens (MoK)" digest,
  English abstract, which names the SwiGLU backward): for routed row f = (t, j)
  sent to expert e,
      h_g = x_t W_gate[e],  h_u = x_t W_up[e],  a = silu(h_g) * h_u,
      y_f = a W_down[e],    silu(z) = z / (1 + exp(-z)).
* weighted combine back to token order: out_t = sum_j g_{t,j} y_{(t,j)}.
* backward for upstream dy (chain rule of the above):
      dg_{t,j} = <dy_t, y_{(t,j)}>          (router-weight gradient)
      G = dy_t W_down[e]^T,  da = g G,
      dh_u = da * silu(h_g),  dh_g = da * h_u * s (1 + h_g (1 - s)),  s = sigmoid(h_g)
      dx_t = sum_j dh_g W_gate[e]^T + dh_u W_up[e]^T
      dW_gate[e] = sum_{f in e} x_t^T dh_g,  dW_up[e] = sum x_t^T dh_u,
      dW_down[e] = sum (g a)^T dy_t.
  The same digest states the router-weight gradient is fused into the SwiGLU
  backward: <dy, a W_down^T ... > is evaluated as <G, a>, which is the same
  number by associativity; both forms are returned.

MXFP8 mode ("Mixture-of-Kittens (MoK)" project summary, Key-concepts table:
MXFP8 weights are pre-quantized): ``fq`` is a fake-quant callable
``fq(array, axis)`` applied to both operands of the forward gate/up and down
products and the backward input-gradient products, along their contraction
axis; weight gradients stay unquantized (reading: MXFP8 is a weight format and
the weight-gradient products have no weight operand). The MXFP8 weight-gradient
variant (``wgrad_fq``) also quantizes the weight-gradient products' operands
along the contraction axis, the expert's rows: blocks of 32 rows in canonical
order per column, the last block of each expert zero-padded.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z / (1.0 + np.exp(-z))


def _ident(a, axis):
    return a


# ----------------------------------------------------------------------------- one expert

def expert_forward(xe, Wg, Wu, Wd, fq=None):
    """Rows xe [n,H] through one SwiGLU expert. Returns h_g, h_u, a, y."""
    fq = fq or _ident
    xq = fq(xe, 1)
    hg = xq @ fq(Wg, 0)
    hu = xq @ fq(Wu, 0)
    a = silu(hg) * hu
    y = fq(a, 1) @ fq(Wd, 0)
    return hg, hu, a, y


def swiglu_backward(G, hg, hu, g):
    """SwiGLU backward for upstream G = dy W_down^T and per-row gate g [n,1].
    Returns dh_g, dh_u and the fused router-weight gradient <G, a> per row."""
    s = sigmoid(hg)
    sl = hg * s
    a = sl * hu
    dw = np.sum(G * a, axis=1)
    da = g * G
    dhu = da * sl
    dhg = da * hu * s * (1.0 + hg * (1.0 - s))
    return dhg, dhu, dw


def rows_fq(fq, a):
    """fq along the row (token) axis of a [n, c], the rows zero-padded to a
    multiple of 32 first: a group's last block holds its tail rows and zeros,
    which leave the block's largest magnitude, and every product, unchanged."""
    n = a.shape[0]
    pad = -n % 32
    ap = np.concatenate([a, np.zeros((pad,) + a.shape[1:])], axis=0) if pad else a
    return fq(ap, 0)[:n]


def expert_backward(xe, dye, g, Wg, Wu, Wd, fq=None, wgrad_fq=None):
    """Backward of one expert for its rows. g is [n,1]. Returns a dict with the
    per-row input gradient dxr, router-weight gradient (fused and direct) and
    this expert's weight gradients. wgrad_fq (MXFP8 weight gradients) quantizes
    both operands of each weight-gradient product along their contraction
    axis, the expert's rows in canonical order: x and dh for dW_gate / dW_up,
    g*a and dy for dW_down."""
    fq = fq or _ident
    hg, hu, a, y = expert_forward(xe, Wg, Wu, Wd, fq)
    G = fq(dye, 1) @ fq(Wd, 1).T
    dhg, dhu, dw = swiglu_backward(G, hg, hu, g)
    dw_direct = np.sum(dye * y, axis=1)
    dxr = fq(dhg, 1) @ fq(Wg, 1).T + fq(dhu, 1) @ fq(Wu, 1).T
    if wgrad_fq is None:
        dWg, dWu, dWd = xe.T @ dhg, xe.T @ dhu, (g * a).T @ dye
    else:
        q = lambda v: rows_fq(wgrad_fq, v)
        dWg, dWu, dWd = q(xe).T @ q(dhg), q(xe).T @ q(dhu), q(g * a).T @ q(dye)
    return dict(dxr=dxr, dw=dw, dw_direct=dw_direct, dWg=dWg, dWu=dWu, dWd=dWd,
                hg=hg, hu=hu, dhg=dhg, dhu=dhu)


# ----------------------------------------------------------------------------- whole layer

def _rows_of(ids_flat, e):
    return np.nonzero(ids_flat == e)[0]


def forward(x, topk_ids, topk_w, Wg, Wu, Wd, fq=None):
    """x [T,H], topk_ids [T,k], topk_w [T,k], Wg/Wu [E,H,I], Wd [E,I,H] (fp64
    values). Returns out [T,H] and the per-routed-row expert outputs y [R,H]."""
    T, k = topk_ids.shape
    H = x.shape[1]
    flat = topk_ids.reshape(-1)
    Y = np.zeros((T * k, H))
    for e in range(Wg.shape[0]):
        rows = _rows_of(flat, e)
        if rows.size:
            Y[rows] = expert_forward(x[rows // k], Wg[e], Wu[e], Wd[e], fq)[3]
    out = np.zeros((T, H))
    for j in range(k):
        out += topk_w[:, j:j + 1].astype(np.float64) * Y[j::k]
    return out, Y


def backward(x, topk_ids, topk_w, Wg, Wu, Wd, dy, fq=None, wgrad_fq=None):
    """Gradients of L = <dy, out>. Returns dict with dx [T,H], dWg, dWu [E,H,I],
    dWd [E,I,H], dw [T,k] (fused form), dw_direct [T,k]."""
    T, k = topk_ids.shape
    flat = topk_ids.reshape(-1)
    wflat = topk_w.reshape(-1).astype(np.float64)
    dx = np.zeros_like(x, dtype=np.float64)
    dWg, dWu, dWd = np.zeros(Wg.shape), np.zeros(Wu.shape), np.zeros(Wd.shape)
    dw = np.zeros(T * k)
    dw_direct = np.zeros(T * k)
    for e in range(Wg.shape[0]):
        rows = _rows_of(flat, e)
        if rows.size == 0:
            continue
        tok = rows // k
        r = expert_backward(x[tok], dy[tok], wflat[rows][:, None], Wg[e], Wu[e], Wd[e], fq, wgrad_fq)
        np.add.at(dx, tok, r["dxr"])
        dWg[e], dWu[e], dWd[e] = r["dWg"], r["dWu"], r["dWd"]
        dw[rows] = r["dw"]
        dw_direct[rows] = r["dw_direct"]
    return dict(dx=dx, dWg=dWg, dWu=dWu, dWd=dWd, dw=dw.reshape(T, k),
                dw_direct=dw_direct.reshape(T, k))


# ----------------------------------------------------------------------------- sampled outputs
# The same definitions evaluated for a subset of tokens or weight columns, so that
# full-size GPU results can be checked at sampled positions.

def token_forward(x_rows, ids_rows, w_rows, expert_w, fq=None):
    """out for selected tokens. x_rows [n,H], ids_rows/w_rows [n,k]; expert_w(e)
    returns (Wg, Wu, Wd) of expert e as fp64."""
    n, k = ids_rows.shape
    out = np.zeros_like(x_rows, dtype=np.float64)
    for e in np.unique(ids_rows):
        t, j = np.nonzero(ids_rows == e)
        Wg, Wu, Wd = expert_w(int(e))
        y = expert_forward(x_rows[t], Wg, Wu, Wd, fq)[3]
        out[t] += w_rows[t, j][:, None].astype(np.float64) * y
    return out


def token_backward(x_rows, dy_rows, ids_rows, w_rows, expert_w, fq=None):
    """dx [n,H] and dw [n,k] for selected tokens."""
    n, k = ids_rows.shape
    dx = np.zeros_like(x_rows, dtype=np.float64)
    dw = np.zeros((n, k))
    for e in np.unique(ids_rows):
        t, j = np.nonzero(ids_rows == e)
        Wg, Wu, Wd = expert_w(int(e))
        r = expert_backward(x_rows[t], dy_rows[t], w_rows[t, j][:, None].astype(np.float64),
                            Wg, Wu, Wd, fq)
        np.add.at(dx, t, r["dxr"])
        dw[t, j] = r["dw"]
    return dx, dw


def expert_wgrad_columns(xe, dye, g, Wg, Wu, Wd, cols, fq=None, wgrad_fq=None):
    """Columns ``cols`` of dW_gate[e], dW_up[e] ([H, len(cols)]) and rows ``cols`` of
    dW_down[e] ([len(cols), H]) from all of expert e's rows (xe, dye, g [n,1]).
    ``fq`` as in expert_backward: it reaches the weight gradients only through
    h (forward product) and G (dA product); the gradient products themselves
    take unquantized operands. Quantization runs along H, so a column subset
    of W_gate/W_up or a row subset of W_down quantizes like the whole.
    ``wgrad_fq`` as in expert_backward: blocks run along the rows, one column
    at a time, so a column subset also quantizes like the whole."""
    fq = fq or _ident
    xq = fq(xe, 1)
    hg = xq @ fq(Wg[:, cols], 0)
    hu = xq @ fq(Wu[:, cols], 0)
    G = fq(dye, 1) @ fq(Wd[cols, :], 1).T
    dhg, dhu, _ = swiglu_backward(G, hg, hu, g)
    a = silu(hg) * hu
    if wgrad_fq is None:
        return xe.T @ dhg, xe.T @ dhu, (g * a).T @ dye
    q = lambda v: rows_fq(wgrad_fq, v)
    return q(xe).T @ q(dhg), q(xe).T @ q(dhu), q(g * a).T @ q(dye)


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F (0 when both are exactly zero, infinite when
    only ref is). The tolerance measure for floating-point outputs: one number
    per output tensor (per expert for the weight gradients)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    nd = np.linalg.norm(got - ref)
    if nr == 0:
        return 0.0 if nd == 0 else float("inf")
    return float(nd / nr)


def rel_rows(got, ref) -> np.ndarray:
    """Per-row form of rel_frobenius: ||got[r] - ref[r]|| / ||ref[r]|| for every
    row r of the leading axis (trailing axes flattened into the row); 0 where
    both rows are exactly zero, infinite where only ref's is. A row that is
    wrong as a whole (another row's values, zeros, a wrong expert) scores about
    1 or more, however many correct rows surround it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    n = ref.shape[0] if ref.ndim else 1
    g2, r2 = got.reshape(n, -1), ref.reshape(n, -1)
    nr = np.linalg.norm(r2, axis=1)
    nd = np.linalg.norm(g2 - r2, axis=1)
    out = np.empty(n)
    zero = nr == 0
    out[~zero] = nd[~zero] / nr[~zero]
    out[zero] = np.where(nd[zero] == 0, 0.0, np.inf)
    return out
