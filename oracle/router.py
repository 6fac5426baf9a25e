"""O5 — the router front-end: logits to top-k expert ids and gate weights, and
the gradient back to the logits (test infrastructure only).

The pages take the top-k expert choice as an input of schedule building
("Mixture-of-Kittens (MoK)" project summary, Functional API) in a sparse layer
where each token activates a few experts ("Mixture-of-Kittens(MoK)란?"
explainer, section 1). They do not spell the router out; this follows the
plainest reading the rest supports, for logits l[t, 0..E-1] (fp32 inputs,
exact in fp64):

  p      = softmax(l) over all E experts
  ids    = the k experts with the largest logits; slot j holds the j-th
           largest, the lower expert index first among equal logits
  w_j    = p[ids_j] / sum_i p[ids_i]          (renormalised over the chosen k)

Backward: the chosen set is piecewise constant in l, so the logit gradient is
the chain rule through the two steps above, written as two vector-Jacobian
products (renormalisation, then softmax).
"""
from __future__ import annotations

import numpy as np


def softmax(l: np.ndarray) -> np.ndarray:
    """Row softmax in fp64, shifted by the row maximum."""
    z = np.asarray(l, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def choose(l: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32: per row, expert indices by descending logit, lower index
    first among equal logits (a stable sort of -l)."""
    l = np.asarray(l, dtype=np.float64)
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route(logits: np.ndarray, k: int):
    """Forward: (ids int32 [T, k], w fp64 [T, k])."""
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    p = softmax(logits)
    ids = choose(logits, k)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return ids, sel / sel.sum(axis=1, keepdims=True)


def route_backward(logits: np.ndarray, ids: np.ndarray, dw: np.ndarray) -> np.ndarray:
    """dL/dl [T, E] fp64 from dL/dw [T, k] for the chosen ids."""
    T, E = logits.shape
    p = softmax(logits)
    idx = ids.astype(np.int64)
    sel = np.take_along_axis(p, idx, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    dw = np.asarray(dw, dtype=np.float64)
    # renormalisation w_j = p_j / S, S = sum_i p_i over the chosen set:
    # dL/dp_j = dw_j / S - sum_i dw_i p_i / S^2 for chosen j, 0 elsewhere
    dsel = dw / S - (dw * sel).sum(axis=1, keepdims=True) / S**2
    dp = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dp, idx, dsel, axis=1)
    # softmax: dL/dl = p * (dL/dp - <p, dL/dp>)
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))
