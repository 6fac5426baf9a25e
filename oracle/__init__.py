"""Plain CPU oracle for one GPU's share of a deterministic MoE training layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP library.

Sources (the pages these functions are written from):

* "Mixture-of-Kittens (MoK)" project summary — Overview, Functional API and the
  Key-concepts table: a deterministic MoE layer, forward and backward, BF16 and
  MXFP8; the caller passes top-k expert ids to schedule building; MXFP8 is a
  weight format pre-quantized before the kernel.
* "Cursor Open-Sources Mixture-of-Kittens (MoK)" digest — English abstract: the
  expert FFN is SwiGLU and the router-weight gradient is computed inside the
  SwiGLU backward.
* "Mixture-of-Kittens(MoK)란?" explainer — section 1 (sparse MoE: each input
  activates a few experts), section 4 ① (one schedule table drives every
  phase), section 4 ③ (drop-free ring buffer, mini-batches, macro-batches,
  backward in reverse).

Modules:
  schedule  — O1, the schedule table (integer result, compared bit-exactly)
  layer     — O2/O3, forward and backward in fp64
  mxfp8     — O4, the MXFP8 codec and fake-quant
  router    — O5, the router front-end (softmax, top-k, renormalisation) and
              its logit gradient

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values fixed outside the oracle (closed forms, brute force, finite
differences, an independent autograd formulation, library casts); none is
"parity unpinned".
"""
from . import schedule, layer, mxfp8, router  # noqa: F401
