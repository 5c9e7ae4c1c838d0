"""Plain CPU oracle of the router that produces ``topk_idx`` and ``topk_weights``.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never does.  It shares no code
with the HIP library (nor with the input generator).

What it computes, and where that is defined
-------------------------------------------
The low_latency_combine page takes the routing as inputs (section "Parameters":
``topk_idx`` holds K distinct ids per token in [0, num_experts + special experts),
``topk_weights`` a float weight per (token, k)); the pages print no router.  The
reading taken here is plain softmax top-K gating over every id a slot may take
(routed and special experts alike):

* ``p = softmax(logits)`` over the ids of one token;
* the K ids of the largest logits (softmax is increasing in the logit), in
  descending order, equal logits ordered by increasing id;
* ``topk_weights = p[topk_idx]``, or, with renormalisation, those K values divided
  by their sum (the same as a softmax over the K selected logits).

The backward maps ``d topk_weights`` to ``d logits`` with the selection held fixed:

* renormalised: ``dl_i = w_i (dw_i - sum_k w_k dw_k)`` for a selected id i, 0 else;
* plain: ``dl_i = p_i ([i selected] dw_i - sum_k w_k dw_k)`` for every id i.

Everything is float64.
"""
import numpy as np


def softmax(logits):
    """Row softmax in float64, shifted by the row maximum."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def select_topk(logits, K):
    """Ids of the K largest logits per row, descending; equal logits by increasing id."""
    z = np.asarray(logits, dtype=np.float64)
    # a stable sort of the negated logits keeps equal values in id order
    order = np.argsort(-z, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def router_fwd(logits, K, renorm):
    """(topk_idx int32 (T, K), topk_weights float64 (T, K))."""
    idx = select_topk(logits, K)
    p = softmax(logits)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def router_bwd(logits, topk_idx, grad_topk_weights, renorm):
    """Gradient of sum(grad_topk_weights * topk_weights) with respect to the logits."""
    p = softmax(logits)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dw = np.asarray(grad_topk_weights, dtype=np.float64)
    w = np.take_along_axis(p, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    s = (w * dw).sum(axis=1, keepdims=True)
    if renorm:
        dl = np.zeros_like(p)
        np.put_along_axis(dl, idx, w * (dw - s), axis=1)
        return dl
    sel = np.zeros_like(p)
    np.put_along_axis(sel, idx, dw, axis=1)
    return p * (sel - s)
