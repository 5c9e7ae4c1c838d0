"""Seeded synthetic inputs for the MoE layer, shared by the tests, the benchmark and
the oracle.  This module holds input synthesis only: random draws, a softmax/top-k
router that turns random logits into routing inputs, and the conversion of the
draws to bf16 storage (done by torch's own dtype cast).  None of the layer's
arithmetic (dispatch, expert FFN, combine, their gradients) lives here.

Every tensor comes back as a numpy array: bf16 tensors as uint16 bit patterns,
``topk_idx`` int32, ``topk_weights`` float32, masks uint8.

The workloads follow the shapes of the pages: the Triton-distributed benchmark
(64 experts, top-8, hidden 1536, ffn 480, 1024..8192 tokens), the
low_latency_combine page (hidden 7168, top-8, zero/copy/constant experts,
activity masks) and the Megatron MoE performance-test proxy models (a
DeepSeek-V3 proxy with fewer experts, Mixtral-8x7B).
"""
from __future__ import annotations

import numpy as np
import torch

# name -> shape and routing recipe
WORKLOADS = {
    # tiny forward-only layer: the oracle finishes it in well under a second
    "tiny": dict(T=256, H=128, F=64, E=8, K=2),
    # Triton-distributed benchmark shape (T is one of 1024, 2048, 4096, 8192)
    "page1": dict(T=8192, H=1536, F=480, E=64, K=8),
    # combine-only stress at the low_latency_combine page's hidden size
    "combine_stress": dict(T=4096, H=7168, E=256, K=8, Z=1, C=1, Q=2),
    # DeepSeek-V3-style proxy with 32 experts, Zipf-skewed routing, one shared expert
    "dsv3_proxy": dict(T=4096, H=7168, F=2048, E=32, K=8, zipf=1.2, shared=True),
    # Mixtral-8x7B-style layer
    "mixtral": dict(T=8192, H=4096, F=14336, E=8, K=2),
    # decode batch of the low_latency_combine page (BS <= 512, H = 7168, top-8,
    # 32 experts in its example), forward only
    "decode": dict(T=512, H=7168, F=2048, E=32, K=8),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 draws -> bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _normal_bf16(rng, shape, std=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits(a)


def router(logits: np.ndarray, K: int, renorm: bool):
    """Softmax over the logits, top-K by descending probability (ties to the lower id),
    weights optionally renormalised to sum to one.  Input synthesis only."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :K]
    w = np.take_along_axis(p, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w.astype(np.float32)


def layer_inputs(T, H, F, E, K, seed=0, Z=0, C=0, Q=0, mask=None, mask_p_false=0.1,
                 mask_active=None, zipf=None, renorm=True, shared=False, grad=True,
                 weights=True):
    """Inputs of one MoE layer step.

    Draw order (fixed): x, router logits, mask, w_gate, w_up, w_down, shared-expert
    weights, constant-expert tensors, grad_out.

    * x ~ N(0,1); router logits ~ N(0,1) over the E+Z+C+Q ids (plus log of a Zipf
      popularity p_e ~ (e+1)^-s over the routed experts when ``zipf`` is s);
    * expert weights ~ N(0, std = 1/sqrt(fan_in)) in the (out, in) layout:
      w_gate, w_up (E, F, H), w_down (E, H, F);
    * mask: None, "1d" (the first ``mask_active`` tokens true) or "2d"
      (Bernoulli(1 - mask_p_false) per slot);
    * constant-expert alpha_1, alpha_2, v ~ N(0,1), shape (Q, H);
    * grad_out ~ N(0,1), shape (T, H).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(T=T, H=H, F=F, E=E, K=K, Z=Z, C=C, Q=Q)
    out["x"] = _normal_bf16(rng, (T, H))
    n_ids = E + Z + C + Q
    logits = rng.standard_normal((T, n_ids), dtype=np.float32).astype(np.float64)
    if zipf is not None:
        pop = np.arange(1, E + 1, dtype=np.float64) ** (-float(zipf))
        pop /= pop.sum()
        logits[:, :E] += np.log(pop)[None, :]
    out["topk_idx"], out["topk_weights"] = router(logits, K, renorm)
    if mask == "1d":
        n_act = T if mask_active is None else int(mask_active)
        m = np.zeros(T, dtype=np.uint8)
        m[:n_act] = 1
        out["mask"] = m
    elif mask == "2d":
        out["mask"] = (rng.random((T, K)) >= mask_p_false).astype(np.uint8)
    else:
        out["mask"] = None
    if weights:
        out["w_gate"] = _normal_bf16(rng, (E, F, H), 1.0 / np.sqrt(H))
        out["w_up"] = _normal_bf16(rng, (E, F, H), 1.0 / np.sqrt(H))
        out["w_down"] = _normal_bf16(rng, (E, H, F), 1.0 / np.sqrt(F))
    if shared:
        out["shared_w_gate"] = _normal_bf16(rng, (1, F, H), 1.0 / np.sqrt(H))
        out["shared_w_up"] = _normal_bf16(rng, (1, F, H), 1.0 / np.sqrt(H))
        out["shared_w_down"] = _normal_bf16(rng, (1, H, F), 1.0 / np.sqrt(F))
    if Q:
        out["const_alpha_1"] = _normal_bf16(rng, (Q, H))
        out["const_alpha_2"] = _normal_bf16(rng, (Q, H))
        out["const_v"] = _normal_bf16(rng, (Q, H))
    if grad:
        out["grad_out"] = _normal_bf16(rng, (T, H))
    return out


def combine_inputs(T=4096, H=7168, E=256, K=8, Z=1, C=1, Q=2, seed=0, mask="2d",
                   mask_p_false=0.1, shared=True, grad=True):
    """Combine-only inputs: routing as in layer_inputs (softmax top-K, not
    renormalised), an expanded expert-output buffer of T*min(E,K) rows ~ N(0,1),
    shared_expert_x and ori_x ~ N(0,1), constant-expert tensors ~ N(0,1).

    Draw order: x (used as ori_x), logits, mask, expert outputs, shared_expert_x,
    constant-expert tensors, grad_out.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(T=T, H=H, E=E, K=K, Z=Z, C=C, Q=Q)
    out["x"] = _normal_bf16(rng, (T, H))
    logits = rng.standard_normal((T, E + Z + C + Q), dtype=np.float32).astype(np.float64)
    out["topk_idx"], out["topk_weights"] = router(logits, K, renorm=False)
    if mask == "2d":
        out["mask"] = (rng.random((T, K)) >= mask_p_false).astype(np.uint8)
    else:
        out["mask"] = None
    out["y"] = _normal_bf16(rng, (T * min(E, K), H))
    out["shared_expert_x"] = _normal_bf16(rng, (T, H)) if shared else None
    if Q:
        out["const_alpha_1"] = _normal_bf16(rng, (Q, H))
        out["const_alpha_2"] = _normal_bf16(rng, (Q, H))
        out["const_v"] = _normal_bf16(rng, (Q, H))
    if grad:
        out["grad_out"] = _normal_bf16(rng, (T, H))
    return out
