"""Shared helpers for the GPU parity tests (oracle side and comparisons)."""
import numpy as np
import torch

import oracle
from quantized_moe_expert_02_amd import synth

REL_L2 = 1e-3
MAX_ABS = 1e-2


def oracle_route(layer, x):
    return oracle.route(layer.dims, x.cpu(), layer.router_w.cpu(),
                        None if layer.router_b is None else layer.router_b.cpu())


def oracle_y(layer, x, tokens=None):
    """Oracle output for a layer (weights on any device); only the experts the
    oracle's own routing selects are copied to the host."""
    r = oracle_route(layer, x)
    if tokens is None:
        need = r.uniq_ids
    else:
        need = np.unique(r.topk_idx[np.asarray(tokens)])
        need = need[need >= 0]  # -1: slots dropped by adaptive top-p
    return oracle.forward(layer, x.cpu(), tokens=tokens, experts_needed=need)


def assert_close(y_gpu: torch.Tensor, y_ref: np.ndarray, what=""):
    g = y_gpu.detach().float().cpu().double().numpy()
    assert g.shape == y_ref.shape, (g.shape, y_ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = g - y_ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(y_ref), 1e-300)
    mx = np.abs(err).max() if err.size else 0.0
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e}"
    return rel, mx


def min_topk_gap(r, k):
    """Smallest gap between the k-th and (k+1)-th logit over tokens."""
    z = np.sort(r.z, axis=1)[:, ::-1]
    if z.shape[1] <= k:
        return np.inf
    return float(np.min(z[:, k - 1] - z[:, k]))


def top_p_margin(r, k, p):
    """Smallest distance, over tokens and slots, between p (the layer's
    binary32 threshold) and a prefix sum of the renormalised slot weights in
    fp64.  The GPU and the oracle take the kept-slot decision in fp64, but
    their exp and summation order may differ in the last bits, so cases must
    keep clear of the threshold.  r: a plain top-k oracle route (z set)."""
    p32 = float(np.float32(p))
    margin = np.inf
    for t in range(r.topk_idx.shape[0]):
        zs = r.z[t, r.topk_idx[t]].astype(np.float64)
        s = 1.0 / (1.0 + np.exp(-zs))
        cum = np.cumsum(s / s.sum())
        margin = min(margin, float(np.min(np.abs(cum - p32))))
    return margin
