"""Seeded synthetic workloads (shapes, dtypes and value distributions only).

This module holds no part of the method's arithmetic: it draws iid Gaussian
tensors from a seeded torch generator. Both the HIP path and the CPU oracle
are fed the same tensors (the oracle through a host copy).

Recipe: ``torch.randn(shape, float32, generator=g) * std`` drawn in the order
Q, K, V (then dO for a backward workload) from ``g.manual_seed(seed)``,
then rounded to the workload dtype (round-to-nearest-even for bf16). Shapes
are [B, S, H, Dh] in original sequence order.

The pages measure end-to-end training of causal transformers and name no
dataset; these iid inputs stand in for attention activations at the
sequence lengths the pages quote (summary page, "Key points": 262,144
tokens on 8 A100s, 786,432 tokens on 16 TPUv4 chips; 8,192 tokens for the
short-sequence case).
"""

import torch

WORKLOADS = {
    # correctness case: fp32 throughout
    "tiny": dict(batch=1, heads=1, seq=256, head_dim=64, dtype=torch.float32, n_dev=4,
                 std=(1.0, 1.0, 1.0), seed=0),
    # the pages' short-sequence case (8,192 tokens), 8 ring devices
    "short": dict(batch=1, heads=16, seq=8192, head_dim=128, dtype=torch.bfloat16, n_dev=8,
                  std=(0.5, 0.5, 0.5), seed=1),
    "mid": dict(batch=1, heads=32, seq=65536, head_dim=128, dtype=torch.bfloat16, n_dev=8,
                std=(0.5, 0.5, 1.0), seed=2),
    # the A100 run's sequence length (262,144) on 8 ring devices
    "long": dict(batch=1, heads=32, seq=262144, head_dim=128, dtype=torch.bfloat16, n_dev=8,
                 std=(0.5, 0.5, 0.5), seed=3),
    # the TPUv4 run's sequence length (786,432) on 16 ring devices, with backward
    "very_long": dict(batch=1, heads=32, seq=786432, head_dim=128, dtype=torch.bfloat16, n_dev=16,
                      std=(0.5, 0.5, 0.5), do_std=1.0, seed=4),
}


def shape_of(w):
    return (w["batch"], w["seq"], w["heads"], w["head_dim"])


def make_inputs(workload, device="cpu", seed=None, with_grad=False, **overrides):
    """Return dict(q, k, v[, do]) for a named workload (or a dict like the
    entries of WORKLOADS), original order, on ``device``."""
    w = dict(WORKLOADS[workload]) if isinstance(workload, str) else dict(workload)
    w.update(overrides)
    g = torch.Generator(device=device)
    g.manual_seed(w["seed"] if seed is None else seed)
    shape = shape_of(w)
    out = {}
    for name, std in zip(("q", "k", "v"), w["std"]):
        out[name] = (torch.randn(shape, dtype=torch.float32, generator=g, device=device) * std).to(w["dtype"])
    if with_grad:
        out["do"] = (torch.randn(shape, dtype=torch.float32, generator=g, device=device)
                     * w.get("do_std", 1.0)).to(w["dtype"])
    return out
