"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic (no quantization, packing or matmul).  The shapes model a
64-layer dense 27B decoder with hidden size 5120 and FFN width 17408 (the
model on the pages: "Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF", the
architecture paragraph; the layer widths are the ones adopted for this
workload).  Trained weights are not used: weights are N(0, 0.02^2) fp32
before quantization and activations are N(0, 1) rounded to fp16.
"""

import numpy as np

WEIGHT_STD = 0.02

# Named workloads: (M, K, N).  K is the reduction (input) width, N the outputs.
WORKLOADS = {
    "tiny_matvec": dict(M=1, K=256, N=512),
    "decode_gate_up": dict(M=1, K=5120, N=17408),
    "verify_down": dict(M=4, K=17408, N=5120),
    "prefill_a8": dict(M=2048, K=5120, N=17408),
}

# One decoder layer's projections for the full decode-step pass: name -> (K, N).
LAYER_PROJECTIONS = [
    ("qkv", 5120, 7168),
    ("out", 5120, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
]
N_LAYERS = 64

WEIGHT_SEED = 0
ACT_SEED = 1


def layer_weight_seed(layer, proj_index):
    return 1000 + 8 * layer + proj_index


def weights(n, k, seed=WEIGHT_SEED, std=WEIGHT_STD):
    """fp32 W [n, k] ~ N(0, std^2), NumPy PCG64 stream ``seed``."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations(m, k, seed=ACT_SEED):
    """fp16 X [m, k] ~ N(0, 1), NumPy PCG64 stream ``seed``."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def weights_device(n, k, seed, device="cuda", std=WEIGHT_STD):
    """fp32 W [n, k] drawn on the device with a seeded torch generator (large shapes)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.empty((n, k), dtype=torch.float32, device=device)
    w.normal_(0.0, std, generator=g)
    return w


def activations_device(m, k, seed, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty((m, k), dtype=torch.float32, device=device)
    x.normal_(0.0, 1.0, generator=g)
    return x.to(torch.float16)
