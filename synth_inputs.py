"""Seeded synthetic inputs for the collectives, shared by tests and the benchmark.

This module only draws numbers and describes workload shapes.  It holds none
of the reduction arithmetic, and it imports neither the oracle nor the HIP
library, so both sides can take their inputs from here.

Workloads follow the pages' own setups: ruCCL README (ja), "CUDA tensor
example" (4 logical ranks on one GPU, 257 FP32 elements), and section 6
"Collective training" (whole gradient lists reduced with Mean); the larger
sizes are the bandwidth workloads this library is measured on.

Draw rule: one generator per workload, ranks drawn in order (rank 0 first).
The batched gradient workload seeds each (tensor t, rank r) on its own as
seed * 1_000_003 + t * R + r, so any tensor can be regenerated alone.
"""

import numpy as np

INT_LIMIT = 1 << 20

# name -> description; "ops" lists the calls each workload exercises
WORKLOADS = {
    "ranks4_257_f32": dict(R=4, N=257, dtype="f32", dist="uniform", seed=0,
                           ops=("all_reduce:sum", "all_reduce:mean", "reduce:sum:0", "broadcast:1")),
    "ranks8_64MiB_f32": dict(R=8, N=16_777_216, dtype="f32", dist="normal", sigma=1.0, seed=1,
                             ops=("all_reduce:sum", "all_reduce:mean")),
    "ranks4_64MiB_i32": dict(R=4, N=16_777_216, dtype="i32", dist="int", seed=2,
                             ops=("all_reduce:sum", "all_reduce:max", "reduce:sum:2", "broadcast:3")),
    "ranks8_256MiB_f32_rs_ag": dict(R=8, N=67_108_864, dtype="f32", dist="normal", sigma=1.0, seed=3,
                                    ops=("reduce_scatter:sum", "all_gather")),
    "ranks4_llama32_grads_f32": dict(R=4, N=None, dtype="f32", dist="normal", sigma=1e-3, seed=4,
                                     ops=("all_reduce_many:mean",)),
}


def transformer_grad_shapes(layers=32, hidden=4096, ffn=11008, vocab=32000):
    """Gradient shapes of a 32-layer transformer: the embedding, then per layer
    four [h,h] projections, two [ffn,h], one [h,ffn] and two [h] norm weights."""
    shapes = [(vocab, hidden)]
    for _ in range(layers):
        shapes += [(hidden, hidden)] * 4
        shapes += [(ffn, hidden)] * 2
        shapes += [(hidden, ffn)]
        shapes += [(hidden,)] * 2
    return shapes


def per_tensor_seed(seed, t, num_ranks, r):
    return seed * 1_000_003 + t * num_ranks + r


# ---------------------------------------------------------------- NumPy (CPU)

def numpy_rank_inputs(R, N, dtype="f32", dist="uniform", seed=0, sigma=1.0):
    """R host arrays of N elements, drawn rank by rank from one generator."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(R):
        if dtype == "i32":
            out.append(rng.integers(-INT_LIMIT, INT_LIMIT + 1, size=N, dtype=np.int64).astype(np.int32))
        elif dist == "normal":
            out.append((rng.standard_normal(N) * sigma).astype(np.float32))
        elif dist == "uniform":
            out.append(rng.uniform(-1.0, 1.0, size=N).astype(np.float32))
        elif dist == "intvalued":
            out.append(rng.integers(-INT_LIMIT, INT_LIMIT + 1, size=N).astype(np.float32))
        else:
            raise ValueError(dist)
    return out


# ---------------------------------------------------------------- torch (GPU)

def torch_rank_inputs(R, N, dtype="f32", dist="uniform", seed=0, sigma=1.0, device="cuda"):
    """R device tensors of N elements, drawn rank by rank from one generator."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    out = []
    for _ in range(R):
        out.append(_torch_draw(torch, g, N, dtype, dist, sigma, device))
    return out


def _torch_draw(torch, g, shape, dtype, dist, sigma, device):
    if isinstance(shape, int):
        shape = (shape,)
    if dtype == "i32":
        return torch.randint(-INT_LIMIT, INT_LIMIT + 1, shape, dtype=torch.int32,
                             generator=g, device=device)
    if dist == "normal":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return t.mul_(sigma) if sigma != 1.0 else t
    if dist == "uniform":
        return torch.rand(shape, generator=g, device=device, dtype=torch.float32).mul_(2).sub_(1)
    if dist == "intvalued":
        return torch.randint(-INT_LIMIT, INT_LIMIT + 1, shape, generator=g,
                             device=device).to(torch.float32)
    raise ValueError(dist)


def torch_tensor_for(seed, t, num_ranks, r, shape, dtype="f32", dist="normal", sigma=1e-3,
                     device="cuda", out=None):
    """Rank r's copy of tensor t of a gradient list, from its own seed.  With
    `out` given, the draw is written into it (no new allocation kept)."""
    import torch
    g = torch.Generator(device=device).manual_seed(per_tensor_seed(seed, t, num_ranks, r))
    x = _torch_draw(torch, g, tuple(shape), dtype, dist, sigma, device)
    if out is not None:
        out.copy_(x)
        return out
    return x
