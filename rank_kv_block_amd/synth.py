"""Seeded synthetic inputs: queries, keys, block tables, planted-block choices.

This module only draws random numbers and shapes them; it holds none of the
predictor's arithmetic, so the oracle and the HIP path can both consume what it
makes.  Every draw is reproducible from (seed, device): torch's counter-based
generators on the GPU for bulk tensors, its CPU generator for permutations and
index samples.
"""

import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, seed, device):
    """N(0, 1) values rounded to bf16."""
    return torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32).to(torch.bfloat16)


def student_t3_bf16(shape, seed, device):
    """Standard Student-t, 3 degrees of freedom (variance 3): z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), in bf16."""
    z = torch.randn((4, *shape), generator=_gen(seed, device), device=device, dtype=torch.float32)
    chi2 = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
    return (z[0] / torch.sqrt(chi2)).to(torch.bfloat16)


def permutation(n, seed):
    """A seeded permutation of 0..n-1 (int32, CPU)."""
    return torch.randperm(n, generator=_gen(seed, "cpu")).to(torch.int32)


def sample_sorted(n, k, seed):
    """k distinct indices from 0..n-1, ascending (int64, CPU)."""
    return torch.randperm(n, generator=_gen(seed, "cpu"))[:k].sort().values
