"""Seeded synthetic inputs for the fused all-reduce + residual + RMSNorm epilogue.

This module only draws random values and stores them as bf16 bit patterns (numpy ``uint16``);
it holds none of the operation's arithmetic. The HIP path and the oracle both take their inputs
from here, so a test can hand the same bits to both.

Workloads are those of the tensor-parallel decode and prefill shapes the pages measure (N partial
sums of a bf16 ``(tokens, hidden)`` activation, a bf16 residual of the same shape and a bf16
weight of length ``hidden``). The pages print no shapes or value distributions, so the draws are
synthetic:

* ``normal``: inputs N(0, 0.5^2), residual N(0, 1), weight 1 + 0.1 * N(0, 1);
* ``stress``: inputs Student-t(3) * 4, with about 1 % of rows all zero (in every input) and about
  1 % of rows set to +-bf16(3e4) with a fair random sign per element; residual and weight as above.

Recipe: ``numpy.random.default_rng(seed)``; draws are made in the order inputs[0..n-1], residual,
weight (then, for ``stress``, the per-row category and sign draws come first); draws are binary32
and are rounded to bf16 by torch's CPU conversion (round to nearest, ties to even).
"""
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Problem", "make_problem", "to_bf16_bits", "stress_m_values", "WORKLOADS"]


def to_bf16_bits(values):
    """bf16 bit patterns (uint16) of a float array, by torch's CPU float32 -> bfloat16 cast."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclass
class Problem:
    """One fused call's inputs as raw bf16 bits: ``inputs`` is a list of n arrays (m, hidden)."""
    inputs: list
    residual: np.ndarray
    weight: np.ndarray
    eps: float
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def n(self):
        return len(self.inputs)

    @property
    def m(self):
        return self.residual.shape[0]

    @property
    def hidden(self):
        return self.residual.shape[1]


def _normal(rng, shape, sigma, mean=0.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make_problem(n, m, hidden, *, seed=0, eps=1e-6, dist="normal", input_sigma=0.5, name=""):
    """Draw one problem of n inputs of shape (m, hidden); see the module docstring for ``dist``."""
    if dist not in ("normal", "stress"):
        raise ValueError(f"unknown dist {dist!r}")
    rng = np.random.default_rng(seed)
    shape = (m, hidden)
    meta = {"seed": seed, "dist": dist}
    if dist == "normal":
        inputs = [to_bf16_bits(_normal(rng, shape, input_sigma)) for _ in range(n)]
    else:
        u = rng.random(m)
        zero_rows = np.nonzero(u < 0.01)[0]
        big_rows = np.nonzero((u >= 0.01) & (u < 0.02))[0]
        big = np.float32(3e4)
        inputs = []
        for _ in range(n):
            x = (rng.standard_t(3, size=shape) * 4.0).astype(np.float32)
            signs = rng.random((len(big_rows), hidden)) < 0.5
            x[big_rows] = np.where(signs, -big, big)
            x[zero_rows] = 0.0
            inputs.append(to_bf16_bits(x))
        meta.update(zero_rows=zero_rows.tolist(), big_rows=big_rows.tolist())
    residual = to_bf16_bits(_normal(rng, shape, 1.0))
    weight = to_bf16_bits(_normal(rng, (hidden,), 0.1, mean=1.0))
    return Problem(inputs, residual, weight, float(eps), name=name, meta=meta)


def stress_m_values(seed=0, count=16):
    """Row counts of the stress workload: ``count`` draws from 1..2048, plus 1, 16, 17 and 2048
    (16/17 straddle the row count at which the automatic path choice changes for n > 4)."""
    rng = np.random.default_rng(seed)
    drawn = rng.integers(1, 2049, count).tolist()
    return sorted(set(drawn) | {1, 16, 17, 2048})


# The workloads of the decode and prefill shapes (n, hidden, row counts, eps, value distribution,
# path). "path" is the path each workload is specified for: 1 one-stage, 2 two-stage, 0 automatic.
WORKLOADS = {
    "small_n4_h4096": dict(n=4, hidden=4096, ms=[8], eps=1e-6, dist="normal", paths=[1]),
    "decode_n8_h7168": dict(n=8, hidden=7168, ms=[1, 2, 4, 8, 16, 32], eps=1e-6, dist="normal",
                            paths=[1]),
    "mid_n4_h7168": dict(n=4, hidden=7168, ms=[64, 256, 1024, 4096], eps=1e-6, dist="normal",
                         paths=[2]),
    "prefill_n8_h8192": dict(n=8, hidden=8192, ms=[8192], eps=1e-5, dist="normal", paths=[1, 2]),
    "stress_n8_h2880": dict(n=8, hidden=2880, ms=None, eps=1e-6, dist="stress", paths=[0]),
    "bandwidth_n8_h7168": dict(n=8, hidden=7168, ms=[2048, 4096, 8192], eps=1e-6, dist="normal",
                               paths=[1, 2]),
}
