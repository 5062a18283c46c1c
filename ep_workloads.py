"""Seeded synthetic workloads for the MoE dispatch / combine path.

This module only draws inputs: hidden states, router top-k indices and gate
weights, and a stand-in for expert outputs.  It holds none of the path's
arithmetic (no counting, placement, quantisation or reduction), so the tests
and the benchmark can feed the same arrays to the HIP library and to the CPU
oracle without the two sharing code.

No public dataset is involved: the pages describe MoE layers with hidden size
7168, top-8 routing over 256 experts, 4096 tokens per rank and group-limited
gates ("Deep Dive - DeepEP", sections "V2's single interface: ElasticBuffer"
and "Logical bandwidth is not a NIC counter"), and these generators reproduce
those shapes and value distributions.

Draw order per workload (numpy PCG64 ``default_rng(seed)``):
  1. x: standard normal fp32 [T, H] times sigma, rounded to bf16 by torch.
  2. routes (uniform distinct / Zipf without replacement / group-limited).
  3. gate logits, standard normal fp32 [T, k] (group-limited: the router
     scores of the chosen experts), softmax in float64, stored as fp32.
  4. mask (Skewed only): exactly floor(frac * T * k) slots set to -1.
  5. y (optional): standard normal fp32 [capacity, H] rounded to bf16, the
     stand-in for expert outputs consumed by combine.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int          # T
    hidden: int              # H
    num_topk: int            # k
    num_experts: int         # E
    num_ranks: int           # R (logical ranks, E % R == 0)
    fp8: bool                # dispatch payload: FP8 e4m3 (+ fp32 scales) or bf16
    routing: str             # "uniform" | "zipf" | "group_limited"
    sigma: float = 1.0       # x ~ N(0, sigma^2)
    seed: int = 0
    alignment: int = 1       # A
    mask_frac: float = 0.0   # fraction of slots set to -1 (exact count)
    zipf_s: float = 1.2
    num_groups: int = 0      # group-limited routing: expert groups
    topk_groups: int = 0     # group-limited routing: groups kept per token

    @property
    def capacity(self) -> int:
        """Worst-case receive rows: every slot valid, every segment padded."""
        return self.num_tokens * self.num_topk + self.num_experts * (self.alignment - 1)

    def describe(self) -> dict:
        return dataclasses.asdict(self)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 128, 2, 8, 2, False, "uniform", seed=1),
    "decode": Workload("decode", 128, 7168, 8, 256, 8, False, "uniform", seed=2),
    "prefill": Workload("prefill", 4096, 7168, 8, 256, 8, True, "uniform", seed=3),
    "skewed": Workload("skewed", 8192, 4096, 6, 64, 8, False, "zipf", seed=4,
                       mask_frac=0.05),
    "large": Workload("large", 16384, 7168, 8, 256, 8, True, "group_limited",
                      sigma=math.sqrt(2.0), seed=5, num_groups=8, topk_groups=4),
}


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns through torch's own conversion (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_CHUNK = 1 << 22


def normal_bf16(rng, shape, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits of standard-normal fp32 draws times sigma (in fp32), drawn
    in fixed-size pieces straight into the output.  The stream is the one a
    single ``rng.standard_normal(shape, dtype=float32)`` call would draw."""
    import torch

    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    buf = np.empty(min(_CHUNK, flat.size), np.float32)
    tout = torch.from_numpy(flat.view(np.int16))
    for lo in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - lo)
        piece = buf[:n]
        rng.standard_normal(n, dtype=np.float32, out=piece)
        if sigma != 1.0:
            piece *= np.float32(sigma)
        tout[lo:lo + n] = torch.from_numpy(piece).to(torch.bfloat16).view(torch.int16)
    return out


def _softmax64(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def _uniform_routes(rng, T, E, k):
    # argsort of iid uniforms is a uniformly random permutation per token;
    # its first k entries are a uniform k-subset in random order.
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def _zipf_routes(rng, T, E, k, s):
    # Successive draws without replacement with p_i ~ (i+1)^-s, done as
    # Gumbel-top-k (equivalent in distribution); slot order = draw order.
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def _group_limited_routes(rng, T, E, k, groups, keep):
    # Router scores s ~ N(0,1); a group's score is its best expert score; the
    # token keeps its `keep` best groups (ties -> lower group index) and picks
    # its top-k experts by score inside them (ties -> lower expert index).
    s = rng.standard_normal((T, E), dtype=np.float32)
    per = E // groups
    gscore = s.reshape(T, groups, per).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :keep]
    allowed = np.zeros((T, groups), bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    masked = np.where(np.repeat(allowed, per, axis=1), s, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :k].astype(np.int32)
    chosen = np.take_along_axis(s, idx, axis=1)
    return idx, chosen


def generate(w: Workload, with_y: bool = True) -> dict:
    """Draw one batch.  Returns numpy arrays:
    x (uint16 bf16 bits [T,H]), topk_idx (int32 [T,k]), topk_weights
    (float32 [T,k]) and, with ``with_y``, y (uint16 bf16 bits [capacity,H])."""
    rng = np.random.default_rng(w.seed)
    T, H, k, E = w.num_tokens, w.hidden, w.num_topk, w.num_experts
    x = normal_bf16(rng, (T, H), w.sigma)
    if w.routing == "uniform":
        idx = _uniform_routes(rng, T, E, k)
        logits = rng.standard_normal((T, k), dtype=np.float32)
    elif w.routing == "zipf":
        idx = _zipf_routes(rng, T, E, k, w.zipf_s)
        logits = rng.standard_normal((T, k), dtype=np.float32)
    elif w.routing == "group_limited":
        idx, logits = _group_limited_routes(rng, T, E, k, w.num_groups, w.topk_groups)
    else:
        raise ValueError(w.routing)
    weights = _softmax64(logits)
    if w.mask_frac > 0:
        n = int(math.floor(w.mask_frac * T * k))
        flat = rng.choice(T * k, size=n, replace=False)
        idx = idx.copy()
        idx.reshape(-1)[flat] = -1
    out = dict(x=x, topk_idx=np.ascontiguousarray(idx, np.int32),
               topk_weights=np.ascontiguousarray(weights, np.float32))
    if with_y:
        out["y"] = normal_bf16(rng, (w.capacity, H))
    return out


def random_routes(rng, T: int, E: int, k: int, mask_prob: float = 0.0) -> np.ndarray:
    """Small random route tables for brute-force tests: distinct experts per
    token, each slot independently set to -1 with probability mask_prob."""
    idx = _uniform_routes(rng, T, E, k)
    if mask_prob > 0:
        idx = np.where(rng.random((T, k)) < mask_prob, -1, idx).astype(np.int32)
    return idx
