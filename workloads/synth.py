"""Seeded synthetic workloads for batch-1 / small-M quantized-MoE decode.

Shapes follow the decode workloads this repository measures:

* ``FP8_GEMV_SMALL``  dense FP8 GEMV, M=1, K=512, N=256.
* ``FP8_GATE_UP``     one expert gate_up at batch 1, K=6144, N=2x2048 (gate||up).
* ``MOE_LAYER``       routed MoE layer, 256 experts, hidden 6144, expert
                      intermediate 2048, top-8 of N(0,1) router logits.
* ``MOE_VERIFY``      the same layer for M in {1,2,4,8} draft tokens whose
                      logits share an equicorrelated component (rho = 0.5).
* ``MOE_LAYER`` extras: bf16 router weights [E, H] (N(0,1)/sqrt(H+800), so the
                      logits come out near N(0,1)) and a shared expert drawn
                      like a routed one (tensor keys T_SH13 / T_SH2).
* ``Q4_STACK``        int4 g32 dense linears K=5120 with N in
                      {5120, 2x17408 (gate||up), 17408->5120}.

Value distributions: activations N(0,1) with two outlier channels scaled x20
(FP8 workloads; the int4 stack has no outliers), master weights 0.02*N(0,1) in
fp32, router logits N(0,1).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "FP8_GEMV_SMALL", "FP8_GATE_UP", "MOE_LAYER", "MOE_VERIFY", "Q4_STACK",
    "T_X", "T_W", "T_W13", "T_W2", "T_LOGITS", "T_OUTLIER", "T_ROUTER", "T_SH13", "T_SH2",
    "router_weights_bf16",
    "LM_HEAD", "generator", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "activation_bf16", "master_weights", "router_logits", "verify_logits",
    "MoEShape", "MOE_SHAPE", "MOE_TP8_SHAPE", "LM_HEAD_V", "Q4_SHAPES", "torch_seed", "master_weights_torch",
]

# workload keys (first spawn-key component)
FP8_GEMV_SMALL = 0
FP8_GATE_UP = 1
MOE_LAYER = 2
MOE_VERIFY = 3
Q4_STACK = 4
LM_HEAD = 5

# tensor keys (second spawn-key component)
T_X = 0
T_W = 1
T_W13 = 2
T_W2 = 3
T_LOGITS = 4
T_OUTLIER = 5
T_ROUTER = 6      # router weights (bf16)
T_SH13 = 7        # shared expert gate||up
T_SH2 = 8         # shared expert down


class MoEShape:
    """Routed-expert bank geometry: E experts, hidden H, intermediate I, top_k."""

    def __init__(self, E: int, H: int, I: int, top_k: int):
        self.E, self.H, self.I, self.top_k = E, H, I, top_k

    def __repr__(self) -> str:
        return f"MoEShape(E={self.E}, H={self.H}, I={self.I}, top_k={self.top_k})"


MOE_SHAPE = MoEShape(E=256, H=6144, I=2048, top_k=8)
# one rank's share of the same layer under 8-way tensor parallelism (I split 8 ways)
MOE_TP8_SHAPE = MoEShape(E=256, H=6144, I=256, top_k=8)
# LM-head GEMV: hidden 6144 to a vocabulary of LM_HEAD_V rows (a parameter: the
# pages give no vocabulary size)
LM_HEAD_V = 151552

# (K, N, silu_mul) for the three linears of one int4 decoder block
Q4_SHAPES = ((5120, 5120, False), (5120, 2 * 17408, True), (17408, 5120, False))


def generator(workload: int, tensor: int, expert: int = 0, seed: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one tensor (one expert) of one workload."""
    ss = np.random.SeedSequence(seed, spawn_key=(int(workload), int(tensor), int(expert)))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the 16-bit patterns.

    Used only to materialise the bf16 activation inputs.  Inputs are finite.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    b = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activation_bf16(M: int, K: int, *, workload: int, seed: int = 0, outliers: int = 2,
                    outlier_scale: float = 20.0) -> np.ndarray:
    """bf16 activations [M,K] ~ N(0,1); ``outliers`` channels (shared by all rows)
    are multiplied by ``outlier_scale`` before rounding to bf16.  Returns uint16 bits."""
    x = generator(workload, T_X, 0, seed).standard_normal((M, K), dtype=np.float32)
    if outliers:
        ch = generator(workload, T_OUTLIER, 0, seed).choice(K, size=outliers, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def master_weights(N: int, K: int, *, workload: int, tensor: int = T_W, expert: int = 0,
                   seed: int = 0, sigma: float = 0.02, out: np.ndarray | None = None) -> np.ndarray:
    """fp32 master weights [N,K] = fp32(sigma * N(0,1)) for one tensor of one expert."""
    g = generator(workload, tensor, expert, seed)
    if out is None:
        out = np.empty((N, K), dtype=np.float32)
    g.standard_normal(out=out.reshape(-1), dtype=np.float32)
    out *= np.float32(sigma)
    return out


def router_logits(M: int, E: int, *, workload: int, seed: int = 0, draw: int = 0) -> np.ndarray:
    """Independent N(0,1) router logits [M,E] (fp32); ``draw`` selects one of many
    pre-generated routing draws."""
    return generator(workload, T_LOGITS, draw, seed).standard_normal((M, E), dtype=np.float32)


def verify_logits(M: int, E: int, *, rho: float = 0.5, workload: int = MOE_VERIFY, seed: int = 0,
                  draw: int = 0) -> np.ndarray:
    """Equicorrelated logits for M draft tokens: l_m = sqrt(rho)*s + sqrt(1-rho)*e_m with a
    shared s ~ N(0,1)^E and independent e_m ~ N(0,1)^E (fp32)."""
    g = generator(workload, T_LOGITS, draw, seed)
    s = g.standard_normal(E)
    e = g.standard_normal((M, E))
    return (np.sqrt(rho) * s[None, :] + np.sqrt(1.0 - rho) * e).astype(np.float32)


def router_weights_bf16(E: int, H: int, *, workload: int = MOE_LAYER, seed: int = 0) -> np.ndarray:
    """bf16 router weights [E, H] = bf16(N(0,1) / sqrt(H + 800)) as uint16 bits: with the
    activation recipe (N(0,1) plus two channels x20) the logits come out near N(0,1)."""
    g = generator(workload, T_ROUTER, 0, seed)
    w = g.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H + 800.0))
    return f32_to_bf16_bits(w)


def torch_seed(workload: int, tensor: int, expert: int = 0, seed: int = 0) -> int:
    """64-bit seed for torch's device generator, derived from the same spawn key."""
    ss = np.random.SeedSequence(seed, spawn_key=(int(workload), int(tensor), int(expert)))
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def master_weights_torch(N: int, K: int, *, workload: int, tensor: int = T_W, expert: int = 0,
                         seed: int = 0, sigma: float = 0.02, device: str = "cuda"):
    """fp32 master weights [N,K] = fp32(sigma * N(0,1)) drawn on the device by torch's
    seeded generator (used for the 10 GB expert bank, where host generation is slow).
    The same (workload, tensor, expert, seed) always gives the same tensor on a given
    device type; copying it to the host gives the CPU side the identical values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(workload, tensor, expert, seed))
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    return w.mul_(sigma)
