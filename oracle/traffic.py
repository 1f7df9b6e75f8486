"""Closed forms for weight traffic: bytes per call, per token, per accepted token.

Test infrastructure (see the package docstring).

[Sionic] intro: decoding one token streams every active weight from HBM once,
so time per forward is at least bytes / bandwidth (the page's example: about
6.65 GB per GPU per token, 0.83 ms at 8 TB/s).  [Sionic] §5 table: under
multi-token prediction one weight read confirms as many tokens as the mean
acceptance length L, so traffic per token is bytes per forward / L
(6.65 GB -> about 1.9 GB at L = 3.5 and about 0.67 GB at L = 10).
"""
from __future__ import annotations

FP8_BLOCK = 128
Q4_GROUP = 32


def fp8_weight_bytes(N: int, K: int) -> int:
    """E4M3 codes plus one fp32 scale per 128-wide block of each row."""
    return N * K + 4 * N * (K // FP8_BLOCK)


def q4_weight_bytes(N: int, K: int) -> int:
    """Packed nibbles plus one fp16 scale per 32-wide group of each row."""
    return N * K // 2 + 2 * N * (K // Q4_GROUP)


def fp8_linear_bytes(M: int, K: int, N: int, silu_mul: bool = False) -> int:
    """Algorithmic bytes of one FP8 GEMV call: weights + scales + bf16 x + bf16 y."""
    n_out = N // 2 if silu_mul else N
    return fp8_weight_bytes(N, K) + 2 * M * K + 2 * M * n_out


def q4_linear_bytes(M: int, K: int, N: int, silu_mul: bool = False) -> int:
    n_out = N // 2 if silu_mul else N
    return q4_weight_bytes(N, K) + 2 * M * K + 2 * M * n_out


def expert_bytes(H: int, I: int) -> int:
    """One routed expert: gate_up [2I, H] plus down [H, I], FP8 with scales."""
    return fp8_weight_bytes(2 * I, H) + fp8_weight_bytes(H, I)


def moe_call_bytes(M: int, n_union: int, H: int, I: int, E: int) -> int:
    """Bytes one MoE decode call must move: each expert in the union of the M
    tokens' routes streamed once, plus bf16 input and output rows and fp32 logits."""
    return n_union * expert_bytes(H, I) + M * (2 * H + 2 * H + 4 * E)


def per_token(bytes_per_call: float, M: int) -> float:
    return bytes_per_call / M


def per_accepted_token(bytes_per_forward: float, acceptance_length: float) -> float:
    """[Sionic] §5: traffic per confirmed token = traffic per forward / L."""
    return bytes_per_forward / acceptance_length


def bandwidth_floor_seconds(bytes_per_forward: float, bandwidth_bytes_per_s: float) -> float:
    """[Sionic] intro: lower bound on a forward = bytes / bandwidth."""
    return bytes_per_forward / bandwidth_bytes_per_s


def fraction_of_peak(achieved: float, peak: float) -> float:
    return achieved / peak
