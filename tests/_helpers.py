"""Shared test helpers: GPU availability, seeded uploads, tolerance checks.

Tolerances (the contract of the decode path):
* quantised activation codes and scales: bit-exact against the oracle;
* GEMV outputs: |y_gpu - y_oracle| <= 2e-3 * S per element, S = sum_k |x~_k w~_k|,
  compared with the unrounded float64 oracle value;
* SiLU(gate)*up outputs: 2e-3 * (1.1 |u| S_g + |silu(g)| S_u) + 2^-8 |h|
  (first-order propagation of the GEMV bound through silu(g)*u, whose
  derivative in g is below 1.1 in magnitude, plus the bf16 output rounding).
"""
import numpy as np
import pytest

REL = 2e-3


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def bf16_to_np(t):
    """bf16 torch tensor -> float64 numpy (exact)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def np_bf16_bits_to_torch(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def assert_gemv_close(y_gpu, y_ref, S, what=""):
    err = np.abs(y_gpu - y_ref)
    bound = REL * S
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside 2e-3*S; worst at {i}: "
                             f"gpu={y_gpu[i]!r} ref={y_ref[i]!r} S={S[i]!r}")
    return float((err / np.maximum(S, 1e-300)).max())


def silu_bound(g, u, Sg, Su, h):
    sg = g / (1.0 + np.exp(-g))
    return REL * (1.1 * np.abs(u) * Sg + np.abs(sg) * Su) + 2.0 ** -8 * np.abs(h)


def assert_silu_close(h_gpu, h_ref, g, u, Sg, Su, what=""):
    err = np.abs(h_gpu - h_ref)
    bound = silu_bound(g, u, Sg, Su, h_ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the SiLU bound; worst at {i}: "
                             f"gpu={h_gpu[i]!r} ref={h_ref[i]!r} bound={bound[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())
