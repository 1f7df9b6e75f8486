"""Routed MoE decode layer: top-k routing, per-expert gate_up -> SiLU*up -> down, weighted combine.

Test infrastructure (see the package docstring).

[Sionic] intro: each token activates only its top-8 experts, and each
activated expert's weights are read once from HBM per forward.  [Sionic] §5 and
§6: a verify pass over several draft tokens (or a batch) reads each weight once
for all of them.  [M1]: a 256-expert MoE with a 2048-wide hidden state.
[CMP]: the routed experts are resident in HBM.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits, bf16_bits_to_f64
from .linear import gemv_fp8, silu_mul
from .quant import act_quant_fp8


def route_topk(logits, top_k: int = 8):
    """Top-k experts per token and their routing weights.

    Reading taken (the pages only say top-8): experts are taken in descending
    logit order, equal logits going to the lower expert id; the weights are a
    softmax over the k selected logits only, w_j = exp(l_j - l_0) / sum_i
    exp(l_i - l_0), in float64.  Logits must be finite.

    Returns (ids int64 [M, k] in slot order, weights float64 [M, k]).
    """
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float32))
    M, E = lg.shape
    assert 1 <= top_k <= E
    assert np.all(np.isfinite(lg)), "router logits must be finite"
    ids = np.empty((M, top_k), dtype=np.int64)
    wts = np.empty((M, top_k), dtype=np.float64)
    for m in range(M):
        taken = np.zeros(E, dtype=bool)
        for j in range(top_k):
            best = -1
            for e in range(E):                       # plain selection: strictly greater wins,
                if taken[e]:                         # so the lowest id keeps a tie
                    continue
                if best < 0 or lg[m, e] > lg[m, best]:
                    best = e
            taken[best] = True
            ids[m, j] = best
        sel = lg[m, ids[m]].astype(np.float64)
        ex = np.exp(sel - sel[0])
        wts[m] = ex / ex.sum()
    return ids, wts


def router_logits(x_bf16_bits, wr_bf16_bits) -> np.ndarray:
    """Router logits l[m, e] = sum_k x[m, k] * Wr[e, k], float64.

    [CMP], section on the 3.05bpw quality (the per-tensor bit allocation of the
    4.05bpw build): the router stays at native precision while the experts are
    quantised.  Reading taken: the router is a bf16 [E, H] weight applied to the
    bf16 layer input (no FP8 quantisation, no bias); the oracle returns the
    exact products summed in float64.  Which experts a token takes is decided
    on the logits the kernel computed (route_topk applied to them): near-equal
    logits may order differently under another summation order.
    """
    x = bf16_bits_to_f64(np.atleast_2d(np.asarray(x_bf16_bits, dtype=np.uint16)))
    w = bf16_bits_to_f64(np.atleast_2d(np.asarray(wr_bf16_bits, dtype=np.uint16)))
    assert x.shape[1] == w.shape[1]
    return x @ w.T


def union_of_experts(ids) -> np.ndarray:
    """Sorted distinct expert ids routed by any token of the call (#U = len)."""
    return np.unique(np.asarray(ids).reshape(-1))


def moe_layer(x_bf16_bits, expert, *, logits=None, ids=None, weights=None, top_k: int = 8, shared=None):
    """One routed MoE layer for M tokens, with an optional shared expert.

    ``expert(e)`` returns the quantised bank entry of expert e as
    (q13 uint8 [2I, H], s13 fp32 [2I, H/128], q2 uint8 [H, I], s2 fp32 [H, I/128]),
    gate rows first in q13.  Either ``logits`` [M, E] or (``ids``, ``weights``)
    [M, k] are given.

    Per token m and slot j (expert e = ids[m, j]):
      xq  = live FP8 quantisation of x[m]
      g|u = gate_up_e(xq)                       (float64, unrounded)
      h   = silu(g) * u                         (float64, unrounded)
      hq  = live FP8 quantisation of bf16(h)    (h crosses to the down GEMV in bf16)
      y   = down_e(hq)                          (float64)
      out[m] = sum_j w[m, j] * y_j              (float64, j in slot order)

    Reading taken: h is handed to the down projection as bf16 and re-quantised
    live exactly like the layer input (the pages fix neither).

    ``shared`` (optional) is a shared expert in the layout of ``expert(e)``:
    [CMP], section on the 3.05bpw quality, lists shared experts beside the
    routed ones (kept at more bits).  Reading taken: every token runs it
    through the same gate_up -> SiLU*up -> bf16 h -> live re-quant -> down
    chain, and its output is added with weight 1 after the routed slots,
    out[m] = sum_j w[m, j] * y_j + y_shared (float64).  Its intermediates are
    returned as ``sh_h``, ``sh_h_bits``, ``sh_hq``, ``sh_hs`` [M, I] (and
    ``sh_hs`` [M, I/128]), ``sh_gate``/``sh_up``/``sh_S_gate``/``sh_S_up``;
    ``S`` then also holds sum_k |hq~_k| |w2~_nk| of the shared expert.

    Returns a dict with ``out`` float64 [M, H] (unrounded), ``S`` [M, H]
    (sum_j |w_j| * sum_k |hq~_k| |w2~_nk|), ``ids``, ``weights``, and the
    per-(token, slot) intermediates ``h`` [M, k, I], ``h_bits`` (bf16),
    ``hq`` [M, k, I], ``hs`` [M, k, I/128], ``S_gate``/``S_up`` [M, k, I],
    ``gate``/``up`` [M, k, I].
    """
    xb = np.atleast_2d(np.asarray(x_bf16_bits, dtype=np.uint16))
    M, H = xb.shape
    if logits is not None:
        ids, weights = route_topk(logits, top_k)
    ids = np.asarray(ids, dtype=np.int64).reshape(M, -1)
    weights = np.asarray(weights, dtype=np.float64).reshape(M, -1)
    k = ids.shape[1]

    qx, sx = act_quant_fp8(xb)
    out = np.zeros((M, H), dtype=np.float64)
    S = np.zeros((M, H), dtype=np.float64)
    res = {}
    for e in union_of_experts(ids):
        q13, s13, q2, s2 = expert(int(e))
        I = q13.shape[0] // 2
        for m, j in zip(*np.nonzero(ids == e)):
            y13, s13err = gemv_fp8(qx[m:m + 1], sx[m:m + 1], q13, s13)
            h = silu_mul(y13, I)[0]
            hb = bf16_bits(h)
            hq, hs = act_quant_fp8(hb[None, :])
            y2, s2err = gemv_fp8(hq, hs, q2, s2)
            res[(m, j)] = (h, hb, hq[0], hs[0], y13[0], s13err[0], y2[0], s2err[0])

    I = next(iter(res.values()))[0].shape[0]
    shp = (M, k, I)
    h_all = np.zeros(shp); hb_all = np.zeros(shp, np.uint16); hq_all = np.zeros(shp, np.uint8)
    hs_all = np.zeros((M, k, I // 128), np.float32)
    gate = np.zeros(shp); up = np.zeros(shp); sg = np.zeros(shp); su = np.zeros(shp)
    for m in range(M):
        for j in range(k):                        # slot order
            h, hb, hq, hs, y13, e13, y2, e2 = res[(m, j)]
            out[m] += weights[m, j] * y2
            S[m] += abs(weights[m, j]) * e2
            h_all[m, j], hb_all[m, j], hq_all[m, j], hs_all[m, j] = h, hb, hq, hs
            gate[m, j], up[m, j] = y13[:I], y13[I:]
            sg[m, j], su[m, j] = e13[:I], e13[I:]
    res_out = {"out": out, "S": S, "ids": ids, "weights": weights, "h": h_all, "h_bits": hb_all,
               "hq": hq_all, "hs": hs_all, "gate": gate, "up": up, "S_gate": sg, "S_up": su,
               "xq": qx, "xs": sx}
    if shared is not None:
        q13, s13, q2, s2 = shared
        Is = q13.shape[0] // 2
        keys = ("sh_h", "sh_h_bits", "sh_hq", "sh_hs", "sh_gate", "sh_up", "sh_S_gate", "sh_S_up")
        acc = {k: [] for k in keys}
        for m in range(M):                        # after the routed slots of token m
            y13, s13err = gemv_fp8(qx[m:m + 1], sx[m:m + 1], q13, s13)
            h = silu_mul(y13, Is)[0]
            hb = bf16_bits(h)
            hq, hs = act_quant_fp8(hb[None, :])
            y2, s2err = gemv_fp8(hq, hs, q2, s2)
            out[m] += y2[0]
            S[m] += s2err[0]
            for k, v in zip(keys, (h, hb, hq[0], hs[0], y13[0, :Is], y13[0, Is:], s13err[0, :Is], s13err[0, Is:])):
                acc[k].append(v)
        for k in keys:
            res_out[k] = np.stack(acc[k])
    return res_out
