"""GPU parity of moe_decode_layer (one launch: route, live act-quant, gate_up +
SiLU*up, h re-quant, down, weighted combine) against the oracle.

Expected values come only from the oracle run on the same seeded inputs: the
master weights are drawn once and quantised independently by the library
(on the GPU) and by the oracle (on the CPU); the test first checks that both
codings agree bit for bit.

Checks per call: routing ids exact, routing weights within 1e-6, h within the
SiLU bound, the live re-quantisation of h bit-exact (the oracle's quantiser
applied to the kernel's own bf16 h must give the kernel's codes and scales,
for every (token, slot) pair and every shared-expert pair), output within
2e-3 * S per element (S = sum_j |w_j| sum_k |h~_k w2~_nk| from the oracle).
The oracle's end-to-end h codes (quantised from its own fp64-derived h) may
still differ in a few places, because h crosses a bf16 rounding computed from
fp32 on the GPU and from fp64 in the oracle; that share is held to at most
2e-3 of the codes.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from _helpers import assert_gemv_close, assert_silu_close, bf16_to_np, need_gpu, np_bf16_bits_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


@pytest.fixture(params=["barrier", "stream"])
def path(request):
    """Run the test with each of the two layer kernels (the library picks one
    by token count; PQ_MOE_PATH forces it)."""
    old = os.environ.get("PQ_MOE_PATH")
    os.environ["PQ_MOE_PATH"] = request.param
    yield request.param
    if old is None:
        del os.environ["PQ_MOE_PATH"]
    else:
        os.environ["PQ_MOE_PATH"] = old


# Oracle codings of the experts drawn so far, shared by the tests of this
# module: (workload, seed, H, I, expert) -> (w13 codes, scales, w2 codes, scales)
_EXPERTS = {}


class Bank:
    """Expert bank with only the experts a test routes to filled in.

    Master weights are drawn per expert from ``workloads``; the GPU copy is
    quantised by the library, the oracle copy by the oracle, and the two are
    checked bit-equal the first time an expert is drawn.  Later tests that
    route to the same expert upload those verified bytes instead of
    quantising again."""

    def __init__(self, pq, E, H, I, workload=workloads.MOE_LAYER, seed=0):
        import torch
        self.pq, self.E, self.H, self.I, self.wl, self.seed = pq, E, H, I, workload, seed
        self.w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device="cuda")
        self.s13 = torch.ones((E, 2 * I, H // 128), dtype=torch.float32, device="cuda")
        self.w2 = torch.zeros((E, H, I), dtype=torch.uint8, device="cuda")
        self.s2 = torch.ones((E, H, I // 128), dtype=torch.float32, device="cuda")
        self.cpu = {}

    def fill(self, experts):
        import torch
        for e in sorted(set(int(v) for v in np.asarray(experts).ravel())):
            if e in self.cpu:
                continue
            key = (self.wl, self.seed, self.H, self.I, e)
            if key in _EXPERTS:
                o13, os13, o2, os2 = _EXPERTS[key]
                self.w13[e].copy_(torch.from_numpy(o13)); self.s13[e].copy_(torch.from_numpy(os13))
                self.w2[e].copy_(torch.from_numpy(o2)); self.s2[e].copy_(torch.from_numpy(os2))
                self.cpu[e] = _EXPERTS[key]
                continue
            m13 = workloads.master_weights(2 * self.I, self.H, workload=self.wl, tensor=workloads.T_W13,
                                           expert=e, seed=self.seed)
            m2 = workloads.master_weights(self.H, self.I, workload=self.wl, tensor=workloads.T_W2,
                                          expert=e, seed=self.seed)
            q13, s13 = self.pq.quantize_fp8(torch.from_numpy(m13).cuda())
            q2, s2 = self.pq.quantize_fp8(torch.from_numpy(m2).cuda())
            self.w13[e].copy_(q13); self.s13[e].copy_(s13); self.w2[e].copy_(q2); self.s2[e].copy_(s2)
            o13, os13 = oracle.block_quant_fp8(m13)
            o2, os2 = oracle.block_quant_fp8(m2)
            assert np.array_equal(q13.cpu().numpy(), o13) and np.array_equal(q2.cpu().numpy(), o2)
            assert np.array_equal(s13.cpu().numpy(), os13) and np.array_equal(s2.cpu().numpy(), os2)
            self.cpu[e] = (o13, os13, o2, os2)
            _EXPERTS[key] = self.cpu[e]
            if self.H * self.I >= (1 << 22):
                print(f"  [bank] expert {e} drawn and quantised ({len(self.cpu)} filled)", flush=True)

    def expert(self, e):
        return self.cpu[e]

    def shared(self):
        """A shared expert with the bank's shapes (drawn like a routed one under
        its own tensor keys); returns the GPU tensors, keeps the oracle's."""
        import torch
        m13 = workloads.master_weights(2 * self.I, self.H, workload=self.wl, tensor=workloads.T_SH13,
                                       seed=self.seed)
        m2 = workloads.master_weights(self.H, self.I, workload=self.wl, tensor=workloads.T_SH2, seed=self.seed)
        q13, s13 = self.pq.quantize_fp8(torch.from_numpy(m13).cuda())
        q2, s2 = self.pq.quantize_fp8(torch.from_numpy(m2).cuda())
        o13, os13 = oracle.block_quant_fp8(m13)
        o2, os2 = oracle.block_quant_fp8(m2)
        assert np.array_equal(q13.cpu().numpy(), o13) and np.array_equal(q2.cpu().numpy(), o2)
        self.sh_cpu = (o13, os13, o2, os2)
        return (q13, s13, q2, s2)


def h_bits(t):
    """bf16 tensor -> uint16 bit patterns (numpy), any shape."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_requant_bit_exact(h, hq, hs, what="h"):
    """The kernel's live re-quantisation of its own bf16 h equals the oracle's
    quantiser applied to the same bits: every code and every scale."""
    I = h.shape[-1]
    hb = h_bits(h).reshape(-1, I)
    qo, so = oracle.act_quant_fp8(hb)
    q = hq.cpu().numpy().reshape(-1, I)
    s = hs.cpu().numpy().reshape(-1, I // 128)
    bad = np.argwhere(q != qo)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ from the oracle's quantisation of the kernel's h, first {bad[:4].tolist()}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{what}: block scales differ from the oracle's"


def _check(pq, bank, x_bits, res, ref, M, k):
    ids = res["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), "routing ids differ"
    assert np.max(np.abs(res["topk_w"].cpu().numpy() - ref["weights"])) <= 1e-6
    I = bank.I
    if "h" in res:
        h = bf16_to_np(res["h"])
        assert_silu_close(h, ref["h"], ref["gate"], ref["up"], ref["S_gate"], ref["S_up"], "h")
        assert_requant_bit_exact(res["h"], res["hq"], res["hs"])
        hq = res["hq"].cpu().numpy()
        diff = np.mean(hq != ref["hq"])
        assert diff <= 2e-3, f"{diff:.2e} of h codes differ from the oracle"
    y = bf16_to_np(res["out"])
    return assert_gemv_close(y, ref["out"], ref["S"], f"out M={M}")


@pytest.mark.parametrize("M,E,H,I,k", [(1, 16, 512, 256, 4), (1, 16, 512, 128, 4), (2, 16, 640, 384, 4), (3, 24, 1024, 512, 8),
                                       (8, 32, 1024, 256, 8)])
def test_moe_small_routed(pq, path, M, E, H, I, k):
    import torch
    bank = Bank(pq, E, H, I, seed=M)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=M)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=M)
    ids, _ = oracle.route_topk(lg, k)
    bank.fill(ids)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=k, debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
    _check(pq, bank, x, res, ref, M, k)


def test_moe_given_routing_with_shared_experts(pq, path):
    import torch
    M, E, H, I, k = 4, 12, 512, 256, 3
    bank = Bank(pq, E, H, I, seed=9)
    ids = np.array([[5, 2, 9], [2, 5, 11], [0, 9, 2], [7, 5, 1]], np.int32)
    w = np.array([[0.5, 0.3, 0.2], [0.6, 0.3, 0.1], [0.4, 0.35, 0.25], [0.9, 0.05, 0.05]], np.float32)
    bank.fill(ids)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=9)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              topk_ids=torch.from_numpy(ids).cuda(), topk_w=torch.from_numpy(w).cuda(), debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, ids=ids, weights=w.astype(np.float64))
    assert_gemv_close(bf16_to_np(res["out"]), ref["out"], ref["S"], "given routing")
    assert_silu_close(bf16_to_np(res["h"]), ref["h"], ref["gate"], ref["up"], ref["S_gate"], ref["S_up"], "h")
    assert_requant_bit_exact(res["h"], res["hq"], res["hs"])


def test_moe_rows_bitwise_independent_of_M(pq):
    """A token's output in an M-token verify call equals the token decoded alone."""
    import torch
    M, E, H, I, k = 6, 20, 1024, 512, 8
    bank = Bank(pq, E, H, I, seed=4)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=4)
    lg = workloads.verify_logits(M, E, workload=workloads.MOE_LAYER, seed=4)
    bank.fill(oracle.route_topk(lg, k)[0])
    xt, lt = np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda()
    full = pq.moe_decode_layer(xt, bank.w13, bank.s13, bank.w2, bank.s2, logits=lt, top_k=k, debug=True)
    for m in range(M):
        one = pq.moe_decode_layer(xt[m:m + 1].contiguous(), bank.w13, bank.s13, bank.w2, bank.s2,
                                  logits=lt[m:m + 1].contiguous(), top_k=k, debug=True)
        assert torch.equal(one["out"][0].view(torch.int16), full["out"][m].view(torch.int16))
        assert torch.equal(one["hq"][0], full["hq"][m])
        assert torch.equal(one["topk_w"][0], full["topk_w"][m])


@pytest.mark.parametrize("M,I,H", [(1, 512, 1024), (3, 512, 1024), (8, 512, 1024), (1, 256, 1024), (2, 128, 1024),
                                   (1, 384, 1024), (3, 2048, 640), (1, 1536, 640), (8, 1024, 896)])
def test_moe_barrier_and_stream_kernels_agree_bitwise(pq, M, I, H):
    """Both layer kernels compute every h row and every output row with the same
    lane split and reduction order, so their results are bitwise equal; short
    down rows (I = 128, 256, 512), which the barrier kernel packs several to a
    step, reduce inside their lane segment in the same order, and longer rows,
    which both kernels carry two to a step, keep each row's order too (H = 640
    and 896 give blocks an odd number of down rows, so some steps carry one)."""
    import torch
    E, k = 24, 8
    bank = Bank(pq, E, H, I, seed=20 + M)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=20 + M)
    lg = workloads.verify_logits(M, E, workload=workloads.MOE_LAYER, seed=20 + M)
    bank.fill(oracle.route_topk(lg, k)[0])
    xt, lt = np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda()
    res = {}
    old = os.environ.get("PQ_MOE_PATH")
    try:
        for p in ("barrier", "stream"):
            os.environ["PQ_MOE_PATH"] = p
            res[p] = pq.moe_decode_layer(xt, bank.w13, bank.s13, bank.w2, bank.s2, logits=lt, top_k=k, debug=True)
            assert pq.workspace_check() == 0
    finally:
        if old is None:
            del os.environ["PQ_MOE_PATH"]
        else:
            os.environ["PQ_MOE_PATH"] = old
    a, b = res["barrier"], res["stream"]
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    assert torch.equal(a["h"].view(torch.int16), b["h"].view(torch.int16))
    assert torch.equal(a["hq"], b["hq"]) and torch.equal(a["hs"], b["hs"])
    if H != 1024:                          # ragged row counts: against the oracle too
        ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
        _check(pq, bank, x, a, ref, M, k)


@pytest.mark.parametrize("M,E,H,I,k,shared", [(1, 16, 1024, 512, 4, False), (2, 16, 640, 384, 4, True),
                                                (1, 256, 6144, 2048, 8, False)])
def test_moe_scale_windows_match_step_loads(pq, monkeypatch, M, E, H, I, k, shared):
    """The barrier kernel's gate_up reads its block scales from per-wave LDS
    windows (filled once per h row by buffer-to-LDS loads); with
    PQ_MOE_SCALES=step it loads them with every step's weights instead.  The
    products and their order are the same, so the results are bitwise equal:
    one chunk per row (four rows rotating through the windows), a ragged
    chunk with a shared expert, and the full-size layer."""
    import torch
    monkeypatch.setenv("PQ_MOE_PATH", "barrier")       # the windows belong to the barrier kernel
    cfg = pq.moe_layer_config(M, H, I, E, k, shared=shared)
    assert cfg["kernel"] == "barrier" and cfg["lds_bytes"] >= 16 * 2048, cfg     # the windows are laid out
    wl = workloads.MOE_LAYER
    bank = Bank(pq, E, H, I, workload=wl, seed=0 if H == 6144 else 40 + M)
    x = workloads.activation_bf16(M, H, workload=wl, seed=40 + M)
    lg = (workloads.router_logits(1, E, workload=wl) if H == 6144
          else workloads.verify_logits(M, E, workload=wl, seed=40 + M))
    ids, _ = oracle.route_topk(lg, k)
    bank.fill(ids)
    sh = bank.shared() if shared else None
    xt, lt = np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda()
    res = {}
    old = os.environ.get("PQ_MOE_SCALES")
    try:
        for mode in ("windows", "step"):
            if mode == "step":
                os.environ["PQ_MOE_SCALES"] = "step"
            res[mode] = pq.moe_decode_layer(xt, bank.w13, bank.s13, bank.w2, bank.s2, logits=lt, top_k=k,
                                            shared=sh, debug=True)
            assert pq.workspace_check() == 0
    finally:
        if old is None:
            os.environ.pop("PQ_MOE_SCALES", None)
        else:
            os.environ["PQ_MOE_SCALES"] = old
    a, b = res["windows"], res["step"]
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    assert torch.equal(a["h"].view(torch.int16), b["h"].view(torch.int16))
    if shared:
        assert torch.equal(a["sh_h"].view(torch.int16), b["sh_h"].view(torch.int16))
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k, shared=bank.sh_cpu if shared else None)
    _check(pq, bank, x, a, ref, M, k)
    if shared:
        _check_shared(a, ref)


def test_moe_deterministic_and_workspace_reuse(pq):
    """Repeated calls are bitwise identical, also interleaved with calls of other
    shapes on the same workspace (counters and the h exchange region must be
    left at zero; M = 1 runs the barrier kernel, M = 2 and 5 the stream kernel)."""
    import torch
    E, H, I, k = 16, 512, 256, 4
    bank = Bank(pq, E, H, I, seed=5)
    bank.fill(range(E))
    outs = {}
    for rep in range(6):
        for M in (1, 5, 2):
            x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=50 + M)
            lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=50 + M)
            r = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                                    logits=torch.from_numpy(lg).cuda(), top_k=k)
            if rep == 0:
                outs[M] = r["out"].clone()
                ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
                assert_gemv_close(bf16_to_np(r["out"]), ref["out"], ref["S"], f"M={M}")
            else:
                assert torch.equal(r["out"].view(torch.int16), outs[M].view(torch.int16))
    assert pq.workspace_check() == 0


def test_moe_bad_expert_id_is_reported(pq, path):
    import torch
    E, H, I = 8, 256, 128
    bank = Bank(pq, E, H, I, seed=6)
    bank.fill([0, 1])
    x = torch.zeros((1, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.tensor([[1, 99]], dtype=torch.int32, device="cuda")
    w = torch.tensor([[0.5, 0.5]], dtype=torch.float32, device="cuda")
    pq.moe_decode_layer(x, bank.w13, bank.s13, bank.w2, bank.s2, topk_ids=ids, topk_w=w)
    assert pq.workspace_check() == -8
    assert pq.workspace_check() == 0          # the record is cleared


def test_moe_watchdog_reports_timeout_and_next_call_is_clean(pq, path):
    """A zero spin budget (set from the host) makes waiting blocks give up
    instead of waiting: the call still ends, the timeout is reported, and the
    next call with the normal budget is correct."""
    import torch
    M, E, H, I, k = 1, 16, 2048, 1024, 4
    bank = Bank(pq, E, H, I, seed=7)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=7)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=7)
    bank.fill(oracle.route_topk(lg, k)[0])
    args = (np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2)
    os.environ["PQ_SPIN_LIMIT"] = "0"
    try:
        pq.moe_decode_layer(*args, logits=torch.from_numpy(lg).cuda(), top_k=k)
    finally:
        del os.environ["PQ_SPIN_LIMIT"]
    assert pq.workspace_check() in (0, -7)
    r = pq.moe_decode_layer(*args, logits=torch.from_numpy(lg).cuda(), top_k=k)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
    assert_gemv_close(bf16_to_np(r["out"]), ref["out"], ref["S"], "after timeout")


@pytest.mark.parametrize("M", [1, 4])
def test_moe_full_size_layer(pq, path, M):
    """256 experts, hidden 6144, intermediate 2048, top-8: the routed MoE layer at
    its real shape (M=1) and a 4-token verify call, every output checked."""
    import torch
    shp = workloads.MOE_SHAPE
    bank = Bank(pq, shp.E, shp.H, shp.I, workload=workloads.MOE_LAYER, seed=0)
    x = workloads.activation_bf16(M, shp.H, workload=workloads.MOE_LAYER if M == 1 else workloads.MOE_VERIFY)
    lg = (workloads.router_logits(1, shp.E, workload=workloads.MOE_LAYER) if M == 1
          else workloads.verify_logits(M, shp.E))
    ids, _ = oracle.route_topk(lg, shp.top_k)
    bank.fill(ids)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=shp.top_k, debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=shp.top_k)
    worst = _check(pq, bank, x, res, ref, M, shp.top_k)
    print(f"full-size M={M} ({path}): union {len(oracle.union_of_experts(ids))} experts, worst |err|/S {worst:.2e}")


@pytest.mark.parametrize("M,kernel,alias,layout", [(2, "stream", False, None), (2, "barrier", True, "barrier"),
                                                   (7, "stream", True, "split"), (8, "stream", True, "split"),
                                                   (8, "stream", True, "full")])
def test_moe_full_size_verify(pq, monkeypatch, M, kernel, alias, layout):
    """Speculative verify at the real shape (256 experts, hidden 6144,
    intermediate 2048, top-8, equicorrelated routing): M = 2 on the library's
    default kernel for two tokens (the stream kernel, x and h side by side)
    and on the barrier kernel (PQ_MOE_PATH=barrier: it always stages h over x,
    after its grid-wide release), M = 7 and 8 on the stream kernel, where x, h and the
    output partials do not fit side by side: by default ("split") the
    first h rows in union order sit apart from x and are staged while other
    waves still stream gate_up, and only the rest overwrite the quantised x;
    with PQ_MOE_ALIAS=full ("full") every h row does.  The test first checks
    that the library really takes that layout.  Every output element is
    checked, the re-quantised h bit for bit."""
    import torch
    shp = workloads.MOE_SHAPE
    if layout == "full":
        monkeypatch.setenv("PQ_MOE_ALIAS", "full")
    if layout == "barrier":
        monkeypatch.setenv("PQ_MOE_PATH", "barrier")
    cfg = pq.moe_layer_config(M, shp.H, shp.I, shp.E, shp.top_k)
    assert cfg["kernel"] == kernel and cfg["alias"] == alias, cfg
    if layout in ("split", "full"):
        P = M * shp.top_k
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        yb = -(-shp.H // cus) * P * 4
        xb, xsb, hsb = M * shp.H, M * (shp.H // 128) * 4, P * (shp.I // 128) * 4
        if layout == "full":     # h codes over x codes, h scales over x scales
            assert cfg["lds_bytes"] == max(xb, P * shp.I) + max(xsb, hsb) + yb, cfg
        else:                    # slots apart from x first, then over x; the scales apart
            apart = (cfg["lds_bytes"] - (xb + xsb + hsb + yb)) // shp.I
            assert P // 2 <= apart < P and (P - apart) * shp.I <= xb, cfg
    bank = Bank(pq, shp.E, shp.H, shp.I, workload=workloads.MOE_LAYER, seed=0)
    x = workloads.activation_bf16(M, shp.H, workload=workloads.MOE_VERIFY, seed=M)
    lg = workloads.verify_logits(M, shp.E, seed=M)
    ids, _ = oracle.route_topk(lg, shp.top_k)
    bank.fill(ids)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=shp.top_k, debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=shp.top_k)
    worst = _check(pq, bank, x, res, ref, M, shp.top_k)
    # each verify row equals the token decoded alone (byte-identical to serial decode)
    xt, lt = np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda()
    for m in (0, M - 1):
        one = pq.moe_decode_layer(xt[m:m + 1].contiguous(), bank.w13, bank.s13, bank.w2, bank.s2,
                                  logits=lt[m:m + 1].contiguous(), top_k=shp.top_k)
        assert torch.equal(one["out"][0].view(torch.int16), res["out"][m].view(torch.int16))
    print(f"full-size verify M={M} ({kernel}, alias={alias}, {layout}): union {len(oracle.union_of_experts(ids))} experts, "
          f"worst |err|/S {worst:.2e}")


@pytest.mark.parametrize("M", [1, 4])
def test_moe_tp8_share_layer(pq, path, M):
    """One GPU's share of the layer under 8-way tensor parallelism: all 256
    experts, hidden 6144, intermediate cut to 2048/8 = 256 columns of gate/up
    and rows of down.  The output is that share's partial sum of the combine;
    every element is checked."""
    import torch
    shp = workloads.MOE_TP8_SHAPE
    bank = Bank(pq, shp.E, shp.H, shp.I, workload=workloads.MOE_LAYER, seed=5)
    x = workloads.activation_bf16(M, shp.H, workload=workloads.MOE_LAYER if M == 1 else workloads.MOE_VERIFY,
                                  seed=5)
    lg = (workloads.router_logits(1, shp.E, workload=workloads.MOE_LAYER, seed=5) if M == 1
          else workloads.verify_logits(M, shp.E, seed=5))
    ids, _ = oracle.route_topk(lg, shp.top_k)
    bank.fill(ids)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=shp.top_k, debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=shp.top_k)
    worst = _check(pq, bank, x, res, ref, M, shp.top_k)
    print(f"tp8 share M={M} ({path}): union {len(oracle.union_of_experts(ids))} experts, worst |err|/S {worst:.2e}")


@pytest.mark.parametrize("E", [16, 200, 256, 1000])
def test_moe_routing_ties_and_signed_zero(pq, E):
    """Equal logits go to the lower expert id; -0 and +0 are equal."""
    import torch
    M, H, I, k = 4, 256, 128, 8
    bank = Bank(pq, E, H, I, seed=11)
    rng = np.random.default_rng(E)
    lg = np.round(rng.standard_normal((M, E)), 1).astype(np.float32)   # many exact ties
    lg[1, :] = 0.0
    lg[1, ::3] = -0.0
    lg[2, :] = 1.5                                                     # everything tied
    lg[3, E - 1] = 9.0
    lg[3, E // 2] = 9.0
    ids_ref, w_ref = oracle.route_topk(lg, k)
    bank.fill(ids_ref)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=11)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=k)
    assert np.array_equal(res["topk_ids"].cpu().numpy(), ids_ref)
    assert np.max(np.abs(res["topk_w"].cpu().numpy() - w_ref)) <= 1e-6
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
    assert_gemv_close(bf16_to_np(res["out"]), ref["out"], ref["S"], f"ties E={E}")


# ---------------------------------------------------------------------------
# The steps either side of the routed layer in the same launch: the router
# GEMV (bf16, native precision) and a shared expert added with weight 1.
# ---------------------------------------------------------------------------

def _check_shared(res, ref):
    """The shared expert's h (SiLU bound) and its re-quantised codes and scales."""
    h = bf16_to_np(res["sh_h"])
    assert_silu_close(h, ref["sh_h"], ref["sh_gate"], ref["sh_up"], ref["sh_S_gate"], ref["sh_S_up"], "shared h")
    assert_requant_bit_exact(res["sh_h"], res["sh_hq"], res["sh_hs"], "shared h")
    diff = np.mean(res["sh_hq"].cpu().numpy() != ref["sh_hq"])
    assert diff <= 2e-3, f"{diff:.2e} of the shared expert's h codes differ"


@pytest.mark.parametrize("M,E,H,I,k", [(1, 16, 512, 256, 4), (3, 24, 1024, 512, 8), (8, 32, 1024, 256, 8)])
def test_moe_shared_expert_given_logits(pq, path, M, E, H, I, k):
    import torch
    bank = Bank(pq, E, H, I, seed=20 + M)
    sh = bank.shared()
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=20 + M)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=20 + M)
    ids, _ = oracle.route_topk(lg, k)
    bank.fill(ids)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              logits=torch.from_numpy(lg).cuda(), top_k=k, shared=sh, debug=True)
    assert pq.workspace_check() == 0
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k, shared=bank.sh_cpu)
    _check(pq, bank, x, res, ref, M, k)
    _check_shared(res, ref)


def _router_case(pq, bank, M, E, H, k, seed, predict=2):
    """Router weights and activations; fills the experts the oracle's own
    logits rank in the top k + ``predict`` of each token (near ties may order
    differently in fp32), returns (x bits, router bits, router tensor)."""
    import torch
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER if M == 1 else workloads.MOE_VERIFY,
                                  seed=seed)
    wr = workloads.router_weights_bf16(E, H, seed=seed)
    lo = oracle.router_logits(x, wr)
    top = np.argsort(-lo, axis=1, kind="stable")[:, :min(E, k + predict)]
    bank.fill(top)
    return x, wr, np_bf16_bits_to_torch(wr)


def _check_router(res, x, wr, bank, k, shared=None):
    """Logits within the fp32 accumulation bound of the oracle's; routing decided on
    the kernel's own logits; the layer output against the oracle run on those
    routes."""
    lg = res["logits"].cpu().numpy()
    lo = oracle.router_logits(x, wr)
    xs = np.abs(workloads.bf16_bits_to_f32(x).astype(np.float64))
    ws = np.abs(workloads.bf16_bits_to_f32(wr).astype(np.float64))
    Sr = xs @ ws.T
    assert np.all(np.abs(lg - lo) <= 1e-4 * Sr), f"router logits: worst {np.max(np.abs(lg - lo) / Sr):.2e} of S"
    ids, w = oracle.route_topk(lg, k)
    assert np.array_equal(res["topk_ids"].cpu().numpy(), ids), "routing ids differ from the top-k of the kernel's logits"
    assert np.max(np.abs(res["topk_w"].cpu().numpy() - w)) <= 1e-6
    ids64, _ = oracle.route_topk(lo.astype(np.float32), k)
    near = np.sort(lo, axis=1)[:, ::-1]
    gap = np.min(np.abs(np.diff(near[:, :k + 1], axis=1)), axis=1)
    for m in range(lg.shape[0]):
        if gap[m] > 1e-3:          # no near tie: the fp64 routing must agree too
            assert np.array_equal(ids[m], ids64[m])
    for e in np.unique(ids):
        assert int(e) in bank.cpu, "the kernel routed to an expert the test did not fill"
    return oracle.moe_layer(x, bank.expert, ids=ids, weights=w, shared=shared)


@pytest.mark.parametrize("M,E,H,I,k,with_shared", [(1, 16, 512, 256, 4, False), (1, 64, 1024, 256, 8, True),
                                                   (2, 32, 1024, 512, 8, True), (5, 40, 512, 256, 6, False),
                                                   (8, 300, 1024, 256, 8, True)])
def test_moe_router_gemv_in_the_launch(pq, path, M, E, H, I, k, with_shared):
    bank = Bank(pq, E, H, I, seed=40 + M)
    sh = bank.shared() if with_shared else None
    x, wr, wrt = _router_case(pq, bank, M, E, H, k, seed=40 + M)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              router_w=wrt, top_k=k, shared=sh, debug=True)
    assert pq.workspace_check() == 0
    ref = _check_router(res, x, wr, bank, k, bank.sh_cpu if with_shared else None)
    assert_requant_bit_exact(res["h"], res["hq"], res["hs"])
    y = bf16_to_np(res["out"])
    assert_gemv_close(y, ref["out"], ref["S"], f"router M={M} E={E} shared={with_shared}")
    if with_shared:
        _check_shared(res, ref)


@pytest.mark.parametrize("M", [1, 4])
def test_moe_full_layer_with_router_and_shared_expert(pq, path, M):
    """256 experts, hidden 6144, intermediate 2048, top-8, the router GEMV and a
    shared expert in the launch, every output checked."""
    shp = workloads.MOE_SHAPE
    bank = Bank(pq, shp.E, shp.H, shp.I, workload=workloads.MOE_LAYER, seed=3)
    sh = bank.shared()
    x, wr, wrt = _router_case(pq, bank, M, shp.E, shp.H, shp.top_k, seed=3, predict=1)
    res = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                              router_w=wrt, top_k=shp.top_k, shared=sh, debug=True)
    assert pq.workspace_check() == 0
    ref = _check_router(res, x, wr, bank, shp.top_k, bank.sh_cpu)
    assert_requant_bit_exact(res["h"], res["hq"], res["hs"])
    worst = assert_gemv_close(bf16_to_np(res["out"]), ref["out"], ref["S"], f"full router+shared M={M}")
    _check_shared(res, ref)
    print(f"full router+shared M={M} ({path}): worst |err|/S {worst:.2e}")


@pytest.mark.parametrize("M", [1, 3])
def test_moe_router_and_shared_kernels_agree_bitwise(pq, M):
    import torch
    E, H, I, k = 48, 1024, 512, 8
    bank = Bank(pq, E, H, I, seed=60 + M)
    sh = bank.shared()
    x, wr, wrt = _router_case(pq, bank, M, E, H, k, seed=60 + M, predict=E)
    outs = []
    for path in ("barrier", "stream"):
        os.environ["PQ_MOE_PATH"] = path
        try:
            r = pq.moe_decode_layer(np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2,
                                    router_w=wrt, top_k=k, shared=sh)
        finally:
            del os.environ["PQ_MOE_PATH"]
        outs.append((r["out"].clone(), r["logits"].clone(), r["topk_ids"].clone()))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    assert torch.equal(outs[0][2], outs[1][2])
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))


def test_moe_router_wait_times_out_then_recovers(pq, path):
    """A spin limit of zero makes the routing waves give up on the logits of
    other blocks (forced from the host: every wait is bounded); the call ends,
    and the next call on the same workspace is correct."""
    M, E, H, I, k = 2, 32, 512, 256, 4
    bank = Bank(pq, E, H, I, seed=70)
    sh = bank.shared()
    x, wr, wrt = _router_case(pq, bank, M, E, H, k, seed=70, predict=E)
    args = (np_bf16_bits_to_torch(x), bank.w13, bank.s13, bank.w2, bank.s2)
    os.environ["PQ_SPIN_LIMIT"] = "0"
    try:
        pq.moe_decode_layer(*args, router_w=wrt, top_k=k, shared=sh)
    finally:
        del os.environ["PQ_SPIN_LIMIT"]
    assert pq.workspace_check() in (0, -7)
    res = pq.moe_decode_layer(*args, router_w=wrt, top_k=k, shared=sh, debug=True)
    assert pq.workspace_check() == 0
    ref = _check_router(res, x, wr, bank, k, bank.sh_cpu)
    assert_requant_bit_exact(res["h"], res["hq"], res["hs"])
    assert_gemv_close(bf16_to_np(res["out"]), ref["out"], ref["S"], "router after timeout")
