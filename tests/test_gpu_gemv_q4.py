"""GPU parity of pq_gemv_q4 (int4 g32 W4A16 GEMV with SiLU*up epilogue) against
the oracle.  Two kernels: the MFMA one (K % 256 == 0, stream-K split with a
cross-wave combine; the default from M = 5, and at M = 4 for layers of >= 48 Mi weights) and the VALU one (K split inside a
block).  PQ_Q4_PATH=valu / =mfma forces either, so both are checked on the
same shapes.

Weights are quantised by the oracle and uploaded; the library's own int4
quantiser is checked bit-equal to it on the same rows.  At the dense-stack
sizes (K = 5120 / 17408, N up to 2 x 17408) the oracle evaluates a seeded
sample of rows (always including the first and last) one by one."""
import os

import numpy as np
import pytest

import oracle
import workloads
from _helpers import (assert_gemv_close, assert_silu_close, bf16_to_np, need_gpu,
                      np_bf16_bits_to_torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


class env:
    """Set one environment variable of the library for a block of code."""

    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = os.environ.get(self.name)
        if self.value is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = str(self.value)

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop(self.name, None)
        else:
            os.environ[self.name] = self.old


def _upload(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _q4_on_gpu(pq, w):
    """Oracle int4 quantisation of w, uploaded; the GPU quantiser must agree."""
    p, s = oracle.q4_quant(w)
    pg, sg = pq.quantize_q4(_upload(w))
    assert np.array_equal(pg.cpu().numpy(), p)
    assert np.array_equal(sg.cpu().numpy().view(np.uint16), s.view(np.uint16))
    return p, s, pg, sg


def _x(M, K, seed):
    x = workloads.activation_bf16(M, K, workload=workloads.Q4_STACK, seed=seed)
    return x, np_bf16_bits_to_torch(x)


class blocks_per_cu:
    """Set PQ_BLOCKS_PER_CU (how many blocks share the rows) for a block of code."""

    def __init__(self, n):
        self.n = n

    def __enter__(self):
        self.old = os.environ.get("PQ_BLOCKS_PER_CU")
        os.environ["PQ_BLOCKS_PER_CU"] = str(self.n)

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("PQ_BLOCKS_PER_CU", None)
        else:
            os.environ["PQ_BLOCKS_PER_CU"] = self.old


@pytest.mark.parametrize("M,K,N,S", [       # S: blocks per CU (None: default)
    (1, 32, 1, None),           # one group, one row
    (2, 96, 37, None),          # 3 groups: a partial 1 KB chunk, ragged N
    (3, 2080, 100, 5),          # 65 groups split 5 ways
    (1, 5120, 640, 8),
    (8, 8704, 64, None),        # largest K allowed at M = 8
    (4, 4096, 300, 2),
    (5, 2048, 129, 1),
    (2, 17408, 40, None),       # 9 chunks per row over 8 waves
    (7, 512, 3000, 2),          # many row tiles, 2 k steps each
    (1, 256, 17, None),         # one k step, ragged tile
])
@pytest.mark.parametrize("path", [None, "valu", "mfma"])
def test_gemv_q4_plain(pq, M, K, N, S, path):
    seed = M * 1000 + K + N
    x, xt = _x(M, K, seed)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=seed)
    p, s, pg, sg = _q4_on_gpu(pq, w)
    with blocks_per_cu(S or 1), env("PQ_Q4_PATH", path):
        y = pq.gemv_q4(xt, pg, sg)
    yo, So = oracle.gemv_q4(x, p, s)
    assert_gemv_close(bf16_to_np(y), yo, So, f"M={M} K={K} N={N} blocks/CU={S} path={path}")


@pytest.mark.parametrize("M,K,N,S", [
    (2, 1024, 70, None),
    (5, 768, 64, 2),
    (1, 4096, 512, 4),
    (8, 2048, 2 * 37, None),    # 37 rows: a ragged 16-row tile, two token sets
    (3, 8192, 2 * 300, 3),
])
@pytest.mark.parametrize("path", [None, "valu", "mfma"])
def test_gemv_q4_silu(pq, M, K, N, S, path):
    seed = M + K + N
    x, xt = _x(M, K, seed)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=seed)
    p, s, pg, sg = _q4_on_gpu(pq, w)
    with blocks_per_cu(S or 1), env("PQ_Q4_PATH", path):
        y = pq.gemv_q4(xt, pg, sg, epi=pq.EPI_SILU_MUL)
    yo, So = oracle.gemv_q4(x, p, s)
    I = N // 2
    h = oracle.silu_mul(yo, I)
    assert_silu_close(bf16_to_np(y), h, yo[:, :I], yo[:, I:], So[:, :I], So[:, I:], f"M={M} S={S}")


def _sample(n_rows, count, seed):
    rng = np.random.default_rng(seed)
    r = rng.choice(n_rows, size=min(count, n_rows), replace=False)
    return np.unique(np.concatenate([r, [0, n_rows - 1]]))


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("layer", [0, 1, 2])
def test_gemv_q4_dense_stack_layers(pq, M, layer):
    """The three layer shapes of the 4-bit dense decode stack at full size, in
    the launch configuration the benchmark times; sampled rows against the oracle."""
    import torch
    K, N, silu = workloads.Q4_SHAPES[layer]
    seed = 7 + layer
    x, xt = _x(M, K, seed)
    wt = workloads.master_weights_torch(N, K, workload=workloads.Q4_STACK, tensor=workloads.T_W,
                                        expert=layer, seed=seed, device="cuda")
    pg, sg = pq.quantize_q4(wt)
    y = bf16_to_np(pq.gemv_q4(xt, pg, sg, epi=pq.EPI_SILU_MUL if silu else pq.EPI_NONE))
    R = N // 2 if silu else N
    rows = _sample(R, 192, seed)
    want_rows = np.concatenate([rows, rows + R]) if silu else rows
    w_rows = wt[torch.from_numpy(want_rows).cuda()].cpu().numpy()
    p, s = oracle.q4_quant(w_rows)
    assert np.array_equal(pg[torch.from_numpy(want_rows).cuda()].cpu().numpy(), p)
    assert np.array_equal(sg[torch.from_numpy(want_rows).cuda()].cpu().numpy().view(np.uint16), s.view(np.uint16))
    yo, So = oracle.gemv_q4(x, p, s)
    if silu:
        n = len(rows)
        h = oracle.silu_mul(yo, n)
        assert_silu_close(y[:, rows], h, yo[:, :n], yo[:, n:], So[:, :n], So[:, n:], f"layer {layer} M={M}")
    else:
        assert_gemv_close(y[:, rows], yo, So, f"layer {layer} M={M}")


@pytest.mark.parametrize("K,path", [(96, None), (512, "valu"), (512, "mfma")])
def test_gemv_q4_decodes_every_nibble(pq, K, path):
    """Row n holds nibble n & 15 at one position, x is 1 there and the fp16 scale
    of that group is chosen per row (normal, subnormal, largest finite, zero):
    y[n] = (nibble - 8) * scale exactly."""
    import torch
    k0 = 45                            # k0 in group 1, odd position (high nibble)
    scales = np.array([1.0, 0.5, 2.0 ** -24, 2.0 ** -14, 65504.0, 0.0, 3.0, 1.0 / 7], np.float16)
    n_rows = 16 * len(scales)
    q = np.zeros((n_rows, K), np.int64)
    q[:, k0] = np.tile(np.arange(16) - 8, len(scales))
    packed = oracle.q4_pack(q)
    sc = np.ones((n_rows, K // 32), np.float16)
    sc[:, 1] = np.repeat(scales, 16)
    x = np.zeros((1, K), np.uint16)
    x[0, k0] = workloads.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    with env("PQ_Q4_PATH", path):
        y = bf16_to_np(pq.gemv_q4(np_bf16_bits_to_torch(x), _upload(packed), _upload(sc)))[0]
    want = q[:, k0] * sc[:, 1].astype(np.float64)
    want_bf16 = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(want.astype(np.float32))).astype(np.float64)
    assert np.array_equal(y, want_bf16)


@pytest.mark.parametrize("K,path", [(2080, None), (2048, "valu"), (2048, "mfma")])
def test_gemv_q4_rows_bitwise_independent_of_M(pq, K, path):
    import torch
    M, N = 6, 512
    x, xt = _x(M, K, 17)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=17)
    p, s, pg, sg = _q4_on_gpu(pq, w)
    with env("PQ_Q4_PATH", path):
        y = pq.gemv_q4(xt, pg, sg, epi=pq.EPI_SILU_MUL)
        for m in range(M):
            ym = pq.gemv_q4(xt[m:m + 1].contiguous(), pg, sg, epi=pq.EPI_SILU_MUL)
            assert torch.equal(ym[0].view(torch.int16), y[m].view(torch.int16))


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_gemv_q4_split_points_change_only_rounding(pq, path):
    """The grid decides where a row's K range is cut between waves; any cut
    agrees with the oracle within the GEMV tolerance, and a repeated call with
    the same grid is bitwise identical."""
    import torch
    M, K, N = 2, 5120, 700
    x, xt = _x(M, K, 23)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=23)
    p, s, pg, sg = _q4_on_gpu(pq, w)
    yo, So = oracle.gemv_q4(x, p, s)
    for n in (1, 2, 3, 8):
        with blocks_per_cu(n), env("PQ_Q4_PATH", path):
            ys = pq.gemv_q4(xt, pg, sg)
            ys2 = pq.gemv_q4(xt, pg, sg)
        assert torch.equal(ys.view(torch.int16), ys2.view(torch.int16))
        assert_gemv_close(bf16_to_np(ys), yo, So, f"blocks/CU={n}")


@pytest.mark.parametrize("K,path", [(1056, None), (1024, "valu"), (1024, "mfma")])
def test_gemv_q4_zero_inputs(pq, K, path):
    import torch
    M, N = 3, 80
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=3)
    p, s = oracle.q4_quant(w)
    xt = np_bf16_bits_to_torch(workloads.activation_bf16(M, K, workload=workloads.Q4_STACK, seed=3))
    with env("PQ_Q4_PATH", path):
        y = pq.gemv_q4(x, _upload(p), _upload(s))
        assert torch.count_nonzero(y.view(torch.int16)) == 0
        y = pq.gemv_q4(xt, _upload(np.full_like(p, 0x88)), _upload(s))     # every code is 0
        assert torch.count_nonzero(y.view(torch.int16)) == 0


@pytest.mark.parametrize("M,K,N,epi", [
    (9, 64, 4, 0),          # M above 8
    (1, 48, 4, 0),          # K not a multiple of 32
    (1, 64, 5, 1),          # odd N under SiLU
    (8, 8736, 4, 0),        # activation does not fit LDS
])
def test_gemv_q4_bad_shapes(pq, M, K, N, epi):
    import torch
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 32), dtype=torch.float16, device="cuda")
    with pytest.raises(pq.PqError) as e:
        pq.gemv_q4(x, w, s, epi=epi)
    assert e.value.status == -2


# ---------------------------------------------------------------------------
# pq_gemv_q4_group: several independent linears in as few launches as LDS allows
# ---------------------------------------------------------------------------

GROUP_SPECS = [(5120, 640, 0), (2080, 2 * 100, 1), (1024, 37, 0), (96, 2 * 9, 1), (4096, 300, 0),
               (512, 4000, 0), (2048, 2 * 513, 1)]     # K / 32 odd for 2080 and 96: the 16-bit scale form


def _group_case(pq, M, specs, seed):
    items, refs = [], []
    for i, (K, N, epi) in enumerate(specs):
        x, xt = _x(M, K, seed + i)
        w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=seed + i)
        p, s, pg, sg = _q4_on_gpu(pq, w)
        items.append((xt, pg, sg, epi))
        refs.append((x, p, s, epi))
    return items, refs


def _check_q4(y, x, p, s, epi, what):
    yo, So = oracle.gemv_q4(x, p, s)
    if epi:
        I = yo.shape[1] // 2
        h = oracle.silu_mul(yo, I)
        assert_silu_close(bf16_to_np(y), h, yo[:, :I], yo[:, I:], So[:, :I], So[:, I:], what)
    else:
        assert_gemv_close(bf16_to_np(y), yo, So, what)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_gemv_q4_group_equals_single_calls(pq, M):
    """One grouped call over linears of mixed shapes, epilogues and scale forms:
    every output is bitwise equal to its own pq_gemv_q4 call on the vector
    kernel (a linear's split does not depend on the other linears), and
    within the oracle's bound."""
    import torch
    specs = GROUP_SPECS if M < 8 else GROUP_SPECS[:4]
    items, refs = _group_case(pq, M, specs, seed=500 + M)
    ys, launches = pq.gemv_q4_group(items)
    assert 2 <= launches <= len(items)          # the two scale forms never share a launch
    with env("PQ_Q4_PATH", "valu"):
        for i, ((xt, pg, sg, epi), y) in enumerate(zip(items, ys)):
            y1 = pq.gemv_q4(xt, pg, sg, epi=epi)
            assert torch.equal(y1.view(torch.int16), y.view(torch.int16)), f"linear {i}: grouped != single call"
    for i, (y, (x, p, s, epi)) in enumerate(zip(ys, refs)):
        _check_q4(y, x, p, s, epi, f"group M={M} linear {i}")


def test_gemv_q4_group_rows_bitwise_independent_of_M(pq):
    import torch
    M = 5
    specs = [(5120, 320, 0), (2048, 2 * 200, 1), (8704, 64, 0)]
    items, _ = _group_case(pq, M, specs, seed=600)
    ys, _ = pq.gemv_q4_group(items)
    for m in range(M):
        one, _ = pq.gemv_q4_group([(xt[m:m + 1].contiguous(), pg, sg, epi) for xt, pg, sg, epi in items])
        for y, y1 in zip(ys, one):
            assert torch.equal(y1[0].view(torch.int16), y[m].view(torch.int16))


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_q4_group_dense_stack_blocks(pq, M):
    """Two blocks of the 4-bit dense decode stack (5120->5120, 5120->2x17408
    with SiLU*up, 17408->5120) at full size in one grouped call, as the
    benchmark issues them: each output bitwise equal to the linear's single
    vector-kernel call, sampled rows against the oracle."""
    import torch
    items, meta = [], []
    for blk in range(2):
        for layer, (K, N, silu) in enumerate(workloads.Q4_SHAPES):
            seed = 70 + 3 * blk + layer
            x, xt = _x(M, K, seed)
            wt = workloads.master_weights_torch(N, K, workload=workloads.Q4_STACK, tensor=workloads.T_W,
                                                expert=3 * blk + layer, seed=seed, device="cuda")
            pg, sg = pq.quantize_q4(wt)
            epi = pq.EPI_SILU_MUL if silu else pq.EPI_NONE
            items.append((xt, pg, sg, epi))
            meta.append((x, wt, pg, sg, K, N, silu, seed))
    ys, launches = pq.gemv_q4_group(items)
    print(f"dense stack, 2 blocks, M={M}: {launches} launches for {len(items)} linears")
    with env("PQ_Q4_PATH", "valu"):
        for (xt, pg, sg, epi), y in zip(items, ys):
            assert torch.equal(pq.gemv_q4(xt, pg, sg, epi=epi).view(torch.int16), y.view(torch.int16))
    for y, (x, wt, pg, sg, K, N, silu, seed) in zip(ys, meta):
        R = N // 2 if silu else N
        rows = _sample(R, 96, seed)
        want_rows = np.concatenate([rows, rows + R]) if silu else rows
        idx = torch.from_numpy(want_rows).cuda()
        p, s = oracle.q4_quant(wt[idx].cpu().numpy())
        assert np.array_equal(pg[idx].cpu().numpy(), p)
        yo, So = oracle.gemv_q4(x, p, s)
        yy = bf16_to_np(y)
        if silu:
            n = len(rows)
            h = oracle.silu_mul(yo, n)
            assert_silu_close(yy[:, rows], h, yo[:, :n], yo[:, n:], So[:, :n], So[:, n:], f"stack SiLU M={M}")
        else:
            assert_gemv_close(yy[:, rows], yo, So, f"stack {K}->{N} M={M}")


def test_gemv_q4_group_two_streams_join_and_overlap_fallback(pq, monkeypatch):
    """A grouped call of several launches alternates them between the
    caller's stream and a second one, joined back at the end: copies queued
    on the caller's stream right after the call see every output final, and
    the bits equal one-stream issue (PQ_Q4_STREAMS=1).  Two linears writing
    the same output from different launches (the two scale forms never share
    one) fall back to one stream in order, so the later linear's values win."""
    import torch
    M = 4
    specs = [(5120, 640, 0), (5120, 2 * 512, 1), (8704, 320, 0), (5120, 640, 0), (2048, 2 * 256, 1)]
    items, _ = _group_case(pq, M, specs, seed=710)
    ys, launches = pq.gemv_q4_group(items)
    copies = [y.clone() for y in ys]                    # queued on the caller's stream, no sync in between
    assert launches >= 2
    monkeypatch.setenv("PQ_Q4_STREAMS", "1")
    ys1, launches1 = pq.gemv_q4_group(items)
    monkeypatch.delenv("PQ_Q4_STREAMS")
    assert launches1 == launches
    for i, (c, y, y1) in enumerate(zip(copies, ys, ys1)):
        assert torch.equal(c.view(torch.int16), y1.view(torch.int16)), f"linear {i}: copy after the call"
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"linear {i}"
    # overlapping outputs: K/32 even and odd, so two launches, one shared y
    (xa, pa, sa, ea), (xb, pb, sb, eb) = _group_case(pq, M, [(1024, 96, 0), (1056, 96, 0)], seed=711)[0]
    shared = torch.empty((M, 96), dtype=torch.bfloat16, device="cuda")
    _, n2 = pq.gemv_q4_group([(xa, pa, sa, ea, shared), (xb, pb, sb, eb, shared)])
    assert n2 == 2
    with env("PQ_Q4_PATH", "valu"):
        want = pq.gemv_q4(xb, pb, sb, epi=eb)
    assert torch.equal(shared.view(torch.int16), want.view(torch.int16))


def test_gemv_q4_group_rejects_bad_linears(pq):
    import torch
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.float16, device="cuda")
    ok = (x, w, s, 0)
    bad = (x, torch.zeros((5, 32), dtype=torch.uint8, device="cuda"), torch.zeros((5, 2), dtype=torch.float16,
                                                                                   device="cuda"), 1)
    with pytest.raises(pq.PqError) as e:
        pq.gemv_q4_group([ok, bad])                  # odd N under SiLU: nothing is launched
    assert e.value.status == -2
