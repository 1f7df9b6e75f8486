"""MI355X (gfx950) quantized-weight decode: Python binding of the C-ABI library.

Every step of the decode path runs in the HIP kernels of ``libpqmoe.so``;
this module only checks tensor metadata, hands raw device pointers and the
current HIP stream to the C calls of ``include/pq.h`` and raises on a
non-zero status.  PyTorch provides device memory and streams.  There is no
CPU fallback: the library must be built (see ``build.py``).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["PqError", "quantize_fp8", "quantize_q4", "gemv_fp8", "gemm_fp8", "gemm_fp8_prequant", "gemv_q4",
           "gemv_q4_group", "moe_decode_layer",
           "moe_decode_layer_noalloc", "gemv_fp8_workspace_bytes", "moe_workspace_bytes", "workspace_check",
           "launches_per_call", "moe_layer_config",
           "stream_probe",
           "EPI_NONE", "EPI_SILU_MUL", "lib"]

EPI_NONE = 0
EPI_SILU_MUL = 1
WS_DATA_OFF = 65536 + (2 << 20)   # start of the workspace's data region (counters and a zeroed region before it)


class PqError(RuntimeError):
    """A pq_* call returned a non-zero pq_status."""

    def __init__(self, what: str, status: int):
        lib = _lib.load()
        msg = lib.pq_strerror(status).decode()
        super().__init__(f"{what}: {msg} (status {status}, hip error {lib.pq_last_hip_error()})")
        self.status = status


def lib():
    return _lib.load()


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise PqError(what, status)


def _need(t, dtype, ndim, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# one zero-initialised workspace per (device, stream); kernels leave it zeroed
_WS: dict = {}


def _workspace(nbytes: int):
    if nbytes == 0:
        return None, 0
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(int(nbytes), 4096), dtype=torch.uint8, device="cuda")
        _check(lib().pq_workspace_init(_p(ws), ws.numel(), _stream()), "pq_workspace_init")
        _WS[key] = ws
    return ws, ws.numel()


def workspace_check() -> int:
    """Synchronise and return (and clear) the error recorded by kernels in the
    current stream's workspace (0 = none)."""
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    ws = _WS.get(key)
    if ws is None:
        return 0
    return lib().pq_workspace_check(_p(ws), _stream())


def launches_per_call(entry_point: str = "moe_decode_layer") -> int:
    """Kernel launches one call of the named C entry point makes."""
    n = lib().pq_launches_per_call(entry_point.encode())
    if n < 0:
        raise PqError("pq_launches_per_call", n)
    return n


def moe_layer_config(M: int, H: int, I: int, E: int, top_k: int, shared: bool = False) -> dict:
    """Which layer kernel and LDS layout a moe_decode_layer call of this shape
    uses on the current device: {"kernel": "barrier"|"stream", "alias": bool,
    "lds_bytes": int}."""
    k, al, lds = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_size_t(0)
    _check(lib().moe_decode_layer_config(M, H, I, E, top_k, int(bool(shared)), ctypes.byref(k), ctypes.byref(al),
                                         ctypes.byref(lds)), "moe_decode_layer_config")
    return {"kernel": ("barrier", "stream")[k.value], "alias": bool(al.value), "lds_bytes": int(lds.value)}


def stream_probe(src, sink) -> None:
    """Stream the bytes of device tensor ``src`` through the weight-stream load
    path and store per-wave checksums into ``sink`` (uint32, >= 16384 words);
    time it with events to get the achievable HBM read bandwidth."""
    _check(lib().pq_stream_probe(_p(src), src.numel() * src.element_size(), _p(sink), _stream()),
           "pq_stream_probe")


def quantize_fp8(t: torch.Tensor):
    """Block-128 FP8 quantisation of bf16 or fp32 rows [R, K] -> (codes uint8, scales fp32)."""
    if t.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("quantize_fp8 takes bf16 or fp32 input")
    _need(t, t.dtype, 2, "t")
    R, K = t.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=t.device)
    scales = torch.empty((R, max(K // 128, 1)), dtype=torch.float32, device=t.device)
    _check(lib().pq_quantize_fp8(_p(t), int(t.dtype == torch.float32), R, K, _p(codes), _p(scales), _stream()),
           "pq_quantize_fp8")
    return codes, scales


def quantize_q4(w: torch.Tensor):
    """int4 g32 quantisation of fp32 [N, K] -> (packed uint8 [N, K/2], scales fp16 [N, K/32])."""
    _need(w, torch.float32, 2, "w")
    N, K = w.shape
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, max(K // 32, 1)), dtype=torch.float16, device=w.device)
    _check(lib().pq_quantize_q4(_p(w), N, K, _p(packed), _p(scales), _stream()), "pq_quantize_q4")
    return packed, scales


def gemv_fp8_workspace_bytes(M: int, K: int, N: int, epi: int = EPI_NONE) -> int:
    return int(lib().pq_gemv_fp8_workspace(M, K, N, epi))


def gemv_fp8(x, w, w_scale, epi: int = EPI_NONE, debug: bool = False, out=None):
    """y = epi(x_q @ w_q^T) with live FP8 quantisation of x.  x bf16 [M,K], w uint8 [N,K],
    w_scale fp32 [N,K/128].  Returns y (bf16 [M,N] or [M,N/2]), or (y, xq, xs) with debug."""
    _need(x, torch.bfloat16, 2, "x")
    _need(w, torch.uint8, 2, "w")
    _need(w_scale, torch.float32, 2, "w_scale")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or w_scale.shape != (N, K // 128):
        raise ValueError("weight / scale shapes do not match x")
    n_out = N // 2 if epi == EPI_SILU_MUL else N
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=x.device)
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device) if debug else None
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if debug else None
    ws, wsn = _workspace(gemv_fp8_workspace_bytes(M, K, N, epi))
    _check(lib().pq_gemv_fp8(_p(x), M, K, _p(w), _p(w_scale), N, epi, _p(y), _p(xq), _p(xs), _p(ws), wsn,
                             _stream()), "pq_gemv_fp8")
    return (y, xq, xs) if debug else y


def gemm_fp8(x, w, w_scale, epi: int = EPI_NONE, debug: bool = False, out=None):
    """Large-M (prefill) block-scaled FP8 GEMM on the matrix cores: x bf16 [M,K] (quantised
    live into the workspace), w uint8 [N,K], w_scale fp32 [N,K/128].  Returns y (bf16 [M,N]
    or [M,N/2] under SiLU*up), or (y, xq, xs) with debug (views of the workspace)."""
    _need(x, torch.bfloat16, 2, "x")
    _need(w, torch.uint8, 2, "w")
    _need(w_scale, torch.float32, 2, "w_scale")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or w_scale.shape != (N, K // 128):
        raise ValueError("weight / scale shapes do not match x")
    n_out = N // 2 if epi == EPI_SILU_MUL else N
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=x.device)
    ws, wsn = _workspace(int(lib().pq_gemm_fp8_workspace(M, K, N, epi)))
    _check(lib().pq_gemm_fp8(_p(x), M, K, _p(w), _p(w_scale), N, epi, _p(y), _p(ws), wsn, _stream()), "pq_gemm_fp8")
    if not debug:
        return y
    off = WS_DATA_OFF
    xq = ws[off:off + M * K].view(M, K)
    off2 = off + (M * K + 255) // 256 * 256
    xs = ws[off2:off2 + M * (K // 128) * 4].view(torch.float32).view(M, K // 128)
    return y, xq, xs


def gemm_fp8_prequant(xq, xs, w, w_scale, epi: int = EPI_NONE, out=None):
    """The GEMM of gemm_fp8 on an activation already quantised (xq uint8 [M,K], xs fp32
    [M,K/128], the rule of quantize_fp8)."""
    _need(xq, torch.uint8, 2, "xq")
    _need(xs, torch.float32, 2, "xs")
    _need(w, torch.uint8, 2, "w")
    _need(w_scale, torch.float32, 2, "w_scale")
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K or w_scale.shape != (N, K // 128) or xs.shape != (M, K // 128):
        raise ValueError("shapes do not match")
    n_out = N // 2 if epi == EPI_SILU_MUL else N
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=xq.device)
    _check(lib().pq_gemm_fp8_prequant(_p(xq), _p(xs), M, K, _p(w), _p(w_scale), N, epi, _p(y), _stream()),
           "pq_gemm_fp8_prequant")
    return y


def gemv_q4(x, w, w_scale, epi: int = EPI_NONE, out=None):
    """W4A16 GEMV: x bf16 [M,K], w uint8 nibbles [N,K/2], w_scale fp16 [N,K/32]."""
    _need(x, torch.bfloat16, 2, "x")
    _need(w, torch.uint8, 2, "w")
    _need(w_scale, torch.float16, 2, "w_scale")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K // 2 or w_scale.shape != (N, K // 32):
        raise ValueError("weight / scale shapes do not match x")
    n_out = N // 2 if epi == EPI_SILU_MUL else N
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=x.device)
    ws, wsn = _workspace(int(lib().pq_gemv_q4_workspace(M, K, N, epi)))
    _check(lib().pq_gemv_q4(_p(x), M, K, _p(w), _p(w_scale), N, epi, _p(y), _p(ws), wsn, _stream()),
           "pq_gemv_q4")
    return y


def gemv_q4_group(items):
    """Several independent int4 GEMVs in as few launches as possible.
    items: list of (x bf16 [M,K], w uint8 [N,K/2], w_scale fp16 [N,K/32], epi)
    or (x, w, w_scale, epi, y); every x has the same M.  Returns (list of y,
    launches made)."""
    if not items:
        return [], 0
    M = items[0][0].shape[0]
    arr = (_lib.Q4Linear * len(items))()
    ys = []
    for i, it in enumerate(items):
        x, w, sc, epi = it[:4]
        _need(x, torch.bfloat16, 2, "x")
        _need(w, torch.uint8, 2, "w")
        _need(sc, torch.float16, 2, "w_scale")
        if x.shape[0] != M:
            raise ValueError("every linear of a group has the same M")
        K, N = x.shape[1], w.shape[0]
        if w.shape[1] != K // 2 or sc.shape != (N, K // 32):
            raise ValueError("weight / scale shapes do not match x")
        n_out = N // 2 if epi == EPI_SILU_MUL else N
        y = it[4] if len(it) > 4 else torch.empty((M, n_out), dtype=torch.bfloat16, device=x.device)
        ys.append(y)
        arr[i] = _lib.Q4Linear(x.data_ptr(), w.data_ptr(), sc.data_ptr(), y.data_ptr(), K, N, epi)
    nl = ctypes.c_int(0)
    _check(lib().pq_gemv_q4_group(arr, len(items), M, ctypes.byref(nl), _stream()), "pq_gemv_q4_group")
    return ys, nl.value


def moe_workspace_bytes(M: int, H: int, I: int, E: int, top_k: int) -> int:
    return int(lib().moe_decode_layer_workspace(M, H, I, E, top_k))


def moe_decode_layer(x, w13, s13, w2, s2, *, logits=None, topk_ids=None, topk_w=None, top_k: int = 8,
                     router_w=None, shared=None, debug: bool = False, out=None):
    """One MoE decode layer in one launch.

    x bf16 [M,H]; w13 uint8 [E,2I,H], s13 fp32 [E,2I,H/128]; w2 uint8 [E,H,I], s2 fp32 [E,H,I/128].
    Routing from ``router_w`` bf16 [E,H] (the router GEMV runs in the launch; its logits are
    returned as ``logits``), from ``logits`` fp32 [M,E], or from given ``topk_ids`` int32 /
    ``topk_w`` fp32 [M,top_k].  ``shared`` = (w13, s13, w2, s2) of one expert of the bank's
    shapes adds a shared expert with weight 1.  Returns a dict with ``out`` (bf16 [M,H]),
    ``topk_ids``, ``topk_w`` and, with debug, ``h`` (bf16 [M*k + M*sh, I]: the (token, slot)
    pairs, then the shared expert's per token), ``hq`` (uint8, same), ``hs`` (fp32 [.., I/128])."""
    _need(x, torch.bfloat16, 2, "x")
    _need(w13, torch.uint8, 3, "w13")
    _need(s13, torch.float32, 3, "s13")
    _need(w2, torch.uint8, 3, "w2")
    _need(s2, torch.float32, 3, "s2")
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    dev = x.device
    lg_out = None
    if router_w is not None:
        _need(router_w, torch.bfloat16, 2, "router_w")
        lg_out = torch.empty((M, E), dtype=torch.float32, device=dev)
        topk_ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
        topk_w = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    elif logits is not None:
        _need(logits, torch.float32, 2, "logits")
        topk_ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
        topk_w = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    else:
        _need(topk_ids, torch.int32, 2, "topk_ids")
        _need(topk_w, torch.float32, 2, "topk_w")
        top_k = topk_ids.shape[1]
    sh = (None,) * 4
    if shared is not None:
        sh = tuple(shared)
        for t, dt, nm in zip(sh, (torch.uint8, torch.float32, torch.uint8, torch.float32),
                             ("shared w13", "shared s13", "shared w2", "shared s2")):
            _need(t, dt, 2, nm)
        if sh[0].shape != w13.shape[1:] or sh[2].shape != w2.shape[1:]:
            raise ValueError("the shared expert must have the routed experts' shapes")
    npairs = M * top_k + (M if shared is not None else 0)
    y = out if out is not None else torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    h = torch.empty((npairs, I), dtype=torch.bfloat16, device=dev) if debug else None
    hq = torch.empty((npairs, I), dtype=torch.uint8, device=dev) if debug else None
    hs = torch.empty((npairs, I // 128), dtype=torch.float32, device=dev) if debug else None
    ws, wsn = _workspace(moe_workspace_bytes(M, H, I, E, top_k))
    lg_arg = lg_out if router_w is not None else logits
    _check(lib().moe_decode_layer_ex(_p(x), M, H, _p(router_w), _p(lg_arg), _p(topk_ids), _p(topk_w), E, top_k, I,
                                     _p(w13), _p(s13), _p(w2), _p(s2), _p(sh[0]), _p(sh[1]), _p(sh[2]), _p(sh[3]),
                                     _p(y), _p(h), _p(hq), _p(hs), _p(ws), wsn, _stream()), "moe_decode_layer_ex")
    res = {"out": y, "topk_ids": topk_ids, "topk_w": topk_w}
    if lg_out is not None:
        res["logits"] = lg_out
    if debug:
        P = M * top_k
        res.update(h=h[:P].view(M, top_k, I), hq=hq[:P].view(M, top_k, I), hs=hs[:P].view(M, top_k, I // 128))
        if shared is not None:
            res.update(sh_h=h[P:], sh_hq=hq[P:], sh_hs=hs[P:])
    return res


def moe_decode_layer_noalloc(x, w13, s13, w2, s2, *, logits=None, topk_ids=None, topk_w=None, top_k: int = 8,
                             router_w=None, shared=None, out=None, status=None):
    """moe_decode_layer through the allocation-free entry point: the layer's
    workspace is the library's static per-GPU scratch, so the call itself
    allocates nothing on the device when ``out``, the routing buffers and
    ``status`` (int32 [4], receives the call's device-side status in element 0)
    are passed in.  Calls that overlap in time on one GPU race."""
    _need(x, torch.bfloat16, 2, "x")
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    dev = x.device
    if router_w is not None or logits is not None:
        if topk_ids is None:
            topk_ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
            topk_w = torch.empty((M, top_k), dtype=torch.float32, device=dev)
    else:
        top_k = topk_ids.shape[1]
    lg = logits
    if router_w is not None and lg is None:
        lg = torch.empty((M, E), dtype=torch.float32, device=dev)
    sh = tuple(shared) if shared is not None else (None,) * 4
    y = out if out is not None else torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    st = status if status is not None else torch.zeros(4, dtype=torch.int32, device=dev)
    _check(lib().moe_decode_layer_noalloc(_p(x), M, H, _p(router_w), _p(lg), _p(topk_ids), _p(topk_w), E, top_k, I,
                                          _p(w13), _p(s13), _p(w2), _p(s2), _p(sh[0]), _p(sh[1]), _p(sh[2]), _p(sh[3]),
                                          _p(y), None, None, None, _p(st), _stream()), "moe_decode_layer_noalloc")
    return {"out": y, "topk_ids": topk_ids, "topk_w": topk_w, "status": st, "logits": lg}


class MoeLayerCall:
    """A prepared MoE layer call for repeated decode steps: output, routing and
    workspace buffers are allocated once and the raw pointers resolved up front,
    so each step is one C call (argument marshalling only).  With ``router_w``
    (bf16 [E,H]) the router GEMV runs in the launch and a step takes only x;
    ``shared`` = (w13, s13, w2, s2) adds a shared expert."""

    def __init__(self, w13, s13, w2, s2, M: int, top_k: int = 8, debug: bool = False, router_w=None,
                 shared=None):
        _need(w13, torch.uint8, 3, "w13")
        _need(s13, torch.float32, 3, "s13")
        _need(w2, torch.uint8, 3, "w2")
        _need(s2, torch.float32, 3, "s2")
        self.E, two_i, self.H = w13.shape
        self.I = two_i // 2
        self.M, self.top_k = M, top_k
        dev = w13.device
        self.w = (w13, s13, w2, s2)
        self.out = torch.empty((M, self.H), dtype=torch.bfloat16, device=dev)
        self.topk_ids = torch.empty((M, top_k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((M, top_k), dtype=torch.float32, device=dev)
        nb = moe_workspace_bytes(M, self.H, self.I, self.E, top_k)
        if nb == 0:
            raise PqError("moe_decode_layer_workspace", -2)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        npairs = M * top_k + (M if shared is not None else 0)
        self.h = torch.empty((npairs, self.I), dtype=torch.bfloat16, device=dev) if debug else None
        self.hq = torch.empty((npairs, self.I), dtype=torch.uint8, device=dev) if debug else None
        self.hs = torch.empty((npairs, self.I // 128), dtype=torch.float32, device=dev) if debug else None
        if router_w is not None:
            _need(router_w, torch.bfloat16, 2, "router_w")
        self.router_w = router_w
        self.logits = torch.empty((M, self.E), dtype=torch.float32, device=dev) if router_w is not None else None
        self.shared = tuple(shared) if shared is not None else (None,) * 4
        self._fn = lib().moe_decode_layer_ex
        _check(lib().pq_workspace_init(_p(self.ws), nb, _stream()), "pq_workspace_init")
        self._fixed = [_p(t) for t in (w13, s13, w2, s2, *self.shared, self.out, self.h, self.hq, self.hs, self.ws)]
        self._ids, self._w = _p(self.topk_ids), _p(self.topk_w)
        self._wr = _p(router_w)
        self._lg = _p(self.logits)

    def __call__(self, x, logits=None, stream=None):
        """x bf16 [M,H] (and logits fp32 [M,E] unless the router runs in the
        launch), contiguous device tensors.  Returns ``out``."""
        w13, s13, w2, s2, a, b, c, d, out, h, hq, hs, ws = self._fixed
        lg = self._lg if self.router_w is not None else _p(logits)
        st = self._fn(_p(x), self.M, self.H, self._wr, lg, self._ids, self._w, self.E, self.top_k, self.I,
                      w13, s13, w2, s2, a, b, c, d, out, h, hq, hs, ws, self.ws.numel(),
                      ctypes.c_void_p(stream) if stream is not None else _stream())
        if st != 0:
            raise PqError("moe_decode_layer_ex", st)
        return self.out

    def check(self) -> int:
        return lib().pq_workspace_check(_p(self.ws), _stream())
