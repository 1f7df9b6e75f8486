"""CPU checks of the C ABI: the library loads, exports every function that
include/pq.h declares, and validates arguments on the host before touching
the GPU."""
import ctypes
import os

import pytest

from quantized_moe_weight_amd import _lib

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libpqmoe.so not built", allow_module_level=True)

PQ_OK, PQ_ERR_NULL, PQ_ERR_SHAPE, PQ_ERR_ALIGN, PQ_ERR_WORKSPACE, PQ_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5

FAKE = ctypes.c_void_p(1 << 20)          # non-null, 16-byte aligned; never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 8)     # misaligned
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_header_function_is_exported(lib):
    names = _lib.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_strerror_covers_every_status(lib):
    for st in range(-9, 1):
        assert b"unknown" not in lib.pq_strerror(st)


def test_launches_per_call_per_entry_point(lib):
    """Every compute entry point is one launch, except pq_gemm_fp8 (the
    activation quantisation, then the GEMM)."""
    f = lib.pq_launches_per_call
    assert f(b"pq_gemm_fp8") == 2
    for name in (b"pq_gemv_fp8", b"pq_gemv_q4", b"moe_decode_layer", b"moe_decode_layer_ex", b"moe_decode_layer_noalloc",
                 b"pq_gemm_fp8_prequant", b"pq_quantize_fp8", b"pq_quantize_q4", b"pq_stream_probe"):
        assert f(name) == 1, name
    assert f(b"pq_strerror") == PQ_ERR_UNSUPPORTED
    assert f(None) == PQ_ERR_NULL


def test_moe_layer_config_host_validation(lib):
    k, al, lds = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_size_t(0)
    g = lib.moe_decode_layer_config
    assert g(1, 6144, 2048, 256, 8, 0, NUL, ctypes.byref(al), ctypes.byref(lds)) == PQ_ERR_NULL
    assert g(0, 6144, 2048, 256, 8, 0, ctypes.byref(k), ctypes.byref(al), ctypes.byref(lds)) == PQ_ERR_SHAPE
    assert g(1, 6000, 2048, 256, 8, 0, ctypes.byref(k), ctypes.byref(al), ctypes.byref(lds)) == PQ_ERR_SHAPE
    # valid shapes stop at the device query on a machine without a gfx950 device
    st = g(8, 6144, 2048, 256, 8, 0, ctypes.byref(k), ctypes.byref(al), ctypes.byref(lds))
    assert st in (PQ_OK, PQ_ERR_UNSUPPORTED, -6)


def test_gemv_fp8_host_validation(lib):
    g = lib.pq_gemv_fp8
    args = lambda x=FAKE, M=1, K=512, w=FAKE, s=FAKE, N=256, epi=0, y=FAKE: (  # noqa: E731
        x, M, K, w, s, N, epi, y, NUL, NUL, NUL, 0, NUL)
    assert g(*args(x=NUL)) == PQ_ERR_NULL
    assert g(*args(y=NUL)) == PQ_ERR_NULL
    assert g(*args(M=0)) == PQ_ERR_SHAPE
    assert g(*args(M=9)) == PQ_ERR_SHAPE
    assert g(*args(K=500)) == PQ_ERR_SHAPE
    assert g(*args(K=32768)) == PQ_ERR_SHAPE
    assert g(*args(N=0)) == PQ_ERR_SHAPE
    assert g(*args(epi=1, N=255)) == PQ_ERR_SHAPE
    assert g(*args(epi=7)) == PQ_ERR_SHAPE
    assert g(*args(w=MIS)) == PQ_ERR_ALIGN
    # valid arguments on a machine without a gfx950 device stop before any launch
    assert g(*args()) in (PQ_ERR_UNSUPPORTED, PQ_OK) or g(*args()) < 0


def test_quantizers_host_validation(lib):
    assert lib.pq_quantize_fp8(NUL, 0, 1, 128, FAKE, FAKE, NUL) == PQ_ERR_NULL
    assert lib.pq_quantize_fp8(FAKE, 0, 1, 100, FAKE, FAKE, NUL) == PQ_ERR_SHAPE
    assert lib.pq_quantize_fp8(FAKE, 0, 0, 128, FAKE, FAKE, NUL) == PQ_ERR_SHAPE
    assert lib.pq_quantize_fp8(MIS, 0, 1, 128, FAKE, FAKE, NUL) == PQ_ERR_ALIGN
    assert lib.pq_quantize_q4(FAKE, 1, 48, FAKE, FAKE, NUL) == PQ_ERR_SHAPE
    assert lib.pq_quantize_q4(NUL, 1, 64, FAKE, FAKE, NUL) == PQ_ERR_NULL


def test_stream_probe_host_validation(lib):
    assert lib.pq_stream_probe(NUL, 64, FAKE, NUL) == PQ_ERR_NULL
    assert lib.pq_stream_probe(FAKE, 64, NUL, NUL) == PQ_ERR_NULL
    assert lib.pq_stream_probe(MIS, 64, FAKE, NUL) == PQ_ERR_ALIGN
    assert lib.pq_stream_probe(FAKE, 0, FAKE, NUL) == PQ_ERR_SHAPE
    assert lib.pq_stream_probe(FAKE, 40, FAKE, NUL) == PQ_ERR_SHAPE


def test_workspace_helpers_host_validation(lib):
    assert lib.pq_workspace_init(NUL, 0, NUL) == PQ_OK
    assert lib.pq_workspace_init(NUL, 64, NUL) == PQ_ERR_NULL
    assert lib.pq_workspace_init(MIS, 64, NUL) == PQ_ERR_ALIGN
    assert lib.pq_workspace_check(NUL, NUL) == PQ_ERR_NULL


def test_gemv_q4_host_validation(lib):
    g = lib.pq_gemv_q4
    args = lambda x=FAKE, M=1, K=512, w=FAKE, s=FAKE, N=256, epi=0, y=FAKE, ws=NUL, wsn=0: (  # noqa: E731
        x, M, K, w, s, N, epi, y, ws, wsn, NUL)
    assert g(*args(x=NUL)) == PQ_ERR_NULL
    assert g(*args(s=NUL)) == PQ_ERR_NULL
    assert g(*args(M=0)) == PQ_ERR_SHAPE
    assert g(*args(M=9)) == PQ_ERR_SHAPE
    assert g(*args(K=48)) == PQ_ERR_SHAPE
    assert g(*args(epi=1, N=7)) == PQ_ERR_SHAPE
    assert g(*args(y=MIS)) == PQ_ERR_ALIGN


def _moe_ex_args(x=FAKE, M=1, H=512, wr=NUL, lg=FAKE, ids=FAKE, w=FAKE, E=16, k=4, I=256,
                 sh=(NUL, NUL, NUL, NUL), out=FAKE, ws=FAKE, wsn=1 << 30):
    return (x, M, H, wr, lg, ids, w, E, k, I, FAKE, FAKE, FAKE, FAKE, *sh, out, NUL, NUL, NUL, ws, wsn, NUL)


def test_moe_layer_host_validation(lib):
    g = lib.moe_decode_layer_ex
    a = _moe_ex_args
    assert g(*a(x=NUL)) == PQ_ERR_NULL
    assert g(*a(ws=NUL)) == PQ_ERR_NULL
    assert g(*a(sh=(FAKE, FAKE, NUL, FAKE))) == PQ_ERR_NULL      # the shared expert: all four or none
    assert g(*a(M=0)) == PQ_ERR_SHAPE
    assert g(*a(M=9)) == PQ_ERR_SHAPE
    assert g(*a(k=9)) == PQ_ERR_SHAPE
    assert g(*a(E=3)) == PQ_ERR_SHAPE                              # fewer experts than top_k
    assert g(*a(E=2000)) == PQ_ERR_SHAPE
    assert g(*a(H=500)) == PQ_ERR_SHAPE
    assert g(*a(I=200)) == PQ_ERR_SHAPE
    assert g(*a(x=MIS)) == PQ_ERR_ALIGN
    assert g(*a(wr=MIS)) == PQ_ERR_ALIGN
    assert g(*a(wsn=1024)) == PQ_ERR_WORKSPACE
    # the plain entry point forwards to the same checks
    p = lib.moe_decode_layer
    assert p(NUL, 1, 512, FAKE, FAKE, FAKE, 16, 4, 256, FAKE, FAKE, FAKE, FAKE, FAKE, NUL, NUL, NUL, FAKE,
             1 << 30, NUL) == PQ_ERR_NULL
    assert p(FAKE, 1, 512, FAKE, FAKE, FAKE, 16, 4, 256, FAKE, FAKE, FAKE, FAKE, FAKE, NUL, NUL, NUL, FAKE,
             1024, NUL) == PQ_ERR_WORKSPACE


def test_moe_workspace_sizes(lib):
    ws = lib.moe_decode_layer_workspace
    assert ws(1, 6144, 2048, 256, 8) > 0
    assert ws(8, 6144, 2048, 256, 8) >= ws(1, 6144, 2048, 256, 8)
    assert ws(0, 6144, 2048, 256, 8) == 0
    assert ws(1, 6144, 2000, 256, 8) == 0


def test_gemm_fp8_host_validation(lib):
    g = lib.pq_gemm_fp8
    args = lambda x=FAKE, M=64, K=512, w=FAKE, s=FAKE, N=256, epi=0, y=FAKE, ws=FAKE, wsn=1 << 30: (  # noqa: E731
        x, M, K, w, s, N, epi, y, ws, wsn, NUL)
    assert g(*args(x=NUL)) == PQ_ERR_NULL
    assert g(*args(M=0)) == PQ_ERR_SHAPE
    assert g(*args(K=300)) == PQ_ERR_SHAPE
    assert g(*args(epi=1, N=255)) == PQ_ERR_SHAPE
    assert g(*args(w=MIS)) == PQ_ERR_ALIGN
    assert g(*args(ws=NUL)) == PQ_ERR_WORKSPACE
    assert g(*args(wsn=4096)) == PQ_ERR_WORKSPACE
    assert lib.pq_gemm_fp8_workspace(64, 512, 256, 0) >= 64 * 512 + 64 * 4 * 4
    assert lib.pq_gemm_fp8_workspace(64, 500, 256, 0) == 0
    q = lib.pq_gemm_fp8_prequant
    assert q(NUL, FAKE, 64, 512, FAKE, FAKE, 256, 0, FAKE, NUL) == PQ_ERR_NULL
    assert q(FAKE, FAKE, 64, 512, FAKE, FAKE, 256, 3, FAKE, NUL) == PQ_ERR_SHAPE
    assert q(FAKE, MIS, 64, 512, FAKE, FAKE, 256, 0, FAKE, NUL) == PQ_ERR_ALIGN


def test_moe_noalloc_host_validation(lib):
    """The allocation-free layer entry point validates like the workspace form
    and refuses, before touching the device, a call whose layer needs more
    than its 4 MiB static scratch."""
    g = lib.moe_decode_layer_noalloc

    def a(x=FAKE, M=1, H=512, E=16, k=4, I=256, status=NUL, sh=(NUL, NUL, NUL, NUL)):
        return (x, M, H, NUL, FAKE, FAKE, FAKE, E, k, I, FAKE, FAKE, FAKE, FAKE, *sh, FAKE, NUL, NUL, NUL, status, NUL)
    PQ_ERR_SCRATCH = -9
    assert g(*a(x=NUL)) == PQ_ERR_NULL
    assert g(*a(sh=(FAKE, NUL, NUL, NUL))) == PQ_ERR_NULL
    assert g(*a(M=9)) == PQ_ERR_SHAPE
    assert g(*a(status=MIS)) == PQ_ERR_ALIGN
    # 8 tokens x 8 slots (+ the shared pair each) at I = 14208: 2.05 MB of h on top of 2.06 MB of fixed
    # regions, a valid workspace-form call (I = 14080 still fits)
    assert lib.moe_decode_layer_workspace(8, 1024, 14208, 16, 8) > 4 << 20
    assert g(*a(M=8, H=1024, I=14208, k=8)) == PQ_ERR_SCRATCH
    assert lib.moe_decode_layer_workspace(8, 1024, 14080, 16, 8) <= 4 << 20
    assert g(*a(M=8, H=1024, I=14080, k=8)) in (PQ_OK, PQ_ERR_UNSUPPORTED, -6)
    # the bench's shapes fit
    assert lib.moe_decode_layer_workspace(8, 6144, 2048, 256, 8) <= 4 << 20
    assert g(*a(M=8, H=6144, I=2048, E=256, k=8)) in (PQ_OK, PQ_ERR_UNSUPPORTED, -6)


def test_gemv_q4_group_host_validation(lib):
    from quantized_moe_weight_amd._lib import Q4Linear
    g = lib.pq_gemv_q4_group
    n = ctypes.c_int(-1)

    def arr(*items):
        a = (Q4Linear * len(items))()
        for i, it in enumerate(items):
            a[i] = Q4Linear(*it)
        return a
    good = (1 << 20, 1 << 20, 1 << 20, 1 << 20, 512, 256, 0)
    assert g(NUL, 0, 1, ctypes.byref(n), NUL) == PQ_OK and n.value == 0     # nothing to do
    assert g(NUL, 2, 1, ctypes.byref(n), NUL) == PQ_ERR_NULL
    assert g(arr(good), -1, 1, NUL, NUL) == PQ_ERR_SHAPE
    assert g(arr(good, (0, 1 << 20, 1 << 20, 1 << 20, 512, 256, 0)), 2, 1, NUL, NUL) == PQ_ERR_NULL
    assert g(arr(good, (1 << 20, 1 << 20, 1 << 20, 1 << 20, 500, 256, 0)), 2, 1, NUL, NUL) == PQ_ERR_SHAPE
    assert g(arr(good, (1 << 20, 1 << 20, 1 << 20, 1 << 20, 512, 255, 1)), 2, 1, NUL, NUL) == PQ_ERR_SHAPE
    assert g(arr(good), 1, 9, NUL, NUL) == PQ_ERR_SHAPE
    assert g(arr(good, ((1 << 20) + 8, 1 << 20, 1 << 20, 1 << 20, 512, 256, 0)), 2, 1, NUL, NUL) == PQ_ERR_ALIGN
    st = g(arr(good, good), 2, 1, ctypes.byref(n), NUL)
    assert st in (PQ_OK, PQ_ERR_UNSUPPORTED, -6)
