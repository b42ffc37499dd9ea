"""C ABI checks that need no GPU: the library loads, exports every function
include/flashnorm.h declares, sizes the packed layout, picks kernel instances
by the M-ladder, and rejects bad arguments before any HIP call."""
import ctypes
import math

import pytest

import rmsnorm_projection_gemm_amd as fn

F32, BF16 = fn.FN_F32, fn.FN_BF16
OK, NULL, SHAPE, ALIGN, DTYPE, EPS, ALIAS = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def lib():
    return fn.load()


def test_exports_every_declared_symbol(lib):
    declared = fn.header_functions()
    assert set(declared) >= {"fn_fold_weights", "fn_norm_proj", "fn_norm_proj_swiglu"}
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in flashnorm.h but not exported"
    # the raw symbol table as well (not only the ctypes wrappers)
    handle = ctypes.CDLL(fn.LIB_PATH)
    for name in declared:
        ctypes.cast(getattr(handle, name), ctypes.c_void_p)


@pytest.mark.parametrize("K,N,dt", [(8, 1, BF16), (4096, 12288, BF16), (40, 37, BF16), (256, 768, F32),
                                    (24, 17, F32), (4096, 0, BF16)])
def test_packed_weight_bytes(lib, K, N, dt):
    kb = 16 if dt == F32 else 32
    assert lib.fn_packed_weight_bytes(K, N, dt) == math.ceil(N / 16) * math.ceil(K / kb) * 1024


@pytest.mark.parametrize("K,N,dt", [(0, 16, BF16), (12, 16, BF16), ((1 << 20) + 8, 16, BF16),
                                    (16, -1, BF16), (16, (1 << 24) + 1, F32), (16, 16, 9)])
def test_packed_weight_bytes_invalid(lib, K, N, dt):
    assert lib.fn_packed_weight_bytes(K, N, dt) == 0


@pytest.mark.parametrize("M,name", [(1, "m16"), (8, "m16"), (16, "m16"), (17, "m32"), (32, "m32"),
                                    (33, "m64"), (64, "m64")])
def test_m_ladder(lib, M, name):
    got = lib.fn_kernel_name(M, 4096, 12288, 0, BF16).decode()
    assert name in got and got.startswith("decode_bf16"), got
    assert lib.fn_kernel_name(M, 4096, 11008, 1, BF16).decode().startswith("decode_swiglu_bf16")


def test_rows_just_past_decode_on_wide_projections(lib):
    # 65..128 rows with at least 512 column blocks: the 128-row rung of the
    # LDS-shared-x decode kernel; 129..256 rows: 128-row prefill tiles; more
    # rows or narrower N: the 256-row prefill tiles
    assert lib.fn_kernel_name(65, 4096, 12288, 0, BF16).decode().startswith("decode_bf16_m128")
    assert lib.fn_kernel_name(128, 4096, 11008, 1, BF16).decode().startswith("decode_swiglu_bf16_m128")
    assert lib.fn_kernel_name(129, 4096, 12288, 0, BF16).decode() == "prefill_bf16_128x128_w4x2"
    assert lib.fn_kernel_name(256, 4096, 11008, 1, BF16).decode() == "prefill_swiglu_bf16_128x128_w4x2"
    assert lib.fn_kernel_name(257, 4096, 12288, 0, BF16).decode().startswith("prefill_bf16_256x")
    # narrow projections (< 512 column blocks): the 64-row rung tiled over the
    # rows up to 256 rows (512 at 192 column blocks or fewer); a narrow SwiGLU
    # pair whose 64-row blocks give at most 256 workgroups: the register-x
    # kernel with a k-split
    assert lib.fn_kernel_name(96, 4096, 8176, 0, BF16).decode() == "decode_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name(256, 4096, 8176, 0, BF16).decode() == "decode_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name(257, 4096, 8176, 0, BF16).decode().startswith("prefill_bf16_256x")
    assert lib.fn_kernel_name(512, 4096, 3072, 0, BF16).decode() == "decode_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name(513, 4096, 3072, 0, BF16).decode().startswith("prefill_bf16_256x128")
    assert lib.fn_kernel_name(128, 4096, 1376, 1, BF16).decode() == "decode_swiglu_bf16_m64_n16_k4_u2"
    assert lib.fn_kernel_name(129, 4096, 1376, 1, BF16).decode() == "decode_swiglu_bf16_m64_xlds_w3_u2"
    assert lib.fn_kernel_name(65, 4096, 2752, 1, BF16).decode() == "decode_swiglu_bf16_m64_xlds_w3_u2"


def test_prefill_w_direct_selection(lib):
    # plain projections over at least 256 tiles of 256 rows with K >= 4096
    # load their W' fragments straight into registers; shorter k loops,
    # smaller grids, SwiGLU pairs and AdaLN keep the LDS ring
    assert lib.fn_kernel_name(4096, 4096, 12288, 0, BF16).decode() == "prefill_bf16_256x256_w2x4_wd"
    assert lib.fn_kernel_name(4096, 4096, 11008, 1, BF16).decode() == "prefill_swiglu_bf16_256x128_w4x2_xl"
    assert lib.fn_kernel_name(8192, 4096, 4096, 0, BF16).decode() == "prefill_bf16_256x256_w2x4_wd"
    assert lib.fn_kernel_name(2000, 1064, 4100, 0, BF16).decode() == "prefill_bf16_256x256_w4x2_xl"
    assert lib.fn_kernel_name(2000, 1064, 2100, 1, BF16).decode() == "prefill_swiglu_bf16_256x128_w4x2_xl"
    assert lib.fn_kernel_name(1000, 4000, 1000, 1, BF16).decode() == "prefill_swiglu_bf16_256x128_w4x2_xl"
    assert lib.fn_kernel_name(1000, 4000, 3000, 0, BF16).decode() == "prefill_bf16_256x128_w4x2_xl"
    assert lib.fn_kernel_name_q8(4096, 4096, 11008, 0).decode() == "prefill_swiglu_bf16_q8_256x128_w4x2_xl"
    assert lib.fn_kernel_name_q8(2000, 2056, 2100, 0).decode() == "prefill_swiglu_bf16_q8_256x128_w4x2_xl"
    assert lib.fn_kernel_name(2000, 2056, 4100, 0, BF16).decode() == "prefill_bf16_256x256_w4x2_xl"
    assert lib.fn_kernel_name(2000, 4104, 4100, 0, BF16).decode() == "prefill_bf16_256x256_w4x2_xl"
    assert lib.fn_kernel_name(4000, 4104, 4100, 0, BF16).decode() == "prefill_bf16_256x256_w2x4_wd"
    assert lib.fn_kernel_name_adaln_ws(4096, 4096, 12288, 4, 0).decode() == "prefill_premod_bf16_256x256_w4x2_xl"
    assert lib.fn_kernel_name(96, 4096, 8192, 0, F32).decode().startswith("decode_f32")


def test_very_wide_projections_take_two_column_blocks_per_wave(lib):
    # up to 16 rows of bf16 with at least 1536 column blocks (an LM head):
    # the register-x decode kernel with two column blocks per wave
    assert lib.fn_kernel_name(16, 4096, 32000, 0, BF16).decode() == "decode_bf16_m16_n32_k1_u4"
    assert lib.fn_kernel_name(1, 4096, 128256, 0, BF16).decode() == "decode_bf16_m16_n32_k1_u4"
    assert lib.fn_kernel_name(8, 4096, 24576, 1, BF16).decode() == "decode_swiglu_bf16_m16_n32_k1_u2"
    assert lib.fn_kernel_name(16, 4096, 24560, 0, BF16).decode() == "decode_bf16_m16_n16_k1_u4"
    assert lib.fn_kernel_name(17, 4096, 32000, 0, BF16).decode().startswith("decode_bf16_m32")
    assert lib.fn_kernel_name(16, 4096, 32000, 0, F32).decode().startswith("decode_f32_m16_n16")


def test_kernel_name_invalid(lib):
    assert lib.fn_kernel_name(0, 4096, 16, 0, BF16) == b"invalid"
    assert lib.fn_kernel_name(4, 12, 16, 0, BF16) == b"invalid"


def _np(lib, x=0x1000, w=0x20000, y=0x40000, M=4, K=16, N=16, eps=1e-6, dt=BF16):
    return lib.fn_norm_proj(x, w, y, M, K, N, eps, dt, None)


def _sw(lib, x=0x1000, wg=0x20000, wu=0x30000, y=0x40000, M=4, K=16, N=16, eps=1e-6, dt=BF16):
    return lib.fn_norm_proj_swiglu(x, wg, wu, y, M, K, N, eps, dt, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(x=None), NULL, "x is NULL"),
    (dict(w=None), NULL, "W_packed"),
    (dict(y=None), NULL, "y is NULL"),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(K=0), SHAPE, "K=0"),
    (dict(K=(1 << 20) + 8), SHAPE, "K="),
    (dict(M=-1), SHAPE, "M=-1"),
    (dict(M=(1 << 22) + 1), SHAPE, "M="),
    (dict(N=-5), SHAPE, "N=-5"),
    (dict(x=0x1008), ALIGN, "x must be 16-byte aligned"),
    (dict(w=0x20004), ALIGN, "packed weights"),
    (dict(y=0x40002), ALIGN, "output"),
    (dict(eps=-1.0), EPS, "eps"),
    (dict(eps=float("nan")), EPS, "eps"),
    (dict(eps=float("inf")), EPS, "eps"),
    (dict(dt=3), DTYPE, "dtype"),
    (dict(y=0x1000), ALIAS, "overlaps"),
    (dict(y=0x1040), ALIAS, "overlaps"),
    (dict(y=0x20000), ALIAS, "overlaps"),
])
def test_norm_proj_rejects(lib, kwargs, status, needle):
    assert _np(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_swiglu_rejects(lib):
    assert _sw(lib, wu=None) == NULL
    assert "W_up_packed" in lib.fn_last_error().decode()
    assert _sw(lib, wg=None) == NULL
    assert _sw(lib, wu=0x30008) == ALIGN
    assert _sw(lib, y=0x30000) == ALIAS
    assert _sw(lib, dt=-1) == DTYPE


def test_empty_calls_touch_nothing(lib):
    # M == 0 or N == 0 is a valid no-op: nothing is launched, pointers unread
    assert _np(lib, x=None, w=None, y=None, M=0) == OK
    assert _np(lib, x=None, w=None, y=None, N=0) == OK
    assert _sw(lib, x=None, wg=None, wu=None, y=None, M=0) == OK
    assert lib.fn_last_error() == b""
    # but shapes are still validated for empty calls
    assert _np(lib, M=0, K=12) == SHAPE


def test_fold_rejects(lib):
    f = lib.fn_fold_weights
    assert f(0x100, None, 0x10000, 16, 16, BF16, None) == NULL
    assert f(0x100, 0x1000, None, 16, 16, BF16, None) == NULL
    assert f(0x101, 0x1000, 0x10000, 16, 16, BF16, None) == ALIGN
    assert f(0x100, 0x1000, 0x10008, 16, 16, BF16, None) == ALIGN
    assert f(0x100, 0x1000, 0x1000, 16, 16, BF16, None) == ALIAS
    assert f(0x100, 0x1000, 0x10000, 20, 16, BF16, None) == SHAPE
    assert f(0x100, 0x1000, 0x10000, 16, 16, 5, None) == DTYPE
    assert f(None, None, None, 16, 0, BF16, None) == OK


def test_chain_helpers_reject(lib):
    assert lib.fn_rmsnorm(None, 0x100, 0x1000, 2, 16, 1e-6, BF16, None) == NULL
    assert lib.fn_rmsnorm(0x1000, 0x100, 0x1000, 2, 16, 1e-6, BF16, None) == ALIAS
    assert lib.fn_rmsnorm(0x1000, 0x100, 0x2000, 2, 16, -1.0, BF16, None) == EPS
    assert lib.fn_silu_mul(0x1000, 0x1000, 2, 8, BF16, None) == ALIAS
    assert lib.fn_silu_mul(0x1001, 0x4000, 2, 8, BF16, None) == ALIGN
    assert lib.fn_silu_mul(None, None, 0, 8, BF16, None) == OK


def test_probes_reject(lib):
    """The measurement probes validate before any HIP call."""
    f = lib.fn_probe_hbm_read
    assert f(None, 1024, 0x1000, 8, None) == NULL
    assert f(0x1000, 1000, 0x1000, 8, None) == SHAPE        # not a multiple of 16
    assert f(0x1000, 0, 0x1000, 8, None) == SHAPE
    assert f(0x1000, 1024, 0x1000, 0, None) == SHAPE
    assert f(0x1000, 1024, 0x1000, 65537, None) == SHAPE
    assert f(0x1008, 1024, 0x1000, 8, None) == ALIGN
    g = lib.fn_probe_mfma_bf16
    assert g(None, 16, 8, None) == NULL
    assert g(0x1000, 0, 8, None) == SHAPE
    assert g(0x1000, (1 << 20) + 1, 8, None) == SHAPE
    assert g(0x1000, 16, 0, None) == SHAPE
    assert g(0x1002, 16, 8, None) == ALIGN


def test_status_strings(lib):
    for s in range(8):
        assert lib.fn_status_string(s)
    assert lib.fn_status_string(99) == b"unknown status"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No CPU fallback: a missing library is an error, not a silent path."""
    monkeypatch.setattr(fn, "_lib", None)
    monkeypatch.setattr(fn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fn.load()


# ------------------------------------------------------------ fp8 weights --
@pytest.mark.parametrize("K,N,want", [(64, 16, 1024), (8, 1, 1024), (72, 17, 4096), (4096, 12288, 50331648)])
def test_packed_fp8_bytes(lib, K, N, want):
    assert lib.fn_packed_fp8_bytes(K, N) == want


@pytest.mark.parametrize("K,N", [(0, 16), (12, 16), (16, -1), ((1 << 20) + 8, 16)])
def test_packed_fp8_bytes_invalid(lib, K, N):
    assert lib.fn_packed_fp8_bytes(K, N) == 0


def test_fp8_kernel_names(lib):
    assert lib.fn_kernel_name_fp8(16, 4096, 12288, 0).decode().startswith("decode_fp8_m16")
    # up to 16 rows of at most 256 column blocks: the register-x tile, k over four waves
    assert lib.fn_kernel_name_fp8(16, 4096, 4096, 0).decode() == "decode_fp8_m16_n16_k4_p4"
    assert lib.fn_kernel_name_fp8(1, 4096, 1376, 1).decode() == "decode_swiglu_fp8_m16_n16_k4_p2"
    assert lib.fn_kernel_name_fp8(16, 4096, 4112, 0).decode().startswith("decode_fp8_m16_xlds")
    assert lib.fn_kernel_name_fp8(17, 4096, 1536, 0).decode().startswith("decode_fp8_m32_xlds")
    assert lib.fn_kernel_name_fp8(17, 4096, 12288, 0).decode().startswith("decode_fp8_m32")
    assert lib.fn_kernel_name_fp8(64, 4096, 11008, 1).decode().startswith("decode_swiglu_fp8_m64")
    # above 64 rows the prefill kernel with fp8 weights
    assert lib.fn_kernel_name_fp8(4096, 4096, 12288, 0).decode() == "prefill_fp8_256x256_w4x2_xl"
    # fewer than 128 tiles of 256 x 256: 256 x 128 tiles
    assert lib.fn_kernel_name_fp8(300, 4096, 12288, 0).decode() == "prefill_fp8_256x128_w4x2_xl"
    # 65..256 rows of a wide projection (>= 512 column blocks): the 64-row
    # decode kernel tiled over the rows; narrower ones too, to 256, 512 or
    # 1024 rows as they narrow
    assert lib.fn_kernel_name_fp8(65, 4096, 12288, 0).decode().startswith("decode_fp8_m64")
    assert lib.fn_kernel_name_fp8(256, 4096, 8192, 1).decode().startswith("decode_swiglu_fp8_m128")
    assert lib.fn_kernel_name_fp8(200, 4096, 8192, 0).decode().startswith("decode_fp8_m64")
    assert lib.fn_kernel_name_fp8(257, 4096, 12288, 0).decode().startswith("prefill_fp8")
    assert lib.fn_kernel_name_fp8(256, 4096, 8176, 0).decode().startswith("decode_fp8_m64")
    assert lib.fn_kernel_name_fp8(257, 4096, 8176, 0).decode().startswith("prefill_fp8")
    assert lib.fn_kernel_name_fp8(512, 4096, 6144, 0).decode().startswith("decode_fp8_m64")
    assert lib.fn_kernel_name_fp8(513, 4096, 6144, 0).decode().startswith("prefill_fp8")
    assert lib.fn_kernel_name_fp8(1024, 4096, 1376, 1).decode().startswith("decode_swiglu_fp8_m128")
    assert lib.fn_kernel_name_fp8(1025, 4096, 1376, 1).decode().startswith("prefill_swiglu_fp8")
    assert lib.fn_kernel_name_fp8(4096, 4096, 12288, 1).decode() == "prefill_swiglu_fp8_256x128_w4x2_xl"
    assert lib.fn_kernel_name_fp8(0, 4096, 16, 0) == b"invalid"


def _np8(lib, x=0x1000, w=0x20000, s=0x30000, y=0x40000, M=4, K=16, N=16, eps=1e-6):
    return lib.fn_norm_proj_fp8(x, w, s, y, M, K, N, eps, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(x=None), NULL, "x is NULL"),
    (dict(w=None), NULL, "W8_packed"),
    (dict(s=None), NULL, "scales"),
    (dict(y=None), NULL, "y is NULL"),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(x=0x1008), ALIGN, "x must be"),
    (dict(w=0x20008), ALIGN, "fp8 weights"),
    (dict(s=0x30002), ALIGN, "scales"),
    (dict(eps=-1.0), EPS, "eps"),
    (dict(y=0x30000), ALIAS, "overlaps"),
    (dict(y=0x20000), ALIAS, "overlaps"),
])
def test_norm_proj_fp8_rejects(lib, kwargs, status, needle):
    assert _np8(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_fp8_swiglu_and_fold_reject(lib):
    sw = lib.fn_norm_proj_swiglu_fp8
    assert sw(0x1000, 0x20000, 0x30000, None, 0x31000, 0x40000, 4, 16, 16, 1e-6, None) == NULL
    assert sw(0x1000, 0x20000, 0x30000, 0x21000, None, 0x40000, 4, 16, 16, 1e-6, None) == NULL
    assert sw(0x1000, 0x20000, 0x30000, 0x21000, 0x31000, 0x31000, 4, 16, 16, 1e-6, None) == ALIAS
    assert sw(None, None, None, None, None, None, 0, 16, 16, 1e-6, None) == OK
    f = lib.fn_fold_weights_fp8
    assert f(0x100, None, 0x10000, 0x20000, 16, 16, BF16, None) == NULL
    assert f(0x100, 0x1000, 0x10000, None, 16, 16, BF16, None) == NULL
    assert f(0x100, 0x1000, 0x10008, 0x20000, 16, 16, BF16, None) == ALIGN
    assert f(0x100, 0x1000, 0x10000, 0x20002, 16, 16, BF16, None) == ALIGN
    assert f(0x100, 0x1000, 0x10000, 0x10000, 16, 16, BF16, None) == ALIAS
    assert f(0x100, 0x1000, 0x1000, 0x20000, 16, 16, BF16, None) == ALIAS
    assert f(0x100, 0x1000, 0x10000, 0x20000, 16, 16, 9, None) == DTYPE
    assert f(None, None, None, None, 16, 0, BF16, None) == OK


def _call(kind=fn.FN_CALL_NORM_PROJ, x=0x1000, wg=0x20000, wu=None, sg=None, su=None, y=0x40000, M=4, K=16, N=16,
          eps=1e-6, dt=BF16, ys=None):
    return fn.FnCall(kind, x, wg, wu, sg, su, y, M, K, N, eps, dt, ys)


def _create(lib, calls):
    arr = (fn.FnCall * max(1, len(calls)))(*calls)
    h = ctypes.c_void_p(0x1234)
    st = lib.fn_step_create(arr, len(calls), ctypes.byref(h))
    return st, h


def test_fn_call_layout_matches_header():
    # kind, 6 pointers, 3 int64, float, enum, pointer: 4 + 4 (pad) + 48 + 24 + 4 + 4 + 8
    assert ctypes.sizeof(fn.FnCall) == 96
    assert fn.FnCall.x.offset == 8 and fn.FnCall.M.offset == 56 and fn.FnCall.eps.offset == 80
    assert fn.FnCall.y_scales.offset == 88


def test_step_create_validates_every_call_first(lib):
    # each bad call is rejected with its entry point's status, prefixed with
    # its index, before any HIP call (none is possible without a GPU)
    st, h = _create(lib, [_call(), _call(K=12)])
    assert st == SHAPE and h.value is None
    assert lib.fn_last_error().decode().startswith("call 1: K=12")
    st, h = _create(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU)])
    assert st == NULL and "call 0: W_up_packed" in lib.fn_last_error().decode()
    st, _ = _create(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_FP8, sg=None)])
    assert st == NULL and "scales" in lib.fn_last_error().decode()
    st, _ = _create(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU_FP8, wu=0x21000, sg=0x30000, su=0x30002)])
    assert st == ALIGN
    st, _ = _create(lib, [_call(y=0x1000)])
    assert st == ALIAS
    st, _ = _create(lib, [_call(eps=-1.0)])
    assert st == EPS
    st, _ = _create(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU_Q8, wu=0x30000)])
    assert st == NULL and "out_scales" in lib.fn_last_error().decode()
    st, _ = _create(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8, wu=0x30000, sg=0x50000, su=0x51000,
                                ys=0x40008)])
    assert st == ALIAS and "out_codes overlaps out_scales" in lib.fn_last_error().decode()
    st, _ = _create(lib, [_call(kind=7)])
    assert st == DTYPE and "call kind" in lib.fn_last_error().decode()
    st, _ = _create(lib, [])
    assert st == SHAPE and "n_calls" in lib.fn_last_error().decode()


def test_step_null_arguments(lib):
    assert lib.fn_step_create(None, 1, ctypes.byref(ctypes.c_void_p())) == NULL
    arr = (fn.FnCall * 1)(_call())
    assert lib.fn_step_create(arr, 1, None) == NULL
    assert lib.fn_step_launch(None, None) == NULL
    assert lib.fn_step_num_kernels(None) == -1
    assert lib.fn_step_destroy(None) == OK


def _create_grouped(lib, calls, n=None):
    arr = (fn.FnCall * max(1, len(calls)))(*calls)
    h = ctypes.c_void_p(0x1234)
    st = lib.fn_step_create_grouped(arr, len(calls) if n is None else n, ctypes.byref(h))
    return st, h


def test_grouped_step_validates_before_any_hip_call(lib):
    # every rejection below is decided on the host, before the call table is
    # allocated (no HIP call is possible without a GPU)
    st, h = _create_grouped(lib, [_call(), _call(K=12)])
    assert st == SHAPE and h.value is None and lib.fn_last_error().decode().startswith("call 1: K=12")
    st, _ = _create_grouped(lib, [_call(), _call(kind=fn.FN_CALL_NORM_PROJ_FP8, x=0x2000, sg=0x30000, y=0x50000)])
    assert st == SHAPE and lib.fn_last_error().decode().startswith("call 1: a grouped step takes calls of one weight")
    st, _ = _create_grouped(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_FP8, sg=0x30000), _call(x=0x2000, y=0x50000)])
    assert st == SHAPE and "one weight type" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU_Q8, wu=0x30000, ys=0x50000)])
    assert st == SHAPE and "their fp8 forms" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [_call(dt=F32)])
    assert st == SHAPE and "bf16 activations of at most 128 rows" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [_call(kind=fn.FN_CALL_NORM_PROJ_SWIGLU_FP8, wu=0x30000, sg=0x50000, su=0x60000,
                                        M=129)])
    assert st == SHAPE and "M=129" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [_call(M=129)])
    assert st == SHAPE and "M=129" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [])
    assert st == SHAPE and "n_calls" in lib.fn_last_error().decode()
    st, _ = _create_grouped(lib, [_call()], n=65536)
    assert st == SHAPE
    assert lib.fn_step_create_grouped(None, 1, ctypes.byref(ctypes.c_void_p())) == NULL
    assert lib.fn_step_create_grouped((fn.FnCall * 1)(_call()), 1, None) == NULL


def test_grouped_step_rejects_calls_that_share_a_written_buffer(lib):
    # x 4x16 bf16 = 128 B, packed 16x16 weights, y 4x16 bf16 = 128 B
    a = dict(x=0x1000, wg=0x20000, y=0x40000)
    b = dict(x=0x2000, wg=0x20000, y=0x50000)            # same weights: read by both, fine
    assert _create_grouped(lib, [_call(M=0, **a), _call(M=0, **b)])[0] == OK
    st, _ = _create_grouped(lib, [_call(**a), _call(x=0x2000, wg=0x30000, y=0x40040)])
    assert st == ALIAS and "at once" in lib.fn_last_error().decode()      # outputs overlap
    st, _ = _create_grouped(lib, [_call(**a), _call(x=0x40000, wg=0x30000, y=0x50000)])
    assert st == ALIAS                                                      # call 1 reads call 0's output
    st, _ = _create_grouped(lib, [_call(**a), _call(x=0x2000, wg=0x30000, y=0x20010)])
    assert st == ALIAS                                                      # call 1 writes call 0's weights
    # a wide input of one call spanning another call's output, with a third
    # call's buffers between them
    st, _ = _create_grouped(lib, [_call(x=0x1000, M=16, K=1024, wg=0x90000, y=0xa0000),
                                  _call(x=0x1100, wg=0x30000, y=0x3000, M=4, K=16, N=16),
                                  _call(x=0x2800, wg=0xb0000, y=0xc0000)])
    assert st == ALIAS
    # fp8 calls: the column scales are inputs too (16 columns: 64 B)
    f8 = fn.FN_CALL_NORM_PROJ_FP8
    st, _ = _create_grouped(lib, [_call(kind=f8, sg=0x30000, M=0),
                                  _call(kind=f8, x=0x2000, sg=0x30000, y=0x50000, M=0)])
    assert st == OK                                                         # shared scales, both read
    st, _ = _create_grouped(lib, [_call(kind=f8, sg=0x30000),
                                  _call(kind=f8, x=0x2000, wg=0x60000, sg=0x70000, y=0x30020)])
    assert st == ALIAS and "at once" in lib.fn_last_error().decode()      # call 1 writes call 0's scales


@pytest.mark.parametrize("fp8", [False, True])
def test_grouped_overlap_check_matches_brute_force(lib, fp8):
    """Random groups of individually valid calls packed into a small address
    range: the grouped step refuses them (FN_ERR_ALIAS) exactly when some
    output of one call overlaps a buffer of another call, which a pairwise
    comparison decides here.  Groups it accepts go on to allocate their
    table (FN_ERR_HIP without a GPU, FN_OK with one)."""
    import random
    rng = random.Random(17 + fp8)
    HIP = 7
    base, arena = 0x100000, 1 << 16

    def packed(K, N):
        return (N + 15) // 16 * ((K + 63) // 64 if fp8 else (K + 31) // 32) * 1024

    def hit(a, b):
        return a[0] < b[0] + b[1] and b[0] < a[0] + a[1]

    seen = {True: 0, False: 0}
    for trial in range(400):
        calls, spans = [], []
        for i in range(rng.randint(2, 5)):
            sw = rng.random() < 0.5
            M, K, N = rng.randint(1, 128 if trial % 2 else 16), 8 * rng.randint(1, 12), rng.randint(1, 40)
            while True:
                at = lambda: base + 16 * rng.randrange(arena // 16)
                x, wg, wu, sg, su, y = at(), at(), at(), at(), at(), at()
                ins = [(x, M * K * 2), (wg, packed(K, N))] + ([(wu, packed(K, N))] if sw else [])
                if fp8:
                    ins += [(sg, N * 4)] + ([(su, N * 4)] if sw else [])
                out = (y, M * N * 2)
                if not any(hit(out, b) for b in ins):   # each call valid on its own
                    break
            kind = ((fn.FN_CALL_NORM_PROJ_SWIGLU_FP8 if sw else fn.FN_CALL_NORM_PROJ_FP8) if fp8 else
                    (fn.FN_CALL_NORM_PROJ_SWIGLU if sw else fn.FN_CALL_NORM_PROJ))
            calls.append(_call(kind=kind, x=x, wg=wg, wu=wu if sw else None, sg=sg if fp8 else None,
                               su=su if fp8 and sw else None, y=y, M=M, K=K, N=N))
            spans.append((ins, out))
        conflict = any(hit(spans[i][1], b) for i in range(len(spans)) for j in range(len(spans)) if i != j
                       for b in spans[j][0] + [spans[j][1]])
        st, h = _create_grouped(lib, calls)
        if st == OK:
            assert lib.fn_step_destroy(h) == OK
        assert (st == ALIAS) == conflict, (trial, st, lib.fn_last_error())
        assert st in (ALIAS, OK, HIP), (trial, st, lib.fn_last_error())
        seen[conflict] += 1
    assert min(seen.values()) >= 40, seen   # both outcomes well represented


def test_grouped_step_of_empty_calls_launches_nothing(lib):
    st, h = _create_grouped(lib, [_call(M=0), _call(N=0, kind=fn.FN_CALL_NORM_PROJ_SWIGLU, wu=0x30000)])
    assert st == OK and h.value is not None
    assert lib.fn_step_num_kernels(h) == 0
    assert lib.fn_step_launch(h, None) == OK
    assert lib.fn_step_destroy(h) == OK


def _q8(lib, x=0x1000, wg=0x20000, wu=0x30000, c=0x40000, s=0x50000, M=4, K=16, N=16, eps=1e-6):
    return lib.fn_norm_proj_swiglu_q8(x, wg, wu, c, s, M, K, N, eps, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(x=None), NULL, "x is NULL"),
    (dict(wu=None), NULL, "gate or up"),
    (dict(c=None), NULL, "out_codes"),
    (dict(s=None), NULL, "out_scales"),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(x=0x1008), ALIGN, "x must be"),
    (dict(wg=0x20008), ALIGN, "packed weights"),
    (dict(s=0x50002), ALIGN, "out_scales"),
    (dict(eps=float("nan")), EPS, "eps"),
    (dict(c=0x1000), ALIAS, "overlaps"),
    (dict(s=0x30000), ALIAS, "overlaps"),
    (dict(s=0x40000), ALIAS, "out_codes overlaps out_scales"),
])
def test_swiglu_q8_rejects(lib, kwargs, status, needle):
    assert _q8(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_swiglu_q8_codes_need_no_alignment_and_empty_is_ok(lib):
    # odd code addresses pass validation (byte stores); empty calls read nothing
    assert _q8(lib, x=None, wg=None, wu=None, c=None, s=None, M=0) == OK
    f = lib.fn_norm_proj_swiglu_fp8_q8
    assert f(0x1000, 0x20000, None, 0x30000, 0x31000, 0x40001, 0x50000, 4, 16, 16, 1e-6, None) == NULL
    assert "s_gate" in lib.fn_last_error().decode()
    assert f(0x1000, 0x20000, 0x21000, 0x30000, 0x31002, 0x40001, 0x50000, 4, 16, 16, 1e-6, None) == ALIGN


def test_q8_kernel_names(lib):
    assert lib.fn_kernel_name_q8(16, 4096, 11008, 0).decode() == "decode_swiglu_bf16_q8_m16_xlds_w3_u2"
    assert lib.fn_kernel_name_q8(64, 4096, 11008, 0).decode().startswith("decode_swiglu_bf16_q8_m64")
    # past 64 rows of projections with at least 512 column blocks: the 64-row
    # tiles repeated over the rows, up to 128 rows (bf16 weights) or 256 (fp8)
    assert lib.fn_kernel_name_q8(65, 4096, 11008, 0).decode().startswith("decode_swiglu_bf16_q8_m64")
    assert lib.fn_kernel_name_q8(128, 4096, 8192, 0).decode().startswith("decode_swiglu_bf16_q8_m64")
    assert lib.fn_kernel_name_q8(129, 4096, 11008, 0).decode() == "prefill_swiglu_bf16_q8_128x128_w4x2"
    assert lib.fn_kernel_name_q8(257, 4096, 11008, 0).decode() == "prefill_swiglu_bf16_q8_256x128_w4x2_xl"
    assert lib.fn_kernel_name_q8(256, 4096, 8176, 0).decode().startswith("decode_swiglu_bf16_q8_m64")
    assert lib.fn_kernel_name_q8(257, 4096, 8176, 0).decode().startswith("prefill_swiglu_bf16_q8")
    assert lib.fn_kernel_name_q8(512, 4096, 2752, 0).decode().startswith("decode_swiglu_bf16_q8_m64")
    assert lib.fn_kernel_name_q8(256, 4096, 11008, 1).decode().startswith("decode_swiglu_fp8_q8_m64")
    assert lib.fn_kernel_name_q8(257, 4096, 11008, 1).decode().startswith("prefill_swiglu_fp8_q8")
    assert lib.fn_kernel_name_q8(257, 4096, 8176, 1).decode().startswith("prefill_swiglu_fp8_q8")
    assert lib.fn_kernel_name_q8(1024, 4096, 1376, 1).decode().startswith("decode_swiglu_fp8_q8_m64")
    assert lib.fn_kernel_name_q8(64, 4096, 11008, 1).decode().startswith("decode_swiglu_fp8_q8_m64")
    assert lib.fn_kernel_name_q8(4096, 4096, 11008, 1).decode() == "prefill_swiglu_fp8_q8_256x128_w4x2_xl"
    assert lib.fn_kernel_name_q8(0, 4096, 16, 0) == b"invalid"


def _ad(lib, x=0x1000, sc=0x10000, idx=0x18000, w=0x20000, b=0x30000, y=0x40000, M=4, K=16, N=16, T=2, eps=1e-6):
    return lib.fn_norm_proj_adaln(x, sc, idx, w, b, y, M, K, N, T, eps, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(x=None), NULL, "x, mod or idx"),
    (dict(sc=None), NULL, "x, mod or idx"),
    (dict(idx=None), NULL, "x, mod or idx"),
    (dict(w=None), NULL, "W_packed or bias"),
    (dict(b=None), NULL, "W_packed or bias"),
    (dict(y=None), NULL, "y is NULL"),
    (dict(T=0), SHAPE, "T=0"),
    (dict(T=1 << 27, K=16), SHAPE, "T="),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(sc=0x10008), ALIGN, "x and mod"),
    (dict(M=17), SHAPE, "at most 16 rows"),
    (dict(idx=0x18002), ALIGN, "idx and bias"),
    (dict(b=0x30002), ALIGN, "idx and bias"),
    (dict(eps=-1.0), EPS, "eps"),
    (dict(y=0x18000), ALIAS, "overlaps"),
    (dict(y=0x30000), ALIAS, "overlaps"),
])
def test_norm_proj_adaln_rejects(lib, kwargs, status, needle):
    assert _ad(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_adaln_swiglu_bias_and_names(lib):
    sw = lib.fn_norm_proj_swiglu_adaln
    assert sw(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, None, 0x31000, 0x40000, 4, 16, 16, 2, 1e-6, None) == NULL
    assert sw(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, 0x21000, None, 0x40000, 4, 16, 16, 2, 1e-6, None) == NULL
    assert sw(None, None, None, None, None, None, None, None, 0, 16, 16, 2, 1e-6, None) == OK
    f = lib.fn_adaln_shift_bias
    assert f(0x1000, 0x2000, None, 2, 16, 16, BF16, None) == NULL
    assert f(0x1001, 0x2000, 0x3000, 2, 16, 16, BF16, None) == ALIGN
    assert f(0x1000, 0x2000, 0x1000, 2, 16, 16, BF16, None) == ALIAS
    assert f(0x1000, 0x2000, 0x3000, 2, 16, 16, 7, None) == DTYPE
    assert f(None, None, None, 0, 16, 16, BF16, None) == OK
    # the one-launch kernel: up to 16 rows
    assert lib.fn_kernel_name_adaln(16, 4096, 11008, 4, 1).decode() == "decode_swiglu_adaln_split_bf16_m16_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln(1, 4096, 12288, 900, 0).decode() == "decode_adaln_bf16_m16_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln(17, 4096, 11008, 4, 0) == b"invalid"
    assert lib.fn_kernel_name_adaln(0, 4096, 16, 4, 0) == b"invalid"


def test_adaln_fold_table_rejects(lib):
    f = lib.fn_adaln_fold_table
    assert f(0x1000, 0x2000, None, 2, 16, BF16, None) == NULL
    assert f(0x1001, 0x2000, 0x3000, 2, 16, BF16, None) == ALIGN
    assert f(0x1000, 0x2000, 0x3002, 2, 16, BF16, None) == ALIGN
    assert f(0x1000, 0x2000, 0x2010, 2, 16, BF16, None) == ALIAS
    assert f(0x1000, 0x2000, 0x3000, 2, 16, 7, None) == DTYPE
    assert f(0x1000, 0x2000, 0x3000, 2, 12, BF16, None) == SHAPE
    assert f(0x1000, 0x2000, 0x3000, 1 << 27, 16, BF16, None) == SHAPE
    assert f(None, None, None, 0, 16, BF16, None) == OK


WORKSPACE = 8


def _adw(lib, x=0x1000, sc=0x10000, idx=0x18000, w=0x20000, b=0x30000, y=0x40000, M=40, K=16, N=16, T=2, eps=1e-6,
         ws=0x100000, wsb=1 << 20):
    return lib.fn_norm_proj_adaln_ws(x, sc, idx, w, b, y, M, K, N, T, eps, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(ws=None), WORKSPACE, "workspace is NULL"),
    (dict(ws=0x100080), WORKSPACE, "256-byte"),
    (dict(wsb=1024), WORKSPACE, "workspace_bytes=1024"),
    (dict(ws=0x40000), ALIAS, "workspace overlaps"),
    (dict(ws=0x1000 - 256), ALIAS, "workspace overlaps"),
    # the one-launch checks come first
    (dict(x=None, ws=None), NULL, "x, mod or idx"),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(T=0), SHAPE, "T=0"),
    (dict(eps=float("nan")), EPS, "eps"),
    (dict(y=0x30000), ALIAS, "output overlaps"),
])
def test_norm_proj_adaln_ws_rejects(lib, kwargs, status, needle):
    assert _adw(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()
    assert lib.fn_status_string(WORKSPACE) == b"workspace missing, misaligned or too small"


def test_adaln_ws_sizes_and_names(lib):
    # the split operand 2*M*K bf16, then one fp32 per row, each rounded up to 256 bytes; none up to 16 rows
    assert lib.fn_adaln_workspace_bytes(16, 4096) == 0
    assert lib.fn_adaln_workspace_bytes(17, 8) == 768 + 256
    assert lib.fn_adaln_workspace_bytes(65, 8) == 2304 + 512
    assert lib.fn_adaln_workspace_bytes(4096, 4096) == 2 * 4096 * 4096 * 2 + 4096 * 4
    assert lib.fn_adaln_workspace_bytes(100, 12) == 0 and lib.fn_adaln_workspace_bytes(-1, 16) == 0
    assert lib.fn_kernel_name_adaln_ws(4096, 4096, 12288, 4, 0).decode() == "prefill_premod_bf16_256x256_w4x2_xl"
    assert (lib.fn_kernel_name_adaln_ws(65, 4096, 11008, 500, 1).decode() ==
            "prefill_swiglu_premod_split_bf16_256x128_w4x2_xl")
    assert lib.fn_kernel_name_adaln_ws(64, 4096, 11008, 4, 1).decode() == "decode_swiglu_premod_split_bf16_m64_xlds_w3_u2"
    # 65..128 rows of wide projections: the 64-row tiles repeated over the rows
    # (not for the split SwiGLU operand)
    assert lib.fn_kernel_name_adaln_ws(65, 4096, 12288, 4, 0).decode() == "decode_premod_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(128, 4096, 8192, 4, 0).decode() == "decode_premod_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(129, 4096, 12288, 4, 0).decode() == "prefill_premod_bf16_128x128_w4x2"
    assert lib.fn_kernel_name_adaln_ws(257, 4096, 12288, 4, 0).decode() == "prefill_premod_bf16_256x256_w4x2_xl"
    assert (lib.fn_kernel_name_adaln_ws(200, 4096, 11008, 4, 1).decode() ==
            "prefill_swiglu_premod_split_bf16_256x128_w4x2_xl")
    assert lib.fn_kernel_name_adaln_ws(256, 4096, 8176, 4, 0).decode() == "decode_premod_bf16_m64_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(257, 4096, 8176, 4, 0).decode().startswith("prefill_premod_bf16")
    assert lib.fn_kernel_name_adaln_ws(65, 4096, 1376, 4, 1).decode().startswith("prefill_swiglu_premod_split")
    assert lib.fn_kernel_name_adaln_ws(16, 4096, 11008, 4, 1).decode() == "decode_swiglu_adaln_split_bf16_m16_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(17, 4096, 12288, 500, 0).decode() == "decode_premod_bf16_m32_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(16, 4096, 12288, 4, 0).decode() == "decode_adaln_bf16_m16_xlds_w3_u2_s5"
    assert lib.fn_kernel_name_adaln_ws(0, 4096, 16, 4, 0) == b"invalid"
    sw = lib.fn_norm_proj_swiglu_adaln_ws
    # SwiGLU: missing up operands, a short workspace, and the empty call (nothing read)
    assert sw(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, None, 0x31000, 0x40000, 100, 16, 16, 2, 1e-6, 0x100000,
              1 << 20, None) == NULL
    assert sw(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, 0x21000, 0x31000, 0x40000, 100, 16, 16, 2, 1e-6, 0x100000,
              16, None) == WORKSPACE
    assert sw(None, None, None, None, None, None, None, None, 0, 16, 16, 2, 1e-6, None, 0, None) == OK


def test_adaln_modulate_rejects(lib):
    f = lib.fn_adaln_modulate
    assert f(None, 0x10000, 0x18000, 0x20000, 0x30000, 4, 16, 2, 1e-6, None) == NULL
    assert f(0x1000, 0x10000, 0x18000, None, 0x30000, 4, 16, 2, 1e-6, None) == NULL
    assert "u or rs" in lib.fn_last_error().decode()
    assert f(0x1000, 0x10000, 0x18000, 0x20008, 0x30000, 4, 16, 2, 1e-6, None) == ALIGN
    assert f(0x1000, 0x10000, 0x18000, 0x20000, 0x30002, 4, 16, 2, 1e-6, None) == ALIGN
    assert f(0x1000, 0x10000, 0x18000, 0x1000, 0x30000, 4, 16, 2, 1e-6, None) == ALIAS
    assert f(0x1000, 0x10000, 0x18000, 0x20000, 0x20010, 4, 16, 2, 1e-6, None) == ALIAS
    assert f(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, 4, 12, 2, 1e-6, None) == SHAPE
    assert f(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, 4, 16, 0, 1e-6, None) == SHAPE
    assert f(0x1000, 0x10000, 0x18000, 0x20000, 0x30000, 4, 16, 2, -1.0, None) == EPS
    assert f(None, None, None, None, None, 0, 16, 2, 1e-6, None) == OK


def _adf(lib, x=0x1000, sc=0x10000, idx=0x18000, w=0x20000, s=0x28000, b=0x30000, y=0x40000, M=4, K=16, N=16, T=2,
         eps=1e-6, ws=0x100000, wsb=512):
    return lib.fn_norm_proj_adaln_fp8_ws(x, sc, idx, w, s, b, y, M, K, N, T, eps, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(ws=None), WORKSPACE, "workspace is NULL"),
    (dict(ws=0x100010), WORKSPACE, "256-byte"),
    (dict(wsb=256), WORKSPACE, "workspace_bytes=256"),
    (dict(ws=0x28000 - 256), ALIAS, "workspace overlaps"),
    (dict(s=None), NULL, "W8_packed, scales or bias"),
    (dict(b=None), NULL, "W8_packed, scales or bias"),
    (dict(x=None), NULL, "x, mod or idx"),
    (dict(s=0x28002), ALIGN, "idx, scales and bias"),
    (dict(w=0x20008), ALIGN, "packed fp8 weights"),
    (dict(K=12), SHAPE, "multiple of 8"),
    (dict(T=0), SHAPE, "T=0"),
    (dict(y=0x28000), ALIAS, "output overlaps"),
])
def test_norm_proj_adaln_fp8_ws_rejects(lib, kwargs, status, needle):
    assert _adf(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_adaln_fp8_sizes_and_names(lib):
    # needed for every M: the (split) operand and 1/RMS, each rounded up to 256 bytes
    assert lib.fn_adaln_prepass_bytes(4, 16) == 256 + 256
    assert lib.fn_adaln_prepass_bytes(5, 16) == 512 + 256
    assert lib.fn_adaln_prepass_bytes(0, 16) == 0
    assert lib.fn_kernel_name_adaln_fp8(16, 4096, 12288, 4, 0).decode() == "decode_fp8_premod_m16_xlds_w3_u8"
    assert (lib.fn_kernel_name_adaln_fp8(64, 4096, 11008, 4, 1).decode() ==
            "decode_swiglu_fp8_premod_split_m64_xlds_w4_u2")
    assert (lib.fn_kernel_name_adaln_fp8(4096, 4096, 11008, 4, 1).decode() ==
            "prefill_swiglu_fp8_premod_split_256x128_w4x2_xl")
    assert lib.fn_kernel_name_adaln_fp8(65, 4096, 12288, 4, 0).decode() == "decode_fp8_premod_m64_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_fp8(256, 4096, 12288, 4, 0).decode() == "decode_fp8_premod_m64_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_fp8(257, 4096, 12288, 4, 0).decode() == "prefill_fp8_premod_256x256_w4x2_xl"
    assert lib.fn_kernel_name_adaln_fp8(256, 4096, 8176, 4, 0).decode() == "decode_fp8_premod_m64_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_fp8(257, 4096, 8176, 4, 0).decode().startswith("prefill_fp8_premod")
    assert (lib.fn_kernel_name_adaln_fp8(128, 4096, 1376, 4, 1).decode() ==
            "decode_swiglu_fp8_premod_split_m64_xlds_w4_u2")
    assert lib.fn_kernel_name_adaln_fp8(129, 4096, 1376, 4, 1).decode().startswith("prefill_swiglu_fp8_premod_split")
    assert (lib.fn_kernel_name_adaln_fp8(128, 4096, 11008, 4, 1).decode() ==
            "decode_swiglu_fp8_premod_split_m64_xlds_w4_u2")
    assert lib.fn_kernel_name_adaln_fp8(129, 4096, 11008, 4, 1).decode().startswith("prefill_swiglu_fp8_premod_split")
    assert lib.fn_kernel_name_adaln_fp8(0, 4096, 16, 4, 0) == b"invalid"
    sw = lib.fn_norm_proj_swiglu_adaln_fp8_ws
    assert sw(0x1000, 0x10000, 0x18000, 0x20000, 0x28000, 0x30000, 0x21000, None, 0x31000, 0x40000, 4, 16, 16, 2,
              1e-6, 0x100000, 512, None) == NULL
    assert "W8_up, s_up or bias_up" in lib.fn_last_error().decode()
    assert sw(None, None, None, None, None, None, None, None, None, None, 0, 16, 16, 2, 1e-6, None, 0, None) == OK


def _adq(lib, x=0x1000, sc=0x10000, idx=0x18000, wg=0x20000, bg=0x30000, wu=0x24000, bu=0x34000, c=0x40000,
         s=0x48000, M=4, K=16, N=16, T=2, eps=1e-6, ws=0x100000, wsb=512):
    return lib.fn_norm_proj_swiglu_adaln_q8_ws(x, sc, idx, wg, bg, wu, bu, c, s, M, K, N, T, eps, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(ws=None), WORKSPACE, "workspace is NULL"),
    (dict(wsb=128), WORKSPACE, "workspace_bytes=128"),
    (dict(ws=0x48000 - 256), ALIAS, "workspace overlaps"),
    (dict(wu=None), NULL, "gate or up weights or bias rows"),
    (dict(bu=None), NULL, "gate or up weights or bias rows"),
    (dict(c=None), NULL, "out_codes or out_scales"),
    (dict(s=0x48002), ALIGN, "out_scales"),
    (dict(bg=0x30002), ALIGN, "idx, scales and bias"),
    (dict(c=0x34000), ALIAS, "an output overlaps"),
    (dict(s=0x40008), ALIAS, "out_codes overlaps out_scales"),
    (dict(T=0), SHAPE, "T=0"),
])
def test_norm_proj_swiglu_adaln_q8_ws_rejects(lib, kwargs, status, needle):
    assert _adq(lib, **kwargs) == status
    assert needle in lib.fn_last_error().decode()


def test_adaln_q8_names_and_fp8(lib):
    assert lib.fn_kernel_name_adaln_q8(16, 4096, 11008, 4, 0).decode() == "decode_swiglu_bf16_q8_premod_m16_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_q8(64, 4096, 11008, 4, 0).decode() == "decode_swiglu_bf16_q8_premod_m64_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_q8(65, 4096, 11008, 4, 0).decode() == "decode_swiglu_bf16_q8_premod_m64_xlds_w3_u2"
    assert lib.fn_kernel_name_adaln_q8(129, 4096, 11008, 4, 0).decode() == "prefill_swiglu_bf16_q8_premod_128x128_w4x2"
    assert lib.fn_kernel_name_adaln_q8(257, 4096, 11008, 4, 0).decode() == "prefill_swiglu_bf16_q8_premod_256x128_w4x2_xl"
    assert lib.fn_kernel_name_adaln_q8(256, 4096, 8176, 4, 0).decode().startswith("decode_swiglu_bf16_q8_premod_m64")
    assert lib.fn_kernel_name_adaln_q8(257, 4096, 8176, 4, 0).decode().startswith("prefill_swiglu_bf16_q8_premod")
    assert lib.fn_kernel_name_adaln_q8(1024, 4096, 1376, 4, 1).decode().startswith("decode_swiglu_fp8_q8_premod_m64")
    assert lib.fn_kernel_name_adaln_q8(256, 4096, 11008, 4, 1).decode() == "decode_swiglu_fp8_q8_premod_m64_xlds_w4_u2"
    assert lib.fn_kernel_name_adaln_q8(257, 4096, 11008, 4, 1).decode().startswith("prefill_swiglu_fp8_q8_premod")
    assert lib.fn_kernel_name_adaln_q8(64, 4096, 11008, 4, 1).decode() == "decode_swiglu_fp8_q8_premod_m64_xlds_w4_u2"
    assert lib.fn_kernel_name_adaln_q8(4096, 4096, 11008, 4, 1).decode() == "prefill_swiglu_fp8_q8_premod_256x128_w4x2_xl"
    assert lib.fn_kernel_name_adaln_q8(0, 4096, 16, 4, 0) == b"invalid"
    f = lib.fn_norm_proj_swiglu_adaln_fp8_q8_ws
    args = [0x1000, 0x10000, 0x18000, 0x20000, 0x22000, 0x30000, 0x24000, 0x26000, 0x34000, 0x40000, 0x48000,
            4, 16, 16, 2, 1e-6, 0x100000, 512, None]
    bad = list(args)
    bad[4] = None
    assert f(*bad) == NULL and "s_gate or s_up" in lib.fn_last_error().decode()
    bad = list(args)
    bad[16] = None
    assert f(*bad) == WORKSPACE
    assert f(None, None, None, None, None, None, None, None, None, None, None, 0, 16, 16, 2, 1e-6, None, 0,
             None) == OK


def test_last_error_is_per_thread(lib):
    """fn_last_error is thread-local: threads failing validation at the same
    time each read their own message (the library is documented thread-safe
    across streams; validation makes no HIP call, so this runs on the CPU)."""
    import threading
    errors = []
    barrier = threading.Barrier(8)

    def worker(k):
        K = 8 * k + 4                       # not a multiple of 8: rejected with K in the message
        barrier.wait()
        for _ in range(200):
            st = lib.fn_norm_proj(0x1000, 0x20000, 0x40000, 4, K, 16, 1e-6, BF16, None)
            msg = lib.fn_last_error().decode()
            if st != SHAPE or f"K={K}" not in msg:
                errors.append((k, st, msg))
                return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(1, 9)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
