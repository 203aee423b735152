"""C-ABI library: loads, exports every declared symbol, and rejects invalid
calls on the host before any HIP call (so these run without a GPU)."""
import pytest

import gemm_scratch_nn_amd as d4r
from gemm_scratch_nn_amd import D4RError, D4R_F32, D4R_F16, D4R_BF16

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 1 << 20            # a 16-byte aligned fake device address
MISALIGNED = (1 << 20) + 4


def test_every_declared_symbol_is_exported():
    names = d4r.declared_functions()
    expected = {"d4r_conv_create", "d4r_conv_destroy", "d4r_conv_output_dims",
                "d4r_conv_workspace_size", "d4r_conv_forward", "d4r_conv_forward_implicit",
                "d4r_conv_backward_data", "d4r_conv_backward_data_implicit",
                "d4r_conv_backward_filter", "d4r_conv_im2col", "d4r_conv_col2im",
                "d4r_conv_bias_grad", "d4r_gemm_workspace_size", "d4r_gemm",
                "d4r_conv_packed_filter_size", "d4r_conv_pack_filter", "d4r_conv_backward_data_packed",
                "d4r_status_string", "d4r_last_error", "d4r_profile_enable",
                "d4r_profile_reset", "d4r_profile_read", "d4r_relu_forward", "d4r_relu_backward",
                "d4r_maxpool_forward", "d4r_maxpool_backward", "d4r_add_bias_rows",
                "d4r_bias_grad_rows", "d4r_softmax", "d4r_softmax_ce_grad", "d4r_sgd_update",
                "d4r_grad_accum", "d4r_conv_forward_ex", "d4r_gemm_bias_act", "d4r_conv_backward",
                "d4r_conv_describe"}
    assert expected <= set(names)
    for n in names:
        assert d4r.exported(n), n
        assert hasattr(d4r, n), f"python binding lacks {n}"


def test_status_strings():
    assert d4r.d4r_status_string(0) == "D4R_OK"
    assert d4r.d4r_status_string(3) == "D4R_ERR_WORKSPACE"
    assert "unknown" in d4r.d4r_status_string(99)


@pytest.mark.parametrize("args", [
    (0, 1, 5, 5, 3, 3, 1, 0, 1),      # batch 0
    (1, 0, 5, 5, 3, 3, 1, 0, 1),      # inC 0
    (1, 1, 5, 5, 3, 3, 0, 0, 1),      # stride 0
    (1, 1, 5, 5, 3, 3, 1, -1, 1),     # negative padding
    (1, 1, 2, 2, 5, 5, 1, 1, 1),      # kernel larger than padded input
    (1, 1, 5, 5, 3, 3, 1, 0, 0),      # outC 0
])
def test_create_rejects_bad_geometry(args):
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_create(*args, D4R_F32)
    assert e.value.status == INVALID


def test_create_rejects_bad_dtype():
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_create(1, 1, 5, 5, 3, 3, 1, 0, 1, 7)
    assert e.value.status == INVALID


def test_create_rejects_2_pow_31():
    # col = 2304 x (64*13*13*100) > 2^31 elements
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_create(6400, 256, 13, 13, 3, 3, 1, 1, 384, D4R_F32)
    assert e.value.status == UNSUPPORTED


@pytest.mark.parametrize("geom,dims", [
    ((32, 3, 224, 224, 11, 11, 4, 2, 96), (55, 55)),
    ((4, 256, 46, 80, 3, 3, 2, 1, 128), (23, 40)),
    ((8, 1, 28, 28, 5, 5, 1, 0, 6), (24, 24)),
    ((1, 1, 7, 5, 3, 2, 3, 1, 1), (3, 2)),
])
def test_output_dims_and_workspace(geom, dims):
    for dt, es in ((D4R_F32, 4), (D4R_BF16, 2)):
        h = d4r.d4r_conv_create(*geom, dt)
        try:
            assert d4r.d4r_conv_output_dims(h) == dims
            B, C, H, W, kH, kW, s, p, O = geom
            col = C * kH * kW * B * dims[0] * dims[1]
            ws = d4r.d4r_conv_workspace_size(h)
            # col (dtype) plus an f32 dcol at least
            assert ws >= col * es + col * 4
            assert ws % 256 == 0
        finally:
            d4r.d4r_conv_destroy(h)


def test_destroy_null_is_ok():
    d4r.d4r_conv_destroy(None)


@pytest.fixture
def handle():
    h = d4r.d4r_conv_create(2, 3, 9, 9, 3, 3, 1, 1, 4, D4R_F32)
    yield h
    d4r.d4r_conv_destroy(h)


def _ws(h):
    return d4r.d4r_conv_workspace_size(h)


def test_forward_argument_errors(handle):
    ws = _ws(handle)
    cases = [
        ((None, FAKE, None, FAKE, FAKE, ws), INVALID),        # x NULL
        ((FAKE, None, None, FAKE, FAKE, ws), INVALID),        # w NULL
        ((FAKE, FAKE, None, None, FAKE, ws), INVALID),        # y NULL
        ((MISALIGNED, FAKE, None, FAKE, FAKE, ws), INVALID),  # x misaligned
        ((FAKE, FAKE, FAKE + 2, FAKE, FAKE, ws), INVALID),    # bias misaligned
        ((FAKE, FAKE, None, FAKE, None, ws), WORKSPACE),      # ws NULL
        ((FAKE, FAKE, None, FAKE, FAKE, ws - 1), WORKSPACE),  # ws short
        ((FAKE, FAKE, None, FAKE, FAKE + 16, ws), INVALID),   # ws not 256-aligned
    ]
    for (x, w, b, y, wsp, nb), code in cases:
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_forward(handle, x, w, b, y, wsp, nb, stream=0)
        assert e.value.status == code, (x, w, b, y, wsp, nb)
        assert d4r.d4r_last_error()


def test_forward_implicit_argument_errors(handle):
    ws = _ws(handle)
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_forward_implicit(handle, None, FAKE, None, FAKE, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_forward_implicit(handle, FAKE, FAKE, None, FAKE, FAKE, ws - 1, stream=0)
    assert e.value.status == WORKSPACE


def test_forward_ex_argument_errors(handle):
    ws = _ws(handle)
    for flags in (4, -1, 8 | d4r.D4R_FWD_RELU):
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_forward_ex(handle, FAKE, FAKE, None, FAKE, flags, FAKE, ws, stream=0)
        assert e.value.status == INVALID, flags
    for flags in (0, 1, 2, 3):
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_forward_ex(handle, FAKE, FAKE, FAKE + 2, FAKE, flags, FAKE, ws, stream=0)
        assert e.value.status == INVALID, flags  # bias misaligned
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_forward_ex(handle, FAKE, FAKE, None, FAKE, flags, FAKE, ws - 1, stream=0)
        assert e.value.status == WORKSPACE, flags
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_forward_ex(None, FAKE, FAKE, None, FAKE, 1, FAKE, ws, stream=0)
    assert e.value.status == INVALID


def test_backward_data_implicit_argument_errors(handle):
    ws = _ws(handle)
    for args, code in [((None, FAKE, FAKE, FAKE, ws), INVALID), ((FAKE, None, FAKE, FAKE, ws), INVALID),
                       ((FAKE, FAKE, None, FAKE, ws), INVALID), ((FAKE, FAKE, FAKE, None, ws), WORKSPACE),
                       ((FAKE, FAKE, FAKE, FAKE, ws - 1), WORKSPACE),
                       ((FAKE, MISALIGNED, FAKE, FAKE, ws), INVALID)]:
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_backward_data_implicit(handle, *args, stream=0)
        assert e.value.status == code, args


def test_backward_argument_errors(handle):
    ws = _ws(handle)
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_backward_data(handle, FAKE, None, FAKE, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_backward_data(handle, FAKE, FAKE, FAKE, FAKE, 10, stream=0)
    assert e.value.status == WORKSPACE
    # reuse_col = 1 requires x == NULL
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_backward_filter(handle, FAKE, FAKE, FAKE, None, 1, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    # reuse_col = 0 requires x
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_backward_filter(handle, None, FAKE, FAKE, None, 0, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_backward_filter(handle, None, FAKE, FAKE, None, 2, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_bias_grad(handle, FAKE, None, FAKE, ws, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_im2col(handle, FAKE, MISALIGNED, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_col2im(handle, None, FAKE, stream=0)
    assert e.value.status == INVALID


def test_combined_backward_argument_errors(handle):
    ws = _ws(handle)
    call = d4r.d4r_conv_backward
    # (x, w, dy, dx, dw, db, reuse_col, ws, nb) -> status
    cases = [
        ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, ws), INVALID),     # x given with reuse_col = 1
        ((None, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, ws), INVALID),     # x missing with reuse_col = 0
        ((None, FAKE, FAKE, FAKE, FAKE, None, 2, FAKE, ws), INVALID),     # reuse_col not 0/1
        ((None, None, FAKE, FAKE, FAKE, None, 1, FAKE, ws), INVALID),     # w NULL
        ((None, FAKE, None, FAKE, FAKE, None, 1, FAKE, ws), INVALID),     # dy NULL
        ((None, FAKE, FAKE, None, FAKE, None, 1, FAKE, ws), INVALID),     # dx NULL
        ((None, FAKE, FAKE, FAKE, None, None, 1, FAKE, ws), INVALID),     # dw NULL
        ((None, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, FAKE, ws), INVALID), # db misaligned
        ((None, FAKE, MISALIGNED, FAKE, FAKE, None, 1, FAKE, ws), INVALID),
        ((None, FAKE, FAKE, FAKE, FAKE, None, 1, None, ws), WORKSPACE),
        ((None, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, ws - 1), WORKSPACE),
    ]
    for args, code in cases:
        with pytest.raises(D4RError) as e:
            call(handle, *args, stream=0)
        assert e.value.status == code, args
    with pytest.raises(D4RError) as e:
        call(None, None, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, ws, stream=0)
    assert e.value.status == INVALID


def test_null_handle():
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_forward(None, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError):
        d4r.d4r_conv_output_dims(None)


@pytest.mark.parametrize("args,code", [
    ((0, 4, 4, 0, D4R_F32), INVALID),
    ((4, 4, 4, 4, D4R_F32), INVALID),
    ((4, 4, 4, -1, D4R_F32), INVALID),
    ((4, 4, 4, 0, 9), INVALID),
    ((1 << 16, 1 << 16, 4, 0, D4R_F16), UNSUPPORTED),
])
def test_gemm_argument_errors(args, code):
    M, K, N, flags, dt = args
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm_workspace_size(M, K, N, flags, dt)
    assert e.value.status == code
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm(M, K, N, flags, dt, FAKE, FAKE, FAKE, None, 0, stream=0)
    assert e.value.status == code


def test_gemm_pointer_and_workspace_errors():
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm(64, 256, 120, 0, D4R_F32, None, FAKE, FAKE, None, 0, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm(64, 256, 120, 0, D4R_F32, FAKE, FAKE, MISALIGNED, None, 0, stream=0)
    assert e.value.status == INVALID
    # a long-K GEMM plans split-K and needs workspace
    need = d4r.d4r_gemm_workspace_size(96, 96800, 363, 2, D4R_F32)
    assert need > 0
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm(96, 96800, 363, 2, D4R_F32, FAKE, FAKE, FAKE, None, 0, stream=0)
    assert e.value.status == WORKSPACE
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm(96, 96800, 363, 2, D4R_F32, FAKE, FAKE, FAKE, FAKE, need - 4, stream=0)
    assert e.value.status == WORKSPACE


def test_gemm_bias_act_argument_errors():
    for args in [(0, 4, 4, 0, D4R_F32), (4, 4, 4, 4, D4R_F32), (4, 4, 4, 0, 9)]:
        with pytest.raises(D4RError) as e:
            d4r.d4r_gemm_bias_act(*args, FAKE, FAKE, FAKE, 1, FAKE, None, 0, stream=0)
        assert e.value.status == INVALID, args
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm_bias_act(64, 256, 120, 2, D4R_F32, FAKE, FAKE, FAKE + 2, 1, FAKE, None, 0, stream=0)
    assert e.value.status == INVALID  # bias misaligned
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm_bias_act(64, 256, 120, 2, D4R_F32, FAKE, None, FAKE, 0, FAKE, None, 0, stream=0)
    assert e.value.status == INVALID
    need = d4r.d4r_gemm_workspace_size(96, 96800, 363, 2, D4R_F32)
    with pytest.raises(D4RError) as e:
        d4r.d4r_gemm_bias_act(96, 96800, 363, 2, D4R_F32, FAKE, FAKE, None, 1, FAKE, FAKE, need - 4, stream=0)
    assert e.value.status == WORKSPACE


def test_profile_recorder_host_side():
    d4r.d4r_profile_reset()
    d4r.d4r_profile_enable(True)
    d4r.d4r_profile_enable(False)
    assert d4r.d4r_profile_read() == []


# ---- the rest of a training step: validation only (no kernel runs here) ----

TRAIN_ERRORS = [
    ("relu_forward negative n", lambda: d4r.d4r_relu_forward(FAKE, FAKE, -1, stream=0)),
    ("relu_forward x NULL", lambda: d4r.d4r_relu_forward(None, FAKE, 8, stream=0)),
    ("relu_forward y misaligned", lambda: d4r.d4r_relu_forward(FAKE, MISALIGNED, 8, stream=0)),
    ("relu_backward dy NULL", lambda: d4r.d4r_relu_backward(FAKE, None, FAKE, 8, stream=0)),
    ("relu_backward dx is x", lambda: d4r.d4r_relu_backward(FAKE, FAKE + 4096, FAKE, 8, stream=0)),
    ("maxpool_forward window > plane", lambda: d4r.d4r_maxpool_forward(FAKE, FAKE, FAKE, 1, 1, 3, 8, 4, 1,
                                                                       stream=0)),
    ("maxpool_forward k 0", lambda: d4r.d4r_maxpool_forward(FAKE, FAKE, FAKE, 1, 1, 8, 8, 0, 1, stream=0)),
    ("maxpool_forward stride 0", lambda: d4r.d4r_maxpool_forward(FAKE, FAKE, FAKE, 1, 1, 8, 8, 2, 0,
                                                                 stream=0)),
    ("maxpool_forward batch < 0", lambda: d4r.d4r_maxpool_forward(FAKE, FAKE, FAKE, -1, 1, 8, 8, 2, 2,
                                                                  stream=0)),
    ("maxpool_forward idx NULL", lambda: d4r.d4r_maxpool_forward(FAKE, FAKE, None, 1, 1, 8, 8, 2, 2, stream=0)),
    ("maxpool_backward dx misaligned", lambda: d4r.d4r_maxpool_backward(FAKE, FAKE, MISALIGNED, 1, 1, 8, 8, 2, 2,
                                                                        stream=0)),
    ("add_bias_rows cols 0", lambda: d4r.d4r_add_bias_rows(FAKE, FAKE, FAKE, 4, 0, stream=0)),
    ("add_bias_rows bias NULL", lambda: d4r.d4r_add_bias_rows(FAKE, None, FAKE, 4, 4, stream=0)),
    ("add_bias_rows 2^31", lambda: d4r.d4r_add_bias_rows(FAKE, FAKE, FAKE, 1 << 16, 1 << 15, stream=0)),
    ("bias_grad_rows db NULL", lambda: d4r.d4r_bias_grad_rows(FAKE, None, 4, 4, stream=0)),
    ("bias_grad_rows db misaligned", lambda: d4r.d4r_bias_grad_rows(FAKE, FAKE + 2, 4, 4, stream=0)),
    ("softmax rows 0", lambda: d4r.d4r_softmax(FAKE, FAKE + 4096, 0, 10, stream=0)),
    ("softmax p overlaps z", lambda: d4r.d4r_softmax(FAKE, FAKE + 16, 4, 10, stream=0)),
    ("softmax_ce labels NULL", lambda: d4r.d4r_softmax_ce_grad(FAKE, None, FAKE + 4096, None, 4, 10, stream=0)),
    ("softmax_ce classes 0", lambda: d4r.d4r_softmax_ce_grad(FAKE, FAKE, FAKE + 4096, None, 4, 0, stream=0)),
    ("softmax_ce dz is z", lambda: d4r.d4r_softmax_ce_grad(FAKE, FAKE + 8192, FAKE, None, 4, 10, stream=0)),
    ("softmax_ce loss inside dz", lambda: d4r.d4r_softmax_ce_grad(FAKE, FAKE + 8192, FAKE + 4096, FAKE + 4100,
                                                                  4, 10, stream=0)),
    ("softmax_ce loss misaligned", lambda: d4r.d4r_softmax_ce_grad(FAKE, FAKE + 8192, FAKE + 4096, FAKE + 16386,
                                                                   4, 10, stream=0)),
    ("sgd negative clip", lambda: d4r.d4r_sgd_update(FAKE, FAKE + 4096, 8, 0.1, -1.0, stream=0)),
    ("sgd NaN clip", lambda: d4r.d4r_sgd_update(FAKE, FAKE + 4096, 8, 0.1, float("nan"), stream=0)),
    ("sgd grad overlaps param", lambda: d4r.d4r_sgd_update(FAKE, FAKE + 16, 8, 0.1, 1.0, stream=0)),
    ("sgd negative n", lambda: d4r.d4r_sgd_update(FAKE, FAKE + 4096, -8, 0.1, 1.0, stream=0)),
    ("grad_accum grad NULL", lambda: d4r.d4r_grad_accum(FAKE, None, 8, stream=0)),
    ("grad_accum overlap", lambda: d4r.d4r_grad_accum(FAKE, FAKE, 8, stream=0)),
]


@pytest.mark.parametrize("name,call", TRAIN_ERRORS, ids=[t[0] for t in TRAIN_ERRORS])
def test_training_step_argument_errors(name, call):
    with pytest.raises(D4RError) as e:
        call()
    assert e.value.status == INVALID, name
    assert d4r.d4r_last_error()


def test_training_step_empty_calls_enqueue_nothing():
    # n = 0 / zero planes / zero rows return before any HIP call; the
    # pointers (an empty tensor has none) are not examined
    d4r.d4r_relu_forward(None, None, 0, stream=0)
    d4r.d4r_relu_backward(None, None, None, 0, stream=0)
    d4r.d4r_maxpool_forward(None, None, None, 0, 3, 8, 8, 2, 2, stream=0)
    d4r.d4r_maxpool_backward(None, None, None, 2, 0, 8, 8, 2, 2, stream=0)
    d4r.d4r_add_bias_rows(None, None, None, 0, 10, stream=0)
    d4r.d4r_sgd_update(None, None, 0, 0.1, 1.0, stream=0)
    d4r.d4r_grad_accum(None, None, 0, stream=0)
    with pytest.raises(D4RError):  # geometry is still checked
        d4r.d4r_maxpool_forward(None, None, None, 0, 3, 8, 8, 9, 2, stream=0)
    with pytest.raises(D4RError):
        d4r.d4r_sgd_update(None, None, 0, 0.1, -1.0, stream=0)


def test_packed_filter_size_and_argument_errors(handle):
    # handle: (2, 3, 9, 9) -> 4 filters 3x3, f32 (Kc = 27)
    assert d4r.d4r_conv_packed_filter_size(handle) == 4 * 27 * 4
    ws = _ws(handle)
    for args, code in [((None, FAKE + (1 << 16)), INVALID), ((FAKE, None), INVALID),
                       ((FAKE, MISALIGNED), INVALID), ((FAKE, FAKE + 16), INVALID)]:  # overlap
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_pack_filter(handle, *args, stream=0)
        assert e.value.status == code, args
    for args, code in [((None, FAKE, FAKE, FAKE, ws), INVALID), ((FAKE, FAKE, FAKE, None, ws), WORKSPACE),
                       ((FAKE, FAKE, FAKE, FAKE, ws - 1), WORKSPACE), ((FAKE, MISALIGNED, FAKE, FAKE, ws), INVALID)]:
        with pytest.raises(D4RError) as e:
            d4r.d4r_conv_backward_data_packed(handle, *args, stream=0)
        assert e.value.status == code, args


def test_describe_reports_the_explicit_one_pass_backward(monkeypatch):
    # AlexNet conv1 f32 (explicit data gradient, 96 output channels): the
    # combined backward reshapes dy once for both GEMMs, with G in the workspace
    def plan():
        h = d4r.d4r_conv_create(32, 3, 224, 224, 11, 11, 4, 2, 96, D4R_F32)
        try:
            return d4r.d4r_conv_describe(h), d4r.d4r_conv_workspace_size(h)
        finally:
            d4r.d4r_conv_destroy(h)
    d, ws = plan()
    assert d["dgrad_implicit"] == "explicit" and d["fused_backward"] == "explicit" and d["fx_wt"] == "1"
    monkeypatch.setenv("D4R_FUSED_EXPLICIT", "0")
    d0, ws0 = plan()
    assert d0["fused_backward"] == "0" and "fx_wt" not in d0
    # G (dy as a 96 x (32*55*55) f32 matrix) and the transposed filter
    assert ws - ws0 >= 32 * 96 * 55 * 55 * 4 + 96 * 363 * 4
    monkeypatch.setenv("D4R_FUSED_EXPLICIT", "1")
    monkeypatch.setenv("D4R_FX_WT", "0")
    d1, ws1 = plan()
    assert d1["fused_backward"] == "explicit" and d1["fx_wt"] == "0" and ws1 <= ws - 96 * 363 * 4
    # LeNet conv2 (16 output channels) and 16-bit layers keep the separate calls
    monkeypatch.delenv("D4R_FUSED_EXPLICIT")
    monkeypatch.delenv("D4R_FX_WT")
    for args in [(64, 6, 12, 12, 5, 5, 1, 0, 16, D4R_F32), (32, 3, 224, 224, 11, 11, 4, 2, 96, D4R_BF16)]:
        h = d4r.d4r_conv_create(*args)
        try:
            assert d4r.d4r_conv_describe(h)["fused_backward"] == "0", args
        finally:
            d4r.d4r_conv_destroy(h)


def test_describe_reports_the_plan(monkeypatch):
    # AlexNet conv4 at batch 64: the multi-image im2col and col2im windows
    h = d4r.d4r_conv_create(64, 384, 13, 13, 3, 3, 1, 1, 384, D4R_F32)
    try:
        d = d4r.d4r_conv_describe(h)
        assert d["dtype"] == "f32" and d["im2col"] == "lds" and int(d["im2col_bb"]) > 1
        assert d["col2im"] == "lds" and int(d["col2im_bb"]) > 1
        assert d["dgrad_implicit"] == "nhwc" and d["fused_backward"] == "1"
        assert int(d["workspace"]) == d4r.d4r_conv_workspace_size(h)
        # the switches are read when the plan is made, as a launch would
        monkeypatch.setenv("D4R_IM2COL_MINBLK", "100000000")
        assert d4r.d4r_conv_describe(h)["im2col_bb"] == "1"
    finally:
        d4r.d4r_conv_destroy(h)
    # the same layer at batch 2: one image per block
    h = d4r.d4r_conv_create(2, 384, 13, 13, 3, 3, 1, 1, 384, D4R_BF16)
    try:
        d = d4r.d4r_conv_describe(h)
        assert d["dtype"] == "bf16" and d["im2col_bb"] == "1" and d["col2im_bb"] == "1"
    finally:
        d4r.d4r_conv_destroy(h)
    # AlexNet conv1: a 227x227 window is too large for the LDS col2im; the
    # data gradient stays explicit (3 input channels) unless the phased form
    # is forced, which then runs all 16 phases
    h = d4r.d4r_conv_create(32, 3, 224, 224, 11, 11, 4, 2, 96, D4R_F32)
    try:
        d = d4r.d4r_conv_describe(h)
        assert d["col2im"] == "gather" and d["dgrad_implicit"] == "explicit"
    finally:
        d4r.d4r_conv_destroy(h)
    monkeypatch.setenv("D4R_DGRAD_PHASED", "force")
    h = d4r.d4r_conv_create(32, 3, 224, 224, 11, 11, 4, 2, 96, D4R_F32)
    try:
        d = d4r.d4r_conv_describe(h)
        assert d["dgrad_implicit"] == "phased" and d["dgrad_phases"] == "16"
    finally:
        d4r.d4r_conv_destroy(h)
    monkeypatch.setenv("D4R_DGRAD_PHASED", "0")
    h = d4r.d4r_conv_create(4, 256, 46, 80, 3, 3, 2, 1, 128, D4R_F32)
    try:
        assert d4r.d4r_conv_describe(h)["dgrad_implicit"] == "explicit"
    finally:
        d4r.d4r_conv_destroy(h)


def test_describe_argument_errors():
    import ctypes
    with pytest.raises(D4RError) as e:
        d4r.d4r_conv_describe(None)
    assert e.value.status == INVALID
    h = d4r.d4r_conv_create(1, 1, 5, 5, 3, 3, 1, 0, 1, D4R_F32)
    try:
        need = ctypes.c_size_t()
        buf = ctypes.create_string_buffer(4)
        st = d4r._c["d4r_conv_describe"](h, buf, 4, ctypes.byref(need))
        assert st == INVALID and need.value > 4 and buf.raw == b"\0" * 4
    finally:
        d4r.d4r_conv_destroy(h)


def test_two_hip_runtimes_are_refused():
    one = ("7f00-7f01 r-xp 0 08:01 1 /usr/lib/python3/site-packages/torch/lib/libamdhip64.so.7\n"
           "7f02-7f03 r--p 0 08:01 1 /usr/lib/python3/site-packages/torch/lib/libamdhip64.so.7\n"
           "7f04-7f05 r-xp 0 08:01 2 /usr/lib/libc.so.6\n")
    d4r.check_single_hip_runtime(one)
    d4r.check_single_hip_runtime("")
    two = one + "7f06-7f07 r-xp 0 08:01 3 /opt/rocm/lib/libamdhip64.so.7\n"
    assert len(d4r.hip_runtimes(two)) == 2
    with pytest.raises(ImportError):
        d4r.check_single_hip_runtime(two)


def test_exports_only_the_declared_c_abi():
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", d4r.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] in "TtWw"}
    assert funcs == set(d4r.declared_functions()), funcs ^ set(d4r.declared_functions())


def test_stream_reference_argument_errors():
    for call in (lambda: d4r.d4r_stream_copy(FAKE, FAKE + (1 << 20), 100, 0),      # not a multiple of 16
                 lambda: d4r.d4r_stream_copy(MISALIGNED, FAKE, 64, 0),
                 lambda: d4r.d4r_stream_copy(FAKE, FAKE + 32, 64, 0),            # overlap
                 lambda: d4r.d4r_stream_fill(MISALIGNED, 0, 64, 0),
                 lambda: d4r.d4r_stream_fill(FAKE, 0, 8, 0)):
        with pytest.raises(D4RError) as e:
            call()
        assert e.value.status == INVALID
    d4r.d4r_stream_copy(FAKE, FAKE, 0, 0)    # nothing to do: no launch
    d4r.d4r_stream_fill(FAKE, 0, 0, 0)


def test_mfma_ceiling_argument_errors():
    far = FAKE + (1 << 20)
    for call in (lambda: d4r.d4r_mfma_ceiling(7, FAKE, far, 1, 1, 0),             # dtype
                 lambda: d4r.d4r_mfma_ceiling(D4R_F32, FAKE, far, 0, 1, 0),       # blocks
                 lambda: d4r.d4r_mfma_ceiling(D4R_F32, FAKE, far, (1 << 20) + 1, 1, 0),
                 lambda: d4r.d4r_mfma_ceiling(D4R_BF16, FAKE, far, 1, 0, 0),      # iters
                 lambda: d4r.d4r_mfma_ceiling(D4R_BF16, None, far, 1, 1, 0),
                 lambda: d4r.d4r_mfma_ceiling(D4R_BF16, FAKE, MISALIGNED, 1, 1, 0),
                 lambda: d4r.d4r_mfma_ceiling(D4R_BF16, FAKE, FAKE + 64, 1, 1, 0)):  # out overlaps src
        with pytest.raises(D4RError) as e:
            call()
        assert e.value.status == INVALID
