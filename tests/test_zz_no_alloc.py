"""d4r_gemm_noalloc (split-K partial sums in the library's own device array,
no allocation) against d4r_gemm with a workspace, through the C ABI.

Two calls in a row on each dtype, the second with a smaller product, both
with plans that split K, so the second call runs on scratch the first one
left behind; the results must equal d4r_gemm's bit for bit (same plan and
kernels) and the oracle within the parity tolerance.  Also: a product whose
partials exceed the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


# (M, K, N, flags): long K, so the planner splits it; the second is smaller
PAIRS = {"f32": [(96, 96800, 363, 2), (16, 36864, 150, 1)],
         "f16": [(256, 14720, 256, 2), (64, 8192, 72, 0)],
         "bf16": [(384, 10816, 640, 2), (128, 4096, 136, 3)]}


def _operands(M, K, N, flags, dt, seed):
    rng = np.random.default_rng(seed)
    a = wl.quantize(rng.normal(size=(K, M) if flags & 1 else (M, K)), dt)
    b = wl.quantize(rng.normal(size=(N, K) if flags & 2 else (K, N)), dt)
    return a, b


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_noalloc_equals_workspace_gemm(dt):
    code = DT_CODE[dt]
    cap = d4r.d4r_gemm_noalloc_scratch_bytes()
    assert cap == 64 << 20
    for i, (M, K, N, flags) in enumerate(PAIRS[dt]):
        wsb = d4r.d4r_gemm_workspace_size(M, K, N, flags, code)
        assert 0 < wsb <= cap, (M, K, N, flags, wsb)      # the case splits K and fits
        a, b = _operands(M, K, N, flags, dt, 300 + i)
        A, B = dev(a), dev(b)
        C0 = torch.full((M, N), float("nan"), device="cuda")
        C1 = torch.full((M, N), float("nan"), device="cuda")
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        print(f"noalloc {dt} call {i}: M={M} K={K} N={N} flags={flags} partials {wsb} bytes", flush=True)
        d4r.d4r_gemm(M, K, N, flags, code, A, B, C0, ws, wsb)
        d4r.d4r_gemm_noalloc(M, K, N, flags, code, A, B, C1)
        torch.cuda.synchronize()
        assert torch.equal(C0, C1), f"call {i}: differs from d4r_gemm"
        err = rel_err(host(C1), oracle.gemm(a.exact, b.exact, M, K, N, flags))
        assert err < TOL[dt], (i, err)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_noalloc_without_split(dt):
    # a plan that does not split K uses no scratch at all
    M, K, N, flags = 200, 64, 300, 0
    code = DT_CODE[dt]
    assert d4r.d4r_gemm_workspace_size(M, K, N, flags, code) == 0
    a, b = _operands(M, K, N, flags, dt, 7)
    C0 = d4r.gemm(dev(a), dev(b), M, K, N, flags)
    C1 = torch.empty((M, N), device="cuda")
    d4r.d4r_gemm_noalloc(M, K, N, flags, code, dev(a), dev(b), C1)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)


def test_noalloc_refuses_oversized_partials():
    # 1536 x 1536 f32 partials over many splits: more than 64 MiB
    M, K, N, flags = 1536, 1 << 18, 1536, 2
    need = d4r.d4r_gemm_workspace_size(M, K, N, flags, d4r.D4R_F32)
    assert need > d4r.d4r_gemm_noalloc_scratch_bytes()
    fake = 1 << 20   # never dereferenced: the call is refused before any launch
    with pytest.raises(d4r.D4RError) as e:
        d4r.d4r_gemm_noalloc(M, K, N, flags, d4r.D4R_F32, fake, fake, fake)
    assert e.value.status == 2 and "scratch" in e.value.msg
