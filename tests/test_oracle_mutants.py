"""The oracle's pins catch plausible mistakes.

Each case copies oracle/oracle.c to a temporary directory, plants one
mistake (a flipped kernel, a wrong channel, a dropped term, a transposed
operand, a typo in an index), builds the copy with gcc, binds it through a
fresh instance of the oracle's Python module and runs the pins of
test_oracle_pins.py against it: at least one pin must fail.  Every planted
mistake keeps all memory accesses in bounds.  The real oracle is untouched.
"""
import importlib.util
import os
import subprocess

import pytest

import test_oracle_pins as pins
import test_oracle_train_pins as tpins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PKG = os.path.join(ROOT, "oracle", "__init__.py")

# (name, function the mistake goes into, original text, mistaken text)
MUTANTS = [
    ("forward flips the kernel", "oracle_conv_forward",
     "double wv = w[((o * C + c) * kH + u) * kW + v];",
     "double wv = w[((o * C + c) * kH + (kH - 1 - u)) * kW + (kW - 1 - v)];"),
    ("forward reads the wrong channel", "oracle_conv_forward",
     "const double *xp = x + (b * C + c) * H * W;",
     "const double *xp = x + (b * C + (C - 1 - c)) * H * W;"),
    ("forward drops the bias", "oracle_conv_forward",
     "yp[t] += bv;", "yp[t] += 0.0 * bv;"),
    ("forward pads on one side only", "oracle_conv_forward",
     "i64 h = i * s - p + u;", "i64 h = i * s + u;"),
    ("filter gradient sums one image", "oracle_conv_backward_filter",
     "for (i64 b = 0; b < B; ++b) {", "for (i64 b = 0; b < 1; ++b) {"),
    ("filter gradient uses the column tap for rows", "oracle_conv_backward_filter",
     "i64 ww = j * s - p + v;", "i64 ww = j * s - p + u % kW;"),
    ("data gradient transposes O and C", "oracle_conv_backward_data",
     "double wv = w[((o * C + c) * kH + u) * kW + v];",
     "double wv = w[((c % O) * C + (o % C)) * kH * kW + u * kW + v];"),
    ("data gradient flips the kernel", "oracle_conv_backward_data",
     "double wv = w[((o * C + c) * kH + u) * kW + v];",
     "double wv = w[((o * C + c) * kH + (kH - 1 - u)) * kW + (kW - 1 - v)];"),
    ("bias gradient drops a pixel", "oracle_conv_backward_bias",
     "acc += gp[t];", "acc += (t > 0) ? gp[t] : 0.0;"),
    ("GEMM swaps the B flag branches", "oracle_gemm",
     "double b = tb ? Bm[n * K + k] : Bm[k * N + n];",
     "double b = tb ? Bm[k * N + n] : Bm[n * K + k];"),
    ("GEMM ignores the A flag", "oracle_gemm",
     "double a = ta ? A[k * M + m] : A[m * K + k];",
     "double a = A[m * K + k];"),
    ("im2col uses u for the column tap", "oracle_im2col_spec",
     "i64 h = i * s - p + u, ww = j * s - p + v;",
     "i64 h = i * s - p + u, ww = j * s - p + u % kW;"),
    ("col2im skips the stride test", "oracle_col2im_spec",
     "if (ti < 0 || ti % s != 0 || ti / s >= OH)",
     "if (ti < 0 || ti / s >= OH)"),
    ("ReLU gradient passes at zero", "oracle_relu_grad",
     "dx[i] = x[i] > 0.0 ? dy[i] : 0.0;", "dx[i] = x[i] >= 0.0 ? dy[i] : 0.0;"),
    ("max pooling keeps the last tied maximum", "oracle_maxpool_forward",
     "if (xp[at] > xp[best])", "if (xp[at] >= xp[best])"),
    ("max-pool backward overwrites overlapping windows", "oracle_maxpool_backward",
     "dp[idx[o]] += dy[o];", "dp[idx[o]] = dy[o];"),
    ("bias-row gradient reads the next column", "oracle_bias_grad_rows",
     "acc += dy[i * cols + j];", "acc += dy[i * cols + (j + 1) % cols];"),
    ("softmax-CE gradient adds the one-hot", "oracle_softmax_ce_grad",
     "dz[i * classes + label[i]] -= 1.0;", "dz[i * classes + label[i]] += 1.0;"),
    ("CE loss sums instead of averaging", "oracle_ce_loss",
     "*loss = total / (double)rows;", "*loss = total;"),
    ("SGD clips only from above", "oracle_sgd",
     "if (g < -clip)\n            g = -clip;", "if (g < -clip)\n            g = g;"),
]


def _mutate(src: str, func: str, old: str, new: str) -> str:
    start = src.index(func + "(")
    nxt = src.find("\nint oracle_", start + 1)
    end = len(src) if nxt < 0 else nxt
    body = src[start:end]
    assert old in body, (func, old)
    return src[:start] + body.replace(old, new, 1) + src[end:]


def _bind(so_path: str, tag: str):
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{tag}", PKG)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.LIB_PATH = so_path
    mod._lib = None
    return mod


def _run_pins(orc) -> list:
    """Run the oracle pins against `orc`; return the names that failed."""
    failed = []
    checks = [("1x1 matmul", lambda: pins.test_forward_1x1_is_matmul(orc))]
    for args in [(3, 1, 1, 1, 1), (5, 2, 2, 0, 4), (4, 3, 1, 3, 1)]:
        checks.append((f"delta {args}", lambda a=args: pins.test_forward_delta_kernel_is_shift(orc, *a)))
    for shape in pins._shapes_tiny()[:6]:
        checks.append((f"torch fwd {shape}", lambda sh=shape: pins.test_forward_matches_torch_f64(orc, sh)))
        checks.append((f"torch bwd {shape}",
                       lambda sh=shape: pins.test_backward_matches_torch_autograd_f64(orc, sh)))
        checks.append((f"im2col {shape}", lambda sh=shape: pins.test_im2col_spec_iota_codes(orc, sh)))
        checks.append((f"col2im {shape}", lambda sh=shape: pins.test_col2im_spec_coverage_and_adjoint(orc, sh)))
    for flags in range(4):
        checks.append((f"gemm {flags}", lambda f=flags: pins.test_gemm_flags_match_numpy(orc, f, 7, 17, 5)))
    for name in sorted(os.listdir(pins.GOLDEN)):
        if name.startswith("conv_") and name.endswith(".json"):
            checks.append((name, lambda n=name: pins.test_golden_conv_fixture(orc, n)))
    for name in dir(tpins):
        if name.startswith("test_"):
            fn = getattr(tpins, name)
            if hasattr(fn, "pytestmark"):  # parametrized: run its first case set
                for mark in fn.pytestmark:
                    if mark.name == "parametrize":
                        for case in mark.args[1]:
                            checks.append((f"{name} {case}", lambda f=fn, c=case: f(orc, *c)))
            else:
                checks.append((name, lambda f=fn: f(orc)))
    for label, fn in checks:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(label)
    return failed


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(so), SRC, "-lm"],
                   check=True)
    assert _run_pins(_bind(str(so), "copy")) == []


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, func, old, new):
    with open(SRC) as f:
        src = f.read()
    c_path = tmp_path / "oracle_mutant.c"
    c_path.write_text(_mutate(src, func, old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-w", "-o", str(so), str(c_path),
                    "-lm"], check=True)
    failed = _run_pins(_bind(str(so), func))
    assert failed, f"no pin caught: {name}"
