"""Helpers for the GPU tests: device copies of seeded inputs and the error
metric.  Marshalling only; all convolution arithmetic on the GPU side runs in
libd4r_conv, and all expected values come from the oracle."""
import numpy as np
import torch

import gemm_scratch_nn_amd as d4r

DT_CODE = {"f32": d4r.D4R_F32, "f16": d4r.D4R_F16, "bf16": d4r.D4R_BF16}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# relative Frobenius tolerances: fp32 inputs; f16 / bf16 inputs with f32 accumulation
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def dev(op, device="cuda"):
    """Operand (workloads.Operand) -> device tensor of its storage dtype."""
    if op.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(op.stored)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(op.stored).view(np.int16)).to(device)
    return t.view(TORCH_DT[op.dtype])


def host(t) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - ref) / nr)


def bits16(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
