"""Helpers for the GPU parity tests: move generator outputs to the device and
compare device results with the oracle."""
import numpy as np
import pytest
import torch

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def require_gpu():
    # GPU tests need a visible GPU: a missing one is a failure, not a skip.
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def dev16(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    """uint16 patterns (or f32 values) -> device tensor of the named dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def dev32(words: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def affine_to_device(case, device):
    x = dev16(case.x, case.act_dtype, device)
    w = dev32(case.packed, device)
    s = dev16(case.scales, case.sb_dtype, device)
    b = dev16(case.biases, case.bias_dtype, device)
    kp = None if case.k_perm is None else torch.from_numpy(np.ascontiguousarray(case.k_perm, dtype=np.int32)).to(device)
    return x, w, s, b, kp


def assert_float_bar(y, ref, what=""):
    import oracle
    rep = oracle.affine_tolerance_report(y, ref)
    print(f"[parity] {what} max_elem={rep['max_elem']:.3e} rel_frob={rep['rel_frob']:.3e}", flush=True)
    assert rep["ok"], f"{what}: {rep}"
    return rep
