"""Helpers shared by the GPU parity tests: moving seeded numpy inputs to the
device, reading results back, and the acceptance check against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def have_gpu() -> bool:
    return torch.cuda.is_available()


def lib():
    import bit_weight_only_awq_amd as awq

    awq.load_library()
    return awq


def dev_f16(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.float16))).cuda()


def dev_u32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.uint32)).view(np.int32)).cuda()


def dev_u16_as_f16(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.uint16)).view(np.float16)).cuda()


def host_u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def host_f16_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def host_f16(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.float16)


def upload_packed(qweight, scales_u16, qzeros):
    return dev_u32(qweight), dev_u16_as_f16(scales_u16), (dev_u32(qzeros) if qzeros is not None else None)


TOL = 1e-3  # |y - y_ref| <= 1e-3 * sum_k |x_k w'_k| per output element


def assert_within_tolerance(y_dev: np.ndarray, y_ref: np.ndarray, d: np.ndarray, what: str = "") -> float:
    from oracle import awq_oracle as O

    r = O.tolerance_ratio(y_dev.astype(np.float64), y_ref, d)
    worst = float(np.max(r)) if r.size else 0.0
    assert np.all(np.isfinite(y_dev.astype(np.float64))), f"{what}: non-finite output"
    assert worst <= TOL, f"{what}: max |y - y_ref| / D = {worst:.3e} > {TOL}"
    return worst
