"""Shared helpers of the GPU parity tests (inputs, device copies, comparisons)."""
import sys

import numpy as np
import torch

from sparse_attention_fp4_cache_amd.workloads import to_bf16_bits

ATOL = 2e-3  # attention: max |gpu - oracle| per output tensor
RTOL = 1e-2  # and max |gpu - oracle| / max |oracle|


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits(x) -> np.ndarray:
    return to_bf16_bits(np.asarray(x, np.float32))


def dev_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def same_bits_f32(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(np.ascontiguousarray(a, np.float32).view(np.int32),
                          np.ascontiguousarray(b, np.float32).view(np.int32))


def attn_close(got_out, ref_out, got_lse, ref_lse, label=""):
    got_out = np.asarray(got_out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    d = np.abs(got_out - ref_out)
    mx = float(d.max()) if d.size else 0.0
    scale = float(np.abs(ref_out).max()) if ref_out.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse)), f"{label}: lse finiteness differs"
    assert np.all(np.asarray(got_lse)[~fin] == -np.inf), label
    dl = np.abs(np.asarray(got_lse, np.float64)[fin] - np.asarray(ref_lse, np.float64)[fin])
    mxl = float(dl.max()) if dl.size else 0.0
    scl = float(np.abs(np.asarray(ref_lse, np.float64)[fin]).max()) if dl.size else 0.0
    say(f"  {label}: out max|d| {mx:.3e} (ref max {scale:.2f}), lse max|d| {mxl:.3e}")
    assert mx <= ATOL and (scale == 0 or mx / scale <= RTOL), f"{label}: out error {mx}"
    assert mxl <= ATOL and (scl == 0 or mxl / scl <= RTOL), f"{label}: lse error {mxl}"
