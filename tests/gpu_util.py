"""Helpers for the GPU parity tests: device transfer and the tolerance bar."""

import os

import numpy as np
import pytest

# max|y - y_oracle| <= TOL_REL_RMS * RMS(y_oracle) for fp16 outputs
TOL_REL_RMS = 1e-2


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def max_err_rel_rms(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(y - ref)) / rms) if rms > 0 else float(np.max(np.abs(y - ref)))


def assert_close(y_fp16, ref, tol=TOL_REL_RMS, what=""):
    e = max_err_rel_rms(np.asarray(y_fp16, np.float16).astype(np.float64), ref)
    log = os.environ.get("Q4W_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(f"{what}\t{e:.3e}\n")
    assert e <= tol, f"{what} max err {e:.3e} x RMS > {tol:.1e}"
    return e
