"""Parity bar shared by the GPU tests: atol = rtol = 5e-3 element by element against the fp64
oracle, plus an absolute RMSE below 5e-3, separately for out and final_state (the tolerances
of the FlashKDA README, section 精度测试, and the RMSE bound of the vLLM #43195 summary,
section 实现拆解 step 4)."""
from __future__ import annotations

import math

import numpy as np
import torch

ATOL = 5e-3
RTOL = 5e-3
RMSE_MAX = 5e-3


def to_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def parity_stats(x, ref) -> dict:
    x = to_f64(x)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    xv, rv = x[m], ref[m]
    d = np.abs(xv - rv)
    bound = ATOL + RTOL * np.abs(rv)
    rms_ref = float(np.sqrt(np.mean(rv * rv))) if rv.size else 0.0
    rmse = float(np.sqrt(np.mean(d * d))) if d.size else 0.0
    return dict(n=int(m.sum()), finite=bool(np.isfinite(xv).all()),
                max_abs=float(d.max()) if d.size else 0.0,
                worst_ratio=float((d / bound).max()) if d.size else 0.0,
                n_bad=int((d > bound).sum()), rmse=rmse,
                nrmse=rmse / rms_ref if rms_ref > 0 else 0.0)


def assert_parity(x, ref, what: str) -> dict:
    s = parity_stats(x, ref)
    msg = (f"{what}: n={s['n']} max|d|={s['max_abs']:.3e} worst d/bound={s['worst_ratio']:.3f} "
           f"bad={s['n_bad']} rmse={s['rmse']:.3e} nrmse={s['nrmse']:.3e}")
    print(msg, flush=True)
    assert s["n"] > 0, f"{what}: nothing compared"
    assert s["finite"], f"{what}: non-finite values\n{msg}"
    assert s["n_bad"] == 0, msg
    assert s["rmse"] < RMSE_MAX and math.isfinite(s["rmse"]), msg
    return s
