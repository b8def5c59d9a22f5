"""Helpers shared by the GPU parity tests: seeded inputs on the device and
error metrics against the float64 oracle."""
import math

import numpy as np

from synth_inputs import make_qkv

# Tolerances for the 16-bit path (float32 accumulation, P and O rounded to
# 16 bits): max |O - O_ref| <= 1e-2, RMSE(O) <= 3e-3, max |LSE - LSE_ref| <= 1e-3.
MAX_ABS = 1e-2
RMSE = 3e-3
LSE_ABS = 1e-3


def device_qkv(B, N, H, d, seed=0, dtype="bf16", outliers=None):
    import torch
    bits, vals = make_qkv(B, N, H, d, seed=seed, dtype=dtype, outliers=outliers)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    dev = [torch.from_numpy(b.view(np.int16)).view(tdt).cuda() for b in bits]
    return dev, vals


def to_f64(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 else t.cpu().numpy().astype(np.float64)


def errors(o, o_ref, lse=None, lse_ref=None):
    diff = o - o_ref
    res = {"max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
           "rmse": float(math.sqrt(np.mean(diff ** 2))) if diff.size else 0.0}
    if lse is not None:
        both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
        d = np.where(both_inf, 0.0, np.abs(lse - lse_ref))
        res["lse_abs"] = float(d.max()) if d.size else 0.0
    return res


def assert_bf16_tolerances(err, tag=""):
    assert err["max_abs"] <= MAX_ABS, (tag, err)
    assert err["rmse"] <= RMSE, (tag, err)
    if "lse_abs" in err:
        assert err["lse_abs"] <= LSE_ABS, (tag, err)
