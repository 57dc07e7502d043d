"""Acceptance checks of a device result against the oracle (test
infrastructure). Tolerances:
  * per-token |lse - lse_ref| <= 2e-3 for every token;
  * |loss - loss_ref| / |loss_ref| <= 1e-4;
  * dH, dW: max|x - ref| <= 1e-2 * max|ref| and cosine(x, ref) >= 0.9999.
"""
from __future__ import annotations

import math

import numpy as np

LSE_ABS = 2e-3
LOSS_REL = 1e-4
GRAD_MAXABS_REL = 1e-2
GRAD_COS = 0.9999


def lse_err(lse, ref):
    lse = np.asarray(lse, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(lse - ref))) if lse.size else 0.0


def loss_rel_err(loss, ref):
    if ref == 0.0:
        return abs(loss)
    return abs(loss - ref) / abs(ref)


def grad_errs(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    mref = float(np.max(np.abs(ref))) if ref.size else 0.0
    mabs = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    nx, nr = np.linalg.norm(x), np.linalg.norm(ref)
    if nx == 0.0 and nr == 0.0:
        cos = 1.0
    elif nx == 0.0 or nr == 0.0:
        cos = 0.0
    else:
        cos = float(np.dot(x, ref) / (nx * nr))
    return mabs, mref, cos


def grad_ok(x, ref):
    mabs, mref, cos = grad_errs(x, ref)
    return mabs <= GRAD_MAXABS_REL * mref and cos >= GRAD_COS, (mabs, mref,
                                                                  cos)


def report(name, **kv):
    parts = []
    for k, v in kv.items():
        parts.append(f"{k}={v:.3e}" if isinstance(v, float) and
                     not math.isnan(v) else f"{k}={v}")
    return f"[{name}] " + " ".join(parts)
