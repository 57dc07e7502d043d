"""Helpers for the GPU tests: move seeded host inputs to the device, run the
HIP path through the C ABI binding, fetch results."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as WL


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run with -m 'not gpu' "
                           "on a CPU-only machine)")
    import vocabulary_projection_cross_amd as vp
    vp._load()
    return vp


def to_device(inp: WL.Inputs, dev="cuda"):
    if inp.workload.dtype == "bf16":
        H = torch.from_numpy(inp.H.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(inp.H).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    return H, W, lab


def run_gpu(vp, H, W, lab, R, dloss=None, ignore_index=-100):
    loss, lse = vp.forward(H, W, lab, R, ignore_index=ignore_index)
    dl = None if dloss is None else torch.tensor([dloss], dtype=torch.float32,
                                                 device=H.device)
    dH, dW = vp.backward(H, W, lab, lse, dl, R, ignore_index=ignore_index)
    torch.cuda.synchronize()
    return (float(loss.item()), lse.cpu().numpy().astype(np.float64),
            dH.cpu().numpy().astype(np.float64),
            dW.cpu().numpy().astype(np.float64))
