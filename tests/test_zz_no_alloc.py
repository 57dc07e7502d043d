"""vpce_forward_noalloc (the allocation-free forward, with its scratch in a
static device array) against vpce_forward, the entry point it is a variant
of, called through the C ABI: two calls in a row, the second with a smaller
input, each bitwise equal to vpce_forward and within the oracle tolerances;
a shape whose scratch would exceed the static array is refused before
anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from oracle import compare as C
from tests.gpu_common import require_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    return require_gpu()


CASES = [
    # (N, d, V, R, dtype): the first fills more of the scratch than the
    # second; the second leaves stale partials of the first behind it
    (5000, 264, 3001, 3, "bf16"),
    (700, 136, 1000, 2, "bf16"),
    (129, 64, 515, 1, "f32"),
]


def _call(vp, H, W, lab, R, loss, lse):
    lib = vp._load()
    st = lib.vpce_forward_noalloc(
        ctypes.c_void_p(H.data_ptr()), ctypes.c_void_p(W.data_ptr()),
        ctypes.c_void_p(lab.data_ptr()), H.shape[0], H.shape[1], W.shape[0],
        R, -100, 0 if H.dtype == torch.bfloat16 else 1,
        ctypes.c_void_p(loss.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_forward_matches_vpce_forward(vp):
    for k, (N, d, V, R, dt) in enumerate(CASES):
        say(f"case noalloc #{k}: N={N} d={d} V={V} R={R} {dt}")
        w = WL.custom(N=N, d=d, V=V, R=R, dtype=dt, w_std=0.3,
                      ignore_frac=0.05, name=f"noalloc{k}")
        inp = WL.make_inputs(w, 40 + k)
        H, W, lab = to_device(inp)
        need = vp.forward_noalloc_bytes(N, d, V, R, H.dtype)
        assert 0 < need <= vp.NOALLOC_SCRATCH_BYTES
        loss_ref, lse_ref = vp.forward(H, W, lab, R)
        loss = torch.full((), float("nan"), dtype=torch.float32,
                          device="cuda")
        lse = torch.full((N,), float("nan"), dtype=torch.float32,
                         device="cuda")
        torch.cuda.synchronize()
        assert _call(vp, H, W, lab, R, loss, lse) == 0
        torch.cuda.synchronize()
        assert torch.equal(loss, loss_ref)
        assert torch.equal(lse, lse_ref)
        rloss, rlse = oracle.forward(inp.H_f64(), inp.W_f64(), inp.labels)
        e_lse = C.lse_err(lse.cpu().numpy(), rlse)
        e_loss = C.loss_rel_err(float(loss.item()), rloss)
        say(C.report(f"noalloc #{k}", lse=e_lse, loss=e_loss))
        assert e_lse <= C.LSE_ABS and e_loss <= C.LOSS_REL


def test_noalloc_forward_refuses_shapes_beyond_its_scratch(vp):
    lib = vp._load()
    A = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(A.data_ptr())
    N, d, V, R = 2_000_000, 16, 1000, 8
    assert lib.vpce_forward_noalloc_bytes(N, d, V, R, 0) > \
        vp.NOALLOC_SCRATCH_BYTES
    torch.cuda.synchronize()
    st = lib.vpce_forward_noalloc(p, p, p, N, d, V, R, -100, 0, p, p, None)
    assert st == 7
    assert b"scratch" in lib.vpce_status_string(st)
    # nothing ran: the buffer the pointers name is untouched
    torch.cuda.synchronize()
    assert bool((A == 0).all())
