"""The shard-level calls against the fp64 oracle.

The move-activations order of Ring-DTP (R ranks, each holding one
vocabulary shard; the R local batches travel round the ring with their
running state, then with their dH) is played on one device: at hop h, rank i
holds batch (i - h) mod R. The result must be the plain cross-entropy of the
concatenated batches, its mean over all their tokens and both gradients.
Partial states are checked after one and two shards against the oracle's
log-sum-exp over just those shards' columns."""
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


def _bounds(V, R):
    base, extra = divmod(V, R)
    b = [0]
    for r in range(R):
        b.append(b[-1] + base + (1 if r < extra else 0))
    return b


def _batches(N, d, V, R, dtype, seed):
    w = WL.Workload(f"ring_{N}x{d}x{V}x{R}_{dtype}", N * R, d, V, R, dtype,
                    w_std=0.05, labels="zipf", zipf_s=1.1, ignore_frac=0.04)
    inp = WL.make_inputs(w, seed)
    H, W, lab = to_device(inp)
    return inp, H, W, lab


@pytest.mark.parametrize("N,d,V,R,dtype", [(384, 136, 1000, 3, "bf16"),
                                           (300, 64, 515, 4, "f32"),
                                           (257, 72, 2600, 2, "bf16")])
def test_move_activations_ring_matches_oracle(vp, N, d, V, R, dtype):
    say(f"case ring move-activations N={N}x{R} d={d} V={V} R={R} {dtype}")
    inp, H, W, lab = _batches(N, d, V, R, dtype, seed=N + R)
    b = _bounds(V, R)
    Hb = [H[k * N:(k + 1) * N] for k in range(R)]
    Lb = [lab[k * N:(k + 1) * N] for k in range(R)]
    Ws = [W[b[i]:b[i + 1]] for i in range(R)]
    state = [vp.state_init(N, H.device) for _ in range(R)]
    for h in range(R):
        for i in range(R):
            k = (i - h) % R
            vp.shard_fold(Hb[k], Ws[i], Lb[k], V, b[i], state[k])
    totals = torch.zeros(2, dtype=torch.float64, device=H.device)
    lse, loss = [], None
    for k in range(R):
        l, loss = vp.state_finish(state[k], Lb[k], totals)
        lse.append(l)
    dH = [torch.zeros((N, d), dtype=torch.float32, device=H.device)
          for _ in range(R)]
    dW = [torch.zeros((b[i + 1] - b[i], d), dtype=torch.float32,
                      device=H.device) for i in range(R)]
    dloss = torch.tensor([1.5], dtype=torch.float32, device=H.device)
    for h in range(R):
        for i in range(R):
            k = (i - h) % R
            vp.shard_backward(Hb[k], Ws[i], Lb[k], lse[k], totals, dloss, V,
                              b[i], dH[k], dW[i])
    torch.cuda.synchronize()
    g_lse = torch.cat(lse).cpu().numpy().astype(np.float64)
    g_dH = torch.cat(dH).cpu().numpy().astype(np.float64)
    g_dW = torch.cat(dW).cpu().numpy().astype(np.float64)
    Hf, Wf = inp.H_f64(), inp.W_f64()
    rloss, rlse = oracle.forward(Hf, Wf, inp.labels)
    rdH, rdW = oracle.backward(Hf, Wf, inp.labels, 1.5)
    e_lse = C.lse_err(g_lse, rlse)
    e_loss = C.loss_rel_err(float(loss.item()), rloss)
    okH, eH = C.grad_ok(g_dH, rdH)
    okW, eW = C.grad_ok(g_dW, rdW)
    n_valid = int(np.sum(inp.labels != -100))
    say(C.report("ring", lse=e_lse, loss=e_loss, dH_maxabs=eH[0],
                 dH_cos=eH[2], dW_maxabs=eW[0], dW_cos=eW[2]))
    assert e_lse <= C.LSE_ABS, e_lse
    assert e_loss <= C.LOSS_REL, (float(loss.item()), rloss)
    assert float(totals[1].item()) == n_valid
    assert okH, eH
    assert okW, eW
    assert np.all(g_dH[inp.labels == -100] == 0.0)


def test_partial_states_are_the_partial_normalisers(vp):
    N, d, V, R = 300, 136, 1000, 3
    say(f"case ring partial states N={N} d={d} V={V} R={R}")
    inp, H, W, lab = _batches(N, d, V, 1, "bf16", seed=21)
    b = _bounds(V, R)
    Hf, Wf = inp.H_f64(), inp.W_f64()
    state = vp.state_init(N, H.device)
    ln2 = float(np.log(2.0))
    for i in range(R):
        vp.shard_fold(H, W[b[i]:b[i + 1]], lab, V, b[i], state)
        torch.cuda.synchronize()
        st = state.cpu().numpy().astype(np.float64)
        got = ln2 * (st[0] + np.log2(st[1]))
        ign = np.full(N, -100, dtype=np.int64)
        _, ref = oracle.forward(Hf, Wf[:b[i + 1]], ign)
        err = float(np.max(np.abs(got - ref)))
        # the target logit is known exactly for tokens whose label lies in the
        # shards folded so far, and NaN for the others
        seen = (inp.labels >= 0) & (inp.labels < b[i + 1])
        z_t = np.einsum("nd,nd->n", Hf[seen], Wf[inp.labels[seen]])
        e_t = float(np.max(np.abs(st[2][seen] - z_t))) if seen.any() else 0.0
        say(f"after shard {i}: lse over [0, {b[i + 1]}) err {err:.2e}, "
            f"target err {e_t:.2e}")
        assert err <= C.LSE_ABS, err
        assert e_t <= 1e-4 * max(1.0, float(np.max(np.abs(z_t)))), e_t
        assert np.all(np.isnan(st[2][~seen]))


def test_move_weights_order_on_shard_calls_matches_forward(vp):
    """The same calls in the move-weights order (one batch meets the shards
    in ascending order) give the loss and lse of vpce_forward up to fp32
    rounding (the splits inside a shard are grouped differently)."""
    N, d, V, R = 513, 264, 2049, 4
    say(f"case ring move-weights order N={N} d={d} V={V} R={R}")
    inp, H, W, lab = _batches(N, d, V, 1, "bf16", seed=5)
    b = _bounds(V, R)
    state = vp.state_init(N, H.device)
    for i in range(R):
        vp.shard_fold(H, W[b[i]:b[i + 1]], lab, V, b[i], state)
    totals = torch.zeros(2, dtype=torch.float64, device=H.device)
    lse, loss = vp.state_finish(state, lab, totals)
    ref_loss, ref_lse = vp.forward(H, W, lab, R)
    torch.cuda.synchronize()
    assert float((lse - ref_lse).abs().max().item()) <= 1e-5
    assert abs(float(loss.item()) - float(ref_loss.item())) <= \
        1e-6 * abs(float(ref_loss.item()))


def test_shard_calls_on_empty_and_all_ignored_batches(vp):
    d, V, R = 64, 700, 2
    say(f"case ring edge cases d={d} V={V} R={R}")
    b = _bounds(V, R)
    dev = torch.device("cuda")
    g = torch.Generator(device="cuda").manual_seed(9)
    W = (torch.randn((V, d), device=dev, generator=g) * 0.1).to(torch.bfloat16)
    totals = torch.zeros(2, dtype=torch.float64, device=dev)
    # an empty batch folds, finishes and back-propagates to nothing
    H0 = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    L0 = torch.empty(0, dtype=torch.int64, device=dev)
    st0 = vp.state_init(0, dev)
    for i in range(R):
        vp.shard_fold(H0, W[b[i]:b[i + 1]], L0, V, b[i], st0)
    lse0, loss0 = vp.state_finish(st0, L0, totals)
    # a batch whose every label is ignored adds no token and no gradient
    N = 300
    H = torch.randn((N, d), device=dev, generator=g).to(torch.bfloat16)
    L = torch.full((N,), -100, dtype=torch.int64, device=dev)
    st = vp.state_init(N, dev)
    for i in range(R):
        vp.shard_fold(H, W[b[i]:b[i + 1]], L, V, b[i], st)
    lse, loss = vp.state_finish(st, L, totals)
    dH = torch.zeros((N, d), dtype=torch.float32, device=dev)
    dW = [torch.zeros((b[i + 1] - b[i], d), dtype=torch.float32, device=dev)
          for i in range(R)]
    for i in range(R):
        vp.shard_backward(H, W[b[i]:b[i + 1]], L, lse, totals, None, V, b[i],
                          dH, dW[i])
    ref_loss, ref_lse = vp.forward(H, W, L, R)
    torch.cuda.synchronize()
    assert lse0.numel() == 0 and float(loss0.item()) == 0.0
    assert totals.tolist() == [0.0, 0.0]
    assert float(loss.item()) == 0.0 and float(ref_loss.item()) == 0.0
    assert float((lse - ref_lse).abs().max().item()) <= 1e-5
    assert bool((dH == 0).all().item())
    assert all(bool((x == 0).all().item()) for x in dW)
