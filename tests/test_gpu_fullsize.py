"""The three large workloads at their full sizes, in the launch configuration
the benchmark times, checked against the fp64 oracle on sampled outputs that
it can compute one at a time:

  * lse and dH rows of sampled tokens (their full logit rows, exact oracle);
  * the mean loss against mean(lse_gpu - t) with the oracle's target logits
    t_i = H_i . W_{y_i} for every token (checks the merge, the target gather
    and the fp64 reduction);
  * dW rows of sampled vocabulary ids (most frequent labels, shard and tile
    boundaries, the last row), from the oracle's formula with the device lse
    as the normaliser (the lse itself is checked on the sampled tokens);
  * dH rows of ignored tokens are exactly zero.
"""
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


def sample_tokens(inp, k, rng):
    N = inp.workload.N
    pick = set(rng.choice(N, size=k, replace=False).tolist())
    pick.update([0, N - 1])
    ign = np.nonzero(inp.labels == -100)[0]
    pick.update(ign[:2].tolist())
    pick.update(inp.outlier_rows[:4].tolist())
    return np.array(sorted(pick))


def sample_vocab(inp, k, rng):
    w = inp.workload
    ok = inp.labels[inp.labels != -100]
    freq = np.bincount(ok, minlength=w.V)
    pick = set(np.argsort(freq)[-4:].tolist())
    for v0, v1 in oracle.shard_bounds(w.V, w.R):
        pick.update([v0, v1 - 1, min(v1 - 1, v0 + 256), min(v1 - 1, v0 + 4096)])
    pick.update(rng.choice(w.V, size=k, replace=False).tolist())
    pick.add(w.V - 1)
    return np.array(sorted(pick))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i", [2, 3, 4])
def test_full_size_sampled(vp, i):
    w = WL.WORKLOADS[i]
    say(f"case full-size {w.name}: generating inputs")
    inp = WL.make_inputs(w, 0)
    H, W, lab = to_device(inp)
    say(f"case full-size {w.name}: GPU forward+backward")
    loss_t, lse_t = vp.forward(H, W, lab, w.R)
    dH_t, dW_t = vp.backward(H, W, lab, lse_t, None, w.R)
    torch.cuda.synchronize()
    loss = float(loss_t.item())
    lse = lse_t.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(123)
    rows = sample_tokens(inp, 48, rng)
    vids = sample_vocab(inp, 24, rng)
    dH_rows = dH_t[torch.from_numpy(rows).cuda()].cpu().numpy()
    dW_rows = dW_t[torch.from_numpy(vids).cuda()].cpu().numpy()
    ign = torch.from_numpy(inp.labels == -100).cuda()
    ign_zero = bool((dH_t[ign] == 0).all().item())
    del dH_t, dW_t, H, W, lab
    torch.cuda.empty_cache()

    say(f"case full-size {w.name}: oracle on samples")
    n_valid = int((inp.labels != -100).sum())
    Wf = inp.W_f64()
    rlse, rdH = oracle.token_rows(inp.H_f64(rows), Wf, inp.labels[rows],
                                  n_valid)
    e_lse = C.lse_err(lse[rows], rlse)
    okH, eH = C.grad_ok(dH_rows, rdH)
    t = oracle.target_logits(_F64Rows(inp, "H"), _F64Rows(inp, "W"),
                             inp.labels)
    valid = inp.labels != -100
    loss_ref = float(np.mean(lse[valid] - t[valid]))
    e_loss = C.loss_rel_err(loss, loss_ref)
    rdW = oracle.vocab_rows_dw(_F64Rows(inp, "H"), Wf[vids], vids,
                               inp.labels, lse, n_valid)
    okW, eW = C.grad_ok(dW_rows, rdW)
    say(C.report(w.name, lse=e_lse, loss=e_loss, dH_maxabs=eH[0],
                 dH_ref=eH[1], dH_cos=eH[2], dW_maxabs=eW[0], dW_ref=eW[1],
                 dW_cos=eW[2]))
    assert np.all(np.isfinite(lse))
    assert e_lse <= C.LSE_ABS
    assert e_loss <= C.LOSS_REL
    assert okH, eH
    assert okW, eW
    assert ign_zero


class _F64Rows:
    """Row access to a workload matrix converted to float64 on demand."""

    def __init__(self, inp, which):
        self.inp, self.which = inp, which
        self.shape = (inp.H if which == "H" else inp.W).shape

    def __getitem__(self, idx):
        return (self.inp.H_f64(idx) if self.which == "H"
                else self.inp.W_f64(idx))
