"""The three large workloads at their full sizes, in the launch configuration
the benchmark times, against the fp64 oracle. No device value enters a
reference:

  * lse of EVERY token against the oracle's lse (stored by
    tests/golden/make_fullsize_lse.py, which calls only the oracle, for the
    same seeded inputs: the input fingerprint is checked first);
  * the mean loss against the oracle's mean loss, and the stored lse and
    target logits against that loss (consistency of the stored files);
  * dH rows of one random token in every 256-token tile, plus the first and
    last tokens, ignored tokens and outlier rows (exact oracle rows);
  * dW rows of sampled vocabulary ids (most frequent labels, shard and tile
    boundaries, the last row, random ids), from the oracle's formula with the
    oracle's own lse as the normaliser;
  * dH rows of ignored tokens are exactly zero.

The N=16384, d=4096, V=128256, R=8 workload is also compared element by
element on all of dH and dW (oracle.backward, about a minute of host BLAS).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from oracle import compare as C
from tests.gpu_common import require_gpu, say, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def vp():
    return require_gpu()


def golden(w, inp):
    with open(os.path.join(GOLDEN, "fullsize_oracle.json")) as f:
        rec = json.load(f)[w.name]
    assert rec["fingerprint"] == WL.fingerprint(inp), \
        "stored oracle values belong to different inputs"
    lse = np.load(os.path.join(GOLDEN, rec["lse"]))
    tgt = np.load(os.path.join(GOLDEN, rec["tgt"]))
    assert lse.shape == (w.N,) and tgt.shape == (w.N,)
    return rec, lse, tgt


def tile_tokens(inp, rng):
    """One random token per 256-token tile, the first and last tokens, two
    ignored tokens and four outlier rows."""
    N = inp.workload.N
    pick = set()
    for t0 in range(0, N, 256):
        pick.add(int(rng.integers(t0, min(N, t0 + 256))))
    pick.update([0, N - 1])
    ign = np.nonzero(inp.labels == WL.IGNORE_INDEX)[0]
    pick.update(ign[:2].tolist())
    pick.update(inp.outlier_rows[:4].tolist())
    return np.array(sorted(pick))


def sample_vocab(inp, k, rng):
    w = inp.workload
    ok = inp.labels[inp.labels != WL.IGNORE_INDEX]
    freq = np.bincount(ok, minlength=w.V)
    pick = set(np.argsort(freq)[-4:].tolist())
    for v0, v1 in oracle.shard_bounds(w.V, w.R):
        pick.update([v0, v1 - 1, min(v1 - 1, v0 + 256), min(v1 - 1, v0 + 319),
                     min(v1 - 1, v0 + 320), min(v1 - 1, v0 + 4096)])
    pick.update(rng.choice(w.V, size=k, replace=False).tolist())
    pick.add(w.V - 1)
    return np.array(sorted(pick))


def dh_rows_oracle(inp, rows, n_valid, chunk=128):
    Wf = inp.W_f64()
    out = []
    lse = []
    for k in range(0, rows.size, chunk):
        r = rows[k:k + chunk]
        l_, dh = oracle.token_rows(inp.H_f64(r), Wf, inp.labels[r], n_valid)
        out.append(dh)
        lse.append(l_)
    return np.concatenate(lse), np.concatenate(out)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i", [2, 3, 4])
def test_full_size_against_stored_oracle(vp, i):
    w = WL.WORKLOADS[i]
    say(f"case full-size {w.name}: generating inputs")
    inp = WL.make_inputs(w, 0)
    rec, rlse, rtgt = golden(w, inp)
    H, W, lab = to_device(inp)
    say(f"case full-size {w.name}: GPU forward+backward")
    loss_t, lse_t = vp.forward(H, W, lab, w.R)
    dH_t, dW_t = vp.backward(H, W, lab, lse_t, None, w.R)
    torch.cuda.synchronize()
    loss = float(loss_t.item())
    lse = lse_t.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(123)
    rows = tile_tokens(inp, rng)
    vids = sample_vocab(inp, 24, rng)
    dH_rows = dH_t[torch.from_numpy(rows).cuda()].cpu().numpy()
    dW_rows = dW_t[torch.from_numpy(vids).cuda()].cpu().numpy()
    ign = torch.from_numpy(inp.labels == WL.IGNORE_INDEX).cuda()
    ign_zero = bool((dH_t[ign] == 0).all().item())
    del dH_t, dW_t, H, W, lab
    torch.cuda.empty_cache()

    valid = inp.labels != WL.IGNORE_INDEX
    n_valid = int(valid.sum())
    assert n_valid == rec["n_valid"]
    # the stored files agree with each other
    assert abs(float(np.mean(rlse[valid] - rtgt[valid])) - rec["loss"]) <= \
        1e-12 * abs(rec["loss"])

    e_lse = C.lse_err(lse, rlse)
    worst = int(np.argmax(np.abs(lse - rlse)))
    e_loss = C.loss_rel_err(loss, rec["loss"])
    say(f"case full-size {w.name}: oracle dH rows ({rows.size}) and dW rows "
        f"({vids.size})")
    slse, rdH = dh_rows_oracle(inp, rows, n_valid)
    okH, eH = C.grad_ok(dH_rows, rdH)
    rdW = oracle.vocab_rows_dw(_F64Rows(inp, "H"), inp.W_f64(vids), vids,
                               inp.labels, rlse, n_valid)
    okW, eW = C.grad_ok(dW_rows, rdW)
    say(C.report(w.name, tokens=w.N, lse=e_lse, worst_token=worst,
                 loss=e_loss, dH_rows=rows.size, dH_maxabs=eH[0],
                 dH_ref=eH[1], dH_cos=eH[2], dW_rows=vids.size,
                 dW_maxabs=eW[0], dW_ref=eW[1], dW_cos=eW[2]))
    # the stored lse is the oracle's: recomputed rows agree to fp64 rounding
    assert np.max(np.abs(slse - rlse[rows])) <= 1e-9
    assert np.all(np.isfinite(lse))
    assert e_lse <= C.LSE_ABS
    assert e_loss <= C.LOSS_REL
    assert okH, eH
    assert okW, eW
    assert ign_zero


@pytest.mark.timeout(900)
def test_n16k_every_gradient_element(vp):
    """N=16384, d=4096, V=128256, R=8 (one vocabulary split per shard, long-K
    256 x 256 product tiles): all of dH and dW against oracle.backward."""
    w = WL.WORKLOADS[2]
    say(f"case every-element {w.name}: generating inputs")
    inp = WL.make_inputs(w, 0)
    rec, rlse, _ = golden(w, inp)
    H, W, lab = to_device(inp)
    say(f"case every-element {w.name}: GPU forward+backward")
    loss_t, lse_t = vp.forward(H, W, lab, w.R)
    dH_t, dW_t = vp.backward(H, W, lab, lse_t, None, w.R)
    torch.cuda.synchronize()
    lse = lse_t.cpu().numpy().astype(np.float64)
    dH = dH_t.cpu().numpy()
    dW = dW_t.cpu().numpy()
    del dH_t, dW_t, H, W, lab
    torch.cuda.empty_cache()
    say(f"case every-element {w.name}: oracle.backward (host BLAS)")
    rdH, rdW = oracle.backward(inp.H_f64(), inp.W_f64(), inp.labels,
                               row_chunk=2048)
    okH, eH = C.grad_ok(dH, rdH)
    okW, eW = C.grad_ok(dW, rdW)
    e_lse = C.lse_err(lse, rlse)
    say(C.report(w.name + " every element", lse=e_lse, dH_maxabs=eH[0],
                 dH_ref=eH[1], dH_cos=eH[2], dW_maxabs=eW[0], dW_ref=eW[1],
                 dW_cos=eW[2]))
    assert e_lse <= C.LSE_ABS
    assert okH, eH
    assert okW, eW


class _F64Rows:
    """Row access to a workload matrix converted to float64 on demand."""

    def __init__(self, inp, which):
        self.inp, self.which = inp, which
        self.shape = (inp.H if which == "H" else inp.W).shape

    def __getitem__(self, idx):
        return (self.inp.H_f64(idx) if self.which == "H"
                else self.inp.W_f64(idx))


@pytest.mark.timeout(900)
def test_v_sweep_at_full_size_keeps_the_workspace(vp):
    """N=65536, d=7168, R=8 (the 1M-context slice's batch) at V = 32000,
    64000, 128256 and 151936: the bytes requested from the allocator during
    one forward + backward, less the inputs and outputs, are exactly the
    workspace, the same for every V; sampled tokens' lse against the oracle
    (their full logit rows)."""
    N, d, R = 65536, 7168, 8
    sizes = {}
    for V in (32000, 64000, 128256, 151936):
        w = WL.custom(N=N, d=d, V=V, R=R, w_std=0.03, labels="zipf",
                      zipf_s=1.1, ignore_frac=0.02, name=f"vsweep_{V}")
        say(f"case V-sweep N={N} d={d} V={V} R={R}: generating inputs")
        inp = WL.make_inputs(w, 0)
        H, W, lab = to_device(inp)
        ws_bytes = vp.workspace_bytes(N, d, V, R, torch.bfloat16)
        io_out = 4 * N + 4 + 4 * N * d + 4 * V * d
        torch.cuda.synchronize()
        base = torch.cuda.memory_stats()["requested_bytes.all.current"]
        torch.cuda.reset_peak_memory_stats()
        loss, lse = vp.forward(H, W, lab, R)
        dH, dW = vp.backward(H, W, lab, lse, None, R)
        torch.cuda.synchronize()
        peak = torch.cuda.memory_stats()["requested_bytes.all.peak"] - base
        rows = np.random.default_rng(V).choice(N, size=16, replace=False)
        glse = lse.cpu().numpy().astype(np.float64)[rows]
        del loss, lse, dH, dW, H, W, lab
        torch.cuda.empty_cache()
        n_valid = int((inp.labels != WL.IGNORE_INDEX).sum())
        rlse, _ = oracle.token_rows(inp.H_f64(rows), inp.W_f64(),
                                    inp.labels[rows], n_valid)
        e_lse = C.lse_err(glse, rlse)
        # the inputs were allocated before the baseline; each call allocates
        # its own workspace (the forward's is freed on return), so the peak
        # above the baseline holds lse, loss, dH, dW and one workspace
        extra = peak - io_out
        say(f"V={V}: peak {peak} workspace {ws_bytes} extra {extra} "
            f"lse_err {e_lse:.3e}")
        sizes[V] = (ws_bytes, extra)
        assert e_lse <= C.LSE_ABS
    assert len({s[0] for s in sizes.values()}) == 1, sizes
    for V, (ws_bytes, extra) in sizes.items():
        assert extra == ws_bytes, (V, extra, ws_bytes)
