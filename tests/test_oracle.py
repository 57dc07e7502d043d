"""Pins for the fp64 oracle: every check compares it with something other than
itself (closed forms, library routines, finite differences, brute force,
invariants of the mathematics). The ``check_*`` helpers take the functions
under test as arguments so that the planted-mistake tests at the bottom can
show that plausible mistakes in the oracle fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import vpce_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(N, d, V, seed=0, w_std=0.5, n_ignored=0, ignore_index=-100):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) * w_std
    y = rng.integers(0, V, size=N)
    if n_ignored:
        y[rng.choice(N, n_ignored, replace=False)] = ignore_index
    return H, W, y


# ----------------------------------------------------------------------------
# pin checks (each raises AssertionError on failure)
# ----------------------------------------------------------------------------

def check_zero_weights(fwd, bwd):
    """W = 0: every logit is 0, so lse = loss = log V exactly, dH = 0 and
    dW_v = dloss/n * sum_valid (1/V - [y_i = v]) H_i."""
    N, d, V = 9, 6, 11
    H, _, y = rand_case(N, d, V, seed=1, n_ignored=2)
    W = np.zeros((V, d))
    loss, lse = fwd(H, W, y)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-14)
    assert abs(loss - math.log(V)) < 1e-14
    dloss = 0.7
    dH, dW = bwd(H, W, y, dloss)
    assert np.all(dH == 0.0)
    valid = y != -100
    n = valid.sum()
    ref = np.zeros((V, d))
    for i in range(N):
        if valid[i]:
            for v in range(V):
                ref[v] += (dloss / n) * (1.0 / V - (y[i] == v)) * H[i]
    assert np.allclose(dW, ref, rtol=1e-12, atol=1e-15)


def check_zero_hidden(fwd, bwd):
    """H = 0: lse = log V, dW = 0, dH_i = dloss/n * (mean_v W_v - W_{y_i})."""
    N, d, V = 7, 5, 13
    _, W, y = rand_case(N, d, V, seed=2, n_ignored=1)
    H = np.zeros((N, d))
    loss, lse = fwd(H, W, y)
    assert np.allclose(lse, math.log(V), atol=1e-14)
    assert abs(loss - math.log(V)) < 1e-14
    dH, dW = bwd(H, W, y, 1.3)
    assert np.all(dW == 0.0)
    valid = y != -100
    n = valid.sum()
    for i in range(N):
        exp_row = (1.3 / n) * (W.mean(axis=0) - W[y[i]]) if valid[i] else 0
        assert np.allclose(dH[i], exp_row, rtol=1e-12, atol=1e-15)


def check_one_hot(fwd, bwd):
    """d = V = 5, W = I, H_i = c e_{k_i}: lse_i = log(e^c + V - 1) and
    l_i = lse_i - c [y_i = k_i]."""
    V = d = 5
    c = 2.5
    k = np.array([0, 3, 4, 4, 1])
    y = np.array([0, 2, 4, 1, 1])
    H = c * np.eye(V)[k]
    W = np.eye(V)
    loss, lse = fwd(H, W, y)
    want = math.log(math.exp(c) + V - 1)
    assert np.allclose(lse, want, atol=1e-14)
    nll = [want - c * (y[i] == k[i]) for i in range(5)]
    assert abs(loss - sum(nll) / 5) < 1e-14


def check_torch(fwd, bwd, R=None):
    """Library routine: torch fp64 cross_entropy with autograd, and
    logsumexp."""
    N, d, V = 37, 12, 53
    H, W, y = rand_case(N, d, V, seed=3, w_std=0.7, n_ignored=5)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    Z = Ht @ Wt.T
    lt = torch.nn.functional.cross_entropy(Z, torch.tensor(y),
                                           ignore_index=-100)
    (lt * 0.9).backward()
    loss, lse = fwd(H, W, y)
    assert abs(loss - lt.item()) <= 1e-13 * abs(lt.item())
    assert np.allclose(lse, torch.logsumexp(Z, 1).detach().numpy(),
                       rtol=1e-14, atol=1e-14)
    dH, dW = bwd(H, W, y, 0.9)
    assert np.allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-15)
    assert np.allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-15)


def check_finite_differences(fwd, bwd):
    """Central differences of the mean loss match dH and dW (rel <= 1e-6)."""
    N, d, V = 3, 4, 5
    H, W, y = rand_case(N, d, V, seed=4, w_std=0.9)
    y[1] = -100
    dH, dW = bwd(H, W, y, 1.0)
    h = 1e-6
    for M, grad in ((H, dH), (W, dW)):
        num = np.zeros_like(M)
        for idx in np.ndindex(M.shape):
            old = M[idx]
            M[idx] = old + h
            lp, _ = fwd(H, W, y)
            M[idx] = old - h
            lm, _ = fwd(H, W, y)
            M[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err <= 1e-6, err


def check_brute_force(fwd, bwd):
    """Pure-Python loops with math.fsum on N <= 4, V <= 8, d <= 4."""
    N, d, V = 4, 3, 8
    H, W, y = rand_case(N, d, V, seed=5, w_std=1.1)
    y[2] = -100
    Z = [[math.fsum(H[i][k] * W[j][k] for k in range(d)) for j in range(V)]
         for i in range(N)]
    lse = []
    for i in range(N):
        mx = max(Z[i])
        lse.append(mx + math.log(math.fsum(math.exp(z - mx) for z in Z[i])))
    valid = [y[i] != -100 for i in range(N)]
    n = sum(valid)
    loss = math.fsum(lse[i] - Z[i][y[i]] for i in range(N) if valid[i]) / n
    got_loss, got_lse = fwd(H, W, y)
    assert abs(got_loss - loss) < 1e-13
    assert np.allclose(got_lse, lse, atol=1e-13)
    G = [[(math.exp(Z[i][j] - lse[i]) - (j == y[i])) / n if valid[i] else 0.0
          for j in range(V)] for i in range(N)]
    dH = [[math.fsum(G[i][j] * W[j][k] for j in range(V)) for k in range(d)]
          for i in range(N)]
    dW = [[math.fsum(G[i][j] * H[i][k] for i in range(N)) for k in range(d)]
          for j in range(V)]
    gH, gW = bwd(H, W, y, 1.0)
    assert np.allclose(gH, dH, atol=1e-14)
    assert np.allclose(gW, dW, atol=1e-14)


def check_golden(fwd, bwd):
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    ns = {"e": math.e, "log": math.log, "__builtins__": {}}
    ev = lambda s: eval(s, ns)  # noqa: E731  (closed forms written by hand)
    H = np.array(g["H"], float)
    W = np.array(g["W"], float)
    y = np.array(g["labels"])
    loss, lse = fwd(H, W, y)
    assert np.allclose(lse, [ev(s) for s in g["expected"]["lse"]], atol=1e-15)
    assert abs(loss - ev(g["expected"]["loss"])) < 1e-15
    dH, dW = bwd(H, W, y, 1.0)
    assert np.allclose(dH, [[ev(s) for s in r] for r in g["expected"]["dH"]],
                       atol=1e-15)
    assert np.allclose(dW, [[ev(s) for s in r] for r in g["expected"]["dW"]],
                       atol=1e-15)


PINS = [check_zero_weights, check_zero_hidden, check_one_hot, check_torch,
        check_finite_differences, check_brute_force, check_golden]


def plain_fwd(H, W, y):
    return oracle.forward(H, W, y)


def plain_bwd(H, W, y, dloss):
    return oracle.backward(H, W, y, dloss)


def sharded(R):
    def f(H, W, y):
        return oracle.forward_sharded(H, W, y, min(R, W.shape[0]))

    def b(H, W, y, dloss):
        _, lse = oracle.forward_sharded(H, W, y, min(R, W.shape[0]))
        return oracle.backward_sharded(H, W, y, lse, min(R, W.shape[0]),
                                       dloss)
    return f, b


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_plain_oracle_pins(pin):
    pin(plain_fwd, plain_bwd)


@pytest.mark.parametrize("R", [2, 3, 5])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_sharded_oracle_pins(pin, R):
    pin(*sharded(R))


# ----------------------------------------------------------------------------
# further properties
# ----------------------------------------------------------------------------

def test_golden_dlogits():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    ns = {"e": math.e, "log": math.log, "__builtins__": {}}
    G = oracle.dlogits(np.array(g["H"], float), np.array(g["W"], float),
                       np.array(g["labels"]))
    want = [[eval(s, ns) for s in r] for r in g["expected"]["G"]]
    assert np.allclose(G, want, atol=1e-15)


def test_scipy_logsumexp():
    H, W, y = rand_case(64, 16, 300, seed=6, w_std=2.0)
    _, lse = oracle.forward(H, W, y, row_chunk=7)
    assert np.allclose(lse, scipy.special.logsumexp(H @ W.T, axis=1),
                       rtol=1e-14, atol=1e-13)


def test_dlogits_row_sums_and_ignored_rows():
    H, W, y = rand_case(40, 8, 33, seed=7, w_std=1.5, n_ignored=6)
    dloss = 2.0
    G = oracle.dlogits(H, W, y, dloss)
    n = (y != -100).sum()
    assert np.abs(G.sum(axis=1)).max() < 1e-15 * 33
    assert np.all(G[y == -100] == 0.0)
    assert G.min() >= -dloss / n - 1e-15
    # the backward's contractions are exactly G W and G^T H
    dH, dW = oracle.backward(H, W, y, dloss)
    assert np.allclose(dH, G @ W, rtol=1e-12, atol=1e-15)
    assert np.allclose(dW, G.T @ H, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("R", [8, 7, 33])
def test_shard_count_invariance(R):
    """Section 3.2: the strip schedule reaches the same values for any shard
    count; R = 7 makes ragged shards, R = V single-column shards."""
    H, W, y = rand_case(50, 10, 33, seed=8, w_std=1.3, n_ignored=4)
    l1, lse1 = oracle.forward(H, W, y)
    lR, lseR = oracle.forward_sharded(H, W, y, R)
    assert abs(l1 - lR) <= 1e-12 * abs(l1)
    assert np.allclose(lseR, lse1, rtol=1e-12)
    dH1, dW1 = oracle.backward(H, W, y, 0.5)
    dHR, dWR = oracle.backward_sharded(H, W, y, lseR, R, 0.5)
    assert np.allclose(dHR, dH1, rtol=1e-12, atol=1e-16)
    assert np.allclose(dWR, dW1, rtol=1e-12, atol=1e-16)


def test_shift_invariance():
    """Appending a ones column to H and a constant-c column to W adds c to
    every logit: lse shifts by c, loss and G are unchanged."""
    H, W, y = rand_case(20, 6, 17, seed=9, n_ignored=3)
    c = 3.7
    H2 = np.hstack([H, np.ones((20, 1))])
    W2 = np.hstack([W, np.full((17, 1), c)])
    l1, lse1 = oracle.forward(H, W, y)
    l2, lse2 = oracle.forward(H2, W2, y)
    assert np.allclose(lse2, lse1 + c, atol=1e-13)
    assert abs(l1 - l2) < 1e-13
    assert np.allclose(oracle.dlogits(H, W, y), oracle.dlogits(H2, W2, y),
                       atol=1e-15)


def test_permutation_invariances():
    H, W, y = rand_case(25, 5, 19, seed=10, n_ignored=2)
    l1, lse1 = oracle.forward(H, W, y)
    dH1, dW1 = oracle.backward(H, W, y, 1.0)
    rng = np.random.default_rng(11)
    pt = rng.permutation(25)
    l2, lse2 = oracle.forward(H[pt], W, y[pt])
    assert abs(l1 - l2) < 1e-13 and np.allclose(lse2, lse1[pt], atol=1e-14)
    dH2, dW2 = oracle.backward(H[pt], W, y[pt], 1.0)
    assert np.allclose(dH2, dH1[pt], atol=1e-15)
    assert np.allclose(dW2, dW1, atol=1e-14)
    pv = rng.permutation(19)          # new row j holds old row pv[j]
    inv = np.argsort(pv)
    y3 = np.where(y == -100, -100, inv[np.where(y == -100, 0, y)])
    l3, lse3 = oracle.forward(H, W[pv], y3)
    assert abs(l1 - l3) < 1e-13 and np.allclose(lse3, lse1, atol=1e-14)
    dH3, dW3 = oracle.backward(H, W[pv], y3, 1.0)
    assert np.allclose(dH3, dH1, atol=1e-15)
    assert np.allclose(dW3, dW1[pv], atol=1e-15)


def test_linear_in_dloss():
    H, W, y = rand_case(12, 4, 9, seed=12, n_ignored=1)
    a = oracle.backward(H, W, y, 1.0)
    b = oracle.backward(H, W, y, -2.5)
    assert np.allclose(b[0], -2.5 * a[0], atol=1e-16)
    assert np.allclose(b[1], -2.5 * a[1], atol=1e-16)


def test_all_ignored_and_invalid_labels():
    H, W, y = rand_case(6, 4, 7, seed=13)
    yi = np.full(6, -100)
    loss, lse = oracle.forward(H, W, yi)
    assert loss == 0.0
    assert np.allclose(lse, scipy.special.logsumexp(H @ W.T, axis=1))
    dH, dW = oracle.backward(H, W, yi, 1.0)
    assert np.all(dH == 0) and np.all(dW == 0)
    ls, _ = oracle.forward_sharded(H, W, yi, 3)
    assert ls == 0.0
    for bad in (7, -1, 1 << 40):
        yb = y.copy()
        yb[2] = bad
        assert math.isnan(oracle.forward(H, W, yb)[0])
        assert math.isnan(oracle.forward_sharded(H, W, yb, 3)[0])


def test_shard_bounds_match_tensor_split():
    for V, R in [(151936, 7), (129280, 8), (32000, 4), (10, 10), (11, 3)]:
        got = [b - a for a, b in oracle.shard_bounds(V, R)]
        want = [len(t) for t in torch.tensor_split(torch.arange(V), R)]
        assert got == want
        b = oracle.shard_bounds(V, R)
        assert b[0][0] == 0 and b[-1][1] == V
        assert all(b[i][1] == b[i + 1][0] for i in range(R - 1))
    with pytest.raises(ValueError):
        oracle.shard_bounds(5, 6)


def test_row_and_vocab_pieces_match_plain():
    """The per-token and per-vocab-row helpers used for full-size sampled
    checks agree with the plain definition."""
    H, W, y = rand_case(30, 7, 41, seed=14, n_ignored=3)
    loss, lse = oracle.forward(H, W, y)
    dH, dW = oracle.backward(H, W, y, 0.8)
    n = int((y != -100).sum())
    rows = np.array([0, 5, 29, 3])
    lse_r, dH_r = oracle.token_rows(H[rows], W, y[rows], n, 0.8)
    assert np.allclose(lse_r, lse[rows], atol=1e-13)
    assert np.allclose(dH_r, dH[rows], atol=1e-15)
    vids = np.array([40, 0, 17])
    dW_r = oracle.vocab_rows_dw(H, W[vids], vids, y, lse, n, 0.8, row_chunk=8)
    assert np.allclose(dW_r, dW[vids], atol=1e-15)
    t = oracle.target_logits(H, W, y)
    ok = y != -100
    assert np.allclose(t[ok], (H @ W.T)[np.nonzero(ok)[0], y[ok]])
    assert abs(np.mean(lse[ok] - t[ok]) - loss) < 1e-13


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# ----------------------------------------------------------------------------

def _fails_some_pin(fwd, bwd):
    failed = []
    for pin in PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


def _mut_bwd(kind):
    def bwd(H, W, y, dloss):
        G = oracle.dlogits(H, W, y, dloss)
        n = max(1, int((np.asarray(y) != -100).sum()))
        V = W.shape[0]
        if kind == "dropped_onehot":
            for i, yy in enumerate(y):
                if yy != -100:
                    G[i, yy] += dloss / n
        elif kind == "wrong_sign":
            G = -G
        elif kind == "transposed_dW":
            dW = (G.T @ H)[::-1]
            return G @ W, dW
        elif kind == "scale_by_N":
            G = G * n / len(y)
        elif kind == "off_by_one_label":
            for i, yy in enumerate(y):
                if yy != -100:
                    G[i, yy] += dloss / n
                    G[i, (yy + 1) % V] -= dloss / n
        return G @ W, G.T @ H
    return bwd


def _mut_fwd(kind):
    def fwd(H, W, y):
        Z = np.asarray(H, float) @ np.asarray(W, float).T
        y = np.asarray(y)
        if kind == "no_max_shift_log2":
            lse = np.log2(np.exp(Z).sum(1))
        elif kind == "mean_over_all":
            lse = scipy.special.logsumexp(Z, axis=1)
            nll = np.array([lse[i] - Z[i, yy] if yy != -100 else 0.0
                            for i, yy in enumerate(y)])
            return float(nll.mean()), lse
        elif kind == "max_only":
            lse = Z.max(1)
        valid = y != -100
        nll = np.array([lse[i] - Z[i, yy] for i, yy in enumerate(y)
                        if yy != -100])
        return float(nll.mean()) if valid.any() else 0.0, lse
    return fwd


@pytest.mark.parametrize("kind", ["dropped_onehot", "wrong_sign",
                                  "transposed_dW", "scale_by_N",
                                  "off_by_one_label"])
def test_planted_backward_mistakes_are_caught(kind):
    assert _fails_some_pin(plain_fwd, _mut_bwd(kind))


@pytest.mark.parametrize("kind", ["no_max_shift_log2", "mean_over_all",
                                  "max_only"])
def test_planted_forward_mistakes_are_caught(kind):
    assert _fails_some_pin(_mut_fwd(kind), plain_bwd)
