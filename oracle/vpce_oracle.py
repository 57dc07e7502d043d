"""Plain, slow, fp64 reference for the vocabulary projection fused with
cross-entropy (Ring-DTP's per-rank computation).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library. numpy only.

Source: "Flattening Every Memory Peak in Long-Context Mixture-of-Experts
Training" (arXiv 2609.14306), section 3.2 "Ring-DTP" and its Figure 3; the
abstract (the method keeps the loss and its gradients exact); section 2 (an
operator must give back the same forward values and gradients as the
implementation it stands in for).

The method reaches, up to rounding order, the ordinary softmax cross-entropy of
the logits Z = H W^T. So the plain functions here (``forward``, ``backward``,
``dlogits``) are that definition written out with the full logit rows
materialised (in row chunks, which changes nothing because rows are
independent). The ``*_sharded`` functions follow the strip schedule of
section 3.2 in the pages' order: per shard a full strip, an online fold of the
running (max, sum-exp) state, the target logit from the owning shard, then the
final negative log-likelihood; backward recomputes strip by strip from the
saved normaliser.

Readings taken where the pages are silent or their formulas were lost in
extraction (each is listed in the design notes):
  * online update: m' = max(m, max_j z_j), s' = s e^(m-m') + sum_j e^(z_j-m'),
    from m = -inf, s = 0 (standard online-softmax form the section cites);
  * final loss per token: l = m + log s - t (t = the target's logit);
  * reduction: mean over tokens whose label is not ignore_index; with no such
    token the loss is 0 and every gradient is 0;
  * a label outside [0, V) that is not ignore_index makes that token's loss
    NaN (so the mean is NaN);
  * shard r of R owns a contiguous vocabulary interval; when R does not divide
    V the first V mod R shards are one row longer;
  * the saved normaliser is the per-token log-sum-exp;
  * dloss is the upstream gradient of the mean loss:
    G_ij = dloss / n_valid * valid_i * (softmax_ij - [j == y_i]),
    dH = G W, dW = G^T H.

Parity pins: closed forms at W = 0 and H = 0, a one-hot closed form,
torch/scipy library routines, central finite differences, brute-force
pure-Python loops, shard-count invariance and symmetry invariants; see
tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def shard_bounds(V: int, R: int):
    """Contiguous vocabulary intervals [v0, v1) of the R shards (section 3.2:
    rank r owns an interval of size V/R). The first V mod R shards get one
    extra row."""
    if R < 1 or R > V:
        raise ValueError("need 1 <= R <= V")
    base, extra = divmod(V, R)
    out, v0 = [], 0
    for r in range(R):
        w = base + (1 if r < extra else 0)
        out.append((v0, v0 + w))
        v0 += w
    return out


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _valid(labels, ignore_index):
    labels = np.asarray(labels, dtype=np.int64)
    return labels != ignore_index


def _mean_reduce(per_token, valid):
    n = int(valid.sum())
    if n == 0:
        return 0.0, 0
    return float(np.sum(per_token[valid]) / n), n


def forward(H, W, labels, ignore_index=IGNORE_INDEX, row_chunk=1024):
    """Plain definition. Returns (loss, lse[N]).

    lse_i = max_j Z_ij + log sum_j exp(Z_ij - max_j Z_ij)   (two-pass, exact)
    l_i   = lse_i - Z_{i, y_i}
    loss  = mean of l_i over tokens with y_i != ignore_index
    """
    H, W = _f64(H), _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    valid = _valid(labels, ignore_index)
    lse = np.empty(N, dtype=np.float64)
    nll = np.zeros(N, dtype=np.float64)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Z = H[r0:r1] @ W.T
        m = Z.max(axis=1)
        lse[r0:r1] = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))
        for i in range(r0, r1):
            if not valid[i]:
                continue
            y = labels[i]
            if 0 <= y < V:
                nll[i] = lse[i] - Z[i - r0, y]
            else:
                nll[i] = np.nan
    loss, _ = _mean_reduce(nll, valid)
    return loss, lse


def dlogits(H, W, labels, dloss=1.0, ignore_index=IGNORE_INDEX):
    """G = d(loss)/dZ, materialised [N x V]; for small inputs only."""
    H, W = _f64(H), _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    valid = _valid(labels, ignore_index)
    n = int(valid.sum())
    Z = H @ W.T
    m = Z.max(axis=1, keepdims=True)
    P = np.exp(Z - m)
    P /= P.sum(axis=1, keepdims=True)
    G = P.copy()
    for i in range(N):
        if valid[i] and 0 <= labels[i] < V:
            G[i, labels[i]] -= 1.0
    scale = (dloss / n) if n else 0.0
    G *= scale
    G[~valid] = 0.0
    return G


def backward(H, W, labels, dloss=1.0, ignore_index=IGNORE_INDEX,
             row_chunk=1024):
    """Plain definition. Returns (dH [N x d], dW [V x d]) with
    G = dloss/n_valid * valid * (softmax(Z) - onehot(y)), dH = G W,
    dW = G^T H."""
    H, W = _f64(H), _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    valid = _valid(labels, ignore_index)
    n = int(valid.sum())
    scale = (dloss / n) if n else 0.0
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Z = H[r0:r1] @ W.T
        m = Z.max(axis=1, keepdims=True)
        P = np.exp(Z - m)
        P /= P.sum(axis=1, keepdims=True)
        for i in range(r0, r1):
            y = labels[i]
            if valid[i] and 0 <= y < V:
                P[i - r0, y] -= 1.0
        G = P * scale
        G[~valid[r0:r1]] = 0.0
        dH[r0:r1] = G @ W
        dW += G.T @ H[r0:r1]
    return dH, dW


def forward_sharded(H, W, labels, R, ignore_index=IGNORE_INDEX):
    """Section 3.2 strip schedule on one rank's batch: R rounds, each forming
    the full strip Z_r = H W_r^T of shard r, folding it into the running
    per-token (m, s) with the online-softmax update, taking the target logit
    from the shard that owns the label, and releasing the strip.
    Returns (loss, lse)."""
    H, W = _f64(H), _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    valid = _valid(labels, ignore_index)
    m = np.full(N, -np.inf)
    s = np.zeros(N)
    t = np.full(N, np.nan)
    for v0, v1 in shard_bounds(V, R):
        Zr = H @ W[v0:v1].T
        m_new = np.maximum(m, Zr.max(axis=1))
        s = s * np.exp(m - m_new) + np.exp(Zr - m_new[:, None]).sum(axis=1)
        m = m_new
        own = (labels >= v0) & (labels < v1)
        idx = np.nonzero(own)[0]
        t[idx] = Zr[idx, labels[idx] - v0]
    lse = m + np.log(s)
    nll = np.where(valid, lse - t, 0.0)
    loss, _ = _mean_reduce(nll, valid)
    return loss, lse


def backward_sharded(H, W, labels, lse, R, dloss=1.0,
                     ignore_index=IGNORE_INDEX):
    """Backward replaying the same rounds: each strip is recomputed, turned
    into G with the saved normaliser lse, and contracted into dH (which stays
    with the batch) and dW_r (the shard's own rows)."""
    H, W = _f64(H), _f64(W)
    lse = _f64(lse)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    valid = _valid(labels, ignore_index)
    n = int(valid.sum())
    scale = (dloss / n) if n else 0.0
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    for v0, v1 in shard_bounds(V, R):
        Zr = H @ W[v0:v1].T
        G = np.exp(Zr - lse[:, None])
        own = valid & (labels >= v0) & (labels < v1)
        idx = np.nonzero(own)[0]
        G[idx, labels[idx] - v0] -= 1.0
        G *= scale
        G[~valid] = 0.0
        dH += G @ W[v0:v1]
        dW[v0:v1] = G.T @ H
    return dH, dW


# ----------------------------------------------------------------------------
# Pieces of the plain definition evaluated for selected tokens or vocabulary
# rows, so that full-size results can be checked one output at a time.
# ----------------------------------------------------------------------------

def target_logits(H, W, labels, ignore_index=IGNORE_INDEX, row_chunk=8192):
    """t_i = H_i . W_{y_i} for tokens whose label is in [0, V); NaN for the
    others."""
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    t = np.full(N, np.nan)
    ok = (labels >= 0) & (labels < V)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        sel = np.nonzero(ok[r0:r1])[0] + r0
        if sel.size:
            t[sel] = np.einsum("ij,ij->i", _f64(H[sel]),
                               _f64(W[labels[sel]]))
    return t


def token_rows(H_rows, W, labels_rows, n_valid, dloss=1.0,
               ignore_index=IGNORE_INDEX):
    """lse and dH for a subset of tokens (their full logit rows), given the
    batch-wide count of non-ignored tokens."""
    H_rows, W = _f64(H_rows), _f64(W)
    labels_rows = np.asarray(labels_rows, dtype=np.int64)
    V = W.shape[0]
    Z = H_rows @ W.T
    m = Z.max(axis=1, keepdims=True)
    E = np.exp(Z - m)
    lse = m[:, 0] + np.log(E.sum(axis=1))
    P = E / E.sum(axis=1, keepdims=True)
    valid = labels_rows != ignore_index
    for i, y in enumerate(labels_rows):
        if valid[i] and 0 <= y < V:
            P[i, y] -= 1.0
    scale = (dloss / n_valid) if n_valid else 0.0
    G = P * scale
    G[~valid] = 0.0
    return lse, G @ W


def vocab_rows_dw(H, W_rows, vocab_ids, labels, lse, n_valid, dloss=1.0,
                  ignore_index=IGNORE_INDEX, row_chunk=8192):
    """dW rows for selected vocabulary ids: dW_v = sum_i G_iv H_i, with
    G_iv = dloss/n_valid * valid_i * (exp(z_iv - lse_i) - [y_i == v]); lse is
    the per-token normaliser of the whole batch."""
    W_rows = _f64(W_rows)
    vocab_ids = np.asarray(vocab_ids, dtype=np.int64)
    labels = np.asarray(labels, dtype=np.int64)
    lse = _f64(lse)
    N = H.shape[0]
    valid = labels != ignore_index
    scale = (dloss / n_valid) if n_valid else 0.0
    out = np.zeros((vocab_ids.size, W_rows.shape[1]))
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Hc = _f64(H[r0:r1])
        Z = Hc @ W_rows.T                      # [rows x k]
        G = np.exp(Z - lse[r0:r1, None])
        G -= (labels[r0:r1, None] == vocab_ids[None, :])
        G *= scale
        G[~valid[r0:r1]] = 0.0
        out += G.T @ Hc
    return out
