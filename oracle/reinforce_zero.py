"""Oracle: group advantage, REINFORCE Zero loss and its gradient (float64, CPU).

TEST INFRASTRUCTURE -- see the package docstring for who may use it.

Source: "vLLM says aligned kernels make asynchronous RL stable at lag 64",
section "REINFORCE Zero removes the mismatch first".

* Advantage: a response's reward minus the mean reward of its group. No
  division by the group's spread, no leave-one-out (literal reading).
* Importance ratio: token level, the learner's probability divided by the
  rollout's recorded probability, i.e. exp(lp - lp_rollout); never clipped
  (the same section argues clipping biases the estimate).
* Tokens are averaged within a response; responses are then averaged over
  all responses in the call (reading taken where the pages stop).
* Plain REINFORCE: the loss minimised is the negative of that average of
  ratio * advantage, so its gradient is -ratio * A * grad(lp) / (N * T_i)
  per token (d ratio / d lp = ratio).

Notation: N responses; response i owns tokens resp_offsets[i] ..
resp_offsets[i+1]-1, T_i of them; group g owns responses group_offsets[g] ..
group_offsets[g+1]-1.

    A_i     = r_i - (1/|g|) sum_{j in g(i)} r_j
    ratio_t = exp(lp_t - lp_rollout_t)
    l_i     = -A_i * (sum_{t in i} ratio_t) / T_i          (per-response loss:
                                                           A_i * ratio_t averaged
                                                           over the response's tokens)
    L       = (1/N) * sum_i l_i
    c_t     = dL/dlp_t = -ratio_t * A_i / (N * T_i)
    G[t, v] = dL/dz[t, v] = c_t * (onehot(y_t)[v] - softmax(z_t)[v])
    dH = G W,  dW = G^T H
"""

import numpy as np

from .lmhead import to_f64, logits


def _check_offsets(off, n_items, what):
    off = np.asarray(off, dtype=np.int64)
    if off.ndim != 1 or off.size < 1 or off[0] != 0 or off[-1] != n_items:
        raise ValueError(f"{what} offsets must start at 0 and end at {n_items}")
    if np.any(np.diff(off) <= 0):
        raise ValueError(f"{what} offsets must be strictly increasing (no empty {what})")
    return off


def group_advantage(rewards, group_offsets):
    """A_i = r_i - mean of the rewards in i's group (float64)."""
    r = np.asarray(rewards, dtype=np.float64)
    off = _check_offsets(group_offsets, r.size, "group")
    A = np.empty_like(r)
    for g in range(off.size - 1):
        s, e = off[g], off[g + 1]
        mean = r[s:e].sum() / (e - s)
        A[s:e] = r[s:e] - mean
    return A


def importance_ratio(lp, lp_rollout):
    """Token-level ratio of learner to rollout probability, unclipped."""
    return np.exp(np.asarray(lp, dtype=np.float64) - np.asarray(lp_rollout, dtype=np.float64))


def reinforce_zero_loss(lp, lp_rollout, advantages, resp_offsets):
    """Returns (resp_loss[N], loss, coef[n_tok]) in float64.

    resp_loss[i] = -A_i * (sum of ratio over response i's tokens) / T_i; it
    does not include the 1/N factor, so it depends on response i alone.
    loss = mean of resp_loss over the N responses.
    coef[t] = dL/dlp_t = -ratio_t * A_i / (N * T_i).
    """
    lp = np.asarray(lp, dtype=np.float64)
    A = np.asarray(advantages, dtype=np.float64)
    off = _check_offsets(resp_offsets, lp.size, "response")
    N = A.size
    if off.size != N + 1:
        raise ValueError("advantages and response offsets disagree on the number of responses")
    ratio = importance_ratio(lp, lp_rollout)
    resp_loss = np.empty(N, dtype=np.float64)
    coef = np.empty(lp.size, dtype=np.float64)
    for i in range(N):
        s, e = off[i], off[i + 1]
        T = e - s
        resp_loss[i] = -A[i] * (ratio[s:e].sum() / T)
        coef[s:e] = -ratio[s:e] * A[i] / (N * T)
    loss = resp_loss.sum() / N
    return resp_loss, loss, coef


def reinforce_zero_objective(H, W, y, lp_rollout, advantages, resp_offsets):
    """L as a function of the head's inputs (used by gradient pins)."""
    from .lmhead import lmhead_logprob

    lp, _ = lmhead_logprob(H, W, y)
    return reinforce_zero_loss(lp, lp_rollout, advantages, resp_offsets)[1]


def reinforce_zero_backward(H, W, y, coef, vocab_chunk=8192):
    """(dH[n_tok, d], dW[vocab, d]) of the loss, given c_t = dL/dlp_t.

    The logits and the log-normaliser are recomputed from H and W; then
    G = c * (onehot(y) - softmax(z)), dH = G W and dW = G^T H in float64.
    dH's sum over the vocabulary is taken one vocabulary chunk at a time so
    that W never has to be widened to float64 all at once.
    """
    H64 = to_f64(H)
    W = np.asarray(W)
    y = np.asarray(y, dtype=np.int64)
    c = np.asarray(coef, dtype=np.float64)
    n, d = H64.shape
    V = W.shape[0]
    if y.shape != (n,) or c.shape != (n,):
        raise ValueError("tokens / coef do not match the rows of H")
    if n and (y.min() < 0 or y.max() >= V):
        raise ValueError("token id out of range")
    z = logits(H64, W, vocab_chunk=vocab_chunk)
    m = z.max(axis=1) if n else np.zeros(0)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1)) if n else np.zeros(0)
    G = -c[:, None] * np.exp(z - lse[:, None])
    G[np.arange(n), y] += c
    dH = np.zeros((n, d), dtype=np.float64)
    dW = np.empty((V, d), dtype=np.float64)
    for v0 in range(0, V, vocab_chunk):
        v1 = min(V, v0 + vocab_chunk)
        Wc = to_f64(W[v0:v1])
        dH += G[:, v0:v1] @ Wc
        dW[v0:v1] = G[:, v0:v1].T @ H64
    return dH, dW


def reinforce_zero_backward_rows(H, W, y, coef, tok_idx, vocab_idx, vocab_chunk=8192):
    """Selected rows of the loss gradient: (dH[tok_idx], dW[vocab_idx]).

    The same definitions as reinforce_zero_backward, evaluated for a subset:
    dH[t] = sum_v G[t, v] W[v] needs token t's full row of G, and
    dW[v] = sum_t G[t, v] H[t] needs column v of G for every token, which in
    turn needs every token's log-normaliser over the whole vocabulary. For
    full-size heads where the full gradient does not fit in memory.
    """
    H64 = to_f64(H)
    W = np.asarray(W)
    y = np.asarray(y, dtype=np.int64)
    c = np.asarray(coef, dtype=np.float64)
    tok_idx = np.asarray(tok_idx, dtype=np.int64)
    vocab_idx = np.asarray(vocab_idx, dtype=np.int64)
    n, d = H64.shape
    V = W.shape[0]
    if y.shape != (n,) or c.shape != (n,):
        raise ValueError("tokens / coef do not match the rows of H")
    if n and (y.min() < 0 or y.max() >= V):
        raise ValueError("token id out of range")
    # log-normaliser of every token in two plain passes over the vocabulary
    # (one chunk of rows at a time): the largest logit, then the sum of
    # exp(z - max); lse = max + log(sum)
    m = np.full(n, -np.inf)
    for v0 in range(0, V, vocab_chunk):
        m = np.maximum(m, (H64 @ to_f64(W[v0:v0 + vocab_chunk]).T).max(axis=1))
    s = np.zeros(n)
    for v0 in range(0, V, vocab_chunk):
        s += np.exp(H64 @ to_f64(W[v0:v0 + vocab_chunk]).T - m[:, None]).sum(axis=1)
    lse = m + np.log(s)
    # dH rows: G[t, :] W over the whole vocabulary
    dH = np.zeros((tok_idx.size, d))
    Ht = H64[tok_idx]
    for v0 in range(0, V, vocab_chunk):
        Wc = to_f64(W[v0:v0 + vocab_chunk])
        G = -c[tok_idx, None] * np.exp(Ht @ Wc.T - lse[tok_idx, None])
        dH += G @ Wc
    dH += c[tok_idx, None] * to_f64(W[y[tok_idx]])
    # dW rows: G[:, v]^T H for the selected vocabulary rows
    Wv = to_f64(W[vocab_idx])
    Gv = -c[:, None] * np.exp(H64 @ Wv.T - lse[:, None])
    Gv += c[:, None] * (y[:, None] == vocab_idx[None, :])
    dW = Gv.T @ H64
    return dH, dW
