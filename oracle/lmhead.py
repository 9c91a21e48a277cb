"""Oracle: logits, log-softmax and the sampled-token logprob (float64, CPU).

TEST INFRASTRUCTURE -- see the package docstring for who may use it.

Definition followed (plain reading; the pages describe the quantity in
words only -- "vLLM Train-Inference Consistency Release Notes", section
"Overview": bitwise-identical logprobs of the sampled tokens between rollout
and training; "vLLM says aligned kernels make asynchronous RL stable at lag
64", section "REINFORCE Zero removes the mismatch first": the rollout
records each sampled token's logprob):

    z[t, v]  = sum_k H[t, k] * W[v, k]                 (LM-head contraction)
    m[t]     = max_v z[t, v]
    lse[t]   = m[t] + log sum_v exp(z[t, v] - m[t])    (log of the normaliser)
    lp[t]    = z[t, y[t]] - lse[t]                     (sampled-token logprob)

Temperature is 1 and nothing is masked. Out-of-range token ids are an
error; NaN and Inf in the inputs propagate.
"""

import numpy as np


def to_f64(a):
    """Exact float64 copy of an input array.

    uint16 arrays hold bfloat16 bit patterns: the 16 bits are the upper half
    of an IEEE binary32, so shifting them up and reinterpreting is exact.
    float32/float64 arrays widen exactly.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype == np.float32 or a.dtype == np.float64:
        return a.astype(np.float64)
    raise TypeError(f"unsupported input dtype {a.dtype}; expected uint16 (bf16 bits), float32 or float64")


def logits(H, W, vocab_chunk=8192):
    """z = H W^T in float64, one vocabulary chunk of W at a time.

    Each z[t, v] is the full dot product of row t of H with row v of W;
    chunking only bounds how much of W is widened to float64 at once.
    """
    H64 = to_f64(H)
    W = np.asarray(W)
    if H64.ndim != 2 or W.ndim != 2 or H64.shape[1] != W.shape[1]:
        raise ValueError(f"shape mismatch: H {H64.shape}, W {W.shape}")
    n, V = H64.shape[0], W.shape[0]
    z = np.empty((n, V), dtype=np.float64)
    for v0 in range(0, V, vocab_chunk):
        v1 = min(V, v0 + vocab_chunk)
        z[:, v0:v1] = H64 @ to_f64(W[v0:v1]).T
    return z


def log_softmax_at(z, y):
    """(lp, lse) of the given token ids for each row of the logits z."""
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    if z.ndim != 2 or y.shape != (z.shape[0],):
        raise ValueError(f"shape mismatch: z {z.shape}, y {y.shape}")
    if y.size and (y.min() < 0 or y.max() >= z.shape[1]):
        raise ValueError("token id out of range")
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    lp = z[np.arange(z.shape[0]), y] - lse
    return lp, lse


def lmhead_logprob(H, W, y, token_block=256, vocab_chunk=8192):
    """Sampled-token logprob and log-normaliser for every row of H.

    H: [n_tok, d], W: [vocab, d] (uint16 = bf16 bits, or float32/float64),
    y: [n_tok] token ids. Returns float64 (lp[n_tok], lse[n_tok]).
    Rows are taken a block at a time so the [block, vocab] float64 logits
    fit in memory; rows are independent, so this does not change any value.
    """
    H = np.asarray(H)
    y = np.asarray(y, dtype=np.int64)
    n = H.shape[0]
    if y.shape != (n,):
        raise ValueError(f"tokens shape {y.shape} does not match {n} rows")
    lp = np.empty(n, dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for t0 in range(0, n, token_block):
        t1 = min(n, t0 + token_block)
        z = logits(H[t0:t1], W, vocab_chunk=vocab_chunk)
        lp[t0:t1], lse[t0:t1] = log_softmax_at(z, y[t0:t1])
    return lp, lse
