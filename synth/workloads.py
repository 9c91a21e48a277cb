"""Workload table and seeded draws (no method arithmetic; see package doc).

Five workloads. Head shapes are those of public model families' output
heads; the pages themselves train a 1.5B reasoning model, Qwen3-4B with a
16K context and larger MoE models ("vLLM says aligned kernels make
asynchronous RL stable at lag 64", section "Reported results include 2.40
times higher throughput"), on math and agentic tool-use tasks that are not
used here. Everything below is synthetic.

Seeds: numpy PCG64(1000 + index) for lengths, rewards, lag noise, subsets,
permutations and chunk points; torch.Generator(device).manual_seed(2000 +
index) for hidden states, head weights and the sampler's Gumbel noise.
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    index: int
    d: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    n_groups: int
    group_size: int
    len_lo: int  # response lengths are uniform integers in [len_lo, len_hi]
    len_hi: int
    h_std: float
    w_std: float
    lag_std: float  # every token's rollout logprob gets N(0, lag_std)
    tail_frac: float  # an i.i.d. Bernoulli(tail_frac) subset additionally gets N(0, tail_std)
    tail_std: float
    reward: tuple  # ("bernoulli", p) or ("uniform",)
    backward: bool
    note: str = field(default="", compare=False)

    @property
    def n_resp(self):
        return self.n_groups * self.group_size


WORKLOADS = {
    w.key: w
    for w in [
        Workload("tiny", 1, 128, 1024, "f32", 2, 4, 8, 32, 1.0, 0.05, 0.01, 0.0, 0.0,
                 ("bernoulli", 0.5), True,
                 "fp32 head small enough for the oracle on every token"),
        Workload("qwen2.5-1.5b-head", 2, 1536, 151936, "bf16", 8, 8, 256, 4096, 1.0, 0.02, 0.02, 0.0, 0.0,
                 ("bernoulli", 0.3), False,
                 "8 prompts x group 8, lengths 256..4096"),
        Workload("qwen3-4b-head", 3, 2560, 151936, "bf16", 4, 8, 2048, 16384, 1.0, 0.02, 0.05, 0.01, 1.0,
                 ("uniform",), False,
                 "4 prompts x group 8, lengths 2048..16384 (16K context), lag-64-like tails"),
        Workload("invariance-stress", 4, 1536, 151936, "bf16", 8, 8, 256, 4096, 1.0, 0.02, 0.02, 0.0, 0.0,
                 ("bernoulli", 0.3), False,
                 "the 1.5B head's shapes, evaluated alone, in permuted batches and as prefill + decode"),
        Workload("large-moe-head", 5, 7168, 129280, "bf16", 4, 16, 512, 8192, 1.0, 0.02, 0.02, 0.0, 0.0,
                 ("bernoulli", 0.4), True,
                 "4 prompts x group 16, lengths 512..8192, forward + loss + backward"),
    ]
}


def torch_dtype(wl):
    import torch

    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


@dataclass
class Layout:
    """Response/group structure and the per-response and per-token draws."""

    lengths: np.ndarray  # int64 [N]
    resp_offsets: np.ndarray  # int64 [N+1]
    group_offsets: np.ndarray  # int32 [G+1]
    rewards: np.ndarray  # float32 [N]
    lag_noise: np.ndarray  # float32 [n_tok]

    @property
    def n_tok(self):
        return int(self.resp_offsets[-1])

    @property
    def n_resp(self):
        return int(self.lengths.size)


def _rng(wl, salt=0):
    return np.random.Generator(np.random.PCG64(1000 + wl.index + 7919 * salt))


def draw_layout(wl, n_groups=None, group_size=None, len_lo=None, len_hi=None, salt=0):
    """Lengths, offsets, rewards and lag noise for a workload.

    The optional overrides give reduced-token instances at a workload's
    head shape (for example one group of 16 responses of 8..64 tokens).
    """
    G = wl.n_groups if n_groups is None else n_groups
    gs = wl.group_size if group_size is None else group_size
    lo = wl.len_lo if len_lo is None else len_lo
    hi = wl.len_hi if len_hi is None else len_hi
    rng = _rng(wl, salt)
    N = G * gs
    lengths = rng.integers(lo, hi, size=N, endpoint=True).astype(np.int64)
    resp_offsets = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(lengths, out=resp_offsets[1:])
    group_offsets = (np.arange(G + 1, dtype=np.int64) * gs).astype(np.int32)
    if wl.reward[0] == "bernoulli":
        rewards = (rng.random(N) < wl.reward[1]).astype(np.float32)
    elif wl.reward[0] == "uniform":
        rewards = rng.random(N).astype(np.float32)
    else:
        raise ValueError(wl.reward)
    n_tok = int(resp_offsets[-1])
    noise = rng.normal(0.0, wl.lag_std, n_tok)
    if wl.tail_frac > 0:
        tail = rng.random(n_tok) < wl.tail_frac
        noise = noise + tail * rng.normal(0.0, wl.tail_std, n_tok)
    return Layout(lengths, resp_offsets, group_offsets, rewards, noise.astype(np.float32))


def draw_head(wl, n_tok, device="cpu", salt=0, chunk_rows=65536):
    """Hidden states H [n_tok, d] and head weights W [vocab, d] as torch tensors.

    Normal draws scaled by the workload's std, then rounded to the
    workload's dtype (torch rounds float32 -> bfloat16 to nearest even).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(2000 + wl.index + 7919 * salt)
    dt = torch_dtype(wl)

    def normal(rows, std):
        out = torch.empty((rows, wl.d), dtype=dt, device=device)
        for r0 in range(0, rows, chunk_rows):
            r1 = min(rows, r0 + chunk_rows)
            x = torch.randn((r1 - r0, wl.d), generator=g, device=device, dtype=torch.float32)
            out[r0:r1] = (x * std).to(dt)
        return out

    W = normal(wl.vocab, wl.w_std)
    H = normal(n_tok, wl.h_std)
    return H, W


def sample_tokens(H, W, wl, salt=0, chunk_rows=2048):
    """Sampled token ids (int32 torch tensor on H's device).

    argmax(logits + Gumbel) draws from softmax(logits) at temperature 1.
    float32 heads: logits in float64 (the workload's "float64 softmax").
    bfloat16 heads: torch's bf16 matmul (fp32 accumulate, bf16 result),
    widened to float32 before the Gumbel noise is added.
    """
    import torch

    device = H.device
    g = torch.Generator(device=device)
    g.manual_seed(3000 + wl.index + 7919 * salt)
    n = H.shape[0]
    out = torch.empty(n, dtype=torch.int32, device=device)
    if H.dtype == torch.float32:
        Wc = W.to(torch.float64)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        if H.dtype == torch.float32:
            z = H[r0:r1].to(torch.float64) @ Wc.T
            u = torch.rand(z.shape, generator=g, device=device, dtype=torch.float64)
        else:
            z = torch.mm(H[r0:r1], W.T).to(torch.float32)
            u = torch.rand(z.shape, generator=g, device=device, dtype=torch.float32)
        u.clamp_(min=torch.finfo(u.dtype).tiny)
        z -= torch.log(-torch.log(u))
        out[r0:r1] = torch.argmax(z, dim=1).to(torch.int32)
        del z, u
    return out


def synthetic_logprobs(n_tok, seed, center=-11.0, spread=2.0):
    """Plausible logprob values (negative, float32) for loss-only tests.

    Stand-ins for a learner's logprobs when the loss stage is tested on its
    own at full size: -|N(center, spread)| keeps them below zero.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    return (-np.abs(rng.normal(center, spread, n_tok))).astype(np.float32)


def token_subset(n_tok, k, seed):
    """k distinct token indices (sorted), seeded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = min(k, n_tok)
    return np.sort(rng.choice(n_tok, size=k, replace=False)).astype(np.int64)


def invariance_plan(layout, n_batches=10, max_batch=64, seed=0):
    """Batches and prefill/decode split points for the invariance stress.

    batches: n_batches random subsets of the responses, of size
    U{1..min(max_batch, N)}, each in random order.
    prefill: per response a prefill length U{1..T_i}; the remaining tokens
    are fed one per decode step.
    """
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    N = layout.n_resp
    batches = []
    for _ in range(n_batches):
        size = int(rng.integers(1, min(max_batch, N), endpoint=True))
        batches.append(rng.permutation(N)[:size].astype(np.int64))
    prefill = np.array([int(rng.integers(1, int(T), endpoint=True)) for T in layout.lengths], dtype=np.int64)
    return batches, prefill
