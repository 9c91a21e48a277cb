"""Seeded synthetic inputs for the sampled-token logprob / REINFORCE Zero path.

This is the one module that both the HIP path's tests and benchmark and the
oracle's tests draw inputs from. It draws random numbers and lays them out
(response lengths and offsets, rewards, lag noise, hidden states, head
weights, sampled tokens, batch permutations). It computes no logprob, no
softmax normaliser, no advantage, no ratio and no loss.

The token sampler stands in for a rollout engine's sampler, which sits
upstream of the path under test: it picks argmax(logits + Gumbel noise),
which draws from softmax(logits) at temperature 1. It forms the logits with
torch's own matmul, not with the HIP library or the oracle. A fault in it
would change which tokens are picked, never whether the two sides agree on
the logprob of a given token.

Rollout logprobs are "exact logprob + lag noise". This module hands out
only the lag noise; whoever builds a rollout record adds it to a logprob it
computed itself (the oracle in parity tests, the HIP path in the benchmark,
where the rollout engine would use the same aligned kernel).
"""

from .workloads import (
    WORKLOADS,
    Workload,
    Layout,
    draw_layout,
    draw_head,
    sample_tokens,
    synthetic_logprobs,
    token_subset,
    invariance_plan,
    torch_dtype,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "Layout",
    "draw_layout",
    "draw_head",
    "sample_tokens",
    "synthetic_logprobs",
    "token_subset",
    "invariance_plan",
    "torch_dtype",
]
