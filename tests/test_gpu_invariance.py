"""Bitwise batch and phase invariance on the 1.5B-head shapes (GPU vs GPU).

Every response of the workload is evaluated
  * inside the full packed batch (the learner's view),
  * alone,
  * inside 10 random permuted batches of 1..64 responses,
  * as a prefill chunk of random length followed by one-token decode steps
    (decode steps batched across the responses still decoding, as a rollout
    engine would, plus a few responses decoded alone at one token per call),
  * on streams restricted to subsets of the CUs, alone and beside another
    call,
and every logprob and every per-response loss must carry identical bits in
every evaluation ("vLLM Train-Inference Consistency Release Notes", section
"Achieving Bitwise Consistency": batch independence, phase consistency).
Advantages are computed once from complete groups and passed in.
"""

import numpy as np
import pytest

from helpers import same_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stress(cuda):
    import torch
    import invariant_token_logprobs_lm_amd as itl
    from synth import WORKLOADS, draw_head, draw_layout, invariance_plan, sample_tokens

    wl = WORKLOADS["invariance-stress"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device=cuda)
    y = sample_tokens(H, W, wl)
    lp, _ = itl.lmhead_logprob(H, W, y)
    lpr = lp + torch.from_numpy(lay.lag_noise).to(cuda)  # rollout record (lagged)
    A = itl.group_advantage(torch.from_numpy(lay.rewards).to(cuda), torch.from_numpy(lay.group_offsets).to(cuda))
    off = torch.from_numpy(lay.resp_offsets).to(cuda)
    rl, _, _ = itl.reinforce_zero_loss(lp, lpr, A, off)
    batches, prefill = invariance_plan(lay, seed=wl.index)
    say(f"[stress] n_tok={lay.n_tok} responses={lay.n_resp}")
    return dict(itl=itl, lay=lay, H=H, W=W, y=y, lp=lp, lpr=lpr, A=A, rl=rl, batches=batches, prefill=prefill)


def _seg(s, i):
    o = s["lay"].resp_offsets
    return slice(int(o[i]), int(o[i + 1]))


def _eval_batch(s, resp_ids):
    """Pack the given responses in the given order; return (lp, resp_loss)."""
    import torch

    itl = s["itl"]
    idx = torch.cat([torch.arange(_seg(s, i).start, _seg(s, i).stop, device=s["H"].device) for i in resp_ids])
    lens = [_seg(s, i).stop - _seg(s, i).start for i in resp_ids]
    off = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=s["H"].device)
    H = s["H"].index_select(0, idx)
    y = s["y"].index_select(0, idx)
    lp, _ = itl.lmhead_logprob(H, s["W"], y)
    A = s["A"][torch.tensor(resp_ids, device=s["H"].device)]
    rl, _, _ = itl.reinforce_zero_loss(lp, s["lpr"].index_select(0, idx), A, off)
    return lp, rl, off


def test_each_response_alone(stress):
    s = stress
    for i in range(s["lay"].n_resp):
        lp, rl, _ = _eval_batch(s, [i])
        assert same_bits(lp, s["lp"][_seg(s, i)]), f"response {i}"
        assert same_bits(rl, s["rl"][i:i + 1]), f"response {i} loss"


def test_permuted_mixed_batches(stress):
    s = stress
    for b, ids in enumerate(s["batches"]):
        ids = [int(i) for i in ids]
        lp, rl, off = _eval_batch(s, ids)
        for k, i in enumerate(ids):
            assert same_bits(lp[int(off[k]):int(off[k + 1])], s["lp"][_seg(s, i)]), f"batch {b} response {i}"
            assert same_bits(rl[k:k + 1], s["rl"][i:i + 1]), f"batch {b} response {i} loss"
        say(f"[stress] batch {b}: {len(ids)} responses bit-identical")


def test_prefill_then_decode(stress):
    import torch

    s = stress
    itl = s["itl"]
    lay = s["lay"]
    dev = s["H"].device
    N = lay.n_resp
    pre = s["prefill"]
    out = torch.full_like(s["lp"], float("nan"))
    # one prefill batch holding every response's first pre[i] tokens
    idx = torch.cat([torch.arange(_seg(s, i).start, _seg(s, i).start + int(pre[i]), device=dev) for i in range(N)])
    lp, _ = itl.lmhead_logprob(s["H"].index_select(0, idx), s["W"], s["y"].index_select(0, idx))
    out[idx] = lp
    # decode: step k feeds token pre[i] + k of every response still decoding
    step = 0
    while True:
        live = [i for i in range(N) if int(pre[i]) + step < int(lay.lengths[i])]
        if not live:
            break
        ids = torch.tensor([_seg(s, i).start + int(pre[i]) + step for i in live], device=dev)
        lp, _ = itl.lmhead_logprob(s["H"].index_select(0, ids), s["W"], s["y"].index_select(0, ids))
        out[ids] = lp
        step += 1
    say(f"[stress] prefill + {step} decode steps")
    assert same_bits(out, s["lp"])
    # a few responses decoded alone, one token per call
    for i in (0, N // 2, N - 1):
        a = _seg(s, i).start + int(pre[i])
        for t in range(a, min(a + 16, _seg(s, i).stop)):
            lp1, _ = itl.lmhead_logprob(s["H"][t:t + 1], s["W"], s["y"][t:t + 1])
            assert same_bits(lp1, s["lp"][t:t + 1])
    # per-response losses from the reassembled logprobs
    rl, _, _ = itl.reinforce_zero_loss(out, s["lpr"], s["A"], torch.from_numpy(lay.resp_offsets).to(dev))
    assert same_bits(rl, s["rl"])


def test_concurrent_stream_load(stress):
    """The same batch on a side stream while another call loads the GPU."""
    import torch

    s = stress
    itl = s["itl"]
    side = torch.cuda.Stream()
    ids = [int(i) for i in s["batches"][0]]
    busy_H = s["H"][:40000]
    busy_y = s["y"][:40000]
    torch.cuda.synchronize()
    itl.lmhead_logprob(busy_H, s["W"], busy_y)  # enqueued on the default stream
    with torch.cuda.stream(side):
        lp, rl, off = _eval_batch(s, ids)
    torch.cuda.synchronize()
    for k, i in enumerate(ids):
        assert same_bits(lp[int(off[k]):int(off[k + 1])], s["lp"][_seg(s, i)])



@pytest.mark.parametrize("mask", ["half the CUs", "8 of every 16 CUs", "32 CUs", "8 CUs"])
def test_cu_masked_streams(cuda, mask):
    """Scheduling perturbation ("vLLM Train-Inference Consistency Release
    Notes", section "Achieving Bitwise Consistency": results must not depend
    on how the work is scheduled): the whole packed batch and three permuted
    batches on a stream restricted to a subset of the CUs
    (hipExtStreamCreateWithCUMask: half, 8 of every 16, 32, 8, each spread
    over the eight XCDs), alone and while another logprob call
    runs on every CU of the default stream; every logprob and per-response
    loss keeps the bits of the unrestricted run. A CU-masked stream takes a
    hardware queue of its own, of which a process has few, so each mask runs
    in a fresh child process (tests/cu_mask_child.py) holding only the
    default stream and that one."""
    import os
    import subprocess
    import sys

    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cu_mask_child.py")
    r = subprocess.run([sys.executable, "-u", child, mask], capture_output=True, text=True, timeout=240)
    for line in r.stdout.splitlines():
        say(line)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
