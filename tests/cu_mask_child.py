"""One CU mask of the scheduling-perturbation test, in a process of its own
(run by tests/test_gpu_invariance.py::test_cu_masked_streams).

Usage: python cu_mask_child.py "<mask name>". Builds the invariance-stress
workload, evaluates the whole packed batch and three permuted batches on the
default stream (every CU), then on a stream restricted to the named CU
subset (hipExtStreamCreateWithCUMask), alone and while another logprob call
runs on the default stream, and compares every logprob and per-response
loss bit for bit. Prints one line per run; exits 1 on the first mismatch.
"""

import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def masks(n_cu):
    """CU subsets by mask bit. The runtime refuses a mask that leaves one of
    the eight XCDs without a CU (bit i falls on XCD i mod 8, as the accepted
    and refused masks show), so every subset here keeps CUs on all eight."""
    return {
        "half the CUs": [i < n_cu // 2 for i in range(n_cu)],
        "8 of every 16 CUs": [i % 16 < 8 for i in range(n_cu)],
        "32 CUs": [i < 32 for i in range(n_cu)],
        "8 CUs": [i < 8 for i in range(n_cu)],
    }


def main(name):
    import torch

    import invariant_token_logprobs_lm_amd as itl
    from synth import WORKLOADS, draw_head, draw_layout, invariance_plan, sample_tokens

    dev = torch.device("cuda:0")
    wl = WORKLOADS["invariance-stress"]
    lay = draw_layout(wl)
    H, W = draw_head(wl, lay.n_tok, device=dev)
    y = sample_tokens(H, W, wl)
    lp0, _ = itl.lmhead_logprob(H, W, y)
    lpr = lp0 + torch.from_numpy(lay.lag_noise).to(dev)
    A = itl.group_advantage(torch.from_numpy(lay.rewards).to(dev), torch.from_numpy(lay.group_offsets).to(dev))
    batches, _ = invariance_plan(lay, seed=wl.index)
    o = lay.resp_offsets
    plan = [list(range(lay.n_resp))] + [[int(i) for i in ids] for ids in batches[:3]]

    def run(ids):
        idx = torch.cat([torch.arange(int(o[i]), int(o[i + 1]), device=dev) for i in ids])
        lens = [int(o[i + 1] - o[i]) for i in ids]
        off = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev)
        lp, _ = itl.lmhead_logprob(H.index_select(0, idx), W, y.index_select(0, idx))
        rl, _, _ = itl.reinforce_zero_loss(lp, lpr.index_select(0, idx), A[torch.tensor(ids, device=dev)], off)
        return lp, rl

    ref = [run(ids) for ids in plan]
    torch.cuda.synchronize()

    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    bits = masks(n_cu)[name]
    n_words = (n_cu + 31) // 32
    words = [0] * n_words
    for b, on in enumerate(bits):
        if on:
            words[b // 32] |= 1 << (b % 32)
    handle = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(n_words),
                                          (ctypes.c_uint32 * n_words)(*words))
    if rc != 0:
        print(f"hipExtStreamCreateWithCUMask returned {rc}")
        return 1
    got = (ctypes.c_uint32 * n_words)()
    rc = hip.hipExtStreamGetCUMask(handle, ctypes.c_uint32(n_words), got)
    print(f"[cu mask] {name}: {sum(bits)} of {n_cu} CUs; mask read back "
          f"{'(unavailable)' if rc != 0 else sum(bin(int(w)).count('1') for w in got)} CUs", flush=True)
    stream = torch.cuda.ExternalStream(handle.value)
    status = 0
    try:
        for concurrent in (False, True):
            torch.cuda.synchronize()
            if concurrent:
                itl.lmhead_logprob(H[:40000], W, y[:40000])  # enqueued on the default stream
            with torch.cuda.stream(stream):
                out = [run(ids) for ids in plan]
            torch.cuda.synchronize()
            same = all(torch.equal(a[0].view(torch.int32), b[0].view(torch.int32)) and
                       torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)) for a, b in zip(out, ref))
            print(f"[cu mask] {name}{', beside a call on every CU' if concurrent else ''}: "
                  f"{len(plan)} batches, {sum(len(r[0]) for r in out)} logprobs, bits {'identical' if same else 'DIFFER'}",
                  flush=True)
            if not same:
                status = 1
            del out
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(handle)
    return status


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
