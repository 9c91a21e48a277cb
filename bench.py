"""Benchmark of the sampled-token logprob + REINFORCE Zero hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]
                    [--no-cpu-baseline] [--no-backward]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM: the fused LM-head logprob (contraction + online
log-sum-exp + gather), the group advantage and the REINFORCE Zero loss with
its per-token coefficients. The default workload is the Qwen3-4B-shaped head
(d = 2560, vocab = 151936, 32 responses of 2048..16384 tokens). The JSON line
also carries the forward on the 1.5B-shaped head (d = 1536) and on the
tiny fp32 head, and a forward + backward figure on the large-MoE-shaped head
(d = 7168, vocab = 129280): with the forward's logits kept in HBM when they
fit (159 GB), else with the backward recomputing them; both are timed when
memory allows.

Prints progress to stderr and ONE JSON line to stdout.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled-token logprobs/sec (fwd, fwd+bwd) at 1 GPU; % bf16 MFMA peak"
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense FP8 matrix-core peak (2 x the bf16 figure)
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU (published 2.5 PFLOP/s)
PEAK_F32_TFLOPS = 157.3  # MI355X dense fp32 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["invariant_token_logprobs_lm_amd/csrc/lmhead.hip",
                  "invariant_token_logprobs_lm_amd/csrc/tile_engine.h",
                  "invariant_token_logprobs_lm_amd/csrc/tile_engine8.h",
                  "invariant_token_logprobs_lm_amd/csrc/itl_config.h",
                  "invariant_token_logprobs_lm_amd/csrc/device_common.h",
                  "invariant_token_logprobs_lm_amd/csrc/lse_fold.h",
                  "invariant_token_logprobs_lm_amd/build.py"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"lmhead_lse_partial8_{workload_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def setup_forward(wl, device):
    import torch
    import invariant_token_logprobs_lm_amd as itl
    from synth import draw_head, draw_layout, sample_tokens

    lay = draw_layout(wl)
    log(f"[bench] {wl.key}: d={wl.d} V={wl.vocab} responses={lay.n_resp} n_tok={lay.n_tok}")
    t0 = time.time()
    H, W = draw_head(wl, lay.n_tok, device=device)
    y = sample_tokens(H, W, wl)
    ws = torch.empty(itl.lmhead_workspace_bytes(lay.n_tok, wl.vocab), dtype=torch.uint8, device=device)
    lp = torch.empty(lay.n_tok, dtype=torch.float32, device=device)
    lse = torch.empty(lay.n_tok, dtype=torch.float32, device=device)
    # The rollout's record: the same aligned kernel (here at the same weights)
    # plus the workload's lag noise.
    itl.lmhead_logprob(H, W, y, logprob=lp, lse=lse, workspace=ws)
    lpr = lp + torch.from_numpy(lay.lag_noise).to(device)
    rewards = torch.from_numpy(lay.rewards).to(device)
    goff = torch.from_numpy(lay.group_offsets).to(device)
    roff = torch.from_numpy(lay.resp_offsets).to(device)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    return dict(lay=lay, H=H, W=W, y=y, ws=ws, lp=lp, lse=lse, lpr=lpr, rewards=rewards, goff=goff, roff=roff)


def forward_step(s, ev=None):
    import invariant_token_logprobs_lm_amd as itl

    if ev is not None:
        ev[0].record()
    itl.lmhead_logprob(s["H"], s["W"], s["y"], logprob=s["lp"], lse=s["lse"], workspace=s["ws"])
    if ev is not None:
        ev[1].record()
    A = itl.group_advantage(s["rewards"], s["goff"])
    return itl.reinforce_zero_loss(s["lp"], s["lpr"], A, s["roff"])


def time_steps(step, steps, warmup):
    import torch

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    head = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for k in range(steps):
        step(head[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    head_ms = [a.elapsed_time(b) for a, b in head]
    return total_ms / steps, sum(head_ms) / steps, wall


def forward_leg(key, device, steps):
    """The forward step (logprob + advantage + loss) on another workload of
    the table, timed like the headline: tokens/s and the logprob kernel's
    fraction of its dtype's matrix-core peak."""
    import torch
    from synth import WORKLOADS

    wl = WORKLOADS[key]
    s = setup_forward(wl, device)
    n_tok = s["lay"].n_tok
    ms_step, ms_head, _ = time_steps(lambda ev: forward_step(s, ev), steps, 2)
    flops = 2.0 * wl.d * wl.vocab * n_tok
    tf = flops / (ms_head * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    log(f"[bench] {key}: step {ms_step:.3f} ms, logprob kernel {ms_head:.3f} ms -> {tf:.1f} TFLOP/s "
        f"({100 * tf / peak:.1f}% of the {wl.dtype} peak)")
    out = {"workload": f"{key} forward logprob + group advantage + REINFORCE Zero loss", "d": wl.d,
           "vocab": wl.vocab, "dtype": wl.dtype, "responses": s["lay"].n_resp, "n_tok": n_tok, "steps": steps,
           "ms_per_step": ms_step, "value": n_tok / (ms_step * 1e-3), "unit": "sampled-token logprobs/s",
           "ms_logprob": ms_head, "tflops_logprob": tf, "frac_peak": tf / peak,
           "peak": f"{peak} TFLOP/s dense {'fp32' if wl.dtype == 'f32' else 'bf16'}"}
    del s
    torch.cuda.empty_cache()
    return out


def setup_backward(wl, device):
    """Inputs of the forward + backward step on a head with a backward."""
    import torch
    import invariant_token_logprobs_lm_amd as itl

    s = setup_forward(wl, device)
    lay = s["lay"]
    s["bws"] = torch.empty(itl.backward_workspace_bytes(lay.n_tok, wl.d, wl.vocab, s["H"].dtype), dtype=torch.uint8,
                           device=device)
    s["dH"] = torch.empty((lay.n_tok, wl.d), dtype=torch.float32, device=device)
    s["dW"] = torch.empty((wl.vocab, wl.d), dtype=torch.float32, device=device)
    return s


def fwd_bwd_step(s, ev=None):
    """Forward logprob, advantage, loss and backward; ev brackets the backward."""
    import invariant_token_logprobs_lm_amd as itl

    rl, L, coef = forward_step(s)
    if ev is not None:
        ev[0].record()
    itl.reinforce_zero_backward(s["H"], s["W"], s["y"], s["lse"], coef, dH=s["dH"], dW=s["dW"], workspace=s["bws"])
    if ev is not None:
        ev[1].record()


def fwd_bwd_keep_step(s, ev=None):
    """The same step with the forward's logits kept in HBM and the backward's
    dlogits formed from them (no recomputed contraction; same bits)."""
    import invariant_token_logprobs_lm_amd as itl

    itl.lmhead_logprob_keep_logits(s["H"], s["W"], s["y"], logits=s["Z"], logprob=s["lp"], lse=s["lse"],
                                   workspace=s["ws"])
    A = itl.group_advantage(s["rewards"], s["goff"])
    rl, L, coef = itl.reinforce_zero_loss(s["lp"], s["lpr"], A, s["roff"])
    if ev is not None:
        ev[0].record()
    itl.reinforce_zero_backward_from_logits(s["H"], s["W"], s["y"], s["lse"], coef, s["Z"], dH=s["dH"], dW=s["dW"],
                                            workspace=s["bws"])
    if ev is not None:
        ev[1].record()


def decode_leg(wl, device, batch_sizes=(1, 8, 64, 128, 256), calls=20):
    """Decode-shaped calls (a rollout engine's step: one new token for each of
    M sequences) on the head: the invariant kernel against a non-invariant
    fast baseline run as a library (hipBLASLt GEMM with bf16 logits, then
    torch log_softmax in fp32 and a gather). Also reports how far the
    baseline's logprob of one fixed token moves with the batch it runs in,
    against the invariant kernel's bit-identical results."""
    import torch
    import invariant_token_logprobs_lm_amd as itl
    from synth import draw_head, draw_layout

    M_max = max(batch_sizes)
    H, W = draw_head(wl, M_max, device=device, salt=3)
    g = torch.Generator(device=device)
    g.manual_seed(4000 + wl.index)
    y = torch.randint(0, wl.vocab, (M_max,), generator=g, device=device, dtype=torch.int32)

    def baseline(Hm, ym):
        z = torch.mm(Hm, W.t())
        return torch.log_softmax(z.float(), dim=1).gather(1, ym.long()[:, None])[:, 0]

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def graph_decode(Hm, ym, ws, steps=16, reps=5):
        """A serving loop's view: `steps` decode calls captured once in a HIP
        graph and replayed (no per-call launch cost on the host). Returns
        the per-call time and whether every replayed call gave the eager
        call's bits."""
        M = Hm.shape[0]
        out = torch.empty((steps, M), dtype=torch.float32, device=device)
        ref = itl.lmhead_logprob(Hm, W, ym, want_lse=False)[0]
        side = torch.cuda.Stream(device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
            for k in range(steps):
                itl.lmhead_logprob(Hm, W, ym, logprob=out[k], workspace=ws, want_lse=False)
        torch.cuda.current_stream(device).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(steps):
                itl.lmhead_logprob(Hm, W, ym, logprob=out[k], workspace=ws, want_lse=False)
        out.zero_()
        ms = timed(graph.replay, reps) / steps
        torch.cuda.synchronize()
        same = bool(torch.equal(out.view(torch.int32), ref.view(torch.int32).expand(steps, M)))
        return ms, same

    Wq8, ws8 = itl.quantize_rows_fp8(W)
    Wq4, ws4 = itl.quantize_rows_mxfp4(W)
    rows = []
    ours_ref = itl.lmhead_logprob(H[:1], W, y[:1], want_lse=False)[0]
    base_ref = baseline(H[:1], y[:1])
    max_base_drift = 0.0
    ours_identical = True
    for M in batch_sizes:
        Hm, ym = H[:M].contiguous(), y[:M].contiguous()
        ws = torch.empty(itl.lmhead_workspace_bytes(M, wl.vocab), dtype=torch.uint8, device=device)
        lp = torch.empty(M, dtype=torch.float32, device=device)
        ms_ours = timed(lambda: itl.lmhead_logprob(Hm, W, ym, logprob=lp, workspace=ws, want_lse=False), calls)
        ms_base = timed(lambda: baseline(Hm, ym), calls)
        Hq = torch.empty((M, wl.d), dtype=torch.uint8, device=device)
        hs = torch.empty(M, dtype=torch.float32, device=device)

        def q8():
            itl.quantize_rows_fp8(Hm, Xq=Hq, scale=hs)
            itl.lmhead_logprob_fp8(Hq, hs, Wq8, ws8, ym, logprob=lp, workspace=ws, want_lse=False)

        def q4():
            itl.quantize_rows_fp8(Hm, Xq=Hq, scale=hs)
            itl.lmhead_logprob_mxfp4(Hq, hs, Wq4, ws4, ym, logprob=lp, workspace=ws, want_lse=False)

        ms_fp8 = timed(q8, calls)
        ms_mx4 = timed(q4, calls)
        ms_graph, graph_same = graph_decode(Hm, ym, ws)
        itl.lmhead_logprob(Hm, W, ym, logprob=lp, workspace=ws, want_lse=False)
        lp_b = baseline(Hm, ym)
        torch.cuda.synchronize()
        ours_identical &= bool(torch.equal(lp[:1].view(torch.int32), ours_ref.view(torch.int32)))
        drift = float((lp_b[:1] - base_ref).abs().max())
        max_base_drift = max(max_base_drift, drift)
        rows.append({"batch": M, "ms_invariant": ms_ours, "ms_baseline": ms_base,
                     "tokens_per_s_invariant": M / (ms_ours * 1e-3), "tokens_per_s_baseline": M / (ms_base * 1e-3),
                     "invariant_over_baseline": ms_base / ms_ours,
                     "ms_invariant_fp8_weights": ms_fp8, "ms_invariant_mxfp4_weights": ms_mx4,
                     "ms_invariant_graph_replay": ms_graph, "graph_replay_bit_identical": graph_same,
                     "max_abs_lp_gap_to_baseline": float((lp - lp_b).abs().max())})
        log(f"[bench] decode M={M}: invariant {ms_ours:.3f} ms ({ms_graph:.3f} ms per call replayed from a graph, "
            f"bits {'identical' if graph_same else 'DIFFER'}), baseline {ms_base:.3f} ms "
            f"(throughput ratio {ms_base / ms_ours:.3f}); with FP8 weights {ms_fp8:.3f} ms, MXFP4 {ms_mx4:.3f} ms")
    return {
        "workload": f"{wl.key} decode-shaped calls (M sequences x 1 token), {calls} calls per point",
        "baseline": "torch.mm (hipBLASLt, bf16 logits) + log_softmax (fp32) + gather; not batch-invariant",
        "points": rows,
        "invariant_token0_bit_identical_across_batches": ours_identical,
        "baseline_token0_max_abs_drift_across_batches": max_base_drift,
    }


def prefill_leg(s, device, chunk=16384, calls=5):
    """Prefill-shaped calls on the same head: one chunk of the batch's tokens
    through the invariant kernel, against the library path an inference
    engine would take (hipBLASLt GEMM to bf16 logits, then torch log_softmax
    in fp32 and a gather; not batch-invariant), and against the library GEMM
    alone. The GEMM alone writes the chunk's logits and does nothing else:
    its rate is the plain contraction's, a practical ceiling for the fused
    kernel's matrix-core work on this shape."""
    import torch
    import invariant_token_logprobs_lm_amd as itl

    H, W, y = s["H"], s["W"], s["y"]
    n = min(chunk, H.shape[0])
    d = H.shape[1]
    V = W.shape[0]
    Hc, yc = H[:n].contiguous(), y[:n].contiguous()
    z = torch.empty((n, V), dtype=H.dtype, device=device)
    ws = torch.empty(itl.lmhead_workspace_bytes(n, V), dtype=torch.uint8, device=device)
    lp = torch.empty(n, dtype=torch.float32, device=device)
    Wt = W.t()

    def gemm():
        torch.mm(Hc, Wt, out=z)

    def fast():
        torch.mm(Hc, Wt, out=z)
        return torch.log_softmax(z.float(), dim=1).gather(1, yc.long()[:, None])[:, 0]

    def ours():
        itl.lmhead_logprob(Hc, W, yc, logprob=lp, workspace=ws, want_lse=False)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    ms_ours, ms_gemm, ms_fast = timed(ours), timed(gemm), timed(fast)
    lp_fast = fast()
    ours()
    torch.cuda.synchronize()
    gap = float((lp - lp_fast).abs().max())
    del z
    flop = 2.0 * d * V * n

    def tf(ms):
        return flop / (ms * 1e-3) / 1e12

    log(f"[bench] prefill chunk of {n} tokens: invariant {ms_ours:.2f} ms ({tf(ms_ours):.0f} TFLOP/s), "
        f"library GEMM alone {ms_gemm:.2f} ms ({tf(ms_gemm):.0f} TFLOP/s), "
        f"GEMM + log_softmax + gather {ms_fast:.2f} ms")
    return {
        "workload": f"first {n} tokens of the batch in one call, {calls} calls per point",
        "baseline": "torch.mm (hipBLASLt, bf16 logits) + log_softmax (fp32) + gather; not batch-invariant",
        "ms_invariant": ms_ours, "ms_library_gemm_only": ms_gemm, "ms_library_path": ms_fast,
        "tflops_invariant": tf(ms_ours), "tflops_library_gemm_only": tf(ms_gemm), "tflops_library_path": tf(ms_fast),
        "invariant_over_library_path": ms_fast / ms_ours,
        "max_abs_lp_gap_to_library_path": gap,
    }


def loss_leg(s, device, calls=20):
    """The group advantage and the REINFORCE Zero loss (with its per-token
    coefficients) on their own: at the benchmark batch, and scaled up to
    ~16.8M tokens as 65,536 responses of 256 tokens, as 2,048 of 8,192, and
    as 2M of 8, groups of 8. The loss runs a token pass (one workgroup per
    2048-token window of the packed batch, summing the response-relative
    segments that start in it: one lane per segment of up to 32 tokens, a
    wavefront up to 256, the workgroup beyond), a finishing pass over chunks
    of 1024 responses and, past one chunk, a final sum; the advantage reduces
    groups of up to 8 with eight lanes each. They move a few bytes per token
    and are HBM-bound in principle; the bytes counted are what the two calls
    must read and write (logprobs, rollout logprobs, coefficients, offsets,
    rewards, advantages, per-response losses). Each case is timed twice: as
    eager calls (host launch cost included, which dominates a small batch)
    and as the same calls captured once in a HIP graph and replayed (the
    device's own time; the figure reported as us_per_call)."""
    import torch
    import invariant_token_logprobs_lm_amd as itl

    def one(lp, lpr, rewards, goff, roff, ws):
        A = itl.group_advantage(rewards, goff)
        return itl.reinforce_zero_loss(lp, lpr, A, roff, workspace=ws)

    def timed(args):
        one(*args)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            one(*args)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    def timed_graph(args, reps=5):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one(*args)  # warm the allocator on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(calls):
                one(*args)
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        del graph
        return a.elapsed_time(b) / (reps * calls)

    def case(name, lp, lpr, rewards, goff, roff):
        n_tok, n_resp, n_grp = lp.numel(), rewards.numel(), goff.numel() - 1
        ws = torch.empty(max(itl.loss_workspace_bytes(n_tok, n_resp), 1), dtype=torch.uint8, device=device)
        args = (lp, lpr, rewards, goff, roff, ws)
        ms_eager = timed(args)
        ms = timed_graph(args)
        nbytes = 12 * n_tok + (8 + 4 + 4 + 4 + 4) * n_resp + 4 * n_grp
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"[bench] advantage + loss, {name}: {ms * 1e3:.1f} us per call replayed from a graph "
            f"({ms_eager * 1e3:.1f} us eager), {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.2f}% of HBM peak)")
        return {"case": name, "n_tok": n_tok, "responses": n_resp, "us_per_call": ms * 1e3,
                "us_per_call_eager": ms_eager * 1e3, "bytes_per_call": nbytes, "gb_per_s": gbs,
                "frac_hbm_peak": gbs / PEAK_HBM_GBS}

    out = [case("benchmark batch", s["lp"], s["lpr"], s["rewards"], s["goff"], s["roff"])]
    g = torch.Generator(device=device)
    g.manual_seed(7)
    for n_resp, T in ((65536, 256), (2048, 8192), (2 * 1024 * 1024, 8)):
        n = n_resp * T
        lp = -torch.rand(n, generator=g, device=device) * 20
        lpr = lp + torch.randn(n, generator=g, device=device) * 0.05
        rewards = torch.rand(n_resp, generator=g, device=device)
        roff = torch.arange(0, n + 1, T, dtype=torch.int64, device=device)
        goff = torch.arange(0, n_resp + 1, 8, dtype=torch.int32, device=device)
        out.append(case(f"{n_resp} responses x {T} tokens", lp, lpr, rewards, goff, roff))
        del lp, lpr, rewards, roff, goff
    return out


def mismatch_leg(s, device, calls=20, n_demo=4096, batch=64):
    """The mismatch diagnostics: (1) itl_mismatch_stats timed on the whole
    batch (learner logprobs, the rollout record with the workload's lag
    noise, the aligned same-weights logprobs); (2) the kernel part of the gap
    at equal weights on a seeded subset of tokens, for two rollouts of the
    same tokens in decode-shaped calls of `batch` tokens: this library
    (aligned) and the fast non-invariant path (bf16 logits + log_softmax)."""
    import torch
    import invariant_token_logprobs_lm_amd as itl
    from synth import token_subset

    lp, lpr = s["lp"], s["lpr"]
    n = lp.shape[0]
    st = torch.empty(len(itl.STAT_FIELDS), dtype=torch.float64, device=device)
    ws = torch.empty(max(itl.mismatch_stats_workspace_bytes(n), 1), dtype=torch.uint8, device=device)
    same = lpr.clone()
    itl.mismatch_stats(lp, lpr, same, stats=st, workspace=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        itl.mismatch_stats(lp, lpr, same, stats=st, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / calls
    full = itl.stats_dict(st)
    log(f"[bench] mismatch stats over {n} tokens: {ms * 1e3:.1f} us/call ({12.0 * n / (ms * 1e-3) / 1e9:.1f} GB/s of "
        f"input); lag k3 {full['kl_k3']:.3e}, weight deviation peak/median {full['deviation_peak_over_median']:.2f}")

    idx = torch.from_numpy(token_subset(n, n_demo, seed=77)).to(device)
    H, W, y = s["H"].index_select(0, idx).contiguous(), s["W"], s["y"].index_select(0, idx).contiguous()
    learner, _ = itl.lmhead_logprob(H, W, y)  # the learner: one call over the whole subset
    aligned = torch.empty_like(learner)
    fast = torch.empty_like(learner)
    for c0 in range(0, n_demo, batch):
        sl = slice(c0, min(c0 + batch, n_demo))
        aligned[sl] = itl.lmhead_logprob(H[sl], W, y[sl], want_lse=False)[0]
        z = torch.mm(H[sl], W.t())
        fast[sl] = torch.log_softmax(z.float(), dim=1).gather(1, y[sl].long()[:, None])[:, 0]
    rows = {}
    for name, roll in (("aligned", aligned), ("fast_non_invariant", fast)):
        # equal weights: the learner's computation at the rollout's weights
        # is the learner's own result, so the whole gap is the kernel part
        d = itl.stats_dict(itl.mismatch_stats(learner, roll, learner))
        rows[name] = {k: d[k] for k in ("kernel_nonzero", "kernel_abs_max", "kernel_kl_k3", "deviation_max",
                                         "deviation_median", "deviation_peak_over_median")}
        log(f"[bench] kernel mismatch, {name} rollout: {int(d['kernel_nonzero'])}/{n_demo} tokens differ, "
            f"max |dlp| {d['kernel_abs_max']:.3e}, weight deviation peak/median {d['deviation_peak_over_median']:.2f}")
    return {
        "kernel": "itl_mismatch_stats (terms + exact median by radix selection + finalize)",
        "n_tok": n,
        "us_per_call": ms * 1e3,
        "input_gb_per_s": 12.0 * n / (ms * 1e-3) / 1e9,
        "stats_full_batch": full,
        "kernel_part_at_equal_weights": {
            "tokens": n_demo,
            "rollout_calls_of": batch,
            "learner": "this library, one call over all the tokens",
            **rows,
        },
    }


def fp8_leg(s, device, steps=5):
    """The same workload on the FP8 (E4M3, per-row scales) head: W quantised
    once (not timed); a step = quantise H + the fp8 logprob kernel."""
    import torch
    import invariant_token_logprobs_lm_amd as itl

    H, W, y, lp_bf16 = s["H"], s["W"], s["y"], s["lp"]
    n, d = H.shape
    V = W.shape[0]
    Wq, ws = itl.quantize_rows_fp8(W)
    Hq = torch.empty((n, d), dtype=torch.uint8, device=device)
    hs = torch.empty(n, dtype=torch.float32, device=device)
    lp = torch.empty(n, dtype=torch.float32, device=device)
    wsp = torch.empty(itl.lmhead_workspace_bytes(n, V), dtype=torch.uint8, device=device)

    def step():
        itl.quantize_rows_fp8(H, Xq=Hq, scale=hs)
        itl.lmhead_logprob_fp8(Hq, hs, Wq, ws, y, logprob=lp, workspace=wsp, want_lse=False)

    step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    q0.record()
    itl.quantize_rows_fp8(H, Xq=Hq, scale=hs)
    q1.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    ms_q = q0.elapsed_time(q1)
    tf = 2.0 * d * V * n / ((ms - ms_q) * 1e-3) / 1e12
    gap = float((lp - lp_bf16).abs().max())
    log(f"[bench] fp8 head: step {ms:.2f} ms (H quantisation {ms_q:.2f} ms) -> {n / (ms * 1e-3):.0f} tokens/s, "
        f"logprob kernel {tf:.1f} TFLOP/s ({100 * tf / PEAK_FP8_TFLOPS:.1f}% of fp8 peak); max |lp_fp8 - lp_bf16| {gap:.3e}")
    del Wq, ws
    # MXFP4 weights (E2M1, E8M0 per 32 along d) against the same E4M3 token rows
    W4, w4s = itl.quantize_rows_mxfp4(W)

    def step4():
        itl.quantize_rows_fp8(H, Xq=Hq, scale=hs)
        itl.lmhead_logprob_mxfp4(Hq, hs, W4, w4s, y, logprob=lp, workspace=wsp, want_lse=False)

    step4()
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        step4()
    b.record()
    torch.cuda.synchronize()
    ms4 = a.elapsed_time(b) / steps
    tf4 = 2.0 * d * V * n / ((ms4 - ms_q) * 1e-3) / 1e12
    gap4 = float((lp - lp_bf16).abs().max())
    log(f"[bench] mxfp4 head: step {ms4:.2f} ms -> {n / (ms4 * 1e-3):.0f} tokens/s, logprob kernel {tf4:.1f} "
        f"TFLOP/s ({100 * tf4 / PEAK_FP8_TFLOPS:.1f}% of the fp8 peak); max |lp_mxfp4 - lp_bf16| {gap4:.3e}")
    return {
        "mxfp4": {"ms_per_step": ms4, "value": n / (ms4 * 1e-3), "tflops_logprob_kernel": tf4,
                  "frac_fp8_peak": tf4 / PEAK_FP8_TFLOPS, "max_abs_lp_gap_to_bf16_head": gap4,
                  "weights": "E2M1 codes + E8M0 scale per 32 along d; tokens E4M3 per-row"},
        "workload": "same tokens and head; W quantised once to E4M3 with per-row scales, H per step",
        "ms_per_step": ms,
        "ms_quantize_h": ms_q,
        "value": n / (ms * 1e-3),
        "unit": "sampled-token logprobs/s",
        "tflops_logprob_kernel": tf,
        "peak_fp8_tflops": PEAK_FP8_TFLOPS,
        "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
        "max_abs_lp_gap_to_bf16_head": gap,
    }


PROBE_SHAPES = {
    0: "v_mfma_f32_32x32x16_bf16, 4x4 block tile per wavefront, one wavefront per SIMD",
    1: "v_mfma_f32_16x16x32_bf16, 8x4 block tile per wavefront, two wavefronts per SIMD "
       "(the bf16 forward's instruction and wavefront tile)",
}


def sustained_mfma_probe(device, shape, blocks=1024, iters=40000):
    """TFLOP/s that a bf16 MFMA shape (PROBE_SHAPES) sustains on this chip
    with operands that change every instruction (random normal bf16 values)
    and no memory traffic: the power-limited ceiling a real contraction
    meets, measured with the probe library (bench_mfma_probe.hip) built
    beside this file."""
    import ctypes
    import torch

    path = os.path.join(ROOT, "libitl_bench_probe.so")
    lib = ctypes.CDLL(path)
    lib.itl_probe_operand_bytes.restype = ctypes.c_size_t
    lib.itl_probe_threads.restype = ctypes.c_int
    lib.itl_probe_threads.argtypes = [ctypes.c_int]
    lib.itl_probe_flops.restype = ctypes.c_double
    lib.itl_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.itl_probe_mfma_bf16.restype = ctypes.c_int
    lib.itl_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    g = torch.Generator(device="cpu").manual_seed(5150)
    n = lib.itl_probe_operand_bytes() // 2
    ops = torch.randn(n, generator=g).to(torch.bfloat16).to(device)
    out = torch.empty(blocks * lib.itl_probe_threads(shape), dtype=torch.float32, device=device)
    st = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    opp, outp = ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr())
    assert lib.itl_probe_mfma_bf16(shape, opp, outp, blocks, 100, st) == 0
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    assert lib.itl_probe_mfma_bf16(shape, opp, outp, blocks, iters, st) == 0
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    tf = lib.itl_probe_flops(shape, blocks, iters) / (ms * 1e-3) / 1e12
    log(f"[bench] matrix-core probe ({PROBE_SHAPES[shape]}; random bf16 operands, no memory traffic): "
        f"{tf:.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:.1f}% of the published peak) in {ms:.1f} ms")
    return tf


def cpu_baseline(wl, n_sample=6144):
    """The float64 oracle timed on a seeded sample of the same workload's
    tokens (forward + loss over the sampled tokens)."""
    import numpy as np
    import torch
    import oracle
    from synth import draw_head, draw_layout, sample_tokens, token_subset

    lay = draw_layout(wl)
    dev = torch.device("cuda:0")
    H, W = draw_head(wl, lay.n_tok, device=dev)
    y = sample_tokens(H, W, wl)
    idx = token_subset(lay.n_tok, n_sample, seed=100 + wl.index)
    it = torch.from_numpy(idx).to(dev)
    Hs = H.index_select(0, it).cpu().view(torch.int16).numpy().view(np.uint16)
    Wh = W.cpu().view(torch.int16).numpy().view(np.uint16)
    ys = y.index_select(0, it).cpu().numpy()
    del H, W
    # the sample's response structure: responses with at least one sampled token
    resp_of = np.searchsorted(lay.resp_offsets, idx, side="right") - 1
    resp_ids, counts = np.unique(resp_of, return_counts=True)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    noise = lay.lag_noise[idx].astype(np.float64)
    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    t0 = time.perf_counter()
    lp, _ = oracle.lmhead_logprob(Hs, Wh, ys)
    A = oracle.group_advantage(lay.rewards, lay.group_offsets)[resp_ids]
    oracle.reinforce_zero_loss(lp, lp + noise, A, off)
    el = time.perf_counter() - t0
    return {
        "value": n_sample / el,
        "unit": "sampled-token logprobs/s",
        "cores": threads if threads else len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{n_sample} seeded tokens of the {wl.key} workload (d={wl.d}, vocab={wl.vocab}): "
                   f"float64 logits over the full vocabulary, log-softmax, gather, and the loss over the "
                   f"{resp_ids.size} responses they fall in; {el:.1f} s"),
        "seconds": el,
    }


def cpu_baseline_fwd_bwd(s, wl, n_sample=192):
    """The float64 oracle's forward + loss + backward timed on a seeded sample
    of the backward workload's tokens: their logprobs over the full
    vocabulary, the loss over the responses they fall in (with the sample's
    own response structure), and dH / dW of that loss (every vocabulary
    row), on the host's cores."""
    import numpy as np
    import torch
    import oracle
    from synth import token_subset

    lay = s["lay"]
    idx = token_subset(lay.n_tok, n_sample, seed=200 + wl.index)
    it = torch.from_numpy(idx).to(s["H"].device)
    Hs = s["H"].index_select(0, it).cpu().view(torch.int16).numpy().view(np.uint16)
    Wh = s["W"].cpu().view(torch.int16).numpy().view(np.uint16)
    ys = s["y"].index_select(0, it).cpu().numpy()
    resp_of = np.searchsorted(lay.resp_offsets, idx, side="right") - 1
    resp_ids, counts = np.unique(resp_of, return_counts=True)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    noise = lay.lag_noise[idx].astype(np.float64)
    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    t0 = time.perf_counter()
    lp, _ = oracle.lmhead_logprob(Hs, Wh, ys)
    A = oracle.group_advantage(lay.rewards, lay.group_offsets)[resp_ids]
    _, _, coef = oracle.reinforce_zero_loss(lp, lp + noise, A, off)
    oracle.reinforce_zero_backward(Hs, Wh, ys, coef)
    el = time.perf_counter() - t0
    return {
        "value": n_sample / el,
        "unit": "sampled tokens/s (forward + backward)",
        "cores": threads if threads else len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{n_sample} seeded tokens of the {wl.key} workload (d={wl.d}, vocab={wl.vocab}): float64 "
                   f"logprobs over the full vocabulary, the loss over the {resp_ids.size} responses they fall in, "
                   f"and dH, dW of that loss (dW over every vocabulary row); {el:.1f} s"),
        "seconds": el,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3-4b-head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-loss", action="store_true")
    ap.add_argument("--no-mismatch", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-other-forward", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="before timing, run one plain 1 GiB device-to-device copy: the reference whose "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path is built and timed on a single MI355X "
              f"(--gpus {args.gpus} requested); multi-GPU sharding is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import WORKLOADS

    device = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    if args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
    s = setup_forward(wl, device)
    n_tok = s["lay"].n_tok
    ms_step, ms_head, wall = time_steps(lambda ev: forward_step(s, ev), args.steps, args.warmup)
    flops = 2.0 * wl.d * wl.vocab * n_tok
    achieved = flops / (ms_head * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms, lmhead {ms_head:.3f} ms -> {achieved:.1f} TFLOP/s "
        f"({100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak), wall {wall:.2f}s")
    traffic = measured_traffic(wl.key)
    sustained = sustained_mfma_probe(device, 1)
    sustained32 = sustained_mfma_probe(device, 0)
    out = {
        "metric": METRIC,
        "value": n_tok / (ms_step * 1e-3),
        "unit": "sampled-token logprobs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.key} forward logprob + group advantage + REINFORCE Zero loss",
            "d": wl.d,
            "vocab": wl.vocab,
            "responses": s["lay"].n_resp,
            "n_tok": n_tok,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "lmhead_lse_partial8 (+ lse_combine)",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "flop_per_launch": flops,
            "ms_per_launch": ms_head,
            "sustained_mfma_probe": {
                "value": sustained,
                "unit": "TFLOP/s",
                "what": PROBE_SHAPES[1] + "; random bf16 operands changing every instruction, no memory traffic "
                        "(power-limited clock)",
                "frac_of_probe": achieved / sustained,
                "other_shape": {"what": PROBE_SHAPES[0], "value": sustained32},
            },
        },
    }
    if not args.no_mismatch:
        out["mismatch"] = mismatch_leg(s, device)
    if not args.no_fp8:
        out["fp8"] = fp8_leg(s, device)
    if not args.no_prefill:
        out["prefill"] = prefill_leg(s, device)
    if not args.no_loss:
        out["loss"] = loss_leg(s, device)
    del s
    torch.cuda.empty_cache()
    if not args.no_other_forward:
        # the other forward workloads of the table: the 1.5B-shaped head, and
        # the tiny fp32 head (launch-bound: a few microseconds per call)
        out["forward_other"] = {k: forward_leg(k, device, args.steps) for k in ("qwen2.5-1.5b-head", "tiny")
                                if k != wl.key}
    if not args.no_decode:
        out["decode"] = decode_leg(wl, device)
        torch.cuda.empty_cache()
    if not args.no_backward:
        wb = WORKLOADS["large-moe-head"]
        sb = setup_backward(wb, device)
        nb = sb["lay"].n_tok
        bsteps = max(1, min(args.steps, 3))
        ms_fb, ms_bwd, wall_b = time_steps(lambda ev: fwd_bwd_step(sb, ev), bsteps, 1)
        fl_alg = 6.0 * wb.d * wb.vocab * nb  # forward 2dV + dH 2dV + dW 2dV per token (recompute not credited)
        tf = fl_alg / (ms_fb * 1e-3) / 1e12
        log(f"[bench] {wb.key} fwd+bwd step {ms_fb:.1f} ms (backward {ms_bwd:.1f} ms) -> {nb / (ms_fb * 1e-3):.0f} "
            f"tokens/s, {tf:.1f} TFLOP/s algorithmic ({100 * tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
        out["fwd_bwd"] = {
            "workload": f"{wb.key} forward logprob + group advantage + REINFORCE Zero loss + backward (dH, dW)",
            "d": wb.d,
            "vocab": wb.vocab,
            "responses": sb["lay"].n_resp,
            "n_tok": nb,
            "steps": bsteps,
            "ms_per_step": ms_fb,
            "ms_backward": ms_bwd,
            "value": nb / (ms_fb * 1e-3),
            "unit": "sampled tokens/s (forward + backward)",
            "tflops_algorithmic": tf,
            "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "path": "the backward recomputes the logits with the forward's contraction",
        }
        # The same step with the logits kept (4 n_tok vocab bytes of HBM)
        # when they fit beside everything else.
        free, _ = torch.cuda.mem_get_info(device)
        z_bytes = nb * ((wb.vocab + 3) // 4 * 4) * 4
        if free > z_bytes + (8 << 30):
            sb["Z"] = torch.empty((nb, (wb.vocab + 3) // 4 * 4), dtype=torch.float32, device=device)
            ms_k, ms_kb, _ = time_steps(lambda ev: fwd_bwd_keep_step(sb, ev), bsteps, 1)
            tfk = fl_alg / (ms_k * 1e-3) / 1e12
            log(f"[bench] {wb.key} fwd+bwd step with kept logits {ms_k:.1f} ms (backward {ms_kb:.1f} ms) -> "
                f"{nb / (ms_k * 1e-3):.0f} tokens/s, {tfk:.1f} TFLOP/s algorithmic "
                f"({100 * tfk / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
            # The faster path is the leg's figure; the recomputing one stays beside it.
            recompute = {k: out["fwd_bwd"][k] for k in ("ms_per_step", "ms_backward", "value", "tflops_algorithmic",
                                                        "frac_bf16_peak")}
            recompute["what"] = "the backward recomputes the logits with the forward's contraction"
            out["fwd_bwd"].update({
                "path": "kept logits: the forward also writes the fp32 logits and the backward forms its dlogits "
                        "from them instead of recomputing the contraction (same dH and dW bits)",
                "logits_bytes": z_bytes,
                "ms_per_step": ms_k,
                "ms_backward": ms_kb,
                "value": nb / (ms_k * 1e-3),
                "tflops_algorithmic": tfk,
                "frac_bf16_peak": tfk / PEAK_BF16_TFLOPS,
                "recompute": recompute,
            })
        else:
            log(f"[bench] kept-logits step skipped: {z_bytes / 2**30:.0f} GiB of logits, {free / 2**30:.0f} GiB free")
        sb.pop("Z", None)
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle's forward + backward on a bounded sample ...")
            out["fwd_bwd"]["cpu_baseline"] = cpu_baseline_fwd_bwd(sb, wb)
            log(f"[bench] oracle fwd+bwd {out['fwd_bwd']['cpu_baseline']['value']:.1f} tokens/s in "
                f"{out['fwd_bwd']['cpu_baseline']['seconds']:.1f}s")
        del sb
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(wl)
        log(f"[bench] oracle {out['cpu_baseline']['value']:.1f} tokens/s in {out['cpu_baseline']['seconds']:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
