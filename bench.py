#!/usr/bin/env python3
"""Throughput of the masked-diffusion loss path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
mdlm_corrupt -> mdlm_compact_masked -> mdlm_fused_head_ce_fwd_bwd (loss and
d_hidden), enqueued on one stream with no host synchronisation.  Each timed
step draws fresh noise (Philox seed = step index), as a training loop would.

Default workload: one sequence of 4,096 tokens, H = 4,096, V = 126,464, bf16
inputs with fp32 accumulation, absorbing noise (eps = 1e-3), aligned logits
(LLaDA-8B-MDLM-LoRA card, Training table: a batch holds sequences no longer
than 4,096 tokens; the base weights are bf16).  Inputs are seeded synthetic data resident in HBM
before timing starts.

Prints ONE JSON line: tokens/s of whole steps, the roofline of the fused
head + CE call (4 M H V flops per call: the logits product and the d_hidden
product, which is also what the call executes with its full workspace, over
its HIP-event time on the launch stream, against the 2.5 PFLOP/s dense bf16
MFMA peak), the
HBM rate of corruption and compaction at 2^27 tokens, and the fp64 CPU oracle
timed on a bounded sample of the same workload.
"""

import argparse
import contextlib
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "corrupted-LM loss fwd+bwd tokens/s at V=126,464; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_VALU_TFLOPS = 157.3   # the fp32 path runs on the vector ALUs
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # ~0.1 s of steps: the GPU's speed settles after the idle set-up
    p.add_argument("--warmup", type=int, default=25)
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--align", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the loss variants (encoder AR term, head-weight gradient, "
                        "row-list modes)")
    p.add_argument("--no-achievable", action="store_true",
                   help="skip the achievable-peak probes (copy, MFMA loop, library GEMM)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip timing the other bf16 workloads (varlen, packed, canvas)")
    p.add_argument("--other-steps", type=int, default=10)
    p.add_argument("--bandwidth-tokens", type=int, default=1 << 27,
                   help="tokens of the corruption/compaction bandwidth run (0 = skip)")
    p.add_argument("--calibrate-copy", type=int, default=0,
                   help="before timing, copy this many MiB once with the probe library's "
                        "copy kernel, so counter runs can scale their byte counts by a "
                        "known transfer")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles",
                                                          "head_ce_traffic.json"),
                   help="measured HBM traffic of the fused call, if current")
    return p.parse_args()


@contextlib.contextmanager
def quiet_host():
    """No Python garbage collection inside a timed region: a collection that
    lands between a start event and the launches after it (when the GPU
    queue is empty) shows up in the event time as a gap with no kernel
    running."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def head_source_sha256():
    """sha256 of the fused call's kernel source, to tie counter results to it."""
    import hashlib
    path = os.path.join(ROOT, "uniform_noise_diffusion_amd", "csrc", "head_ce.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def to_device(inp, dev):
    import torch
    x0 = torch.from_numpy(inp.x0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    if inp.wl.dtype == "bf16":
        h = torch.from_numpy(inp.hidden_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(inp.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        h = torch.from_numpy(inp.hidden).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    return x0, cu, h, W


def gpu_steps(args, inp, dev):
    import torch
    from uniform_noise_diffusion_amd.pipeline import MdlmLossStep
    wl = inp.wl
    align = wl.align if args.align is None else args.align
    x0, cu, h, W = to_device(inp, dev)
    dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=dtype, device=dev)

    def one(seed, ev=None):
        # (events on torch's current stream, which the calls are launched on)
        if ev is not None:
            ev[0].record()
        step.corrupt(x0, cu, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab)
        step.compact(x0, cu, align)
        if ev is not None:
            ev[1].record()
        step.head_ce(h, W, wl.softcap, row_ce=False)
        if ev is not None:
            ev[2].record()

    K = args.steps
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # (the host's garbage collection runs before the warm-up steps, so that
    # only the synchronize separates them from the timed steps: after an idle
    # spell the GPU's next tens of milliseconds of work run measurably slower)
    with quiet_host():
        for i in range(args.warmup):
            one(1_000_000 + i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(K):
            one(i, evs[i])
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    head_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    losses = []
    rows = []
    # scored-row counts of the timed seeds, recomputed after the timed region
    for i in range(K):
        step.corrupt(x0, cu, i, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab)
        step.compact(x0, cu, align)
        rows.append(int(step.n_rows.item()))
    step.head_ce(h, W, wl.softcap)
    torch.cuda.synchronize()
    losses.append(float(step.loss.item()))
    if not all(np.isfinite(losses)):
        raise RuntimeError("non-finite loss")
    return dict(total_ms=total_ms, wall_s=wall, head_ms=head_ms, step_ms=step_ms, rows=rows,
                align=align)


def bandwidth(n_tokens, dev, reps=10, doc_mean=None):
    """Corruption and compaction at a bandwidth-sized stream of 2^27 tokens:
    documents of 4,096 tokens (32,768 documents), or lognormal lengths with
    arithmetic mean ``doc_mean`` (sigma 1, clipped to [16, 4096])."""
    import torch
    import workloads as WL
    from uniform_noise_diffusion_amd.pipeline import MdlmLossStep
    if doc_mean is None:
        L = 4096
        n = n_tokens // L * L
        cu = torch.arange(0, n + 1, L, dtype=torch.int32, device=dev)
    else:
        n = n_tokens
        cu = torch.from_numpy(
            WL.lognormal_stream_offsets(5000 + doc_mean, doc_mean, n).astype(np.int32)).to(dev)
    n_docs = cu.numel() - 1
    g = torch.Generator(device=dev).manual_seed(0)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=dev, generator=g)
    step = MdlmLossStep(n, n_docs, 64, 64, device=dev, head_workspace_bytes=0, want_grad=False)
    # the one-pass call: the same outputs as the two calls
    from uniform_noise_diffusion_amd import binding as B
    ws = torch.empty(B.mdlm_corrupt_compact_workspace_bytes(n), dtype=torch.uint8, device=dev)

    def fused(seed):
        B.mdlm_corrupt_compact(x0, cu, seed, 1e-3, 0, 126336, 126464, 0, step.xt, step.corrupted,
                               step.p_doc, step.doc_counts, step.row_idx, step.tgt, step.w,
                               step.n_rows, ws)
    # The two forms are timed alternately (call i of each on the same seed),
    # right behind an untimed warm-up of about 0.1 s that is queued with no
    # wait in between: when the GPU has been idle, even for a few
    # milliseconds, calls of this size drift in time over the next tens of
    # milliseconds (up to 20% slower, then settling).
    ec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    ef = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    with quiet_host():
        for i in range(100):
            step.corrupt(x0, cu, i, 1e-3, 0, 126336, 126464)
            step.compact(x0, cu, 0)
            fused(i)
        for i in range(reps):
            ec[i][0].record()
            step.corrupt(x0, cu, 100 + i, 1e-3, 0, 126336, 126464)
            ec[i][1].record()
            step.compact(x0, cu, 0)
            ec[i][2].record()
            ef[i][0].record()
            fused(100 + i)
            ef[i][1].record()
        torch.cuda.synchronize()
    # medians over the repetitions (the per-repetition times are reported too)
    r_cor = [a.elapsed_time(b) * 1e3 for a, b, _ in ec]
    r_cmp = [b.elapsed_time(c) * 1e3 for _, b, c in ec]
    t_cor = float(np.median(r_cor)) * 1e-6
    t_cmp = float(np.median(r_cmp)) * 1e-6
    r_fused = [a.elapsed_time(b) * 1e3 for a, b in ef]
    t_fused = float(np.median(r_fused)) * 1e-6
    # (each fused call repeats the two-call pair's seed: the same rows)
    m = m_fused = int(step.n_rows.item())
    b_fused = 9.0 * n + 12.0 * m_fused
    # algorithmic bytes: corrupt reads x0 (4 B) and writes xt (4 B) and the
    # mask (1 B) per token; compact reads the mask (1 B) per token and, per
    # scored row, the target (4 B) and writes row, target and weight (12 B)
    b_cor = 9.0 * n
    b_cmp = 1.0 * n + 16.0 * m
    return dict(docs="4096 each" if doc_mean is None else f"lognormal mean {doc_mean}",
                n_tokens=n, n_docs=n_docs, scored_rows=m,
                corrupt_us=t_cor * 1e6, corrupt_GBs=b_cor / t_cor / 1e9,
                corrupt_frac=b_cor / t_cor / 1e9 / PEAK_HBM_GBS,
                compact_us=t_cmp * 1e6, compact_GBs=b_cmp / t_cmp / 1e9,
                compact_frac=b_cmp / t_cmp / 1e9 / PEAK_HBM_GBS,
                fused_us=t_fused * 1e6, fused_GBs=b_fused / t_fused / 1e9,
                fused_frac=b_fused / t_fused / 1e9 / PEAK_HBM_GBS,
                two_calls_us=(t_cor + t_cmp) * 1e6,
                timing=(f"medians over {reps} calls (HIP events on the launch stream), the "
                        "two-call pair and the one call alternating right behind 100 untimed "
                        "rounds; "
                        "per call below, in us"),
                corrupt_us_per_call=[round(x, 1) for x in r_cor],
                compact_us_per_call=[round(x, 1) for x in r_cmp],
                fused_us_per_call=[round(x, 1) for x in r_fused],
                fused_what=("mdlm_corrupt_compact (corruption writing per-tile counts, then "
                            "the row list without a count pass); algorithmic bytes 9 per token "
                            "(x0 read, xt and mask written) + 12 per scored row (row, target, "
                            "weight written; the target is the token already read) -- the "
                            "least any implementation moves; this one also reads the mask and "
                            "x0 again (5 bytes per token)"))


def achievable(dev, gemm_shape=None):
    """Measured achievable peaks on this GPU, beside the datasheet ones: the
    one-pass streaming copy and the MFMA issue loop of libmdlm_probe.so, and
    (context only) a library bf16 GEMM of the forward logits' shape."""
    import torch
    from uniform_noise_diffusion_amd import probe
    n = 2 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    probe.copy(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        probe.copy(a, b)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(4 * cus * 8, dtype=torch.float32, device=dev)
    probe.mfma(out, 4 * cus, 2000)
    torch.cuda.synchronize()
    e0.record()
    fl = probe.mfma(out, 4 * cus, 20000)
    e1.record()
    torch.cuda.synchronize()
    mfma_tf = fl / (e0.elapsed_time(e1) * 1e-3) / 1e12
    res = dict(copy_GBs=copy_gbs, mfma_bf16_tflops=mfma_tf,
               how=("copy: 2 GiB, one 16-byte element per thread, mean of 5; mfma: "
                    f"{4 * cus} workgroups x 8 waves, 8 independent 32x32x16 bf16 MFMA chains "
                    "per wave from registers (no memory traffic)"))
    if gemm_shape is not None:
        V, H, M = gemm_shape
        A = torch.randn(V, H, device=dev).to(torch.bfloat16)
        B = torch.randn(M, H, device=dev).to(torch.bfloat16)
        C = A @ B.t().contiguous()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            C = A @ B.t().contiguous()
        e1.record()
        torch.cuda.synchronize()
        res["library_gemm_tflops"] = 2.0 * V * H * M * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res["library_gemm"] = (f"torch.matmul (hipBLASLt) bf16 [{V} x {H}] x [{H} x {M}], the "
                               "forward logits' shape, output written; context, not a target")
        del A, B, C
        # the library's rate on a large square product, where it is at its best
        S = 8192
        A = torch.randn(S, S, device=dev).to(torch.bfloat16)
        B = torch.randn(S, S, device=dev).to(torch.bfloat16)
        C = A @ B
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            C = A @ B
        e1.record()
        torch.cuda.synchronize()
        res["library_gemm_square_tflops"] = 2.0 * S ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res["library_gemm_square"] = (f"torch.matmul (hipBLASLt) bf16 {S} x {S} x {S}; context "
                                      "for what a library GEMM reaches on this GPU")
        del A, B, C
    return res


def _timed(fn, reps):
    """Mean seconds per call of `reps` calls of fn (HIP events), queued right
    behind untimed calls worth about 0.1 s with no wait in between: after
    even a short idle spell the GPU's next tens of milliseconds of work run
    at a drifting speed."""
    import torch
    a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    fn()
    b0.record()
    torch.cuda.synchronize()
    warm = int(min(50, max(2, np.ceil(100.0 / max(a0.elapsed_time(b0), 1e-3)))))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    with quiet_host():
        for _ in range(warm):
            fn()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3


def variants(inp, dev, n_bw, reps=5):
    """The loss variants on the same workload: the encoder AR term (every-token
    causal rows of mdlm_compact_rows, then the fused head on them), the
    head-weight gradient call, the fused call with a backward that recomputes
    the logits (a workspace just short of the preferred size), the fused call
    on one eighth of the vocabulary (one GPU's share of a vocabulary-parallel
    head), and mdlm_compact_rows' other modes and the corrective mixture at
    the bandwidth size."""
    import torch
    from uniform_noise_diffusion_amd import binding as B
    from uniform_noise_diffusion_amd.pipeline import MdlmLossStep
    wl = inp.wl
    x0, cu, h, W = to_device(inp, dev)
    out = {}
    if wl.dtype != "bf16":
        return out
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, device=dev)
    HV = float(wl.H) * wl.V
    # encoder AR term: lambda * causal next-token CE over the clean sequence
    step.compact_rows(x0, cu, 1, B.MDLM_WEIGHT_MEAN, 0.5, corrupted=None)
    t_rows = _timed(lambda: step.compact_rows(x0, cu, 1, B.MDLM_WEIGHT_MEAN, 0.5,
                                              corrupted=None), reps)
    m = int(step.n_rows.item())
    t_head = _timed(lambda: step.head_ce(h, W, wl.softcap, row_ce=False), reps)
    out["encoder_ar_term"] = dict(
        rows=m, compact_rows_us=t_rows * 1e6, head_ms=t_head * 1e3,
        head_algorithmic_tflops=4 * m * HV / t_head / 1e12,
        what="mdlm_compact_rows(every token, shifted, mean weights x 0.5) then "
             "mdlm_fused_head_ce_fwd_bwd on those rows")
    # head-weight gradient on the masked rows of seeds 0..reps-1
    ws = torch.empty(B.mdlm_head_ce_dw_workspace_bytes(wl.n_tokens, wl.H, wl.V),
                     dtype=torch.uint8, device=dev)
    dW = torch.empty((wl.V, wl.H), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    # the same call with a workspace one 256-column chunk short of G over the
    # whole vocabulary: the backward then recomputes the logits (in two
    # vocabulary chunks) instead of using the forward pass's stash
    ws_rc = torch.empty(B.mdlm_head_ce_workspace_bytes(wl.n_tokens, wl.H, wl.V, B.MDLM_BF16)
                        - wl.n_tokens * 256 * 2, dtype=torch.uint8, device=dev)
    t_dw, t_plain, t_rc, rows = [], [], [], []
    for seed in range(reps):
        step.corrupt(x0, cu, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab)
        step.compact(x0, cu, wl.align)
        rows.append(int(step.n_rows.item()))
        t_dw.append(_timed(lambda: B.mdlm_fused_head_ce_fwd_bwd_dw(
            h, W, step.row_idx, step.tgt, step.w, step.n_rows, wl.n_tokens, wl.softcap, loss,
            None, step.d_hidden, dW, ws), 2))
        t_plain.append(_timed(lambda: step.head_ce(h, W, wl.softcap, row_ce=False), 2))
        t_rc.append(_timed(lambda: B.mdlm_fused_head_ce_fwd_bwd(
            h, W, step.row_idx, step.tgt, step.w, step.n_rows, wl.n_tokens, wl.softcap, loss,
            None, step.d_hidden, ws_rc), 2))
    rows = np.array(rows, dtype=np.float64)
    out["head_recompute_backward"] = dict(
        seeds=f"0..{reps - 1}", mean_rows=float(rows.mean()),
        ms_per_call=float(np.mean(t_rc)) * 1e3,
        ms_per_call_with_stash=float(np.mean(t_plain)) * 1e3,
        algorithmic_tflops=float((4 * rows * HV).sum() / np.sum(t_rc) / 1e12),
        executed_tflops=float((6 * rows * HV).sum() / np.sum(t_rc) / 1e12),
        what="mdlm_fused_head_ce_fwd_bwd with a workspace one 256-column chunk short of "
             "the preferred size: the backward recomputes the logit tiles (6 M H V "
             "executed) instead of using the forward pass's stash")
    out["head_weight_gradient"] = dict(
        seeds=f"0..{reps - 1}", mean_rows=float(rows.mean()),
        ms_per_call=float(np.mean(t_dw)) * 1e3,
        ms_per_call_without_dw=float(np.mean(t_plain)) * 1e3,
        algorithmic_tflops=float((6 * rows * HV).sum() / np.sum(t_dw) / 1e12),
        dw_gemm_tflops=float((2 * rows * HV).sum() / (np.sum(t_dw) - np.sum(t_plain)) / 1e12),
        what="mdlm_fused_head_ce_fwd_bwd_dw (loss, d_hidden and dW fp32 [V, H]); the dW "
             "product's rate is 2 M H V over the time the call adds")
    # one GPU's share of a vocabulary-parallel head over 8 GPUs: the fused
    # call on the first V/8 rows of W, targets folded into the shard (the
    # all-reduces of the row statistics and of d_hidden that the sharded
    # head adds are not included)
    V8 = wl.V // 8
    W8 = W[:V8]
    ws8 = torch.empty(B.mdlm_head_ce_workspace_bytes(wl.n_tokens, wl.H, V8, B.MDLM_BF16),
                      dtype=torch.uint8, device=dev)
    t8, rows8 = [], []
    for seed in range(reps):
        step.corrupt(x0, cu, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab)
        step.compact(x0, cu, wl.align)
        rows8.append(int(step.n_rows.item()))
        tg8 = torch.remainder(step.tgt, V8)
        t8.append(_timed(lambda: B.mdlm_fused_head_ce_fwd_bwd(
            h, W8, step.row_idx, tg8, step.w, step.n_rows, wl.n_tokens, wl.softcap, loss, None,
            step.d_hidden, ws8), 2))
    rows8 = np.array(rows8, dtype=np.float64)
    out["head_vocab_shard_of_8"] = dict(
        V_shard=V8, seeds=f"0..{reps - 1}", mean_rows=float(rows8.mean()),
        ms_per_call=float(np.mean(t8)) * 1e3,
        algorithmic_tflops=float((4 * rows8 * wl.H * V8).sum() / np.sum(t8) / 1e12),
        what="mdlm_fused_head_ce_fwd_bwd on W[:V/8] (one GPU's share of a vocabulary-parallel "
             "head over 8 GPUs); the collectives of the sharded head are not included")
    del step, ws, dW, ws_rc, ws8
    if n_bw:
        L = 4096
        n = n_bw // L * L
        cu2 = torch.arange(0, n + 1, L, dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev).manual_seed(0)
        x2 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=dev, generator=g)
        s2 = MdlmLossStep(n, n // L, 64, 64, device=dev, head_workspace_bytes=0, want_grad=False)
        s2.corrupt(x2, cu2, 7, 1e-3, 1, 126336, 126464)
        res = {}
        for name, kw in (("causal_mean", dict(weighting=B.MDLM_WEIGHT_MEAN, corrupted=None)),
                         ("masked_example_mean_clipped",
                          dict(weighting=B.MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED, weight_clip=5.0))):
            t = _timed(lambda: s2.compact_rows(x2, cu2, 1, **kw), reps)
            mm = int(s2.n_rows.item())
            mask_bytes = 0 if kw.get("corrupted", True) is None else n
            alg = mask_bytes + 16.0 * mm
            res[name] = dict(us=t * 1e6, rows=mm, algorithmic_GBs=alg / t / 1e9,
                             frac=alg / t / 1e9 / PEAK_HBM_GBS)
        res["what"] = (f"mdlm_compact_rows at {n} tokens in documents of 4,096 (shifted); "
                       "algorithmic bytes: the mask (1 B per token, if any) + 16 B per row")
        out["compact_rows_hbm"] = res
        # the corrective mixture: corruption with a replaced share, then its row list
        mix = {}
        seeds = iter(range(1000, 2000))
        t = _timed(lambda: s2.corrupt_mixture(x2, cu2, next(seeds), 1e-3, 0.25, 126336,
                                              126464), reps)
        mix["corrupt_mixture"] = dict(us=t * 1e6, algorithmic_GBs=9.0 * n / t / 1e9,
                                      frac=9.0 * n / t / 1e9 / PEAK_HBM_GBS)
        for name, c in (("compact_corrective", 0.0), ("compact_corrective_clean", 0.1)):
            t = _timed(lambda: s2.compact_corrective(x2, cu2, 0, 0.5, c), reps)
            mm = int(s2.n_rows.item())
            alg = n + 16.0 * mm
            mix[name] = dict(us=t * 1e6, rows=mm, algorithmic_GBs=alg / t / 1e9,
                             frac=alg / t / 1e9 / PEAK_HBM_GBS)
        mix["what"] = (f"mdlm_corrupt_mixture (mixture_prob 0.25) and mdlm_compact_corrective "
                       f"(noise_token_wt 0.5, clean_token_wt 0 and 0.1) at {n} tokens in "
                       "documents of 4,096 (aligned); algorithmic bytes: corruption 9 B per "
                       "token, compaction the codes (1 B per token) + 16 B per row")
        out["corrective_mixture_hbm"] = mix
    return out


def other_workloads(dev, steps, warmup):
    """The other bf16 workloads, each timed like the default one (whole steps
    on one stream, Philox seed = step index): llada8b-varlen-12docs,
    nemotron3b-packed-16384 with aligned and shifted logits, and
    diffusiongemma-canvas-8x1024.  For each: ms per step (aggregate and
    median), tokens/s, and the fused call's 4 M H V rate against the bf16
    peak."""
    import torch
    import workloads as WL
    out = {}
    inp = None
    for k, align in ((3, None), (4, 0), (4, 1), (5, None)):
        wl = WL.make_workload(k)
        log(f"other workload {wl.name} (align {wl.align if align is None else align})")
        if inp is None or inp.wl.index != k:
            inp = None
            torch.cuda.empty_cache()
            inp = WL.generate(wl)
        a = argparse.Namespace(steps=steps, warmup=warmup, align=align)
        r = gpu_steps(a, inp, dev)
        rows = np.array(r["rows"], dtype=np.float64)
        head_s = np.array(r["head_ms"]) * 1e-3
        fl = 4.0 * rows * wl.H * wl.V
        tf = fl.sum() / head_s.sum() / 1e12
        name = wl.name + ("-shifted" if r["align"] == 1 and wl.align == 0 else "")
        out[name] = dict(
            n_tokens=wl.n_tokens, H=wl.H, V=wl.V, softcap=wl.softcap,
            noise="absorb" if wl.noise == 0 else "uniform",
            align="aligned" if r["align"] == 0 else "shifted", steps=steps,
            mean_scored_rows=float(rows.mean()), ms_per_step=r["total_ms"] / steps,
            median_ms_per_step=float(np.median(r["step_ms"])),
            tokens_per_s=wl.n_tokens * steps / (r["total_ms"] * 1e-3),
            head_ms_per_call=float(head_s.mean() * 1e3), head_tflops=float(tf),
            head_frac_of_bf16_peak=float(tf / PEAK_BF16_TFLOPS))
    del inp
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, seconds, align):
    """The fp64 oracle, as it stands, timed over whole steps of the workload:
    corruption, the row list and the head + CE forward and gradient over
    every scored row, for Philox seeds 0, 1, ... (the seeds of the timed GPU
    steps) until about `seconds` have been spent, at least one step.  The
    rate is the workload's tokens over the median step time."""
    import oracle
    wl = inp.wl
    steps = []
    spent = 0.0
    seed = 0
    while True:
        t0 = time.perf_counter()
        xt, corrupted, p, _ = oracle.corrupt(inp.x0, inp.cu_seqlens, seed, wl.eps, wl.noise,
                                             wl.mask_id, wl.rand_vocab)
        rows, tgt, w = oracle.compact(corrupted, inp.x0, inp.cu_seqlens, p, align)
        t1 = time.perf_counter()
        oracle.head_ce(inp.hidden, inp.W, rows, tgt, w, wl.softcap)
        t2 = time.perf_counter()
        steps.append(dict(seed=seed, rows=int(rows.shape[0]), corrupt_compact_s=t1 - t0,
                          head_s=t2 - t1, step_s=t2 - t0))
        spent += t2 - t0
        seed += 1
        if spent >= seconds or seed >= 20:
            break
    med = float(np.median([x["step_s"] for x in steps]))
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) or os.cpu_count()
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=wl.n_tokens / med, unit="tokens/s", cores=cores, kind="oracle",
                host_cpus=os.cpu_count(), cpu_model=cpu_model, seconds_per_step=med,
                steps=steps,
                sample=(f"{len(steps)} whole oracle steps of {wl.name} (Philox seeds "
                        f"0..{len(steps) - 1}): fp64 corruption, row list and head + CE "
                        f"forward and d_hidden over every scored row; rate = "
                        f"{wl.n_tokens} tokens / median step time ({spent:.1f} s in all; "
                        "corruption and the row list single-threaded numpy, the head's "
                        f"matrix products on {cores} BLAS threads)"))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library runs the loss path on a single "
              "MI355X and has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as WL
    from uniform_noise_diffusion_amd import binding
    binding.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    wl = WL.make_workload(args.workload)
    log(f"generating workload {wl.name}: N={wl.n_tokens} H={wl.H} V={wl.V}")
    inp = WL.generate(wl)
    if args.calibrate_copy:
        # one dispatch of the probe library's copy kernel over a known byte
        # count, for scaling counter runs
        from uniform_noise_diffusion_amd import probe
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        probe.copy(src, dst)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del src, dst
    log("timing steps")
    r = gpu_steps(args, inp, dev)
    K = args.steps
    rows = np.array(r["rows"], dtype=np.float64)
    head_s = np.array(r["head_ms"]) * 1e-3
    flops_alg = 4.0 * rows * wl.H * wl.V
    achieved = flops_alg.sum() / head_s.sum() / 1e12
    total_s = r["total_ms"] * 1e-3
    value = wl.n_tokens * K / total_s
    log(f"steps: {r['total_ms'] / K:.3f} ms/step, head+CE {head_s.mean() * 1e3:.3f} ms/call, "
        f"mean scored rows {rows.mean():.0f}, {achieved:.1f} TFLOP/s")
    # the counters' bytes belong to the workload they were taken on, and to
    # the kernels as they were then: they are reported only while the source
    # of the fused call's kernels is byte for byte the one they were counted on
    traffic, traffic_note = None, "no counter file"
    if args.traffic_json and os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            t = json.load(f)
        src = head_source_sha256()
        if t.get("workload") != wl.name:
            traffic_note = f"counted on {t.get('workload')}, not this workload"
        elif t.get("source_sha256") != src:
            traffic_note = (f"not reported: the kernels changed since the counters were taken "
                            f"(counted at {t.get('counted_at', '?')})")
        else:
            traffic = t.get("bytes_per_call")
            traffic_note = (f"FETCH_SIZE and WRITE_SIZE per call from {os.path.basename(args.traffic_json)}"
                            f", counted at {t.get('counted_at', '?')} on the same kernel source "
                            f"(sha256 {src[:12]})")
    bf16 = wl.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_VALU_TFLOPS
    roofline = dict(bound="mfma" if bf16 else "alu", achieved=achieved, peak=peak,
                    unit="TFLOP/s", frac=achieved / peak, traffic=traffic,
                    traffic_note=traffic_note, kernel="mdlm_fused_head_ce_fwd_bwd",
                    ms_per_call=float(head_s.mean() * 1e3),
                    algorithmic_flops_per_call=float(flops_alg.mean()))
    step_s = np.array(r["step_ms"]) * 1e-3
    per_seed = [dict(seed=i, rows=int(rows[i]), step_ms=float(step_s[i] * 1e3),
                     head_ms=float(head_s[i] * 1e3),
                     head_tflops=float(flops_alg[i] / head_s[i] / 1e12))
                for i in range(K)]
    med_step = float(np.median(step_s))
    out = dict(metric=METRIC, value=value, unit="tokens/s", n_gpus=1, steps=K,
               warmup=args.warmup, ms_per_step=r["total_ms"] / K, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16" if wl.dtype == "bf16" else "f32",
               data="synthetic",
               config=dict(workload=wl.name, global_batch=wl.n_docs, seq_len=wl.n_tokens,
                           H=wl.H, V=wl.V, noise="absorb" if wl.noise == 0 else "uniform",
                           align="aligned" if r["align"] == 0 else "shifted",
                           softcap=wl.softcap, eps=wl.eps, seeds=f"0..{K - 1}",
                           mean_scored_rows=float(rows.mean()), parallelism="none (1 GPU)"),
               roofline=roofline,
               median=dict(ms_per_step=med_step * 1e3, tokens_per_s=wl.n_tokens / med_step,
                           head_ms=float(np.median(head_s) * 1e3),
                           what=("median over the timed steps (each step's HIP events on the "
                                 "launch stream); `value` is the aggregate over all of them, "
                                 "the expectation over the noise draw")),
               per_seed=per_seed)
    if not args.no_achievable:
        log("measuring achievable peaks")
        ach = achievable(dev, (wl.V, wl.H, int(round(rows.mean()))))
        out["achievable"] = ach
        if bf16:
            roofline["frac_of_achievable"] = achieved / ach["mfma_bf16_tflops"]
    if args.bandwidth_tokens:
        log("timing corruption/compaction bandwidth")
        out["corrupt_compact_hbm"] = bandwidth(args.bandwidth_tokens, dev)
        out["corrupt_compact_hbm_lognormal296"] = bandwidth(args.bandwidth_tokens, dev,
                                                            doc_mean=296)
        if "achievable" in out:
            for k in ("corrupt_compact_hbm", "corrupt_compact_hbm_lognormal296"):
                for op in ("corrupt", "compact"):
                    out[k][f"{op}_frac_of_achievable_copy"] = (
                        out[k][f"{op}_GBs"] / out["achievable"]["copy_GBs"])
    if not args.no_other_workloads and args.workload == 2:
        out["other_workloads"] = other_workloads(dev, args.other_steps, 10)
    if not args.no_variants:
        log("timing the loss variants")
        out["variants"] = variants(inp, dev, args.bandwidth_tokens)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, r["align"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
