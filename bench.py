"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole path on synthetic, seeded inputs resident in HBM:
  * chunked prefill of a 128k-token sequence: B=1, H=32, T=131072, dk=dv=128, bf16 q/k/v
    (q, k unit-norm), fp32 per-channel log_alpha = -softplus(N(0,1)), fp32 beta =
    sigmoid(N(0,1)), zero initial state, chunk 64, output o and the final state;
  * one batched decode step: 256 sequences x 32 heads, fp32 128x128 states ~ N(0, 0.02),
    raw bf16 activations -> width-4 short conv with cache (q, k, v) -> decode step with
    in-kernel L2 normalisation of q and k.
`value` is prefill tokens/s; the decode state-update GB/s is reported beside it, and so are the
same 128k tokens prefilled as 32 packed prompts of seeded lengths (kda_chunk_prefill_varlen)
and with Gated DeltaNet's per-head gate (KDA_FLAG_SCALAR_GATE).
The training backward (kda_chunk_prefill_backward) is timed on the chunked-prefill training
shape (B=4, H=32, T=4096): fed with the chunk-end states that the training forward
(kda_chunk_prefill_states) saves, and as the self-contained call that runs the forward again,
with the plain forward on the same inputs beside them; the same tokens as 12 packed documents
(kda_chunk_prefill_varlen with 64-token checkpoints, then kda_chunk_prefill_varlen_backward);
and the training step with the per-head gate and with the q/k L2 norm.
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_BYTES_PER_TH = 1540          # q,k,v,o bf16 (4 x 256) + log_alpha fp32 (512) + beta (4)
PREFILL_GDN_BYTES_PER_TH = 1032      # the same with one gate per (token, head): log_alpha fp32 (4)
DECODE_BYTES_PER_SH = 132612         # state read+write 8*K*V + q,k,v,o (1024) + log_alpha (512) + beta
# backward per token-head: q, k, v, dO bf16 (4 x 256) + log_alpha (512) + beta (4) read;
# dq, dk, dv, dlog_alpha fp32 (4 x 512) + dbeta (4) written; with the chunk-end states
# handed in, those are read too (K x V fp32 per 64 tokens: 1024)
BACKWARD_BYTES_PER_TH = 1024 + 512 + 4 + 2048 + 4
BACKWARD_STATES_BYTES_PER_TH = BACKWARD_BYTES_PER_TH + 128 * 128 * 4 // 64


# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE on the default workload,
# scaled by a known-size streaming kernel in the same run (factors 2.0 and 1.0 on this GPU).  A
# figure is reported only while the kernel sources still hash to what was profiled.
MEASURED_TRAFFIC = {
    "prefill": {"sources": ("kda_prefill.hip", "kda_device.h"), "sha": "a4ab46f5ccfff747", "bytes": 16.389e9},
    "decode": {"sources": ("kda_decode.hip", "kda_device.h"), "sha": "7bca8c2b29273684", "bytes": 1.087e9},
    # the backward call with the chunk-end states given: bwd_prep, bwd_scan, bwd_cc, bwd_ck
    "backward": {"sources": ("kda_backward.hip", "kda_device.h"), "sha": "28d1e459b9f0f3e9", "bytes": 8.877e9},
}


# MFMA counters of the 128k prefill call (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
# SQ_INSTS_VALU_MFMA_MOPS_BF16 ...; busy % = busy cycles / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)),
# reported only while the kernel sources hash to what was profiled.
MEASURED_MFMA = {"sources": ("kda_prefill.hip", "kda_device.h"), "sha": "a4ab46f5ccfff747",
                 "prep_busy_pct": 8.1, "scan_busy_pct": 24.1, "call_busy_pct": 16.1, "issued_flop_per_call": 1.441e12}


def measured_mfma(default_workload):
    import hashlib
    h = hashlib.sha256()
    for name in MEASURED_MFMA["sources"]:
        with open(os.path.join(ROOT, "linear_attention_recurrence_kda_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if not (default_workload and h.hexdigest()[:16] == MEASURED_MFMA["sha"]):
        return None
    return {k: v for k, v in MEASURED_MFMA.items() if k not in ("sources", "sha")}


def measured_traffic(key, default_workload):
    import hashlib
    ent = MEASURED_TRAFFIC[key]
    h = hashlib.sha256()
    for name in ent["sources"]:
        with open(os.path.join(ROOT, "linear_attention_recurrence_kda_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return ent["bytes"] if default_workload and h.hexdigest()[:16] == ent["sha"] else None


def prefill_flops_per_th(C, K=128, V=128):
    # chunk WY form, triangles exploited: A, P, the solve on [V|K], P U, three state products
    return C * (3 * K + 2 * V) + 6 * K * V


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=131072)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--decode-batch", type=int, default=256)
    ap.add_argument("--flagged-steps", type=int, default=1,
                    help="also time the training step with the per-head gate and with the q/k L2 norm "
                         "(0 skips them, so that a profile's backward rows hold the default call only)")
    ap.add_argument("--long-T", type=int, default=524288,
                    help="tokens of the long single-sequence prefill timed beside the headline (0: skip)")
    ap.add_argument("--cpu-segment", type=int, default=8192,
                    help="tokens of the oracle's CPU-baseline segment (32 heads)")
    ap.add_argument("--cpu-repeats", type=int, default=16,
                    help="times the segment is chained through the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-B", type=int, default=4, help="batch of the backward timing (0: skip)")
    ap.add_argument("--bwd-T", type=int, default=4096, help="tokens per sequence of the backward timing")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size kernel "
                         "that scales the FETCH_SIZE/WRITE_SIZE counters of a profiling run)")
    return ap.parse_args()


def cpu_baseline(args):
    """The fp64 oracle, as it stands, on a bounded sample of the same prefill workload:
    one seeded 32-head segment chained `cpu_repeats` times with the state carried, on
    every host core (OpenMP over heads).  Inputs are converted to fp64 before timing."""
    import numpy as np
    from linear_attention_recurrence_kda_amd import datagen as D
    from oracle import oracle as O
    H, seg, reps = 32, args.cpu_segment, args.cpu_repeats
    inp = {n: np.ascontiguousarray(x, dtype=np.float64)
           for n, x in D.np_kda_inputs(1, seg, H, 128, 128, "bf16", seed=0).items()}
    threads = O.host_threads()
    O.c_prefill(**{n: x[:, :16] for n, x in inp.items()}, nthreads=threads)   # load the library
    state = None
    t0 = time.perf_counter()
    for _ in range(reps):
        _, state = O.c_prefill(**inp, init_state=state, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": seg * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"fp64 token loop, B=1 H=32 dk=dv=128: a {seg}-token segment chained "
                      f"{reps}x ({seg * reps} tokens), {dt:.1f} s wall"}


def cpu_backward_baseline(T=4096, heads=8):
    """The oracle's fp64 gradient (np_prefill_backward, a NumPy token loop on one core) on a
    bounded sample of the backward workload: `heads` heads of one T-token sequence, each run
    on its own (the oracle keeps every state of the sequence)."""
    import numpy as np
    from linear_attention_recurrence_kda_amd import datagen as D
    from oracle import oracle as O
    inp = D.np_kda_inputs(1, T, heads, 128, 128, "bf16", seed=0)
    do = np.random.default_rng(1).normal(0, 1, (1, T, heads, 128))
    t0 = time.perf_counter()
    for hh in range(heads):
        one = {n: np.ascontiguousarray(x[:, :, hh:hh + 1]) for n, x in inp.items()}
        O.np_prefill_backward(one["q"], one["k"], one["v"], one["log_alpha"], one["beta"], do[:, :, hh:hh + 1])
    dt = time.perf_counter() - t0
    return {"value": T * heads / 32 / dt, "unit": "tokens/s (32 heads)", "cores": 1, "kind": "oracle",
            "sample": f"fp64 reverse token loop (NumPy), B=1 T={T}, {heads} heads of dk=dv=128 one at a "
                      f"time, {dt:.1f} s wall; token-heads/s divided by 32"}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard over heads/sequences, see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from linear_attention_recurrence_kda_amd import datagen as D
    from linear_attention_recurrence_kda_amd import kda

    dev = torch.device("cuda:0")
    H, dk, dv, T, C = 32, 128, 128, args.T, args.chunk
    x = D.torch_kda_inputs(1, T, H, dk, dv, dev, "bf16", seed=0)
    o = torch.empty(1, T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.prefill_workspace_size(1, T, H, dk, dv, C, kda.KDA_BF16), dtype=torch.uint8, device=dev)

    Bd = args.decode_batch
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    state = 0.02 * torch.randn(Bd, H, dk, dv, device=dev, generator=g)
    dx = {n: torch.randn(Bd, 1, H * dk, device=dev, generator=g).to(torch.bfloat16) for n in ("q", "k", "v")}
    cw = {n: (torch.rand(H * dk, 4, device=dev, generator=g) - 0.5) for n in ("q", "k", "v")}
    cache = {n: torch.randn(Bd, 3, H * dk, device=dev, generator=g).to(torch.bfloat16) for n in ("q", "k", "v")}
    dla = -torch.nn.functional.softplus(torch.randn(Bd, H, dk, device=dev, generator=g))
    dbeta = torch.sigmoid(torch.randn(Bd, H, device=dev, generator=g))
    dy = {n: torch.empty_like(dx[n]) for n in dx}
    do = torch.empty(Bd, H, dv, dtype=torch.bfloat16, device=dev)

    def prefill():
        kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=C,
                          out=o, final_state=fs, workspace=ws)

    def decode():
        for n in ("q", "k", "v"):
            kda.short_conv(dx[n], cw[n], None, None, cache[n], out=dy[n])
        kda.decode_step(dy["q"].view(Bd, H, dk), dy["k"].view(Bd, H, dk), dy["v"].view(Bd, H, dv),
                        dla, dbeta, state, l2norm_qk=True, out=do)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        prefill()
        e[1].record()
        e[2].record()
        decode()
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sorted(a.elapsed_time(b) for a, b, _, _ in ev)
    dec_ms = sorted(c.elapsed_time(d) for _, _, c, d in ev)
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    # decode state update alone (the bandwidth-bound kernel): each launch bracketed by its
    # own events on the launch stream, so the figure is the kernel's duration
    reps = max(10, args.steps)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in dev_ev:
        a_.record()
        kda.decode_step(dy["q"].view(Bd, H, dk), dy["k"].view(Bd, H, dk), dy["v"].view(Bd, H, dv),
                        dla, dbeta, state, l2norm_qk=True, out=do)
        b_.record()
    torch.cuda.synchronize()
    dstep_ms = sum(a_.elapsed_time(b_) for a_, b_ in dev_ev) / reps

    # the same decode step fused into one launch (three convolutions at T = 1 with their
    # caches, the L2 norm and the state update): kda_decode_step_fused
    dxf = {n: dx[n].view(Bd, H * dk) for n in dx}
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in fev:
        a_.record()
        kda.decode_step_fused(dxf["q"], dxf["k"], dxf["v"], cw["q"], cw["k"], cw["v"], cache["q"],
                              cache["k"], cache["v"], dla, dbeta, state, H, l2norm_qk=True, out=do)
        b_.record()
    torch.cuda.synchronize()
    fused_ms = sum(a_.elapsed_time(b_) for a_, b_ in fev) / reps
    # and replayed from a graph: 8 fused steps captured once (a decode loop with no
    # per-launch host work), timed over whole replays
    def fused_step():
        kda.decode_step_fused(dxf["q"], dxf["k"], dxf["v"], cw["q"], cw["k"], cw["v"], cache["q"],
                              cache["k"], cache["v"], dla, dbeta, state, H, l2norm_qk=True, out=do)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(8):
            fused_step()
    graph.replay()
    torch.cuda.synchronize()
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a_, b_ in gev:
        a_.record()
        graph.replay()
        b_.record()
    torch.cuda.synchronize()
    graph_step_ms = sum(a_.elapsed_time(b_) for a_, b_ in gev) / (5 * 8)
    del graph

    # how the headline call scanned: the plan its segmented scan left at the end of the
    # workspace (segments per head by the library's rule; heads whose boundaries all had a
    # forgetting tail), and the same call as single chains (KDA_FLAG_SERIAL_SCAN) beside it
    G = 1
    while H * G < 64 and ((T + C - 1) // C) // (2 * G) >= 64:
        G *= 2
    seg_heads = 0
    if G > 1:
        plan = ws[ws.numel() - H * G * 4:].view(torch.int32).view(H, G).cpu()
        seg_heads = int((plan[:, 0] == 1).sum())

    def prefill_serial():
        kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=C,
                          out=o, final_state=fs, workspace=ws, serial_scan=True)
    prefill_serial()
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in sev:
        a_.record()
        prefill_serial()
        b_.record()
    torch.cuda.synchronize()
    serial_ms = sum(a_.elapsed_time(b_) for a_, b_ in sev) / reps
    scan_line = {"segments_per_head": G, "segmented_heads": seg_heads, "heads": H,
                 "single_chain_ms": serial_ms, "single_chain_tokens_per_s": T / (serial_ms * 1e-3)}

    # the same 128k tokens served as 32 prompts packed end to end (kda_chunk_prefill_varlen):
    # seeded cut points, so lengths vary from a few tokens to several thousand
    Nv = 32
    gcut = torch.Generator()
    gcut.manual_seed(2)
    cuts = torch.sort(torch.randperm(T - 1, generator=gcut)[:Nv - 1] + 1).values
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), cuts, torch.full((1,), T)]).to(torch.int32)
    lens = (cu[1:] - cu[:-1]).tolist()
    cu_d = cu.to(dev)
    xv = {n: t[0] for n, t in x.items()}
    fsv = torch.empty(Nv, H, dk, dv, dtype=torch.float32, device=dev)
    wsv = torch.empty(kda.prefill_varlen_workspace_size(Nv, T, H, dk, dv, C, kda.KDA_BF16), dtype=torch.uint8,
                      device=dev)

    def prefill_varlen():
        kda.chunk_prefill_varlen(xv["q"], xv["k"], xv["v"], xv["log_alpha"], xv["beta"], cu_d, chunk_size=C,
                                 out=o[0], final_state=fsv, workspace=wsv)
    prefill_varlen()
    vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in vev:
        a_.record()
        prefill_varlen()
        b_.record()
    torch.cuda.synchronize()
    varlen_ms = sum(a_.elapsed_time(b_) for a_, b_ in vev) / reps
    del wsv

    # Gated DeltaNet's per-head gate on the same tokens (kda_chunk_prefill with
    # KDA_FLAG_SCALAR_GATE): log_alpha [1, T, H], the first channel's gate
    la_h = x["log_alpha"][..., 0].contiguous()

    def prefill_gdn():
        kda.chunk_prefill(x["q"], x["k"], x["v"], la_h, x["beta"], chunk_size=C, out=o, final_state=fs,
                          workspace=ws, scalar_gate=True)
    prefill_gdn()
    gdn_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a_, b_ in gdn_ev:
        a_.record()
        prefill_gdn()
        b_.record()
    torch.cuda.synchronize()
    gdn_ms = sum(a_.elapsed_time(b_) for a_, b_ in gdn_ev) / reps
    del la_h

    # the long-context end of the pages' range: one 512k-token sequence, 32 heads, timed
    # after the headline workload (its inputs replace the 128k ones in HBM)
    long_line = None
    if args.long_T > 0:
        TL = args.long_T
        del x, o, ws, xv
        xl = D.torch_kda_inputs(1, TL, H, dk, dv, dev, "bf16", seed=3)
        ol = torch.empty(1, TL, H, dv, dtype=torch.bfloat16, device=dev)
        wsl = torch.empty(kda.prefill_workspace_size(1, TL, H, dk, dv, C, kda.KDA_BF16), dtype=torch.uint8,
                          device=dev)

        def prefill_long():
            kda.chunk_prefill(xl["q"], xl["k"], xl["v"], xl["log_alpha"], xl["beta"], chunk_size=C,
                              out=ol, final_state=fs, workspace=wsl)
        prefill_long()
        lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
        for a_, b_ in lev:
            a_.record()
            prefill_long()
            b_.record()
        torch.cuda.synchronize()
        long_ms = sum(a_.elapsed_time(b_) for a_, b_ in lev) / len(lev)
        long_gbs = PREFILL_BYTES_PER_TH * TL * H / (long_ms * 1e-3) / 1e9
        long_line = {"B": 1, "T": TL, "H": H, "ms": long_ms, "tokens_per_s": TL / (long_ms * 1e-3),
                     "algorithmic_GBps": long_gbs, "hbm_frac": long_gbs / HBM_PEAK_GBS}
        del xl, ol, wsl

    # the training backward on the chunked-prefill training shape: dq, dk, dv, dlog_alpha, dbeta
    # and dinit for L = <dO, o> + <dS_T, S_T>.  A training step runs the forward that saves the
    # chunk-end states, then the backward that takes them; the backward that runs the forward
    # again, and the plain forward, are timed beside it
    bwd_line = None
    if args.bwd_B > 0:
        Bb, Tb = args.bwd_B, args.bwd_T
        xb = D.torch_kda_inputs(Bb, Tb, H, dk, dv, dev, "bf16", seed=4)
        gb = torch.Generator(device=dev)
        gb.manual_seed(5)
        dob = torch.randn(Bb, Tb, H, dv, device=dev, generator=gb).to(torch.bfloat16)
        dfb = torch.randn(Bb, H, dk, dv, device=dev, generator=gb)
        fargs = (xb["q"], xb["k"], xb["v"], xb["log_alpha"], xb["beta"])
        bargs = fargs + (dob,)
        ob = torch.empty(Bb, Tb, H, dv, dtype=torch.bfloat16, device=dev)
        fsb = torch.empty(Bb, H, dk, dv, dtype=torch.float32, device=dev)
        ckb = torch.empty(Bb * (Tb // 64), H, dk, dv, dtype=torch.float32, device=dev)
        wfb = torch.empty(max(kda.prefill_workspace_size(Bb, Tb, H, dk, dv, c, kda.KDA_BF16) for c in (64, C)),
                          dtype=torch.uint8, device=dev)
        wsg = torch.empty(kda.backward_workspace_size(Bb, Tb, H, dk, dv, kda.KDA_BF16, states_given=True),
                          dtype=torch.uint8, device=dev)
        wsr = torch.empty(kda.backward_workspace_size(Bb, Tb, H, dk, dv, kda.KDA_BF16), dtype=torch.uint8,
                          device=dev)

        def forward_states():
            kda.chunk_prefill_states(*fargs, chunk_size=64, state_interval=64, chunk_states=ckb, out=ob,
                                     final_state=fsb, workspace=wfb)

        def backward():
            return kda.chunk_prefill_backward(*bargs, d_final_state=dfb, workspace=wsg, chunk_states=ckb)

        def backward_recompute():
            return kda.chunk_prefill_backward(*bargs, d_final_state=dfb, workspace=wsr)

        def forward():
            kda.chunk_prefill(*fargs, chunk_size=C, out=ob, final_state=fsb, workspace=wfb)

        def timed(fn, n=5):
            fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for a_, b_ in ev:
                a_.record()
                fn()
                b_.record()
            torch.cuda.synchronize()
            return sum(a_.elapsed_time(b_) for a_, b_ in ev) / n
        fst_ms = timed(forward_states)
        bwd_ms = timed(backward)                 # reads the states forward_states left in ckb
        rec_ms = timed(backward_recompute)
        fwd_ms = timed(forward)

        # the same tokens as 12 documents packed end to end (seeded cut points): the packed
        # training forward with 64-token checkpoints, then the packed backward fed with them
        NP = 12
        cuts = np.sort(np.random.default_rng(6).choice(np.arange(1, Bb * Tb), NP - 1, replace=False))
        cu_np = np.concatenate([[0], cuts, [Bb * Tb]]).astype(np.int32)
        plen = np.diff(cu_np)
        cup = torch.from_numpy(cu_np).to(dev)
        pk = tuple(x.view(Bb * Tb, *x.shape[2:]) for x in fargs)
        dop = dob.view(Bb * Tb, H, dv)
        dfp = torch.randn(NP, H, dk, dv, device=dev, generator=gb)
        ckp = torch.empty(int((plen // 64).sum()), H, dk, dv, dtype=torch.float32, device=dev)
        fsp = torch.empty(NP, H, dk, dv, dtype=torch.float32, device=dev)
        wfp = torch.empty(kda.prefill_varlen_workspace_size(NP, Bb * Tb, H, dk, dv, 64, kda.KDA_BF16),
                          dtype=torch.uint8, device=dev)
        wsp = torch.empty(kda.varlen_backward_workspace_size(NP, Bb * Tb, H, dk, dv, kda.KDA_BF16, states_given=True),
                          dtype=torch.uint8, device=dev)

        def forward_states_packed():
            kda.chunk_prefill_varlen(*pk, cup, chunk_size=64, state_interval=64, chunk_states=ckp,
                                     out=ob.view(Bb * Tb, H, dv), final_state=fsp, workspace=wfp)

        def backward_packed():
            return kda.chunk_prefill_varlen_backward(*pk, cup, dop, d_final_state=dfp, chunk_states=ckp,
                                                     workspace=wsp)
        pfst_ms = timed(forward_states_packed)
        pbwd_ms = timed(backward_packed)
        packed_line = {"documents": NP, "len_min": int(plen.min()), "len_max": int(plen.max()),
                       "forward_states_ms": pfst_ms, "ms": pbwd_ms, "training_step_ms": pfst_ms + pbwd_ms,
                       "training_step_tokens_per_s": Bb * Tb / ((pfst_ms + pbwd_ms) * 1e-3)}
        del ckp, fsp, wfp, wsp, dfp

        # the same training step with each forward flag: Gated DeltaNet's per-head gate
        # (log_alpha [B,T,H]) and the q/k L2 norm inside the calls (raw rows)
        def flagged_step(flags, la):
            args_f = (xb["q"], xb["k"], xb["v"], la, xb["beta"])
            wsf = torch.empty(kda.backward_workspace_size(Bb, Tb, H, dk, dv, kda.KDA_BF16, states_given=True,
                                                          **flags), dtype=torch.uint8, device=dev)

            def fwd():
                kda.chunk_prefill_states(*args_f, chunk_size=64, state_interval=64, chunk_states=ckb, out=ob,
                                         final_state=fsb, workspace=wfb, **flags)

            def bwd():
                return kda.chunk_prefill_backward(*args_f, dob, d_final_state=dfb, workspace=wsf, chunk_states=ckb,
                                                  **flags)
            f_ms, b_ms = timed(fwd), timed(bwd)
            return {"forward_states_ms": f_ms, "ms": b_ms, "training_step_ms": f_ms + b_ms,
                    "training_step_tokens_per_s": Bb * Tb / ((f_ms + b_ms) * 1e-3)}
        gate_line = l2_line = None
        if args.flagged_steps:
            gate_line = flagged_step({"scalar_gate": True}, xb["log_alpha"][..., 0].contiguous())
            l2_line = flagged_step({"l2norm_qk": True}, xb["log_alpha"])
        bth = Bb * Tb * H
        bwd_gbs = BACKWARD_STATES_BYTES_PER_TH * bth / (bwd_ms * 1e-3) / 1e9
        default_bwd = (Bb == 4 and Tb == 4096)    # the shape the measured traffic was taken on
        bwd_line = {"B": Bb, "T": Tb, "H": H, "dk": dk, "dv": dv, "dtype": "bf16",
                    "ms": bwd_ms, "tokens_per_s": Bb * Tb / (bwd_ms * 1e-3),
                    "forward_states_ms": fst_ms,
                    "training_step_ms": fst_ms + bwd_ms,
                    "training_step_tokens_per_s": Bb * Tb / ((fst_ms + bwd_ms) * 1e-3),
                    "ms_recompute": rec_ms,
                    "forward_ms_same_inputs": fwd_ms,
                    "backward_over_forward": bwd_ms / fwd_ms,
                    "packed": packed_line,
                    "per_head_gate": gate_line,
                    "l2norm_qk": l2_line,
                    "roofline": {"bound": "hbm", "achieved": bwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": bwd_gbs / HBM_PEAK_GBS,
                                 "traffic": measured_traffic("backward", default_bwd),
                                 "algorithmic_bytes": BACKWARD_STATES_BYTES_PER_TH * bth,
                                 "kernel": "kda_chunk_prefill_backward call with the chunk-end states given "
                                           "(bwd_prep, bwd_scan, bwd_cc, bwd_ck)"}}
        del xb, dob, dfb, ob, fsb, ckb, wfb, wsg, wsr

    # achievable streaming bandwidth on this GPU: a plain elementwise kernel over 1 GiB
    # (read 1 GiB, write 1 GiB), the reference point beside the nominal 8 TB/s
    cn = (1 << 30) // 4
    csrc = torch.ones(cn, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    torch.mul(csrc, 1.0, out=cdst)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a_, b_ in cev:
        a_.record()
        torch.mul(csrc, 1.0, out=cdst)
        b_.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * cn * 4 / (min(a_.elapsed_time(b_) for a_, b_ in cev) * 1e-3) / 1e9
    del csrc, cdst

    th = T * H
    default_wl = (T == 131072 and C == 64 and Bd == 256)
    pre_traffic = measured_traffic("prefill", default_wl)
    dec_traffic = measured_traffic("decode", default_wl)
    tok_s = T / (pre_avg * 1e-3)
    pre_gbs = PREFILL_BYTES_PER_TH * th / (pre_avg * 1e-3) / 1e9
    pre_tflops = prefill_flops_per_th(C) * th / (pre_avg * 1e-3) / 1e12
    dec_gbs = DECODE_BYTES_PER_SH * Bd * H / (dstep_ms * 1e-3) / 1e9

    line = {
        "metric": "KDA prefill tokens/s at 128k (MFMA %) + decode state-update GB/s (HBM %)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm bf16, log_alpha=-softplus(N(0,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": f"kda_prefill_T{T}_B1_H32_dk128_dv128_chunk{C} + kda_decode_B{Bd}_H32",
                   "prefill": {"B": 1, "T": T, "H": H, "dk": dk, "dv": dv, "chunk": C},
                   "decode": {"B": Bd, "H": H, "dk": dk, "dv": dv, "conv_width": 4}},
        "copy_GBps_measured": copy_gbs,
        "prefill": {"ms": pre_avg, "ms_min": pre_ms[0], "tokens_per_s": tok_s,
                    "algorithmic_GBps": pre_gbs, "hbm_frac": pre_gbs / HBM_PEAK_GBS,
                    "hbm_frac_of_copy": pre_gbs / copy_gbs,
                    "model_tflops": pre_tflops, "mfma_frac": pre_tflops / MFMA_BF16_PEAK_TFLOPS,
                    "mfma_counters": measured_mfma(default_wl),
                    "roofline_frac": max(pre_gbs / HBM_PEAK_GBS, pre_tflops / MFMA_BF16_PEAK_TFLOPS),
                    "scan": scan_line},
        "prefill_varlen": {"N": Nv, "T_total": T, "len_min": min(lens), "len_max": max(lens), "ms": varlen_ms,
                           "tokens_per_s": T / (varlen_ms * 1e-3),
                           "algorithmic_GBps": PREFILL_BYTES_PER_TH * th / (varlen_ms * 1e-3) / 1e9,
                           "hbm_frac": PREFILL_BYTES_PER_TH * th / (varlen_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "prefill_scalar_gate": {"ms": gdn_ms, "tokens_per_s": T / (gdn_ms * 1e-3),
                                "algorithmic_GBps": PREFILL_GDN_BYTES_PER_TH * th / (gdn_ms * 1e-3) / 1e9,
                                "hbm_frac": PREFILL_GDN_BYTES_PER_TH * th / (gdn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "prefill_long": long_line,
        "backward": bwd_line,
        "decode": {"step_ms_with_conv": dec_avg, "fused_step_ms": fused_ms, "fused_step_graph_ms": graph_step_ms,
                   "fused_tokens_per_s": Bd / (fused_ms * 1e-3), "state_update_ms": dstep_ms,
                   "state_update_GBps": dec_gbs, "hbm_frac": dec_gbs / HBM_PEAK_GBS,
                   "hbm_frac_of_copy": dec_gbs / copy_gbs,
                   "tokens_per_s": Bd / (dec_avg * 1e-3),
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_gbs / HBM_PEAK_GBS, "traffic": dec_traffic,
                                "algorithmic_bytes": DECODE_BYTES_PER_SH * Bd * H,
                                "kernel": "decode_step_kernel"}},
        "roofline": {"bound": "hbm", "achieved": pre_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pre_gbs / HBM_PEAK_GBS, "traffic": pre_traffic,
                     "algorithmic_bytes": PREFILL_BYTES_PER_TH * th,
                     "kernel": "kda_chunk_prefill call (prep_kernel, seg_plan_kernel, scan_kernel passes 2 and 0)"},
    }
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)          # a streaming kernel (copy_ would be a DMA memcpy)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = {"read": n * 4, "write": n * 4}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args)
        if bwd_line is not None:
            bwd_line["cpu_baseline"] = cpu_backward_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
