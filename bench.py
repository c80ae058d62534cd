#!/usr/bin/env python3
"""Benchmark of the KDA forward on one MI355X.

A step is one chunkwise prefill (kda_chunk_fwd) of the headline workload
B=8, H=32, T=8192, d_k=d_v=128, bf16 q/k/v/o, fp32 gates and state, chunk 64,
S0 = NULL (65,536 tokens), with inputs already resident in HBM.  `value` is
prefill tokens/s (B*T per step).  The same run also measures the decode
workload (256 sequences x 32 heads, fp32 state of 512 MiB, 128 chained
kda_decode_step calls) and reports its steps/s, and the multi-token decode
workload (the same states, 256 sequences of U{1..8} new tokens, one
kda_recurrent_fwd_varlen call updating them in place) and the Gated DeltaNet
prefill (the headline shapes with one gate per token and head,
kda_gdn_chunk_fwd), the prefill of raw layer inputs with the in-kernel
input transforms (q/k L2 norm, beta sigmoid, the -5 sigmoid gate), and the
backward (kda_backward: every input gradient) of the headline prefill.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, published

PREFILL = dict(B=8, T=8192, H=32, dk=128, dv=128, io="bf16", chunk=64)
DECODE = dict(N=256, H=32, dk=128, dv=128, io="bf16", steps=128)
# multi-token decode: 256 sequences of U{1..8} tokens (seed 0) on resident states
RECURRENT = dict(n_seq=256, lo=1, hi=8, H=32, dk=128, dv=128, io="bf16", calls=20)
BACKWARD_CALLS = 5


def backward_alg_flops(B, T, H, dk, dv):
    """fp32 flops per head-token of the recurrence's backward, per state
    element: the forward's decay, predict and write (1 + 2 + 2) and the
    backward's read (dS += q do^T, dq: 2 + 2), de (2), dk (two terms, 4),
    dSbar (2), dg (2) and the decay of dS (1): 20 d_k d_v."""
    return B * T * H * 20 * dk * dv


def backward_alg_bytes(B, T, H, dk, dv, io):
    """q, k, v, d_out in the I/O type, log_alpha and beta in fp32 read once;
    dq, dk, dv, dlog_alpha and dbeta in fp32 written once."""
    e = 2 if io == "bf16" else 4
    return B * T * H * (e * (2 * dk + 2 * dv) + 4 * dk + 4 + 4 * (3 * dk + dv) + 4)


def prefill_alg_bytes(B, T, H, dk, dv, io, with_S0=False, with_S_final=True, gate_dims=None):
    """Inputs read once and outputs written once: q, k (dk), v, o (dv) in the
    I/O type, log_alpha (dk per token and head, or 1 for Gated DeltaNet) and
    beta in fp32, plus the fp32 states."""
    e = 2 if io == "bf16" else 4
    per_ht = e * (2 * dk + 2 * dv) + 4 * (dk if gate_dims is None else gate_dims) + 4
    states = B * H * dk * dv * 4 * (int(with_S0) + int(with_S_final))
    return B * T * H * per_ht + states


def prefill_alg_flops(B, T, H, dk, dv, C=64):
    """Chunkwise method per head-token: 6 dk dv + 2C(3dk + 2dv) + C^2/3."""
    return B * T * H * (6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles",
                            "traffic_chunk_kda_gdn_b8_h32_t8192_decode_recurrent_n256_h32.md")
CSRC = os.path.join(HERE, "gated_delta_rule_06_amd", "csrc")


BWD_TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_backward_b8_h32_t8192.md")


def measured_traffic(kernel="chunk", source="chunk.hip", path=TRAFFIC_FILE):
    """HBM bytes per launch of one kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when the
    kernel's source has changed since the counters were taken."""
    import hashlib
    try:
        txt = open(path).read()
        src = hashlib.sha256(open(os.path.join(CSRC, source), "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in txt.splitlines() if ":" in l and not l.startswith("#"))
    fields = {k.strip("- `*").strip(): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("%s_source_sha256" % kernel) != src:
        return None
    try:
        return float(fields["%s_traffic_bytes_per_launch" % kernel])
    except (KeyError, ValueError):
        return None


def decode_alg_bytes(N, H, dk, dv, io):
    e = 2 if io == "bf16" else 4
    return N * H * (2 * dk * dv * 4 + e * (2 * dk + 2 * dv) + 4 * dk + 4)


def recurrent_alg_bytes(tokens, n_seq, H, dk, dv, io):
    """Every state read and written once, every token's inputs read and its
    output written once."""
    e = 2 if io == "bf16" else 4
    return n_seq * H * dk * dv * 4 * 2 + tokens * H * ((2 * dk + 2 * dv) * e + dk * 4 + 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chains", type=int, default=160,
                    help="chains of the prefill workload the oracle runs for the CPU baseline")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the KDA library runs on a single MI355X, "
               "and no multi-GPU path exists; got --gpus %d, WORLD_SIZE %d" % (args.gpus, world))
        print(msg, file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_06_amd import inputs, kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)   # the stream the binding launches on
    P = PREFILL
    log("generating prefill inputs", P)
    d = inputs.prefill_inputs(P["B"], P["T"], P["H"], P["dk"], P["dv"], io=P["io"], seed=0,
                              with_S0=False, device=dev)
    out = torch.empty((P["B"], P["T"], P["H"], P["dv"]), dtype=torch.bfloat16, device=dev)
    Sf = torch.empty((P["B"], P["H"], P["dk"], P["dv"]), dtype=torch.float32, device=dev)
    # the call's workspace, allocated once as a serving loop would (256 chains
    # on 256 CUs take one workgroup per chain; it is not read on this shape)
    ws_pf = torch.empty(kda.chunk_fwd_workspace_size(P["B"], P["T"], P["H"], P["dk"], P["dv"]),
                        dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=None, out=out, S_final=Sf,
                      workspace=ws_pf)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy of %d MiB done" % args.calib_copy_mib)
        del a, b

    # ---------------------------------------------------------------- decode
    D = DECODE
    log("generating decode inputs", D)
    dd = inputs.decode_inputs(D["N"], D["H"], D["dk"], D["dv"], D["steps"], io=D["io"], seed=0,
                              device=dev)
    S = dd["S"]
    o_dec = torch.empty((D["N"], D["H"], D["dv"]), dtype=torch.bfloat16, device=dev)

    def decode_run():
        for t in range(D["steps"]):
            kda.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["g"][t], dd["beta"][t], S,
                            out=o_dec)

    decode_run()   # warm-up run
    torch.cuda.synchronize()
    # The 128 steps as one HIP graph (the serving loop's launch path): captured
    # once, then checked bit for bit against the same steps run eagerly from
    # the same state, then timed by replays (HIP events around each replay).
    S_init = S.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_run()
    torch.cuda.synchronize()
    S.copy_(S_init)
    decode_run()
    torch.cuda.synchronize()
    S_eager, o_eager = S.clone(), o_dec.clone()
    S.copy_(S_init)
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(S, S_eager) and torch.equal(o_dec, o_eager)):
        raise RuntimeError("decode graph replay differs from the eager steps")
    del S_eager, o_eager, S_init
    graph.replay()   # one more untimed replay
    torch.cuda.synchronize()
    dk_ms = []
    dec_walls = []
    for _ in range(args.decode_reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        dec_walls.append(time.perf_counter() - t0)
        dk_ms.append(a.elapsed_time(b) / D["steps"])
    dec_wall = float(np.median(dec_walls))
    dec_steps_s = D["steps"] / dec_wall
    dec_kernel_ms = float(np.mean(dk_ms))
    dec_b = decode_alg_bytes(D["N"], D["H"], D["dk"], D["dv"], D["io"])
    dec_gbs = dec_b / (dec_kernel_ms * 1e-3) / 1e9
    log("decode: %.1f steps/s (wall, 128 steps per graph replay), %.2f us per step, %.0f GB/s"
        % (dec_steps_s, dec_kernel_ms * 1e3, dec_gbs))
    del dd, S, graph
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- multi-token decode
    R = RECURRENT
    lens = inputs.varlen_lengths(R["n_seq"], R["lo"], R["hi"], seed=0)
    log("generating multi-token decode inputs", R, "tokens", int(lens.sum()))
    dr = inputs.varlen_inputs(lens, R["H"], R["dk"], R["dv"], io=R["io"], seed=0, with_S0=True,
                              device=dev)
    Sr = dr["S0"]
    o_rec = torch.empty((dr["T_total"], R["H"], R["dv"]), dtype=torch.bfloat16, device=dev)

    def rec_call():
        kda.recurrent_fwd_varlen(dr["q"], dr["k"], dr["v"], dr["g"], dr["beta"], dr["cu_seqlens"],
                                 S0=Sr, S_final=Sr, out=o_rec)

    for _ in range(5):
        rec_call()
    torch.cuda.synchronize()
    evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(R["calls"])]
    t0 = time.perf_counter()
    for a, b in evr:
        a.record(stream)
        rec_call()
        b.record(stream)
    torch.cuda.synchronize()
    rec_wall = (time.perf_counter() - t0) / R["calls"]
    rec_ms = float(np.mean([a.elapsed_time(b) for a, b in evr]))
    rec_b = recurrent_alg_bytes(int(lens.sum()), R["n_seq"], R["H"], R["dk"], R["dv"], R["io"])
    rec_gbs = rec_b / (rec_ms * 1e-3) / 1e9
    log("multi-token decode: %.2f us/call (wall), kernel %.2f us avg, %.0f GB/s"
        % (rec_wall * 1e6, rec_ms * 1e3, rec_gbs))
    rec_tokens = int(lens.sum())
    del dr, Sr, o_rec
    torch.cuda.empty_cache()

    # gates of the fast-forgetting leg (drawn now, away from the timed legs)
    strong = {"g": d["g"].clone()}
    inputs.strong_gate_channels(strong, 8, -5.0, -2.0, seed=0)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- Gated DeltaNet prefill
    log("generating Gated DeltaNet prefill inputs (one gate per token and head)")
    dg = inputs.prefill_inputs(P["B"], P["T"], P["H"], P["dk"], P["dv"], io=P["io"], seed=0,
                               with_S0=False, device=dev, gate="gdn")

    def gdn_step():
        kda.chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], S0=None, out=out, S_final=Sf,
                      workspace=ws_pf)

    for _ in range(args.warmup):
        gdn_step()
    torch.cuda.synchronize()
    evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evg:
        a.record(stream)
        gdn_step()
        b.record(stream)
    torch.cuda.synchronize()
    gdn_wall = (time.perf_counter() - t0) / args.steps
    tokens = P["B"] * P["T"]
    gdn_ms = float(np.mean([a.elapsed_time(b) for a, b in evg]))
    gdn_b = prefill_alg_bytes(P["B"], P["T"], P["H"], P["dk"], P["dv"], P["io"], gate_dims=1)
    gdn_gbs = gdn_b / (gdn_ms * 1e-3) / 1e9
    log("gdn prefill: %.3f ms/step (wall), kernel %.3f ms avg, %.3e tokens/s, %.0f GB/s"
        % (gdn_wall * 1e3, gdn_ms, tokens / gdn_wall, gdn_gbs))

    # ---------------------------------------------------------------- headline prefill
    # Timed right after the Gated DeltaNet prefill (the same kernel family,
    # about 17 ms of back-to-back launches): at the start of a burst after
    # idle the engine clock drops to about 1.7 GHz and recovers to about
    # 2.2 GHz over some 25 launches of this kernel, while the kernel's cycle
    # count per launch stays the same (GRBM_GUI_ACTIVE per dispatch,
    # profiles/).  The launch times of the warm-up and timed steps are printed
    # to stderr.
    warm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.warmup)]
    for a, b in warm_ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = 1e3 * wall / args.steps
    avg_kernel_ms = float(np.mean(kern_ms))
    tokens = P["B"] * P["T"]
    value = tokens / (wall / args.steps)
    alg_b = prefill_alg_bytes(P["B"], P["T"], P["H"], P["dk"], P["dv"], P["io"])
    alg_f = prefill_alg_flops(P["B"], P["T"], P["H"], P["dk"], P["dv"])
    achieved = alg_b / (avg_kernel_ms * 1e-3) / 1e9
    log("prefill: %.3f ms/step (wall), kernel %.3f ms avg (min %.3f), %.3e tokens/s, %.0f GB/s"
        % (ms_per_step, avg_kernel_ms, min(kern_ms), value, achieved))
    log("prefill launch ms, warm-up:", " ".join("%.3f" % a.elapsed_time(b) for a, b in warm_ev))
    log("prefill launch ms, timed:", " ".join("%.3f" % x for x in kern_ms))

    # ---------------------------------------------------------------- fast-forgetting channels
    # The same workload with 8 of the 128 key channels of every head redrawn
    # at log alpha ~ U[-5, -2] per token (up to e^-320 over a chunk); the
    # gates were drawn before the headline, so the two legs run back to back.
    def strong_step():
        kda.chunk_fwd(d["q"], d["k"], d["v"], strong["g"], d["beta"], S0=None, out=out,
                      S_final=Sf, workspace=ws_pf)

    # A longer warm-up than the headline's, in one burst with the timed
    # launches: a few launches after an idle gap the engine clock dips under
    # this heavier load (launch times rise by up to 40% and recover over some
    # 20 launches, while the cycles per launch stay 1.06x the plain kernel's),
    # so the leg runs 30 untimed launches and then the timed ones with no
    # synchronisation in between, and averages the timed ones only.
    n_warm_s = max(args.warmup, 30)
    evs_s = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_warm_s + args.steps)]
    for a, b in evs_s:
        a.record(stream)
        strong_step()
        b.record(stream)
    torch.cuda.synchronize()
    sg_all = [a.elapsed_time(b) for a, b in evs_s]
    sg_launch = sg_all[n_warm_s:]
    sg_ms = float(np.mean(sg_launch))
    log("prefill, 8 of 128 channels at log alpha ~ U[-5,-2]: kernel %.3f ms avg (%.3f x the "
        "plain inputs)" % (sg_ms, sg_ms / avg_kernel_ms))
    log("fast-forgetting launch ms, warm-up:", " ".join("%.3f" % x for x in sg_all[:n_warm_s]))
    log("fast-forgetting launch ms, timed:", " ".join("%.3f" % x for x in sg_launch))
    del strong
    del d, dg
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- fused input transforms
    log("generating raw layer inputs for the in-kernel transforms")
    dr0 = inputs.prefill_inputs(P["B"], P["T"], P["H"], P["dk"], P["dv"], io=P["io"], seed=0,
                                with_S0=False, device=dev)
    dr0 = inputs.raw_layer_inputs(dr0, P["H"], P["dk"], seed=0, device=dev, gate_mu=-6.0)

    def fused_step():
        kda.chunk_fwd(dr0["q"], dr0["k"], dr0["v"], dr0["g"], dr0["beta"], S0=None, out=out,
                      S_final=Sf, qk_l2norm=True, beta_sigmoid=True, A_log=dr0["A_log"],
                      gate_bias=dr0["gate_bias"], workspace=ws_pf)

    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evf:
        a.record(stream)
        fused_step()
        b.record(stream)
    torch.cuda.synchronize()
    fu_wall = (time.perf_counter() - t0) / args.steps
    fu_ms = float(np.mean([a.elapsed_time(b) for a, b in evf]))
    fu_b = alg_b + P["H"] * 4 + P["H"] * P["dk"] * 4          # plus A_log and the gate bias
    fu_gbs = fu_b / (fu_ms * 1e-3) / 1e9
    log("fused prefill: %.3f ms/step (wall), kernel %.3f ms avg, %.3e tokens/s, %.0f GB/s"
        % (fu_wall * 1e3, fu_ms, tokens / fu_wall, fu_gbs))
    del dr0
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the other prefill configs
    def timed_calls(fn, n, warm=5):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    c2 = inputs.CONFIGS["prefill_h16_s0"]
    log("generating the B1 H16 T4096 prefill with S0")
    d2 = inputs.prefill_inputs(c2["B"], c2["T"], c2["H"], c2["dk"], c2["dv"], io=c2["io"], seed=0,
                               with_S0=True, device=dev)
    c2_ms = timed_calls(lambda: kda.chunk_fwd(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"],
                                              S0=d2["S0"]), 20)
    c2_b = prefill_alg_bytes(c2["B"], c2["T"], c2["H"], c2["dk"], c2["dv"], c2["io"], with_S0=True)
    c2_chunks = c2["T"] // 64
    log("prefill B1 H16 T4096 + S0: %.1f us per launch (%d chains of %d chunks on %d CUs)"
        % (c2_ms * 1e3, c2["B"] * c2["H"], c2_chunks, 256))
    del d2
    c5 = inputs.CONFIGS["varlen_16seq_h32"]
    lens5 = inputs.varlen_lengths(c5["n_seq"], c5["lo"], c5["hi"], seed=0)
    log("generating the 16-sequence packed prefill (%d tokens)" % int(lens5.sum()))
    d5 = inputs.varlen_inputs(lens5, c5["H"], c5["dk"], c5["dv"], io=c5["io"], seed=0,
                              long_channels=c5["long_channels"], device=dev)
    c5_tokens = int(lens5.sum())
    ws5 = torch.empty(kda.lib.kda_chunk_fwd_varlen_workspace_size(
        c5["n_seq"], c5_tokens, c5["H"], c5["dk"], c5["dv"], 64, 1), dtype=torch.uint8, device=dev)
    c5_ms = timed_calls(lambda: kda.chunk_fwd_varlen(d5["q"], d5["k"], d5["v"], d5["g"], d5["beta"],
                                                     d5["cu_seqlens"], workspace=ws5), 5, warm=2)
    # the balanced schedule's plan, as the kernels left it in the workspace:
    # workgroups launched, slice length and total in chunks
    w5 = ws5[:24].cpu().numpy()
    c5_wg = int(w5[:4].view(np.uint32)[0])
    c5_slice, c5_total = (int(x) for x in w5[8:24].view(np.int64))
    # the same call with one workgroup per (sequence, head) chain, for comparison
    c5_chain_ms = timed_calls(lambda: kda.chunk_fwd_varlen(
        d5["q"], d5["k"], d5["v"], d5["g"], d5["beta"], d5["cu_seqlens"], balanced=False), 5,
        warm=2)
    c5_b = c5_tokens * c5["H"] * 1540 + c5["n_seq"] * c5["H"] * c5["dk"] * c5["dv"] * 4
    c5_longest = int(-(-int(lens5.max()) // 64))
    log("varlen 16 sequences: %.2f ms per launch, %.0f GB/s (%d workgroups, slices of %d of %d "
        "chunks; longest chain %d); one workgroup per chain: %.2f ms"
        % (c5_ms, c5_b / (c5_ms * 1e-3) / 1e9, c5_wg, c5_slice, c5_total, c5_longest,
           c5_chain_ms))
    del d5, ws5
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- backward
    log("generating backward inputs (the prefill workload plus dL/dout)")
    dbw = inputs.prefill_inputs(P["B"], P["T"], P["H"], P["dk"], P["dv"], io=P["io"], seed=0,
                                with_S0=False, device=dev)
    inputs.grad_inputs(dbw, seed=0, with_dS_final=False, device=dev)
    ws_bw = torch.empty(kda.backward_workspace_size(P["B"], P["T"], P["H"], P["dk"], P["dv"]),
                        dtype=torch.uint8, device=dev)

    def bwd_call():
        kda.backward(dbw["q"], dbw["k"], dbw["v"], dbw["g"], dbw["beta"], dbw["d_out"],
                     want_dS0=False, workspace=ws_bw)

    # the engine clock is still climbing over the first few calls of a burst
    # after the lighter legs before it (launch times fall by some 10% over six)
    bw_ms = timed_calls(bwd_call, BACKWARD_CALLS, warm=6)
    bw_f = backward_alg_flops(P["B"], P["T"], P["H"], P["dk"], P["dv"])
    bw_b = backward_alg_bytes(P["B"], P["T"], P["H"], P["dk"], P["dv"], P["io"])
    bw_tf = bw_f / (bw_ms * 1e-3) / 1e12
    bw_gbs = bw_b / (bw_ms * 1e-3) / 1e9
    log("backward: %.2f ms per call, %.0f GB/s algorithmic (%.1f%% of HBM), %.1f TFLOP/s of the "
        "recurrence's fp32 flops" % (bw_ms, bw_gbs, 100 * bw_gbs / HBM_PEAK_GBS, bw_tf))
    bw_ws_gb = ws_bw.numel() / 1e9
    del dbw, ws_bw
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        from gated_delta_rule_06_amd.inputs import to_host
        d = inputs.prefill_inputs(P["B"], P["T"], P["H"], P["dk"], P["dv"], io=P["io"], seed=0,
                                  with_S0=False, device=dev)
        step_out, step_S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
        torch.cuda.synchronize()
        n = max(1, min(args.cpu_chains, P["B"] * P["H"]))
        rng = np.random.default_rng(1)
        ids = sorted(rng.choice(P["B"] * P["H"], size=n, replace=False).tolist())
        # gather the sampled chains as a [n, T, 1, d] batch
        sel = lambda t: np.stack([to_host(t[c // P["H"], :, c % P["H"]].contiguous())
                                  for c in ids])[:, :, None]
        q, k, v, g = sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["g"])
        beta = np.stack([to_host(d["beta"][c // P["H"], :, c % P["H"]].contiguous())
                         for c in ids])[:, :, None]
        # the host cores this process may use, capped at the CPU share a
        # one-GPU job gets (OMP_NUM_THREADS is set to it on the GPU hosts)
        affinity = oracle.default_threads()
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or affinity
        threads = max(1, min(affinity, share))
        log("oracle: %d chains x %d tokens on %d threads" % (n, P["T"], threads))
        t0 = time.perf_counter()
        outs, Sref = oracle.forward(q, k, v, g, beta, threads=threads)
        cpu_wall = time.perf_counter() - t0
        head_tokens = n * P["T"]
        cpu = {"value": head_tokens / P["H"] / cpu_wall, "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": "%d of the %d (sequence, head) chains of the B8 H32 T8192 d128 workload "
                         "(%d head-tokens, fp64 sequential recurrence); tokens/s counts a token "
                         "as all %d heads, i.e. head-tokens/s / %d; wall %.2f s; %d threads "
                         "(host affinity %d cores, OMP_NUM_THREADS %s)"
                         % (n, P["B"] * P["H"], head_tokens, P["H"], P["H"], cpu_wall, threads,
                            affinity, os.environ.get("OMP_NUM_THREADS", "unset"))}
        go = np.stack([step_out[c // P["H"], :, c % P["H"]].float().cpu().numpy() for c in ids])
        gs = np.stack([step_S[c // P["H"], c % P["H"]].cpu().numpy() for c in ids])
        ro = np.stack(outs)
        rel = lambda a, b: float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))
        parity = {"chains": n, "rel_l2_o": rel(go, ro), "rel_l2_S": rel(gs, Sref)}
        log("oracle %.2f s -> %.3e tokens/s; parity %s" % (cpu_wall, cpu["value"], parity))

    rec = {
        "metric": "KDA prefill tokens/s (B8 H32 T8192 d128) + decode steps/s, % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: L2-normalised Gaussian q/k, Gaussian v, "
                "log_alpha=-exp(N(-3,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "prefill_b8_h32_t8192", "B": P["B"], "T": P["T"], "H": P["H"],
                   "d_k": P["dk"], "d_v": P["dv"], "chunk": P["chunk"], "io": "bf16",
                   "state": "fp32", "S0": None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("chunk", "chunk.hip"),
                     "kernel": "chunk_fwd_kernel<128,128,bf16>",
                     "alg_bytes_per_launch": alg_b, "avg_launch_ms": avg_kernel_ms,
                     "alg_tflops": alg_f / (avg_kernel_ms * 1e-3) / 1e12,
                     "mfma_frac": alg_f / (avg_kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "decode": {"workload": "decode_n256_h32", "launch": "one HIP graph of the 128 steps",
                   "steps_per_s": dec_steps_s,
                   "tokens_per_s": dec_steps_s * D["N"], "ms_per_step": 1e3 / dec_steps_s,
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "traffic": measured_traffic("decode", "decode.hip"),
                                "alg_bytes_per_launch": dec_b,
                                "avg_launch_ms": dec_kernel_ms}},
        "strong_gate_prefill": {"workload": "prefill_b8_h32_t8192, 8 of 128 key channels per "
                                            "head at log_alpha ~ U[-5,-2]",
                                "warmup": max(args.warmup, 30),
                                "avg_launch_ms": sg_ms, "vs_plain": sg_ms / avg_kernel_ms,
                                "tokens_per_s": tokens / (sg_ms * 1e-3)},
        "gdn_prefill": {"workload": "gated_deltanet_prefill_b8_h32_t8192",
                        "tokens_per_s": tokens / gdn_wall, "ms_per_step": gdn_wall * 1e3,
                        "roofline": {"bound": "hbm", "achieved": gdn_gbs, "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": gdn_gbs / HBM_PEAK_GBS,
                                     "traffic": measured_traffic("gdn", "chunk.hip"),
                                     "kernel": "chunk_fwd_kernel<128,128,bf16,scalar gate>",
                                     "alg_bytes_per_launch": gdn_b, "avg_launch_ms": gdn_ms}},
        "fused_prefill": {"workload": "prefill_b8_h32_t8192_raw_inputs_in_kernel_transforms",
                          "transforms": "q/k L2 norm, beta sigmoid, -5 sigmoid gate",
                          "tokens_per_s": tokens / fu_wall, "ms_per_step": fu_wall * 1e3,
                          "roofline": {"bound": "hbm", "achieved": fu_gbs, "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": fu_gbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic("fused", "chunk.hip"),
                                       "kernel": "chunk_fwd_kernel<128,128,bf16,transforms>",
                                       "alg_bytes_per_launch": fu_b, "avg_launch_ms": fu_ms}},
        "prefill_h16_t4096_s0": {
            "workload": "prefill_b1_h16_t4096_with_S0", "avg_launch_ms": c2_ms,
            "tokens_per_s": c2["B"] * c2["T"] / (c2_ms * 1e-3),
            "achieved_gbs": c2_b / (c2_ms * 1e-3) / 1e9, "alg_bytes_per_launch": c2_b,
            "bound": "latency: 16 chains of %d serial chunks on 256 CUs" % c2_chunks,
            "us_per_chunk_step": c2_ms * 1e3 / c2_chunks},
        "varlen_16seq_h32": {
            "workload": "varlen_16_sequences_U1024_65536_h32", "tokens": c5_tokens,
            "avg_launch_ms": c5_ms, "tokens_per_s": c5_tokens / (c5_ms * 1e-3),
            "achieved_gbs": c5_b / (c5_ms * 1e-3) / 1e9, "alg_bytes_per_launch": c5_b,
            "frac_hbm": c5_b / (c5_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "longest_chain_chunks": c5_longest,
            "schedule": "balanced: %d workgroups, %d chunks laid end to end per head and cut "
                        "into slices of %d" % (c5_wg, c5_total, c5_slice),
            "us_per_slice_chunk": c5_ms * 1e3 / c5_slice,
            "traffic": measured_traffic("varlen", "chunk.hip"),
            "one_workgroup_per_chain_ms": c5_chain_ms},
        "recurrent": {"workload": "multi_token_decode_n256_h32_len1to8",
                      "tokens_per_call": rec_tokens, "calls": R["calls"],
                      "us_per_call": rec_wall * 1e6, "tokens_per_s": rec_tokens / rec_wall,
                      "roofline": {"bound": "hbm", "achieved": rec_gbs, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": rec_gbs / HBM_PEAK_GBS,
                                   "traffic": measured_traffic("recurrent", "recurrent.hip"),
                                   "kernel": "recurrent_fwd_kernel<128,128,bf16>",
                                   "alg_bytes_per_launch": rec_b, "avg_launch_ms": rec_ms}},
        "backward": {"workload": "backward_b8_h32_t8192 (dq, dk, dv, dlog_alpha, dbeta)",
                     "avg_launch_ms": bw_ms, "tokens_per_s": tokens / (bw_ms * 1e-3),
                     "workspace_gb": bw_ws_gb,
                     "roofline": {"bound": "hbm", "achieved": bw_gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": bw_gbs / HBM_PEAK_GBS,
                                  "traffic": measured_traffic("backward", "backward_chunk.hip",
                                                              BWD_TRAFFIC_FILE),
                                  "kernel": "bwd_chunk_kernel<KDA> (chunkwise, MFMA, bf16 I/O)",
                                  "alg_flops_per_launch": bw_f, "alg_bytes_per_launch": bw_b,
                                  "recurrence_fp32_tflops": bw_tf,
                                  "avg_launch_ms": bw_ms}},
        "parity_sample": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
