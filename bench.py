#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule mixer on one MI355X.

Headline (the JSON `value`): chunked prefill throughput at T = 65,536 tokens,
B = 1, 16 key heads / 48 value heads, head dim 128, random fp32 initial state,
fp32 outputs and final state -- one `gdn_chunk_fwd` launch per step, inputs
resident in HBM.  The same run also times, as extra legs in the same JSON line:
  decode  one batched decode step, 256 sequences, fp32 state [256,48,128,128]
          updated in place (state GB/s), plus the batch-mode conv-state update,
          a 4-tokens-per-sequence step (gdn_decode_tokens) and the whole mixer
          step in one launch (gdn_decode_mixer_step);
  mixer   the full mixer at T = 8192: conv + SiLU + L2 -> chunked rule -> gated
          RMSNorm, as four launches and as one gdn_mixer_fwd call (the conv
          front inside the prep kernel);
  varlen  packed prefill of 262,144 tokens in 24 sequences (cu_seqlens);
  backward  gdn_backward (the rule's gradients) on 8 x 1024 and 1 x 8192 tokens.
  latency   the core recurrence at T = 512 (zero state): median and min of
          single launches;
  ceilings  what this device sustains: a 1 GiB device copy, a streaming
          in-place pass over the decode step's 805 MB of states
          (gdn_calib_stream_inplace: each piece read and written back once)
          and a dense fp16 MFMA loop (gdn_calib_mfma_loop), beside the
          published peaks.
Two more prefill timings, not the headline: o written in bf16
(`prefill_bf16_o`) and the gates formed from bf16 projections (`prefill_gated`).
`roofline` covers the prefill launch (one `gdn_chunk_fwd`: the parallel prep
kernel, then the sequential scan kernel, back to back on one stream):
algorithmic bytes per launch over the launch duration measured with HIP events
on the launch stream, against the 8 TB/s HBM3E peak (the arithmetic intensity,
~136 flop/B, is below the MFMA ridge); `mfma` gives the same launch against the
2.5 PFLOP/s dense fp16/bf16 MFMA peak.  `traffic` is the HBM bytes per launch
that rocprofv3's FETCH_SIZE + WRITE_SIZE counters recorded (scaled by the
counters' reading for a plain 1 GiB copy), taken from profiles/ and reported
only while the prefill source is the one they were taken on.  `cpu_baseline`
times the fp64 CPU oracle on a bounded prefix of the same prefill input on this
host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs prefill,decode,...]
(`--legs copy` adds a plain 1 GiB device copy, the calibration kernel for the
HBM byte counters.)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s @T=64K (% MFMA peak); decode-step state GB/s (% HBM)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0          # dense fp16 / bf16 MFMA, MI355X
HK, HV, D, C = 16, 48, 128, 64
# algorithmic work per token of the chunked rule (chunk 64): Gram products per
# key head + (W, U~, intra-chunk O: 3 dv (C+1)) + (K S0^T, Q S0^T, S update: 6 dk dv)
# per value head
FLOP_PER_TOKEN = HK * 2 * D * C + HV * (3 * D * (C + 1) + 6 * D * D)      # 6,178,816
# bytes per token: q, k, v bf16; g, beta fp32; o fp32
BYTES_PER_TOKEN = HK * D * 2 * 2 + HV * D * 2 + HV * 4 * 2 + HV * D * 4   # 45,440
STATE_BYTES = HV * D * D * 4                                              # 3,145,728
DECODE_N = 256                                                            # sequences of the decode leg


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_leg(fn, steps, warmup):
    """Run fn `warmup` times, then `steps` times bracketed by HIP events on the
    current stream.  Returns (mean event ms, wall ms per step)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = sum(s.elapsed_time(e) for s, e in evs) / steps
    return ev, wall


def leg_prefill(args, ops, synth, torch):
    T = 65536
    log(f"[prefill] drawing inputs T={T}")
    ci = synth.chunk_inputs_torch(1002, T, h0_std=0.02)
    q, k, v, g, b, h0 = ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], ci["h0"]
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_bytes(1, T, HK, HV), dtype=torch.uint8,
                     device="cuda")

    def step():
        ops.gdn_chunk_fwd(q, k, v, g, b, initial_state=h0, final_state=fs, o=o, n_seqs=1,
                          workspace=ws)

    ev, wall = time_leg(step, args.steps, args.warmup)
    bytes_launch = T * BYTES_PER_TOKEN + 2 * STATE_BYTES
    flops_launch = T * FLOP_PER_TOKEN
    res = dict(tokens=T, event_ms=ev, wall_ms=wall, tokens_per_s=T / (wall * 1e-3),
               alg_bytes=bytes_launch, alg_flops=flops_launch,
               hbm_gbps=bytes_launch / (ev * 1e-3) / 1e9,
               mfma_tflops=flops_launch / (ev * 1e-3) / 1e12)
    log(f"[prefill] {ev:.3f} ms/launch, {res['tokens_per_s'] / 1e6:.2f} M tok/s, "
        f"{res['hbm_gbps']:.0f} GB/s alg, {res['mfma_tflops']:.1f} TFLOP/s alg")

    if "bf16o" not in args.prefill_forms:
        return res, ci
    # the same launch with o written in bf16 (gdn_chunk_fwd_bf16o); not the headline
    o16 = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")

    def step16():
        ops.gdn_chunk_fwd(q, k, v, g, b, initial_state=h0, final_state=fs, o=o16, n_seqs=1,
                          workspace=ws)

    ev16, _ = time_leg(step16, args.steps, args.warmup)
    res.update(bf16o_event_ms=ev16, bf16o_tokens_per_s=T / (ev16 * 1e-3))
    log(f"[prefill] bf16 o: {ev16:.3f} ms/launch, {res['bf16o_tokens_per_s'] / 1e6:.2f} M tok/s")

    if "gated" not in args.prefill_forms:
        return res, ci
    # the same launch with the gates formed from bf16 projections (gdn_chunk_fwd_gated)
    gi = synth.gate_inputs(1007, T)
    ga = torch.from_numpy(gi.a.view("int16")).view(torch.bfloat16).cuda()
    gb = torch.from_numpy(gi.b.view("int16")).view(torch.bfloat16).cuda()
    A_log, dt_bias = torch.from_numpy(gi.A_log).cuda(), torch.from_numpy(gi.dt_bias).cuda()

    def step_gated():
        ops.gdn_chunk_fwd_gated(q, k, v, ga, gb, A_log, dt_bias, initial_state=h0, final_state=fs,
                                o=o, n_seqs=1, workspace=ws)

    evg, _ = time_leg(step_gated, args.steps, args.warmup)
    res.update(gated_event_ms=evg, gated_tokens_per_s=T / (evg * 1e-3))
    log(f"[prefill] gates from projections: {evg:.3f} ms/launch")
    return res, ci


def leg_decode(args, ops, synth, torch):
    N = DECODE_N
    log(f"[decode] drawing inputs N={N}")
    di = synth.decode_inputs_torch(1003, N)
    o = torch.empty((N, HV, D), dtype=torch.float32, device="cuda")

    def step():
        ops.gdn_decode_step(di["q"], di["k"], di["v"], di["g"], di["beta"], di["state"], o=o)

    ev, wall = time_leg(step, args.steps, args.warmup)
    sbytes = 2 * N * STATE_BYTES
    y = torch.empty((N, HK * 2 * D + HV * D), dtype=torch.bfloat16, device="cuda")

    def conv_step():
        ops.gdn_conv1d_fwd(di["x"], di["conv_w"], y=y, conv_state=di["conv_state"], n_seqs=N,
                           n_l2_heads=2 * HK)

    cev, cwall = time_leg(conv_step, args.steps, args.warmup)
    cbytes = N * y.shape[1] * 2 * 2 + N * y.shape[1] * 3 * 2 * 2 + y.shape[1] * 4 * 2

    # several tokens per sequence in one pass over the state (gdn_decode_tokens)
    NT = 4
    gen = torch.Generator(device="cuda").manual_seed(1005)

    def unit(shape):
        a = torch.randn(shape, generator=gen, device="cuda")
        return (a / a.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    tq, tk = unit((N * NT, HK, D)), unit((N * NT, HK, D))
    tv = torch.randn((N * NT, HV, D), generator=gen, device="cuda").to(torch.bfloat16)
    tg = torch.rand((N * NT, HV), generator=gen, device="cuda") * -0.1
    tb = torch.sigmoid(torch.randn((N * NT, HV), generator=gen, device="cuda"))
    to = torch.empty((N * NT, HV, D), dtype=torch.float32, device="cuda")

    def tokens_step():
        ops.gdn_decode_tokens(tq, tk, tv, tg, tb, di["state"], NT, o=to)

    tev, twall = time_leg(tokens_step, args.steps, args.warmup)

    # the whole mixer's decode step in one launch (gdn_decode_mixer_step) against
    # the three launches it replaces (batch conv, decode step, gated norm)
    z = torch.randn((N, HV, D), generator=gen, device="cuda").to(torch.bfloat16)
    nw = 1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")
    mo = torch.empty((N, HV, D), dtype=torch.float32, device="cuda")
    yv = y.view(N, 2 * HK + HV, D)

    def fused_step():
        ops.gdn_decode_mixer_step(di["x"], di["conv_w"], di["conv_state"], di["g"], di["beta"], z,
                                  nw, di["state"], Hk=HK, out=mo)

    def unfused_step():
        ops.gdn_conv1d_fwd(di["x"], di["conv_w"], y=y, conv_state=di["conv_state"], n_seqs=N,
                           n_l2_heads=2 * HK)
        ops.gdn_decode_step(yv[:, :HK], yv[:, HK:2 * HK], yv[:, 2 * HK:], di["g"], di["beta"],
                            di["state"], o=o)
        ops.gdn_gated_rmsnorm(o, z, nw, out=mo)

    fev, _ = time_leg(fused_step, args.steps, args.warmup)
    uev, _ = time_leg(unfused_step, args.steps, args.warmup)
    C = y.shape[1]
    fbytes = sbytes + N * C * 2 + 2 * N * C * 3 * 2 + C * 4 * 2 + N * HV * D * (2 + 4) + 2 * N * HV * 4
    res = dict(n_seqs=N, event_ms=ev, wall_ms=wall, state_bytes=sbytes,
               state_gbps=sbytes / (ev * 1e-3) / 1e9,
               frac_hbm=sbytes / (ev * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               conv_event_ms=cev, conv_alg_bytes=cbytes, conv_gbps=cbytes / (cev * 1e-3) / 1e9,
               tokens_n=NT, tokens_event_ms=tev,
               tokens_state_gbps=sbytes / (tev * 1e-3) / 1e9,
               tokens_per_s=N * NT / (tev * 1e-3),
               fused_event_ms=fev, unfused_event_ms=uev, fused_alg_bytes=fbytes,
               fused_gbps=fbytes / (fev * 1e-3) / 1e9)
    log(f"[decode] {ev:.3f} ms/step, state {res['state_gbps']:.0f} GB/s "
        f"({100 * res['frac_hbm']:.1f}% of HBM); conv update {cev * 1e3:.1f} us; "
        f"{NT} tokens/sequence: {tev:.3f} ms, {res['tokens_per_s'] / 1e6:.2f} M tok/s; "
        f"whole mixer step fused {fev:.3f} ms ({res['fused_gbps']:.0f} GB/s alg) vs "
        f"three launches {uev:.3f} ms")
    return res


def leg_mixer(args, ops, synth, torch):
    T = 8192
    log(f"[mixer] drawing inputs T={T}")
    mi = synth.mixer_inputs_torch(1001, T)
    y = torch.empty((T, (2 * HK + HV) * D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    out = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    yv = y.view(T, 2 * HK + HV, D)

    def step():
        ops.gdn_conv1d_fwd(mi["x"], mi["conv_w"], y=y, n_seqs=1, n_l2_heads=2 * HK)
        ops.gdn_chunk_fwd(yv[:, :HK], yv[:, HK:2 * HK], yv[:, 2 * HK:], mi["g"], mi["beta"],
                          final_state=fs, o=o, n_seqs=1)
        ops.gdn_gated_rmsnorm(o, mi["z"], mi["norm_w"], out=out)

    ev, wall = time_leg(step, args.steps, args.warmup)

    # the same mixer in one call, the conv front inside the prep kernel (gdn_mixer_fwd)
    ws = torch.empty(ops.gdn_mixer_fwd_workspace_bytes(1, T, HK, HV), dtype=torch.uint8,
                     device="cuda")

    def fused_step():
        ops.gdn_mixer_fwd(mi["x"], mi["conv_w"], mi["g"], mi["beta"], mi["z"], mi["norm_w"], Hk=HK,
                          final_state=fs, n_seqs=1, out=out, workspace=ws)

    fev, fwall = time_leg(fused_step, args.steps, args.warmup)
    res = dict(tokens=T, event_ms=ev, wall_ms=wall, tokens_per_s=T / (wall * 1e-3),
               fused_event_ms=fev, fused_tokens_per_s=T / (fwall * 1e-3))
    log(f"[mixer] {ev:.3f} ms/step, {res['tokens_per_s'] / 1e6:.2f} M tok/s; "
        f"one call with the conv front fused: {fev:.3f} ms, "
        f"{res['fused_tokens_per_s'] / 1e6:.2f} M tok/s")
    return res


def leg_varlen(args, ops, synth, torch):
    lens = synth.varlen_lengths(1004)
    T = int(lens.sum())
    log(f"[varlen] drawing inputs T={T} N={len(lens)}")
    ci = synth.chunk_inputs_torch(1004, T, lengths=lens, h0_std=0.02)
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((len(lens), HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_bytes(len(lens), T, HK, HV), dtype=torch.uint8,
                     device="cuda")

    def step():
        ops.gdn_chunk_fwd(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], initial_state=ci["h0"],
                          final_state=fs, o=o, cu_seqlens=ci["cu_seqlens"], workspace=ws)

    ev, wall = time_leg(step, max(2, args.steps // 2), max(1, args.warmup // 2))
    bytes_launch = T * BYTES_PER_TOKEN + 2 * len(lens) * STATE_BYTES
    res = dict(tokens=T, n_seqs=len(lens), event_ms=ev, wall_ms=wall,
               tokens_per_s=T / (wall * 1e-3), hbm_gbps=bytes_launch / (ev * 1e-3) / 1e9,
               mfma_tflops=T * FLOP_PER_TOKEN / (ev * 1e-3) / 1e12)
    log(f"[varlen] {ev:.3f} ms/launch, {res['tokens_per_s'] / 1e6:.2f} M tok/s")
    return res


# matrix products per (chunk of 64 tokens, value head) of the chunked
# backward, counted as fp32 16x16x4 products (2,048 flops each; the gradient
# pass's products with S0 and dS_C run as split-bf16 16x16x32 products and are
# counted by the fp32 work they stand for), masked blocks included:
#   per-chunk pass   Q K^T, K K^T: 640 per key head = 640 / 3 per value head
#   forward chain    K S0^T 128, T R 40, K^T (D U) 128 per 16-channel tile x 8
#   reverse chain    K dS^T 128, P^T dO 40, T^T dU 40, the dS update 256, x 8
#   gradient pass    dP and dA 640, the S0 / dS_C products 3,072, the
#                    (dP o M), W products 1,280, K K^T 320 / 3
BWD_MFMA_PER_CHUNK_HEAD = 640 / 3 + 8 * 296 + 8 * 464 + 640 + 3072 + 1280 + 320 / 3
FP32_MFMA_PEAK_TFLOPS = 157.3       # dense fp32 matrix, MI355X


def leg_backward(args, ops, synth, torch):
    """gdn_backward over two training-shaped batches: 8 sequences of 1024
    tokens, and one sequence of 8192 (the longest chain)."""
    res = {}
    for N, L in ((8, 1024), (1, 8192)):
        T = N * L
        log(f"[backward] drawing inputs N={N} L={L}")
        ci = synth.chunk_inputs_torch(1008, T, lengths=[L] * N, h0_std=0.02)
        bs = synth.backward_seeds_torch(1009, T, N)
        d_o, dhT = bs["d_o"], bs["dhT"]
        ws = torch.empty(ops.gdn_backward_workspace_bytes(N, T, HV), dtype=torch.uint8, device="cuda")

        def step():
            ops.gdn_backward(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], d_o,
                             initial_state=ci["h0"], grad_final_state=dhT,
                             cu_seqlens=ci["cu_seqlens"], workspace=ws)

        ev, wall = time_leg(step, max(2, args.steps // 4), 1)
        chunk_heads = N * ((L + C - 1) // C) * HV
        flops = chunk_heads * BWD_MFMA_PER_CHUNK_HEAD * 2048
        r = dict(tokens=T, n_seqs=N, event_ms=ev, wall_ms=wall, tokens_per_s=T / (ev * 1e-3),
                 mfma_fp32_tflops=flops / (ev * 1e-3) / 1e12, workspace_bytes=ws.numel())
        log(f"[backward] {N} x {L}: {ev:.3f} ms/call, {r['tokens_per_s'] / 1e6:.3f} M tok/s, "
            f"{r['mfma_fp32_tflops']:.1f} TFLOP/s fp32 matrix, workspace {ws.numel() / T / 1024:.0f} KiB/token")
        res[f"{N}x{L}"] = r
        del ws, ci, bs, d_o, dhT
    return res


def leg_copy(args, torch):
    """A plain device-to-device copy of 1 GiB: reads and writes exactly 2^30
    bytes each, the reference for scaling the HBM byte counters."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ev, wall = time_leg(lambda: dst.copy_(src), max(2, args.steps // 4), 1)
    log(f"[copy] 1 GiB copy {ev:.3f} ms, {2 * n / (ev * 1e-3) / 1e9:.0f} GB/s")
    return dict(bytes=2 * n, event_ms=ev)


def leg_latency(args, ops, synth, torch):
    """The core recurrence at T = 512 (B = 1, zero initial state, fp32 o and
    final state): a latency figure, each launch bracketed by its own events."""
    T = 512
    log(f"[latency] drawing inputs T={T}")
    ci = synth.chunk_inputs_torch(1000, T)
    o = torch.empty((T, HV, D), dtype=torch.float32, device="cuda")
    fs = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_bytes(1, T, HK, HV), dtype=torch.uint8,
                     device="cuda")

    def step():
        ops.gdn_chunk_fwd(ci["q"], ci["k"], ci["v"], ci["g"], ci["beta"], final_state=fs, o=o,
                          n_seqs=1, workspace=ws)

    for _ in range(max(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    n = max(args.steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for s, e in evs:
        s.record()
        step()
        e.record()
        e.synchronize()
    ts = sorted(s.elapsed_time(e) for s, e in evs)
    med, mn = ts[len(ts) // 2], ts[0]
    bytes_launch = T * BYTES_PER_TOKEN + STATE_BYTES      # zero initial state: S_T only
    res = dict(tokens=T, median_ms=med, min_ms=mn, tokens_per_s=T / (med * 1e-3),
               hbm_frac=bytes_launch / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               mfma_frac=T * FLOP_PER_TOKEN / (med * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS)
    log(f"[latency] T={T}: median {med * 1e3:.1f} us, min {mn * 1e3:.1f} us per launch")
    return res


def leg_ceilings(args, ops, torch):
    """Measured ceilings of this device beside the published peaks: a 1 GiB
    device copy (HBM) and the dense fp16 MFMA loop."""
    cp = leg_copy(args, torch)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_blocks, n_iter = 4 * cus, 4096
    out = torch.empty(4 * n_blocks, dtype=torch.float32, device="cuda")
    flops = ops.gdn_calib_mfma_loop(n_iter, n_blocks, out)[1]
    ev, _ = time_leg(lambda: ops.gdn_calib_mfma_loop(n_iter, n_blocks, out), 5, 2)
    tflops = flops / (ev * 1e-3) / 1e12
    # the decode step's states, streamed in place (4 work-groups per CU)
    buf = torch.zeros(DECODE_N * STATE_BYTES // 4, dtype=torch.float32, device="cuda")
    sbytes = ops.gdn_calib_stream_inplace(buf, 4 * cus)
    sev, _ = time_leg(lambda: ops.gdn_calib_stream_inplace(buf, 4 * cus), 10, 3)
    del buf
    sgbps = sbytes / (sev * 1e-3) / 1e9
    log(f"[ceilings] copy {cp['bytes'] / (cp['event_ms'] * 1e-3) / 1e9:.0f} GB/s; "
        f"streaming in place {sgbps:.0f} GB/s ({sbytes / 2e6:.0f} MB); "
        f"MFMA loop {tflops:.0f} TFLOP/s ({n_blocks} x 4 waves x {n_iter} x 8 products)")
    return dict(copy_gbps=cp["bytes"] / (cp["event_ms"] * 1e-3) / 1e9, copy_event_ms=cp["event_ms"],
                stream_gbps=sgbps, stream_event_ms=sev,
                mfma_tflops=tflops, mfma_event_ms=ev, mfma_blocks=n_blocks, mfma_iters=n_iter)


PREFILL_SOURCES = ("gated_delta_rule_09_amd/csrc/chunk.hip", "gated_delta_rule_09_amd/csrc/common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_T65536_traffic.json")


def prefill_source_sha():
    """Hash of the prefill sources' code: // comments and blank lines are
    dropped, so a comment edit does not invalidate the counter figures."""
    h = hashlib.sha256()
    for rel in PREFILL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter runs, or None
    when they were taken on different prefill sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != prefill_source_sha():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(ci, seconds, torch):
    """The fp64 oracle on a prefix of the prefill input, all 48 heads."""
    import numpy as np
    import oracle

    def host_bf16(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)

    threads = len(os.sched_getaffinity(0))
    q, k, v = host_bf16(ci["q"]), host_bf16(ci["k"]), host_bf16(ci["v"])
    g, b = ci["g"].cpu().numpy(), ci["beta"].cpu().numpy()
    h0 = ci["h0"].cpu().numpy()
    # calibrate on 256 tokens, then size the sample for ~`seconds` of work
    t0 = time.perf_counter()
    oracle.recurrence(q[:256], k[:256], v[:256], g[:256], b[:256], h0, n_threads=threads)
    rate = 256 / (time.perf_counter() - t0)
    Ts = int(min(q.shape[0], max(512, rate * seconds)))
    Ts -= Ts % 64
    log(f"[cpu] oracle on {Ts} tokens x {HV} heads, {threads} threads")
    t0 = time.perf_counter()
    oracle.recurrence(q[:Ts], k[:Ts], v[:Ts], g[:Ts], b[:Ts], h0, n_threads=threads)
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": f"first {Ts} tokens of the T=65536 prefill input, all 48 value heads, "
                      f"fp64 sequential recurrence, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="prefill,latency,decode,mixer,varlen,backward,ceilings")
    ap.add_argument("--prefill-forms", default="fp32,bf16o,gated",
                    help="prefill launch forms timed by the prefill leg (fp32 is always timed)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the mixer shards by heads or sequences with no "
              "exchange; the figures here are for a single MI355X (--gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_09_amd import ops, synth
    torch.cuda.set_device(0)
    ops.lib()
    legs = args.legs.split(",")
    out = {}
    ci = None
    if "prefill" in legs:
        out["prefill"], ci = leg_prefill(args, ops, synth, torch)
    if "latency" in legs:
        out["latency"] = leg_latency(args, ops, synth, torch)
    if "decode" in legs:
        out["decode"] = leg_decode(args, ops, synth, torch)
    if "mixer" in legs:
        out["mixer"] = leg_mixer(args, ops, synth, torch)
    if "varlen" in legs:
        out["varlen"] = leg_varlen(args, ops, synth, torch)
    if "backward" in legs:
        out["backward"] = leg_backward(args, ops, synth, torch)
    if "copy" in legs:
        out["copy"] = leg_copy(args, torch)
    if "ceilings" in legs:
        out["ceilings"] = leg_ceilings(args, ops, torch)

    pre = out.get("prefill")
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"] if pre else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["wall_ms"] if pre else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands, f32 accumulate, f32 state",
        "data": "synthetic",
        "config": {"workload": "chunked prefill B=1 T=65536 Hk=16 Hv=48 d=128, fp32 S0, "
                               "fp32 o + final state", "tokens": 65536, "chunk": C,
                   "parallelism": "single GPU"},
    }
    if pre:
        line["roofline"] = {"bound": "hbm", "achieved": round(pre["hbm_gbps"], 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(pre["hbm_gbps"] / HBM_PEAK_GBPS, 4),
                            "traffic": measured_traffic(),
                            "kernel": "chunk_prep_kernel + chunk_scan_kernel (one gdn_chunk_fwd)",
                            "launch_ms": round(pre["event_ms"], 4)}
        line["mfma"] = {"achieved": round(pre["mfma_tflops"], 1), "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(pre["mfma_tflops"] / MFMA_PEAK_TFLOPS, 4)}
        if "bf16o_event_ms" in pre:
            line["prefill_bf16_o"] = {"launch_ms": round(pre["bf16o_event_ms"], 4),
                                      "tokens_per_s": round(pre["bf16o_tokens_per_s"], 1)}
        if "gated_event_ms" in pre:
            line["prefill_gated"] = {"launch_ms": round(pre["gated_event_ms"], 4),
                                     "tokens_per_s": round(pre["gated_tokens_per_s"], 1)}
    if "latency" in out:
        la = out["latency"]
        line["latency_T512"] = {"median_ms": round(la["median_ms"], 4),
                                "min_ms": round(la["min_ms"], 4),
                                "tokens_per_s": round(la["tokens_per_s"], 1),
                                "hbm_frac": round(la["hbm_frac"], 4),
                                "mfma_frac": round(la["mfma_frac"], 4)}
    if "ceilings" in out:
        ce = out["ceilings"]
        line["ceilings"] = {"copy_GBps": round(ce["copy_gbps"], 1),
                            "copy_frac_of_peak": round(ce["copy_gbps"] / HBM_PEAK_GBPS, 4),
                            "stream_inplace_GBps": round(ce["stream_gbps"], 1),
                            "stream_inplace_frac_of_peak": round(ce["stream_gbps"] / HBM_PEAK_GBPS, 4),
                            "mfma_loop_TFLOPs": round(ce["mfma_tflops"], 1),
                            "mfma_loop_frac_of_peak": round(ce["mfma_tflops"] / MFMA_PEAK_TFLOPS, 4)}
    if "decode" in out:
        d = out["decode"]
        line["decode"] = {"state_GBps": round(d["state_gbps"], 1),
                          "frac_hbm": round(d["frac_hbm"], 4),
                          "launch_ms": round(d["event_ms"], 4),
                          "conv_update_ms": round(d["conv_event_ms"], 4),
                          "tokens4": {"launch_ms": round(d["tokens_event_ms"], 4),
                                      "tokens_per_s": round(d["tokens_per_s"], 1),
                                      "state_GBps": round(d["tokens_state_gbps"], 1)},
                          "mixer_step": {"fused_ms": round(d["fused_event_ms"], 4),
                                         "three_launches_ms": round(d["unfused_event_ms"], 4),
                                         "alg_GBps": round(d["fused_gbps"], 1)}}
    if "mixer" in out:
        line["mixer_T8192"] = {"tokens_per_s": round(out["mixer"]["tokens_per_s"], 1),
                               "ms": round(out["mixer"]["event_ms"], 4),
                               "fused": {"tokens_per_s": round(out["mixer"]["fused_tokens_per_s"], 1),
                                         "ms": round(out["mixer"]["fused_event_ms"], 4)}}
    if "varlen" in out:
        vl = out["varlen"]
        line["varlen_262144x24"] = {"tokens_per_s": round(vl["tokens_per_s"], 1),
                                    "ms": round(vl["event_ms"], 4),
                                    "hbm_frac": round(vl["hbm_gbps"] / HBM_PEAK_GBPS, 4),
                                    "mfma_frac": round(vl["mfma_tflops"] / MFMA_PEAK_TFLOPS, 4)}
    if "backward" in out:
        for key, bw in out["backward"].items():
            line[f"backward_{key}"] = {
                "ms": round(bw["event_ms"], 4), "tokens_per_s": round(bw["tokens_per_s"], 1),
                "mfma_fp32_tflops": round(bw["mfma_fp32_tflops"], 2),
                "mfma_fp32_frac": round(bw["mfma_fp32_tflops"] / FP32_MFMA_PEAK_TFLOPS, 4),
                "workspace_bytes_per_token": round(bw["workspace_bytes"] / bw["tokens"])}
    if ci is not None and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(ci, args.cpu_seconds, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
