#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step is one kda_chunk_fwd over the long-context prefill workload
(B1 H32 T65536, dk = dv = 128, chunk 64, bf16 q/k/v, fp32 alpha/beta/state,
o in bf16).  `value` is prefill tokens/s over the timed steps, bracketed by
HIP events on the launch stream.  The same number of steps then runs as the
call's two halves, kda_chunk_fwd_intra and kda_chunk_fwd_inter, with events
between them: they time each kernel for the roofline figures (the events add
a little: "ms_per_step_as_two_halves").  The decode workload (256 sequences x H32, 128
in-place steps) is measured in the same run and reported under "decode" as
state GB/s.  Inputs are seeded synthetic data already resident in HBM when a
timed region starts.

The line also carries the roofline of the dominant kernel (algorithmic bytes
or flops per launch / measured average launch time, against MI355X peaks),
the same for every kernel, the fp64 CPU oracle timed on a bounded sample of
the workload on this host, and ("variants") the time of one call with each
option of kda_chunk_fwd_ex / kda_decode_step_ex on the same workloads, of the
gated layer with fused inputs in a 1 GiB workspace (kda_chunk_fwd_windowed_ex),
of the packed variable-length workload (in one piece, and in a 2 GiB workspace
through kda_chunk_fwd_windowed), of one 2^20-token sequence over the same 32
heads, and of one sequence's decode steps issued one by one and replayed as one
HIP graph.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode state GB/s (dk=dv=128), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak


def algorithmic(dk, dv, chunk, qkv_bytes=2, o_bytes=2):
    """Per-unit algorithmic costs of the path (what the method itself must move or compute)."""
    in_bytes = 2 * dk * qkv_bytes + dv * qkv_bytes + dk * 4 + 4   # q, k, v, alpha, beta
    return {
        # intra-chunk kernel: reads every input once
        "intra_bytes_per_token_head": in_bytes,
        # inter-chunk kernel: W S, Qtilde S, Kbar^T U (2 dk dv flops each) and the causal
        # P U (triangle counted at half: C dv)
        "inter_flops_per_token_head": 6 * dk * dv + chunk * dv,
        "prefill_bytes_per_token_head": in_bytes + dv * o_bytes,
        "state_bytes_per_seq_head": dk * dv * 4,
        # decode: state read + written once, plus the token's q, k, v, alpha, beta and o
        "decode_bytes_per_head_step": 2 * dk * dv * 4 + in_bytes + dv * o_bytes,
    }


# HBM bytes per launch of each kernel on the workloads above, from two rocprofv3
# counter passes over this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by what the same counter reads for a calibration dispatch that
# reads and writes 1 GiB (--copy-calibration): FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.
# A figure is reported only while the kernel sources hash to the value it was
# measured on; after any change it is null until the counters are taken again.
KERNEL_SOURCES = {
    "prefill": ["kda_prefill.hip", "kda_quads.h", "kda_kernels.h"],
    "decode": ["kda_decode.hip", "kda_quads.h", "kda_kernels.h"],
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {  # kernel: (sources, sha256[:16] of the sources, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "kda_intra_kernel": ("prefill", "70cc7a22baa70465", 1343686.4, 2379672.3),
    "kda_range_kernel": ("prefill", "70cc7a22baa70465", 702832.7, 29740.0),
    "kda_range_scan_kernel": ("prefill", "70cc7a22baa70465", 14367.6, 14336.0),
    "kda_inter_kernel": ("prefill", "70cc7a22baa70465", 1205855.9, 526451.9),
    "kda_decode_kernel": ("decode", "36ee23fa6ad7684f", 267578.0, 526427.7),
}


def source_sha(which):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, "linear_attention_sequence_gated_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(kernel):
    """Measured HBM bytes per launch, or None if the kernel changed since."""
    if kernel not in TRAFFIC:
        return None
    which, sha, fetch_kib, write_kib = TRAFFIC[kernel]
    if source_sha(which) != sha:
        return None
    return int((fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024)


def roof(bound, amount, seconds, unit, kernel, traffic=None):
    peak = HBM_PEAK_GBS if unit == "GB/s" else MFMA_F16_PEAK_TFLOPS
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = amount / seconds / scale
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, heads, target_s=12.0):
    """Oracle tokens/s on a leading slice of the prefill workload, all heads."""
    from oracle import kda_oracle

    def run(tokens):
        sl = {k: inp[k][:, :tokens] for k in ("q", "k", "v", "alpha", "beta")}
        t0 = time.perf_counter()
        kda_oracle.forward(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"])
        return time.perf_counter() - t0

    probe = 256
    dt = run(probe)
    T = inp["q"].shape[1]
    tokens = int(min(T, max(probe, probe * target_s / max(dt, 1e-6))))
    tokens = max(64, tokens // 64 * 64)
    dt = run(tokens)
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": kda_oracle.threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {tokens} tokens of the prefill workload, all {heads} heads "
                      f"({tokens * heads} token-heads), fp64 token-by-token, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first calls after the inputs are drawn run ~2.5 % slower than the
    # steady state (2.098 against 2.040-2.050 ms per step with 10 or 30
    # warm-up calls): 20 by default
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the timing of the option variants")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one MI355X only (--gpus {args.gpus}, WORLD_SIZE {world}): this KDA "
              "library runs on one GPU; heads, sequences and value columns would shard across GPUs "
              "with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_sequence_gated_amd as kda
    import workloads
    PREFILL_CFG, DECODE_CFG = workloads.LONG_CONTEXT_PREFILL, workloads.DECODE
    from linear_attention_sequence_gated_amd import build as kbuild

    if not os.path.exists(kbuild.LIB):
        kbuild.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---- prefill -------------------------------------------------------------
    w = workloads.CONFIGS[PREFILL_CFG]
    log(f"generating {w.name} inputs")
    host = workloads.config_inputs(PREFILL_CFG)
    d = {k: (v.to(dev) if v is not None else None) for k, v in host.items()}
    pre = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                      chunk_size=w.chunk, o_dtype=torch.bfloat16)
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        pre.run()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    e_begin, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_begin.record(stream)
    for _ in range(args.steps):
        pre.run()   # one kda_chunk_fwd
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_begin.elapsed_time(e_end) / args.steps
    # the same number of steps again as the call's two halves with events
    # between them, for the time of each kernel
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps as two halves")
    for i in range(args.steps):
        ev[i][0].record(stream)
        pre.intra()
        ev[i][1].record(stream)
        pre.inter()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    intra_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    inter_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    halves_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    tokens = w.batch * w.seqlen
    th = tokens * w.heads
    alg = algorithmic(w.dk, w.dv, w.chunk)
    intra_roof = roof("hbm", th * alg["intra_bytes_per_token_head"], intra_ms / 1e3, "GB/s",
                      "kda_intra_kernel", traffic("kda_intra_kernel"))
    # the inter-chunk pass is one kernel, or three when the call cuts its
    # sequences into chunk ranges (range maps, start-state scan, ranged walk)
    plan = kda.chunk_plan(d["q"], d["v"], d["cu_seqlens"], chunk_size=w.chunk)
    inter_kernels = (["kda_range_kernel", "kda_range_scan_kernel", "kda_inter_kernel"] if plan["range_chunks"] > 0
                     else ["kda_inter_kernel"])
    t_parts = [traffic(k) for k in inter_kernels]
    t_out = None if None in t_parts else sum(t_parts)
    inter_roof = roof("mfma", th * alg["inter_flops_per_token_head"], inter_ms / 1e3, "TFLOP/s",
                      " + ".join(inter_kernels), t_out)
    step_bytes = th * alg["prefill_bytes_per_token_head"] + w.batch * w.heads * alg["state_bytes_per_seq_head"]
    t_in = traffic("kda_intra_kernel")
    step_roof = roof("hbm", step_bytes, step_ms / 1e3, "GB/s", "kda_chunk_fwd (whole step)",
                     t_in + t_out if t_in is not None and t_out is not None else None)
    # ---- prefill variants (kda_chunk_fwd_ex options), whole call ----------------
    variants = {}
    if not args.no_variants:
        def time_call(fn, reps=5, warm=3):
            # a fresh call object's first runs touch its new workspace (several
            # GiB): they are left out
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        log("timing prefill variants")
        g = torch.Generator(device=dev).manual_seed(7)
        base = dict(chunk_size=w.chunk, o_dtype=torch.bfloat16, o=pre.o, final_state=pre.final_state)
        args0 = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])

        def time_variant(inputs, **opts):   # one marshalled call per variant, its own workspace
            pv = kda.Prefill(*inputs, **base, **opts)
            ms = time_call(pv.run)
            del pv
            return ms

        plain_ms = time_variant(args0)
        variants["prefill_plain"] = {"ms": round(plain_ms, 4)}
        every = 4096
        ck = torch.empty((w.batch, w.seqlen // every, w.heads, w.dk, w.dv), dtype=torch.float32, device=dev)
        ms = time_variant(args0, checkpoints=ck, ckpt_every=every)
        variants["prefill_checkpoints"] = {"ms": round(ms, 4), "every_tokens": every,
                                           "checkpoints": ck.shape[1], "vs_plain": round(ms / plain_ms, 4)}
        gate = torch.randn(d["v"].shape, generator=g, device=dev).to(d["v"].dtype)
        wn = torch.ones(w.dv, device=dev)
        ms = time_variant(args0, gate=gate, norm_weight=wn, norm_eps=1e-5)
        variants["prefill_output_gate"] = {"ms": round(ms, 4), "vs_plain": round(ms / plain_ms, 4)}
        al = torch.randn(d["alpha"].shape, generator=g, device=dev) + 4.0
        bl = torch.randn(d["beta"].shape, generator=g, device=dev)
        argsf = (d["q"], d["k"], d["v"], al, bl, d["S0"], d["cu_seqlens"])
        ms = time_variant(argsf, fuse_inputs=True, gate=gate, norm_weight=wn, norm_eps=1e-5)
        variants["prefill_fused_inputs_and_gate"] = {"ms": round(ms, 4), "vs_plain": round(ms / plain_ms, 4)}
        # the same gated layer in a 1 GiB workspace (kda_chunk_fwd_windowed_ex:
        # the sequence runs in windows that resume from the state)
        wsg = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        ms_g = time_call(lambda: kda.chunk_fwd_windowed(
            d["q"], d["k"], d["v"], al, bl, wsg, d["S0"], d["cu_seqlens"], o=pre.o, final_state=pre.final_state,
            chunk_size=w.chunk, o_dtype=torch.bfloat16, check_range=False, fuse_inputs=True, gate=gate,
            norm_weight=wn, norm_eps=1e-5))
        variants["prefill_fused_inputs_and_gate_windowed"] = {
            "ms": round(ms_g, 4), "workspace_bytes": int(wsg.numel()), "vs_one_piece": round(ms_g / ms, 4)}
        del wsg
        a_s = d["alpha"][..., 0].contiguous()
        argss = (d["q"], d["k"], d["v"], a_s, d["beta"], d["S0"], d["cu_seqlens"])
        ms = time_variant(argss, alpha_scalar=True)
        variants["prefill_scalar_gate"] = {"ms": round(ms, 4), "vs_plain": round(ms / plain_ms, 4)}
        ms = time_variant(args0, decay_floor=0.6)
        variants["prefill_decay_floor"] = {"ms": round(ms, 4), "floor": 0.6, "vs_plain": round(ms / plain_ms, 4)}
        del ck, gate, al, bl, a_s
    del pre, d
    torch.cuda.empty_cache()
    if not args.no_variants:
        # packed variable-length prefill with prefix-cache resume: 64 sequences
        # (the workload's seeded lengths), H16, nonzero initial states; inputs
        # drawn on the device with the workload's recipe, o in bf16
        wp = workloads.CONFIGS[workloads.PACKED_VARLEN_RESUME]
        log(f"generating {wp.name} inputs on the device")
        dp = workloads.device_inputs(workloads.PACKED_VARLEN_RESUME, dev)
        ptok = int(dp["q"].shape[1])
        pp = kda.Prefill(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dp["S0"], dp["cu_seqlens"],
                         chunk_size=wp.chunk, o_dtype=torch.bfloat16)
        ms = time_call(pp.run, reps=3)
        variants["prefill_packed_varlen_resume"] = {
            "ms": round(ms, 4), "tokens": ptok, "sequences": wp.packed_seqs, "heads": wp.heads,
            "tokens_per_s": round(ptok / (ms / 1e3), 1),
            "token_heads_per_s": round(ptok * wp.heads / (ms / 1e3), 1),
            "workspace_bytes": int(pp.workspace.numel())}
        # the same call in a 2 GiB workspace (kda_chunk_fwd_windowed: whole
        # sequences grouped, long ones in windows resuming from their state)
        wsw = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        cu_host = dp["cu_seqlens"].cpu()
        ms_w = time_call(lambda: kda.chunk_fwd_windowed(
            dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], wsw, dp["S0"], dp["cu_seqlens"], o=pp.o,
            final_state=pp.final_state, chunk_size=wp.chunk, o_dtype=torch.bfloat16, check_range=False,
            cu_seqlens_host=cu_host), reps=3)
        variants["prefill_packed_varlen_resume_windowed"] = {
            "ms": round(ms_w, 4), "workspace_bytes": int(wsw.numel()), "vs_one_piece": round(ms_w / ms, 4)}
        del pp, dp, wsw
        torch.cuda.empty_cache()
        # one sequence of 2^20 tokens over the long-context heads (the
        # million-token context), drawn on the device with the same recipe
        log("generating a 2^20-token sequence on the device")
        dm = workloads.device_shape_inputs(1 << 20, w.heads, w.dk, w.dv, w.dtype, dev, alpha_mu=w.alpha_mu, seed=11)
        pm = kda.Prefill(dm["q"], dm["k"], dm["v"], dm["alpha"], dm["beta"], None, None, chunk_size=w.chunk,
                         o_dtype=torch.bfloat16)
        ms = time_call(pm.run, reps=3)
        variants["prefill_one_million_tokens"] = {
            "ms": round(ms, 4), "tokens": 1 << 20, "heads": w.heads,
            "tokens_per_s": round((1 << 20) / (ms / 1e3), 1),
            "vs_long_context_per_token": round((ms / (1 << 20)) / (plain_ms / w.seqlen), 4),
            "workspace_bytes": int(pm.workspace.numel())}
        del pm, dm
        torch.cuda.empty_cache()

    # ---- decode --------------------------------------------------------------
    wd = workloads.CONFIGS[DECODE_CFG]
    log(f"generating {wd.name} inputs")
    dh = workloads.decode_inputs(DECODE_CFG, steps=args.decode_steps)
    dd = {k: v.to(dev) for k, v in dh.items()}
    state = dd["S0"].clone()
    o_dec = torch.empty(dd["v"].shape[1:], dtype=torch.bfloat16, device=dev)

    def dstep(t):
        kda.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["alpha"][t], dd["beta"][t], state,
                        o=o_dec, o_dtype=torch.bfloat16)

    for t in range(min(3, args.decode_steps)):
        dstep(t)
    state.copy_(dd["S0"])  # the timed run starts from the pristine state
    torch.cuda.synchronize()
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.decode_steps + 1)]
    log(f"timing {args.decode_steps} decode steps")
    dev_ev[0].record(stream)
    for t in range(args.decode_steps):
        dstep(t)
        dev_ev[t + 1].record(stream)
    torch.cuda.synchronize()
    dec_ms = dev_ev[0].elapsed_time(dev_ev[-1]) / args.decode_steps
    units = wd.decode_seqs * wd.heads
    dec_bytes = units * alg["decode_bytes_per_head_step"]
    state_bytes = units * 2 * wd.dk * wd.dv * 4
    dec_roof = roof("hbm", dec_bytes, dec_ms / 1e3, "GB/s", "kda_decode_kernel",
                    traffic("kda_decode_kernel"))
    decode = {
        "workload": f"decode {wd.decode_seqs} seqs x H{wd.heads} dk=dv={wd.dk}, "
                    f"{args.decode_steps} in-place steps (bf16 q/k/v/o, fp32 alpha/beta/state)",
        "value": round(state_bytes / (dec_ms / 1e3) / 1e9, 1), "unit": "GB/s (state read + write)",
        "ms_per_step": round(dec_ms, 4),
        "tokens_per_s": round(wd.decode_seqs / (dec_ms / 1e3), 1),
        "roofline": dec_roof,
    }
    if not args.no_variants:
        log("timing decode variants")
        N0, H0 = wd.decode_seqs, wd.heads
        # N distinct pool entries drawn at random from a pool twice that size (a
        # strided choice such as every other entry interleaves unevenly over HBM)
        pool = torch.empty((2 * N0, H0, wd.dk, wd.dv), dtype=torch.float32, device=dev)
        pick = torch.randperm(2 * N0, generator=torch.Generator().manual_seed(11))[:N0]
        pool[pick.to(dev)] = dd["S0"]
        slots = pick.to(torch.int32).to(dev)
        gate = torch.zeros(dd["v"].shape[1:], dtype=dd["v"].dtype, device=dev)
        wn = torch.ones(wd.dv, device=dev)

        def dtime(fn, reps=min(32, args.decode_steps)):
            for t in range(min(3, reps)):
                fn(t)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in range(reps):
                fn(t)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms = dtime(lambda t: kda.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["alpha"][t], dd["beta"][t],
                                             pool, o=o_dec, o_dtype=torch.bfloat16, state_slots=slots))
        variants["decode_paged_pool"] = {"ms": round(ms, 4), "vs_plain": round(ms / dec_ms, 4),
                                         "GB/s": round(state_bytes / (ms / 1e3) / 1e9, 1)}
        ms = dtime(lambda t: kda.decode_step(dd["q"][t], dd["k"][t], dd["v"][t], dd["alpha"][t], dd["beta"][t],
                                             pool, o=o_dec, o_dtype=torch.bfloat16, state_slots=slots,
                                             fuse_inputs=True, gate=gate, norm_weight=wn, norm_eps=1e-5))
        variants["decode_paged_fused_inputs_and_gate"] = {"ms": round(ms, 4), "vs_plain": round(ms / dec_ms, 4),
                                                          "GB/s": round(state_bytes / (ms / 1e3) / 1e9, 1)}
        del pool, slots, gate
        # one sequence (H heads, 2 MiB of state): the steps are launch-bound;
        # the same steps issued one by one and replayed as one HIP graph
        st1 = dd["S0"][:1].clone()
        o1 = torch.empty((1, H0, wd.dv), dtype=torch.bfloat16, device=dev)

        def step1(t):
            kda.decode_step(dd["q"][t][:1], dd["k"][t][:1], dd["v"][t][:1], dd["alpha"][t][:1], dd["beta"][t][:1],
                            st1, o=o1, o_dtype=torch.bfloat16)

        nst = args.decode_steps
        ms_eager = dtime(step1, reps=nst)
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for t in range(min(3, nst)):
                step1(t)
        gs.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for t in range(nst):
                step1(t)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / nst
        variants["decode_one_sequence_hip_graph"] = {
            "heads": H0, "steps": nst, "eager_ms_per_step": round(ms_eager, 4),
            "graph_ms_per_step": round(ms_graph, 4), "eager_over_graph": round(ms_eager / ms_graph, 2)}
        del graph, st1, o1
    del dd, state
    torch.cuda.empty_cache()

    calib = None
    if args.copy_calibration:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB: the reference
        # dispatch for scaling FETCH_SIZE / WRITE_SIZE, and the practical
        # read+write bandwidth of this GPU
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ce[0].record(stream)
        for _ in range(4):
            torch.mul(src, 2.0, out=dst)
        ce[1].record(stream)
        torch.cuda.synchronize()
        cms = ce[0].elapsed_time(ce[1]) / 4
        calib = {"kernel": "torch.mul fp32, 1 GiB in + 1 GiB out", "ms": round(cms, 4),
                 "GB/s": round(2 * (1 << 30) / (cms / 1e3) / 1e9, 1)}
        del src, dst

    # ---- CPU baseline (oracle) ------------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(host, w.heads)

    kernels = {"kda_intra_kernel": dict(intra_roof, ms_per_launch=round(intra_ms, 4)),
               "inter_chunk_pass": dict(inter_roof, ms_per_launch=round(inter_ms, 4), plan=plan),
               "kda_decode_kernel": dict(dec_roof, ms_per_launch=round(dec_ms, 4))}
    dominant = intra_roof if intra_ms >= inter_ms else inter_roof
    out = {
        "metric": METRIC,
        "value": round(tokens / (step_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_as_two_halves": round(halves_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"long-context prefill B{w.batch} H{w.heads} T{w.seqlen} dk=dv={w.dk} "
                               f"chunk {w.chunk} (bf16 q/k/v/o, fp32 alpha/beta/state; fp16 matrix-core "
                               "operands, fp32 accumulation)",
                   "batch": w.batch, "seq_len": w.seqlen, "heads": w.heads, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk},
        "roofline": dominant,
        "step_roofline": step_roof,
        "kernels": kernels,
        "decode": decode,
        "cpu_baseline": cpu,
        "variants": variants or None,
        "copy_calibration": calib,
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
