"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * gdn_chunk_fwd on the prefill workload (B=4, H=16, T=4096, d_k=d_v=128,
    bf16 q/k/v, fp32 state, chunk 64): gate, intra-chunk WY, state scan and
    output kernels, final state written;
  * gdn_decode_step on the decode workload (B=256, H=32, d=128, one bf16 token
    per sequence, fp32 state updated in place; the state comes from a
    512-token chunked forward over the seeded warm-up tokens).

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize(); each call is bracketed by HIP events on the stream
it runs on.  Before each call a 512 MiB scratch read evicts the 256 MB
last-level cache (outside the events), so inputs come from HBM.  The flush
reads rather than writes: a write flush leaves up to 256 MB of dirty lines in
the memory-side cache, and their write-back lands on whichever kernel runs
next (``--flush write`` measures that case, ``--flush none`` warm caches).

Prints ONE JSON line.  ``value`` is chunked-forward tokens/s (prefill tokens
per second of gdn_chunk_fwd); decode steps/s ride along in ``decode``.
``roofline`` is for the decode kernel, the dominant kernel of the step (one
kernel per call, so its event time is its launch duration); ``chunk_roofline``
gives the chunked forward's fractions of the HBM and bf16 MFMA peaks.
``cpu_baseline`` is the float64 oracle timed on this host's cores over the
whole prefill batch.

``long_context`` and ``varlen`` report the chunked forward's throughput on the
long-context workload (B=1, H=16, T=65536, log alpha / 64) and the packed
variable-length workload (32 sequences, the generator's lengths, 16 query/key
heads serving 32 value heads), timed the same way.  Their inputs are drawn on
the device from a seed with the generator's shapes and distributions (the
kernels' time does not depend on the values; the parity tests run these
workloads on the generator's exact inputs).

``block`` times the GDN block's prologue and epilogue kernels and a whole
block (prologue, chunked forward, epilogue) on the prefill shape with bf16
projections drawn on the device, and gives each kernel's algorithmic bytes
(every input read once, every output written once) as a fraction of HBM
peak.

``chunk_fwd_f32`` times the chunked forward with fp32 inputs on the prefill
shape (the chained form, every product on fp32 MFMA), with the algorithmic
flops as a fraction of the fp32 MFMA peak.

``chunk_bwd`` times the backward pass (gdn_chunk_bwd) on the prefill shape,
with its products' flops as a fraction of the fp32 MFMA peak (the backward
computes in fp32; with bf16 inputs some products run on the bf16 MFMA with
their fp32 factor split hi + lo, still counted here against the fp32 peak).

``kda_decode`` times the per-channel-gate decode step (one decay rate per key
channel) on the decode shape, with its HBM fraction.

``decode_graph`` times a 64-step batch-1 decode loop launched eagerly and
replayed as one captured HIP graph (host wall time per step).

``roofline.traffic`` is the decode kernel's HBM bytes per launch from the
rocprofv3 FETCH_SIZE and WRITE_SIZE counters (profiles/decode_kernel.traffic.json),
each scaled by what the counter reads for a plain 1 GiB read + 1 GiB write
elementwise kernel; it is null when the decode source has changed since the
counters were taken.  ``--calibrate-copy`` adds that plain kernel to the run
(and reports its bandwidth) so a counter pass over this script sees both.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15      # flop/s, dense bf16 MFMA
MFMA_F32_PEAK = 157.3e12     # flop/s, dense fp32 MFMA

# Algorithmic work (per unit = (sequence, value head); per token-unit):
# q, k, v, o in bf16 (4 x 128 x 2 bytes) + alpha, beta fp32 (8 bytes).
PREFILL_BYTES_PER_TOKEN_UNIT = 4 * 128 * 2 + 8
# Chunked delta-rule operations per token and head, C = 64, r = d = 128:
# 4 C r + 3 C d + 6 r d ("Attention as Matrix Algebra", section 8 and 9).
PREFILL_FLOPS_PER_TOKEN_UNIT = 4 * 64 * 128 + 3 * 64 * 128 + 6 * 128 * 128
# Decode per unit: state read + write (2 x 128 x 128 x 4 bytes), q k v o
# (4 x 128 x 2 bytes), alpha, beta (8 bytes).
DECODE_BYTES_PER_UNIT = 2 * 128 * 128 * 4 + 4 * 128 * 2 + 8
DECODE_FLOPS_PER_UNIT = 6 * 128 * 128


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel.traffic.json")
DECODE_SOURCE = os.path.join(ROOT, "gated_delta_rule_03_amd", "csrc", "decode.hip")


def decode_traffic():
    """Counter-measured HBM bytes per decode launch, if taken on this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(DECODE_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


CHUNK_COUNTERS_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_B4_H16_T4096_d128.counters.json")
CHUNK_SOURCES = {n: os.path.join(ROOT, "gated_delta_rule_03_amd", "csrc", n) for n in ("prep.hip", "scan.hip")}


def chunk_counters():
    """Counter figures of the prefill chunked forward's kernels (MFMA busy,
    MFMA flop, HBM bytes), if taken on the current prep.hip and scan.hip."""
    try:
        with open(CHUNK_COUNTERS_FILE) as f:
            rec = json.load(f)
        for name, path in CHUNK_SOURCES.items():
            with open(path, "rb") as f:
                if rec["source_sha256"].get(name) != hashlib.sha256(f.read()).hexdigest():
                    return None
    except (OSError, ValueError, KeyError):
        return None
    call = rec["call"]
    return {"mfma_busy_frac": call["mfma_busy_frac_time_weighted"], "mfma_flop_executed": call["mfma_flop"],
            "hbm_bytes": call["hbm_bytes"], "traffic_over_algorithmic": call["traffic_over_algorithmic"],
            "kernel_us": call["kernel_us"],
            "per_kernel_mfma_busy": {k: v["mfma_busy_frac"] for k, v in rec["kernels"].items()}}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, torch, dev):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, gi):
    """The oracle as it stands, on this host's cores: the whole prefill batch
    (the headline), and bounded samples of the other workloads, each timed
    on the float64 recurrence alone (not input generation).

    long context: all 16 heads over its first 8,192 tokens;
    packed batch: every head of its first 8 sequences;
    decode: one step of 32 of the 256 sequences (1,024 of 8,192 units) from a
    random fp32 state, and the 512-token warm-up forward of the same 1,024
    units.  Rates are per token of the full workload (a token carries every
    head) and, for decode, per full-batch step.
    """
    import oracle
    threads = oracle.cpu_threads()

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    dt = timed(lambda: oracle.forward(w.q, w.k, w.v, w.alpha, w.beta, return_o=True, threads=threads))
    tokens = w.B * w.T
    out = {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"whole prefill batch (B={w.B}, T={w.T}, H={w.spec.H_v}, d=128; "
                     f"{tokens * w.spec.H_v} token-units) in {dt:.2f} s, float64"}
    others = {}
    # long context, the first 8,192 tokens of all 16 heads
    wl = gi.generate(gi.config(4, T=8192, name="long-cpu-sample"))
    dt = timed(lambda: oracle.forward(wl.q, wl.k, wl.v, wl.alpha, wl.beta, return_o=True, threads=threads))
    units = wl.spec.H_v * wl.T
    others["long_context"] = {"tokens_per_s": wl.T / dt, "token_units_per_s": units / dt,
                              "sample": f"first {wl.T} of 65536 tokens, all 16 heads ({units} token-units) "
                                        f"in {dt:.2f} s"}
    # packed batch, first 8 sequences, all 32 heads
    wv = gi.generate(gi.config(5))
    sel = [(i, j) for i in range(8) for j in range(wv.spec.H_v)]
    n_tok = int(wv.cu_seqlens[8])
    dt = timed(lambda: oracle.forward(wv.q, wv.k, wv.v, wv.alpha, wv.beta, cu_seqlens=wv.cu_seqlens,
                                      units=sel, threads=threads))
    others["varlen"] = {"tokens_per_s": n_tok / dt, "token_units_per_s": n_tok * wv.spec.H_v / dt,
                        "sample": f"8 of 32 packed sequences ({n_tok} tokens x 32 heads) in {dt:.2f} s"}
    # decode: 32 of 256 sequences
    s3 = gi.config(3, B=32, name="decode-cpu-sample")
    wd = gi.generate(s3)
    state = gi.random_state((32, s3.H_v, 128, 128), seed=3, scale=0.3)
    dt = timed(lambda: oracle.decode(state, wd.q, wd.k, wd.v, wd.alpha, wd.beta, threads=threads))
    others["decode_step"] = {"steps_per_s": (32 * s3.H_v) / dt / 8192, "units_per_s": 32 * s3.H_v / dt,
                             "sample": f"one step of 32 of 256 sequences (1,024 units) in {dt:.3f} s"}
    ww = gi.generate(gi.decode_warmup_spec(s3))
    dt = timed(lambda: oracle.forward(ww.q, ww.k, ww.v, ww.alpha, ww.beta, return_o=False, threads=threads))
    others["decode_warmup"] = {"tokens_per_s": 32 * ww.T / dt, "token_units_per_s": 32 * ww.T * s3.H_v / dt,
                               "sample": f"512-token forward of 32 sequences x 32 heads in {dt:.2f} s"}
    out["other_workloads"] = others
    del wl, wv, wd, ww, state
    return out


def device_inputs(torch, dev, spec, n_tokens, B, seed):
    """Inputs with ``spec``'s shapes and distributions, drawn on the device.

    q, k ~ N(0, 1) scaled to unit length per token and head (q then by
    1/sqrt(d_k)), v ~ N(0, 1), rounded to bf16 (kept in fp32 for an fp32
    spec); log alpha = -softplus(N(0, 1))
    * A_h * s with A_h = exp(U(-4, 0)) per value head, beta = sigmoid(N(0, 1)).
    """
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    T = n_tokens // B
    q = torch.randn((B, T, spec.H_qk, spec.d_k), generator=g, device=dev)
    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    q = (torch.nn.functional.normalize(q, dim=-1) / spec.d_k ** 0.5).to(dt)
    k = torch.nn.functional.normalize(torch.randn((B, T, spec.H_qk, spec.d_k), generator=g, device=dev),
                                      dim=-1).to(dt)
    v = torch.randn((B, T, spec.H_v, spec.d_v), generator=g, device=dev).to(dt)
    A_h = torch.exp(torch.rand((spec.H_v,), generator=g, device=dev) * 4.0 - 4.0)
    z_a = torch.randn((B, T, spec.H_v), generator=g, device=dev)
    alpha = torch.exp(-torch.nn.functional.softplus(z_a) * A_h * spec.log_alpha_scale)
    beta = torch.sigmoid(torch.randn((B, T, spec.H_v), generator=g, device=dev))
    return q, k, v, alpha.float().contiguous(), beta.float().contiguous()


def timed_calls(args, torch, stream, evict, call):
    """Median seconds of ``call`` over several calls, each after an eviction."""
    ms = []
    for i in range(2 + max(3, args.steps // 4)):
        evict(4)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    return statistics.median(ms) * 1e-3


def extra_workloads(args, gi, gdn, torch, dev, stream, evict):
    """Chunked-forward throughput on the long-context and variable-length
    workloads.  The long-context workload is also timed through the
    segment-parallel form, as given (16 heads) and at two heads (one GPU's
    share of an eight-way head split), next to the one-pass scan; at two
    heads also with fp32 inputs (the chained kernels)."""
    out = {}
    cases = (("long_context", gi.config(4), None), ("long_context_2heads",
             gi.config(4, H_qk=2, H_v=2, name="long-2heads"), None),
             ("long_context_2heads_f32", gi.config(4, H_qk=2, H_v=2, dtype="f32", name="long-2heads-f32"), None),
             ("varlen", gi.config(5), None))
    for key, spec, _ in cases:
        if spec.packed_seqs:
            lengths = gi.packed_lengths(spec)
            n_tokens, B = int(sum(lengths)), 1
            cu = torch.tensor([0] + list(itertools.accumulate(lengths)), dtype=torch.int32, device=dev)
            n_seqs = len(lengths)
        else:
            n_tokens, B, cu, n_seqs = spec.B * spec.T, spec.B, None, spec.B
        log(f"bench: {spec.name} workload, {n_tokens} tokens")
        q, k, v, alpha, beta = device_inputs(torch, dev, spec, n_tokens, B, seed=spec.seed)
        o = torch.empty_like(v)
        hT = torch.empty((n_seqs, spec.H_v, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)
        n_arg = n_seqs if cu is not None else 0
        f32 = spec.dtype == "f32"
        dims = (B, n_tokens // B, spec.H_qk, spec.H_v, spec.d_k, spec.d_v, gdn.GDN_F32 if f32 else gdn.GDN_BF16,
                spec.chunk, n_arg)
        plan = gdn.chunk_fwd_plan_segments(*dims)
        # the one-pass scan, the planned form, and (long context) fixed segment lengths
        forms = [0] if plan == 0 else [0, plan]
        if key.startswith("long_context"):
            forms += [s for s in (32, 64, 128) if s not in forms]
        times = {}
        for seg in forms:
            need = gdn.chunk_fwd_segmented_workspace_bytes(*dims, seg)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def call():
                gdn.chunk_fwd(q, k, v, alpha, beta, chunk=spec.chunk, cu_seqlens=cu, o=o, hT=hT, workspace=ws,
                              seg_chunks=seg, stream=stream)

            times[seg] = timed_calls(args, torch, stream, evict, call)
            del ws
        t = times[plan]
        units = n_seqs * spec.H_v
        flops = n_tokens * spec.H_v * PREFILL_FLOPS_PER_TOKEN_UNIT
        esz = 4 if f32 else 2
        byts = n_tokens * (2 * spec.H_qk * spec.d_k * esz + 2 * spec.H_v * spec.d_v * esz + 8 * spec.H_v) + \
            units * spec.d_k * spec.d_v * 4
        out[key] = {"workload": f"{spec.name}: B={B} tokens={n_tokens} sequences={n_seqs} H_qk={spec.H_qk} "
                                f"H_v={spec.H_v} d={spec.d_k} {'fp32' if f32 else 'bf16'} chunk {spec.chunk}",
                    "tokens_per_s": n_tokens / t, "us_per_call": t * 1e6,
                    "hbm_frac": byts / t / HBM_PEAK,
                    ("mfma_f32_frac" if f32 else "mfma_frac"): flops / t / (MFMA_F32_PEAK if f32 else MFMA_BF16_PEAK),
                    "segment_chunks": plan,
                    "inputs": "drawn on the device with the generator's shapes and distributions"}
        if len(forms) > 1:
            out[key]["us_by_segment_chunks"] = {str(sg): tm * 1e6 for sg, tm in times.items()}
        del q, k, v, alpha, beta, o, hT
    return out


def kda_decode_workload(args, gdn, torch, dev, stream, evict, Dd, state):
    """The per-channel-gate decode step on the decode shape: the same q, k, v,
    beta and a copy of the state, with one decay rate per key channel."""
    B, _, H, D = Dd["v"].shape
    g = torch.Generator(device=dev)
    g.manual_seed(91)
    alpha = 0.8 + 0.2 * torch.rand((B, 1, H, D), generator=g, device=dev)
    st = state.clone()
    o = torch.empty_like(Dd["v"])
    ms = []
    for i in range(2 + max(3, args.steps // 2)):
        evict(6)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gdn.kda_decode_step(Dd["q"], Dd["k"], Dd["v"], alpha, Dd["beta"], st, o=o, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    t = statistics.median(ms) * 1e-3
    nbytes = B * H * (DECODE_BYTES_PER_UNIT + (D - 1) * 4)  # + the rates beyond one scalar
    del st
    return {"kda_decode": {
        "workload": f"per-channel gate decode step B={B} H={H} d={D} bf16, fp32 state in place",
        "us_per_step": t * 1e6, "bytes": nbytes, "GBps": nbytes / t / 1e9, "hbm_frac": nbytes / t / HBM_PEAK,
    }}


def kda_chunk_workload(args, gdn, gi, torch, dev, stream, evict):
    """The per-channel-gate chunked forward on the prefill shape (B=4, T=4096,
    H=16, d=128, bf16, chunk 64): q, k, v, beta as the prefill workload,
    one decay rate per key channel drawn uniform in [0.8, 1)."""
    spec = gi.config(2)
    B, T = spec.B, spec.T
    q, k, v, _, beta = device_inputs(torch, dev, spec, B * T, B, seed=spec.seed + 7)
    g = torch.Generator(device=dev)
    g.manual_seed(92)
    alpha = 0.8 + 0.2 * torch.rand((B, T, spec.H_v, spec.d_k), generator=g, device=dev)
    o = torch.empty_like(v)
    hT = torch.empty((B, spec.H_v, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.kda_chunk_fwd_workspace_bytes(B, T, spec.H_qk, spec.H_v, spec.d_k, spec.d_v, gdn.GDN_BF16,
                                                       64, 0), dtype=torch.uint8, device=dev)
    log("bench: per-channel-gate chunked forward, prefill shape")

    def call():
        gdn.kda_chunk_fwd(q, k, v, alpha, beta, chunk=64, o=o, hT=hT, workspace=ws, stream=stream)

    t = timed_calls(args, torch, stream, evict, call)
    tokens, units = B * T, B * spec.H_v
    # q, k, v, o in bf16, the rates (d_k fp32) and beta per token-unit, the final states
    nbytes = tokens * spec.H_v * (4 * 128 * 2 + 128 * 4 + 4) + units * 128 * 128 * 4
    flops = tokens * spec.H_v * PREFILL_FLOPS_PER_TOKEN_UNIT
    del q, k, v, alpha, beta, o, hT, ws
    return {"kda_chunk": {
        "workload": f"per-channel gate chunked forward B={B} T={T} H={spec.H_v} d=128 bf16 chunk 64",
        "tokens_per_s": tokens / t, "us_per_call": t * 1e6, "bytes": nbytes,
        "hbm_frac": nbytes / t / HBM_PEAK, "mfma_frac": flops / t / MFMA_BF16_PEAK,
    }}


def chunk_fwd_f32_workload(args, gdn, gi, torch, dev, stream, evict):
    """The chunked forward with fp32 inputs on the prefill shape (B=4, T=4096,
    H=16, d=128, chunk 64): the prefill workload's inputs widened to fp32.
    Off the bf16 staged path, this runs the chained form (every product on
    fp32 MFMA)."""
    spec = gi.config(2)
    B, T = spec.B, spec.T
    q, k, v, alpha, beta = device_inputs(torch, dev, spec, B * T, B, seed=spec.seed + 11)
    q, k, v = q.float(), k.float(), v.float()
    o = torch.empty_like(v)
    hT = torch.empty((B, spec.H_v, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.chunk_fwd_workspace_bytes(B, T, spec.H_qk, spec.H_v, spec.d_k, spec.d_v, gdn.GDN_F32,
                                                   64, 0), dtype=torch.uint8, device=dev)
    log("bench: chunked forward, fp32 inputs, prefill shape")

    def call():
        gdn.chunk_fwd(q, k, v, alpha, beta, chunk=64, o=o, hT=hT, workspace=ws, stream=stream)

    t = timed_calls(args, torch, stream, evict, call)
    tokens, units = B * T, B * spec.H_v
    # q, k, v, o in fp32, alpha and beta per token-unit, the final states
    nbytes = tokens * spec.H_v * (4 * 128 * 4 + 8) + units * 128 * 128 * 4
    flops = tokens * spec.H_v * PREFILL_FLOPS_PER_TOKEN_UNIT
    del q, k, v, alpha, beta, o, hT, ws
    return {"chunk_fwd_f32": {
        "workload": f"chunked forward B={B} T={T} H={spec.H_v} d=128 fp32 inputs, chunk 64",
        "tokens_per_s": tokens / t, "us_per_call": t * 1e6, "bytes": nbytes, "flops": flops,
        "hbm_frac": nbytes / t / HBM_PEAK, "mfma_f32_frac": flops / t / MFMA_F32_PEAK,
    }}


def chunk_bwd_workload(args, gdn, gi, torch, dev, stream, evict):
    """The backward pass (gdn_chunk_bwd) on the prefill shape (B=4, T=4096,
    H=16, d=128, bf16, chunk 64): the prefill workload's inputs and an
    upstream gradient d_o ~ N(0, 1) in bf16; all gradients in fp32."""
    spec = gi.config(2)
    B, T = spec.B, spec.T
    q, k, v, alpha, beta = device_inputs(torch, dev, spec, B * T, B, seed=spec.seed + 9)
    g = torch.Generator(device=dev)
    g.manual_seed(93)
    d_o = torch.randn((B, T, spec.H_v, spec.d_v), generator=g, device=dev).bfloat16()
    ws = torch.empty(gdn.chunk_bwd_workspace_bytes(B, T, spec.H_qk, spec.H_v, spec.d_k, spec.d_v, gdn.GDN_BF16,
                                                   64, 0), dtype=torch.uint8, device=dev)
    log("bench: backward pass, prefill shape")

    def call():
        gdn.chunk_bwd(q, k, v, alpha, beta, d_o, chunk=64, workspace=ws, stream=stream)

    t = timed_calls(args, torch, stream, evict, call)
    del q, k, v, alpha, beta, d_o, ws
    # products per (chunk of 64, value head), triangular ones at half size:
    # 8 C d_k d_v (K S, the state update, K dS', the two dS terms, dO S^T,
    # dY S^T, U dS'^T) + 2.5 C^2 d_v (T X, P^T dO, M^T dU, dO U^T, dY U^T)
    # + 3 C^2 d_k (K K^T, Q K^T, (dP.Gamma) K, (dP.Gamma)^T Q, (dG + dG^T) K)
    C, dk, dv = 64, spec.d_k, spec.d_v
    flops = 2 * (8 * C * dk * dv + 2.5 * C * C * dv + 3 * C * C * dk) * (T // C) * B * spec.H_v
    return {"chunk_bwd": {
        "workload": f"backward pass B={B} T={T} H={spec.H_v} d=128 bf16 inputs, fp32 gradients, chunk 64",
        "tokens_per_s": B * T / t, "us_per_call": t * 1e6, "flops": flops,
        "mfma_f32_frac": flops / t / MFMA_F32_PEAK,
    }}


def decode_graph_workload(args, gdn, torch, dev, stream):
    """A serving loop of 64 decode steps at batch 1 (H=32, d=128, bf16), launched
    eagerly and as one captured HIP graph: the per-step time shows the launch
    overhead that a graph removes at this size."""
    steps, B, H, D = 64, 1, 32, 128
    g = torch.Generator(device=dev)
    g.manual_seed(93)
    ops = []
    for _ in range(steps):
        q = torch.randn((B, 1, H, D), generator=g, device=dev)
        k = torch.nn.functional.normalize(torch.randn((B, 1, H, D), generator=g, device=dev), dim=-1)
        ops.append(((q * D ** -0.5).bfloat16(), k.bfloat16(), torch.randn((B, 1, H, D), generator=g, device=dev).bfloat16(),
                    0.9 + 0.1 * torch.rand((B, 1, H), generator=g, device=dev),
                    torch.rand((B, 1, H), generator=g, device=dev)))
    state = torch.zeros((B, H, D, D), device=dev)
    outs = [torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=dev) for _ in range(steps)]

    def loop():
        for s_ in range(steps):
            gdn.decode_step(*ops[s_], state, o=outs[s_])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()

    def timed(fn, reps=5):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts) / steps
    loop()
    t_eager = timed(loop)
    t_graph = timed(graph.replay)
    return {"decode_graph": {
        "workload": f"{steps} decode steps, B={B} H={H} d={D} bf16, host wall time per step",
        "eager_us_per_step": t_eager * 1e6, "graph_us_per_step": t_graph * 1e6,
    }}


def block_workload(args, gdn, torch, dev, stream, evict):
    """The block prologue and epilogue kernels, and a whole block (prologue,
    chunked forward, epilogue), on the prefill shape with bf16 projections."""
    B, T, H, D = 4, 4096, 16, 128
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    rn = lambda *shape: torch.randn(shape, generator=g, device=dev)
    q_raw, k_raw, v_raw, g_raw = (rn(B, T, H, D).bfloat16() for _ in range(4))
    conv = [0.5 * rn(H * D, 4) for _ in range(3)]
    bias = [0.1 * rn(H * D) for _ in range(3)]
    a_raw, b_raw = rn(B, T, H), rn(B, T, H)
    log_A = torch.log(torch.rand(H, generator=g, device=dev) * 15.5 + 0.5)
    nw = 1.0 + 0.1 * rn(D)
    outs = (torch.empty_like(q_raw), torch.empty_like(k_raw), torch.empty_like(v_raw),
            torch.empty((B, T, H), device=dev), torch.empty((B, T, H), device=dev))
    o = torch.empty_like(v_raw)
    y = torch.empty_like(v_raw)
    hT = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.chunk_fwd_workspace_bytes(B, T, H, H, D, D, gdn.GDN_BF16, 64, 0), dtype=torch.uint8,
                     device=dev)

    def prologue():
        gdn.block_prologue(q_raw, k_raw, v_raw, *conv, a_raw, b_raw, log_A, conv_q_bias=bias[0],
                           conv_k_bias=bias[1], conv_v_bias=bias[2], v_norm_weight=nw, q_scale=D ** -0.5,
                           out=outs, stream=stream)

    def epilogue():
        gdn.block_epilogue(o, g_raw, o_norm_weight=nw, y=y, stream=stream)

    def whole():
        prologue()
        q, k, v, al, be = outs
        gdn.chunk_fwd(q, k, v, al, be, chunk=64, o=o, hT=hT, workspace=ws, stream=stream)
        epilogue()

    def timed(fn):
        ms = []
        for i in range(2 + max(3, args.steps // 2)):
            evict(5)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        return statistics.median(ms) * 1e-3

    tokens = B * T
    row = H * D * 2  # one token's projections of one tensor, bf16
    pro_bytes = tokens * (3 * row * 2 + H * 4 * 4)  # q, k, v in and out; a, b in; alpha, beta out
    epi_bytes = tokens * 3 * row                    # o, g in; y out
    t_pro, t_epi, t_all = timed(prologue), timed(epilogue), timed(whole)
    return {"block": {
        "workload": f"B={B} T={T} H={H} d={D} bf16 projections (q/k/v convolution width 4)",
        "prologue_us": t_pro * 1e6, "prologue_GBps": pro_bytes / t_pro / 1e9,
        "prologue_hbm_frac": pro_bytes / t_pro / HBM_PEAK, "prologue_bytes": pro_bytes,
        "epilogue_us": t_epi * 1e6, "epilogue_GBps": epi_bytes / t_epi / 1e9,
        "epilogue_hbm_frac": epi_bytes / t_epi / HBM_PEAK, "epilogue_bytes": epi_bytes,
        "whole_block_us": t_all * 1e6, "whole_block_tokens_per_s": tokens / t_all,
    }}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read",
                    help="what runs before each call to evict the last-level cache")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long-context and variable-length throughput lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by (sequence, head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_03_amd as gdn
    import gdn_inputs as gi

    dev = torch.device("cuda:0")
    gdn.load()

    # ---------------- inputs, resident in HBM before timing ----------------
    log("bench: generating prefill inputs")
    wp = gi.generate(gi.config(2))
    P = {n: to_dev(getattr(wp, n), torch, dev) for n in ("q", "k", "v", "alpha", "beta")}
    B, T, H, D = wp.B, wp.T, wp.spec.H_v, wp.spec.d_k
    o_p = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    hT_p = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    need = gdn.chunk_fwd_workspace_bytes(B, T, H, H, D, D, gdn.GDN_BF16, 64, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    log("bench: decode state from a 512-token chunked forward over the seeded warm-up")
    spec3 = gi.config(3)
    warm = gi.generate(gi.decode_warmup_spec(spec3))
    Wd = {n: to_dev(getattr(warm, n), torch, dev) for n in ("q", "k", "v", "alpha", "beta")}
    _, state = gdn.chunk_fwd(Wd["q"], Wd["k"], Wd["v"], Wd["alpha"], Wd["beta"], chunk=64)
    del Wd, warm
    wd = gi.generate(spec3)
    Dd = {n: to_dev(getattr(wd, n), torch, dev) for n in ("q", "k", "v", "alpha", "beta")}
    o_d = torch.empty((spec3.B, 1, spec3.H_v, spec3.d_v), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    flush = None if args.flush == "none" else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def evict(tag):
        if flush is None:
            return
        if args.flush == "write":
            flush.fill_(tag)
        else:
            torch.sum(flush.view(torch.int64), dim=0, keepdim=True, out=flush_sink)

    def chunk_call():
        gdn.chunk_fwd(P["q"], P["k"], P["v"], P["alpha"], P["beta"], chunk=64, o=o_p, hT=hT_p,
                      workspace=ws, stream=stream)

    def decode_call():
        gdn.decode_step(Dd["q"], Dd["k"], Dd["v"], Dd["alpha"], Dd["beta"], state, o=o_d,
                        stream=stream)

    def step(record):
        evict(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        chunk_call()
        e1.record(stream)
        evict(2)
        e2 = torch.cuda.Event(enable_timing=True)
        e3 = torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        decode_call()
        e3.record(stream)
        record.append((e0, e1, e2, e3))

    log(f"bench: {args.warmup} warm-up steps")
    rec = []
    for _ in range(args.warmup):
        step(rec)
    torch.cuda.synchronize()
    rec = []
    log(f"bench: {args.steps} timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    chunk_ms = [a.elapsed_time(b) for a, b, _, _ in rec]
    dec_ms = [c.elapsed_time(d) for _, _, c, d in rec]
    chunk_s = statistics.median(chunk_ms) * 1e-3
    dec_s = statistics.median(dec_ms) * 1e-3
    dec_mean_s = statistics.fmean(dec_ms) * 1e-3

    copy_gbps = None
    if args.calibrate_copy:
        log("bench: calibration copy, 1 GiB read + 1 GiB write")
        c_src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        c_dst = torch.empty_like(c_src)
        cms = []
        for _ in range(3):
            evict(3)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.mul(c_src, 1.0, out=c_dst)
            e1.record(stream)
            torch.cuda.synchronize()
            cms.append(e0.elapsed_time(e1))
        copy_gbps = 2 * c_src.numel() * 4 / (statistics.median(cms) * 1e-3) / 1e9
        del c_src, c_dst

    extra = {}
    if not args.no_extra:
        extra = extra_workloads(args, gi, gdn, torch, dev, stream, evict)
        extra.update(block_workload(args, gdn, torch, dev, stream, evict))
        extra.update(kda_decode_workload(args, gdn, torch, dev, stream, evict, Dd, state))
        extra.update(kda_chunk_workload(args, gdn, gi, torch, dev, stream, evict))
        extra.update(chunk_fwd_f32_workload(args, gdn, gi, torch, dev, stream, evict))
        extra.update(chunk_bwd_workload(args, gdn, gi, torch, dev, stream, evict))
        extra.update(decode_graph_workload(args, gdn, torch, dev, stream))

    tokens = B * T
    units = B * H
    prefill_bytes = tokens * H * PREFILL_BYTES_PER_TOKEN_UNIT + units * D * D * 4
    prefill_flops = tokens * H * PREFILL_FLOPS_PER_TOKEN_UNIT
    dec_units = spec3.B * spec3.H_v
    dec_bytes = dec_units * DECODE_BYTES_PER_UNIT

    result = {
        "metric": "GDN chunked-fwd tokens/s (H=16,d=128,T=4096) + decode steps/s; % roofline",
        "value": tokens / chunk_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (chunk_s + dec_s) * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "chunked forward B=4 H=16 T=4096 d_k=d_v=128 bf16 chunk 64 "
                        "+ decode step B=256 H=32 d=128 (fp32 state in place)",
            "global_batch": B, "seq_len": T, "heads": H, "head_dim": D, "chunk": 64,
            "decode_batch": spec3.B, "decode_heads": spec3.H_v,
            "cache": {"none": "warm", "read": "cold (512 MiB read before each call)",
                      "write": "cold (512 MiB write before each call)"}[args.flush],
        },
        "decode": {
            "steps_per_s": 1.0 / dec_s,
            "tokens_per_s": spec3.B / dec_s,
            "us_per_step": dec_s * 1e6,
            "hbm_frac": dec_bytes / dec_s / HBM_PEAK,
        },
        "chunk_fwd": {
            "us_per_call": chunk_s * 1e6,
            "us_p10": float(np.percentile(chunk_ms, 10)) * 1e3,
            "us_p90": float(np.percentile(chunk_ms, 90)) * 1e3,
        },
        "roofline": {
            "kernel": "decode_kernel<bf16>",
            "bound": "hbm",
            "achieved": dec_bytes / dec_mean_s / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": dec_bytes / dec_mean_s / HBM_PEAK,
            "traffic": decode_traffic(),
        },
        "chunk_roofline": {
            "algorithmic_bytes": prefill_bytes,
            "algorithmic_flops": prefill_flops,
            "hbm_frac": prefill_bytes / chunk_s / HBM_PEAK,
            "mfma_frac": prefill_flops / chunk_s / MFMA_BF16_PEAK,
            "achieved_GBps": prefill_bytes / chunk_s / 1e9,
            "achieved_TFLOPs": prefill_flops / chunk_s / 1e12,
            "counters": chunk_counters(),
        },
        "wall_s_timed_region": wall,
    }
    result.update(extra)
    if copy_gbps is not None:
        result["calibration_copy_GBps"] = copy_gbps
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (float64 oracle on host cores)")
        result["cpu_baseline"] = cpu_baseline(wp, gi)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
