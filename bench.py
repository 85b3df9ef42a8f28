"""Benchmark of the KDA core on one MI355X.

One step = one ``kda_chunk_fwd`` call over the varlen_64 workload (64 packed
sequences, lengths U{128..16384}, 530,033 tokens, H=32, d_k=d_v=128, chunk 64,
bf16 q/k/v/z/beta, per-sequence fp32 initial and final states) with its inputs
already resident in HBM: the largest prefill configuration that fits one GPU.
The prefill_8k and prefill_128k configurations, the decode workload (512
sequences x 32 heads, fp32 state of 1 GiB updated in place, 64 steps with
fresh inputs), the speculative window and the fused layer are timed alongside.
Prints one JSON line.

Roofline figures use algorithmic counts per (token, head) at d = 128, C = 64
(derived from eq. (1) and the chunkwise form of eqs. (3)-(4) of "Kimi K3
Technical Report: Open Frontier Intelligence" §2.1.1):
  prefill bytes  = 5 x 256 (q, k, v, z, o in bf16) + 2 (beta) = 1282, plus the
                   fp32 initial and final state per (sequence, head);
  prefill FLOPs  = 6 d_k d_v + (3C - 1) d_k + 2C d_v = 139136;
  decode bytes   = 2 x 64 KiB (fp32 state read + write) + 1282.
Timing uses HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_delta_rule_20_amd as kda  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix, published (no sparsity)
METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode state-update % HBM BW"


def prefill_counts(T, H, Dk, Dv, N, C=64, elem=2):
    per_tok_bytes = elem * (3 * Dk + 2 * Dv) + elem          # q, k, z, v, o + beta
    state_bytes = 2 * N * H * Dk * Dv * 4                     # h0 read + hT write
    flops = (6 * Dk * Dv + (3 * C - 1) * Dk + 2 * C * Dv) * T * H
    return per_tok_bytes * T * H + state_bytes, flops


def decode_counts(N, H, Dk, Dv, elem=2):
    return N * H * (2 * Dk * Dv * 4 + elem * (3 * Dk + 2 * Dv) + elem), N * H * 7 * Dk * Dv


_C_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def source_digest(files):
    """First 16 hex digits of sha256 over the listed csrc files with comments
    removed and whitespace collapsed (string literals kept), so that a change
    to a comment does not retire a profile taken on the same code.  None if a
    file is missing."""
    h = hashlib.sha256()
    for f in files:
        src = os.path.join(ROOT, "gated_delta_rule_20_amd", "csrc", f)
        if not os.path.exists(src):
            return None
        with open(src) as fh:
            h.update(code_tokens(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def code_tokens(text):
    """C/C++ source with // and /* */ comments removed (string and character
    literals kept as written) and every run of whitespace made one space."""
    text = _C_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(text.split())


def profiled_traffic(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (copy-calibrated), read from profiles/hbm_traffic_pmc.txt.  Returns None
    when the kernel sources no longer match the digest that was profiled."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_pmc.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if not line.startswith("record "):
            continue
        fields = dict(kv.split("=", 1) for kv in line.split()[1:])
        if fields.get("name") != name:
            continue
        d = source_digest(fields["files"].split(","))
        return int(fields["traffic_bytes"]) if d is not None and d == fields["digest"] else None
    return None


def time_calls(fn, n, stream):
    """Run fn(i) n times, each bracketed by HIP events on `stream`; returns
    (per-call ms list, wall ms of the whole region)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def bench_prefill(steps, warmup, n_sets=3, ckpt_every=0, name="prefill_8k", keep_inputs=False):
    """One kda_chunk_fwd call per step over a prefill workload (fixed-length or
    packed).  n_sets independent input sets rotate so that no step reads the
    previous step's inputs from the 256 MB last-level cache (one set is enough
    once a set is many times that size).  ckpt_every > 0 also writes a
    prefix-state checkpoint every ckpt_every chunks (slots for the whole
    sequence)."""
    w = W.WORKLOADS[name]
    import dataclasses
    sets = []
    for i in range(n_sets):
        inp = W.make_prefill(dataclasses.replace(w, seed=w.seed + 17 * i), device="cuda")
        cu = inp["cu_seqlens"]
        N = cu.numel() - 1 if cu is not None else inp["q"].shape[0]
        o = torch.empty_like(inp["v"])
        hT = torch.empty_like(inp["h0"])
        nws = kda.chunk_fwd_workspace_size(inp["q"], inp["v"], cu_seqlens=cu, N=N if cu is not None else None)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        ck = None
        if ckpt_every > 0:
            B, T, H, Dk = inp["q"].shape
            slots = max(1, T // (64 * ckpt_every))
            ck = torch.empty((B, slots, H, Dk, inp["v"].shape[-1]), dtype=torch.float32, device="cuda")
        sets.append((inp, o, hT, ws, ck))
    stream = torch.cuda.current_stream()

    def call(i):
        inp, o, hT, ws, ck = sets[i % n_sets]
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], A_log=inp["A_log"],
                      g_min=inp["g_min"], cu_seqlens=inp["cu_seqlens"], initial_state=inp["h0"], out=o,
                      final_state=hT, workspace=ws, stream=stream, checkpoints=ck, checkpoint_every=ckpt_every)

    for i in range(warmup):
        call(i)
    per_call, wall = time_calls(call, steps, stream)
    inp0 = sets[0][0]
    tokens = W.n_tokens(inp0)
    H, Dk = inp0["q"].shape[-2:]
    Dv = inp0["v"].shape[-1]
    N = inp0["h0"].shape[0]
    nbytes, flops = prefill_counts(tokens, H, Dk, Dv, N)
    ms = sum(per_call) / len(per_call)
    n_ck = 0
    if ckpt_every > 0:  # slots strictly inside the sequence are written
        T = inp0["q"].shape[1]
        n_ck = N * H * min(sets[0][4].shape[1], (T - 1) // (64 * ckpt_every))
    out = dict(ms=ms, ms_min=min(per_call), ms_median=statistics.median(per_call), wall_ms=wall, tokens=tokens,
               sequences=N, bytes=nbytes + 4 * Dk * Dv * n_ck, flops=flops, shape=(tokens, H, Dk, Dv),
               checkpoint_states=n_ck)
    if keep_inputs:
        out["inputs"] = inp0
    del sets
    return out


def prefill_line(r, kernel, traffic_name):
    """Throughput, HBM roofline and MFMA-rate figures of one prefill measurement."""
    sec = r["ms"] / 1e3
    achieved = r["bytes"] / sec / 1e9
    tflops = r["flops"] / sec / 1e12
    return {
        "ms_per_call": r["ms"], "ms_min": r["ms_min"], "ms_median": r["ms_median"],
        "tokens": r["tokens"], "sequences": r["sequences"], "tokens_per_s": r["tokens"] / sec,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(traffic_name),
                     "algorithmic_bytes": r["bytes"]},
        "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "algorithmic_flops": r["flops"]},
    }


def bench_decode(warmup_rounds=1):
    w = W.WORKLOADS["decode_512"]
    d = W.make_decode(w, device="cuda")
    state = d["state"]
    steps = d["steps"]
    outs = [torch.empty_like(st["v"]) for st in steps]
    stream = torch.cuda.current_stream()

    def call(i):
        st = steps[i]
        kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=d["A_log"],
                           g_min=d["g_min"], out=outs[i], stream=stream)

    for _ in range(warmup_rounds):
        for i in range(len(steps)):
            call(i)
    per_call, wall = time_calls(call, len(steps), stream)
    N, H, Dk = steps[0]["q"].shape
    Dv = steps[0]["v"].shape[-1]
    nbytes, flops = decode_counts(N, H, Dk, Dv)
    us = 1e3 * sum(per_call) / len(per_call)
    return dict(us=us, us_min=1e3 * min(per_call), us_median=1e3 * statistics.median(per_call), steps=len(steps),
                N=N, H=H, bytes=nbytes, flops=flops)


def spec_counts(N, H, Dk, Dv, n_replayed, T_new, elem=2):
    """Algorithmic bytes of one replay call: the state read and written once, the
    replayed tokens' k, g, v, beta, and the new window's q, k, g, v, beta and o."""
    state = 2 * N * H * Dk * Dv * 4
    replay = n_replayed * H * (2 * Dk + Dv + 1) * elem
    new = N * T_new * H * (3 * Dk + 2 * Dv + 1) * elem
    return state + replay + new


def bench_spec(T_new=4, calls=None, warmup_rounds=1):
    """decode_512_spec: one replay call per speculative step (fresh inputs per call)."""
    w = W.WORKLOADS["decode_512_spec"]
    d = W.make_spec_decode(w, device="cuda", T_new=T_new, calls=calls)
    state = d["state"]
    cl = d["calls"]
    outs = [torch.empty_like(c["v"]) for c in cl]
    stream = torch.cuda.current_stream()

    def call(i):
        c = cl[i]
        kda.recurrent_replay(c["q"], c["k"], c["v"], c["z"], c["beta"], state,
                             replay=(c["k_r"], c["v_r"], c["z_r"], c["beta_r"]), n_replay=c["n_replay"],
                             n_commit=1, A_log=d["A_log"], g_min=d["g_min"], out=outs[i], stream=stream)

    for _ in range(warmup_rounds):
        for i in range(len(cl)):
            call(i)
    per_call, _ = time_calls(call, len(cl), stream)
    N, T, H, Dk = cl[0]["q"].shape
    Dv = cl[0]["v"].shape[-1]
    n_rep = sum(int(c["n_replay"].sum()) for c in cl) / len(cl)
    nbytes = spec_counts(N, H, Dk, Dv, n_rep, T)
    us = 1e3 * sum(per_call) / len(per_call)
    return dict(us=us, us_median=1e3 * statistics.median(per_call), us_min=1e3 * min(per_call), calls=len(cl),
                N=N, H=H, T_new=T, T_replay=cl[0]["k_r"].shape[1], mean_replayed=n_rep / N, bytes=nbytes)


def layer_counts(tokens, N, H, Dk, Dv, W=4, elem=2):
    """Algorithmic bytes of the fused layer: per (token, head) the projections
    q, k, v before the convolution, the decay logits z, the beta logit, the gate
    logits and the output (eq. (2) and eq. (6) inputs and output); per
    (sequence, head) the fp32 state read and written and the convolution state
    read and written; the filters once."""
    per_tok = elem * (3 * Dk + 3 * Dv) + elem
    per_seq = 2 * Dk * Dv * 4 + 2 * (W - 1) * (2 * Dk + Dv) * elem
    return per_tok * tokens * H + per_seq * N * H + H * (2 * Dk + Dv) * W * 4 + H * Dv * 4


def bench_layer_prefill(steps, warmup, n_sets=3):
    """prefill_8k shapes through the fused layer (prologue and epilogue in the kernels)."""
    import dataclasses
    w = W.WORKLOADS["prefill_8k"]
    sets = []
    for i in range(n_sets):
        d = W.make_layer(dataclasses.replace(w, seed=w.seed + 17 * i), "cuda", N=w.B, T=w.T, H=w.H)
        f = kda.Fusion(conv_weight=d["conv_weight"], conv_state=d["conv_state"],
                       conv_state_out=torch.empty_like(d["conv_state"]), qk_eps=1e-6, gate=d["gate"],
                       o_norm_weight=d["o_norm_weight"], o_eps=1e-6)
        nws = kda.chunk_fwd_workspace_size(d["q_pre"], d["v_pre"], prologue=True)
        sets.append((d, f, torch.empty_like(d["v_pre"]), torch.empty_like(d["state"]),
                     torch.empty(nws, dtype=torch.uint8, device="cuda")))
    stream = torch.cuda.current_stream()

    def call(i):
        d, f, o, hT, ws = sets[i % n_sets]
        kda.chunk_fwd(d["q_pre"], d["k_pre"], d["v_pre"], d["z"], d["beta_logit"], A_log=d["A_log"],
                      g_min=d["g_min"], initial_state=d["state"], out=o, final_state=hT, workspace=ws,
                      stream=stream, fusion=f)

    for i in range(warmup):
        call(i)
    per_call, _ = time_calls(call, steps, stream)
    B, T, H, Dk = sets[0][0]["q_pre"].shape
    Dv = sets[0][0]["v_pre"].shape[-1]
    ms = sum(per_call) / len(per_call)
    nbytes = layer_counts(B * T, B, H, Dk, Dv)
    return dict(ms=ms, ms_min=min(per_call), ms_median=statistics.median(per_call), tokens=B * T, bytes=nbytes,
                shape=(B, T, H, Dk, Dv))


def bench_layer_decode(warmup_rounds=1, steps=64):
    """decode_512 shapes through the fused layer: 64 steps with fresh inputs,
    the recurrent and convolution states updated in place."""
    w = W.WORKLOADS["decode_512"]
    d = W.make_layer(w, "cuda", N=w.B, T=steps, H=w.H)
    per = [{n: d[n][:, t].contiguous() for n in ("q_pre", "k_pre", "v_pre", "z", "beta_logit", "gate")}
           for t in range(steps)]
    for n in ("q_pre", "k_pre", "v_pre", "z", "beta_logit", "gate"):
        del d[n]
    state, cs = d["state"], d["conv_state"]
    fus = [kda.Fusion(conv_weight=d["conv_weight"], conv_state=cs, qk_eps=1e-6, gate=x["gate"],
                      o_norm_weight=d["o_norm_weight"], o_eps=1e-6) for x in per]
    outs = [torch.empty_like(x["v_pre"]) for x in per]
    stream = torch.cuda.current_stream()

    def call(i):
        x = per[i]
        kda.recurrent_step(x["q_pre"], x["k_pre"], x["v_pre"], x["z"], x["beta_logit"], state, A_log=d["A_log"],
                           g_min=d["g_min"], out=outs[i], stream=stream, fusion=fus[i])

    for _ in range(warmup_rounds):
        for i in range(steps):
            call(i)
    per_call, _ = time_calls(call, steps, stream)
    N, H, Dk = per[0]["q_pre"].shape
    Dv = per[0]["v_pre"].shape[-1]
    us = 1e3 * sum(per_call) / len(per_call)
    return dict(us=us, us_min=1e3 * min(per_call), us_median=1e3 * statistics.median(per_call), steps=steps,
                N=N, H=H, bytes=layer_counts(N, N, H, Dk, Dv))


def layer_spec_counts(N, H, Dk, Dv, n_replayed, T_new, W=4, elem=2):
    """Algorithmic bytes of one fused replay call: the fp32 state and the
    convolution state read and written once; per replayed token its q, k, v
    projections, z and beta logit (q only feeds the convolution); per new token
    the same plus the gate logits and the output; the filters once."""
    C = 2 * Dk + Dv
    state = 2 * N * H * Dk * Dv * 4 + 2 * N * H * (W - 1) * C * elem
    replay = n_replayed * H * (2 * Dk + Dv + Dk + 1) * elem
    new = N * T_new * H * (3 * Dk + 3 * Dv + 1) * elem
    return state + replay + new + H * C * W * 4 + H * Dv * 4


def bench_layer_spec(T_new=4, calls=16, warmup_rounds=1):
    """decode_512_spec shapes through the fused layer: per call the accepted
    drafts of a cached window are replayed and a new window (bonus + drafts)
    runs, both from pre-convolution projections with the eq. (2) prologue and
    the eq. (6) epilogue in the kernel; the recurrent and convolution states
    are updated in place at the bonus token (fresh inputs per call)."""
    w = W.WORKLOADS["decode_512_spec"]
    Tr = w.T - 1
    base = W.make_layer(w, "cuda", N=w.B, T=1, H=w.H)
    state, cs = base["state"], base["conv_state"]
    cpu = torch.Generator().manual_seed(w.seed + 7)
    lo, hi = w.len_range
    names = ("q_pre", "k_pre", "v_pre", "z", "beta_logit")
    cl = []
    for i in range(calls):
        d = W.make_layer(w, "cuda", N=w.B, T=Tr + T_new, H=w.H, seed_offset=i + 1)
        del d["state"]
        x = {f"{n}_r": d[n][:, :Tr].contiguous() for n in names}
        x.update({n: d[n][:, Tr:].contiguous() for n in names})
        x["gate"] = d["gate"][:, Tr:].contiguous()
        x["n_replay"] = torch.randint(lo, hi + 1, (w.B,), generator=cpu, dtype=torch.int32).to("cuda")
        cl.append(x)
        del d
    fus = [kda.Fusion(conv_weight=base["conv_weight"], conv_state=cs, qk_eps=1e-6, gate=x["gate"],
                      o_norm_weight=base["o_norm_weight"], o_eps=1e-6) for x in cl]
    outs = [torch.empty_like(x["v_pre"]) for x in cl]
    stream = torch.cuda.current_stream()

    def call(i):
        x = cl[i]
        kda.recurrent_replay(x["q_pre"], x["k_pre"], x["v_pre"], x["z"], x["beta_logit"], state,
                             replay=(x["k_pre_r"], x["v_pre_r"], x["z_r"], x["beta_logit_r"]),
                             n_replay=x["n_replay"], n_commit=1, A_log=base["A_log"], g_min=base["g_min"],
                             q_r=x["q_pre_r"], out=outs[i], stream=stream, fusion=fus[i])

    for _ in range(warmup_rounds):
        for i in range(calls):
            call(i)
    per_call, _ = time_calls(call, calls, stream)
    N, T, H, Dk = cl[0]["q_pre"].shape
    Dv = cl[0]["v_pre"].shape[-1]
    n_rep = sum(int(x["n_replay"].sum()) for x in cl) / calls
    us = 1e3 * sum(per_call) / len(per_call)
    return dict(us=us, us_median=1e3 * statistics.median(per_call), us_min=1e3 * min(per_call), calls=calls,
                N=N, H=H, T_new=T, T_replay=Tr, mean_replayed=n_rep / N,
                bytes=layer_spec_counts(N, H, Dk, Dv, n_rep, T))


def copy_calibration(steps, nbytes=1 << 30):
    """A plain device-to-device copy of known size (for scaling the HBM
    FETCH_SIZE / WRITE_SIZE counters: it reads and writes nbytes each)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    per_call, _ = time_calls(lambda i: dst.copy_(src), steps, stream)
    ms = sum(per_call) / len(per_call)
    return {"copy_bytes_each_way": nbytes, "ms": ms, "GBps_read_plus_write": 2 * nbytes / (ms / 1e3) / 1e9}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(inp, max_threads=16, min_seconds=10.0, max_seconds=30.0):
    """The fp64 oracle on the host cores over the headline workload, streamed
    one head at a time (every packed sequence of that head in one oracle call,
    OpenMP over the sequences), heads taken in order until at least
    min_seconds of oracle time have accumulated or every head is done, and
    stopped early once max_seconds would be passed.  Only the oracle calls are
    timed (not the copies to the host).  Reported as tokens/s of the whole
    workload: (token-heads per second) / H.  Reported baseline only."""
    import oracle
    cu = inp["cu_seqlens"]
    H = inp["q"].shape[-2]
    flat = lambda t: t.reshape((-1,) + tuple(t.shape[-2:])) if t.dim() == 4 else t
    q, k, v, z = (flat(inp[x]) for x in ("q", "k", "v", "z"))
    b = inp["beta"].reshape(-1, H)
    T = q.shape[0]
    cu_np = (cu.to("cpu", torch.int64).numpy() if cu is not None
             else (torch.arange(inp["q"].shape[0] + 1, dtype=torch.int64) * inp["q"].shape[1]).numpy())
    N = cu_np.size - 1
    threads = min(max_threads, os.cpu_count() or 1)
    host = lambda t: t.detach().to("cpu", torch.float64).numpy()
    total, used, heads = 0.0, threads, 0
    for h in range(H):
        sl = slice(h, h + 1)
        args = [host(x[:, sl]) for x in (q, k, v, z)] + [host(b[:, sl])]
        h0 = host(inp["h0"][:, sl])
        A = host(inp["A_log"][sl])
        t0 = time.perf_counter()
        _, _, used = oracle.forward(*args, cu_seqlens=cu_np, h0=h0, A_log=A, g_min=inp["g_min"], nthreads=threads,
                                    return_threads=True)
        dt = time.perf_counter() - t0
        total, heads = total + dt, heads + 1
        if total >= min_seconds or total * (heads + 1) / heads > max_seconds:
            break
    return {"value": T * heads / H / total, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{heads} of {H} heads of the headline workload ({N} sequences, {T} tokens each head), "
                      f"fp64, {total:.1f} s of oracle time, scaled to all {H} heads",
            "host_cpus": os.cpu_count(), "host_cpu_model": cpu_model()}


def measured_peaks():
    """Peaks measured on this device as references beside the published ones:
    a bf16 GEMM at 8192^3 (torch.matmul, hipBLASLt) and a 1 GiB device copy."""
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b_ = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        torch.matmul(a, b_)
    per_call, _ = time_calls(lambda i: torch.matmul(a, b_), 10, stream)
    gemm_ms = statistics.median(per_call)
    del a, b_
    cp = copy_calibration(10)
    return {"bf16_gemm_8192_tflops": 2 * 8192 ** 3 / (gemm_ms / 1e3) / 1e12,
            "copy_1GiB_read_plus_write_gbs": cp["GBps_read_plus_write"]}


def log(msg):
    """Progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


PREFILL_KERNELS = ("kda_chunk_fwd (from 128 (sequence, head) pairs at bf16, d_k = 128: intra_chunk_kernel in pair "
                   "mode, the chain inside it; below: intra_chunk_kernel + chain_kernel; chunk_table_kernel for "
                   "packed input)")
HEADLINE = "varlen_64"


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured GEMM / copy reference peaks")
    ap.add_argument("--no-spec", action="store_true", help="skip the speculative-decoding replay measurement")
    ap.add_argument("--no-other", action="store_true", help="skip the prefill_8k and prefill_128k measurements")
    ap.add_argument("--no-layer", action="store_true", help="skip the fused-layer (prologue / epilogue) measurements")
    ap.add_argument("--mode", choices=["all", "varlen", "prefill", "prefill128k", "decode", "spec", "layer", "copy"],
                    default="all",
                    help="every mode but 'all' runs one part only (for profiler runs: varlen = the headline "
                         "varlen_64 call, prefill = prefill_8k); the JSON line of the benchmark contract is "
                         "printed in mode 'all'")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    kda.load_library()
    if args.mode == "copy":
        print(json.dumps(copy_calibration(args.steps)))
        return
    if args.mode == "decode":
        dc = bench_decode()
        print(json.dumps({k: v for k, v in dc.items()}))
        return
    if args.mode == "spec":
        print(json.dumps(bench_spec()))
        return
    if args.mode == "layer":
        lp = bench_layer_prefill(args.steps, args.warmup)
        ld = bench_layer_decode()
        ls = bench_layer_spec()
        print(json.dumps({"prefill_ms": lp["ms"], "decode_us": ld["us"], "spec_us": ls["us"]}))
        return
    if args.mode in ("varlen", "prefill", "prefill128k"):
        name = {"varlen": "varlen_64", "prefill": "prefill_8k", "prefill128k": "prefill_128k"}[args.mode]
        r = bench_prefill(args.steps, args.warmup, n_sets=3 if name == "prefill_8k" else 1, name=name)
        print(json.dumps({"workload": name, "ms": r["ms"], "ms_min": r["ms_min"],
                          "tokens_per_s": r["tokens"] / (r["ms"] / 1e3)}))
        return

    # headline: the largest prefill configuration (530,033 packed tokens; one input set of ~17 GB
    # is far larger than the 256 MB last-level cache, so no rotation is needed)
    hv = bench_prefill(args.steps, args.warmup, n_sets=1, name=HEADLINE, keep_inputs=not args.no_cpu_baseline)
    line = prefill_line(hv, PREFILL_KERNELS, "varlen")
    log(f"{HEADLINE}: {hv['ms']:.3f} ms per call")
    tokens, H, Dk, Dv = hv["shape"]
    result = {
        "metric": METRIC,
        "value": line["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hv["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"varlen_64: {hv['sequences']} packed sequences (cu_seqlens), lengths U{{128..16384}}, "
                               f"{tokens} tokens, H={H} d_k={Dk} d_v={Dv} chunk=64, bf16 q/k/v/z/beta, per-sequence "
                               "fp32 initial+final states, eq.(5) gate in-kernel",
                   "global_batch": hv["sequences"], "seq_len": tokens, "parallelism": "none (1 GPU)"},
        "roofline": line["roofline"],
        "mfma": line["mfma"],
        "ms_min": hv["ms_min"],
        "ms_median": hv["ms_median"],
        "wall_ms": hv["wall_ms"],
    }
    inputs = hv.pop("inputs", None)
    pf = None
    if not args.no_other:
        pf = bench_prefill(args.steps, args.warmup, n_sets=3, name="prefill_8k")
        result["prefill_8k"] = {"workload": "prefill_8k: B=1 T=8192 H=32 d=128 chunk=64, bf16, fp32 initial+final "
                                            "state; three input sets rotate", **prefill_line(pf, PREFILL_KERNELS, "prefill")}
        ck = bench_prefill(args.steps, args.warmup, ckpt_every=8, name="prefill_8k")
        result["prefill_with_checkpoints"] = {
            "workload": "prefill_8k with a prefix-state checkpoint every 8 chunks (512 tokens), fp32 slots",
            "ms_per_step": ck["ms"], "ms_median": ck["ms_median"], "tokens_per_s": ck["tokens"] / (ck["ms"] / 1e3),
            "checkpoint_states_written": ck["checkpoint_states"],
            "hbm_GBps": ck["bytes"] / (ck["ms"] / 1e3) / 1e9, "algorithmic_bytes": ck["bytes"],
            "overhead_vs_plain": ck["ms"] / pf["ms"] - 1.0,
        }
        log(f"prefill_8k: {pf['ms'] * 1e3:.1f} us per call, with checkpoints {ck['ms'] * 1e3:.1f} us")
        p128 = bench_prefill(max(3, args.steps // 4), 1, n_sets=1, name="prefill_128k")
        log(f"prefill_128k: {p128['ms']:.3f} ms per call")
        result["prefill_128k"] = {"workload": "prefill_128k: B=1 T=131072 H=32 d=128, 5% of decay channels forced "
                                              "each way", **prefill_line(p128, PREFILL_KERNELS, "prefill128k")}
        torch.cuda.empty_cache()
    if not args.no_decode:
        dc = bench_decode()
        log(f"decode_512: {dc['us']:.1f} us per step")
        gbs = dc["bytes"] / (dc["us"] / 1e6) / 1e9
        result["decode"] = {
            "workload": f"decode_512: N={dc['N']} x 1 token, H={dc['H']}, d=128, fp32 state 1 GiB in place, "
                        f"{dc['steps']} steps with fresh inputs",
            "us_per_step": dc["us"], "us_min": dc["us_min"], "us_median": dc["us_median"],
            "tokens_per_s": dc["N"] / (dc["us"] / 1e6),
            "roofline": {"bound": "hbm", "kernel": "replay_kernel (one-token window)", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": profiled_traffic("decode"), "algorithmic_bytes": dc["bytes"]},
        }
    if not args.no_spec:
        sp = bench_spec()
        gbs = sp["bytes"] / (sp["us"] / 1e6) / 1e9
        window = {}
        for tn in (1, 2, 4, 8):
            r = bench_spec(T_new=tn, calls=8)
            window[str(tn)] = round(r["us"], 1)
        log(f"decode_512_spec: {sp['us']:.1f} us per call; by new window {window}")
        result["spec_decode"] = {
            "workload": f"decode_512_spec: N={sp['N']}, H={sp['H']}, d=128, cached drafts {sp['T_replay']} "
                        f"(mean {sp['mean_replayed']:.2f} accepted and replayed), new window {sp['T_new']} "
                        f"(bonus + drafts), bonus committed, {sp['calls']} calls with fresh inputs",
            "us_per_call": sp["us"], "us_median": sp["us_median"], "us_min": sp["us_min"],
            # committed per call and sequence: the accepted drafts replayed plus the bonus token
            "committed_tokens_per_s": sp["N"] * (sp["mean_replayed"] + 1) / (sp["us"] / 1e6),
            "roofline": {"bound": "hbm", "kernel": "replay_kernel", "achieved": gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": profiled_traffic("spec"),
                         "algorithmic_bytes": sp["bytes"]},
            "us_per_call_by_new_window": window,
        }
    if not args.no_layer:
        lp = bench_layer_prefill(args.steps, args.warmup)
        ld = bench_layer_decode()
        ls = bench_layer_spec()
        lp_gbs = lp["bytes"] / (lp["ms"] / 1e3) / 1e9
        ld_gbs = ld["bytes"] / (ld["us"] / 1e6) / 1e9
        ls_gbs = ls["bytes"] / (ls["us"] / 1e6) / 1e9
        log(f"layer: prefill {lp['ms'] * 1e3:.1f} us, decode {ld['us']:.1f} us, spec {ls['us']:.1f} us")
        B_, T_, H_, Dk_, Dv_ = lp["shape"]
        result["layer"] = {
            "what": "eq. (2) prologue (ShortConv width 4, Swish, L2Norm, Sigmoid beta) and eq. (6) epilogue "
                    "(RMSNorm, Sigmoid output gate) fused around the recurrence; dense projections not included",
            "prefill": {"workload": f"prefill_8k shapes (B={B_} T={T_} H={H_} d={Dk_}) from pre-convolution "
                                    "projections, bf16", "ms_per_call": lp["ms"], "ms_median": lp["ms_median"],
                        "tokens_per_s": lp["tokens"] / (lp["ms"] / 1e3),
                        "vs_core_call": lp["ms"] / pf["ms"] if pf else None,
                        "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd with fusion", "achieved": lp_gbs,
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lp_gbs / HBM_PEAK_GBS,
                                     "traffic": profiled_traffic("layer_prefill"), "algorithmic_bytes": lp["bytes"]}},
            "decode": {"workload": f"decode_512 shapes (N={ld['N']} x 1 token, H={ld['H']}, d=128), fp32 state and "
                                   f"bf16 convolution state in place, {ld['steps']} steps with fresh inputs",
                       "us_per_step": ld["us"], "us_median": ld["us_median"],
                       "tokens_per_s": ld["N"] / (ld["us"] / 1e6),
                       "roofline": {"bound": "hbm", "kernel": "replay_kernel (fused variant, one-token window)",
                                    "achieved": ld_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": ld_gbs / HBM_PEAK_GBS, "traffic": profiled_traffic("layer_decode"),
                                    "algorithmic_bytes": ld["bytes"]}},
            "spec": {"workload": f"decode_512_spec shapes (N={ls['N']}, H={ls['H']}, d=128): cached drafts "
                                 f"{ls['T_replay']} (mean {ls['mean_replayed']:.2f} accepted and replayed), new "
                                 f"window {ls['T_new']}, bonus committed, {ls['calls']} calls with fresh inputs",
                     "us_per_call": ls["us"], "us_median": ls["us_median"], "us_min": ls["us_min"],
                     "roofline": {"bound": "hbm", "kernel": "replay_kernel (fused variant)", "achieved": ls_gbs,
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ls_gbs / HBM_PEAK_GBS,
                                  "traffic": profiled_traffic("layer_spec"), "algorithmic_bytes": ls["bytes"]}},
        }
        torch.cuda.empty_cache()
    if not args.no_peaks:
        pk = measured_peaks()
        log(f"measured peaks: {pk}")
        result["measured_peaks"] = pk
        result["roofline"]["frac_of_measured_copy"] = result["roofline"]["achieved"] / pk["copy_1GiB_read_plus_write_gbs"]
        result["mfma"]["frac_of_measured_gemm"] = result["mfma"]["achieved"] / pk["bf16_gemm_8192_tflops"]
        if "decode" in result:
            d = result["decode"]["roofline"]
            d["frac_of_measured_copy"] = d["achieved"] / pk["copy_1GiB_read_plus_write_gbs"]
    if not args.no_cpu_baseline and inputs is not None:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(inputs)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.0f} tokens/s on {result['cpu_baseline']['cores']} threads")
    print(json.dumps(result))


if __name__ == "__main__":
    main()
