"""Benchmark of the Gated DeltaNet layer core on one MI355X.

One step = one gdn_layer_core call (prologue + recurrence, every step of the
hot path) over the prefill workload: B=1, T=4096, Hk=16, Hv=32, Dk=Dv=128,
conv K=4, zero conv and recurrent state, seeded synthetic inputs resident in
HBM before timing.  The timed steps rotate over 4 sets of inputs and outputs
(qkv, a, b, y, state and conv-state outputs: 401 MB together, more than the
256 MB last-level cache), so each step reads inputs the previous steps did
not leave in that cache; the single-set (warm) step time is reported beside
it.  Before the warm-up, 0.3 s of untimed steps bring the GPU to its loaded
clock state (its first milliseconds of work run measurably slower).
Metric: recurrence tokens/s*head = B*T*Hv / step time.

Also measured in the same run (same JSON line):
  * roofline of the timed step (its two launches: the chunk preparation with
    the prologue fused in, and the sequential pass): algorithmic fp32 flops
    against the fp32 peak, computed on the matrix cores (the f32 matrix
    instruction for W S^T, bf16 products of exact plane splits elsewhere);
    the f32 and bf16 matrix flops those launches issue (rocprofv3 counters,
    committed under profiles/) against those peaks; HBM traffic;
  * the chunked recurrence alone (one gdn_recurrent_chunked call on prepared
    inputs), the same roofline;
  * a plain device copy (read + write) as the practical HBM ceiling;
  * batched decode, B=64, T=1 (layer core, 8 rotating sets of state and conv
    state, 1 GiB, so the 256 MB last-level cache cannot hold them) -> HBM
    roofline of its recurrence kernel;
  * the prologue kernel and the output epilogue (gated RMS normalisation of
    y, gdn_gated_rmsnorm) on the prefill workload, each over 4 rotating
    buffer sets larger together than the last-level cache -> HBM roofline;
    and the gated layer core (gdn_layer_core_gated) step time;
  * single-token decode B=1 (per-call time, warm and cold, marshalled once,
    replayed from a HIP graph) beside the floor of a plain copy of its 2 MiB
    state in the same graph form, and the long batched prefill B=4, T=32768
    (layer core and chunked recurrence);
  * a speculative-verify window (B=64, T=4, state emitted after 1..4 steps)
    and per-key-gate decode (B=64, T=1), both HBM-bound, rotating state sets;
  * the CPU oracle on a bounded sample of the prefill workload, one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_prep_amd", "csrc")
KERNEL_SOURCES = {
    "layer_core": ["chunked.hip"],
    "chunked_recurrence": ["chunked.hip"],
    "recurrent_chunk_kernel": ["recurrent.hip"],
    "recurrent_step_kernel": ["recurrent.hip"],
    "prep_kernel": ["prep.hip"],
    "gated_rmsnorm_kernel": ["epilogue.hip"],
}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector alike)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix
F32_MATRIX_PEAK_TFLOPS = 157.3 # MI355X dense f32 matrix
R_HBM = 4                      # rotating buffer sets for the HBM-bound kernels
R_IN = 4                       # rotating input/output sets of the timed prefill step
SETTLE_S = 0.3                 # untimed steps before the warm-up: the GPU's loaded clock state


def source_digest(kernel):
    """sha256 of a kernel's source file and the shared device headers."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["gdn_device.h", "gdn_launch.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_counter(kernel, workload, key="traffic_bytes"):
    """A per-launch figure from the committed counter summary
    (profiles/traffic.txt: HBM traffic bytes, or issued bf16 matrix flops),
    or None when the kernel's source changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            kv = dict(x.split("=", 1) for x in line.split())
            if kv.get("kernel") == kernel and kv.get("workload") == workload and key in kv:
                if kv.get("source_sha256") != source_digest(kernel):
                    return None
                return int(kv[key])
    return None


def measured_traffic(kernel, workload):
    return measured_counter(kernel, workload, "traffic_bytes")


def host_cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else the platform string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-long", action="store_true", help="skip the B=4 T=32768 long-prefill leg")
    ap.add_argument("--kernel-only", default=None,
                    choices=[None, "recurrent", "prep", "decode", "copy", "chunked", "epilogue", "layer", "verify",
                             "per_key_decode", "long", "per_key"],
                    help="launch only this kernel (for counter collection)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path needs no collectives; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_recurrence_prep_amd import binding, inputs

    assert torch.cuda.is_available(), "no GPU visible"
    binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.kernel_only == "long":       # the long-prefill layer-core step alone
        bench_long_prefill(args, torch, dev, up, inputs, binding, np, launches=max(args.steps, 1))
        return
    if args.kernel_only == "per_key":    # the per-key chunked recurrence alone
        bench_per_key_prefill(args, torch, dev, up, inputs, binding, np, launches=max(args.steps, 1))
        return

    # ------------------------------------------------------------ prefill
    w = inputs.WORKLOADS["prefill"]
    B, T, Hk, Hv, Dk, Dv, K = (w[k] for k in ("B", "T", "Hk", "Hv", "Dk", "Dv", "K"))
    C = 2 * Hk * Dk + Hv * Dv
    qs, ks = inputs.scales(Dk)
    eps = 1e-6
    raw = inputs.workload("prefill")
    d = {k: up(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state")}
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    s_out = torch.empty(B, Hv, Dv, Dk, dtype=torch.float32, device=dev)
    cs_out = torch.empty(B, K - 1, C, dtype=torch.int16, device=dev)
    ws = torch.empty(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), dtype=torch.uint8,
                     device=dev)
    # the timed step's rotating sets: the same inputs in fresh buffers, own outputs
    in_sets = [dict(qkv=d["qkv"].clone(), a=d["a"].clone(), b=d["b"].clone(), y=torch.empty_like(y),
                    s=torch.empty_like(s_out), cs=torch.empty_like(cs_out)) for _ in range(R_IN)]

    def step(i=None):
        if i is None:      # the single resident set (warm)
            binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                               d["dt_bias"], d["state"], s_out, y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                               q_scale=qs, k_scale=ks, eps=eps)
            return
        x = in_sets[i % R_IN]
        binding.layer_core(x["qkv"], d["conv_w"], d["conv_state"], x["cs"], x["a"], x["b"], d["A_log"],
                           d["dt_bias"], d["state"], x["s"], x["y"], ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                           q_scale=qs, k_scale=ks, eps=eps)

    # prologue outputs for timing the recurrence kernel alone
    pq = torch.empty(B, T, Hk, Dk, dtype=torch.int16, device=dev)
    pk = torch.empty_like(pq)
    pv = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    pg = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    pb = torch.empty_like(pg)

    def prep_only():
        binding.prep(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                     d["dt_bias"], pq, pk, pv, pg, pb, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs,
                     k_scale=ks, eps=eps)

    def rec_only():
        binding.recurrent(pq, pk, pv, pg, pb, None, s_out, y)

    cws = torch.empty(max(binding.recurrent_chunked_workspace_bytes(B, T, Hk, Hv, Dk, Dv), 1),
                      dtype=torch.uint8, device=dev)

    def chunked_only():
        binding.recurrent_chunked(pq, pk, pv, pg, pb, None, s_out, y, cws)

    # the output epilogue (gated RMS normalisation of y) on the same workload
    gate = inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=w["id"], with_y=False)
    gz, gw = up(gate["z"]), up(gate["norm_weight"])
    out = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)

    # The HBM-bound kernels are timed over R_HBM rotating buffer sets (each
    # >= 100 MB, together more than the 256 MB last-level cache), so every
    # launch streams its operands from HBM rather than from that cache.
    prep_sets = [dict(qkv=d["qkv"].clone(), q=torch.empty_like(pq), k=torch.empty_like(pk),
                      v=torch.empty_like(pv), g=torch.empty_like(pg), b=torch.empty_like(pb))
                 for _ in range(R_HBM)]

    def prep_rot(i):
        p_ = prep_sets[i % R_HBM]
        binding.prep(p_["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                     d["dt_bias"], p_["q"], p_["k"], p_["v"], p_["g"], p_["b"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                     q_scale=qs, k_scale=ks, eps=eps)

    epi_sets = [dict(y=torch.empty_like(y), z=gz.clone(), out=torch.empty_like(out)) for _ in range(R_HBM)]

    def epilogue_rot(i):
        e_ = epi_sets[i % R_HBM]
        binding.gated_rmsnorm(e_["y"], e_["z"], gw, e_["out"], eps=eps)

    def step_gated():
        binding.layer_core_gated(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                                 d["dt_bias"], gz, gw, d["state"], s_out, out, ws, Hk=Hk, Hv=Hv, Dk=Dk,
                                 Dv=Dv, q_scale=qs, k_scale=ks, eps=eps, norm_eps=eps)

    prep_only()
    torch.cuda.synchronize()

    if args.kernel_only:
        return kernel_only(args, torch, dev, prep_rot, rec_only, up, inputs, binding, np, chunked_only,
                           epilogue_rot, epi_sets, y, step)

    # Settle: the GPU runs its first milliseconds of work at lower clocks
    # (measured: the same step takes about 191 us in its first 40 calls and
    # about 167 us from then on), so untimed steps run for SETTLE_S seconds
    # (synchronised every 20 steps, so the queue never runs ahead) before the
    # warm-up and the timed steps.
    t_settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle0 < SETTLE_S:
        for _ in range(20):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle0
    for i in range(max(args.warmup, R_IN)):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] prefill settle {n_settle} steps ({settle_s:.2f} s), warmup done ({max(args.warmup, R_IN)})",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    value = B * T * Hv / (ms_step * 1e-3)
    warm_us = time_kernel(torch, stream, step, args.steps)
    print(f"[bench] prefill layer core {ms_step * 1e3:.1f} us/step ({R_IN} rotating sets), "
          f"{warm_us:.1f} us/step warm (one set)", file=sys.stderr, flush=True)

    # dominant work alone, events on the stream it runs on: the chunked
    # recurrence (chunk_prep_kernel + chunk_seq_kernel), then for reference
    # the per-step form the layer core uses for short sequences, and the prologue
    chunk_us = time_kernel(torch, stream, chunked_only, args.steps)
    step_form_us = time_kernel(torch, stream, rec_only, max(3, args.steps // 4))
    prep_us = time_rotating(torch, stream, prep_rot, max(args.steps, 2 * R_HBM))
    for e_ in epi_sets:
        e_["y"].copy_(y)            # the layer core's y as the epilogue's input
    epi_us = time_rotating(torch, stream, epilogue_rot, max(args.steps, 2 * R_HBM))
    gated_us = time_kernel(torch, stream, step_gated, args.steps)
    epi_bytes = 3 * B * T * Hv * Dv * 2 + Dv * 2
    flops = 7 * B * T * Hv * Dk * Dv
    achieved_tflops = flops / (chunk_us * 1e-6) / 1e12
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    copy = bench_copy(torch, dev, stream)
    rec_bytes = (2 * B * T * Hk * Dk * 2 + B * T * Hv * Dv * 2 + 2 * B * T * Hv * 4 + B * T * Hv * Dv * 2
                 + B * Hv * Dv * Dk * 4)
    prep_bytes = (B * T * C * 2 + C * K * 2 + 2 * B * T * Hv * 2 + 2 * Hv * 4 + 2 * B * T * Hk * Dk * 2
                  + B * T * Hv * Dv * 2 + 2 * B * T * Hv * 4 + B * (K - 1) * C * 2)
    print(f"[bench] layer core step {step_tflops:.1f} TFLOP/s ({step_tflops / FP32_PEAK_TFLOPS:.1%} of fp32 peak); "
          f"device copy {copy['GBs_1GiB']:.0f} GB/s", file=sys.stderr, flush=True)
    print(f"[bench] chunked recurrence {chunk_us:.1f} us ({achieved_tflops:.1f} TFLOP/s, "
          f"{achieved_tflops / FP32_PEAK_TFLOPS:.1%} of fp32 peak); per-step form {step_form_us:.1f} us; "
          f"prep kernel {prep_us:.1f} us ({prep_bytes / prep_us / 1e3:.0f} GB/s)", file=sys.stderr, flush=True)
    print(f"[bench] epilogue {epi_us:.1f} us ({epi_bytes / epi_us / 1e3:.0f} GB/s); "
          f"gated layer core {gated_us:.1f} us/step", file=sys.stderr, flush=True)

    # ------------------------------------------------------------- decode
    decode = bench_decode(args, torch, dev, up, inputs, binding, np)
    serving = bench_verify_and_per_key(args, torch, dev, up, inputs, binding, np)
    decode1 = bench_decode_b1(args, torch, dev, up, inputs, binding, np)
    per_key_prefill = bench_per_key_prefill(args, torch, dev, up, inputs, binding, np)
    long_prefill = None if args.no_long else bench_long_prefill(args, torch, dev, up, inputs, binding, np)

    # -------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(raw, Hk, Hv, Dk, Dv, qs, ks, eps)

    line = {
        "metric": "recurrence tokens/s*head (prefill T=4096, layer core incl. prologue)",
        "value": value,
        "unit": "token*head/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 q/k/v/y storage)",
        "data": "synthetic (seeded)",
        "config": {"workload": "prefill B=1 T=4096 Hk=16 Hv=32 Dk=Dv=128 K=4, zero conv/recurrent state",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": roofline_step(flops, ms_step * 1e3, step_tflops, B, T, Hk, Hv, Dk, Dv, C, K),
        "recurrence_chunked_alone": {
            "kernel": "chunk_prep_kernel<0, 2> + chunk_seq_kernel<1> (gdn_recurrent_chunked on prepared q/k/v/g/beta)",
            "avg_launch_us": chunk_us, "achieved": achieved_tflops, "unit": "TFLOP/s",
            "frac_fp32": achieved_tflops / FP32_PEAK_TFLOPS,
            "traffic": measured_traffic("chunked_recurrence", "prefill_T4096"), "traffic_algorithmic": rec_bytes,
            "bf16_matrix_flops": measured_counter("chunked_recurrence", "prefill_T4096", "mfma_bf16_flops"),
            "f32_matrix_flops": measured_counter("chunked_recurrence", "prefill_T4096", "mfma_f32_flops")},
        "prefill_warm_us_per_step": warm_us,
        "device_copy": copy,
        "recurrence_per_step_form": {"kernel": "recurrent_chunk_kernel<128,32>", "avg_launch_us": step_form_us,
                                     "achieved_TFLOPs": flops / (step_form_us * 1e-6) / 1e12},
        "prologue": {"kernel": "prep_kernel<128,4>", "avg_launch_us": prep_us,
                     "buffers": f"{R_HBM} rotating sets (inputs and outputs exceed the last-level cache)",
                     "bytes_per_launch": prep_bytes, "achieved_GBs": prep_bytes / prep_us / 1e3,
                     "traffic": measured_traffic("prep_kernel", "prefill_T4096"),
                     "frac_hbm": prep_bytes / prep_us / 1e3 / HBM_PEAK_GBS},
        "epilogue": {"kernel": "gated_rmsnorm_kernel<16,1>", "avg_launch_us": epi_us,
                     "buffers": f"{R_HBM} rotating sets (inputs and outputs exceed the last-level cache)",
                     "bytes_per_launch": epi_bytes, "achieved_GBs": epi_bytes / epi_us / 1e3,
                     "traffic": measured_traffic("gated_rmsnorm_kernel", "prefill_T4096"),
                     "frac_hbm": epi_bytes / epi_us / 1e3 / HBM_PEAK_GBS,
                     "layer_core_gated_us": gated_us},
        "decode_b64": decode,
        "decode_b1": decode1,
        "long_prefill_b4": long_prefill,
        "verify_window_b64": serving["verify_window"],
        "per_key_decode_b64": serving["per_key_decode"],
        "per_key_prefill_b1": per_key_prefill,
        "cpu_baseline": cpu,
        "wall_s_timed": t_wall,
        "settle": {"steps": n_settle, "seconds": settle_s,
                   "note": "untimed steps before the warm-up, bringing the GPU to its loaded clock state"},
    }
    print(json.dumps(line), flush=True)


def roofline_step(flops, step_us, step_tflops, B, T, Hk, Hv, Dk, Dv, C, K):
    """Roofline of the timed step (its two launches).  The work is fp32
    arithmetic, 7 Dk Dv flop per token*head, computed on the matrix cores:
    W S^T on the f32 matrix instruction, the other products in bf16 on exact
    plane splits of the f32 operands.  The algorithmic fp32 rate against the
    fp32 peak, and the f32 and bf16 matrix flops the launches issue (counters)
    against those peaks."""
    mf = measured_counter("layer_core", "prefill_T4096", "mfma_bf16_flops")
    mf32 = measured_counter("layer_core", "prefill_T4096", "mfma_f32_flops")
    # algorithmic bytes: qkv, a, b, conv weights read; y, state, conv-state tail written
    alg = B * T * C * 2 + 2 * B * T * Hv * 2 + C * K * 2 + B * T * Hv * Dv * 2 + B * Hv * Dv * Dk * 4 \
        + B * (K - 1) * C * 2
    return {"bound": "mfma", "kernel": "chunk_prep_kernel<4, 2> + chunk_seq_kernel<1> (gdn_layer_core step)",
            "dtype": "fp32 arithmetic on matrix cores (f32 instruction; bf16 on exact plane splits)",
            "achieved": step_tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": step_tflops / FP32_PEAK_TFLOPS,
            "traffic": measured_traffic("layer_core", "prefill_T4096"), "traffic_algorithmic": alg,
            "flops_per_launch": flops, "avg_launch_us": step_us,
            "bf16_matrix": None if mf is None else {
                "flops_per_launch": mf, "achieved": mf / (step_us * 1e-6) / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": mf / (step_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS},
            "f32_matrix": None if mf32 is None else {
                "flops_per_launch": mf32, "achieved": mf32 / (step_us * 1e-6) / 1e12, "peak": F32_MATRIX_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": mf32 / (step_us * 1e-6) / 1e12 / F32_MATRIX_PEAK_TFLOPS}}


def bench_copy(torch, dev, stream):
    """A plain device copy (read + write), the practical HBM ceiling: 256 MiB
    and 1 GiB buffers, two destinations alternating."""
    out = {}
    for name, nbytes in (("256MiB", 256 << 20), ("1GiB", 1 << 30)):
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = [torch.empty_like(src) for _ in range(2)]
        ctr = iter(range(1 << 30))
        us = time_kernel(torch, stream, lambda: dst[next(ctr) % 2].copy_(src), 10)
        out[f"GBs_{name}"] = 2 * nbytes / us / 1e3
        del src, dst
    out["note"] = "torch copy_ of a device buffer, bytes read + written per microsecond"
    return out


def time_rotating(torch, stream, fn, n):
    """Average launch time of fn(i), i = 0..n-1 (fn rotates buffer sets)."""
    for i in range(R_HBM):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def time_kernel(torch, stream, fn, n, warm=5):
    """Average time of fn() over n back-to-back calls, after warm untimed
    calls (a freshly allocated set of buffers runs its first calls slower)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def bench_decode(args, torch, dev, up, inputs, binding, np):
    """Batched decode B=64, T=1 through the layer core, rotating 8 state sets."""
    B, T, Hk, Hv, Dk, Dv, K = 64, 1, 16, 32, 128, 128, 4
    C = 2 * Hk * Dk + Hv * Dv
    qs, ks = inputs.scales(Dk)
    R = 8
    raw = inputs.layer_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K, workload_id=2, state=True,
                           conv_state=True)
    common = {k: up(raw[k]) for k in ("conv_w", "A_log", "dt_bias")}
    sets = []
    for r in range(R):
        sets.append(dict(qkv=up(raw["qkv"]).clone(), a=up(raw["a"]).clone(), b=up(raw["b"]).clone(),
                         cs=up(raw["conv_state"]).clone(), st=up(raw["state"]).clone()))
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    ws = torch.empty(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), dtype=torch.uint8,
                     device=dev)
    # recurrence kernel alone: q,k,v,g,beta prepared once per set
    pq = torch.empty(B, T, Hk, Dk, dtype=torch.int16, device=dev)
    pk, pv = torch.empty_like(pq), torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    pg = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    pb = torch.empty_like(pg)
    binding.prep(sets[0]["qkv"], common["conv_w"], sets[0]["cs"], None, sets[0]["a"], sets[0]["b"],
                 common["A_log"], common["dt_bias"], pq, pk, pv, pg, pb, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                 q_scale=qs, k_scale=ks)

    def step(i):
        s = sets[i % R]
        binding.layer_core(s["qkv"], common["conv_w"], s["cs"], s["cs"], s["a"], s["b"], common["A_log"],
                           common["dt_bias"], s["st"], s["st"], y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                           q_scale=qs, k_scale=ks)

    def rec(i):
        s = sets[i % R]
        binding.recurrent(pq, pk, pv, pg, pb, s["st"], s["st"], y)

    stream = torch.cuda.current_stream(dev)
    n = args.decode_steps
    out = {}
    for name, fn in (("layer_core", step), ("recurrent", rec)):
        for i in range(2 * R):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        out[name] = a.elapsed_time(b) * 1e3 / n
    state_bytes = 2 * B * Hv * Dv * Dk * 4
    rec_bytes = state_bytes + 2 * B * T * Hk * Dk * 2 + 2 * B * T * Hv * Dv * 2 + 2 * B * T * Hv * 4
    core_bytes = (state_bytes + B * T * C * 2 + 2 * B * (K - 1) * C * 2 + C * K * 2 + 2 * B * T * Hv * 2
                  + B * T * Hv * Dv * 2)
    gbs = rec_bytes / out["recurrent"] / 1e3
    print(f"[bench] decode B=64: layer core {out['layer_core']:.1f} us, recurrent kernel "
          f"{out['recurrent']:.1f} us ({gbs:.0f} GB/s)", file=sys.stderr, flush=True)
    return {
        "workload": "decode B=64 T=1 Hk=16 Hv=32 Dk=Dv=128, 8 rotating state sets (1 GiB)",
        "value": B * T * Hv / (out["layer_core"] * 1e-6),
        "unit": "token*head/s",
        "us_per_step": out["layer_core"],
        "layer_core_GBs": core_bytes / out["layer_core"] / 1e3,
        "roofline": {"bound": "hbm", "kernel": "recurrent_step_kernel<128, false, false>", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("recurrent_step_kernel", "decode_B64"),
                     "bytes_per_launch": rec_bytes, "avg_launch_us": out["recurrent"]},
    }


def bench_verify_and_per_key(args, torch, dev, up, inputs, binding, np):
    """Two serving-side uses of the per-step form, B=64 Hk=16 Hv=32
    Dk=Dv=128, over rotating state sets: a speculative-verify window (T=4,
    the state emitted after 1, 2, 3 and 4 steps) and decode (T=1) with the
    per-key decay gate g [B,T,Hv,Dk]."""
    B, Hk, Hv, Dk, Dv = 64, 16, 32, 128, 128
    stream = torch.cuda.current_stream(dev)
    sb = B * Hv * Dv * Dk * 4                      # one state set, bytes
    res = {}
    for name, T, R, per_key, steps in (("verify_window", 4, 2, False, [1, 2, 3, 4]),
                                       ("per_key_decode", 1, 8, True, [])):
        raw = inputs.recurrence_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, workload_id=7, state=True)
        # unit-scale keys keep the state bounded over the repeated in-place steps
        q = (up(raw["q_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
        k = (up(raw["k_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
        v = up(raw["v"])
        g = (torch.full((B, T, Hv, Dk), 0.9, device=dev) if per_key
             else torch.full((B, T, Hv), 0.9, device=dev))
        beta = torch.full((B, T, Hv), 0.5, device=dev)
        y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
        sets = [dict(st=up(raw["state"]).clone(),
                     snaps=torch.empty(len(steps), B, Hv, Dv, Dk, device=dev) if steps else None)
                for _ in range(R)]

        def fn(i, steps=steps, sets=sets, q=q, k=k, v=v, g=g, beta=beta, y=y, per_key=per_key):
            s_ = sets[i % len(sets)]
            if steps:
                binding.recurrent_snapshots(q, k, v, g, beta, s_["st"], s_["st"], y, steps, s_["snaps"])
            else:
                binding.recurrent_per_key(q, k, v, g, beta, s_["st"], s_["st"], y)

        for i in range(2 * R):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(args.decode_steps // 2, 10)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / n
        nbytes = (2 + len(steps)) * sb + 2 * B * T * Hk * Dk * 2 + 2 * B * T * Hv * Dv * 2 + B * T * Hv * 4 \
            + B * T * Hv * (Dk if per_key else 1) * 4
        gbs = nbytes / us / 1e3
        kern = "recurrent_step_kernel<128, %s, %s>" % ("true" if per_key else "false", "true" if steps else "false")
        res[name] = {"workload": f"B={B} T={T} Hk={Hk} Hv={Hv} Dk=Dv={Dk}, {R} rotating state sets"
                                 + (f", snapshots after {steps} steps" if steps else ", per-key gate"),
                     "kernel": kern, "avg_launch_us": us, "bytes_per_launch": nbytes, "achieved_GBs": gbs,
                     "frac_hbm": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("recurrent_step_kernel", f"{name}_B64")}
        print(f"[bench] {name}: {us:.1f} us ({gbs:.0f} GB/s, {gbs / HBM_PEAK_GBS:.0%} of HBM)", file=sys.stderr,
              flush=True)
    return res


def serving_kernel(name, torch, dev, up, inputs, binding):
    """One launch of the verify-window (snapshots) or per-key-decode call of
    bench_verify_and_per_key, rotating its state sets (for counter passes)."""
    B, Hk, Hv, Dk, Dv = 64, 16, 32, 128, 128
    T, R, per_key, steps = (4, 2, False, [1, 2, 3, 4]) if name == "verify" else (1, 8, True, [])
    raw = inputs.recurrence_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, workload_id=7, state=True)
    q = (up(raw["q_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
    k = (up(raw["k_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
    v = up(raw["v"])
    g = torch.full((B, T, Hv, Dk), 0.9, device=dev) if per_key else torch.full((B, T, Hv), 0.9, device=dev)
    beta = torch.full((B, T, Hv), 0.5, device=dev)
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    sets = [dict(st=up(raw["state"]).clone(),
                 snaps=torch.empty(len(steps), B, Hv, Dv, Dk, device=dev) if steps else None) for _ in range(R)]
    ctr = iter(range(1 << 30))

    def fn():
        s_ = sets[next(ctr) % R]
        if steps:
            binding.recurrent_snapshots(q, k, v, g, beta, s_["st"], s_["st"], y, steps, s_["snaps"])
        else:
            binding.recurrent_per_key(q, k, v, g, beta, s_["st"], s_["st"], y)
    return fn


def bench_per_key_prefill(args, torch, dev, up, inputs, binding, np, launches=None):
    """The per-key decay gate g [B,T,Hv,Dk] over a prefill-length sequence
    (B=1 T=4096 Hk=16 Hv=32 Dk=Dv=128): the chunked matrix-core form, the
    per-step form with k, q and the gate rows staged through LDS, and the
    staging-free per-step kernel (reached through the snapshot entry point
    with one snapshot, of the final state).  With ``launches``: only that
    many chunked calls (for counter passes)."""
    B, T, Hk, Hv, Dk, Dv = 1, 4096, 16, 32, 128, 128
    raw = inputs.recurrence_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, workload_id=8, state=True)
    # unit-norm-scale keys and queries, beta in (0, 1)
    q = (up(raw["q_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
    k = (up(raw["k_raw"]).view(torch.bfloat16).float() / Dk ** 0.5).to(torch.bfloat16)
    v, st = up(raw["v"]), up(raw["state"])
    beta = torch.sigmoid(up(raw["b"]).view(torch.bfloat16).float())
    g = up(inputs.per_key_gate(B=B, T=T, Hv=Hv, Dk=Dk, workload_id=8))
    s_out = torch.empty_like(st)
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    snap = torch.empty(1, B, Hv, Dv, Dk, device=dev)
    stream = torch.cuda.current_stream(dev)

    ws = torch.empty(binding.recurrent_chunked_per_key_workspace_bytes(B, T, Hk, Hv, Dk, Dv), dtype=torch.uint8,
                     device=dev)

    def chunked():
        binding.recurrent_chunked_per_key(q, k, v, g, beta, st, s_out, y, ws)

    def staged():
        binding.recurrent_per_key(q, k, v, g, beta, st, s_out, y)

    def staging_free():
        binding.recurrent_snapshots(q, k, v, g, beta, st, s_out, y, [T], snap)

    if launches is not None:
        for _ in range(launches):
            chunked()
        torch.cuda.synchronize()
        print(f"[bench] kernel-only per_key: {launches} launches", file=sys.stderr, flush=True)
        return None
    out = {}
    for name, fn in (("chunked", chunked), ("staged", staged), ("staging_free", staging_free)):
        fn()
        torch.cuda.synchronize()
        out[name] = time_kernel(torch, stream, fn, 30 if name == "chunked" else 10,
                                warm=20 if name == "chunked" else 3)
    flops = 7 * B * T * Hv * Dk * Dv
    tf = flops / (out["chunked"] * 1e-6) / 1e12
    print(f"[bench] per-key prefill B=1 T=4096: chunked {out['chunked']:.1f} us ({tf:.1f} TFLOP/s), per-step "
          f"staged {out['staged']:.1f} us, staging-free {out['staging_free']:.1f} us", file=sys.stderr, flush=True)
    # algorithmic bytes: q, k, v, the gate rows, beta and the state read; y and the state written
    alg = (2 * B * T * Hk * Dk * 2 + B * T * Hv * Dv * 2 + B * T * Hv * Dk * 4 + B * T * Hv * 4
           + 2 * B * Hv * Dv * Dk * 4 + B * T * Hv * Dv * 2)
    return {"workload": f"B={B} T={T} Hk={Hk} Hv={Hv} Dk=Dv={Dk}, per-key gate U[0.3, 1), random state",
            "kernel": "chunk_prep_kernel<0, 1, true> + chunk_seq_kernel<1, true> (gdn_recurrent_chunked_per_key)",
            "traffic": measured_traffic("chunked_recurrence", "per_key_prefill_B1_T4096"),
            "traffic_algorithmic": alg,
            "avg_launch_us": out["chunked"], "achieved_TFLOPs": tf, "frac_fp32_peak": tf / FP32_PEAK_TFLOPS,
            "per_step_staged_us": out["staged"], "per_step_staging_free_us": out["staging_free"]}


def bench_decode_b1(args, torch, dev, up, inputs, binding, np):
    """Single-token decode B=1, T=1 (Hk=16 Hv=32 Dk=Dv=128): microseconds per
    call over 1000 back-to-back calls, warm (one state, updated in place) and
    cold (256 rotating states, 512 MiB, beyond the last-level cache); the
    recurrence alone and the layer core."""
    B, T, Hk, Hv, Dk, Dv, K = 1, 1, 16, 32, 128, 128, 4
    qs, ks = inputs.scales(Dk)
    raw = inputs.layer_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K, workload_id=1, state=True, conv_state=True)
    d = {k: up(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias")}
    R = 256
    states = [up(raw["state"]).clone() for _ in range(R)]
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    ws = torch.empty(max(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), 1), dtype=torch.uint8,
                     device=dev)
    pq = torch.empty(B, T, Hk, Dk, dtype=torch.int16, device=dev)
    pk, pv = torch.empty_like(pq), torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    pg = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    pb = torch.empty_like(pg)
    binding.prep(d["qkv"], d["conv_w"], d["conv_state"], None, d["a"], d["b"], d["A_log"], d["dt_bias"], pq, pk,
                 pv, pg, pb, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)

    def rec(st):
        binding.recurrent(pq, pk, pv, pg, pb, st, st, y)

    def core(st):
        binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], d["conv_state"], d["a"], d["b"], d["A_log"],
                           d["dt_bias"], st, st, y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)

    stream = torch.cuda.current_stream(dev)
    n = 1000
    out = {}
    for name, fn in (("recurrent", rec), ("layer_core", core)):
        for mode, pick in (("warm", lambda i: states[0]), ("cold", lambda i: states[i % R])):
            for i in range(R):
                fn(pick(i))
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n):
                fn(pick(i))
            b.record(stream)
            torch.cuda.synchronize()
            out[f"{name}_{mode}_us"] = a.elapsed_time(b) * 1e3 / n
    # the same calls marshalled once (binding.bind) and issued back to back:
    # the host cost is then the C entry point and the kernel launches only
    for name, fn in (("recurrent", rec), ("layer_core", core)):
        fname = binding.recurrent if name == "recurrent" else binding.layer_core
        calls = []
        for i in range(R):
            st = states[i]
            if name == "recurrent":
                calls.append(binding.bind(fname, pq, pk, pv, pg, pb, st, st, y))
            else:
                calls.append(binding.bind(fname, d["qkv"], d["conv_w"], d["conv_state"], d["conv_state"], d["a"],
                                          d["b"], d["A_log"], d["dt_bias"], st, st, y, ws, Hk=Hk, Hv=Hv, Dk=Dk,
                                          Dv=Dv, q_scale=qs, k_scale=ks))
        for c in calls:
            c()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            calls[i % R]()
        b.record(stream)
        torch.cuda.synchronize()
        out[f"{name}_bound_us"] = a.elapsed_time(b) * 1e3 / n
        del calls
    # the same calls captured in a HIP graph (a decode loop replayed without
    # host launch cost): 100 calls per graph, rotating the cold state ring
    side = torch.cuda.Stream()
    for name, fn in (("recurrent", rec), ("layer_core", core)):
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for i in range(100):
                fn(states[i % R])
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(100):
                fn(states[i % R])
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        out[f"{name}_graph_us"] = a.elapsed_time(b) * 1e3 / 1000
        del graph
    # the floor: a plain device copy of one 2 MiB state into another (the
    # bytes the step must move, less q/k/v/g/beta/y), back to back over the
    # same cold ring, eager and replayed from a graph of 100 copies
    dst = [torch.empty_like(states[0]) for _ in range(2)]

    def copy_state(st, i=[0]):
        i[0] += 1
        dst[i[0] % 2].copy_(st)
    for i in range(R):
        copy_state(states[i])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        copy_state(states[i % R])
    b.record(stream)
    torch.cuda.synchronize()
    out["copy_state_eager_us"] = a.elapsed_time(b) * 1e3 / n
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(100):
            copy_state(states[i % R])
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(100):
            copy_state(states[i % R])
    graph.replay()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(10):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    out["copy_state_graph_us"] = a.elapsed_time(b) * 1e3 / 1000
    del graph
    print(f"[bench] decode B=1 floor: 2 MiB state copy {out['copy_state_eager_us']:.2f} us eager, "
          f"{out['copy_state_graph_us']:.2f} us in a graph", file=sys.stderr, flush=True)
    print(f"[bench] decode B=1: recurrence {out['recurrent_warm_us']:.2f} us warm / {out['recurrent_cold_us']:.2f} us "
          f"cold / {out['recurrent_bound_us']:.2f} us bound / {out['recurrent_graph_us']:.2f} us in a graph; "
          f"layer core {out['layer_core_warm_us']:.2f} / {out['layer_core_cold_us']:.2f} / "
          f"{out['layer_core_bound_us']:.2f} / {out['layer_core_graph_us']:.2f} us per call",
          file=sys.stderr, flush=True)
    out["workload"] = ("decode B=1 T=1 Hk=16 Hv=32 Dk=Dv=128; 1000 back-to-back calls; warm = one state in place, "
                       "cold = 256 rotating states (512 MiB)")
    out["note"] = ("per-call time of back-to-back calls (device time plus any host launch gap); *_bound_us: the "
                   "cold calls marshalled once with binding.bind and issued back to back; *_graph_us: the same calls "
                   "captured in a HIP graph of 100 calls over the cold state ring and replayed; copy_state_*: the "
                   "floor, a plain device copy of one 2 MiB state (4 MiB moved) in the same two forms")
    return out


def bench_long_prefill(args, torch, dev, up, inputs, binding, np, launches=None):
    """Long batched prefill B=4, T=32768 (Hk=16 Hv=32 Dk=Dv=128, random
    recurrent state): the layer core per step, and its chunked recurrence
    alone against the fp32 peak.  With ``launches``: only that many
    layer-core steps (for counter passes)."""
    w = inputs.WORKLOADS["long"]
    B, T, Hk, Hv, Dk, Dv, K = (w[k] for k in ("B", "T", "Hk", "Hv", "Dk", "Dv", "K"))
    C = 2 * Hk * Dk + Hv * Dv
    qs, ks = inputs.scales(Dk)
    raw = inputs.workload("long")
    d = {k: up(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state")}
    del raw
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    s_out = torch.empty(B, Hv, Dv, Dk, dtype=torch.float32, device=dev)
    cs_out = torch.empty(B, K - 1, C, dtype=torch.int16, device=dev)
    ws = torch.empty(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), dtype=torch.uint8, device=dev)
    pq = torch.empty(B, T, Hk, Dk, dtype=torch.int16, device=dev)
    pk, pv = torch.empty_like(pq), torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)
    pg = torch.empty(B, T, Hv, dtype=torch.float32, device=dev)
    pb = torch.empty_like(pg)
    cws = torch.empty(binding.recurrent_chunked_workspace_bytes(B, T, Hk, Hv, Dk, Dv), dtype=torch.uint8,
                      device=dev)

    def step():
        binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                           d["dt_bias"], d["state"], s_out, y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                           q_scale=qs, k_scale=ks)

    def chunked():
        binding.recurrent_chunked(pq, pk, pv, pg, pb, d["state"], s_out, y, cws)

    if launches is not None:
        for _ in range(launches):
            step()
        torch.cuda.synchronize()
        print(f"[bench] kernel-only long: {launches} launches", file=sys.stderr, flush=True)
        return None
    binding.prep(d["qkv"], d["conv_w"], d["conv_state"], None, d["a"], d["b"], d["A_log"], d["dt_bias"], pq, pk,
                 pv, pg, pb, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    stream = torch.cuda.current_stream(dev)
    n = 6
    step_us = time_kernel(torch, stream, step, n)
    chunk_us = time_kernel(torch, stream, chunked, n)
    flops = 7 * B * T * Hv * Dk * Dv
    tf = flops / (chunk_us * 1e-6) / 1e12
    print(f"[bench] long prefill B=4 T=32768: layer core {step_us / 1e3:.2f} ms/step; chunked recurrence "
          f"{chunk_us / 1e3:.2f} ms ({tf:.1f} TFLOP/s, {tf / FP32_PEAK_TFLOPS:.1%} of fp32 peak)",
          file=sys.stderr, flush=True)
    # algorithmic bytes of the layer-core step: qkv, a, b, conv weights and the state read; y, the state and
    # the conv state written
    alg = (B * T * C * 2 + 2 * B * T * Hv * 2 + C * K * 2 + B * Hv * Dv * Dk * 4
           + B * T * Hv * Dv * 2 + B * Hv * Dv * Dk * 4 + B * (K - 1) * C * 2)
    return {"workload": "long prefill B=4 T=32768 Hk=16 Hv=32 Dk=Dv=128 K=4, random recurrent state",
            "kernel": "chunk_prep_kernel<4, 2> + chunk_seq_pairs_kernel (two waves per 16-row state tile)",
            "traffic": measured_traffic("layer_core", "long_prefill_B4_T32768"), "traffic_algorithmic": alg,
            "ms_per_step": step_us / 1e3, "value": B * T * Hv / (step_us * 1e-6), "unit": "token*head/s",
            "chunked_recurrence_ms": chunk_us / 1e3, "chunked_TFLOPs": tf, "frac_fp32_peak": tf / FP32_PEAK_TFLOPS,
            "steps_timed": n}


def cpu_baseline(raw, Hk, Hv, Dk, Dv, qs, ks, eps):
    """The oracle (as it stands) on a bounded sample of the prefill workload:
    the full layer core (prologue of the head's channels + recurrence) for
    a fixed set of v-heads over all T tokens, on one host thread."""
    import numpy as np

    import oracle
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    heads = list(range(Hv))
    T = raw["qkv"].shape[1]
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    oracle.lib()
    # whole passes over the workload until at least 10 s of CPU time (one pass
    # takes a few seconds on the host)
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < 10.0:
        for hv in heads:
            hk = hv // (Hv // Hk)
            ch = (list(range(hk * Dk, (hk + 1) * Dk)) + list(range(Hk * Dk + hk * Dk, Hk * Dk + (hk + 1) * Dk))
                  + list(range(2 * Hk * Dk + hv * Dv, 2 * Hk * Dk + (hv + 1) * Dv)))
            oracle.layer_core(np.ascontiguousarray(raw["qkv"][..., ch]), np.ascontiguousarray(raw["conv_w"][ch]),
                              None, np.ascontiguousarray(raw["a"][..., hv:hv + 1]),
                              np.ascontiguousarray(raw["b"][..., hv:hv + 1]), raw["A_log"][hv:hv + 1].copy(),
                              raw["dt_bias"][hv:hv + 1].copy(), None, Hk=1, Hv=1, Dk=Dk, Dv=Dv,
                              q_scale=qs, k_scale=ks, eps=eps)
        passes += 1
    dt = time.perf_counter() - t0
    print(f"[bench] cpu oracle: {passes} passes of {len(heads)} heads x {T} tokens in {dt:.1f} s",
          file=sys.stderr, flush=True)
    return {"value": passes * len(heads) * T / dt, "unit": "token*head/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} whole passes over the prefill workload, each computed per v-head (all {len(heads)}): "
                      f"prologue of the head's channels + recurrence over all {T} tokens, fp64, one thread",
            "seconds": dt, "passes": passes, "host": host_cpu_model(), "host_cpus": os.cpu_count()}


def kernel_only(args, torch, dev, prep_rot, rec_only, up, inputs, binding, np, chunked_only, epilogue_rot,
                epi_sets, y, step):
    """Launch one kernel a few times (for rocprofv3 counter passes), in the
    configuration the benchmark times (rotating sets for the prefill step,
    prep and epilogue)."""
    n = max(args.steps, 1)
    ctr = iter(range(1 << 30))
    if args.kernel_only == "layer":
        def fn():
            step(next(ctr))
    elif args.kernel_only in ("verify", "per_key_decode"):
        fn = serving_kernel(args.kernel_only, torch, dev, up, inputs, binding)
    elif args.kernel_only == "recurrent":
        fn = rec_only
    elif args.kernel_only == "chunked":
        fn = chunked_only
    elif args.kernel_only == "prep":
        def fn():
            prep_rot(next(ctr))
    elif args.kernel_only == "epilogue":
        rec_only()
        for e_ in epi_sets:
            e_["y"].copy_(y)

        def fn():
            epilogue_rot(next(ctr))
    elif args.kernel_only == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)   # 256 MiB
        dst = torch.empty_like(src)

        def fn():
            dst.copy_(src)
    else:
        B, T, Hk, Hv, Dk, Dv = 64, 1, 16, 32, 128, 128
        pq = torch.zeros(B, T, Hk, Dk, dtype=torch.int16, device=dev)
        pk, pv = torch.zeros_like(pq), torch.zeros(B, T, Hv, Dv, dtype=torch.int16, device=dev)
        pg = torch.ones(B, T, Hv, dtype=torch.float32, device=dev)
        pb = torch.zeros_like(pg)
        st = torch.zeros(B, Hv, Dv, Dk, dtype=torch.float32, device=dev)
        yy = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=dev)

        def fn():
            binding.recurrent(pq, pk, pv, pg, pb, st, st, yy)
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    print(f"[bench] kernel-only {args.kernel_only}: {n} launches", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
