"""Decode-step benchmark: tokens/s on one MI355X and the fraction of the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2b|8b|2b_long|tiny]

One "step" is one kd_step: a whole decode step of the batch-1 decoder, run as one persistent
kernel launch. The default workload is the 2B-class decoder. Its 512-token prompt is fed one
token per step to fill the KV cache; this is untimed. Then W warm-up decode steps and K timed
decode steps follow, each feeding back the greedy token of the step before.

Printed on stdout, as one JSON line:
  value          tokens/s over the timed steps (batch 1: one token per step), inputs resident in HBM
  roofline       algorithmic bytes per step (every weight, the KV cache over 0..p, the KV write,
                 the logits) divided by the kernel's mean duration. The duration comes from HIP
                 events on the launch stream; the peak is the HBM spec of 8 TB/s.
  cpu_baseline   the CPU oracle, run for a bounded number of decode steps on the host cores
Everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "batch-1 decode tokens/sec on 1 MI355X + % of HBM bytes/token roofline"
KERNEL_SOURCES = ("kd_device.h", "kd_plan.h", "kd_api.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bandwidth_bound_transformer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this kernel."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def cpu_baseline(wl, weights, dec, torch, n_steps: int, first_pos: int, first_token: int):
    """Time the oracle on decode steps of the same workload, starting from the GPU's KV cache."""
    from oracle import decoder as ref
    from threadpoolctl import threadpool_info

    m = wl.model
    o = ref.Oracle(m, weights, batch=1, max_seq=first_pos + n_steps + 1)
    kv = dec.kv_view()[:, :, 0, :, :first_pos].float().cpu().numpy()
    o.k_cache[0, :, :, :first_pos] = kv[:, 0]
    o.v_cache[0, :, :, :first_pos] = kv[:, 1]
    del kv
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tok = first_token
    t0 = time.perf_counter()
    for i in range(n_steps):
        logits = o.step_one(0, tok, first_pos + i)
        tok = int(ref.greedy_token(logits[None])[0])
    dt = time.perf_counter() - t0
    return {
        "value": n_steps / dt,
        "unit": "tok/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_steps} decode steps of workload {wl.name} at positions {first_pos}..{first_pos + n_steps - 1}, "
                  f"float64 numpy oracle, {dt:.1f} s",
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="2b", choices=["tiny", "2b", "8b", "2b_long"])
    ap.add_argument("--cpu-steps", type=int, default=3, help="oracle decode steps timed for cpu_baseline (0: skip)")
    ap.add_argument("--trace", action="store_true", help="after timing, trace one step and print its phase breakdown")
    ap.add_argument("--trace-out", default=None, help="with --trace: also save the raw timestamp buffer (.npy)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before decoding, copy MIB MiB once with a plain device copy; HBM-traffic counters read on "
                         "that copy calibrate the counters read on the decode kernel (profiling runs only)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path (asked for {max(args.gpus, world)}).",
              file=sys.stderr)
        return 2

    import torch

    import workloads
    from bandwidth_bound_transformer_amd import kd, roofline

    wl = workloads.get(args.workload)
    m = wl.model
    decode_steps = wl.decode_steps
    if args.warmup + args.steps > decode_steps:
        args.steps = decode_steps - args.warmup
        log(f"steps capped at {args.steps}: the workload has {decode_steps} decode steps")
    assert args.steps > 0

    t0 = time.perf_counter()
    weights = workloads.make_weights(m, seed=wl.weight_seed)
    log(f"weights generated in {time.perf_counter() - t0:.1f} s")
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst
    dec = kd.Decoder(m, weights, max_seq=wl.max_seq, device="cuda:0")
    info = kd.kd_get_info(dec.handle)
    log(f"kd_init done: {info}")
    stream = torch.cuda.current_stream()

    # fill the KV cache: the prompt fed one token per step, or the seeded pre-filled values
    if wl.prefill_len > 0:
        kv_host = np.zeros((m.n_layers, 2, 1, m.n_kv_heads, dec.s_alloc, m.head_dim),
                           np.uint16 if m.kv_dtype == "bf16" else np.float32)
        workloads.fill_kv_prefill(wl, kv_host)
        flat = torch.from_numpy(kv_host.reshape(-1).view(np.int16 if m.kv_dtype == "bf16" else np.float32))
        dec.kv.view(torch.int16 if m.kv_dtype == "bf16" else torch.float32).copy_(flat)
        del kv_host, flat
        dec.tokens.fill_(int(workloads.make_first_tokens(wl)[0]))
        dec.positions.fill_(wl.prefill_len)
    else:
        prompt = torch.as_tensor(workloads.make_prompt(wl, 0), device=dec.device)
        dec.positions.zero_()
        for p in range(wl.prompt_len):
            dec.tokens.copy_(prompt[p : p + 1])
            dec.step(write_logits=False)
    torch.cuda.synchronize()
    if dec.status():
        log(f"device status {dec.status():#x} after prefill")
        return 1

    for _ in range(args.warmup):
        dec.step()
    torch.cuda.synchronize()
    first_pos = int(dec.positions.item())
    first_token = int(dec.tokens.item())

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    whole0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        dec.step(stream=stream)
        ev[i][1].record(stream)
    whole1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    status = dec.status()
    if status:
        log(f"device status {status:#x} during the timed steps")
        return 1

    elapsed_ms = whole0.elapsed_time(whole1)
    per_step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    positions = range(first_pos, first_pos + args.steps)
    alg_bytes = np.array([roofline.step_bytes(m, 1, p).total for p in positions], np.float64)
    achieved_gbps = float(alg_bytes.mean() / (per_step_us.mean() * 1e-6) / 1e9)
    tok_s = args.steps / (elapsed_ms * 1e-3)
    bound_tok_s = roofline.tokens_per_s_bound(PEAK_HBM_GBPS * 1e9, float(alg_bytes.mean()))
    log(f"{args.steps} steps in {elapsed_ms:.2f} ms (wall {t_wall * 1e3:.1f} ms): {tok_s:.1f} tok/s, "
        f"kernel mean {per_step_us.mean():.1f} us (p50 {np.percentile(per_step_us, 50):.1f}, "
        f"p99 {np.percentile(per_step_us, 99):.1f}), {achieved_gbps:.0f} GB/s algorithmic, "
        f"roofline {bound_tok_s:.0f} tok/s")

    if args.trace:
        from bandwidth_bound_transformer_amd import trace as tr

        stride = kd.kd_trace(dec.handle, None, 0)
        buf = torch.zeros(stride * info["workgroups"], dtype=torch.int64, device=dec.device)
        kd.kd_trace(dec.handle, buf, buf.numel())
        for _ in range(3):
            dec.step()
        torch.cuda.synchronize()
        kd.kd_trace(dec.handle, None, 0)
        raw = buf.cpu().numpy()
        log("phase breakdown of one traced step:\n" + tr.summary(raw, m.n_layers, info["workgroups"]))
        log(tr.critical_path(raw, m.n_layers, info["workgroups"]))
        if args.trace_out:
            np.save(args.trace_out, raw)

    cpu = None
    if args.cpu_steps > 0:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(wl, weights, dec, torch, args.cpu_steps, first_pos, first_token)
        log(f"cpu oracle: {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    traffic = measured_traffic(wl.name)
    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "layers": m.n_layers, "d_model": m.d_model, "q_heads": m.n_q_heads, "kv_heads": m.n_kv_heads,
            "head_dim": m.head_dim, "ffn": m.ffn_dim, "vocab": m.vocab, "weight_dtype": m.weight_dtype,
            "kv_dtype": m.kv_dtype, "batch": 1, "positions": [first_pos, first_pos + args.steps - 1],
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "decode_step_kernel",
            "algorithmic_bytes_per_launch": round(float(alg_bytes.mean())),
            "kernel_mean_us": round(float(per_step_us.mean()), 2),
        },
        "roofline_tok_s": round(bound_tok_s, 1),
        "frac_of_roofline_tok_s": round(tok_s / bound_tok_s, 4),
        "itl_us": {"p50": round(float(np.percentile(per_step_us, 50)), 2), "p99": round(float(np.percentile(per_step_us, 99)), 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    dec.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
