"""Decode-step benchmark: tokens/s on one MI355X and the fraction of the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2b|8b|2b_long|tiny|11b_x56]

One "step" is one kd_step: a whole decode step of every session. At batch 1 it is one persistent
kernel launch; for the 56 lockstep sessions it is one tick, a fixed kernel sequence on one stream.
The default workload is the 2B-class decoder at batch 1. Its 512-token prompt is fed one token per
step to fill the KV cache; this is untimed. Pre-filled workloads write the seeded cache contents
instead. Then W warm-up steps and K timed steps follow, each feeding back the greedy tokens of
the step before.

Printed on stdout, as one JSON line:
  value          tokens/s over the timed steps (B tokens per step, all sessions), inputs resident in HBM
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
METRIC_SESSIONS = "aggregate decode tokens/sec of lockstep sessions on 1 MI355X + p99 tick latency"
KERNEL_SOURCES = ("kd_device.h", "kd_plan.h", "kd_pack.h")  # what defines the batch-1 step kernel and its weight layout
BATCH_SOURCES = ("kd_batch.h", "kd_batch_host.h")  # the lockstep-sessions kernels and their launch plan


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "bandwidth_bound_transformer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this kernel."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash(sources):
        return None
    return float(val.group(1))


def cpu_baseline(wl, weights, dec, torch, max_steps: int, min_seconds: float, first_pos: int, first_token: int):
    """Time the oracle on decode steps of session 0 of the same workload, from the GPU's KV cache:
    steps until ``min_seconds`` have passed, or ``max_steps`` of them."""
    from oracle import decoder as ref
    from threadpoolctl import threadpool_info

    m = wl.model
    o = ref.Oracle(m, weights, batch=1, max_seq=first_pos + max_steps + 1)
    for l in range(m.n_layers):
        kv = dec.kv_view()[l, :, 0, :, :first_pos].float().cpu().numpy()
        o.k_cache[0, l, :, :first_pos] = kv[0]
        o.v_cache[0, l, :, :first_pos] = kv[1]
    del kv
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tok = first_token
    n_steps = 0
    t0 = time.perf_counter()
    while n_steps < max_steps:
        logits = o.step_one(0, tok, first_pos + n_steps)
        tok = int(ref.greedy_token(logits[None])[0])
        n_steps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": n_steps / dt,
        "unit": "tok/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n_steps} decode steps of session 0 of workload {wl.name} at positions "
                  f"{first_pos}..{first_pos + n_steps - 1}, float64 numpy oracle, {dt:.1f} s",
    }


def nearest_rank(values, q: float) -> float:
    """Nearest-rank percentile: the ceil(q n)-th smallest value."""
    v = np.sort(np.asarray(values, np.float64))
    return float(v[max(0, int(np.ceil(q * len(v))) - 1)])


def fill_prefilled_cache(wl, dec, torch) -> None:
    """Write the seeded pre-filled K/V values of every session, one layer at a time."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads

    m = wl.model
    storage = np.uint16 if m.kv_dtype == "bf16" else np.float32
    view_dtype = torch.int16 if m.kv_dtype == "bf16" else torch.float32
    host = np.zeros((2, wl.batch, m.n_kv_heads, wl.prefill_len, m.head_dim), storage)
    kv = dec.kv_view().view(view_dtype)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for l in range(m.n_layers):
            def work(job, l=l):
                s, b, g = job
                host[s, b, g] = workloads.kv_prefill_block(wl, l, s, b, g)

            list(pool.map(work, [(s, b, g) for s in range(2) for b in range(wl.batch) for g in range(m.n_kv_heads)]))
            kv[l, :, :, :, : wl.prefill_len] = torch.from_numpy(host.view(np.int16 if m.kv_dtype == "bf16" else np.float32))
            if (l + 1) % 8 == 0 or l + 1 == m.n_layers:
                log(f"pre-filled cache: {l + 1}/{m.n_layers} layers ({time.perf_counter() - t0:.1f} s)")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="2b", choices=["tiny", "2b", "8b", "2b_long", "11b_x56"])
    ap.add_argument("--cpu-steps", type=int, default=30,
                    help="most oracle decode steps (of one session) timed for cpu_baseline; 0 skips it")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="cpu_baseline stops stepping the oracle once this much time has passed")
    ap.add_argument("--trace", action="store_true", help="after timing, trace one step and print its phase breakdown")
    ap.add_argument("--trace-out", default=None, help="with --trace: also save the raw timestamp buffer (.npy)")
    ap.add_argument("--trace-json", default=None,
                    help="with --trace: also write the traced step as Chrome trace-event JSON (Perfetto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before decoding, copy MIB MiB once with a plain device copy; HBM-traffic counters read on "
                         "that copy calibrate the counters read on the decode kernel (profiling runs only)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path (asked for {max(args.gpus, world)}).",
              file=sys.stderr)
        return 2

    import torch

    import workloads
    from bandwidth_bound_transformer_amd import kd, roofline

    wl = workloads.get(args.workload)
    m = wl.model
    B = wl.batch
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
    dec = kd.Decoder(m, weights, max_seq=wl.max_seq, batch=B, device="cuda:0")
    info = kd.kd_get_info(dec.handle)
    log(f"kd_init done: {info}")
    stream = torch.cuda.current_stream()

    # fill the KV cache: the prompt fed one token per step, or the seeded pre-filled values
    if wl.prefill_len > 0:
        fill_prefilled_cache(wl, dec, torch)
        dec.tokens.copy_(torch.from_numpy(workloads.make_first_tokens(wl)))
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
    first_pos = int(dec.positions[0].item())
    first_token = int(dec.tokens[0].item())

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
    alg_bytes = np.array([roofline.step_bytes(m, B, p).total for p in positions], np.float64)
    achieved_gbps = float(alg_bytes.mean() / (per_step_us.mean() * 1e-6) / 1e9)
    tok_s = args.steps * B / (elapsed_ms * 1e-3)
    bound_tok_s = roofline.tokens_per_s_bound(PEAK_HBM_GBPS * 1e9, float(alg_bytes.mean()), B)
    p99 = nearest_rank(per_step_us, 0.99)
    log(f"{args.steps} steps x {B} sessions in {elapsed_ms:.2f} ms (wall {t_wall * 1e3:.1f} ms): {tok_s:.1f} tok/s, "
        f"step mean {per_step_us.mean():.1f} us (p50 {np.percentile(per_step_us, 50):.1f}, "
        f"p99 {p99:.1f}), {achieved_gbps:.0f} GB/s algorithmic, roofline {bound_tok_s:.0f} tok/s")

    if args.trace and B == 1:
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
        if args.trace_json:
            with open(args.trace_json, "w") as f:
                json.dump(tr.to_chrome_trace(raw, m.n_layers, info["workgroups"]), f)

    cpu = None
    if args.cpu_steps > 0:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(wl, weights, dec, torch, args.cpu_steps, args.cpu_seconds, first_pos, first_token)
        log(f"cpu oracle: {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    traffic = measured_traffic(wl.name, KERNEL_SOURCES if B == 1 else BATCH_SOURCES)
    out = {
        "metric": METRIC if B == 1 else METRIC_SESSIONS,
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
            "kv_dtype": m.kv_dtype, "batch": B, "positions": [first_pos, first_pos + args.steps - 1],
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "decode_step_kernel" if B == 1 else "one tick (the kd_step kernel sequence)",
            "algorithmic_bytes_per_launch": round(float(alg_bytes.mean())),
            "kernel_mean_us": round(float(per_step_us.mean()), 2),
        },
        "roofline_tok_s": round(bound_tok_s, 1),
        "frac_of_roofline_tok_s": round(tok_s / bound_tok_s, 4),
        "itl_us": {"p50": round(float(np.percentile(per_step_us, 50)), 2), "p99": round(p99, 2)},
        "cpu_baseline": cpu,
    }
    if B > 1:
        out["tick_latency_ms"] = {"p50": round(float(np.percentile(per_step_us, 50)) / 1e3, 4), "p99": round(p99 / 1e3, 4),
                                  "max": round(float(per_step_us.max()) / 1e3, 4)}
    print(json.dumps(out), flush=True)
    dec.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
