"""Decode-step benchmark: tokens/s on one MI355X and the fraction of the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b|2b|2b_long|tiny|11b_x56|8b_fp8|2b_fp8|8b_int8|2b_int8|11b_x56_fp8|11b_x56_int8]

One "step" is one kd_step: a whole decode step of every session. At batch 1 it is one persistent
kernel launch; for the 56 lockstep sessions it is one tick, a fixed kernel sequence on one stream.
The default workload is the Llama-3-8B-shaped decoder at batch 1, the largest batch-1 workload.
Its prompt is fed one token per step to fill the KV cache; this is untimed. Pre-filled workloads
write the seeded cache contents instead. Then W warm-up steps and K timed steps follow, each
feeding back the greedy tokens of the step before. The same positions are then run once more as
one kd_generate call (the resident loop), timed as a whole.

Printed on stdout, as one JSON line:
  value          tokens/s over the timed steps (B tokens per step, all sessions), inputs resident in HBM
  roofline       algorithmic bytes per step (every weight, the KV cache over 0..p, the KV write,
                 the logits) divided by the kernel's mean duration. The duration comes from HIP
                 events on the launch stream; the peak is the HBM spec of 8 TB/s.
  stream_ceiling the read rate of a plain streaming kernel on the same GPU in the same run, and
                 the decode kernel's achieved rate as a fraction of it
  cpu_baseline   the CPU oracle, run for a bounded number of decode steps on the host cores
  extra          the 2B batch-1 workload, and the 8B and 2B with FP8 and with int8 weights, measured the
                 same way in the same run (default run only)
  ttft           batch-1 prompts (bf16, fp8, int8): time to the first token with kd_prefill (the prompt on the matrix
                 cores), beside the time the same prompt takes one step per token
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


def measure(wl, args, torch, kd, roofline, steps: int, warmup: int, trace: bool, cpu_steps: int):
    """Build the decoder of workload wl, fill its cache, time `steps` kd_step calls after `warmup`
    untimed ones, then the same positions as one kd_generate call. Returns (result dict, decoder,
    weights, first position, first token); the caller closes the decoder."""
    import workloads

    m = wl.model
    B = wl.batch
    if warmup + steps > wl.decode_steps:
        steps = wl.decode_steps - warmup
        log(f"{wl.name}: steps capped at {steps}: the workload has {wl.decode_steps} decode steps")
    assert steps > 0
    t0 = time.perf_counter()
    weights = workloads.make_weights(m, seed=wl.weight_seed)
    log(f"{wl.name}: weights generated in {time.perf_counter() - t0:.1f} s")
    # batch-1 prompts also run through kd_prefill (the matrix cores, 128 positions a pass)
    chunk = getattr(args, "prefill_chunk", 128) if (B == 1 and m.weight_dtype in ("bf16", "fp8", "int8") and wl.prompt_len > 0) else 0
    dec = kd.Decoder(m, weights, max_seq=wl.max_seq, batch=B, device="cuda:0", prefill_chunk=chunk)
    info = kd.kd_get_info(dec.handle)
    log(f"{wl.name}: kd_init done: {info}")
    stream = torch.cuda.current_stream()

    # fill the KV cache: the prompt fed one token per step (timed), then, where set up, through
    # kd_prefill (timed: the time to the first token), or the seeded pre-filled values
    ttft = None
    if wl.prefill_len > 0:
        view_dtype = torch.int16 if m.kv_dtype == "bf16" else torch.float32
        workloads.fill_kv_prefill_device(wl, dec.kv_view().view(view_dtype), torch, log=log)
        dec.tokens.copy_(torch.from_numpy(workloads.make_first_tokens(wl)))
        dec.positions.fill_(wl.prefill_len)
    else:
        prompt = torch.as_tensor(workloads.make_prompt(wl, 0), device=dec.device)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dec.positions.zero_()
        torch.cuda.synchronize()
        a.record(stream)
        for p in range(wl.prompt_len):
            dec.tokens.copy_(prompt[p : p + 1])
            dec.step(write_logits=False, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        stepwise_ms = a.elapsed_time(b)
        first_stepwise = int(dec.tokens[0].item())
        log(f"{wl.name}: prompt of {wl.prompt_len} tokens one step each: {stepwise_ms:.2f} ms")
        if chunk:
            runs = []
            for _ in range(2):  # the second run is reported; the first warms the kernels
                dec.positions.zero_()
                torch.cuda.synchronize()
                a.record(stream)
                dec.prefill(prompt, stream=stream)
                b.record(stream)
                torch.cuda.synchronize()
                runs.append(a.elapsed_time(b))
            ttft = {
                "ms": round(runs[-1], 3),
                "prompt_tokens": wl.prompt_len,
                "prefill_tok_s": round(wl.prompt_len / (runs[-1] * 1e-3), 1),
                "chunk_positions": chunk,
                "stepwise_prompt_ms": round(stepwise_ms, 2),
                "same_first_token_as_stepwise": int(dec.tokens[0].item()) == first_stepwise,
                # the whole prefill against the matrix cores' dense bf16 peak (algorithmic flops:
                # every projection per position, causal attention, the last position's LM head)
                "roofline": {"bound": "mfma", "unit": "TFLOP/s",
                             "achieved": round(roofline.prefill_flops(m, wl.prompt_len) / (runs[-1] * 1e-3) / 1e12, 1),
                             "peak": roofline.MI355X_BF16_DENSE_FLOPS / 1e12,
                             "frac": round(roofline.prefill_flops(m, wl.prompt_len) / (runs[-1] * 1e-3)
                                           / roofline.MI355X_BF16_DENSE_FLOPS, 4)},
                "what": "kd_prefill of the whole prompt (prompt tokens in HBM) to the first greedy token",
            }
            log(f"{wl.name}: time to first token via kd_prefill: {runs} ms")
    torch.cuda.synchronize()
    if dec.status():
        raise RuntimeError(f"{wl.name}: device status {dec.status():#x} after prefill")

    for _ in range(warmup):
        dec.step()
    torch.cuda.synchronize()
    first_pos = int(dec.positions[0].item())
    first_token = int(dec.tokens[0].item())
    tokens0, positions0 = dec.tokens.clone(), dec.positions.clone()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    whole0, whole1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    whole0.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        dec.step(stream=stream)
        ev[i][1].record(stream)
    whole1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    status = dec.status()
    if status:
        raise RuntimeError(f"{wl.name}: device status {status:#x} during the timed steps")
    tokens_steps = dec.tokens.clone()

    elapsed_ms = whole0.elapsed_time(whole1)
    per_step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    positions = range(first_pos, first_pos + steps)
    alg_bytes = np.array([roofline.step_bytes(m, B, p).total for p in positions], np.float64)
    achieved_gbps = float(alg_bytes.mean() / (per_step_us.mean() * 1e-6) / 1e9)
    tok_s = steps * B / (elapsed_ms * 1e-3)
    bound_tok_s = roofline.tokens_per_s_bound(PEAK_HBM_GBPS * 1e9, float(alg_bytes.mean()), B)
    p99 = nearest_rank(per_step_us, 0.99)
    log(f"{wl.name}: {steps} steps x {B} sessions in {elapsed_ms:.2f} ms (wall {t_wall * 1e3:.1f} ms): {tok_s:.1f} tok/s, "
        f"step mean {per_step_us.mean():.1f} us (p50 {np.percentile(per_step_us, 50):.1f}, "
        f"p99 {p99:.1f}), {achieved_gbps:.0f} GB/s algorithmic, roofline {bound_tok_s:.0f} tok/s")

    # the same positions again, as one resident call (the cache is rewritten with the same values)
    dec.tokens.copy_(tokens0)
    dec.positions.copy_(positions0)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    dec.generate(steps, stream=stream)
    g1.record(stream)
    torch.cuda.synchronize()
    if dec.status():
        raise RuntimeError(f"{wl.name}: device status {dec.status():#x} during kd_generate")
    same = bool(torch.equal(dec.tokens, tokens_steps))
    gen_ms = g0.elapsed_time(g1)
    resident = {"tok_s": round(steps * B / (gen_ms * 1e-3), 2), "itl_us_mean": round(gen_ms * 1e3 / steps, 2),
                "same_tokens_as_kd_step": same}
    log(f"{wl.name}: kd_generate of the same {steps} steps: {resident}")

    if trace and B == 1:
        from bandwidth_bound_transformer_amd import trace as tr

        stride = kd.kd_trace(dec.handle, None, 0)
        buf = torch.zeros(stride * info["workgroups"], dtype=torch.int64, device=dec.device)
        kd.kd_trace(dec.handle, buf, buf.numel())
        dec.tokens.copy_(tokens0)
        dec.positions.copy_(positions0)
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
    if cpu_steps > 0:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(wl, weights, dec, torch, cpu_steps, args.cpu_seconds, first_pos, first_token)
        log(f"cpu oracle: {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    res = {
        "workload": wl.name,
        "tok_s": tok_s,
        "steps": steps,
        "elapsed_ms": elapsed_ms,
        "per_step_us": per_step_us,
        "alg_bytes": float(alg_bytes.mean()),
        "achieved_gbps": achieved_gbps,
        "bound_tok_s": bound_tok_s,
        "p99_us": p99,
        "first_pos": first_pos,
        "resident": resident,
        "cpu": cpu,
        "ttft": ttft,
    }
    del weights
    return res, dec


def stream_ceiling(torch, kd, gib: int = 4, reps: int = 10) -> float:
    """Read rate (GB/s) of the library's plain streaming kernel over a gib GiB buffer of random bytes,
    like the weights and caches it is compared with."""
    nbytes = gib << 30
    g = torch.Generator(device="cuda:0")
    g.manual_seed(1)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0", generator=g)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        kd.kd_stream_read(buf, nbytes, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        kd.kd_stream_read(buf, nbytes, stream)
    b.record(stream)
    torch.cuda.synchronize()
    gbps = reps * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    log(f"stream ceiling: {gbps:.0f} GB/s reading {gib} GiB")
    return gbps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="8b", choices=["tiny", "2b", "8b", "2b_long", "11b_x56", "2b_fp8", "8b_fp8", "2b_int8", "8b_int8",
                                                    "11b_x56_fp8", "11b_x56_int8"])
    ap.add_argument("--prefill-chunk", type=int, default=128,
                    help="prompt positions per kd_prefill pass for batch-1 workloads (2..128)")
    ap.add_argument("--extra", default=None,
                    help="comma-separated workloads measured after the headline one and reported under 'extra' "
                         "(default: 2b when the headline is the default 8b, else none; 'none' for none)")
    ap.add_argument("--extra-steps", type=int, default=500, help="timed steps of each extra workload")
    ap.add_argument("--tick-budget-ms", type=float, default=160.0,
                    help="lockstep sessions: a tick longer than this misses its deadline (the pages' 160 ms tick)")
    ap.add_argument("--cpu-steps", type=int, default=30,
                    help="most oracle decode steps (of one session) timed for cpu_baseline; 0 skips it")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="cpu_baseline stops stepping the oracle once this much time has passed")
    ap.add_argument("--no-stream-ceiling", action="store_true", help="skip the plain stream-read measurement")
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

    try:
        r, dec = measure(wl, args, torch, kd, roofline, args.steps, args.warmup, args.trace, args.cpu_steps)
    except RuntimeError as e:
        log(str(e))
        return 1
    dec.close()
    del dec
    torch.cuda.empty_cache()

    extra_names = args.extra
    if extra_names is None:
        extra_names = "2b,8b_fp8,2b_fp8,8b_int8,2b_int8" if args.workload == "8b" else "none"
    extra = {}
    for name in [n for n in extra_names.split(",") if n and n != "none"]:
        try:
            e, d2 = measure(workloads.get(name), args, torch, kd, roofline, args.extra_steps, args.warmup, False, 0)
        except RuntimeError as err:
            log(str(err))
            return 1
        d2.close()
        del d2
        torch.cuda.empty_cache()
        extra[name] = {
            "value": round(e["tok_s"], 2),
            "unit": "tok/s",
            "steps": e["steps"],
            "ms_per_step": round(e["elapsed_ms"] / e["steps"], 4),
            "positions": [e["first_pos"], e["first_pos"] + e["steps"] - 1],
            "roofline_frac": round(e["achieved_gbps"] / PEAK_HBM_GBPS, 4),
            "achieved_gbps": round(e["achieved_gbps"], 1),
            "frac_of_roofline_tok_s": round(e["tok_s"] / e["bound_tok_s"], 4),
            "roofline_tok_s": round(e["bound_tok_s"], 1),
            "itl_us": {"p50": round(float(np.percentile(e["per_step_us"], 50)), 2),
                       "p99": round(nearest_rank(e["per_step_us"], 0.99), 2)},
            "resident": e["resident"],
            "ttft": e["ttft"],
            "weight_dtype": workloads.get(name).model.weight_dtype,
            "traffic": measured_traffic(name, KERNEL_SOURCES if workloads.get(name).batch == 1 else BATCH_SOURCES),
        }

    ceiling = None if args.no_stream_ceiling else stream_ceiling(torch, kd)
    per_step_us = r["per_step_us"]
    traffic = measured_traffic(wl.name, KERNEL_SOURCES if B == 1 else BATCH_SOURCES)
    out = {
        "metric": METRIC if B == 1 else METRIC_SESSIONS,
        "value": round(r["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(r["elapsed_ms"] / r["steps"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic: fp32 FMAs on bf16 weights at batch 1; bf16 (hi/lo) matrix-core products otherwise
        "dtype": "f32" if B == 1 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "layers": m.n_layers, "d_model": m.d_model, "q_heads": m.n_q_heads, "kv_heads": m.n_kv_heads,
            "head_dim": m.head_dim, "ffn": m.ffn_dim, "vocab": m.vocab, "weight_dtype": m.weight_dtype,
            "kv_dtype": m.kv_dtype, "batch": B, "positions": [r["first_pos"], r["first_pos"] + r["steps"] - 1],
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["achieved_gbps"], 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(r["achieved_gbps"] / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "decode_step_kernel" if B == 1 else "one tick (the kd_step kernel sequence)",
            "algorithmic_bytes_per_launch": round(r["alg_bytes"]),
            "kernel_mean_us": round(float(per_step_us.mean()), 2),
        },
        "stream_ceiling": None if ceiling is None else {
            "achieved_gbps": round(ceiling, 1),
            "frac_of_stream_ceiling": round(r["achieved_gbps"] / ceiling, 4),
            "kernel": "stream_read_kernel (kd_stream_read, 4 GiB of random bytes, 16-byte non-temporal loads)",
        },
        "roofline_tok_s": round(r["bound_tok_s"], 1),
        "frac_of_roofline_tok_s": round(r["tok_s"] / r["bound_tok_s"], 4),
        "itl_us": {"p50": round(float(np.percentile(per_step_us, 50)), 2), "p99": round(r["p99_us"], 2)},
        "resident": r["resident"],
        "ttft": r["ttft"],
        "cpu_baseline": r["cpu"],
        "extra": extra or None,
    }
    if ceiling is not None:
        for e in extra.values():
            e["frac_of_stream_ceiling"] = round(e["achieved_gbps"] / ceiling, 4)
    if B > 1:
        budget_us = args.tick_budget_ms * 1e3
        med = float(np.percentile(per_step_us, 50))
        out["tick_latency_ms"] = {"p50": round(med / 1e3, 4), "p99": round(r["p99_us"] / 1e3, 4),
                                  "max": round(float(per_step_us.max()) / 1e3, 4)}
        out["deadline"] = {
            "budget_ms": args.tick_budget_ms,
            "ticks": int(len(per_step_us)),
            "missed_ticks": int(np.sum(per_step_us > budget_us)),
            "missed_session_ticks": int(np.sum(per_step_us > budget_us)) * B,
            "ticks_over_1.1x_median": int(np.sum(per_step_us > 1.1 * med)),
        }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
