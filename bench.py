"""MLA decode benchmark on one MI355X: one JSON line.

A step is the whole decode path for one batch: mla_append_absorb (= mla_cache_append of the
step's new tokens and mla_absorb_q, in one launch), mla_decode_split + mla_decode_combine
(= mla_decode_attn), mla_out_proj.
The default workload is DeepSeek-V2-shaped bf16 decode at batch 64 with context lengths
drawn uniformly from [1024, 32768] (synthetic, seeded).  Inputs are resident in HBM before
the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--workload NAME] [--no-cpu-baseline]

Before the W warm-up steps, untimed steps run for at least MS milliseconds (default 300): from
idle the GPU's clocks take ~100 steps to settle, and the timed steps measure the steady state.

value       query tokens decoded per second (B*Sq per step / mean step time)
roofline    the split-K decode kernel: latent-cache bytes it must read per launch (1152 B per
            visible cached token in bf16, 580 B in fp8 incl. the scale) / its mean duration,
            against 8 TB/s; durations from HIP events on the launch stream.  traffic = HBM bytes
            per launch measured by rocprofv3 counters (profiles/decode_hbm_traffic.md), null
            when the kernel source differs from the one those counters were taken on
cpu_baseline the fp64 oracle on the host cores, on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
METRIC = "MLA decode tokens/s + latent-cache GB/s & TFLOP/s (% peak) at B=64, 32k ctx"


def algorithmic(w, kv_lens):
    """Bytes the decode kernel must read (the latent cache rows of every visible token) and
    the FLOPs of the latent-space attention: 2*H*(2*d_c + d_R) per visible (query, token)."""
    kv = kv_lens.astype(np.int64)
    tokens = int(kv.sum())
    per_tok = w.row * (1 if w.dtype == "fp8" else 2 if w.dtype == "bf16" else 4) + (4 if w.dtype == "fp8" else 0)
    visible = 0
    for j in range(w.sq):
        visible += int((kv - w.sq + j + 1).sum())
    flops = visible * 2 * w.heads * (2 * w.d_c + w.d_r)
    return tokens * per_tok, flops, tokens


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a calibration copy), or None when that summary was
    taken on a different decode.hip than the one built here."""
    import hashlib
    src = os.path.join(ROOT, "mla_latent_kv_40_amd", "csrc", "decode.hip")
    prof = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
    if not os.path.exists(prof):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for line in open(prof):
        f = line.split()
        if len(f) == 6 and f[0] == "traffic" and f[1] == kernel and f[2] == workload and f[5] == sha:
            return int(f[3])
    return None


def cpu_baseline(w, bt, budget_s=20.0):
    """Time the fp64 oracle on whole sequences near the batch's mean length until ~budget."""
    import oracle.mla_oracle as orc
    from mla_latent_kv_40_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    kv = bt.kv_lens.astype(np.int64)
    order = np.argsort(np.abs(kv - kv.mean()))
    done, toks, t0 = 0, 0, time.perf_counter()
    picked = []
    for b in order:
        s = wl.draw_sequence(w, int(b), int(kv[b]))
        orc.decode(s["c"], s["k_r"], s["q_c"], s["q_r"], bt.weights["W_UK"], bt.weights["W_UV"], int(kv[b]),
                   w.softmax_scale, w.rope_base)
        done += w.sq
        toks += int(kv[b])
        picked.append(int(kv[b]))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(picked)} of {w.batch} sequences (kv_len {picked}, nearest the batch mean "
                      f"{kv.mean():.0f}), all {w.heads} heads, fp64 numpy, {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the warm-up steps (the GPU leaves "
                         "its idle clocks over the first ~100 steps)")
    ap.add_argument("--workload", default="dsv2_b64_l1k_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device-to-device copy 3 times (scales HBM counters)")
    a = ap.parse_args()
    if a.calibrate_copy:
        import torch
        x = torch.empty(1 << 28, dtype=torch.uint8, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 28, "runs": 3}))
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the decode path is a single-GPU "
              "kernel; a multi-GPU split would shard whole sequences per GPU.", file=sys.stderr)
        return 2

    import torch
    from mla_latent_kv_40_amd import harness, workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = wl.get(a.workload)
    print(f"[bench] workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    t = time.perf_counter()
    bt = wl.draw_batch(w)
    seqs = harness.draw_all_sequences(w, bt)
    st = harness.DecodeState(w, bt, seqs, device="cuda:0")
    del seqs
    st.fill_context()
    print(f"[bench] setup {time.perf_counter() - t:.1f} s, cache {st.cache.numel() * st.cache.element_size() / 1e9:.2f} GB",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        st.append_absorb()
        if ev is not None:
            ev[0].record(stream)
        st.decode_split()
        if ev is not None:
            ev[1].record(stream)
        st.decode_combine()
        st.out_proj()

    # a GPU coming out of idle runs the first ~100 steps ~10% slower while its clocks ramp up;
    # steady-state throughput is measured after an untimed settle period and the warm-up steps
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < a.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms_per_step = wall * 1e3 / a.steps

    bytes_alg, flops, tokens = algorithmic(w, bt.kv_lens)
    k_s = float(split_ms.mean()) * 1e-3
    gbs = bytes_alg / k_s / 1e9
    tflops = flops / k_s / 1e12
    peak_mfma = PEAK_FP8_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
    # the kernel is bound by whichever roof it is closer to
    bound_hbm = gbs / PEAK_HBM_GBS >= tflops / peak_mfma
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)} if bound_hbm else
            {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak_mfma, "unit": "TFLOP/s",
             "frac": round(tflops / peak_mfma, 4)})
    roof["kernel"] = "decode_mfma_fp8_kernel" if w.dtype == "fp8" else "decode_mfma_bf16_kernel"
    roof["traffic"] = measured_traffic(roof["kernel"], w.name)
    value = w.batch * w.sq / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "settle": {"steps": settle_steps, "ms": a.settle_ms}, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1) latents/queries, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "batch": w.batch, "sq": w.sq, "kv_tokens": tokens,
                   "kv_len_min": int(bt.kv_lens.min()), "kv_len_max": int(bt.kv_lens.max()),
                   "heads": w.heads, "d_c": w.d_c, "d_r": w.d_r, "page_tokens": 64, "parallelism": "none"},
        "roofline": roof,
        "decode_split": {"ms": round(float(split_ms.mean()), 4), "ms_min": round(float(split_ms.min()), 4),
                         "cache_GBps": round(gbs, 1), "cache_frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4),
                         "TFLOPs": round(tflops, 1), "mfma_frac": round(tflops / peak_mfma, 4),
                         "bytes": bytes_alg, "flops": flops},
    }
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, bt)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
