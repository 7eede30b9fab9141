"""MLA decode benchmark on one MI355X: one JSON line.

A step is the whole decode path for one batch: mla_append_absorb (= mla_cache_append of the
step's new tokens and mla_absorb_q, in one launch), mla_decode_split + mla_decode_combine
(= mla_decode_attn), mla_out_proj.
The default workload is DeepSeek-V2-shaped bf16 decode at batch 64 with context lengths
drawn uniformly from [1024, 32768] (synthetic, seeded).  Inputs are resident in HBM before
the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--workload NAME]
                    [--no-cpu-baseline] [--no-configs] [--warm]

Timing.  Before every step (settle, warm-up and timed) a 512 MiB buffer is written, outside
the timed events, so that no step starts with the latent cache in the 256 MB last-level cache
(a decode step of one layer follows other layers' work in a model).  Each timed step is
bracketed by HIP events on the launch stream: step (all kernels), split (K1), combine (K2).
Untimed steps run for at least MS milliseconds first (default 300): from idle the GPU's clocks
take ~100 steps to settle.  --warm adds the same measurement without the buffer writes.

value       query tokens decoded per second: B*Sq / mean step time (flushed steps)
roofline    the split-K decode (K1 split + K2 combine): latent-cache bytes it must read per step
            (1152 B per cached token in bf16, 580 B in fp8 incl. the scale, 578.25 B with tile scales) / mean(K1 + K2),
            against 8 TB/s; the K1-only figure alongside.  traffic = HBM bytes per step of K1 + K2
            from rocprofv3 counters (profiles/decode_hbm_traffic.md), null when the kernel source
            differs from the one those counters were taken on
configs     the same measurement (shorter) for each DeepSeek-V2-shaped workload and the tiny
            fp32 case, with its bound and roofline fraction, and the oracle's max error / tolerance
            on the sequences its CPU sample covers
cpu_baseline the fp64 oracle on the host cores, on a bounded sample of the same workload
attainable  what the box reaches on plain work (with the configs): a 1 GiB copy, read streams
            of ~1 GB (plain vector loads, and the split's buffer->LDS loads and LDS ring without
            its arithmetic), the vendor bf16 GEMM and a loop of the split's matrix instructions;
            and the split-K decode's read and matrix rates against the best of them
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_TFLOPS = 157.3
METRIC = "MLA decode tokens/s + latent-cache GB/s & TFLOP/s (% peak) at B=64, 32k ctx"
FLUSH_BYTES = 512 << 20
# the five decode workloads, smallest first (the first is latency-bound)
CONFIGS = ["tiny_f32", "dsv2_b16_l4k", "dsv2_b64_l1k_32k", "dsv2_b32_l8k_sq4", "dsv2_b128_l8k_fp8"]
# measured alongside them: every context at 32768, a chunked prefill step (512 new tokens per
# sequence) and the fp8 step with the block-scaled cache
EXTRA_CONFIGS = ["dsv2_b64_l32k", "dsv2_b4_l8k_sq512", "dsv2_b128_l8k_fp8b"]


def algorithmic(w, kv_lens):
    """Bytes the decode must read (the latent cache rows of every cached token) and the FLOPs of
    the latent-space attention: 2*H*(2*d_c + d_R) per visible (query, token)."""
    kv = kv_lens.astype(np.int64)
    tokens = int(kv.sum())
    per_tok = w.cache_bytes_per_token   # row bytes plus the scales' share
    visible = 0
    for j in range(w.sq):
        visible += int(np.maximum(kv - w.sq + j + 1, 0).sum())
    flops = visible * 2 * w.heads * (2 * w.d_c + w.d_r)
    return int(round(tokens * per_tok)), flops, tokens


def measured_traffic(workload):
    """HBM bytes per step of the split and combine kernels on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a calibration copy), or None
    when that summary was taken on a different decode.hip than the one built here."""
    import hashlib
    src = os.path.join(ROOT, "mla_latent_kv_40_amd", "csrc", "decode.hip")
    prof = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
    if not os.path.exists(prof):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for line in open(prof):
        f = line.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == workload and f[4] == sha:
            return int(f[2])
    return None


READ_CLOCK = True   # --no-clock: no rocm-smi child (under a profiler, whose preload covers children)


def gpu_clock_mhz():
    """Current shader clock of GPU 0 from rocm-smi (None if it cannot be read or --no-clock)."""
    if not READ_CLOCK:
        return None
    smi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        r = subprocess.run([smi, "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return None
    for card in d.values():
        for k, v in card.items():
            if "sclk" in k.lower() and "clock" in k.lower():
                try:
                    return float(str(v).strip("()Mhz MHz"))
                except ValueError:
                    pass
    return None


def cpu_baseline(w, bt, seqs_gpu_out, budget_s=20.0, heads=None):
    """Time the fp64 oracle on whole sequences near the batch's mean length until ~budget, and
    compare its outputs with the GPU's (max error / tolerance of the oracle gate, 4x for fp8)."""
    import oracle.mla_oracle as orc
    from mla_latent_kv_40_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    kv = bt.kv_lens.astype(np.int64)
    order = np.argsort(np.abs(kv - kv.mean()), kind="stable")
    done, t0 = 0, time.perf_counter()
    picked = []
    worst = 0.0
    factor = 4.0 if w.fp8 else 1.0
    hs = list(range(w.heads)) if heads is None else list(heads)
    for b in order:
        b = int(b)
        if w.d_model is not None:   # the tiny case starts at hidden states
            W = bt.weights
            L = int(kv[b])
            C, KR, qC, qR = orc.project_from_hidden(W["x"], W["W_down"], W["W_KR"], W["W_Q"], W["W_QR"], w.heads,
                                                    w.d_h, w.d_r, list(range(L - w.sq, L)))
            s = {"c": C, "k_r": KR, "q_c": qC, "q_r": qR}
        else:
            s = wl.draw_sequence(w, b, int(kv[b]))
        ref = orc.decode(s["c"], s["k_r"], s["q_c"], s["q_r"], bt.weights["W_UK"], bt.weights["W_UV"], int(kv[b]),
                         w.softmax_scale, w.rope_base, heads=hs)
        done += w.sq
        picked.append(int(kv[b]))
        rows = slice(b * w.sq, (b + 1) * w.sq)
        for k in ("o", "o_lat", "lse"):
            got = seqs_gpu_out[k][rows][:, hs].astype(np.float64)
            tol = factor * (2e-2 * float(np.max(np.abs(ref[k]))) + 1e-3)
            worst = max(worst, float(np.max(np.abs(got - ref[k]))) / tol)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    scale = w.heads / len(hs)
    return {"value": done / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(picked)} of {w.batch} sequences (kv_len {picked[:24]}{' ...' if len(picked) > 24 else ''}, "
                      f"nearest the batch mean {kv.mean():.0f}), {len(hs)} of {w.heads} heads (rate scaled to all "
                      f"heads), fp64 numpy, {dt:.1f} s",
            "max_err_over_tol": round(worst, 4)}


def run_workload(name, steps, warmup, settle_ms, flush, warm, cpu_budget, log):
    import torch
    from mla_latent_kv_40_amd import harness, workloads as wl

    w = wl.get(name)
    log(f"[bench] workload {w.name}: {w.description}")
    t = time.perf_counter()
    bt = wl.draw_batch(w)
    if w.d_model is not None:
        W = {k: np.asarray(v, dtype=np.float64) for k, v in bt.weights.items()}
        L = int(bt.kv_lens[0])
        x = W["x"]
        xq = x[L - w.sq:L]
        seqs = [{"c": (x @ W["W_down"]).astype(np.float32), "k_r": (x @ W["W_KR"]).astype(np.float32),
                 "q_c": (xq @ W["W_Q"]).reshape(w.sq, w.heads, w.d_h).astype(np.float32),
                 "q_r": (xq @ W["W_QR"]).reshape(w.sq, w.heads, w.d_r).astype(np.float32)}]
    else:
        seqs = harness.draw_all_sequences(w, bt)
    st = harness.DecodeState(w, bt, seqs, device="cuda:0")
    del seqs
    st.fill_context()
    log(f"[bench] setup {time.perf_counter() - t:.1f} s, cache {st.cache.numel() * st.cache.element_size() / 1e9:.2f} GB")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st.append_absorb()
        if ev is not None:
            ev[1].record(stream)
        st.decode_split()
        if ev is not None:
            ev[2].record(stream)
        st.decode_combine()
        if ev is not None:
            ev[3].record(stream)
        st.out_proj()
        if ev is not None:
            ev[4].record(stream)

    def timed(n, with_flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if with_flush:
                flush.fill_(i & 255)
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = np.array([[e[0].elapsed_time(e[4]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
        return ms, wall

    # settle (the clocks leave their idle state) and warm up, under the same conditions as the
    # timed steps
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(10):
            flush.fill_(settle_steps & 255)
            step()
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        flush.fill_(i & 255)
        step()
    torch.cuda.synchronize()
    ms, wall = timed(steps, True)
    # the shader clock under this load: queue ~200 ms of steps, read the clock while they run
    n_clk = max(1, int(200.0 / max(float(ms[:, 0].mean()), 1e-3)))
    for i in range(n_clk):
        flush.fill_(i & 255)
        step()
    clk = gpu_clock_mhz()
    torch.cuda.synchronize()

    bytes_alg, flops, tokens = algorithmic(w, bt.kv_lens)
    step_ms, k1_ms, k2_ms = ms[:, 0], ms[:, 1], ms[:, 2]
    k12_ms = k1_ms + k2_ms
    peak_mfma = PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    intensity = flops / bytes_alg
    hbm_bound = intensity < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)

    def roof(t_ms):
        gbs = bytes_alg / (t_ms * 1e-3) / 1e9
        tfl = flops / (t_ms * 1e-3) / 1e12
        if hbm_bound:
            return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
        return {"bound": "mfma", "achieved": round(tfl, 1), "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(tfl / peak_mfma, 4)}

    def pct(x):
        return {"mean": round(float(x.mean()), 4), "median": round(float(np.median(x)), 4),
                "p10": round(float(np.percentile(x, 10)), 4), "p90": round(float(np.percentile(x, 90)), 4),
                "min": round(float(x.min()), 4)}

    k1_name = ("decode_mfma_fp8_kernel" if w.fp8 else "decode_mfma_bf16_kernel" if w.dtype == "bf16"
               else "decode_generic_kernel")
    r = {
        "workload": w.name, "batch": w.batch, "sq": w.sq, "dtype": w.dtype, "kv_tokens": tokens,
        "kv_len_min": int(bt.kv_lens.min()), "kv_len_max": int(bt.kv_lens.max()),
        "tokens_per_s": round(w.batch * w.sq / (float(step_ms.mean()) * 1e-3), 1),
        "ms_per_step": round(float(step_ms.mean()), 4), "wall_ms_per_step_incl_flush": round(wall * 1e3 / steps, 4),
        "step_ms": pct(step_ms), "k1_split_ms": pct(k1_ms), "k2_combine_ms": pct(k2_ms), "k1_k2_ms": pct(k12_ms),
        "bytes": bytes_alg, "flops": flops, "flop_per_byte": round(intensity, 1),
        "roofline": dict(roof(float(k12_ms.mean())), kernel=f"{k1_name} + combine_kernel"),
        "roofline_k1_only": dict(roof(float(k1_ms.mean())), kernel=k1_name),
        "mfma_frac_k1_k2": round(flops / (float(k12_ms.mean()) * 1e-3) / 1e12 / peak_mfma, 4),
        "sclk_mhz_under_load": clk, "settle_steps": settle_steps,
    }
    if warm:
        ms_w, _ = timed(steps, False)
        r["warm_no_flush"] = {"ms_per_step": round(float(ms_w[:, 0].mean()), 4),
                              "k1_k2_ms": pct(ms_w[:, 1] + ms_w[:, 2])}
    if cpu_budget > 0:
        log(f"[bench] cpu baseline (fp64 oracle, ~{cpu_budget:.0f} s) ...")
        got = {"o": st.out.float().cpu().numpy(), "o_lat": st.o_lat.cpu().numpy(), "lse": st.lse.cpu().numpy()}
        # a head subset keeps one oracle sequence within the budget (many query rows per sequence
        # cost the oracle Sq times a decode)
        n_heads = w.heads if (cpu_budget >= 10 and w.sq <= 4) else (16 if w.sq <= 4 else 4)
        heads = None if n_heads >= w.heads else list(range(0, w.heads, w.heads // n_heads))
        r["cpu_baseline"] = cpu_baseline(w, bt, got, budget_s=cpu_budget, heads=heads)
    del st
    torch.cuda.empty_cache()
    return r


def kv_cache_comparison(name, steps, flush, log, kv_heads=(128, 8)):
    """The same batch (lengths, pages) decoded from a per-head key/value cache: multi-head attention
    (128 key/value heads of width 128, 65,536 B per token in bf16) and grouped-query attention
    (8 key/value heads, 4,096 B per token), with mla_kv_decode_attn.  Cache contents are random
    (timing only); the split + combine time per step against the bytes each token holds."""
    import torch
    from mla_latent_kv_40_amd import binding as B, workloads as wl

    w = wl.get(name)
    bt = wl.draw_batch(w)
    kv = bt.kv_lens.astype(np.int64)
    tokens = int(kv.sum())
    cfg = B.Config(num_heads=w.heads, d_c=w.d_c, d_r=w.d_r, d_h=128, d_v=128, softmax_scale=128 ** -0.5)
    table = torch.from_numpy(bt.block_table).to("cuda:0")
    lens = torch.from_numpy(bt.kv_lens).to("cuda:0")
    q = torch.randn((w.batch, w.heads, 128), dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty((w.batch, w.heads, 128), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda:0")
    out = {}
    for h_kv in kv_heads:
        per_tok = 2 * h_kv * 128 * 2
        log(f"[bench] per-head key/value cache, {h_kv} key/value heads: {tokens * per_tok / 1e9:.1f} GB")
        k = torch.randn((bt.num_blocks, h_kv, 64, 128), dtype=torch.bfloat16, device="cuda:0")
        v = torch.randn((bt.num_blocks, h_kv, 128, 64), dtype=torch.bfloat16, device="cuda:0")
        ws = B.mla_kv_decode_workspace_size(cfg, h_kv, w.batch, bt.max_blocks)
        work = torch.empty(ws, dtype=torch.uint8, device="cuda:0")
        stream = torch.cuda.current_stream()

        def run():
            B.mla_kv_decode_attn(cfg, h_kv, q, k, v, bt.num_blocks, table, bt.max_blocks, lens, w.batch, work, ws,
                                 o, lse)
        for i in range(3):
            flush.fill_(i & 255)
            run()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            flush.fill_(i & 255)
            evs[i][0].record(stream)
            run()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        gbs = tokens * per_tok / (ms.mean() * 1e-3) / 1e9
        out[f"{'mha' if h_kv == w.heads else 'gqa'}_{h_kv}_kv_heads"] = {
            "bytes_per_token": per_tok, "cache_GB": round(tokens * per_tok / 1e9, 2),
            "ms_mean": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
            "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4),
            "tokens_per_s": round(w.batch / (ms.mean() * 1e-3), 1)}
        del k, v, work
        torch.cuda.empty_cache()
    return out


def model_width_measurement(name, steps, flush, log, d_model=5120):
    """The projections on either side of the decode for the default batch's step (T = B query rows,
    B new tokens), from d_model = 5120 (DeepSeek-V2's hidden size): mla_append_absorb_hidden (reads
    [W_down | W_KR] and [W_Q | W_QR], 257 MB) and mla_out_proj_folded (reads W_O' = H*d_c*d_model
    values, 671 MB).  Weights are random (timing only); bandwidth = weight bytes / time."""
    import torch
    from mla_latent_kv_40_amd import binding as B, harness, workloads as wl

    w = wl.get(name)
    bt = wl.draw_batch(w)
    cfg = harness.config_for(w)
    T = w.batch * w.sq
    H = w.heads
    dev = dict(dtype=torch.bfloat16, device="cuda:0")
    cache = torch.empty((bt.num_blocks, 64, w.row), **dev)
    table = torch.from_numpy(bt.block_table).to("cuda:0")
    h = torch.randn((T, d_model), **dev)
    w_dkv = torch.randn((w.d_c + w.d_r, d_model), **dev) * d_model ** -0.5
    w_q = torch.randn((H * (w.d_h + w.d_r), d_model), **dev) * d_model ** -0.5
    w_uk = torch.randn((w.d_c, H * w.d_h), **dev) * w.d_c ** -0.5
    kv = bt.kv_lens.astype(np.int64)
    pos = torch.from_numpy((kv - 1).astype(np.int32)).to("cuda:0")
    seq = torch.arange(T, dtype=torch.int32, device="cuda:0")
    q_abs = torch.empty((T, H, w.row), **dev)
    ws = B.mla_hidden_workspace_size(cfg, d_model, T, T)
    work = torch.empty(ws, dtype=torch.uint8, device="cuda:0")
    o_lat = torch.randn((T, H, w.d_c), dtype=torch.float32, device="cuda:0") * 0.05
    w_fold = torch.randn((d_model, H * w.d_c), **dev) * (H * w.d_c) ** -0.5
    out = torch.empty((T, d_model), **dev)
    wso = max(B.mla_out_proj_folded_workspace_size(cfg, d_model, T), 256)
    work_o = torch.empty(wso, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    calls = {
        "append_absorb_hidden": (lambda: B.mla_append_absorb_hidden(
            cfg, d_model, h, w_dkv, cache, None, bt.num_blocks, pos, seq, table, w.batch, bt.max_blocks, T, h, w_q,
            pos, w_uk, q_abs, T, work, ws), (w_dkv.numel() + w_q.numel() + w_uk.numel()) * 2),
        "out_proj_folded": (lambda: B.mla_out_proj_folded(cfg, d_model, o_lat, w_fold, out, T, work_o, wso),
                            w_fold.numel() * 2),
    }
    res = {"d_model": d_model, "rows": T}
    for key, (fn, wbytes) in calls.items():
        for i in range(3):
            flush.fill_(i & 255)
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            flush.fill_(i & 255)
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        gbs = wbytes / (ms.mean() * 1e-3) / 1e9
        res[key] = {"ms_mean": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
                    "weight_bytes": int(wbytes), "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench] {key}: {ms.mean():.3f} ms, {gbs:.0f} GB/s of weights")
    return res


ATTAINABLE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_kv_40_amd",
                              "libmla_attainable.so")
LOOP_FLOP = {0: 32 * 32 * 16 * 2, 1: 32 * 32 * 64 * 2}   # per instruction: bf16, scaled fp8
LDS_PER_CU = 163840


def mfma_loop_rates(log, settle_ms=300.0):
    """The matrix rate the chip sustains: libmla_attainable's loop of independent matrix
    instructions (no memory traffic) on every compute unit, launched back to back for settle_ms
    before 20 timed launches (median).  One workgroup of four waves per compute unit (all of its
    LDS reserved, the decode split's occupancy), and two per compute unit."""
    import ctypes
    import torch
    if not os.path.exists(ATTAINABLE_LIB):
        raise RuntimeError(f"{ATTAINABLE_LIB} is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(ATTAINABLE_LIB)
    fn = L.mla_attainable_mfma_loop
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda:0")
    r = {}
    for kind, name, iters in ((0, "bf16", 2048), (1, "fp8", 1024)):
        for per_cu in (1, 2):
            wgs, it = cus * per_cu, iters // per_cu

            def launch():
                rc = fn(kind, wgs, it, LDS_PER_CU // per_cu, out.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mla_attainable_mfma_loop returned {rc}")
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < settle_ms * 1e-3:
                for _ in range(20):
                    launch()
                torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for e0, e1 in evs:
                e0.record(stream); launch(); e1.record(stream)
            torch.cuda.synchronize()
            ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
            flop = wgs * 4 * it * 4 * LOOP_FLOP[kind]
            key = f"{name}_mfma_loop_TFLOPs" + ("" if per_cu == 1 else "_2wg_per_cu")
            r[key] = round(flop / (ms * 1e-3) / 1e12, 1)
    del out
    log(f"[bench] matrix-instruction loop: {r}")
    return r


READ_CHUNK = 36864   # one chunk of libmla_attainable's read streams (a bf16 half page)


def read_rates(log, settle_ms=200.0):
    """The HBM read bandwidth the chip sustains: libmla_attainable's read streams over a
    ~1.06 GB buffer (bytes read / time, median of 20 launches after settle_ms of launches back
    to back).  `read_vgpr` uses plain vector loads at 1, 4 and 8 workgroups per compute unit;
    `read_lds` the decode split's buffer->LDS loads and four-stage LDS ring at one workgroup per
    compute unit, the split's occupancy."""
    import ctypes
    import torch
    L = ctypes.CDLL(ATTAINABLE_LIB)
    fn = L.mla_attainable_read
    fn.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = cus * READ_CHUNK * 112          # a multiple of every workgroup count below
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    out = torch.empty(8 * cus * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    r = {}
    for kind, name, per_cu in ((0, "read_vgpr", 1), (0, "read_vgpr", 4), (0, "read_vgpr", 8), (1, "read_lds", 1)):
        wgs = cus * per_cu

        def launch():
            rc = fn(kind, buf.data_ptr(), nbytes, wgs, out.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"mla_attainable_read returned {rc}")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_ms * 1e-3:
            for _ in range(10):
                launch()
            torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in evs:
            e0.record(stream); launch(); e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
        key = f"{name}_GBps" + ("" if kind == 1 else f"_{per_cu}wg_per_cu")
        r[key] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, out
    log(f"[bench] read streams: {r}")
    return r


def attainable(log):
    """What the box reaches, next to the published peaks: a 1 GiB device-to-device copy (bytes
    read + written / time), an 8192^3 bf16 matrix product (torch.matmul, i.e. the vendor GEMM
    library) and the plain matrix-instruction loop (mfma_loop_rates).  Reference points only:
    none is part of the decode path."""
    import torch
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for _ in range(3):
        y.copy_(x)
    for a, b in evs:
        a.record(); y.copy_(x); b.record()
    torch.cuda.synchronize()
    copy_ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    del x, y
    n = 8192
    A = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    Bm = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):
        C = A @ Bm
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in evs:
        a.record(); C = A @ Bm; b.record()
    torch.cuda.synchronize()
    mm_ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    del A, Bm, C
    r = {"copy_GBps": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
         "bf16_gemm_8192_TFLOPs": round(2 * n ** 3 / (mm_ms * 1e-3) / 1e12, 1)}
    r.update(read_rates(log))
    r.update(mfma_loop_rates(log))
    log(f"[bench] attainable: {r}")
    return r


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the warm-up steps (the GPU leaves "
                         "its idle clocks over the first ~100 steps)")
    ap.add_argument("--workload", default="dsv2_b64_l1k_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration measurements")
    ap.add_argument("--no-clock", action="store_true", help="do not read the shader clock with rocm-smi")
    ap.add_argument("--warm", action="store_true", help="also time the steps without the cache flush")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device-to-device copy 3 times (scales HBM counters)")
    a = ap.parse_args()
    global READ_CLOCK
    READ_CLOCK = not a.no_clock
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
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the decode path is measured on "
              "one GPU; a multi-GPU run would shard whole sequences per GPU and is not provided.", file=sys.stderr)
        return 2

    import torch

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    main_r = run_workload(a.workload, a.steps, a.warmup, a.settle_ms, flush, a.warm,
                          0.0 if a.no_cpu_baseline else 20.0, log)
    configs = {}
    if not a.no_configs:
        for name in CONFIGS + EXTRA_CONFIGS:
            if name == a.workload:
                configs[name] = {k: main_r[k] for k in ("tokens_per_s", "ms_per_step", "k1_k2_ms", "roofline",
                                                        "flop_per_byte", "sclk_mhz_under_load")}
                if "cpu_baseline" in main_r:
                    configs[name]["max_err_over_tol"] = main_r["cpu_baseline"]["max_err_over_tol"]
                continue
            r = run_workload(name, 50, 10, 100.0, flush, False, 0.0 if a.no_cpu_baseline else 3.0, log)
            configs[name] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "k1_k2_ms", "roofline",
                                               "flop_per_byte", "sclk_mhz_under_load")}
            if "cpu_baseline" in r:
                configs[name]["max_err_over_tol"] = r["cpu_baseline"]["max_err_over_tol"]
                configs[name]["oracle_sample"] = r["cpu_baseline"]["sample"]

    kv_cmp = None
    if not a.no_configs and a.workload == "dsv2_b64_l1k_32k":
        kv_cmp = kv_cache_comparison(a.workload, 10, flush, log)
        kv_cmp["mla_latent"] = {"bytes_per_token": 1152, "ms_mean_k1_k2": main_r["k1_k2_ms"]["mean"],
                                "tokens_per_s_k1_k2": round(main_r["batch"] / (main_r["k1_k2_ms"]["mean"] * 1e-3), 1)}

    width = None
    if not a.no_configs and a.workload == "dsv2_b64_l1k_32k":
        width = model_width_measurement(a.workload, 20, flush, log)
    reach = attainable(log) if not a.no_configs else None

    roof = dict(main_r["roofline"])
    roof["traffic"] = measured_traffic(main_r["workload"])
    line = {
        "metric": METRIC, "value": main_r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "settle": {"steps": main_r["settle_steps"], "ms": a.settle_ms},
        "ms_per_step": main_r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": main_r["dtype"],
        "data": "synthetic (seeded N(0,1) latents/queries, N(0,1/fan_in) weights)",
        "config": {"workload": main_r["workload"], "batch": main_r["batch"], "sq": main_r["sq"],
                   "kv_tokens": main_r["kv_tokens"], "kv_len_min": main_r["kv_len_min"],
                   "kv_len_max": main_r["kv_len_max"], "heads": 128, "d_c": 512, "d_r": 64, "page_tokens": 64,
                   "parallelism": "none", "llc_flush_bytes_between_steps": FLUSH_BYTES},
        "roofline": roof,
        "roofline_k1_only": main_r["roofline_k1_only"],
        "timing_ms": {k: main_r[k] for k in ("step_ms", "k1_split_ms", "k2_combine_ms", "k1_k2_ms")},
        "wall_ms_per_step_incl_flush": main_r["wall_ms_per_step_incl_flush"],
        "mfma_frac_k1_k2": main_r["mfma_frac_k1_k2"],
        "sclk_mhz_under_load": main_r["sclk_mhz_under_load"],
        "bytes_per_step": main_r["bytes"], "flops_per_step": main_r["flops"],
    }
    if "warm_no_flush" in main_r:
        line["warm_no_flush"] = main_r["warm_no_flush"]
    if configs:
        line["configs"] = configs
    if kv_cmp:
        line["kv_cache_comparison"] = kv_cmp
    if width:
        line["model_width_projections"] = width
    if reach:
        # the split-K decode's matrix rate (K1 + K2, algorithmic FLOPs) against the loop's
        loop = reach["fp8_mfma_loop_TFLOPs" if main_r["dtype"].startswith("fp8") else "bf16_mfma_loop_TFLOPs"]
        tfl = main_r["flops"] / (main_r["k1_k2_ms"]["mean"] * 1e-3) / 1e12
        reach["k1_k2_TFLOPs"] = round(tfl, 1)
        reach["k1_k2_of_mfma_loop"] = round(tfl / loop, 4)
        # the split-K decode's latent-cache read rate (K1 + K2) against the best read stream
        gbps = main_r["bytes"] / (main_r["k1_k2_ms"]["mean"] * 1e-3) / 1e9
        best = max(v for k, v in reach.items() if k.startswith("read_"))
        reach["k1_k2_GBps"] = round(gbps, 1)
        reach["k1_k2_of_best_read_stream"] = round(gbps / best, 4)
        line["attainable"] = reach
    if "cpu_baseline" in main_r:
        line["cpu_baseline"] = main_r["cpu_baseline"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
