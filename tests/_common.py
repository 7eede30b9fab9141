"""Shared helpers for the GPU parity tests (input synthesis for the tiny case, oracle runs,
tolerance checks).  Nothing here is imported by the library."""
from __future__ import annotations

import sys
from typing import Dict, List, Optional

import numpy as np

import oracle.mla_oracle as orc
from mla_latent_kv_40_amd import workloads as wl


def bound(ref: np.ndarray, factor: float = 1.0) -> float:
    """max|gpu - oracle| allowed: 2e-2 * max|oracle| + 1e-3 (x4 for fp8 caches)."""
    return factor * (2e-2 * float(np.max(np.abs(ref))) + 1e-3)


def check(name: str, got, ref, factor: float = 1.0, extra_rel: Optional[float] = None) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    tol = bound(ref, factor)
    print(f"  {name}: max err {err:.3e}  tol {tol:.3e}  ratio {err / tol:.3f}  max|ref| {np.max(np.abs(ref)):.3e}",
          flush=True)
    assert err <= tol, f"{name}: max err {err:.3e} > tol {tol:.3e}"
    if extra_rel is not None:
        t2 = extra_rel * float(np.max(np.abs(ref))) + 1e-6
        assert err <= t2, f"{name}: max err {err:.3e} > {t2:.3e} (expected accuracy of this path)"
    return err / tol


def tiny_sequences(w: wl.Workload, bt: wl.Batch) -> List[Dict[str, np.ndarray]]:
    """GPU inputs of the tiny case, which starts from hidden states x: the latent, raw
    positional key and the two query parts, projected here in fp64 and handed over as fp32."""
    W = {k: np.asarray(v, dtype=np.float64) for k, v in bt.weights.items()}
    L = int(bt.kv_lens[0])
    x = W["x"]
    c = (x @ W["W_down"]).astype(np.float32)
    kr = (x @ W["W_KR"]).astype(np.float32)
    xq = x[L - w.sq:L]
    qc = (xq @ W["W_Q"]).reshape(w.sq, w.heads, w.d_h).astype(np.float32)
    qr = (xq @ W["W_QR"]).reshape(w.sq, w.heads, w.d_r).astype(np.float32)
    return [{"c": c, "k_r": kr, "q_c": qc, "q_r": qr}]


def oracle_for(w: wl.Workload, bt: wl.Batch, seqs, b: int, heads=None, weights=None) -> Dict[str, np.ndarray]:
    W = weights if weights is not None else bt.weights
    s = seqs[b]
    return orc.decode(s["c"], s["k_r"], s["q_c"], s["q_r"], W["W_UK"], W["W_UV"], int(bt.kv_lens[b]),
                      w.softmax_scale, w.rope_base, heads=heads)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()
