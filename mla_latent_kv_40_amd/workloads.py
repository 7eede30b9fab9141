"""Seeded synthetic inputs for MLA decode (shared by the GPU path's harness and by the tests).

This module only *draws* inputs: random normals, integer lengths, block-table
permutations, and the rounding of those draws to the number format that is
handed across the C ABI (bf16 or fp32).  It contains none of the method's
arithmetic (no projection, RoPE, attention or quantisation), so the oracle and
the HIP path can both take their inputs from here without sharing any of the
computation they are compared on.

Shapes follow DeepSeek-V2 (latent width d_c = 512 is the figure the talentme
"Multi-head Latent Attention" card gives under "Core Definition"); the tiny
fp32 case follows the numpy snippet of the katajob interview page ("code":
d_model 512, 8 heads, head dim 64, latent 64, 10 tokens).

Random streams
--------------
* global stream  ``PCG64(SeedSequence([seed, 0]))``: lengths, block-table
  permutation, weights (and x for the tiny case), in that order;
* per-sequence stream ``PCG64(SeedSequence([seed, 1, b]))``: the latents c,
  the raw positional keys k_R, the content query q^C and the positional query
  q^R of sequence b, in that order.

Per-sequence streams let a check regenerate one sequence without drawing the
whole batch.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BLOCK = 64  # tokens per cache page


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    sq: int                 # new query tokens per sequence in one step
    heads: int
    d_h: int                # per-head content (nope) dim of q and k
    d_r: int                # decoupled RoPE dim
    d_c: int                # latent dim
    d_v: int                # per-head value dim
    dtype: str              # "f32" | "bf16" | "fp8" | "fp8b" (cache format; activations bf16 for fp8:
                            # "fp8" one scale per token, "fp8b" one power-of-two scale per tile of
                            # 32 tokens x 32 columns)
    ctx_lo: int             # context before the step's new tokens (inclusive range)
    ctx_hi: int
    d_model: Optional[int] = None   # set only for the tiny case, whose inputs start at x
    rope_base: float = 10000.0
    description: str = ""

    @property
    def row(self) -> int:
        return self.d_c + self.d_r

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(d_h + d_R): content and positional keys concatenated.
        return 1.0 / float(np.sqrt(self.d_h + self.d_r))

    @property
    def act_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"

    @property
    def fp8(self) -> bool:
        return self.dtype in ("fp8", "fp8b")

    @property
    def cache_bytes_per_token(self) -> float:
        """Row bytes plus the scales' share: 4 per token (fp8), 36 scales x 4 bytes per 64-token
        page (fp8b)."""
        if self.dtype == "fp8":
            return self.row + 4.0
        if self.dtype == "fp8b":
            return self.row + 4.0 * 2 * (self.row // 32) / BLOCK
        return self.row * (2.0 if self.dtype == "bf16" else 4.0)


def _ds(name, seed, batch, sq, dtype, lo, hi, desc):
    return Workload(name=name, seed=seed, batch=batch, sq=sq, heads=128, d_h=128, d_r=64,
                    d_c=512, d_v=128, dtype=dtype, ctx_lo=lo, ctx_hi=hi, description=desc)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload(
        name="tiny_f32", seed=0, batch=1, sq=1, heads=8, d_h=64, d_r=16, d_c=64, d_v=64,
        dtype="f32", ctx_lo=9, ctx_hi=9, d_model=512,
        description="1 sequence of 10 tokens (9 cached + 1 new), d_model 512, H 8, d_h 64, "
                    "d_c 64, d_R 16, fp32, inputs from x"),
    "dsv2_b16_l4k": _ds("dsv2_b16_l4k", 1, 16, 1, "bf16", 4095, 4095,
                        "DeepSeek-V2 shapes, bf16, B=16, every context 4096"),
    "dsv2_b64_l1k_32k": _ds("dsv2_b64_l1k_32k", 2, 64, 1, "bf16", 1023, 32767,
                            "DeepSeek-V2 shapes, bf16, B=64, context U[1024, 32768]"),
    "dsv2_b64_l32k": _ds("dsv2_b64_l32k", 2, 64, 1, "bf16", 32767, 32767,
                         "DeepSeek-V2 shapes, bf16, B=64, every context 32768"),
    "dsv2_b32_l8k_sq4": _ds("dsv2_b32_l8k_sq4", 3, 32, 4, "bf16", 8192, 8192,
                            "DeepSeek-V2 shapes, bf16, B=32, context 8192 + 4 causal new tokens"),
    "dsv2_b128_l8k_fp8": _ds("dsv2_b128_l8k_fp8", 4, 128, 1, "fp8", 8191, 8191,
                             "DeepSeek-V2 shapes, fp8 e4m3 cache with per-token scale, B=128, "
                             "context 8192"),
    # the same step and inputs with the block-scaled fp8 cache (32 x 32 tiles, power-of-two scales)
    "dsv2_b128_l8k_fp8b": _ds("dsv2_b128_l8k_fp8b", 4, 128, 1, "fp8b", 8191, 8191,
                              "DeepSeek-V2 shapes, fp8 e4m3 cache with a power-of-two scale per tile of "
                              "32 tokens x 32 columns, B=128, context 8192"),
    # not one of the decode configurations: a chunk of prompt tokens extended in one step
    "dsv2_b4_l8k_sq512": _ds("dsv2_b4_l8k_sq512", 5, 4, 512, "bf16", 8192, 8192,
                             "DeepSeek-V2 shapes, bf16, chunked prefill: B=4, context 8192 + a chunk of "
                             "512 causal new tokens"),
}


def get(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller batch, lengths, ...)."""
    w = WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); result kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _as_input(w: Workload, x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    return x if w.act_dtype == "f32" else round_bf16(x)


def _global_rng(w: Workload) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0])))


def _seq_rng(w: Workload, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 1, b])))


@dataclasses.dataclass
class Batch:
    """Everything the step needs except the per-sequence tensors (drawn lazily)."""
    w: Workload
    kv_lens: np.ndarray        # [B] int32, tokens visible to the last query (context + sq)
    block_table: np.ndarray    # [B, max_blocks] int32 physical page ids (-1 past the end)
    num_blocks: int            # pool size
    weights: Dict[str, np.ndarray]   # W_UK [d_c, H*d_h], W_UV [d_c, H*d_v] (+ tiny-case extras)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def draw_batch(w: Workload) -> Batch:
    """Lengths, a shuffled page pool, and weights ~ N(0, 1/fan_in)."""
    g = _global_rng(w)
    if w.ctx_lo == w.ctx_hi:
        ctx = np.full(w.batch, w.ctx_lo, dtype=np.int64)
    else:
        ctx = g.integers(w.ctx_lo, w.ctx_hi, size=w.batch, endpoint=True)
    kv_lens = (ctx + w.sq).astype(np.int32)
    nblk = (kv_lens.astype(np.int64) + BLOCK - 1) // BLOCK
    pool = int(nblk.sum())
    perm = g.permutation(pool).astype(np.int32)
    max_blocks = int(nblk.max())
    table = np.full((w.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += int(nblk[b])
    H, dh, dv, dc, dr = w.heads, w.d_h, w.d_v, w.d_c, w.d_r
    weights: Dict[str, np.ndarray] = {}

    def normal(shape, fan_in):
        return _as_input(w, g.standard_normal(shape, dtype=np.float32) / np.float32(np.sqrt(fan_in)))

    if w.d_model is not None:
        dm = w.d_model
        L = int(kv_lens[0])
        weights["x"] = _as_input(w, g.standard_normal((L, dm), dtype=np.float32))
        weights["W_down"] = normal((dm, dc), dm)
        weights["W_UK"] = normal((dc, H * dh), dc)
        weights["W_UV"] = normal((dc, H * dv), dc)
        weights["W_QR"] = normal((dm, H * dr), dm)
        weights["W_Q"] = normal((dm, H * dh), dm)
        weights["W_KR"] = normal((dm, dr), dm)
        weights["W_O"] = normal((H * dv, dm), H * dv)
    else:
        weights["W_UK"] = normal((dc, H * dh), dc)
        weights["W_UV"] = normal((dc, H * dv), dc)
    return Batch(w=w, kv_lens=kv_lens, block_table=table, num_blocks=pool, weights=weights)


def draw_sequence(w: Workload, b: int, kv_len: int) -> Dict[str, np.ndarray]:
    """Per-sequence draws: c [L, d_c], k_R before RoPE [L, d_R], q^C [Sq, H, d_h], q^R [Sq, H, d_R].

    Only for workloads that start from the latent (not the tiny case, which starts at x).
    All values ~ N(0, 1), rounded to the input format.
    """
    assert w.d_model is None
    g = _seq_rng(w, b)
    L = int(kv_len)
    c = _as_input(w, g.standard_normal((L, w.d_c), dtype=np.float32))
    kr = _as_input(w, g.standard_normal((L, w.d_r), dtype=np.float32))
    qc = _as_input(w, g.standard_normal((w.sq, w.heads, w.d_h), dtype=np.float32))
    qr = _as_input(w, g.standard_normal((w.sq, w.heads, w.d_r), dtype=np.float32))
    return {"c": c, "k_r": kr, "q_c": qc, "q_r": qr}


def draw_hidden(w: Workload, d_model: int, kv_lens) -> Dict[str, np.ndarray]:
    """Hidden-state inputs for a DeepSeek-V2-shaped workload run from the model width: the
    projection weights W_down [d_model, d_c], W_KR [d_model, d_R], W_Q [d_model, H*d_h],
    W_QR [d_model, H*d_R], the output projection W_O [H*d_v, d_model] (all ~ N(0, 1/fan_in)) and
    hidden states x_b [kv_len_b, d_model] ~ N(0, 1) per sequence, rounded to the input format.
    Drawn from their own streams (PCG64(SeedSequence([seed, 2])) for the weights,
    [seed, 3, b] for sequence b), so the other draws of the workload are unchanged."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 2])))
    H, dh, dv, dc, dr = w.heads, w.d_h, w.d_v, w.d_c, w.d_r

    def normal(shape, fan_in):
        return _as_input(w, g.standard_normal(shape, dtype=np.float32) / np.float32(np.sqrt(fan_in)))

    out = {"W_down": normal((d_model, dc), d_model), "W_KR": normal((d_model, dr), d_model),
           "W_Q": normal((d_model, H * dh), d_model), "W_QR": normal((d_model, H * dr), d_model),
           "W_O": normal((H * dv, d_model), H * dv)}
    for b, L in enumerate(np.asarray(kv_lens)):
        gb = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 3, b])))
        out[f"x{b}"] = _as_input(w, gb.standard_normal((int(L), d_model), dtype=np.float32))
    return out
