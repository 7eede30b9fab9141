"""Device-side driver for one MLA decode step through libmla (used by the tests and bench.py).

Torch provides device memory and the stream; every computation is a libmla call:

    setup (untimed)  mla_cache_append of each sequence's context tokens
    step             mla_append_absorb (the Sq new tokens per sequence into the cache, and the
                     folded queries; or mla_cache_append then mla_absorb_q)
                     -> mla_decode_attn -> mla_out_proj

Inputs come from ``workloads`` (seeded draws, no method arithmetic).  The tiny fp32 case
starts from hidden states; its caller passes the per-sequence latent and query tensors.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import binding as B
from . import workloads as wl


def config_for(w: wl.Workload) -> B.Config:
    return B.Config(num_heads=w.heads, d_c=w.d_c, d_r=w.d_r, d_h=w.d_h, d_v=w.d_v,
                    softmax_scale=w.softmax_scale, rope_base=w.rope_base,
                    cache_dtype=w.dtype, act_dtype=w.act_dtype)


class DecodeState:
    """All device buffers of one workload: paged cache, tables, weights, step inputs/outputs."""

    def __init__(self, w: wl.Workload, batch: wl.Batch, seqs: List[Dict[str, np.ndarray]],
                 device: str = "cuda", weights: Optional[Dict[str, np.ndarray]] = None):
        import torch
        self.torch = torch
        self.w, self.batch, self.device = w, batch, device
        self.cfg = config_for(w)
        act = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
        self.act = act
        Bn, Sq, H = w.batch, w.sq, w.heads
        self.T = Bn * Sq
        kv = batch.kv_lens.astype(np.int64)
        W = weights if weights is not None else batch.weights

        def dev(x, dt=act):
            return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)

        # paged cache
        nb = batch.num_blocks
        if w.fp8:
            self.cache = torch.empty((nb, wl.BLOCK, w.row), dtype=torch.uint8, device=device)
            shape = (nb, wl.BLOCK) if w.dtype == "fp8" else (nb, wl.BLOCK // 32, w.row // 32)
            self.cache_scale = torch.empty(shape, dtype=torch.float32, device=device)
        else:
            self.cache = torch.empty((nb, wl.BLOCK, w.row), dtype=act, device=device)
            self.cache_scale = None
        self.block_table = dev(batch.block_table, torch.int32)
        self.kv_lens = dev(batch.kv_lens, torch.int32)
        self.w_uk = dev(W["W_UK"])
        self.w_uv = dev(W["W_UV"])

        # context tokens (positions 0 .. kv_len - Sq - 1) and the step's new tokens
        ctx_c, ctx_k, ctx_pos, ctx_seq = [], [], [], []
        new_c, new_k, new_pos, new_seq = [], [], [], []
        qn, qr = [], []
        for b in range(Bn):
            L = int(kv[b])
            s = seqs[b]
            n_ctx = max(L - Sq, 0)
            ctx_c.append(s["c"][:n_ctx]); ctx_k.append(s["k_r"][:n_ctx])
            ctx_pos.append(np.arange(n_ctx, dtype=np.int32)); ctx_seq.append(np.full(n_ctx, b, np.int32))
            # the step's new tokens sit at positions L - Sq .. L - 1; with L < Sq the first ones
            # have negative positions: no such token exists, the append skips them (zero rows here)
            idx = np.arange(L - Sq, L)
            ok = (idx >= 0)[:, None]
            new_c.append(np.where(ok, s["c"][np.maximum(idx, 0)], 0).astype(s["c"].dtype))
            new_k.append(np.where(ok, s["k_r"][np.maximum(idx, 0)], 0).astype(s["k_r"].dtype))
            new_pos.append(idx.astype(np.int32)); new_seq.append(np.full(Sq, b, np.int32))
            qn.append(s["q_c"]); qr.append(s["q_r"])
        self._ctx = (np.concatenate(ctx_c), np.concatenate(ctx_k), np.concatenate(ctx_pos), np.concatenate(ctx_seq))
        self.new_c = dev(np.concatenate(new_c))
        self.new_k = dev(np.concatenate(new_k))
        self.new_pos = dev(np.concatenate(new_pos), torch.int32)     # = query positions
        self.new_seq = dev(np.concatenate(new_seq), torch.int32)
        self.q_nope = dev(np.concatenate(qn).reshape(self.T, H, w.d_h))
        self.q_rope = dev(np.concatenate(qr).reshape(self.T, H, w.d_r))

        # outputs and scratch
        self.q_abs = torch.empty((self.T, H, w.row), dtype=act, device=device)
        self.o_lat = torch.empty((self.T, H, w.d_c), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.T, H), dtype=torch.float32, device=device)
        self.out = torch.empty((self.T, H, w.d_v), dtype=act, device=device)
        self.ws_bytes = B.mla_decode_workspace_size(self.cfg, Bn, Sq, batch.max_blocks)
        if self.ws_bytes == 0:
            raise RuntimeError("mla_decode_workspace_size rejected the configuration")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    # ------------------------------------------------------------------ setup
    def fill_context(self, chunk_tokens: int = 1 << 18) -> None:
        """Append every sequence's context tokens (untimed setup), in chunks."""
        torch = self.torch
        c, k, pos, seq = self._ctx
        for t0 in range(0, len(pos), chunk_tokens):
            t1 = min(len(pos), t0 + chunk_tokens)
            cd = torch.from_numpy(np.ascontiguousarray(c[t0:t1])).to(self.device, self.act)
            kd = torch.from_numpy(np.ascontiguousarray(k[t0:t1])).to(self.device, self.act)
            pd = torch.from_numpy(pos[t0:t1]).to(self.device)
            sd = torch.from_numpy(seq[t0:t1]).to(self.device)
            self.append(cd, kd, pd, sd, t1 - t0)
        torch.cuda.synchronize()
        self._ctx = None

    # ------------------------------------------------------------------ calls
    def append(self, c, k, pos, seq, n, stream=None) -> None:
        B.mla_cache_append(self.cfg, self.cache, self.cache_scale, self.batch.num_blocks, c, k, pos, seq,
                           self.block_table, self.w.batch, self.batch.max_blocks, n, stream)

    def absorb(self, stream=None) -> None:
        B.mla_absorb_q(self.cfg, self.q_nope, self.q_rope, self.new_pos, self.w_uk, self.q_abs, self.T, stream)

    def append_absorb(self, stream=None) -> None:
        """The step's new tokens into the cache and the folded queries, in one call."""
        B.mla_append_absorb(self.cfg, self.cache, self.cache_scale, self.batch.num_blocks, self.new_c, self.new_k,
                            self.new_pos, self.new_seq, self.block_table, self.w.batch, self.batch.max_blocks, self.T,
                            self.q_nope, self.q_rope, self.new_pos, self.w_uk, self.q_abs, self.T, stream)

    def decode(self, stream=None) -> None:
        B.mla_decode_attn(self.cfg, self.q_abs, self.cache, self.cache_scale, self.batch.num_blocks,
                          self.block_table, self.batch.max_blocks, self.kv_lens, self.w.batch, self.w.sq,
                          self.workspace, self.ws_bytes, self.o_lat, self.lse, stream)

    def _dargs(self):
        return (self.cfg, self.q_abs, self.cache, self.cache_scale, self.batch.num_blocks,
                self.block_table, self.batch.max_blocks, self.kv_lens, self.w.batch, self.w.sq, self.workspace,
                self.ws_bytes, self.o_lat, self.lse)

    def decode_split(self, stream=None) -> None:
        B.mla_decode_split(*self._dargs(), stream)

    def decode_combine(self, stream=None) -> None:
        B.mla_decode_combine(*self._dargs(), stream)

    def out_proj(self, stream=None) -> None:
        B.mla_out_proj(self.cfg, self.o_lat, self.w_uv, self.out, self.T, stream)

    def step(self, stream=None, fused: bool = True) -> None:
        """One decode step: append the new tokens, fold the query, attend, project out.
        fused=False makes the append and the absorption two calls."""
        if fused:
            self.append_absorb(stream)
        else:
            self.append(self.new_c, self.new_k, self.new_pos, self.new_seq, self.T, stream)
            self.absorb(stream)
        self.decode(stream)
        self.out_proj(stream)


def draw_all_sequences(w: wl.Workload, batch: wl.Batch) -> List[Dict[str, np.ndarray]]:
    return [wl.draw_sequence(w, b, int(batch.kv_lens[b])) for b in range(w.batch)]
