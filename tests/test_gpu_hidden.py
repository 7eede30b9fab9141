"""GPU parity of the projections on either side of the latent-space decode, through the C ABI:

* mla_append_absorb_hidden: the layer runs from hidden states (the context is written through it,
  then one decode step), against oracle.project_from_hidden followed by oracle.decode;
* mla_fold_output_weights + mla_out_proj_folded: the output in the model width with W_UV folded
  into W_O, against the oracle's unfolded o W_O.

Cases: the tiny fp32 workload (d_model 512) and DeepSeek-V2 shapes with d_model 5120, the
model width of DeepSeek-V2 (the pages give none for these workloads), bf16 and fp8 caches, and
d_model 1040 with a bf16 cache (the generic row products).
"""
import numpy as np
import pytest

import oracle.mla_oracle as orc
from mla_latent_kv_40_amd import binding as B, harness, workloads as wl
from _common import check, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)


class HiddenRun:
    """Device state of a batch that starts at hidden states: each sequence's context is written by
    mla_append_absorb_hidden (T = 0), then one step writes the Sq new tokens and folds the queries."""

    def __init__(self, w, kv_lens, d_model, W, xs, chunk=200):
        self.w, self.d_model = w, d_model
        self.cfg = harness.config_for(w)
        act = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
        self.act = act
        dev = lambda a, dt=act: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
        kv = np.asarray(kv_lens, dtype=np.int64)
        Bn, Sq, H = len(kv), w.sq, w.heads
        self.B, self.T = Bn, Bn * Sq
        nblk = (kv + 63) // 64
        self.num_blocks = int(nblk.sum())
        perm = np.random.default_rng(w.seed + 99).permutation(self.num_blocks).astype(np.int32)
        self.max_blocks = int(nblk.max())
        table = np.full((Bn, self.max_blocks), -1, np.int32)
        off = 0
        for b in range(Bn):
            table[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += int(nblk[b])
        self.block_table = dev(table, torch.int32)
        self.kv_lens = dev(kv.astype(np.int32), torch.int32)
        if w.fp8:
            self.cache = torch.empty((self.num_blocks, 64, w.row), dtype=torch.uint8, device="cuda")
            shape = (self.num_blocks, 64) if w.dtype == "fp8" else (self.num_blocks, 2, w.row // 32)
            self.cache_scale = torch.empty(shape, dtype=torch.float32, device="cuda")
        else:
            self.cache = torch.empty((self.num_blocks, 64, w.row), dtype=act, device="cuda")
            self.cache_scale = None
        # transposed projection weights: row j holds the weights of output j
        self.w_dkv_t = dev(np.concatenate([W["W_down"], W["W_KR"]], axis=1).T)
        self.w_q_t = dev(np.concatenate([W["W_Q"], W["W_QR"]], axis=1).T)
        self.w_uk, self.w_uv, self.w_o = dev(W["W_UK"]), dev(W["W_UV"]), dev(W["W_O"])
        self.q_abs = torch.empty((self.T, H, w.row), dtype=act, device="cuda")
        self.o_lat = torch.empty((self.T, H, w.d_c), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((self.T, H), dtype=torch.float32, device="cuda")
        self.out = torch.empty((self.T, H, w.d_v), dtype=act, device="cuda")
        # context: positions 0 .. kv_len - Sq - 1 of each sequence, in chunks
        hs, ps, ss = [], [], []
        for b in range(Bn):
            L = int(kv[b])
            hs.append(xs[b][:L - Sq]); ps.append(np.arange(L - Sq)); ss.append(np.full(L - Sq, b))
        h_ctx, p_ctx, s_ctx = np.concatenate(hs), np.concatenate(ps), np.concatenate(ss)
        for t0 in range(0, len(p_ctx), chunk):
            t1 = min(len(p_ctx), t0 + chunk)
            self.call(dev(h_ctx[t0:t1]), dev(p_ctx[t0:t1], torch.int32), dev(s_ctx[t0:t1], torch.int32), t1 - t0,
                      None, None, 0)
        # the step: new tokens at kv_len - Sq .. kv_len - 1, query rows at the same positions
        self.h_new = dev(np.concatenate([xs[b][int(kv[b]) - Sq:int(kv[b])] for b in range(Bn)]))
        self.p_new = dev(np.concatenate([np.arange(int(kv[b]) - Sq, int(kv[b])) for b in range(Bn)]), torch.int32)
        self.s_new = dev(np.repeat(np.arange(Bn), Sq), torch.int32)
        self.call(self.h_new, self.p_new, self.s_new, self.T, self.h_new, self.p_new, self.T)
        ws = B.mla_decode_workspace_size(self.cfg, Bn, Sq, self.max_blocks)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        B.mla_decode_attn(self.cfg, self.q_abs, self.cache, self.cache_scale, self.num_blocks, self.block_table,
                          self.max_blocks, self.kv_lens, Bn, Sq, self.ws, ws, self.o_lat, self.lse)
        B.mla_out_proj(self.cfg, self.o_lat, self.w_uv, self.out, self.T)
        torch.cuda.synchronize()

    def call(self, h_kv, pos, seq, n, h_q, q_pos, T):
        ws = B.mla_hidden_workspace_size(self.cfg, self.d_model, n, T)
        assert ws > 0
        buf = torch.empty(ws, dtype=torch.uint8, device="cuda")
        B.mla_append_absorb_hidden(self.cfg, self.d_model, h_kv, self.w_dkv_t, self.cache, self.cache_scale,
                                   self.num_blocks, pos, seq, self.block_table, self.B, self.max_blocks, n, h_q,
                                   self.w_q_t, q_pos, self.w_uk, self.q_abs, T, buf, ws)

    def folded_output(self):
        """W_O' on the device, then out [T, d_model] = o_lat . W_O'."""
        H, dc = self.w.heads, self.w.d_c
        self.w_fold_t = torch.empty((self.d_model, H * dc), dtype=self.act, device="cuda")
        B.mla_fold_output_weights(self.cfg, self.d_model, self.w_uv, self.w_o, self.w_fold_t)
        out = torch.empty((self.T, self.d_model), dtype=self.act, device="cuda")
        ws = B.mla_out_proj_folded_workspace_size(self.cfg, self.d_model, self.T)
        buf = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")
        B.mla_out_proj_folded(self.cfg, self.d_model, self.o_lat, self.w_fold_t, out, self.T, buf, ws)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()


def oracle_from_hidden(w, W, x, L, heads=None):
    C, KR, qC, qR = orc.project_from_hidden(x[:L], W["W_down"], W["W_KR"], W["W_Q"], W["W_QR"], w.heads, w.d_h,
                                            w.d_r, list(range(L - w.sq, L)))
    ref = orc.decode(C, KR, qC, qR, W["W_UK"], W["W_UV"], L, w.softmax_scale, w.rope_base, heads=heads)
    ref["q_abs"] = orc.absorbed_query(qC, qR, W["W_UK"], list(range(L - w.sq, L)), w.rope_base)
    return ref


def test_tiny_f32_layer_from_hidden_states():
    log("case tiny_f32 from hidden states through mla_append_absorb_hidden, folded output projection")
    w = wl.get("tiny_f32")
    bt = wl.draw_batch(w)
    W = bt.weights
    L = int(bt.kv_lens[0])
    run = HiddenRun(w, [L], w.d_model, W, [W["x"]], chunk=4)
    ref = oracle_from_hidden(w, W, W["x"], L)
    got = {"o": run.out.cpu().numpy(), "o_lat": run.o_lat.cpu().numpy(), "lse": run.lse.cpu().numpy(),
           "q_abs": run.q_abs.cpu().numpy()}
    for k in ("o", "o_lat", "lse", "q_abs"):   # fp32 throughout: ~1e-6 relative expected
        check(f"tiny hidden {k}", got[k], ref[k], extra_rel=1e-4)
    out = run.folded_output()
    check("tiny folded model output", out, orc.model_output(ref["o"], W["W_O"]), extra_rel=1e-4)
    Wf = orc.fold_output_weights(W["W_UV"], W["W_O"], w.heads)              # [H, d_c, d_model]
    got_f = run.w_fold_t.cpu().numpy().reshape(w.d_model, w.heads, w.d_c).transpose(1, 2, 0)
    check("tiny folded weights", got_f, Wf, extra_rel=1e-4)


@pytest.mark.parametrize("fmt,d_model", [("bf16", 5120), ("fp8", 5120), ("fp8b", 5120), ("bf16", 1040)])
def test_dsv2_layer_from_hidden_states(fmt, d_model):
    """d_model 5120 takes the matrix-core projections; 1040 (a multiple of 16, not of 64) the
    generic row products for both projections and the folded output."""
    lengths = [300, 65, 1, 130]
    name = {"bf16": "dsv2_b16_l4k", "fp8": "dsv2_b128_l8k_fp8", "fp8b": "dsv2_b128_l8k_fp8b"}[fmt]
    w = wl.get(name, batch=len(lengths), seed=91)
    fp8 = w.fp8
    log(f"case DeepSeek-V2 shapes from hidden states, d_model {d_model}, cache {fmt}, lengths {lengths}")
    bt = wl.draw_batch(w)
    Hd = wl.draw_hidden(w, d_model, lengths)
    W = dict(Hd, W_UK=bt.weights["W_UK"], W_UV=bt.weights["W_UV"])
    xs = [Hd[f"x{b}"] for b in range(len(lengths))]
    run = HiddenRun(w, lengths, d_model, W, xs)
    f = 4.0 if fp8 else 1.0
    heads = list(range(0, 128, 5))
    o = run.out.float().cpu().numpy()
    o_lat = run.o_lat.cpu().numpy()
    lse = run.lse.cpu().numpy()
    q_abs = run.q_abs.float().cpu().numpy()
    out = run.folded_output()
    for b, L in enumerate(lengths):
        ref = oracle_from_hidden(w, W, xs[b], L, heads=heads)
        check(f"b{b} q_abs", q_abs[b:b + 1][:, heads], ref["q_abs"][:, heads])
        check(f"b{b} o", o[b:b + 1][:, heads], ref["o"], f)
        check(f"b{b} o_lat", o_lat[b:b + 1][:, heads], ref["o_lat"], f)
        check(f"b{b} lse", lse[b:b + 1][:, heads], ref["lse"], f)
        full = oracle_from_hidden(w, W, xs[b], L)
        check(f"b{b} folded model output", out[b:b + 1], orc.model_output(full["o"], W["W_O"]), f)
    # the folded weights of a few heads against the oracle's fold (one bf16 rounding)
    got_f = run.w_fold_t.float().cpu().numpy().reshape(d_model, w.heads, w.d_c)
    for i in (0, 77, 127):
        ref_i = orc.fold_output_weights(W["W_UV"][:, i * w.d_v:(i + 1) * w.d_v], W["W_O"][i * w.d_v:(i + 1) * w.d_v], 1)[0]
        err = np.abs(got_f[:, i, :].T - ref_i)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref_i) + 1e-6), i
