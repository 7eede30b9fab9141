"""GPU invariance and adversarial checks (through the C ABI):

* split-count invariance: the same batch decoded with different numbers of token ranges
  (the test-only override MLA_FORCE_SPLITS) agrees within a bound derived from the rounding
  that a different cut changes, and every run passes the oracle gate; the range-size override
  MLA_SPLIT_TOKENS reproduces the equivalent range count bit for bit;
* query rows that see no token (kv_len < Sq) give the defined empty result, the others the
  oracle's;
* needle tokens in the longest sequence of the full-size long-context workloads, at the bench's
  launch configuration: at t = 0, at a range boundary and in the sequence's last page.
"""
import os

import numpy as np
import pytest

import oracle.mla_oracle as orc
from mla_latent_kv_40_amd import binding as B, harness, workloads as wl
from _common import STORAGE_SHARE, bound, cache_rows, check, dsv2, host, log, oracle_for, run_state
from test_gpu_parity import compare_seq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)


def decode_with_ranges(st, G, var="MLA_FORCE_SPLITS"):
    """mla_decode_attn on the state's inputs with the test-only override `var` = G (None: the
    default count), a fresh NaN-filled workspace and NaN-filled outputs."""
    old = {k: os.environ.pop(k, None) for k in ("MLA_FORCE_SPLITS", "MLA_SPLIT_TOKENS")}
    if G is not None:
        os.environ[var] = str(G)
    try:
        ws_bytes = B.mla_decode_workspace_size(st.cfg, st.w.batch, st.w.sq, st.batch.max_blocks)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        ws.view(torch.float32)[: ws_bytes // 4].fill_(float("nan"))
        st.o_lat.fill_(float("nan"))
        st.lse.fill_(float("nan"))
        B.mla_decode_attn(st.cfg, st.q_abs, st.cache, st.cache_scale, st.batch.num_blocks, st.block_table,
                          st.batch.max_blocks, st.kv_lens, st.w.batch, st.w.sq, ws, ws_bytes, st.o_lat, st.lse)
        torch.cuda.synchronize()
        return st.o_lat.cpu().numpy().copy(), st.lse.cpu().numpy().copy(), ws_bytes
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def weighted_spread(w, bt, seqs, b, heads):
    """Per (query, head, latent column): D = sum_t w_t |c_t - o| and A = sum_t w_t |c_t| over the
    oracle's softmax weights w_t (fp64, scores by the absorbed route), with c_t the latent rows
    the kernel reads (dequantised for an fp8 cache).  They scale the rounding bound below."""
    s = seqs[b]
    L = int(bt.kv_lens[b])
    t = np.arange(L)
    rows = cache_rows(w, bt, seqs, b)
    pos_q = L - w.sq + np.arange(w.sq)
    qa = orc.absorbed_query(s["q_c"], s["q_r"], bt.weights["W_UK"], pos_q, w.rope_base)[:, list(heads)]
    sc = np.einsum("jhk,tk->jht", qa, rows) * w.softmax_scale
    sc = np.where((t[None, :] <= pos_q[:, None])[:, None, :], sc, -np.inf)
    wt = np.exp(sc - sc.max(-1, keepdims=True))
    wt /= wt.sum(-1, keepdims=True)
    C = rows[:, :w.d_c]
    o = np.einsum("jht,tc->jhc", wt, C)
    D = np.einsum("jht,jhtc->jhc", wt, np.abs(C[None, None] - o[:, :, None, :]))
    A = np.einsum("jht,tc->jhc", wt, np.abs(C))
    return D, A, float(np.abs(C).max())


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8b"])
def test_split_count_invariance(fmt):
    """A different cut changes each segment's softmax reference and so the rounding of the
    probabilities fed to the value product (bf16: relative 2^-9, and l sums the same rounded
    values; fp8: hi + lo/16 e4m3 terms, relative 2^-8, l summed unrounded) and of the bf16
    segment partials (2^-9).  With u the probability rounding, per latent column of one query
    and head a run is within u' (D + A) of exact attention over the same inputs (u' = u/(1-u)
    plus the partial rounding), so two runs differ by at most 2 u' (D + A) (+1e-6 max|c| for the
    fp32 sums).  lse moves only with l: by at most 2 u'.  Ranges tried: the fewest the page table
    allows, an odd count that is not a multiple of the XCD count, the default, and one page per
    range."""
    log(f"case split-count invariance, cache {fmt}: lengths [20000, 9000, 3001, 777, 65]")
    lengths = [20000, 9000, 3001, 777, 65]
    w, bt, seqs = dsv2(5, lengths, seed=71, fmt=None if fmt == "bf16" else fmt)
    fp8 = w.fp8
    st = run_state(w, bt, seqs)
    cap = w.batch * bt.max_blocks
    runs = {}
    for G in (1, 37, None, cap):
        o_lat, lse, ws = decode_with_ranges(st, G)
        runs[G] = (o_lat, lse)
        log(f"  ranges {G if G is not None else 'default'}: workspace {ws} B")
        assert np.all(np.isfinite(o_lat)) and np.all(np.isfinite(lse)), G
    u = 2.0 ** -9
    up = (2.0 ** -8 + u) if fp8 else (u / (1 - u) + u)
    heads = list(range(0, 128, 7))
    for b in range(w.batch):
        D, A, cmax = weighted_spread(w, bt, seqs, b, heads)
        bound_o = 2 * up * (D + A) + 1e-6 * cmax
        bound_l = 2 * (2.0 ** -8 if fp8 else u / (1 - u)) + 1e-5
        ref = oracle_for(w, bt, seqs, b, heads=heads)
        for G, (o_lat, lse) in runs.items():
            g_o = o_lat[b:b + 1][:, heads]
            g_l = lse[b:b + 1][:, heads]
            d_o = np.abs(g_o - runs[None][0][b:b + 1][:, heads])
            d_l = np.abs(g_l - runs[None][1][b:b + 1][:, heads])
            ratio = max(float(np.max(d_o / bound_o)), float(np.max(d_l / bound_l)))
            log(f"  b{b} ranges {G}: max |diff| / bound {ratio:.3f} (o_lat {np.max(d_o):.2e}, lse {np.max(d_l):.2e})")
            assert np.all(d_o <= bound_o) and np.all(d_l <= bound_l), (b, G)
            f = 4.0 if fp8 else 1.0
            check(f"b{b} ranges {G} o_lat", g_o, ref["o_lat"], f)
            check(f"b{b} ranges {G} lse", g_l, ref["lse"], f)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_split_tokens_override_equals_range_count(fmt):
    """MLA_SPLIT_TOKENS = n gives G = ceil(64 * B * max_blocks / n) ranges: the same cut as
    MLA_FORCE_SPLITS = G, so the two runs agree bit for bit."""
    lengths = [20000, 9000, 3001, 777, 65]
    log(f"case split-tokens override, cache {fmt}: lengths {lengths}")
    w, bt, seqs = dsv2(5, lengths, seed=72, fmt=None if fmt == "bf16" else fmt)
    st = run_state(w, bt, seqs)
    cap_tokens = 64 * w.batch * bt.max_blocks
    for n in (cap_tokens // 37, 4096, 64 * 3):
        G = -(-cap_tokens // n)
        o_t, l_t, ws_t = decode_with_ranges(st, n, var="MLA_SPLIT_TOKENS")
        o_g, l_g, ws_g = decode_with_ranges(st, G)
        log(f"  {n} tokens per range -> {G} ranges: workspace {ws_t} B")
        assert ws_t == ws_g
        assert np.array_equal(o_t, o_g) and np.array_equal(l_t, l_g), (n, G)


@pytest.mark.parametrize("fmt,pages", [("bf16", 1021), ("fp8", 510)])
def test_page_table_at_capacity(fmt, pages):
    """One range holding as many pages as the split kernel's LDS page table takes: a single
    sequence of `pages` full pages with the range count forced to 1.  The planner keeps one range
    while B (max_blocks + w) fits the table (1,024 entries with w = 3 for bf16, 512 with w = 2
    for fp8), i.e. up to 1,021 and 510 pages; the workspace size (one partial slot) shows that
    it did.  Needles (latent x4) at t = 0, in the middle and on the last token make a lost or
    misplaced page visible."""
    L = 64 * pages
    log(f"case page table at capacity, cache {fmt}: one sequence of {pages} pages ({L} tokens), one range")
    w, bt, seqs = dsv2(1, [L], seed=79, fmt=None if fmt == "bf16" else fmt)
    seqs[0]["c"] = seqs[0]["c"].copy()
    for t in (0, L // 2, L - 1):
        seqs[0]["c"][t] = seqs[0]["c"][t] * 4.0
    old = os.environ.get("MLA_FORCE_SPLITS")
    os.environ["MLA_FORCE_SPLITS"] = "1"
    try:
        st = run_state(w, bt, seqs)
        got = host(st)
    finally:
        if old is None:
            os.environ.pop("MLA_FORCE_SPLITS", None)
        else:
            os.environ["MLA_FORCE_SPLITS"] = old
    one_slot = 128 * 512 * 2 + 128 * 2 * 4          # bf16 partial O and (m, l) of one slot
    assert st.ws_bytes == one_slot, st.ws_bytes     # a single range (both parts 256-byte aligned)
    compare_seq(w, bt, seqs, got, 0, heads=range(0, 128, 16), factor=4.0 if w.fp8 else 1.0, tag="capacity ")


@pytest.mark.parametrize("fmt", ["bf16", "fp8b", "bf16-generic"])
def test_query_rows_without_tokens(fmt):
    """kv_len < Sq: query j sits at p = kv_len - Sq + j; rows with p < 0 see no token and give
    o_lat = 0, lse = -inf (and a zero layer output); rows with p >= 0 attend to tokens 0 .. p,
    i.e. equal a one-query decode of length p + 1 (the causal multi-query reduction); also in a
    non-DeepSeek-V2 head shape (the generic kernels).  With the
    tile-scaled cache the rows are also checked against the oracle on the rows the cache holds
    (1x), and the exact oracle at 4x where the storage alone leaves the kernel its 1x share."""
    log(f"case kv_len < Sq: lengths [2, 3, 1, 9], Sq=4, cache {fmt}")
    shape = dict(heads=16, d_h=64, d_r=32, d_c=128, d_v=64) if fmt == "bf16-generic" else None
    w, bt, seqs = dsv2(4, [2, 3, 1, 9], sq=4, seed=73, fmt="fp8b" if fmt == "fp8b" else None, shape=shape)
    st = run_state(w, bt, seqs)
    got = host(st)
    for b in range(w.batch):
        L = int(bt.kv_lens[b])
        s = seqs[b]
        deq = cache_rows(w, bt, seqs, b) if w.fp8 else None
        for j in range(w.sq):
            row = b * w.sq + j
            p = L - w.sq + j
            if p < 0:
                assert np.all(got["o_lat"][row] == 0.0) and np.all(np.isneginf(got["lse"][row])), (b, j)
                assert np.all(got["o"][row] == 0.0), (b, j)
                continue
            ref = orc.decode(s["c"], s["k_r"], s["q_c"][j:j + 1], s["q_r"][j:j + 1], bt.weights["W_UK"],
                             bt.weights["W_UV"], p + 1, w.softmax_scale, w.rope_base)
            if deq is None:
                for k in ("o", "o_lat", "lse"):
                    check(f"b{b} j{j} {k}", got[k][row:row + 1], ref[k])
                continue
            rd = orc.decode(deq[:p + 1, :w.d_c], deq[:p + 1, w.d_c:], s["q_c"][j:j + 1], s["q_r"][j:j + 1],
                            bt.weights["W_UK"], bt.weights["W_UV"], p + 1, w.softmax_scale, w.rope_base,
                            keys_rotated=True)
            for k in ("o", "o_lat", "lse"):
                check(f"b{b} j{j} {k} vs dequantised cache", got[k][row:row + 1], rd[k])
                if np.max(np.abs(rd[k] - ref[k])) <= STORAGE_SHARE * bound(ref[k], 4.0):
                    check(f"b{b} j{j} {k}", got[k][row:row + 1], ref[k], 4.0)


def range_boundary_page(bt, b, G, w_seg=3):
    """A page of sequence b at which the default cut (G ranges, per-segment cost w_seg pages)
    starts a new range, or None: page x of the r-th non-empty sequence sits at cost position
    first_page + x + w_seg (r + 1), and range g starts at floor(g C / G)."""
    n = (bt.kv_lens.astype(np.int64) + 63) // 64
    nz = n > 0
    C = int(n.sum() + w_seg * nz.sum())
    first = int(n[:b].sum())
    r = int(nz[:b].sum())
    lo = first + w_seg * (r + 1)
    for g in range(1, G):
        c = g * C // G
        if lo < c < lo + int(n[b]):
            return c - lo
    return None


@pytest.mark.parametrize("name", ["dsv2_b64_l1k_32k", "dsv2_b64_l32k"])
def test_full_size_needles(name):
    """The full-size long-context workloads at the bench's launch configuration, with three
    needles (latent x4, exact in bf16) in the longest sequence: at t = 0, on the first token of a
    page where a range starts, and on the sequence's last token.  A dropped, duplicated or
    misplaced page holding one moves the output of the heads it dominates far past the gate."""
    w = wl.get(name)
    bt = wl.draw_batch(w)
    b = int(np.argmax(bt.kv_lens))
    L = int(bt.kv_lens[b])
    G = torch.cuda.get_device_properties(0).multi_processor_count
    x = range_boundary_page(bt, b, G)
    assert x is not None
    spots = [0, 64 * x, L - 1]
    log(f"case full-size needles {name}: sequence {b} (kv_len {L}), needles at {spots}")
    seqs = harness.draw_all_sequences(w, bt)
    heads = list(range(0, 128, 4))
    plain = oracle_for(w, bt, seqs, b, heads=heads)
    seqs[b]["c"] = seqs[b]["c"].copy()
    for t in spots:
        seqs[b]["c"][t] = seqs[b]["c"][t] * 4.0
    st = run_state(w, bt, seqs)
    got = host(st)
    assert np.all(np.isfinite(got["o"]))
    ref = oracle_for(w, bt, seqs, b, heads=heads)
    # the needles move the output by far more than the gate allows, so losing one would fail
    moved = float(np.max(np.abs(ref["o_lat"] - plain["o_lat"])))
    tol = 2e-2 * float(np.max(np.abs(ref["o_lat"]))) + 1e-3
    log(f"  needles move o_lat by {moved:.3e} (gate {tol:.3e})")
    assert moved > 10 * tol
    for k in ("o", "o_lat", "lse"):
        check(f"needles b{b} {k}", got[k][b:b + 1][:, heads], ref[k])


@pytest.mark.parametrize("lengths,sq,fmt", [([1064, 364], 64, "bf16"), ([256], 256, "bf16"), ([700, 333], 333, "bf16"),
                                            ([1064, 364], 64, "fp8b"), ([256], 256, "fp8")])
def test_chunked_extend_and_prefill(lengths, sq, fmt):
    """Many query rows per sequence: a chunk of Sq new tokens (positions kv_len - Sq ..) appended
    and attended causally in one step, up to a whole prompt (kv_len = Sq: prefill).  The range
    count falls to CUs / Sq, so each query row's workgroup streams its sequence's pages.  The fp8
    cases append the chunk in the step (for tile scales, runs of up to 32 tokens per tile) and
    take the fp8 gate (the oracle on the rows the cache holds at 1x as well)."""
    log(f"case chunked extend / prefill: lengths {lengths}, Sq={sq}, cache {fmt}")
    w, bt, seqs = dsv2(len(lengths), lengths, sq=sq, seed=97, fmt=None if fmt == "bf16" else fmt)
    st = run_state(w, bt, seqs)
    got = host(st)
    assert np.all(np.isfinite(got["o"]))
    heads = list(range(3, 128, 25))
    for b in range(w.batch):
        if w.fp8:
            compare_seq(w, bt, seqs, got, b, heads=heads, factor=4.0, tag=f"Sq={sq} ")
            continue
        ref = oracle_for(w, bt, seqs, b, heads=heads)
        rows = slice(b * sq, (b + 1) * sq)
        for k in ("o", "o_lat", "lse"):
            check(f"b{b} Sq={sq} {k}", got[k][rows][:, heads], ref[k])
