"""C-ABI checks that need no GPU: the library loads, exports every entry point declared in
include/mla.h, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from mla_latent_kv_40_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_0-9]+\s*\*?\s*(mla_[a-z_0-9]+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmla.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert set(syms) == set(B.EXPORTS), syms
    for s in syms:
        assert hasattr(L, s), s
    assert B.mla_abi_version() == B.ABI_VERSION


def cfg(**kw):
    base = dict(num_heads=128, d_c=512, d_r=64, d_h=128, d_v=128, softmax_scale=192 ** -0.5,
                cache_dtype="bf16", act_dtype="bf16")
    base.update(kw)
    return B.Config(**base)


FAKE = 1 << 20   # aligned non-null address: never dereferenced because validation fails first


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=32), B.MLA_ERR_INVALID_ARG),
    (dict(d_c=500), B.MLA_ERR_INVALID_ARG),
    (dict(num_heads=0), B.MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), B.MLA_ERR_INVALID_ARG),
    (dict(cache_dtype="fp8", act_dtype="f32"), B.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype="bf16", act_dtype="f32"), B.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype="fp8", num_heads=64), B.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype="fp8b", act_dtype="f32"), B.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype="fp8b", num_heads=64), B.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype="f32", act_dtype="f32", num_heads=256, d_c=64, d_r=16, d_h=64, d_v=64),
     B.MLA_ERR_UNSUPPORTED),
])
def test_config_validation(L, kw, code):
    c = cfg(**kw)
    assert B.mla_out_proj(c, FAKE, FAKE, FAKE, 4, stream=0, check=False) == code
    assert B.mla_decode_workspace_size(c, 4, 1, 8) == 0


def test_pointer_and_size_validation(L):
    c = cfg()
    # null / misaligned pointers
    assert B.mla_absorb_q(c, 0, FAKE, FAKE, FAKE, FAKE, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_absorb_q(c, FAKE + 8, FAKE, FAKE, FAKE, FAKE, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_out_proj(c, FAKE, FAKE, FAKE, -1, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    # zero-size work is a no-op that touches nothing
    assert B.mla_out_proj(c, 0, 0, 0, 0, stream=0, check=False) == B.MLA_OK
    assert B.mla_absorb_q(c, 0, 0, 0, 0, 0, 0, stream=0, check=False) == B.MLA_OK
    # the scale pointer must be given exactly for fp8 caches
    c8 = cfg(cache_dtype="fp8")
    dec = [100, FAKE, 512, FAKE, 64, 1, FAKE, 1 << 30, FAKE, FAKE]
    assert B.mla_decode_attn(c8, FAKE, FAKE, None, *dec, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    c8b = cfg(cache_dtype="fp8b")
    assert B.mla_decode_attn(c8b, FAKE, FAKE, None, *dec, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_cache_append(c8b, FAKE, None, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 3, stream=0,
                              check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_cache_append(c8b, FAKE, FAKE + 4, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 3, stream=0,
                              check=False) == B.MLA_ERR_INVALID_ARG          # misaligned scales
    assert B.mla_decode_attn(c, FAKE, FAKE, FAKE, *dec, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_cache_append(c, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 3, stream=0,
                              check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_cache_append(c, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 3, stream=0,
                              check=False) == B.MLA_ERR_INVALID_ARG


def test_append_absorb_validation(L):
    c = cfg()
    app = [FAKE, None, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4]      # cache .. max_blocks (bf16: no scale)
    absq = [FAKE, FAKE, FAKE, FAKE, FAKE]                          # q_nope, q_rope, q_pos, w_uk, q_abs
    # either half's validation fails the whole call before anything is launched
    assert B.mla_append_absorb(c, *app, 3, 0, FAKE, FAKE, FAKE, FAKE, 4, stream=0,
                               check=False) == B.MLA_ERR_INVALID_ARG          # null q_nope
    assert B.mla_append_absorb(c, *app, 3, FAKE + 8, FAKE, FAKE, FAKE, FAKE, 4, stream=0,
                               check=False) == B.MLA_ERR_INVALID_ARG          # misaligned q_nope
    assert B.mla_append_absorb(c, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 3, *absq, 4, stream=0,
                               check=False) == B.MLA_ERR_INVALID_ARG          # scale for a bf16 cache
    assert B.mla_append_absorb(c, *app, -1, *absq, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_append_absorb(c, *app, 3, *absq, -1, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    c8 = cfg(cache_dtype="fp8")
    assert B.mla_append_absorb(c8, *app, 3, *absq, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    # nothing to do on either side is a no-op that touches nothing
    assert B.mla_append_absorb(c, *app, 0, 0, 0, 0, 0, 0, 0, stream=0, check=False) == B.MLA_OK


def test_decode_workspace_checks(L):
    c = cfg()
    ws = B.mla_decode_workspace_size(c, 64, 1, 512)
    assert ws > 0 and ws % 256 == 0
    # more queries per sequence or more sequences never need less scratch
    assert B.mla_decode_workspace_size(c, 64, 4, 512) >= ws
    assert B.mla_decode_workspace_size(c, 128, 1, 512) >= ws
    args = [c, FAKE, FAKE, None, 100, FAKE, 512, FAKE, 64, 1]
    assert B.mla_decode_attn(*args, 0, ws, FAKE, FAKE, stream=0, check=False) == B.MLA_ERR_WORKSPACE
    assert B.mla_decode_attn(*args, FAKE, ws - 256, FAKE, FAKE, stream=0, check=False) == B.MLA_ERR_WORKSPACE
    assert B.mla_decode_attn(*args, FAKE + 16, ws, FAKE, FAKE, stream=0, check=False) == B.MLA_ERR_WORKSPACE
    bad = [c, FAKE, FAKE, None, 100, FAKE, 512, FAKE, 64, 0]
    assert B.mla_decode_attn(*bad, FAKE, ws, FAKE, FAKE, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_decode_attn(c, FAKE, FAKE, None, 100, FAKE, 512, FAKE, 0, 1, 0, 0, 0, 0, stream=0,
                             check=False) == B.MLA_OK


def test_every_pointer_is_checked_for_alignment(L):
    """Each array argument must be 16-byte aligned (the header's convention): a pointer 4 bytes
    off is rejected before anything is launched, argument by argument."""
    c, c8 = cfg(), cfg(cache_dtype="fp8")
    ws = B.mla_decode_workspace_size(c, 64, 1, 512)
    ws8 = B.mla_decode_workspace_size(c8, 64, 1, 512)
    # decode: q_abs, cache, cache_scale, block_table, kv_lens, o_lat, lse
    for conf, w, scale in ((c, ws, None), (c8, ws8, FAKE)):
        good = dict(q=FAKE, cache=FAKE, scale=scale, bt=FAKE, kv=FAKE, o=FAKE, lse=FAKE)
        def call(**kw):
            a = dict(good, **kw)
            return B.mla_decode_attn(conf, a["q"], a["cache"], a["scale"], 100, a["bt"], 512, a["kv"], 64, 1,
                                     FAKE, w, a["o"], a["lse"], stream=0, check=False)
        for k in good:
            if good[k] is None:
                continue
            assert call(**{k: good[k] + 4}) == B.MLA_ERR_INVALID_ARG, k
    # append: cache, cache_scale, c_kv, k_r, pos, seq_of, block_table
    names = ["cache", "scale", "c", "k", "pos", "seq", "bt"]
    for k in names:
        a = {n: FAKE for n in names}
        a[k] += 4
        assert B.mla_cache_append(c8, a["cache"], a["scale"], 8, a["c"], a["k"], a["pos"], a["seq"], a["bt"], 2, 4,
                                  3, stream=0, check=False) == B.MLA_ERR_INVALID_ARG, k
    # absorb: q_nope, q_rope, q_pos, w_uk, q_abs
    for i in range(5):
        a = [FAKE] * 5
        a[i] += 4
        assert B.mla_absorb_q(c, *a, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG, i
    # out_proj: o_lat, w_uv, out
    for i in range(3):
        a = [FAKE] * 3
        a[i] += 4
        assert B.mla_out_proj(c, *a, 4, stream=0, check=False) == B.MLA_ERR_INVALID_ARG, i


def test_forced_split_count_changes_only_the_workspace(L, monkeypatch):
    """MLA_FORCE_SPLITS (test-only) sets the number of token ranges; the workspace follows it,
    clamped to one range per page at most."""
    c = cfg()
    base = B.mla_decode_workspace_size(c, 4, 1, 100)
    monkeypatch.setenv("MLA_FORCE_SPLITS", "1")
    one = B.mla_decode_workspace_size(c, 4, 1, 100)
    monkeypatch.setenv("MLA_FORCE_SPLITS", "400")
    many = B.mla_decode_workspace_size(c, 4, 1, 100)
    monkeypatch.setenv("MLA_FORCE_SPLITS", "100000")
    capped = B.mla_decode_workspace_size(c, 4, 1, 100)
    monkeypatch.setenv("MLA_FORCE_SPLITS", "junk")
    ignored = B.mla_decode_workspace_size(c, 4, 1, 100)
    assert one < base < many == capped      # 4 sequences x 100 pages: at most 400 ranges
    assert ignored == base


def test_split_tokens_override_sets_the_range_size(L, monkeypatch):
    """MLA_SPLIT_TOKENS = n (test-only) asks for ranges of about n tokens of the block tables'
    capacity: G = ceil(64 * B * max_blocks / n), so the workspace equals the one for that many
    forced ranges.  MLA_FORCE_SPLITS wins when both are set."""
    c = cfg()
    monkeypatch.delenv("MLA_FORCE_SPLITS", raising=False)

    def size(force=None, tokens=None):
        for k, v in (("MLA_FORCE_SPLITS", force), ("MLA_SPLIT_TOKENS", tokens)):
            if v is None:
                monkeypatch.delenv(k, raising=False)
            else:
                monkeypatch.setenv(k, str(v))
        return B.mla_decode_workspace_size(c, 4, 1, 100)   # capacity 400 pages = 25,600 tokens

    base = size()
    for n, G in ((25_600, 1), (1 << 30, 1), (6_400, 4), (6_399, 5), (700, 37), (64, 400), (1, 400)):
        assert size(tokens=n) == size(force=G), (n, G)
    assert size(force=3, tokens=64) == size(force=3)
    assert size(tokens="junk") == size(tokens=0) == base


def test_status_strings(L):
    for code in range(5):
        assert B.mla_status_string(code).startswith("MLA_")
    assert "UNKNOWN" in B.mla_status_string(99)


def test_noalloc_decode_validation(L):
    """mla_decode_attn_noalloc validates like mla_decode_attn and rejects a launch whose partials
    exceed its fixed 64 MiB scratch, before touching the device."""
    c = cfg()
    assert B.mla_decode_workspace_size(c, 2048, 1, 4) > B.NOALLOC_SCRATCH_BYTES
    assert B.mla_decode_attn_noalloc(c, FAKE, FAKE, None, 100, FAKE, 4, FAKE, 2048, 1, FAKE, FAKE, stream=0,
                                     check=False) == B.MLA_ERR_WORKSPACE
    assert B.mla_decode_attn_noalloc(c, FAKE + 4, FAKE, None, 100, FAKE, 4, FAKE, 2, 1, FAKE, FAKE, stream=0,
                                     check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_decode_attn_noalloc(c, FAKE, FAKE, None, 100, FAKE, 4, FAKE, 0, 1, FAKE, FAKE, stream=0,
                                     check=False) == B.MLA_OK
    c8 = cfg(cache_dtype="fp8")
    assert B.mla_decode_attn_noalloc(c8, FAKE, FAKE, None, 100, FAKE, 4, FAKE, 2, 1, FAKE, FAKE, stream=0,
                                     check=False) == B.MLA_ERR_INVALID_ARG


def test_hidden_and_folded_calls_validate_first(L):
    c = cfg()
    ws = B.mla_hidden_workspace_size(c, 5120, 8, 8)
    assert ws > 0 and B.mla_hidden_workspace_size(c, 5121, 8, 8) == 0
    # either side may be empty (context written without queries, or queries only)
    assert 0 < B.mla_hidden_workspace_size(c, 5120, 200, 0) and 0 < B.mla_hidden_workspace_size(c, 5120, 0, 4)
    assert B.mla_hidden_workspace_size(c, 5120, 0, 0) > 0
    assert B.mla_out_proj_folded_workspace_size(c, 5120, 0) > 0
    app = [FAKE, None, 8, FAKE, FAKE, FAKE, 2, 4]          # cache .. max_blocks (bf16: no scale)
    good = dict(h_kv=FAKE, w_dkv_t=FAKE, h_q=FAKE, w_q_t=FAKE, q_pos=FAKE, w_uk=FAKE, q_abs=FAKE, ws=FAKE)

    def call(conf=c, d_model=5120, n=8, T=8, ws_bytes=ws, **kw):
        a = dict(good, **kw)
        return B.mla_append_absorb_hidden(conf, d_model, a["h_kv"], a["w_dkv_t"], *app, n, a["h_q"], a["w_q_t"],
                                          a["q_pos"], a["w_uk"], a["q_abs"], T, a["ws"], ws_bytes, stream=0,
                                          check=False)
    assert call(h_kv=0) == B.MLA_ERR_INVALID_ARG
    assert call(w_q_t=FAKE + 4) == B.MLA_ERR_INVALID_ARG
    assert call(d_model=100) == B.MLA_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 512) == B.MLA_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == B.MLA_ERR_WORKSPACE
    assert call(q_pos=0) == B.MLA_ERR_INVALID_ARG              # the absorption half's own check
    assert call(n=0, T=0) == B.MLA_OK
    # folded output projection
    assert B.mla_fold_output_weights(c, 5120, FAKE, 0, FAKE, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
    wso = B.mla_out_proj_folded_workspace_size(c, 5120, 64)
    assert wso > 0
    assert B.mla_out_proj_folded(c, 5120, FAKE, FAKE, FAKE, 64, FAKE, wso - 512, stream=0,
                                 check=False) == B.MLA_ERR_WORKSPACE
    assert B.mla_out_proj_folded(c, 5120, FAKE + 4, FAKE, FAKE, 64, FAKE, wso, stream=0,
                                 check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_out_proj_folded(c, 5120, 0, 0, 0, 0, 0, 0, stream=0, check=False) == B.MLA_OK


def test_kv_cache_decode_validation(L):
    c = B.Config(num_heads=128, d_c=512, d_r=64, d_h=128, d_v=128, softmax_scale=128 ** -0.5)
    assert B.mla_kv_decode_workspace_size(c, 8, 64, 512) > 0
    assert B.mla_kv_decode_workspace_size(c, 3, 64, 512) == 0          # 128 heads do not group by 3
    assert B.mla_kv_decode_workspace_size(c, 4, 64, 512) == 0          # groups of 32: unsupported
    ws = B.mla_kv_decode_workspace_size(c, 8, 4, 16)
    args = [c, 8, FAKE, FAKE, FAKE, 100, FAKE, 16, FAKE, 4]
    assert B.mla_kv_decode_attn(*args, FAKE, ws - 256, FAKE, FAKE, stream=0, check=False) == B.MLA_ERR_WORKSPACE
    assert B.mla_kv_decode_attn(c, 8, FAKE + 4, *args[3:], FAKE, ws, FAKE, FAKE, stream=0,
                                check=False) == B.MLA_ERR_INVALID_ARG
    assert B.mla_kv_decode_attn(c, 8, FAKE, FAKE, 0, *args[5:], FAKE, ws, FAKE, FAKE, stream=0,
                                check=False) == B.MLA_ERR_INVALID_ARG
    c8 = B.Config(num_heads=128, d_c=512, d_r=64, d_h=128, d_v=128, softmax_scale=0.1, cache_dtype="fp8")
    assert B.mla_kv_decode_attn(c8, 8, *args[2:], FAKE, ws, FAKE, FAKE, stream=0,
                                check=False) == B.MLA_ERR_UNSUPPORTED


def test_size_limits(L):
    """The documented size limits: at most 2^20 query rows, appended tokens and batch entries per
    call, 2^24 pages in the pool or a table row, and split plans of at most 2^23 workgroups.
    Sizes past them are refused before anything is launched, and the size queries stay exact
    (no wrap-around) up to them."""
    rows, pages = 1 << 20, 1 << 24
    for fmt in ("bf16", "fp8", "fp8b"):
        c = cfg(cache_dtype=fmt)
        sc = None if fmt == "bf16" else FAKE
        # at the limits the sizes are real (huge) byte counts, past them 0
        one = B.mla_decode_workspace_size(c, 1, rows, 1)
        assert one >= rows * 128 * 512 * 2
        assert B.mla_decode_workspace_size(c, 1, rows + 1, 1) == 0
        assert B.mla_decode_workspace_size(c, 2, rows // 2 + 1, 1) == 0
        wide = B.mla_decode_workspace_size(c, 128, 1, pages)
        assert wide >= 128 * pages // 1024 * 128 * 512 * 2         # one partial per range of <= 1024 pages
        assert B.mla_decode_workspace_size(c, 128, 1, pages + 1) == 0
        assert B.mla_decode_workspace_size(c, rows, 1, pages) == 0  # plan past 2^23 workgroups
        for b, sq, mb in [(2**31 - 1, 1, 1), (1, 2**31 - 1, 1), (2**31 - 1, 2**31 - 1, 2**31 - 1), (-1, 1, 1)]:
            assert B.mla_decode_workspace_size(c, b, sq, mb) == 0
        dec = lambda b, sq, nb, mb: B.mla_decode_attn(c, FAKE, FAKE, sc, nb, FAKE, mb, FAKE, b, sq, FAKE,
                                                      1 << 62, FAKE, FAKE, stream=0, check=False)
        assert dec(rows + 1, 1, 100, 8) == B.MLA_ERR_INVALID_ARG
        assert dec(1024, 1025, 100, 8) == B.MLA_ERR_INVALID_ARG
        assert dec(4, 1, pages + 1, 8) == B.MLA_ERR_INVALID_ARG
        assert dec(4, 1, 100, pages + 1) == B.MLA_ERR_INVALID_ARG
        assert dec(rows, 1, 100, pages) == B.MLA_ERR_UNSUPPORTED   # refused before any launch
        assert B.mla_decode_attn_noalloc(c, FAKE, FAKE, sc, 100, FAKE, pages, FAKE, rows, 1, FAKE, FAKE,
                                         stream=0, check=False) == B.MLA_ERR_UNSUPPORTED
        app = lambda nb, batch, mb, n: B.mla_cache_append(c, FAKE, sc, nb, FAKE, FAKE, FAKE, FAKE, FAKE, batch,
                                                          mb, n, stream=0, check=False)
        assert app(pages + 1, 2, 4, 3) == B.MLA_ERR_INVALID_ARG
        assert app(8, rows + 1, 4, 3) == B.MLA_ERR_INVALID_ARG
        assert app(8, 2, pages + 1, 3) == B.MLA_ERR_INVALID_ARG
        assert app(8, 2, 4, rows + 1) == B.MLA_ERR_INVALID_ARG
        assert B.mla_absorb_q(c, FAKE, FAKE, FAKE, FAKE, FAKE, rows + 1, stream=0,
                              check=False) == B.MLA_ERR_INVALID_ARG
        assert B.mla_out_proj(c, FAKE, FAKE, FAKE, rows + 1, stream=0, check=False) == B.MLA_ERR_INVALID_ARG
        assert B.mla_hidden_workspace_size(c, 5120, rows, rows) > 0
        assert B.mla_hidden_workspace_size(c, 5120, rows + 1, 1) == 0
        assert B.mla_hidden_workspace_size(c, 5120, 1, rows + 1) == 0
        assert B.mla_hidden_workspace_size(c, 1 << 20, rows, rows) > 0
        assert B.mla_out_proj_folded_workspace_size(c, 1 << 20, rows) > 0
        assert B.mla_out_proj_folded_workspace_size(c, 5120, rows + 1) == 0
        assert B.mla_out_proj_folded(c, 5120, FAKE, FAKE, FAKE, rows + 1, FAKE, 1 << 62, stream=0,
                                     check=False) == B.MLA_ERR_INVALID_ARG
    kv = B.Config(num_heads=128, d_c=512, d_r=64, d_h=128, d_v=128, softmax_scale=128 ** -0.5)
    assert B.mla_kv_decode_workspace_size(kv, 8, rows // 128, 16) > 0
    assert B.mla_kv_decode_workspace_size(kv, 8, rows // 128 + 1, 16) > 0      # 2^24 pairs is the limit
    assert B.mla_kv_decode_workspace_size(kv, 8, rows, 16) == 0                # 2^27 pairs
    assert B.mla_kv_decode_workspace_size(kv, 128, 8192, pages) == 0           # 2^30 work items
    assert B.mla_kv_decode_workspace_size(kv, 8, 4, pages + 1) == 0
    kvd = lambda n, b, nb, mb: B.mla_kv_decode_attn(kv, n, FAKE, FAKE, FAKE, nb, FAKE, mb, FAKE, b, FAKE,
                                                    1 << 62, FAKE, FAKE, stream=0, check=False)
    assert kvd(8, rows + 1, 100, 16) == B.MLA_ERR_INVALID_ARG
    assert kvd(8, 4, pages + 1, 16) == B.MLA_ERR_INVALID_ARG
    assert kvd(8, rows, 100, 16) == B.MLA_ERR_UNSUPPORTED
    assert kvd(128, 8192, 100, pages) == B.MLA_ERR_UNSUPPORTED


def test_attainable_library_exports_and_validates():
    """libmla_attainable (the matrix-instruction loop the benchmark times) exports what its
    header declares and rejects bad arguments before any HIP call."""
    path = os.path.join(ROOT, "mla_latent_kv_40_amd", "libmla_attainable.so")
    if not os.path.exists(path):
        pytest.fail("libmla_attainable.so is not built (run __graft_entry__.build())")
    src = open(os.path.join(ROOT, "include", "mla_attainable.h")).read()
    syms = set(re.findall(r"^\s*[A-Za-z_0-9]+\s*\*?\s*(mla_[a-z_0-9]+)\s*\(", src, re.M))
    assert syms == {"mla_attainable_mfma_loop", "mla_attainable_read"}
    L = ctypes.CDLL(path)
    rd = L.mla_attainable_read
    rd.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    rd.restype = ctypes.c_int32
    chunk = 36864
    for args in [(2, FAKE, 256 * chunk, 256, FAKE), (-1, FAKE, 256 * chunk, 256, FAKE),
                 (0, FAKE, 256 * chunk, 0, FAKE), (1, FAKE, 256 * chunk, (1 << 16) + 1, FAKE),
                 (0, FAKE, 0, 256, FAKE), (1, FAKE, -chunk, 1, FAKE),
                 (0, FAKE, 256 * chunk + 4, 256, FAKE), (1, FAKE, 255 * chunk, 256, FAKE),
                 (0, FAKE, (1 << 31) // chunk * chunk + chunk, 1, FAKE),   # one slice above 2^31 - 1 bytes
                 (0, None, 256 * chunk, 256, FAKE), (1, FAKE, 256 * chunk, 256, None),
                 (0, FAKE + 16, 256 * chunk, 256, FAKE), (1, FAKE, 256 * chunk, 256, FAKE + 4)]:
        assert rd(*args, None) == -1, args
    fn = L.mla_attainable_mfma_loop
    fn.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    for args in [(2, 256, 16, 0, FAKE), (-1, 256, 16, 0, FAKE), (0, 0, 16, 0, FAKE), (0, (1 << 20) + 1, 16, 0, FAKE),
                 (0, 256, -1, 0, FAKE), (1, 256, (1 << 20) + 1, 0, FAKE), (0, 256, 16, 163841, FAKE),
                 (1, 256, 16, -1, FAKE), (0, 256, 16, 0, None), (1, 256, 16, 0, FAKE + 4)]:
        assert fn(*args, None) == -1, args
