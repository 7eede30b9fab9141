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
    assert B.mla_abi_version() == B.ABI_VERSION == 3


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


def test_status_strings(L):
    for code in range(5):
        assert B.mla_status_string(code).startswith("MLA_")
    assert "UNKNOWN" in B.mla_status_string(99)
