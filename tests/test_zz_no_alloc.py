"""mla_decode_attn_noalloc (the decode entry point that allocates nothing: its split-K partials
live in a fixed 64 MiB device array inside the library) against mla_decode_attn with a caller
workspace: bit-identical o_lat and lse, on two calls in a row, the second with a smaller
batch, and the size limit enforced before anything is launched."""
import numpy as np
import pytest

from mla_latent_kv_40_amd import binding as B
from _common import dsv2, log, run_state

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)


def _noalloc(st):
    st.o_lat.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    B.mla_decode_attn_noalloc(st.cfg, st.q_abs, st.cache, st.cache_scale, st.batch.num_blocks, st.block_table,
                              st.batch.max_blocks, st.kv_lens, st.w.batch, st.w.sq, st.o_lat, st.lse)
    torch.cuda.synchronize()
    return st.o_lat.clone(), st.lse.clone()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8b"])
def test_noalloc_equals_decode_attn_twice(fmt):
    log(f"case mla_decode_attn_noalloc vs mla_decode_attn, cache {fmt}: a batch of 6, then a batch of 2")
    f = None if fmt == "bf16" else fmt
    big = dsv2(6, [5000, 3001, 77, 1, 640, 2049], seed=81, fmt=f)
    small = dsv2(2, [130, 64], seed=83, fmt=f)
    states = [run_state(*big), run_state(*small)]   # each ran mla_decode_attn with its own workspace
    for st in states:
        assert st.ws_bytes <= B.NOALLOC_SCRATCH_BYTES
    refs = [(st.o_lat.clone(), st.lse.clone()) for st in states]
    for st, (o_ref, l_ref) in zip(states, refs):      # big first, then the smaller one
        o, l = _noalloc(st)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # and the big one again after the small one left its partials in the shared array
    o, l = _noalloc(states[0])
    assert torch.equal(o, refs[0][0]) and torch.equal(l, refs[0][1])


def test_noalloc_rejects_batches_beyond_its_scratch():
    w, bt, seqs = dsv2(2, [100, 70], seed=85)
    st = run_state(w, bt, seqs)
    # a batch whose partials exceed 64 MiB: 2048 sequences need (G + B - 1) slots of 129 KiB
    big_b, max_blocks = 2048, 4
    need = B.mla_decode_workspace_size(st.cfg, big_b, 1, max_blocks)
    assert need > B.NOALLOC_SCRATCH_BYTES
    kv = torch.zeros(big_b, dtype=torch.int32, device="cuda")
    table = torch.zeros((big_b, max_blocks), dtype=torch.int32, device="cuda")
    o_lat = torch.empty((big_b, 128, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((big_b, 128), dtype=torch.float32, device="cuda")
    st_code = B.mla_decode_attn_noalloc(st.cfg, st.q_abs, st.cache, None, st.batch.num_blocks, table, max_blocks, kv,
                                        big_b, 1, o_lat, lse, check=False)
    assert st_code == B.MLA_ERR_WORKSPACE
