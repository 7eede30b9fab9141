"""A decode step captured in a HIP graph (through torch.cuda.graph around the C-ABI calls) and
replayed: every replay, with eager work and synchronisations between them, gives bit for bit the
eager step's outputs.  The library's calls enqueue kernels only (no allocation, no memset, no
host synchronisation inside a call), so a serving loop may capture them; the lazily set kernel
attributes are set by the eager warm-up before the capture."""
import numpy as np
import pytest

from _common import dsv2, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("fmt", ["bf16", "fp8b"])
def test_step_replayed_from_a_graph(fmt):
    from mla_latent_kv_40_amd import harness
    log(f"case decode step in a HIP graph, cache {fmt}: lengths [3000, 65, 1, 700], three replays")
    w, bt, seqs = dsv2(4, [3000, 65, 1, 700], seed=95, fmt=None if fmt == "bf16" else fmt)
    st = harness.DecodeState(w, bt, seqs, device="cuda")
    st.fill_context()
    cache0 = st.cache.clone()
    scale0 = st.cache_scale.clone() if st.cache_scale is not None else None

    def restore():   # the step appends its new tokens: start every run from the same cache
        st.cache.copy_(cache0)
        if scale0 is not None:
            st.cache_scale.copy_(scale0)

    def outputs():
        return [st.out.clone(), st.o_lat.clone(), st.lse.clone(), st.q_abs.clone(), st.cache.clone()]

    restore()
    st.step()
    torch.cuda.synchronize()
    ref = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        restore()
        st.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    for k in range(3):
        restore()
        for t in (st.out, st.o_lat, st.lse, st.q_abs):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        same = [torch.equal(a, b) for a, b in zip(ref, got)]
        log(f"  replay {k}: out, o_lat, lse, q_abs, cache bit-identical to the eager step: {same}")
        assert all(same), k
        # eager work between the replays
        restore()
        st.step()
        torch.cuda.synchronize()
        assert torch.equal(st.o_lat, ref[1])
