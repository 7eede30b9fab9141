"""GPU parity of the per-head key/value cache decode (mla_kv_decode_attn, the multi-head and
grouped-query layout MLA replaces), through the C ABI, against oracle.attention."""
import numpy as np
import pytest

import oracle.mla_oracle as orc
from mla_latent_kv_40_amd import binding as B, workloads as wl
from _common import check, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)


def kv_cfg():
    return B.Config(num_heads=128, d_c=512, d_r=64, d_h=128, d_v=128, softmax_scale=128 ** -0.5)


@pytest.mark.parametrize("h_kv", [128, 64, 32, 16, 8])   # 1, 2, 4, 8 and 16 query heads per key/value head
def test_kv_cache_decode(h_kv):
    lengths = [1, 63, 64, 65, 200, 3000, 0]
    log(f"case per-head key/value cache decode: H=128, H_kv={h_kv}, lengths {lengths}")
    H, d = 128, 128
    rng = np.random.default_rng(200 + h_kv)
    kv = np.asarray(lengths, dtype=np.int32)
    nblk = np.maximum((kv + 63) // 64, 1)
    pool = int(nblk.sum())
    perm = rng.permutation(pool).astype(np.int32)
    max_blocks = int(nblk.max())
    table = np.full((len(kv), max_blocks), -1, np.int32)
    off = 0
    for b in range(len(kv)):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += int(nblk[b])
    k_pages = np.zeros((pool, h_kv, 64, d), np.float32)
    v_pages = np.zeros((pool, h_kv, d, 64), np.float32)   # value pages stored transposed
    Ks, Vs = [], []
    for b, L in enumerate(kv):
        K = wl.round_bf16(rng.standard_normal((L, h_kv, d), dtype=np.float32))
        V = wl.round_bf16(rng.standard_normal((L, h_kv, d), dtype=np.float32))
        t = np.arange(L)
        pg = table[b, t // 64]
        k_pages[pg, :, t % 64] = K
        v_pages[pg, :, :, t % 64] = V
        Ks.append(K)
        Vs.append(V)
    q = wl.round_bf16(rng.standard_normal((len(kv), H, d), dtype=np.float32))
    dev = lambda x, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    cfg = kv_cfg()
    ws = B.mla_kv_decode_workspace_size(cfg, h_kv, len(kv), max_blocks)
    assert ws > 0
    work = torch.empty(ws, dtype=torch.uint8, device="cuda")
    work.view(torch.float32)[: ws // 4].fill_(float("nan"))
    o = torch.full((len(kv), H, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((len(kv), H), float("nan"), dtype=torch.float32, device="cuda")
    B.mla_kv_decode_attn(cfg, h_kv, dev(q), dev(k_pages), dev(v_pages), pool, dev(table, torch.int32), max_blocks,
                         dev(kv, torch.int32), len(kv), work, ws, o, lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b, L in enumerate(kv):
        ref = orc.attention(q[b], Ks[b], Vs[b], cfg.softmax_scale)
        if L == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        check(f"b{b} (kv_len {L}) o", o[b], ref["o"])
        check(f"b{b} (kv_len {L}) lse", lse[b], ref["lse"])
