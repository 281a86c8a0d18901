"""Seeded random problems through every path, against the oracle (needs an MI355X).

Each case draws batch or packed segments, head count, lengths, storage layout and the Q
scale granularity, then checks: quantized bytes and scales bit-exact, BF16 output within
the method's tolerance of the oracle, and the fused-Q forward equal to the two-pass one.
"""
import numpy as np
import pytest
import torch

from oracle import sattn as O
from quantized_attention_video_amd import binding as B
from quantized_attention_video_amd import workloads as W

pytestmark = pytest.mark.gpu

MAX_REL, MAE = 1e-2, 1e-3


def _problem(seed):
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    H = int(rng.choice([1, 2, 3, 5, 9, 12, 20]))  # 9..23 heads: unequal heads per XCD (8 XCDs)
    rows = 32 if seed % 2 else 64
    varlen = bool(rng.integers(0, 2))
    if varlen:
        nseg = int(rng.integers(1, 5))
        lq = [int(x) for x in rng.integers(0, 400, nseg)]
        lk = [int(x) for x in rng.integers(0, 900, nseg)]
        lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)
        cu_q, cu_k = [0] + list(np.cumsum(lq)), [0] + list(np.cumsum(lk))
        q = torch.randn((cu_q[-1], H, 128), generator=g)
        k = torch.randn((cu_k[-1], H, 128), generator=g) + 2.0 * torch.randn((H, 128), generator=g)
        v = torch.randn((cu_k[-1], H, 128), generator=g)
        layout = "packed"
    else:
        nseg = int(rng.integers(1, 4))
        layout = str(rng.choice(["blhd", "bhld", "fused"]))
        Lq, Lk = int(rng.integers(1, 500)), int(rng.integers(1, 1100))
        if layout == "fused":  # one [B, L, 3, H, D] projection output: as many keys as queries
            Lk = Lq
        cu_q, cu_k = [i * Lq for i in range(nseg + 1)], [i * Lk for i in range(nseg + 1)]
        q = torch.randn((nseg, Lq, H, 128), generator=g)
        k = torch.randn((nseg, Lk, H, 128), generator=g) + 2.0 * torch.randn((H, 128), generator=g)
        v = torch.randn((nseg, Lk, H, 128), generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    if layout == "bhld":
        q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    elif layout == "fused":
        f = torch.stack([q, k, v], dim=2).contiguous()
        q, k, v = f[:, :, 0], f[:, :, 1], f[:, :, 2]
    return dict(H=H, rows=rows, varlen=varlen, nseg=nseg, cu_q=[int(x) for x in cu_q],
                cu_k=[int(x) for x in cu_k], q=q, k=k, v=v, layout=layout, sm=float(rng.uniform(0.05, 0.12)))


def _to_cuda(t):
    """Device copy with the same strides (fused slices keep their projection stride)."""
    if t.is_contiguous() or t.dim() != 4:
        return t.cuda()
    base = t.as_strided((t.untyped_storage().nbytes() // 2,), (1,), 0).cuda()
    return base.as_strided(t.shape, t.stride(), t.storage_offset())


@pytest.mark.parametrize("seed", range(20))
def test_random_problem(seed):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    p = _problem(1000 + seed)
    H, rows = p["H"], p["rows"]
    q, k, v = (_to_cuda(p[n]) for n in "qkv")
    if p["varlen"]:
        cq = torch.tensor(p["cu_q"], dtype=torch.int32, device="cuda")
        ck = torch.tensor(p["cu_k"], dtype=torch.int32, device="cuda")
        quant = B.sattn_quantize_qkv(q, k, v, cq, ck, q_scale_rows=rows)
        out = B.sattn_fwd_varlen(quant, cq, ck, q.shape[0], p["sm"])
        kv = B.sattn_quantize_kv(q, k, v, cq, ck, q_scale_rows=rows)
        fused = B.sattn_fwd_fused(kv, q, p["sm"], cq, ck, Lk=k.shape[0])
    else:
        Bn, Lq, Lk = q.shape[0], q.shape[1], k.shape[1]
        quant = B.sattn_quantize_qkv(q, k, v, q_scale_rows=rows)
        out = B.sattn_fwd(quant, Bn, H, Lq, Lk, p["sm"])
        kv = B.sattn_quantize_kv(q, k, v, q_scale_rows=rows)
        fused = B.sattn_fwd_fused(kv, q, p["sm"], Lk=Lk)
    torch.cuda.synchronize()
    label = f"seed {seed}: H={H} rows={rows} {p['layout']} cu_q={p['cu_q']} cu_k={p['cu_k']}"
    assert torch.equal(fused, out), label

    oq = O.quantize(*(W.packed_float64(p[n]) for n in "qkv"), p["cu_q"], p["cu_k"], q_rows=rows)
    dense_L = None if p["varlen"] else p["cu_q"][1]
    bq = B.segment_blocks(p["cu_q"], dense_L)
    bk = B.segment_blocks(p["cu_k"], None if p["varlen"] else p["cu_k"][1])
    qt, kt, vt = (getattr(quant, n).cpu().numpy() for n in ("q", "k", "v"))
    qs = quant.q_scale.view(H, quant.qblk_cap, 64 // rows).cpu().numpy()
    ks = quant.k_scale.cpu().numpy()
    for si, seg in enumerate(oq):
        Lq_s, Lk_s = seg["q8"].shape[0], seg["k8"].shape[0]
        nq, nk, nsc = -(-Lq_s // 64), -(-Lk_s // 64), -(-Lq_s // rows)
        for h in range(H):
            assert np.array_equal(B.untile_qk(qt[h, bq[si]:bq[si] + nq])[:Lq_s], seg["q8"][:, h].astype(np.int8)), label
            assert np.array_equal(B.untile_qk(kt[h, bk[si]:bk[si] + nk])[:Lk_s], seg["k8"][:, h].astype(np.int8)), label
            assert np.array_equal(B.untile_v(vt[h, bk[si]:bk[si] + nk])[:Lk_s], seg["v8"][:, h]), label
            assert np.array_equal(qs[h, bq[si]:bq[si] + nq].reshape(-1)[:nsc], seg["q_scale"][h].astype(np.float32))
            assert np.array_equal(ks[h, bk[si]:bk[si] + nk], seg["k_scale"][h].astype(np.float32)), label
    ref = O.attention(oq, p["sm"])
    got = out.float().cpu().numpy().reshape(-1, H, 128).astype(np.float64)
    for si, (a, b) in enumerate(O.segments(p["cu_q"])):
        if b == a:
            continue
        for h in range(H):
            err = np.abs(got[a:b, h] - ref[a:b, h])
            scale = np.max(np.abs(ref[a:b, h]))
            if scale == 0:
                assert np.all(got[a:b, h] == 0), label
                continue
            assert np.max(err) <= MAX_REL * scale, f"{label} seg {si} head {h}: max rel {np.max(err) / scale:.3e}"
            assert np.mean(err) <= MAE, f"{label} seg {si} head {h}: mae {np.mean(err):.3e}"
