"""sattn_quantize_qkv_noalloc (the quantizer with the library's per-device scratch array as
its workspace) against sattn_quantize_qkv, through the C ABI (needs an MI355X): every
output buffer bit-identical, on two calls in a row, the second with a smaller problem."""
import pytest
import torch

from quantized_attention_video_amd import binding as B

pytestmark = pytest.mark.gpu

NAMES = ("q", "q_scale", "k", "k_scale", "k_mean", "v", "v_scale")


def _zeroed(nseg, tq, tk, H, rows=64):
    out = B.alloc_quantized(nseg, tq, tk, H, q_scale_rows=rows)
    for n in NAMES:
        getattr(out, n).zero_()  # blocks beyond the segments are never written: compare them too
    return out


def _problem(seed, packed):
    g = torch.Generator().manual_seed(seed)
    if packed:
        lens = [1900, 700, 1, 333]
        cu = [0]
        for n in lens:
            cu.append(cu[-1] + n)
        H, T = 24, cu[-1]
        q, k, v = (torch.randn((T, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
        c = torch.tensor(cu, dtype=torch.int32, device="cuda")
        return dict(q=q, k=k, v=v, cu=c, nseg=len(lens), tq=T, tk=T, H=H)
    H, L, Bn = 3, 300, 2
    q, k, v = (torch.randn((Bn, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    return dict(q=q, k=k, v=v, cu=None, nseg=Bn, tq=Bn * L, tk=Bn * L, H=H)


def _check(p, rows):
    ref = _zeroed(p["nseg"], p["tq"], p["tk"], p["H"], rows)
    got = _zeroed(p["nseg"], p["tq"], p["tk"], p["H"], rows)
    B.sattn_quantize_qkv(p["q"], p["k"], p["v"], p["cu"], p["cu"], out=ref)
    B.sattn_quantize_qkv_noalloc(p["q"], p["k"], p["v"], got, p["cu"], p["cu"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(getattr(got, n), getattr(ref, n)), n


def test_noalloc_equals_the_workspace_form_twice_the_second_smaller():
    assert torch.cuda.is_available()
    assert B.sattn_noalloc_scratch_bytes() == 16 << 20
    big, small = _problem(1, True), _problem(2, False)
    assert B.sattn_quant_query(big["nseg"], big["tq"], big["tk"], big["H"]).quant_workspace_bytes > \
        B.sattn_quant_query(small["nseg"], small["tq"], small["tk"], small["H"]).quant_workspace_bytes
    _check(big, 64)
    _check(small, 32)  # the scratch array keeps the first call's sums: none may leak into this one


def test_noalloc_rejects_a_workspace_beyond_the_array():
    n = 9000  # segment-heads: 9000 * 2 KiB of statistics > 16 MiB
    out = B.alloc_quantized(n, n, n, 1)
    cu = torch.arange(n + 1, dtype=torch.int32, device="cuda")
    x = torch.zeros((n, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SattnError) as e:
        B.sattn_quantize_qkv_noalloc(x, x, x, out, cu, cu)
    assert e.value.status == B.SATTN_ENOSPACE
