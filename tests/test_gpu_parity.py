"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bars: quantized bytes and scales bit-exact; INT32 accumulators and FP32 scores bit-exact;
BF16 output within max|o - r| / max|r| <= 1e-2 and mean|o - r| <= 1e-3 per (segment,
head) — the tolerance stated for this method — plus exact invariants of the program.
"""
import functools
import sys

import numpy as np
import pytest
import torch

from oracle import sattn as O
from quantized_attention_video_amd import binding as B
from quantized_attention_video_amd import workloads as W

pytestmark = pytest.mark.gpu

MAX_REL = 1e-2
MAE = 1e-3


def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sample_rows(L, full_below=2100):
    """All rows of short sequences; of long ones the first, middle and last 64-row blocks
    plus one row of every 128-query tile, its position in the tile varying from tile to tile
    (so that every wave and lane position of the attention workgroups is reached)."""
    if L <= full_below:
        return np.arange(L)
    mid = (L // 2) // 64 * 64
    last = (L - 1) // 64 * 64
    per_tile = np.arange(0, L, 128) + (np.arange(0, L, 128) // 128 * 37) % 128
    return np.unique(np.concatenate([np.arange(0, 64), np.arange(mid, mid + 64), np.arange(last, L),
                                     per_tile[per_tile < L]]))


def _tensor_cu(cu):
    return torch.tensor(cu, dtype=torch.int32, device="cuda")


def gpu_run(inp, sm_scale, q_scale_rows=64):
    """Quantize + forward on the GPU for a workload input dict; returns (quant, out)."""
    w = inp["workload"]
    dev = W.to_device(inp)
    if w.varlen:
        cq, ck = _tensor_cu(inp["cu_q"]), _tensor_cu(inp["cu_k"])
        quant = B.sattn_quantize_qkv(dev["q"], dev["k"], dev["v"], cq, ck, q_scale_rows=q_scale_rows)
        out = B.sattn_fwd_varlen(quant, cq, ck, dev["q"].shape[0], sm_scale)
    else:
        quant = B.sattn_quantize_qkv(dev["q"], dev["k"], dev["v"], q_scale_rows=q_scale_rows)
        Bn, Lq, H = dev["q"].shape[:3]
        out = B.sattn_fwd(quant, Bn, H, Lq, dev["k"].shape[1], sm_scale)
    torch.cuda.synchronize()
    return quant, out


@functools.lru_cache(maxsize=8)
def case(name, q_scale_rows=64):
    """GPU results and oracle quantization of one workload (cached for the session)."""
    _need_gpu()
    w = W.get(name)
    _say(f"[case] {name} (Q scale per {q_scale_rows} rows): generate + GPU")
    inp = W.make_inputs(w)
    quant, out = gpu_run(inp, w.sm_scale, q_scale_rows)
    _say(f"[case] {name}: oracle quantize")
    q64, k64, v64 = (W.packed_float64(inp[n]) for n in "qkv")
    oq = O.quantize(q64, k64, v64, inp["cu_q"], inp["cu_k"], q_rows=q_scale_rows)
    return dict(w=w, inp=inp, quant=quant, out=out, oq=oq)


def _blocks(cu, w):
    return B.segment_blocks(cu, None if w.varlen else (cu[1] - cu[0]))


NAMES = ["fixed_q128_kv192", "dense_h8_l4096", "ragged_b2_h16_l1000", "ragged_b2_h16_l2049", "varlen_h24_4seg",
         "h3_video_l37810"]


def _assert_quantized_equal(quant, oq, bq, bk, H):
    """Every quantized byte and scale of every segment equals the oracle's (bq, bk: first
    quantized block of each segment)."""
    qt, kt, vt = (getattr(quant, n).cpu().numpy() for n in ("q", "k", "v"))
    qs, ks = quant.q_scale.cpu().numpy(), quant.k_scale.cpu().numpy()
    km, vs = quant.k_mean.cpu().numpy(), quant.v_scale.cpu().numpy()
    for si, seg in enumerate(oq):
        Lq, Lk = seg["q8"].shape[0], seg["k8"].shape[0]
        nq, nk = -(-Lq // 64), -(-Lk // 64)
        assert np.array_equal(km[si], seg["k_mean"].astype(np.float32)), f"k_mean seg {si}"
        assert np.array_equal(vs[si], seg["v_scale"].astype(np.float32)), f"v_scale seg {si}"
        for h in range(H):
            gq = B.untile_qk(qt[h, bq[si]:bq[si] + nq])
            gk = B.untile_qk(kt[h, bk[si]:bk[si] + nk])
            gv = B.untile_v(vt[h, bk[si]:bk[si] + nk])
            assert np.array_equal(gq[:Lq], seg["q8"][:, h, :].astype(np.int8)), f"q8 seg {si} head {h}"
            assert np.array_equal(gk[:Lk], seg["k8"][:, h, :].astype(np.int8)), f"k8 seg {si} head {h}"
            assert np.array_equal(gv[:Lk], seg["v8"][:, h, :]), f"v8 seg {si} head {h}"
            assert not gq[Lq:].any() and not gk[Lk:].any() and not gv[Lk:].any(), "padding must be zero"
            assert np.array_equal(qs[h, bq[si]:bq[si] + nq], seg["q_scale"][h].astype(np.float32))
            assert np.array_equal(ks[h, bk[si]:bk[si] + nk], seg["k_scale"][h].astype(np.float32))


@pytest.mark.parametrize("name", NAMES)
def test_quantized_buffers_bit_exact(name):
    c = case(name)
    w, inp = c["w"], c["inp"]
    _assert_quantized_equal(c["quant"], c["oq"], _blocks(inp["cu_q"], w), _blocks(inp["cu_k"], w), w.H)


def debug_run(c, seg, head, q0, q1, step=1, nep=0):
    """sattn_debug_scores for one (segment, head) of a cached case, as the case was run."""
    w, inp, quant = c["w"], c["inp"], c["quant"]
    if w.varlen:
        cq, ck = _tensor_cu(inp["cu_q"]), _tensor_cu(inp["cu_k"])
        lk = inp["cu_k"][seg + 1] - inp["cu_k"][seg]
        r = B.sattn_debug_scores(quant, w.sm_scale, seg, head, q0, q1, step, ld=lk, nep=nep, cu_seqlens_q=cq,
                                 cu_seqlens_k=ck)
    else:
        r = B.sattn_debug_scores(quant, w.sm_scale, seg, head, q0, q1, step, Lq=inp["q"].shape[1],
                                 Lk=inp["k"].shape[1], nep=nep)
    torch.cuda.synchronize()
    return r


def _seg_rows(c, seg):
    cu = c["inp"]["cu_q"]
    return cu[seg + 1] - cu[seg]


def assert_scores_exact(c, seg, head, q0, q1, step):
    """INT32 accumulators and FP32 scores of the sampled rows bit-exact against the oracle,
    and the checkpoint run's output rows bit-identical to the forward's."""
    w = c["w"]
    rows = np.arange(q0, min(q1, _seg_rows(c, seg)), step)
    r = debug_run(c, seg, head, q0, q1, step)
    _say(f"[scores] {w.name} seg {seg} head {head}: {len(rows)} rows x {r['acc'].shape[1]} keys")
    r_acc, r_s = O.scores(c["oq"][seg], head, w.sm_scale, rows)
    acc, sc = r["acc"][:len(rows)].cpu().numpy(), r["s"][:len(rows)].cpu().numpy()
    bad = np.argwhere(acc.astype(np.int64) != r_acc.astype(np.int64))
    assert len(bad) == 0, f"INT32 accumulators differ at {len(bad)} (row, key) pairs, first {bad[:5].tolist()}"
    bad = np.argwhere(sc != r_s.astype(np.float32))
    assert len(bad) == 0, f"FP32 scores differ at {len(bad)} (row, key) pairs, first {bad[:5].tolist()}"
    if w.varlen:
        base = c["inp"]["cu_q"][seg]
        got, ref = r["out"][base + rows, head], c["out"][base + rows, head]
    else:
        got, ref = r["out"][seg, rows, head], c["out"][seg, rows, head]
    assert torch.equal(got, ref), "the checkpoint run's output rows differ from the forward's"


# (workload, segment, head, first row, row step): all rows of the small shapes; one row of
# every 128-query tile (the position in the tile moving by one from tile to tile) of the
# long sequences, in the launch configuration the throughput benchmark times.
SCORE_CASES = [("fixed_q128_kv192", 0, 0, 0, 1), ("dense_h8_l4096", 0, 5, 3, 13), ("ragged_b2_h16_l1000", 1, 9, 0, 1),
               ("ragged_b2_h16_l2049", 1, 3, 0, 1), ("ragged_b2_h16_l2049", 0, 15, 5, 3),
               ("h3_video_l37810", 0, 0, 0, 129), ("h3_video_l37810", 0, 17, 64, 129),
               ("h3_video_l37810", 0, 31, 127, 129),
               ("varlen_h24_4seg", 0, 0, 11, 129), ("varlen_h24_4seg", 0, 23, 100, 129),
               ("varlen_h24_4seg", 1, 7, 0, 65), ("varlen_h24_4seg", 2, 12, 0, 7), ("varlen_h24_4seg", 3, 5, 0, 1),
               ("varlen_h24_4seg", 3, 18, 0, 1)]


@pytest.mark.parametrize("name,seg,head,q0,step", SCORE_CASES)
def test_scores_bit_exact(name, seg, head, q0, step):
    assert_scores_exact(case(name), seg, head, q0, _seg_rows(case(name), seg), step)


def _check_output(got, ref, label):
    for h in range(ref.shape[1]):
        err = np.abs(got[:, h] - ref[:, h])
        scale = np.max(np.abs(ref[:, h]))
        assert np.max(err) <= MAX_REL * scale, f"{label} head {h}: max rel {np.max(err) / scale:.3e}"
        assert np.mean(err) <= MAE, f"{label} head {h}: mae {np.mean(err):.3e}"


@functools.lru_cache(maxsize=4)
def oracle_rows(name, q_scale_rows=64):
    """The oracle's output on the sampled rows of every segment and head: (rows, ref)."""
    c = case(name, q_scale_rows)
    oq = c["oq"]
    rows = {si: _sample_rows(seg["q8"].shape[0]) for si, seg in enumerate(oq)}
    _say(f"[oracle] {name}: attention on {sum(len(r) for r in rows.values())} rows of each of {c['w'].H} heads")
    return rows, O.attention(oq, c["w"].sm_scale, rows=rows)


@pytest.mark.parametrize("name", NAMES)
def test_output_within_tolerance(name):
    c = case(name)
    w, inp = c["w"], c["inp"]
    out = c["out"].float().cpu()
    rows, ref = oracle_rows(name)
    for si, (a, b) in enumerate(O.segments(inp["cu_q"])):
        if w.varlen:
            got = out[a:b].numpy()
        else:
            got = out[si].numpy()
        _check_output(got[rows[si]].astype(np.float64), ref[si], f"{name} seg {si}")
    assert torch.isfinite(c["out"].float()).all()


@pytest.mark.parametrize("name", NAMES)
def test_quantization_error_against_exact_attention(name):
    """A diagnostic of the method rather than of the kernel: the relative L2 distance of the
    GPU output from textbook FP64 softmax attention on the same BF16 inputs (the pages'
    own accuracy measure), printed beside the kernel's distance from the oracle, and held
    to the oracle's own sanity bound of 5e-2.  The kernel's distance from the oracle must
    be a small fraction of the method's distance from exact attention."""
    c = case(name)
    w, oq, inp = c["w"], c["oq"], c["inp"]
    q64, k64, v64 = (W.packed_float64(inp[n]) for n in "qkv")
    out = c["out"].float().cpu().numpy().astype(np.float64)
    rows, ref = oracle_rows(name)
    d_ex = d_or = n_ex = 0.0
    for si, ((a, b), (ka, kb)) in enumerate(zip(O.segments(inp["cu_q"]), O.segments(inp["cu_k"]))):
        if b == a or kb == ka:
            continue
        r = rows[si]
        ex = O.softmax_attention_exact(q64[a:b][r], k64[ka:kb], v64[ka:kb], w.sm_scale)
        got = (out[a:b] if w.varlen else out[si])[r]
        d_ex += float(np.sum((got - ex) ** 2))
        d_or += float(np.sum((got - ref[si]) ** 2))
        n_ex += float(np.sum(ex ** 2))
    rl2_exact, rl2_oracle = (d_ex / n_ex) ** 0.5, (d_or / n_ex) ** 0.5
    _say(f"[diag] {name}: rel-L2 vs exact FP64 attention {rl2_exact:.4f}, vs the oracle {rl2_oracle:.2e}")
    assert rl2_exact <= 5e-2
    assert rl2_oracle <= 0.1 * rl2_exact


# ---------------------------------------------------------------- per-warp (32-row) Q scales
Q32_NAMES = ["fixed_q128_kv192", "ragged_b2_h16_l1000", "ragged_b2_h16_l2049", "varlen_h24_4seg"]


@pytest.mark.parametrize("name", Q32_NAMES)
def test_q32_quantized_buffers_bit_exact(name):
    c = case(name, 32)
    w, quant, oq, inp = c["w"], c["quant"], c["oq"], c["inp"]
    qt, kt = quant.q.cpu().numpy(), quant.k.cpu().numpy()
    qs = quant.q_scale.view(w.H, quant.qblk_cap, 2).cpu().numpy()
    ks = quant.k_scale.cpu().numpy()
    bq, bk = _blocks(inp["cu_q"], w), _blocks(inp["cu_k"], w)
    for si, seg in enumerate(oq):
        Lq, Lk = seg["q8"].shape[0], seg["k8"].shape[0]
        nq, nk, n32 = -(-Lq // 64), -(-Lk // 64), -(-Lq // 32)
        assert seg["q_scale"].shape[1] == n32
        for h in range(w.H):
            gq = B.untile_qk(qt[h, bq[si]:bq[si] + nq])
            assert np.array_equal(gq[:Lq], seg["q8"][:, h, :].astype(np.int8)), f"q8 seg {si} head {h}"
            assert not gq[Lq:].any(), "padding must be zero"
            halves = qs[h, bq[si]:bq[si] + nq].reshape(-1)
            assert np.array_equal(halves[:n32], seg["q_scale"][h].astype(np.float32)), f"q_scale seg {si} head {h}"
            assert not halves[n32:].any(), "the scale of an empty half is 0"
            gk = B.untile_qk(kt[h, bk[si]:bk[si] + nk])
            assert np.array_equal(gk[:Lk], seg["k8"][:, h, :].astype(np.int8)), f"k8 seg {si} head {h}"
            assert np.array_equal(ks[h, bk[si]:bk[si] + nk], seg["k_scale"][h].astype(np.float32))


@pytest.mark.parametrize("name,seg,head,q0,step", [("fixed_q128_kv192", 0, 0, 0, 1), ("ragged_b2_h16_l1000", 1, 9, 0, 1),
                                                   ("ragged_b2_h16_l2049", 0, 3, 0, 1), ("varlen_h24_4seg", 0, 3, 31, 129),
                                                   ("varlen_h24_4seg", 2, 20, 0, 5)])
def test_q32_scores_bit_exact(name, seg, head, q0, step):
    c = case(name, 32)
    assert_scores_exact(c, seg, head, q0, _seg_rows(c, seg), step)


@pytest.mark.parametrize("name", Q32_NAMES)
def test_q32_output_within_tolerance(name):
    c = case(name, 32)
    w, inp = c["w"], c["inp"]
    out = c["out"].float().cpu()
    rows, ref = oracle_rows(name, 32)
    for si, (a, b) in enumerate(O.segments(inp["cu_q"])):
        got = out[a:b].numpy() if w.varlen else out[si].numpy()
        _check_output(got[rows[si]].astype(np.float64), ref[si], f"{name} (32-row Q scales) seg {si}")
    assert torch.isfinite(c["out"].float()).all()


# ---------------------------------------------------------------- Q preparation fused into the forward
@pytest.mark.parametrize("name,rows", [("fixed_q128_kv192", 64), ("dense_h8_l4096", 64), ("ragged_b2_h16_l1000", 64),
                                       ("ragged_b2_h16_l2049", 32), ("varlen_h24_4seg", 64), ("varlen_h24_4seg", 32),
                                       ("h3_video_l37810", 64)])
def test_fused_q_forward_equals_two_pass(name, rows):
    """sattn_fwd_fused (Q quantized inside the attention launch, read from the BF16 view,
    projection-strided for the video layout) gives the two-pass output bit for bit, and
    the K/V-only preparation writes the same K/V buffers as the full one."""
    c = case(name, rows)
    w, inp, quant = c["w"], c["inp"], c["quant"]
    dev = W.to_device(inp)
    _say(f"[fused] {name}: K/V-only quantize + fused forward")
    if w.varlen:
        cq, ck = _tensor_cu(inp["cu_q"]), _tensor_cu(inp["cu_k"])
        kv = B.sattn_quantize_kv(dev["q"], dev["k"], dev["v"], cq, ck, q_scale_rows=rows)
        out = B.sattn_fwd_fused(kv, dev["q"], w.sm_scale, cq, ck, Lk=dev["k"].shape[0])
    else:
        kv = B.sattn_quantize_kv(dev["q"], dev["k"], dev["v"], q_scale_rows=rows)
        out = B.sattn_fwd_fused(kv, dev["q"], w.sm_scale, Lk=dev["k"].shape[1])
    torch.cuda.synchronize()
    assert kv.q is None and kv.q_scale is None
    for n in ("k_mean", "v_scale"):
        assert torch.equal(getattr(kv, n), getattr(quant, n)), n
    bk = _blocks(inp["cu_k"], w)  # capacity blocks beyond the segments are never written
    for si, (a, b) in enumerate(O.segments(inp["cu_k"])):
        blk = slice(bk[si], bk[si] + -(-(b - a) // 64))
        for n in ("k", "k_scale", "v"):
            assert torch.equal(getattr(kv, n)[:, blk], getattr(quant, n)[:, blk]), f"{n} seg {si}"
    assert torch.equal(out, c["out"])


def test_varlen_equals_per_segment_dense():
    _need_gpu()
    rng = torch.Generator().manual_seed(7)
    lens = [70, 1, 0, 129, 300, 64]
    T, H = sum(lens), 3
    q, k, v = (torch.randn((T, H, 128), generator=rng).to(torch.bfloat16) for _ in range(3))
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    cq = _tensor_cu(cu)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    quant = B.sattn_quantize_qkv(qd, kd, vd, cq, cq)
    joint = B.sattn_fwd_varlen(quant, cq, cq, T, 128 ** -0.5)
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if b == a:
            continue
        qs, ks, vs = (t[a:b].unsqueeze(0) for t in (qd, kd, vd))
        part = B.sattn_fwd(B.sattn_quantize_qkv(qs, ks, vs), 1, H, b - a, b - a, 128 ** -0.5)
        assert torch.equal(joint[a:b], part[0]), f"segment {s}"


def test_v_power_of_two_scaling_is_exact():
    c = case("ragged_b2_h16_l1000")
    w = c["w"]
    inp = dict(c["inp"])
    inp["v"] = inp["v"] * 8.0  # exact in BF16
    _, out = gpu_run(inp, w.sm_scale)
    assert torch.equal(out.float(), c["out"].float() * 8.0)


def test_head_permutation_permutes_output():
    """Heads are independent: permuting the heads of Q, K and V permutes the output heads
    bit for bit (although other workgroups, on other XCDs, now compute each head)."""
    _need_gpu()
    g = torch.Generator().manual_seed(17)
    H, L = 11, 333
    q, k, v = (torch.randn((2, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    perm = torch.randperm(H, generator=g).cuda()
    out = B.sattn_fwd(B.sattn_quantize_qkv(q, k, v), 2, H, L, L, 0.09)
    qp, kp, vp = (t[:, :, perm] for t in (q, k, v))  # strided views: the head stride is not H*D
    outp = B.sattn_fwd(B.sattn_quantize_qkv(*(t.contiguous() for t in (qp, kp, vp))), 2, H, L, L, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(outp, out[:, :, perm])


def test_k_mean_shift_changes_nothing_on_the_gpu():
    """K -> K + b with a dyadic per-(head, channel) b, K on a 1/16 grid and L a power of two,
    so every mean and every K - mean is exact: the INT8 K codes and scales, the INT32
    scores and the output are bit-identical (the K-smoothing invariance, on the GPU)."""
    _need_gpu()
    g = torch.Generator().manual_seed(19)
    H, L = 3, 256
    q = torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16)
    k = (torch.randint(-128, 128, (1, L, H, 128), generator=g) / 16.0).to(torch.bfloat16)
    v = torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16)
    b = (torch.randint(-64, 65, (H, 128), generator=g) / 16.0)
    k2 = (k.float() + b).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + b)  # still exact in BF16
    qa, qb = (B.sattn_quantize_qkv(q.cuda(), kk.cuda(), v.cuda()) for kk in (k, k2))
    torch.cuda.synchronize()
    assert torch.equal(qb.k_mean.cpu(), qa.k_mean.cpu() + b[None])
    nb = L // 64  # the blocks written (the buffers hold one more of capacity, never written)
    assert torch.equal(qb.k[:, :nb], qa.k[:, :nb]) and torch.equal(qb.k_scale[:, :nb], qa.k_scale[:, :nb])
    for h in range(H):
        ra = B.sattn_debug_scores(qa, 0.0884, 0, h, 0, L, Lq=L, Lk=L)
        rb = B.sattn_debug_scores(qb, 0.0884, 0, h, 0, L, Lq=L, Lk=L)
        torch.cuda.synchronize()
        assert torch.equal(ra["acc"], rb["acc"]) and torch.equal(ra["s"], rb["s"])
        assert torch.equal(ra["out"][:, :, h], rb["out"][:, :, h])


def test_two_streams_at_once_match_one_after_the_other():
    """The library keeps no state between calls: two problems quantized and attended on two
    streams at the same time give the same bits as the same calls made one after another."""
    _need_gpu()
    g = torch.Generator().manual_seed(31)
    probs = []
    for H, L in ((4, 700), (3, 1100)):
        probs.append(tuple(torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3)))

    def run(p):
        q, k, v = p
        H, L = q.shape[2], q.shape[1]
        return B.sattn_fwd(B.sattn_quantize_qkv(q, k, v), 1, H, L, L, 0.09)

    seq = [run(p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = [None, None]
    for _ in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs[i] = run(probs[i])
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(outs, seq))


def test_quantize_and_forward_replay_from_a_captured_graph():
    """The whole step captured in one HIP graph (no memset nodes: the library issues none)
    and replayed with new inputs copied into the captured buffers: every replay equals the
    eager result for those inputs, with eager work and synchronisations in between."""
    _need_gpu()
    g = torch.Generator().manual_seed(37)
    H, L = 3, 600
    q, k, v = (torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    quant = B.sattn_quantize_qkv(q, k, v)  # buffers reused by the captured calls
    out = torch.empty((1, L, H, 128), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side, as torch recommends
        B.sattn_quantize_qkv(q, k, v, out=quant)
        B.sattn_fwd(quant, 1, H, L, L, 0.09, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.sattn_quantize_qkv(q, k, v, out=quant)
        B.sattn_fwd(quant, 1, H, L, L, 0.09, out=out)
    for _ in range(3):
        new = [torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
        ref = B.sattn_fwd(B.sattn_quantize_qkv(*new), 1, H, L, L, 0.09)  # eager, fresh buffers
        torch.cuda.synchronize()
        for dst, src in zip((q, k, v), new):
            dst.copy_(src)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_repeated_launches_are_bitwise_identical():
    c = case("dense_h8_l4096")
    w = c["w"]
    _, out = gpu_run(c["inp"], w.sm_scale)
    for _ in range(20):
        o2 = B.sattn_fwd(c["quant"], 1, 8, 4096, 4096, w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, out)


def test_many_tiny_segments_beyond_the_sorted_schedule():
    """5,000 packed segments of 0..6 queries and 0..9 keys: more segments than the
    longest-first schedule sorts (4,096), so the launch keeps the input order; one
    statistics block per segment-head.  Bytes and output against the oracle."""
    _need_gpu()
    rng = np.random.default_rng(5)
    lq, lk = rng.integers(0, 7, 5000), rng.integers(0, 10, 5000)
    cu_q, cu_k = [0] + [int(x) for x in np.cumsum(lq)], [0] + [int(x) for x in np.cumsum(lk)]
    g = torch.Generator().manual_seed(5)
    H = 2
    q = torch.randn((cu_q[-1], H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((cu_k[-1], H, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((cu_k[-1], H, 128), generator=g).to(torch.bfloat16)
    cq, ck = _tensor_cu(cu_q), _tensor_cu(cu_k)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda(), cq, ck)
    out = B.sattn_fwd_varlen(quant, cq, ck, cu_q[-1], 0.1)
    torch.cuda.synchronize()
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu_q, cu_k)
    # a per-segment K mean enters the scores as a per-query constant, to which the softmax is
    # blind: only the bytes show whether every segment's statistics are the right ones
    _assert_quantized_equal(quant, oq, B.segment_blocks(cu_q, None), B.segment_blocks(cu_k, None), H)
    ref = O.attention(oq, 0.1)
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.max(err) <= MAX_REL * np.max(np.abs(ref)) and np.mean(err) <= MAE
    empty_k = np.repeat(lk == 0, lq)
    assert np.all(got[empty_k] == 0)


def test_degenerate_values():
    """Zero scales everywhere they can occur: segment 0 has K constant over its tokens (the
    smoothed K is zero, every k_scale 0, every score 0: uniform attention); segment 1 has an
    all-zero 64-query block (q_scale 0) and an all-zero V channel (v_scale 0)."""
    _need_gpu()
    g = torch.Generator().manual_seed(11)
    H, L = 2, 300
    q = torch.randn((2, L, H, 128), generator=g)
    k = torch.randn((2, L, H, 128), generator=g)
    v = torch.randn((2, L, H, 128), generator=g)
    k[0] = torch.randn((1, H, 128), generator=g)  # constant over segment 0's tokens
    q[1, 64:128] = 0.0
    v[1, :, :, 5] = 0.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    out = B.sattn_fwd(quant, 2, H, L, L, 0.0884)
    torch.cuda.synchronize()
    assert not quant.k_scale[:, :5].any()  # segment 0's five K blocks
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(got[1, :, :, 5] == 0)
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), [0, L, 2 * L], [0, L, 2 * L])
    ref = O.attention(oq, 0.0884)
    for si in range(2):
        _check_output(got[si], ref[si * L:(si + 1) * L], f"degenerate seg {si}")
    # uniform attention: every query of segment 0 sees the same weights, so all its rows agree
    assert np.all(got[0] == got[0, :1])


@pytest.mark.parametrize("sm_scale", [1e-4, 1.0, 4.0])
def test_extreme_softmax_scales(sm_scale):
    """Nearly flat (sm_scale 1e-4: every P close to 1, O close to the mean of V) and sharply
    peaked rows (1.0 and 4.0: score spans of tens to hundreds in base 2, so most P underflow
    E4M3 and one or two keys carry each row), against the oracle."""
    _need_gpu()
    g = torch.Generator().manual_seed(13)
    H, Lq, Lk = 2, 200, 333
    q = torch.randn((1, Lq, H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((1, Lk, H, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((1, Lk, H, 128), generator=g).to(torch.bfloat16)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    out = B.sattn_fwd(quant, 1, H, Lq, Lk, sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)[0]
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), [0, Lq], [0, Lk])
    ref = O.attention(oq, sm_scale)
    _check_output(got, ref, f"sm_scale {sm_scale}")


def test_blocks_too_small_for_a_finite_reciprocal():
    """Values at the bottom of the binary32 range (a Q block, all of one segment's K, a V
    channel below ~1e-36, where 127/amax or 448/amax overflows): zero blocks and channels,
    byte for byte as the oracle; the fused-Q forward agrees; the output stays finite."""
    _need_gpu()
    g = torch.Generator().manual_seed(41)
    H, L = 2, 200
    q = torch.randn((2, L, H, 128), generator=g)
    k = torch.randn((2, L, H, 128), generator=g)
    v = torch.randn((2, L, H, 128), generator=g)
    q[0, 64:128] *= 1e-38  # one Q block
    k[1] *= 1e-38          # all of segment 1's K: mean and smoothed K that small too
    v[0, :, :, 9] *= 1e-37  # one V channel
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    quant = B.sattn_quantize_qkv(qd, kd, vd)
    out = B.sattn_fwd(quant, 2, H, L, L, 0.0884)
    kv = B.sattn_quantize_kv(qd, kd, vd)
    fused = B.sattn_fwd_fused(kv, qd, 0.0884, Lk=L)
    torch.cuda.synchronize()
    cu = [0, L, 2 * L]
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu, cu)
    assert oq[0]["q_scale"][0, 1] == 0 and not oq[1]["k_scale"].any() and oq[0]["v_scale"][0, 9] == 0
    _assert_quantized_equal(quant, oq, B.segment_blocks(cu, L), B.segment_blocks(cu, L), H)
    assert torch.equal(fused, out)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    ref = O.attention(oq, 0.0884)
    for si in range(2):
        _check_output(got[si], ref[si * L:(si + 1) * L], f"tiny values seg {si}")


def test_thousand_launches_of_the_fixed_shape_agree():
    """The pages' fixed shape (B=1, H=1, 128 queries, 192 keys in three K64 epochs) run
    1,000 times back to back on one stream: every output identical to the first."""
    c = case("fixed_q128_kv192")
    w = c["w"]
    outs = torch.empty((1000, 1, 128, 1, 128), dtype=torch.bfloat16, device="cuda")
    for i in range(1000):
        B.sattn_fwd(c["quant"], 1, 1, 128, 192, w.sm_scale, out=outs[i])
    torch.cuda.synchronize()
    assert torch.equal(outs, c["out"].expand_as(outs))


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (5, 64), (64, 65), (300, 3), (257, 1000), (31, 129), (33, 63), (127, 191),
                                   (128, 128), (129, 576), (200, 897), (96, 1280)])
def test_small_shapes_and_untouched_padding(Lq, Lk):
    _need_gpu()
    g = torch.Generator().manual_seed(Lq * 1000 + Lk)
    H, Bn = 2, 2
    q = torch.randn((Bn, Lq, H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((Bn, Lk, H, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((Bn, Lk, H, 128), generator=g).to(torch.bfloat16)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    # write into the middle of a larger canary-filled tensor: nothing else may change
    big = torch.full((Bn, Lq + 3, H + 1, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, 1:Lq + 1, :H, 64:192]
    B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09, out=view)
    torch.cuda.synchronize()
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[:, 1:Lq + 1, :H, 64:192] = False
    assert torch.all(big[mask] == 7.0)
    cu_q = [0, Lq, 2 * Lq]
    cu_k = [0, Lk, 2 * Lk]
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu_q, cu_k)
    ref = O.attention(oq, 0.09)
    got = view.float().cpu().reshape(-1, H, 128).numpy().astype(np.float64)
    for s in range(Bn):
        _check_output(got[s * Lq:(s + 1) * Lq], ref[s * Lq:(s + 1) * Lq], f"Lq={Lq} Lk={Lk} seg {s}")


def test_queries_without_keys_give_zeros():
    _need_gpu()
    g = torch.Generator().manual_seed(3)
    cu_q, cu_k = [0, 5, 10, 80], [0, 0, 7, 7]
    q = torch.randn((80, 2, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((7, 2, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((7, 2, 128), generator=g).to(torch.bfloat16)
    cq, ck = _tensor_cu(cu_q), _tensor_cu(cu_k)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda(), cq, ck)
    out = B.sattn_fwd_varlen(quant, cq, ck, 80, 0.1).float().cpu().numpy()
    assert np.all(out[0:5] == 0) and np.all(out[10:80] == 0)
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu_q, cu_k)
    ref = O.attention(oq, 0.1)
    _check_output(out[5:10].astype(np.float64), ref[5:10], "seg 1")
    assert np.all(ref[0:5] == 0) and np.all(ref[10:] == 0)
    # the fused-Q forward on the same packed batch (empty key segments included)
    kv = B.sattn_quantize_kv(q.cuda(), k.cuda(), v.cuda(), cq, ck)
    fused = B.sattn_fwd_fused(kv, q.cuda(), 0.1, cq, ck, Lk=7).float().cpu().numpy()
    assert np.array_equal(fused, out)


@pytest.mark.timeout(600)
def test_long_key_sequence_reads_scales_through_the_scalar_cache():
    """More than 2048 key blocks per segment: the kernel reads the K block scales through
    the scalar cache instead of copying them to LDS.  Output vs the oracle; the fused-Q
    forward on the same inputs is bit-identical."""
    _need_gpu()
    g = torch.Generator().manual_seed(77)
    H, Lq, Lk = 2, 200, 2048 * 64 + 1000
    q = torch.randn((1, Lq, H, 128), generator=g).to(torch.bfloat16)
    k = (torch.randn((1, Lk, H, 128), generator=g) + 1.5).to(torch.bfloat16)
    v = torch.randn((1, Lk, H, 128), generator=g).to(torch.bfloat16)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    quant = B.sattn_quantize_qkv(qd, kd, vd)
    out = B.sattn_fwd(quant, 1, H, Lq, Lk, 0.0884)
    kv = B.sattn_quantize_kv(qd, kd, vd)
    fused = B.sattn_fwd_fused(kv, qd, 0.0884, Lk=Lk)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    _say("[oracle] long key sequence: 200 rows x 132,072 keys x 2 heads")
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), [0, Lq], [0, Lk])
    ref = O.attention(oq, 0.0884)
    _check_output(out[0].float().cpu().numpy().astype(np.float64), ref, "Lk=132072")


@pytest.mark.timeout(900)
def test_large_shape_sampled_heads():
    """The 74K-token, 56-head shape in the bench's launch configuration: every quantized byte
    and scale of three heads bit-exact, and sampled output rows of those heads in
    tolerance.  The oracle runs on the three heads only (quantization and attention are
    per head), the GPU on all 56."""
    _need_gpu()
    w = W.get("h3_video_l74000_h56")
    _say(f"[case] {w.name}: generate + GPU")
    inp = W.make_inputs(w)
    quant, out = gpu_run(inp, w.sm_scale)
    heads = [0, 29, 55]
    _say(f"[case] {w.name}: oracle on heads {heads}")
    sub = {n: W.packed_float64(inp[n][:, :, heads]) for n in "qkv"}
    oq = O.quantize(sub["q"], sub["k"], sub["v"], inp["cu_q"], inp["cu_k"])
    seg = oq[0]
    nblk = -(-w.Lq // 64)
    qt = quant.q.view(w.H, -1, 8192)
    kt = quant.k.view(w.H, -1, 8192)
    vt = quant.v.view(w.H, -1, 8192)
    qs = quant.q_scale.view(w.H, -1)
    ks = quant.k_scale.view(w.H, -1)
    km = quant.k_mean.cpu().numpy()[0]
    vsc = quant.v_scale.cpu().numpy()[0]
    assert np.array_equal(km[heads], seg["k_mean"].astype(np.float32)), "k_mean"
    assert np.array_equal(vsc[heads], seg["v_scale"].astype(np.float32)), "v_scale"
    for j, h in enumerate(heads):
        got_q = B.untile_qk(qt[h, :nblk].cpu().numpy())[:w.Lq]
        got_k = B.untile_qk(kt[h, :nblk].cpu().numpy())[:w.Lk]
        got_v = B.untile_v(vt[h, :nblk].cpu().numpy())[:w.Lk]
        assert np.array_equal(got_q, seg["q8"][:, j, :].astype(np.int8)), f"q8 head {h}"
        assert np.array_equal(got_k, seg["k8"][:, j, :].astype(np.int8)), f"k8 head {h}"
        assert np.array_equal(got_v, seg["v8"][:, j, :].astype(np.uint8)), f"v8 head {h}"
        assert np.array_equal(qs[h, :nblk].cpu().numpy(), seg["q_scale"][j].astype(np.float32)), f"q_scale {h}"
        assert np.array_equal(ks[h, :nblk].cpu().numpy(), seg["k_scale"][j].astype(np.float32)), f"k_scale {h}"
    # one score row in about every second 128-query tile of head 29, bit-exact
    srows = np.arange(3, w.Lq, 257)
    r = B.sattn_debug_scores(quant, w.sm_scale, 0, 29, 3, w.Lq, 257, Lq=w.Lq, Lk=w.Lk)
    torch.cuda.synchronize()
    r_acc, r_s = O.scores(seg, heads.index(29), w.sm_scale, srows)
    assert np.array_equal(r["acc"].cpu().numpy().astype(np.int64), r_acc.astype(np.int64)), "INT32 scores, head 29"
    assert np.array_equal(r["s"].cpu().numpy(), r_s.astype(np.float32)), "FP32 scores, head 29"
    assert torch.equal(r["out"][0, srows, 29], out[0, srows, 29])
    rows = _sample_rows(w.Lq)
    ref = O.attention(oq, w.sm_scale, rows={0: rows})[0]
    got = out[0][rows][:, heads].float().cpu().numpy().astype(np.float64)
    _check_output(got, ref, w.name)
    assert torch.isfinite(out.float()).all()



# ---------------------------------------------------------------- per-epoch checkpoints
EPS_MFMA = 2.0 ** -11  # error of one FP8 matrix instruction, relative to the magnitudes it adds
def _ulp32(x):
    """Spacing of binary32 values at |x| (elementwise, FP64)."""
    x = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 23)


def _e4m3_midpoint_distance(x):
    """Relative distance of x > 0 from the nearest rounding midpoint of the E4M3 grid
    (4 significant bits, subnormal spacing 2^-9)."""
    x = np.asarray(x, dtype=np.float64)
    step = np.where(x >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(x, 2.0 ** -6))) - 3), 2.0 ** -9)
    mid = (np.floor(x / step) + 0.5) * step
    return np.abs(x - mid) / np.maximum(x, 1e-300)


@pytest.mark.parametrize("name,seg,head,q0,step", [("fixed_q128_kv192", 0, 0, 0, 1), ("ragged_b2_h16_l1000", 1, 4, 2, 7),
                                                   ("ragged_b2_h16_l2049", 0, 11, 0, 13), ("varlen_h24_4seg", 3, 9, 0, 1)])
def test_epoch_checkpoints_against_the_oracle(name, seg, head, q0, step):
    """The per-epoch checkpoints of the Phase 2B report's "Exactness" list, from the forward
    kernel's own registers, against the oracle's recurrence on the same rows:
      * running max m: exact (both are maxima of the same binary32 scores);
      * rescale factor alpha: 0 on the first epoch, 1 where m did not change, else within the
        error of the hardware exp2 of fl32(m - m') (2^-22 relative + the argument's rounding);
      * E4M3 probability bytes: identical, except where the FP64 448 P lies within the GPU's
        bound on its exponent-argument error of an E4M3 rounding midpoint (each such key is
        printed with its distance);
      * denominator (units of 448 P): within a bound derived from the FP32 partial sums;
      * running output RO: within a bound built from the per-instruction precision of the
        FP8 matrix instruction (E4M3 products are exact, but the instruction adds its 64
        products and the accumulator with less than FP32 precision: about 2^-14 of the sum
        of their magnitudes on gfx950, measured; the bound allows 2^-11), the rescale and
        the flipped bytes;
      * the epilogue's final reciprocal 1 / (448 d): the correctly rounded binary32
        reciprocal of the kernel's own d, and within d's bound of the oracle's.
    The hardware exp2 is not correctly rounded, so alpha, d and RO cannot be compared bit
    for bit."""
    c = case(name)
    w = c["w"]
    oseg = c["oq"][seg]
    L = _seg_rows(c, seg)
    Lk = oseg["k8"].shape[0]
    nep = -(-Lk // 64)
    rows = np.arange(q0, L, step)
    r = debug_run(c, seg, head, q0, L, step, nep=nep)
    g = {k: v[:len(rows)].cpu().numpy() for k, v in r.items() if k != "out"}
    _, S = O.scores(oseg, head, w.sm_scale, rows)
    vv = oseg["v8val"][:, head, :]
    cps = []
    O.online_softmax_pv(S, vv, checkpoints=cps)
    log2_448 = float(np.float32(np.log2(448.0)))
    flips = 0
    ro_bound = np.zeros((len(rows), 128))  # bound on |RO_gpu - RO_oracle| after the epoch
    d_rel = 0.0                            # accumulated relative error of the rescale factors in d
    for e, cp in enumerate(cps):
        m, alpha, p8, ro = cp["m"], cp["alpha"], cp["p"], cp["RO"]
        k0, k1 = 64 * e, min(64 * e + 64, Lk)
        assert np.array_equal(g["m"][:, e], m.astype(np.float32)), f"m, epoch {e}"
        ga = g["alpha"][:, e].astype(np.float64)
        if e == 0:
            assert np.all(ga == 0)
            eps_a = np.zeros(len(rows))
        else:
            prev = cps[e - 1]["m"]
            same = prev == m
            assert np.all(ga[same] == 1.0), f"alpha != 1 where m did not change, epoch {e}"
            eps_a = np.where(same, 0.0, 2.0 ** -22 + np.log(2) * _ulp32(prev - m) / 2)
            assert np.all(np.abs(ga - alpha) <= alpha * eps_a), f"alpha, epoch {e}"
        # the GPU's exponent argument fl32(acc*sigma - fl32(m' - log2 448)) against the exact
        # S - m' + log2 448: the roundings of S, of m' - log2 448 (with the binary32 log2 448)
        # and of the argument, then the hardware exp2 (2^-22 relative)
        Se = S[:, k0:k1]
        mm = (m - log2_448).astype(np.float32).astype(np.float64)
        arg = Se - m[:, None] + np.log2(448.0)
        eps = np.log(2) * (_ulp32(Se) + _ulp32(mm)[:, None] + _ulp32(arg) + 2.0 ** -20) / 2 + 2.0 ** -22
        p448 = 448.0 * np.exp2(Se - m[:, None])
        ref_b = O.e4m3_encode(p8)
        got_b = g["p8"][:, e, :k1 - k0]
        diff = np.argwhere(got_b != ref_b)
        for i, j in diff:
            dist = _e4m3_midpoint_distance(p448[i, j])
            _say(f"[p8] {name} epoch {e} row {rows[i]} key {k0 + j}: 448P = {p448[i, j]:.9g}, "
                 f"{dist:.2e} from a rounding midpoint (bound {eps[i, j]:.2e}), bytes {got_b[i, j]} vs {ref_b[i, j]}")
            assert dist <= eps[i, j], "an E4M3 byte differs away from a rounding midpoint"
            assert abs(int(got_b[i, j]) - int(ref_b[i, j])) == 1, "a flip moves by more than one E4M3 step"
        flips += len(diff)
        # d in units of 448 P: each term within eps; FP32 partial sums of 8, then 4 and 2, the
        # rescale and the two half-waves (about 14 roundings per epoch); the rescale factors' errors
        d_rel = d_rel + float(np.max(eps_a))
        dref = 448.0 * cp["d"]
        tol_d = dref * (float(np.max(eps)) + d_rel + 14 * (e + 1) * 2.0 ** -24)
        assert np.all(np.abs(g["d"][:, e] - dref) <= tol_d), f"d, epoch {e}"
        # RO: the previous error rescaled, the rescale's rounding and alpha's error on the
        # previous RO, one matrix instruction's error on its accumulator and 64 exact products
        # (EPS_MFMA of their magnitudes), and the bytes that flipped
        gp = O.e4m3_decode(got_b)
        prev_ro = cps[e - 1]["RO"] if e else np.zeros_like(ro)
        terms = (np.abs(prev_ro) + ro_bound) * alpha[:, None] + np.abs(p8) @ np.abs(vv[k0:k1])
        ro_bound = (ro_bound * alpha[:, None] * (1 + eps_a[:, None]) + np.abs(prev_ro) * alpha[:, None] *
                    (eps_a[:, None] + 2.0 ** -24) + EPS_MFMA * terms + np.abs(gp - p8) @ np.abs(vv[k0:k1]))
        err = np.abs(g["ro"][:, e, :] - ro)
        assert np.all(err <= ro_bound * 1.001 + 1e-30), f"RO, epoch {e}: max excess {np.max(err - ro_bound):.3e}"
    _say(f"[checkpoints] {name} seg {seg} head {head}: {len(rows)} rows x {nep} epochs, {flips} E4M3 bytes at "
         f"rounding midpoints")
    assert flips <= max(2, 1e-4 * len(rows) * Lk), "too many probability bytes differ"
    # the final reciprocal: the correctly rounded binary32 1/x of the kernel's own final d
    # (units of 448 P), and within d's bound of the oracle's 1 / (448 d)
    rcp = r["rcp"][:len(rows)].cpu().numpy()
    d_last = g["d"][:, nep - 1].astype(np.float32)
    assert np.array_equal(rcp, np.float32(1.0) / d_last), "rcp is not fl32(1 / d)"
    ref_rcp = 1.0 / (448.0 * cps[-1]["d"])
    assert np.all(np.abs(rcp - ref_rcp) <= ref_rcp * (tol_d / dref + 2.0 ** -24)), "rcp against the oracle"


# ---------------------------------------------------------------- key split of small grids
def _ntile(Lq):
    return -(-(-(-Lq // 64) * 64) // 128)


def _split_plan(Bn, H, Lq, Lk):
    """The library's rule: the work items of each XCD's last dispatch round (two workgroups
    per CU, cus/8 CUs per XCD; the whole grid when it is shorter than a round) are split
    into k = 4 or 2 pieces when k of them each get a CU of their own and the keys span at
    least 8 k epochs.  Returns (split tiles, pieces); (0, 1) when nothing is split."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_xcd = -(-H // 8) * Bn * _ntile(Lq)
    last = per_xcd % (cus // 4)
    tiles = min(H, 8) * last
    for k, cap in ((4, 64), (2, 128)):
        if last and k * last <= cus // 8 and -(-Lk // 64) >= 8 * k and tiles <= cap:
            return tiles, k
    return 0, 1


def _split_last(Bn, H, Lq, Lk):
    return _split_plan(Bn, H, Lq, Lk)[0]


def _splits(Bn, H, Lq, Lk):
    return _split_last(Bn, H, Lq, Lk) > 0


def _counter_bytes(tiles):
    """The split workspace starts with one 32-bit counter per tile, padded to 256 bytes."""
    return -(-tiles * 4 // 256) * 256


def _close_bf16(a, b):
    """Within one BF16 rounding of each other, plus 2^-10 of the row's largest magnitude.  The
    split changes only the order in which O and d accumulate; a matrix instruction's
    accumulation error is relative to the magnitudes it sums, not to the result, so an output
    element that cancels to near zero (1e-7 against a row maximum of 0.07) can move by more
    than its own BF16 step while staying 1e-8 of the row's scale."""
    a, b = a.float(), b.float()
    row = torch.maximum(a.abs(), b.abs()).amax(dim=-1, keepdim=True)
    return bool(torch.all((a - b).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), b.abs()) + 2.0 ** -10 * row + 1e-30))


def _split_inputs(Bn, H, Lq, Lk, seed, loud_rows=0.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((Bn, Lq, H, 128), generator=g)
    if loud_rows:  # a share of the query rows scaled by 8: large, late running maxima
        q[torch.rand((Bn, Lq), generator=g) < loud_rows] *= 8.0
    k = torch.randn((Bn, Lk, H, 128), generator=g)
    v = torch.randn((Bn, Lk, H, 128), generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def _split_oracle_check(out, q, k, v, sm_scale, label, rows=None, q_rows=64):
    Bn, Lq, H = q.shape[:3]
    Lk = k.shape[1]
    cu_q, cu_k = [Lq * i for i in range(Bn + 1)], [Lk * i for i in range(Bn + 1)]
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu_q, cu_k, q_rows=q_rows)
    sel = {s: (np.arange(Lq) if rows is None else rows) for s in range(Bn)}
    ref = O.attention(oq, sm_scale, rows=sel)
    got = out.float().cpu().numpy().astype(np.float64)
    for s in range(Bn):
        _check_output(got[s][sel[s]], ref[s], f"{label} seg {s}")


@pytest.mark.parametrize("Bn,H,Lq,Lk,pieces", [(1, 1, 128, 4096, 4), (1, 2, 1000, 2049, 4), (1, 8, 2048, 1024, 2),
                                              (2, 1, 200, 37810, 4), (1, 8, 1024, 1100, 2)])
def test_key_split_long_keys(Bn, H, Lq, Lk, pieces):
    """sattn_fwd with its forward workspace on a grid small enough that 2 or 4 pieces of
    every query tile get a CU of their own: the tile's keys are split between that many
    workgroups (each later one first takes the running max over the earlier keys, so every
    E4M3 probability is the sequential recurrence's) and the pieces merge.  20 calls in a
    row give identical bits and leave the counters at zero; the result differs from the
    unsplit forward only by the order of the O and d sums, equals the fused-Q forward's
    split bit for bit, and meets the oracle's tolerance (5% of the query rows scaled by 8)."""
    _need_gpu()
    assert _split_plan(Bn, H, Lq, Lk)[1] == pieces
    q, k, v = _split_inputs(Bn, H, Lq, Lk, seed=Bn * 1000 + H * 100 + Lk, loud_rows=0.05)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    plain = B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09)
    ws = B.split_workspace(Bn, H, Lq, Lk)
    outs = [B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09, workspace=ws) for _ in range(20)]
    torch.cuda.synchronize()
    ncnt = _counter_bytes(_split_last(Bn, H, Lq, Lk))
    assert not ws[:ncnt].any(), "the split counters must be left at zero"
    assert ws[ncnt:].any(), "the split did not run (no partials in the workspace)"
    out = outs[0]
    assert all(torch.equal(o, out) for o in outs[1:])
    assert _close_bf16(out, plain)
    # the fused-Q forward splits by the same rule (its Q operands are ready before the second
    # half's running-max pass): the same bits
    qd = q.cuda()
    kv = B.sattn_quantize_kv(qd, k.cuda(), v.cuda())
    ws2 = B.split_workspace(Bn, H, Lq, Lk)
    fused = B.sattn_fwd_fused(kv, qd, 0.09, Lk=Lk, workspace=ws2)
    torch.cuda.synchronize()
    assert not ws2[:ncnt].any() and ws2[ncnt:].any()
    assert torch.equal(fused, out), "fused-Q split differs from the two-pass split"
    rows = None if Lq * Lk <= 2_100_000 else np.unique(np.r_[0:8, Lq - 8:Lq, np.arange(0, Lq, 37)])
    _split_oracle_check(out, q, k, v, 0.09, f"split B={Bn} H={H} Lq={Lq} Lk={Lk}", rows)


def test_key_split_with_32_row_q_scales():
    """The split with one Q scale per 32 query rows (each wave's own scale; the pieces'
    running-max passes use it too): 4 pieces of one tile, against the unsplit forward and
    the oracle's 32-row program, and the fused-Q split bit for bit."""
    _need_gpu()
    Bn, H, Lq, Lk = 1, 1, 128, 4096
    assert _split_plan(Bn, H, Lq, Lk)[1] == 4
    q, k, v = _split_inputs(Bn, H, Lq, Lk, seed=3232, loud_rows=0.05)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    quant = B.sattn_quantize_qkv(qd, kd, vd, q_scale_rows=32)
    plain = B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09)
    ws = B.split_workspace(Bn, H, Lq, Lk)
    out = B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09, workspace=ws)
    kv = B.sattn_quantize_kv(qd, kd, vd, q_scale_rows=32)
    ws2 = B.split_workspace(Bn, H, Lq, Lk)
    fused = B.sattn_fwd_fused(kv, qd, 0.09, Lk=Lk, workspace=ws2)
    torch.cuda.synchronize()
    ncnt = _counter_bytes(_split_last(Bn, H, Lq, Lk))
    assert not ws[:ncnt].any() and ws[ncnt:].any()
    assert torch.equal(fused, out)
    assert _close_bf16(out, plain)
    _split_oracle_check(out, q, k, v, 0.09, "split, 32-row Q scales", q_rows=32)


def test_key_split_of_the_last_round():
    """B=2, H=16, L=2,049: 17 query tiles per (sequence, head), 544 workgroups, 32 more than
    fit at once, so each XCD's last round holds 4 tiles: those are split (their halves then
    run on CUs of their own).  20 calls give identical bits, the counters are left at
    zero; the output differs from the unsplit one only by the summation order of the split
    tiles and meets the oracle's tolerance on the sampled rows of every head."""
    name = "ragged_b2_h16_l2049"
    c = case(name)
    inp, quant, w = c["inp"], c["quant"], c["w"]
    Bn, Lq, H = inp["q"].shape[:3]
    Lk = inp["k"].shape[1]
    tiles, pieces = _split_plan(Bn, H, Lq, Lk)
    assert tiles == 32 and pieces == 4
    ws = B.split_workspace(Bn, H, Lq, Lk)
    outs = [B.sattn_fwd(quant, Bn, H, Lq, Lk, w.sm_scale, workspace=ws) for _ in range(20)]
    torch.cuda.synchronize()
    ncnt = _counter_bytes(tiles)
    assert not ws[:ncnt].any() and ws[ncnt:].any(), "the last round was not split"
    out = outs[0]
    assert all(torch.equal(o, out) for o in outs[1:])
    assert _close_bf16(out, c["out"])
    rows, ref = oracle_rows(name)
    got = out.float().cpu()
    for si in range(len(O.segments(inp["cu_q"]))):
        _check_output(got[si].numpy()[rows[si]].astype(np.float64), ref[si], f"{name} last-round split seg {si}")


@pytest.mark.parametrize("name", ["dense_h8_l4096", "ragged_b2_h16_l1000"])
def test_key_split_not_taken_on_full_grids(name):
    """Grids of 256 workgroups (32 per XCD, one dispatch round; split, their 64 halves would
    share the XCD's 32 CUs) run unsplit even with a workspace: the same bits as without
    one, the workspace untouched."""
    c = case(name)
    inp, quant, w = c["inp"], c["quant"], c["w"]
    Bn, Lq, H = inp["q"].shape[:3]
    Lk = inp["k"].shape[1]
    assert not _splits(Bn, H, Lq, Lk)
    ws = B.split_workspace(Bn, H, Lq, Lk)
    out = B.sattn_fwd(quant, Bn, H, Lq, Lk, w.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    assert not ws.any()
    assert torch.equal(out, c["out"])


@pytest.mark.parametrize("Lq,Lk", [(64, 1025), (129, 1088), (200, 1345), (96, 1280), (257, 1000), (33, 4097)])
def test_key_split_small_shapes(Lq, Lk):
    """Split forward on shapes around tile and epoch boundaries (odd epoch counts, a one-key
    tail, partial query tiles), against the oracle and the unsplit forward."""
    _need_gpu()
    g = torch.Generator().manual_seed(Lq * 7 + Lk)
    H, Bn = 3, 2
    assert _splits(Bn, H, Lq, Lk)
    q = torch.randn((Bn, Lq, H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((Bn, Lk, H, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((Bn, Lk, H, 128), generator=g).to(torch.bfloat16)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    plain = B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09)
    ws = B.split_workspace(Bn, H, Lq, Lk)
    split = B.sattn_fwd(quant, Bn, H, Lq, Lk, 0.09, workspace=ws)
    torch.cuda.synchronize()
    ncnt = _counter_bytes(_split_last(Bn, H, Lq, Lk))
    assert not ws[:ncnt].any() and ws[ncnt:].any()
    assert _close_bf16(split, plain)
    cu_q, cu_k = [0, Lq, 2 * Lq], [0, Lk, 2 * Lk]
    oq = O.quantize(W.packed_float64(q), W.packed_float64(k), W.packed_float64(v), cu_q, cu_k)
    ref = O.attention(oq, 0.09)
    got = split.float().cpu().reshape(-1, H, 128).numpy().astype(np.float64)
    for s in range(Bn):
        _check_output(got[s * Lq:(s + 1) * Lq], ref[s * Lq:(s + 1) * Lq], f"split Lq={Lq} Lk={Lk} seg {s}")


def test_key_split_replays_from_a_captured_graph():
    """The split forward captured in a HIP graph with its workspace: each replay (eager work
    and synchronisations between them) equals the eager split result, and the counters stay
    zero."""
    _need_gpu()
    g = torch.Generator().manual_seed(43)
    H, L = 2, 1100
    assert _splits(1, H, L, L)
    q, k, v = (torch.randn((1, L, H, 128), generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    quant = B.sattn_quantize_qkv(q, k, v)
    ws = B.split_workspace(1, H, L, L)
    ref = B.sattn_fwd(quant, 1, H, L, L, 0.09, workspace=ws).clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.sattn_fwd(quant, 1, H, L, L, 0.09, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.sattn_fwd(quant, 1, H, L, L, 0.09, out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert not ws[:_counter_bytes(_split_last(1, H, L, L))].any()
        B.sattn_fwd(quant, 1, H, L, L, 0.09, workspace=ws)  # eager work between the replays
        torch.cuda.synchronize()
