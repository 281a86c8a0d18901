"""Pins of the FP64 oracle against facts that do not depend on the oracle itself.

Each test names the property it checks; together they are chosen so that a dropped term,
a wrong sign or index, or a transposed operand anywhere in oracle/sattn.py fails one.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sattn as O
from oracle.codecs import bf16, e4m3, e4m3_decode, fl32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")


def _bf16_randn(rng, shape, scale=1.0):
    return bf16(rng.standard_normal(shape) * scale)


# ---------------------------------------------------------------- T1: reduces to textbook
@pytest.mark.parametrize("epoch", [64, 7, 1, 1000])
def test_identity_rounding_equals_textbook_softmax(epoch):
    rng = np.random.default_rng(11)
    L, H, D = 150, 2, 128
    q, k, v = (rng.standard_normal((L, H, D)) for _ in range(3))
    q *= 3.0  # peaked rows make the running max move
    sm = D ** -0.5
    got = O.attention_identity(q, k, v, sm, epoch=epoch)
    ref = O.softmax_attention_exact(q, k, v, sm)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- T2: rows sum to one
def test_online_denominator_normalises_probabilities():
    rng = np.random.default_rng(12)
    S = rng.standard_normal((40, 300)) * 6.0
    cps = []
    O.online_softmax_pv(S, np.zeros((300, 4)), quantize_p=True, checkpoints=cps)
    m, d = cps[-1]["m"], cps[-1]["d"]
    assert np.array_equal(m, S.max(axis=1))
    total = np.exp2(S - m[:, None]).sum(axis=1) / d
    assert np.max(np.abs(total - 1.0)) <= 1e-14
    assert len(cps) == math.ceil(300 / 64)


# ---------------------------------------------------------------- T3: K-mean shift invariance
def test_k_mean_shift_leaves_codes_and_scores_unchanged():
    rng = np.random.default_rng(13)
    L, H, D = 128, 2, 128  # L a power of two: the mean is exact
    q = _bf16_randn(rng, (L, H, D))
    k = rng.integers(-128, 128, (L, H, D)) / 16.0  # on a 1/16 grid, |k| <= 8
    v = _bf16_randn(rng, (L, H, D))
    b = rng.integers(-64, 65, (H, D)) / 16.0  # dyadic per-channel bias, |b| <= 4
    k2 = k + b[None]
    assert np.array_equal(bf16(k2), k2)  # the shifted K is still exact in BF16
    cu = [0, L]
    a = O.quantize(q, k, v, cu, cu)[0]
    c = O.quantize(q, k2, v, cu, cu)[0]
    assert np.array_equal(c["k_mean"], a["k_mean"] + b)
    assert np.array_equal(a["k8"], c["k8"]) and np.array_equal(a["k_scale"], c["k_scale"])
    for h in range(H):
        acc_a, s_a = O.scores(a, h, D ** -0.5)
        acc_c, s_c = O.scores(c, h, D ** -0.5)
        assert np.array_equal(acc_a, acc_c) and np.array_equal(s_a, s_c)
    assert np.array_equal(O.attention([a], D ** -0.5), O.attention([c], D ** -0.5))
    # without rounding, the textbook output ignores a per-channel K shift entirely
    o1 = O.attention_identity(q, k, v, D ** -0.5)
    o2 = O.attention_identity(q, k2, v, D ** -0.5)
    assert np.max(np.abs(o1 - o2)) <= 1e-12


def test_k_mean_is_subtracted_per_channel_not_per_token():
    # a K whose channels have different means but whose tokens are all equal: smoothing
    # must turn it into zeros (a per-token mean would leave it non-zero)
    L, H, D = 64, 1, 128
    k = np.broadcast_to(np.arange(D, dtype=np.float64) / 4.0, (L, H, D)).copy()
    km, kp = O.k_smooth(k)
    assert np.array_equal(km[0], np.arange(D) / 4.0)
    assert np.all(kp == 0.0)


# ---------------------------------------------------------------- T4: grid-exact special case
def _grid_exact_problem(rng, L=128, H=2, D=128):
    """Q, K, V for which every quantizer is the identity and every P*448 is an E4M3 value."""
    q = np.zeros((L, H, D))
    k = np.zeros((L, H, D))
    q[:, :, 0] = 127.0  # per-block Q amax 127 -> scale 1; K[:, 0] = 0 so it adds nothing
    k[0::2, :, 1] = 127.0  # K amax 127 in every block; Q[:, 1] = 0 so it adds nothing
    k[1::2, :, 1] = -127.0
    # channels 2..9: small +-1 patterns, K tokens in negated pairs (zero channel mean)
    q[:, :, 2:10] = rng.integers(-1, 2, (L, H, 8))
    kk = rng.integers(-1, 2, (L // 2, H, 8))
    k[0::2, :, 2:10] = kk
    k[1::2, :, 2:10] = -kk
    k[:, :, 10] = np.where(np.arange(L) % 4 < 2, 1.0, -1.0)[:, None]  # non-symmetric extra term
    q[:, :, 10] = rng.integers(0, 2, (L, H))
    # V on the E4M3 grid with per-channel amax exactly 448
    grid = e4m3_decode(np.arange(0, 0x7F))
    grid = np.concatenate([grid, -grid])
    v = rng.choice(grid, (L, H, D))
    v[0, :, :] = 448.0
    return q, k, v


def test_grid_exact_case_equals_brute_force():
    rng = np.random.default_rng(14)
    q, k, v = _grid_exact_problem(rng)
    L, H, D = q.shape
    sm = float(np.float32(math.log(2.0)))
    assert O.sm_scale_log2(sm) == 1.0  # so sigma = 1 and scores are integers
    seg = O.quantize(q, k, v, [0, L], [0, L])[0]
    assert np.all(seg["q_scale"] == 1.0) and np.all(seg["k_scale"] == 1.0)
    assert np.array_equal(seg["q8"], q) and np.array_equal(seg["k8"], k)
    assert np.all(seg["v_scale"] == 1.0) and np.array_equal(seg["v8val"], v)
    for h in range(H):
        acc, S = O.scores(seg, h, sm)
        assert np.array_equal(acc, q[:, h] @ k[:, h].T)  # Q K^T, not K Q^T
        assert np.array_equal(S, acc)
        assert np.max(S.max(axis=1) - S.min(axis=1)) <= 15  # P*448 stays on the grid
    got = O.attention([seg], sm)
    # brute force in base e: softmax(q k^T ln2) = base-2 softmax of the integer scores
    ref = O.softmax_attention_exact(q, k, v, math.log(2.0))
    assert np.max(np.abs(got - bf16(ref))) == 0.0


# ---------------------------------------------------------------- quantizer closed forms
def test_int8_block_scale_and_ties():
    x = np.zeros((64, 1, 128))
    x[0, 0, :4] = np.array([0.5, 1.5, 2.5, 127.0]) / 8.0  # amax = 127/8 -> scale 1/8, inv 8
    x[1, 0, 0] = -2.5 / 8.0
    codes, scales = O.quantize_int8_blocks(x)
    assert scales[0, 0] == 0.125
    assert codes[0, 0, :4].tolist() == [0.0, 2.0, 2.0, 127.0]  # round half to even
    assert codes[1, 0, 0] == -2.0


def test_int8_blocks_are_per_64_tokens_and_partial_tail():
    rng = np.random.default_rng(15)
    x = fl32(rng.standard_normal((70, 2, 128)))
    x[65, 1, 3] = 100.0  # only the second (6-token) block of head 1 sees it
    codes, scales = O.quantize_int8_blocks(x)
    assert scales.shape == (2, 2)
    assert scales[1, 1] == fl32(100.0 / 127.0)
    assert scales[0, 1] == fl32(np.max(np.abs(x[64:, 0])) / 127.0)
    assert scales[1, 0] == fl32(np.max(np.abs(x[:64, 1])) / 127.0)
    assert codes[65, 1, 3] == 127.0 and np.max(np.abs(codes)) == 127.0


def test_zero_blocks_and_channels():
    x = np.zeros((64, 1, 128))
    codes, scales = O.quantize_int8_blocks(x)
    assert np.all(codes == 0) and scales[0, 0] == 0.0
    v8, vals, vs = O.quantize_v(x)
    assert np.all(v8 == 0) and np.all(vs == 0)


def test_blocks_too_small_for_a_finite_reciprocal_are_zero():
    """The edge of the binary32 range, where 127/amax (448/amax for V) overflows: such a
    block or channel is a zero one (scale 0, codes 0), while one just above the edge is
    quantized as usual (its largest value at code 127, or at E4M3 448)."""
    flt_max = float(np.finfo(np.float32).max)
    edge_q, edge_v = 127.0 / flt_max, 448.0 / flt_max  # about 3.7e-37 and 1.3e-36
    x = np.zeros((128, 1, 128))
    x[0, 0, 0], x[1, 0, 5] = bf16(0.5 * edge_q), -bf16(0.25 * edge_q)  # block 0: below the edge
    x[64, 0, 3] = bf16(4.0 * edge_q)  # block 1: above it
    x[65, 0, 7] = -bf16(2.0 * edge_q)
    codes, scales = O.quantize_int8_blocks(x)
    assert scales[0, 0] == 0 and not codes[:64].any()
    assert scales[0, 1] == fl32(bf16(4.0 * edge_q) / 127.0) > 0
    assert codes[64, 0, 3] == 127 and codes[65, 0, 7] == -64
    v = np.zeros((10, 1, 128))
    v[:, 0, 0] = bf16(0.5 * edge_v) * np.linspace(-1, 1, 10)  # channel 0: below the edge
    v[:, 0, 1] = bf16(4.0 * edge_v) * np.linspace(-1, 1, 10)  # channel 1: above it
    v8, vals, vs = O.quantize_v(v)
    assert vs[0, 0] == 0 and not np.any(vals[:, 0, 0])
    assert vs[0, 1] > 0 and np.max(np.abs(vals[:, 0, 1])) == 448.0


def test_v_channel_scale_exact_case():
    v = np.zeros((10, 1, 128))
    v[:, 0, 5] = np.arange(10) * 0.25  # amax 2.25 -> scale fl32(2.25/448), inv fl32(448/2.25)
    v[3, 0, 7] = -7.0  # amax 7 -> inv = 64, values exact: 7*64 = 448
    codes, vals, vs = O.quantize_v(v)
    assert vs[0, 7] == fl32(7.0 / 448.0) and vals[3, 0, 7] == -448.0
    assert vals[9, 0, 5] == 448.0 and vs[0, 5] == fl32(2.25 / 448.0)
    assert np.array_equal(vals[:, 0, 5], e4m3(fl32(np.arange(10) * 0.25 * fl32(448.0 / 2.25))))


# ---------------------------------------------------------------- closed forms of attention
def test_zero_queries_give_the_mean_of_v():
    rng = np.random.default_rng(16)
    L, H, D = 200, 2, 128
    q = np.zeros((L, H, D))
    k = _bf16_randn(rng, (L, H, D))
    v = _bf16_randn(rng, (L, H, D))
    seg = O.quantize(q, k, v, [0, L], [0, L])[0]
    got = O.attention([seg], D ** -0.5)
    # all scores are 0 -> every P is 1 -> P8 = 448 exactly -> O = mean of dequantized V8*v_scale
    mean = seg["v8val"].mean(axis=0) * seg["v_scale"]
    assert np.array_equal(got, np.broadcast_to(bf16(mean), got.shape))


def test_single_key_returns_its_value():
    rng = np.random.default_rng(17)
    q = _bf16_randn(rng, (5, 1, 128))
    k = _bf16_randn(rng, (1, 1, 128))
    v = _bf16_randn(rng, (1, 1, 128))
    seg = O.quantize(q, k, v, [0, 5], [0, 1])[0]
    got = O.attention([seg], 0.1)
    ref = seg["v8val"][0, 0] * seg["v_scale"][0]
    assert np.array_equal(got[:, 0], np.broadcast_to(bf16(ref), (5, 128)))


def test_queries_without_keys_give_zeros():
    rng = np.random.default_rng(18)
    q = _bf16_randn(rng, (3, 1, 128))
    empty = np.zeros((0, 1, 128))
    seg = O.quantize(q, empty, empty, [0, 3], [0, 0])[0]
    assert np.all(O.attention([seg], 0.1) == 0.0)


# ---------------------------------------------------------------- T6: close to exact attention
def test_quantized_program_tracks_exact_attention():
    rng = np.random.default_rng(19)
    L, H, D = 512, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    k = k + bf16(rng.standard_normal((H, D)) * 2.0)[None]
    seg = O.quantize(q, k, v, [0, L], [0, L])[0]
    got = O.attention([seg], D ** -0.5)
    ref = O.softmax_attention_exact(q, k, v, D ** -0.5)
    assert O.rel_l2(got, ref) <= 5e-2


# ---------------------------------------------------------------- T7: exact invariants
def test_v_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(20)
    L, H, D = 130, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    base = O.attention(O.quantize(q, k, v, [0, L], [0, L]), D ** -0.5)
    for p in (3, -5):
        got = O.attention(O.quantize(q, k, v * 2.0 ** p, [0, L], [0, L]), D ** -0.5)
        assert np.array_equal(got, base * 2.0 ** p)


def test_varlen_equals_separate_segments():
    rng = np.random.default_rng(21)
    lens = [70, 1, 0, 129]
    T, H, D = sum(lens), 2, 128
    q, k, v = (_bf16_randn(rng, (T, H, D)) for _ in range(3))
    k[70:71] += 5.0  # segments get different K means
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    joint = O.attention(O.quantize(q, k, v, cu, cu), D ** -0.5)
    parts = [O.attention(O.quantize(q[a:b], k[a:b], v[a:b], [0, b - a], [0, b - a]), D ** -0.5)
             for a, b in O.segments(cu)]
    assert np.array_equal(joint, np.concatenate(parts, axis=0))


def test_head_permutation_permutes_output():
    rng = np.random.default_rng(22)
    L, H, D = 90, 3, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    perm = [2, 0, 1]
    a = O.attention(O.quantize(q, k, v, [0, L], [0, L]), D ** -0.5)
    b = O.attention(O.quantize(q[:, perm], k[:, perm], v[:, perm], [0, L], [0, L]), D ** -0.5)
    assert np.array_equal(a[:, perm], b)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(23)
    L, H, D = 200, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    quant = O.quantize(q, k, v, [0, L], [0, L])
    full = O.attention(quant, D ** -0.5)
    rows = np.array([0, 5, 63, 64, 130, 199])
    sub = O.attention(quant, D ** -0.5, rows={0: rows})[0]
    assert np.array_equal(sub, full[rows])


# ---------------------------------------------------------------- per-warp (32-row) Q scales
def test_q32_scales_are_per_32_rows_and_partial_tail():
    rng = np.random.default_rng(30)
    x = fl32(rng.standard_normal((70, 2, 128)))
    x[40, 1, 7] = 50.0  # rows 32..63 of head 1 only
    x[69, 0, 2] = -80.0  # the 6-row tail block of head 0 only
    codes, scales = O.quantize_int8_blocks(x, 32)
    assert scales.shape == (2, 3)
    assert scales[1, 1] == fl32(50.0 / 127.0) and scales[0, 2] == fl32(80.0 / 127.0)
    for h in range(2):
        for b, (a, e) in enumerate([(0, 32), (32, 64), (64, 70)]):
            assert scales[h, b] == fl32(np.max(np.abs(x[a:e, h])) / 127.0)
    # rows 0..31 keep the codes of their own scale: the outlier at row 40 does not touch them
    c0, _ = O.quantize_int8_blocks(x[:32], 32)
    assert np.array_equal(codes[:32], c0)


def test_q32_doubling_one_half_doubles_only_its_scores():
    """Q rows 32..63 times 2 (exact in BF16): with 32-row scales their codes stay, their
    scale doubles, so their scores double exactly and the other rows' scores do not move.
    With one scale per 64 rows the codes of rows 0..31 would change."""
    rng = np.random.default_rng(31)
    L, H, D = 100, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    q2 = q.copy()
    q2[32:64] *= 2.0
    a = O.quantize(q, k, v, [0, L], [0, L], q_rows=32)[0]
    b = O.quantize(q2, k, v, [0, L], [0, L], q_rows=32)[0]
    assert np.array_equal(a["q8"], b["q8"])
    assert np.array_equal(b["q_scale"][:, 1], 2.0 * a["q_scale"][:, 1])
    assert np.array_equal(np.delete(b["q_scale"], 1, axis=1), np.delete(a["q_scale"], 1, axis=1))
    for h in range(H):
        _, sa = O.scores(a, h, D ** -0.5)
        _, sb = O.scores(b, h, D ** -0.5)
        assert np.array_equal(sb[32:64], 2.0 * sa[32:64])
        assert np.array_equal(np.delete(sb, np.s_[32:64], axis=0), np.delete(sa, np.s_[32:64], axis=0))
    c64 = O.quantize(q2, k, v, [0, L], [0, L])[0]
    assert not np.array_equal(c64["q8"][:32], a["q8"][:32])


def test_q32_equals_q64_when_halves_share_their_amax():
    rng = np.random.default_rng(32)
    L, H, D = 128, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    q[0::32, :, 5] = 9.0  # the largest |q| of every 32-row half, per head: equal halves
    s32 = O.quantize(q, k, v, [0, L], [0, L], q_rows=32)[0]
    s64 = O.quantize(q, k, v, [0, L], [0, L])[0]
    assert np.array_equal(s32["q8"], s64["q8"])
    assert np.array_equal(s32["q_scale"], np.repeat(s64["q_scale"], 2, axis=1))
    assert np.array_equal(O.attention([s32], D ** -0.5), O.attention([s64], D ** -0.5))


def test_q32_program_tracks_exact_attention():
    rng = np.random.default_rng(33)
    L, H, D = 512, 2, 128
    q, k, v = (_bf16_randn(rng, (L, H, D)) for _ in range(3))
    k = k + bf16(rng.standard_normal((H, D)) * 2.0)[None]
    got = O.attention(O.quantize(q, k, v, [0, L], [0, L], q_rows=32), D ** -0.5)
    ref = O.softmax_attention_exact(q, k, v, D ** -0.5)
    assert O.rel_l2(got, ref) <= 5e-2


# ---------------------------------------------------------------- the pages' shape facts
def test_pages_shape_facts():
    facts = json.load(open(GOLDEN))["facts"]
    fs = facts["fixed_shape"]
    assert O.epochs(fs["Lk"]) == fs["key_epochs"] and O.EPOCH == fs["epoch_keys"]
    rng = np.random.default_rng(24)
    q = _bf16_randn(rng, (fs["Lq"], fs["H"], fs["D"]))
    k = _bf16_randn(rng, (fs["Lk"], fs["H"], fs["D"]))
    cps = []
    seg = O.quantize(q, k, k, [0, fs["Lq"]], [0, fs["Lk"]])[0]
    _, S = O.scores(seg, 0, fs["D"] ** -0.5)
    O.online_softmax_pv(S, seg["v8val"][:, 0], checkpoints=cps)
    assert len(cps) == fs["key_epochs"]
    from quantized_attention_video_amd import workloads as W
    h3 = facts["h3_packed_tokens"]
    assert W.get("h3_video_l37810").Lq == h3["tokens"]
    assert W.get("varlen_h24_4seg").seqlens[0] == h3["tokens"] and h3["text_tokens"] in W.get("varlen_h24_4seg").seqlens
    w1 = W.get("fixed_q128_kv192")
    assert (w1.B, w1.H, w1.Lq, w1.Lk) == (fs["B"], fs["H"], fs["Lq"], fs["Lk"])
