"""FP64 oracle of the quantized attention program (test infrastructure only).

Sources (the pages): "H3 Performance Roadmap", the Sage2 phase
decomposition (K smoothing, Q/K INT8 quantization, V transpose/FP8 quantization, fused
mainloop) and "Phase 4: Dense Sage-Compatible Attention" (per-warp INT8 Q/K, FP8 V
policy, K smoothing); "Phase 2B Aligned Numerical Prototype",
sections "Decision" (three increasing K64 epochs over KV=192) and "Exactness" (INT32 to
FP32 QK scores, per-epoch online-softmax m and d, E4M3 probability words, FP32 rescale
values, PV partials into FP32 RO, final reciprocal, BF16 output).

Where the pages leave a step open, the plainest reading is taken:
  * the K mean is taken per (sequence, head, channel) over that sequence's keys, summed
    in FP64 and rounded once to FP32; the smoothed K is rounded once to FP32;
  * Q and smoothed K are quantized per 64-token block (symmetric, RNE, codes in
    [-127, 127], scale = fl32(amax/127), multiply by fl32(127/amax)); the "per-warp"
    policy of the roadmap's Phase 4 is also available for Q as one scale per 32 query
    rows (the rows one of four QK warps owns in a 128-query tile), K staying per 64;
  * V is quantized per (sequence, head, channel): scale fl32(amax/448), multiply by
    fl32(448/amax), E4M3 RNE;
  * a Q/K block or V channel whose amax is 0, or so small that its binary32 reciprocal
    overflows (fl32(127/amax) or fl32(448/amax) = inf), gets scale 0 and zero codes;
  * sm_scale and log2(e) are folded into the per-block score scale
    sigma = fl32(fl32(q_scale * c) * k_scale) with c = fl32(sm_scale * log2 e);
  * the score is fl32(acc * sigma), acc the exact integer dot product;
  * the online softmax runs in base 2 over 64-key epochs in increasing key order:
    m' = max(m, max S), alpha = 2^(m - m') (0 for the first epoch), P = 2^(S - m'),
    d = d*alpha + sum P (unquantized P), P8 = e4m3(448 P), RO = RO*alpha + P8 . V8;
  * O = bf16(RO / d * v_scale / 448), evaluated in FP64 and rounded once.
Everything between the explicit roundings is FP64.  Both the pages' FP16 PV partials
and the GPU's FP32 accumulators are replaced here by exact FP64 sums.

Every array is float64 unless stated; token-major [T, H, D] layouts; segments are given
by Python lists of prefix sums (cu_seqlens).
"""
import math

import numpy as np

from .codecs import bf16, e4m3, e4m3_decode, e4m3_encode, fl32, rne

LOG2E = 1.4426950408889634  # the float64 nearest to log2(e)
BLOCK = 64  # tokens per Q/K quantization block
EPOCH = 64  # keys per online-softmax epoch


# ----------------------------------------------------------------------------- helpers
def segments(cu):
    """[(start, end)] of each segment of a prefix-sum list."""
    cu = [int(c) for c in cu]
    return list(zip(cu[:-1], cu[1:]))


def sm_scale_log2(sm_scale):
    """c = fl32(sm_scale * log2 e), with sm_scale first taken as binary32 (the C API's float)."""
    return float(fl32(float(np.float32(sm_scale)) * LOG2E))


def quantize_int8_blocks(x, block=None):
    """Symmetric INT8 quantization of [L, H, D] per `block`-token block (default 64) and head.

    Returns codes [L, H, D] (float64 integers in [-127, 127]) and scales [H, nblk].
    scale = fl32(amax/127) and inv = fl32(127/amax) are each one correctly rounded
    binary32 operation: the float64 quotient of two binary32 operands rounded again to
    binary32 equals the correctly rounded binary32 quotient, because 53 >= 2*24 + 2.
    x*inv is exact in float64 (24 + 24 bits), so fl32 applies the single rounding.
    An all-zero block gets scale 0 and codes 0, and so does a block whose amax is too
    small for a finite binary32 reciprocal (fl32(127/amax) = inf, amax < 127/FLT_MAX,
    about 3.7e-37): the pages leave it open, and x*inf would make NaN codes.
    """
    block = BLOCK if block is None else block
    L, H, D = x.shape
    nblk = -(-L // block)
    codes = np.zeros_like(x)
    scales = np.zeros((H, nblk))
    for b in range(nblk):
        blk = x[b * block:(b + 1) * block]  # [n, H, D]; the last block may be partial
        amax = np.max(np.abs(blk), axis=(0, 2))  # [H]
        safe = np.where(amax > 0, amax, 1.0)
        with np.errstate(over="ignore"):
            inv_all = fl32(127.0 / safe)
        nz = (amax > 0) & np.isfinite(inv_all)
        scale = np.where(nz, fl32(safe / 127.0), 0.0)
        inv = np.where(nz, inv_all, 0.0)
        q = np.clip(rne(fl32(blk * inv[None, :, None])), -127.0, 127.0)
        codes[b * block:(b + 1) * block] = q
        scales[:, b] = scale
    return codes, scales


def k_smooth(k):
    """Per-channel mean of K over the segment's tokens and the smoothed K' (both FP32 values).

    k_mean[h, c] = fl32(fl64(sum_t K[t, h, c]) / L): the sum is accumulated in FP64 (exact
    for inputs whose magnitudes span fewer than 53 - 8 - log2(L) binades, which holds for
    the workloads here), divided in FP64 and rounded once to binary32 (both steps are
    correctly rounded, so any reduction order that keeps the sum exact agrees).
    K' = fl32(K - k_mean).  An empty segment has mean 0.
    """
    L = k.shape[0]
    if L == 0:
        return np.zeros(k.shape[1:]), k.copy()
    mean = fl32(np.sum(k, axis=0) / L)
    return mean, fl32(k - mean[None])


def quantize_v(v):
    """Per-(head, channel) E4M3 quantization of V [L, H, D] over the segment's tokens.

    Returns (codes uint8 [L, H, D], values float64 [L, H, D], v_scale [H, D]).
    """
    L, H, D = v.shape
    amax = np.max(np.abs(v), axis=0) if L else np.zeros((H, D))
    safe = np.where(amax > 0, amax, 1.0)
    with np.errstate(over="ignore"):
        inv_all = fl32(448.0 / safe)
    nz = (amax > 0) & np.isfinite(inv_all)  # as for INT8: no finite reciprocal, a zero channel
    scale = np.where(nz, fl32(safe / 448.0), 0.0)
    inv = np.where(nz, inv_all, 0.0)
    vals = e4m3(fl32(v * inv[None]))
    return e4m3_encode(vals), vals, scale


def quantize(q, k, v, cu_q, cu_k, q_rows=None):
    """Quantize packed Q/K/V ([T, H, D] float64 holding BF16 values) per segment.

    q_rows: query rows per Q scale, 64 (default, one per 64-token block) or 32 (the
    per-warp variant).  Returns a list with one dict per segment: q8 [Lq, H, D], q_scale
    [H, ceil(Lq/q_rows)], q_rows, k_mean [H, D], k8 [Lk, H, D], k_scale [H, nkblk], v8
    (uint8 codes) [Lk, H, D], v8val [Lk, H, D], v_scale [H, D].
    """
    q_rows = BLOCK if q_rows is None else q_rows
    out = []
    for (qs, qe), (ks, ke) in zip(segments(cu_q), segments(cu_k)):
        q8, qsc = quantize_int8_blocks(q[qs:qe], q_rows)
        km, kp = k_smooth(k[ks:ke])
        k8, ksc = quantize_int8_blocks(kp)
        v8, v8val, vsc = quantize_v(v[ks:ke])
        out.append(dict(q8=q8, q_scale=qsc, q_rows=q_rows, k_mean=km, k8=k8, k_scale=ksc, v8=v8, v8val=v8val,
                        v_scale=vsc))
    return out


# ----------------------------------------------------------------------------- scores
def block_sigma(q_scale_h, k_scale_h, c32):
    """sigma[bq, bk] = fl32(fl32(q_scale[bq] * c) * k_scale[bk]) (bq a block of q_rows queries)."""
    a = fl32(q_scale_h * c32)
    return fl32(a[:, None] * k_scale_h[None, :])


def scores(seg, h, sm_scale, rows=None):
    """Exact INT32 accumulators and FP32 scores (log2 units) of one segment and head.

    acc[i, j] = sum_c q8[i, c] k8[j, c] (exact: |acc| <= 128*127^2 < 2^53, so the FP64
    product below is exact); S = fl32(acc * sigma).  `rows` selects query rows.
    """
    q8 = seg["q8"][:, h, :]
    k8 = seg["k8"][:, h, :]
    Lq, Lk = q8.shape[0], k8.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    acc = q8[rows] @ k8.T
    sig = block_sigma(seg["q_scale"][h], seg["k_scale"][h], sm_scale_log2(sm_scale))
    sig_rows = sig[rows // seg.get("q_rows", BLOCK)]  # [nrows, nkblk]
    sig_full = np.repeat(sig_rows, BLOCK, axis=1)[:, :Lk]
    return acc, fl32(acc * sig_full)


# ----------------------------------------------------------------------------- softmax
def online_softmax_pv(S, vvals, quantize_p=True, epoch=EPOCH, checkpoints=None):
    """Online base-2 softmax over key epochs, accumulating RO = sum P8 V.

    S: [n, Lk] scores in log2 units; vvals: [Lk, D].  Returns (RO [n, D], d [n]).
    With quantize_p the probabilities enter the PV product as e4m3(448 P); without,
    as P itself (the "identity rounding" mode used by the pins).  If `checkpoints` is a
    list, one dict per epoch (m, d, alpha, p8 or p, RO) is appended to it.
    """
    n, Lk = S.shape
    m = np.full(n, -np.inf)
    d = np.zeros(n)
    RO = np.zeros((n, vvals.shape[1]))
    for e0 in range(0, Lk, epoch):
        Se = S[:, e0:e0 + epoch]
        m_new = np.maximum(m, np.max(Se, axis=1))
        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - m_new))
        P = np.exp2(Se - m_new[:, None])
        d = d * alpha + np.sum(P, axis=1)
        Pq = e4m3(448.0 * P) if quantize_p else P
        RO = RO * alpha[:, None] + Pq @ vvals[e0:e0 + epoch]
        m = m_new
        if checkpoints is not None:
            checkpoints.append(dict(m=m.copy(), d=d.copy(), alpha=alpha, p=Pq, RO=RO.copy()))
    return RO, d


def attention(quant, sm_scale, rows=None):
    """Quantized attention output for every segment and head.

    quant: the list returned by `quantize`.  Returns O as float64 BF16 values
    [sum Lq, H, D] (or, with `rows` = {segment index: row indices}, a dict
    {segment: [len(rows), H, D]}).  A segment with queries but no keys yields zeros.
    """
    outs = {}
    for si, seg in enumerate(quant):
        Lq, H, D = seg["q8"].shape
        r = np.arange(Lq) if rows is None else np.asarray(rows.get(si, []), dtype=np.int64)
        o = np.zeros((len(r), H, D))
        if len(r) and seg["k8"].shape[0]:
            for h in range(H):
                _, S = scores(seg, h, sm_scale, r)
                RO, d = online_softmax_pv(S, seg["v8val"][:, h, :])
                o[:, h, :] = bf16(RO / d[:, None] * seg["v_scale"][h][None, :] / 448.0)
        outs[si] = o
    if rows is not None:
        return outs
    return np.concatenate([outs[i] for i in range(len(quant))], axis=0)


def attention_identity(q, k, v, sm_scale, epoch=EPOCH):
    """The same online recurrence with every rounding removed (one segment, [L, H, D])."""
    Lq, H, D = q.shape
    o = np.zeros((Lq, H, D))
    for h in range(H):
        S = (q[:, h, :] @ k[:, h, :].T) * (sm_scale * LOG2E)
        RO, d = online_softmax_pv(S, v[:, h, :], quantize_p=False, epoch=epoch)
        o[:, h, :] = RO / d[:, None]
    return o


def softmax_attention_exact(q, k, v, sm_scale):
    """Textbook softmax(q k^T sm_scale) v in FP64 for one segment, [L, H, D]."""
    Lq, H, D = q.shape
    o = np.zeros((Lq, H, D))
    for h in range(H):
        z = (q[:, h, :] @ k[:, h, :].T) * sm_scale
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=1, keepdims=True)
        o[:, h, :] = w @ v[:, h, :]
    return o


def rel_l2(a, b):
    """||a - b|| / ||b|| over all elements."""
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def epochs(Lk):
    """Number of 64-key epochs the recurrence takes over Lk keys."""
    return math.ceil(Lk / EPOCH)
