"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case replaces one piece of oracle/sattn.py (or a codec it uses) with a plausible wrong
version — a dropped term, a wrong sign, a transposed operand, a wrong block size or axis,
a missing factor — and runs the pins of tests/test_oracle_pins.py that should notice.  At
least one of them has to fail; if all pass, the pins have a blind spot for that mistake.
The mutants live only in this file and only while a case runs (monkeypatch).
"""
import numpy as np
import pytest

import test_oracle_pins as P
from oracle import sattn as O
from oracle.codecs import e4m3, fl32


def _softmax_variant(d_no_alpha=False, alpha_inverted=False, old_max=False, ro_no_alpha=False, pad=False,
                     epoch_override=None, scale_after_e4m3=False, d_from_p8=False):
    """The oracle's online recurrence with one deliberate error switched on."""

    def f(S, vvals, quantize_p=True, epoch=None, checkpoints=None):
        epoch = epoch_override or epoch or O.EPOCH
        if pad and S.shape[1] % epoch:
            extra = epoch - S.shape[1] % epoch
            S = np.concatenate([S, np.zeros((S.shape[0], extra))], axis=1)
            vvals = np.concatenate([vvals, np.zeros((extra, vvals.shape[1]))], axis=0)
        n, Lk = S.shape
        m = np.full(n, -np.inf)
        d = np.zeros(n)
        RO = np.zeros((n, vvals.shape[1]))
        for e0 in range(0, Lk, epoch):
            Se = S[:, e0:e0 + epoch]
            m_new = np.maximum(m, np.max(Se, axis=1))
            first = np.isneginf(m)
            alpha = np.where(first, 0.0, np.exp2((m_new - m) if alpha_inverted else (m - m_new)))
            ref = np.where(first, m_new, m) if old_max else m_new
            Pe = np.exp2(Se - ref[:, None])
            if scale_after_e4m3:  # quantized on [0, 1] (subnormals from 2^-6 down), then scaled
                Pq = 448.0 * e4m3(Pe) if quantize_p else Pe
            else:
                Pq = e4m3(448.0 * Pe) if quantize_p else Pe
            psum = np.sum(Pq, axis=1) / 448.0 if (d_from_p8 and quantize_p) else np.sum(Pe, axis=1)
            d = (d + psum) if d_no_alpha else (d * alpha + psum)
            RO = (RO + Pq @ vvals[e0:e0 + epoch]) if ro_no_alpha else (RO * alpha[:, None] + Pq @ vvals[e0:e0 + epoch])
            m = m_new
            if checkpoints is not None:
                checkpoints.append(dict(m=m.copy(), d=d.copy(), alpha=alpha, p=Pq, RO=RO.copy()))
        return RO, d

    return f


def _quantize_v_per_head(v):
    L, H, D = v.shape
    amax = np.max(np.abs(v), axis=(0, 2))[:, None] * np.ones((1, D))  # one scale per head
    safe = np.where(amax > 0, amax, 1.0)
    inv = np.where(amax > 0, fl32(448.0 / safe), 0.0)
    vals = e4m3(fl32(v * inv[None]))
    from oracle.codecs import e4m3_encode
    return e4m3_encode(vals), vals, np.where(amax > 0, fl32(safe / 448.0), 0.0)


def _k_smooth_per_token(k):
    mean = fl32(np.mean(k, axis=2))  # over channels instead of tokens
    return mean, fl32(k - mean[:, :, None])


def _quantize_v_per_token(v):
    L, H, D = v.shape
    amax = np.max(np.abs(v), axis=2, keepdims=True)  # per token instead of per channel
    safe = np.where(amax > 0, amax, 1.0)
    inv = np.where(amax > 0, fl32(448.0 / safe), 0.0)
    vals = e4m3(fl32(v * inv))
    scale = np.where(amax[0] > 0, fl32(safe[0] / 448.0), 0.0) * np.ones((H, D))
    from oracle.codecs import e4m3_encode
    return e4m3_encode(vals), vals, scale


def _scores_q_k_swapped(seg, h, sm_scale, rows=None):
    q8, k8 = seg["q8"][:, h, :], seg["k8"][:, h, :]
    rows = np.arange(q8.shape[0]) if rows is None else np.asarray(rows)
    acc = k8[rows] @ q8.T  # the roles of Q and K exchanged
    sig = O.block_sigma(seg["q_scale"][h], seg["k_scale"][h], O.sm_scale_log2(sm_scale))
    sig_full = np.repeat(sig[rows // O.BLOCK], O.BLOCK, axis=1)[:, :k8.shape[0]]
    return acc, fl32(acc * sig_full)


def _block_sigma_without_k(q_scale_h, k_scale_h, c32):
    a = fl32(q_scale_h * c32)
    return fl32(a[:, None] * np.ones_like(k_scale_h)[None, :])


def _attention_variant(drop_448=False, drop_v_scale=False):
    real = O.attention

    def f(quant, sm_scale, rows=None):
        out = real(quant, sm_scale, rows)
        # undo the oracle's own epilogue factor and re-apply a wrong one
        if rows is not None:
            return out
        o = np.zeros_like(out)
        base = 0
        for seg in quant:
            Lq, H, D = seg["q8"].shape
            for h in range(H):
                if seg["k8"].shape[0] == 0:
                    continue
                _, S = O.scores(seg, h, sm_scale)
                RO, d = O.online_softmax_pv(S, seg["v8val"][:, h, :])
                vs = np.ones(D) if drop_v_scale else seg["v_scale"][h]
                div = 1.0 if drop_448 else 448.0
                o[base:base + Lq, h, :] = P.bf16(RO / d[:, None] * vs[None, :] / div)
            base += Lq
        return o

    return f


def _rne_half_away(x):
    return np.where(np.asarray(x) >= 0, np.floor(np.asarray(x) + 0.5), np.ceil(np.asarray(x) - 0.5))


def _e4m3_three_bits(x):
    from oracle.codecs import _round_to_bits
    x = np.asarray(x, dtype=np.float64)
    return np.clip(_round_to_bits(x, 3, -9), -448.0, 448.0)


def _scores_ignoring_q_rows(seg, h, sm_scale, rows=None):
    q8, k8 = seg["q8"][:, h, :], seg["k8"][:, h, :]
    rows = np.arange(q8.shape[0]) if rows is None else np.asarray(rows)
    acc = q8[rows] @ k8.T
    sig = O.block_sigma(seg["q_scale"][h], seg["k_scale"][h], O.sm_scale_log2(sm_scale))
    sig_full = np.repeat(sig[np.minimum(rows // O.BLOCK, sig.shape[0] - 1)], O.BLOCK, axis=1)[:, :k8.shape[0]]
    return acc, fl32(acc * sig_full)


def _quantize_ignoring_q_rows(q, k, v, cu_q, cu_k, q_rows=None):
    out = _REAL_QUANTIZE(q, k, v, cu_q, cu_k)
    for seg in out:
        seg["q_rows"] = q_rows or O.BLOCK
        if q_rows == 32:  # one 64-row scale reported twice
            seg["q_scale"] = np.repeat(seg["q_scale"], 2, axis=1)[:, :-(-seg["q8"].shape[0] // 32)]
    return out


_REAL_QUANTIZE = O.quantize

PINS_ATTN = [
    lambda: P.test_identity_rounding_equals_textbook_softmax(64),
    lambda: P.test_identity_rounding_equals_textbook_softmax(7),
    P.test_online_denominator_normalises_probabilities,
    P.test_grid_exact_case_equals_brute_force,
    P.test_zero_queries_give_the_mean_of_v,
    P.test_single_key_returns_its_value,
    P.test_quantized_program_tracks_exact_attention,
]
PINS_QUANT = [
    P.test_k_mean_shift_leaves_codes_and_scores_unchanged,
    P.test_k_mean_is_subtracted_per_channel_not_per_token,
    P.test_int8_block_scale_and_ties,
    P.test_int8_blocks_are_per_64_tokens_and_partial_tail,
    P.test_zero_blocks_and_channels,
    P.test_v_channel_scale_exact_case,
    P.test_grid_exact_case_equals_brute_force,
    P.test_quantized_program_tracks_exact_attention,
    P.test_pages_shape_facts,
]

PINS_Q32 = [
    P.test_q32_scales_are_per_32_rows_and_partial_tail,
    P.test_q32_doubling_one_half_doubles_only_its_scores,
    P.test_q32_equals_q64_when_halves_share_their_amax,
    P.test_q32_program_tracks_exact_attention,
]

MUTANTS = {
    "denominator not rescaled": (lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(d_no_alpha=True)),
                                 PINS_ATTN),
    "rescale factor inverted": (lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(alpha_inverted=True)),
                                PINS_ATTN),
    "probabilities against the old max": (lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(old_max=True)),
                                          PINS_ATTN),
    "output not rescaled": (lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(ro_no_alpha=True)),
                            PINS_ATTN),
    "partial epoch padded with zero scores": (lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(pad=True)),
                                              PINS_ATTN),
    "P quantized before the 448 scaling": (
        lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(scale_after_e4m3=True)), PINS_ATTN),
    "denominator summed from the quantized probabilities": (
        lambda mp: mp.setattr(O, "online_softmax_pv", _softmax_variant(d_from_p8=True)), PINS_ATTN),
    "epoch of 32 keys": (lambda mp: (mp.setattr(O, "EPOCH", 32),
                                     mp.setattr(O, "online_softmax_pv", _softmax_variant(epoch_override=32))),
                         PINS_ATTN + [P.test_pages_shape_facts]),
    "K mean over channels": (lambda mp: mp.setattr(O, "k_smooth", _k_smooth_per_token), PINS_QUANT),
    "Q/K blocks of 32 tokens": (lambda mp: mp.setattr(O, "BLOCK", 32), PINS_QUANT),
    "INT8 ties away from zero": (lambda mp: mp.setattr(O, "rne", _rne_half_away), PINS_QUANT),
    "V scaled per token": (lambda mp: mp.setattr(O, "quantize_v", _quantize_v_per_token), PINS_QUANT),
    "V scaled per head instead of per channel": (lambda mp: mp.setattr(O, "quantize_v", _quantize_v_per_head),
                                                 PINS_QUANT),
    "Q and K exchanged in the scores": (lambda mp: mp.setattr(O, "scores", _scores_q_k_swapped), PINS_ATTN),
    "score scale without k_scale": (lambda mp: mp.setattr(O, "block_sigma", _block_sigma_without_k), PINS_ATTN),
    "softmax scale without log2 e": (lambda mp: mp.setattr(O, "sm_scale_log2", lambda s: float(fl32(np.float32(s)))),
                                     PINS_ATTN),
    "epilogue without the 1/448": (lambda mp: mp.setattr(O, "attention", _attention_variant(drop_448=True)), PINS_ATTN),
    "epilogue without v_scale": (lambda mp: mp.setattr(O, "attention", _attention_variant(drop_v_scale=True)),
                                 PINS_ATTN),
    "E4M3 with three significant bits": (lambda mp: mp.setattr(O, "e4m3", _e4m3_three_bits), PINS_ATTN + PINS_QUANT),
    "32-row Q scales read with the 64-row block index": (lambda mp: mp.setattr(O, "scores", _scores_ignoring_q_rows),
                                                          PINS_Q32),
    "32-row Q scales computed over 64 rows": (lambda mp: mp.setattr(O, "quantize", _quantize_ignoring_q_rows),
                                             PINS_Q32),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    patch, pins = MUTANTS[name]
    patch(monkeypatch)
    caught = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin fails when the oracle has this mistake: {name}"
