"""The C-ABI library without a GPU: it loads, exports what include/sattn.h declares, and its
host-side validation returns the documented status before touching the device."""
import ctypes
import os
import re

import pytest

from quantized_attention_video_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")

# Never dereferenced: every call below fails validation before any HIP call.
FAKE = 0x10000
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"SATTN_API\s+[\w\s\*]+?\b(sattn_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert B.status_string(B.SATTN_OK) == "ok"
    assert B.status_string(B.SATTN_ENOSPACE) == "buffer or workspace too small"
    assert B.status_string(99) == "unknown status"


def test_quant_query_sizes():
    s = B.sattn_quant_query(1, 37810, 37810, 32)
    assert s.qblk_cap == 37810 // 64 + 1 == 591
    assert s.q_bytes == 32 * 591 * 8192 and s.q_scale_bytes == 32 * 591 * 2 * 4  # room for 32-row scales
    assert s.k_mean_bytes == 32 * 128 * 4 and s.v_bytes == s.k_bytes
    v = B.sattn_quant_query(4, 47638, 47638, 24)
    assert v.kblk_cap == 47638 // 64 + 4
    assert v.fwd_workspace_bytes >= 4 * 4 + 5 * 4
    with pytest.raises(B.SattnError) as e:
        B.sattn_quant_query(0, 10, 10, 1)
    assert e.value.status == B.SATTN_EINVAL
    with pytest.raises(B.SattnError) as e:
        B.sattn_quant_query(1, 10, 10, 1, 64)
    assert e.value.status == B.SATTN_EUNSUPPORTED


def test_capacity_bound_covers_every_segment_layout():
    # blocks of segment s start at cu[s]//64 + s; the last one must end inside the capacity
    import random
    rng = random.Random(5)
    for _ in range(2000):
        lens = [rng.choice([0, 1, 63, 64, 65, rng.randint(0, 5000)]) for _ in range(rng.randint(1, 12))]
        cu = [0]
        for n in lens:
            cu.append(cu[-1] + n)
        cap = cu[-1] // 64 + len(lens)
        ends = [cu[s] // 64 + s + -(-lens[s] // 64) for s in range(len(lens))]
        starts = [cu[s] // 64 + s for s in range(len(lens))]
        assert max(ends) <= cap
        assert all(ends[s] <= starts[s + 1] for s in range(len(lens) - 1))


def _quant_struct(cap=100, ptr=FAKE, rows=64):
    return B.QKVQuant(ptr, ptr, ptr, ptr, ptr, ptr, ptr, cap, cap, rows)


def _in(ptr=FAKE, sb=0, st=128, sh=128):
    return B.BF16In(ptr, sb, st, sh)


def _out(ptr=FAKE, sb=0, st=128, sh=128):
    return B.BF16Out(ptr, sb, st, sh)


def test_quantize_validation():
    L = B.lib()
    q = _quant_struct()

    def call(qv=_in(), kv=_in(), vv=_in(), nseg=1, H=1, D=128, Lq=64, Lk=64, cuq=None, cuk=None, out=q, ws=FAKE,
             wsb=1 << 20):
        return L.sattn_quantize_qkv(qv, kv, vv, nseg, H, D, Lq, Lk, cuq, cuk, ctypes.byref(out) if out else None,
                                    ws, wsb, None)

    assert call(D=64) == B.SATTN_EUNSUPPORTED
    assert call(nseg=0) == B.SATTN_EINVAL
    assert call(Lq=-1) == B.SATTN_EINVAL
    assert call(qv=_in(ptr=0)) == B.SATTN_EINVAL
    assert call(kv=_in(ptr=MISALIGNED)) == B.SATTN_EINVAL
    assert call(vv=_in(st=100)) == B.SATTN_EINVAL  # token stride not a multiple of 8
    assert call(cuq=FAKE) == B.SATTN_EINVAL  # only one of the two cu_seqlens
    assert call(out=None) == B.SATTN_EINVAL
    assert call(ws=None) == B.SATTN_EINVAL
    assert call(out=_quant_struct(cap=1)) == B.SATTN_ENOSPACE
    assert call(wsb=16) == B.SATTN_ENOSPACE
    for rows in (1, 16, 48, 128, -32):
        assert call(out=_quant_struct(rows=rows)) == B.SATTN_EINVAL
    # statistics blocks (one per segment-head here) plus Q blocks beyond a 1-D grid of 2^32 - 1
    big = dict(nseg=65535, H=65535, Lq=1, Lk=1, out=_quant_struct(cap=1 << 40), wsb=1 << 62)
    assert call(**big) == B.SATTN_EUNSUPPORTED


def test_fwd_validation():
    L = B.lib()
    q = _quant_struct()
    f = L.sattn_fwd
    assert f(ctypes.byref(q), 1, 1, 64, 64, 64, 0.1, _out(), None, 0, None) == B.SATTN_EUNSUPPORTED
    assert f(ctypes.byref(q), 0, 1, 64, 64, 128, 0.1, _out(), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(q), 1, 1, 64, 64, 128, 0.0, _out(), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(q), 1, 1, 64, 64, 128, float("nan"), _out(), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(q), 1, 1, 64, 64, 128, 0.1, _out(ptr=MISALIGNED), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(q), 1, 1, 64, 64, 128, 0.1, _out(st=4), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(_quant_struct(cap=0)), 2, 1, 64, 64, 128, 0.1, _out(), None, 0, None) == B.SATTN_ENOSPACE
    assert f(None, 1, 1, 64, 64, 128, 0.1, _out(), None, 0, None) == B.SATTN_EINVAL
    assert f(ctypes.byref(_quant_struct(rows=16)), 1, 1, 64, 64, 128, 0.1, _out(), None, 0, None) == B.SATTN_EINVAL
    # 2^31 - 1 queries of 8 heads: 1.3e8 workgroups, beyond one dispatch's 32-bit work-item count
    assert f(ctypes.byref(_quant_struct(cap=1 << 40)), 1, 8, (1 << 31) - 1, 64, 128, 0.1, _out(), None, 0, None) \
        == B.SATTN_EUNSUPPORTED
    assert f(ctypes.byref(q), 1, 1, 64, 64, 128, 0.1, _out(), MISALIGNED, 1 << 20, None) == B.SATTN_EINVAL
    v = L.sattn_fwd_varlen
    assert v(ctypes.byref(q), FAKE, FAKE, 2, 100, 100, 1, 128, 0.1, _out(), FAKE, 4, None) == B.SATTN_ENOSPACE
    assert v(ctypes.byref(q), None, FAKE, 2, 100, 100, 1, 128, 0.1, _out(), FAKE, 1024, None) == B.SATTN_EINVAL
    assert v(ctypes.byref(q), FAKE, FAKE, 2, 100, 100, 1, 128, 0.1, _out(), None, 1024, None) == B.SATTN_EINVAL
    assert v(ctypes.byref(q), FAKE, FAKE, 2, 100, -1, 1, 128, 0.1, _out(), FAKE, 1024, None) == B.SATTN_EINVAL
    g = L.sattn_fwd_fused  # (kv, q, cu_q, cu_k, nseg, H, Lq, Lk, D, sm_scale, o, workspace, bytes, stream)
    assert g(ctypes.byref(q), _in(), None, None, 1, 1, 64, 64, 64, 0.1, _out(), None, 0, None) == B.SATTN_EUNSUPPORTED
    assert g(ctypes.byref(q), _in(ptr=MISALIGNED), None, None, 1, 1, 64, 64, 128, 0.1, _out(), None, 0, None) \
        == B.SATTN_EINVAL
    # dense: the workspace is optional (the key split) but must be aligned; packed: required
    assert g(ctypes.byref(q), _in(), None, None, 1, 1, 64, 64, 128, 0.1, _out(), MISALIGNED, 1 << 20, None) \
        == B.SATTN_EINVAL
    assert g(ctypes.byref(q), _in(), FAKE, FAKE, 2, 1, 100, 100, 128, 0.1, _out(), None, 1024, None) == B.SATTN_EINVAL
    assert g(ctypes.byref(q), _in(), FAKE, FAKE, 2, 1, 100, 100, 128, 0.1, _out(), FAKE, 4, None) == B.SATTN_ENOSPACE


def test_noalloc_validation():
    """The allocation-free quantizer validates like the workspace form, and rejects a problem
    whose workspace exceeds its scratch array before any device call."""
    L = B.lib()
    assert L.sattn_noalloc_scratch_bytes() == 16 << 20
    f = L.sattn_quantize_qkv_noalloc

    def call(nseg=1, H=1, Lq=64, Lk=64, cu=None, out=None, D=128):
        out = _quant_struct() if out is None else out
        return f(_in(), _in(), _in(), nseg, H, D, Lq, Lk, cu, cu, ctypes.byref(out), None)

    assert call(D=64) == B.SATTN_EUNSUPPORTED
    assert call(nseg=0) == B.SATTN_EINVAL
    assert call(Lk=-1) == B.SATTN_EINVAL
    assert call(out=_quant_struct(rows=16)) == B.SATTN_EINVAL
    assert call(out=_quant_struct(cap=1)) == B.SATTN_ENOSPACE
    n = 9000  # segment-heads whose statistics (2 KiB each) exceed the 16 MiB array
    assert call(nseg=n, Lq=n, Lk=n, cu=FAKE, out=_quant_struct(cap=1 << 20)) == B.SATTN_ENOSPACE
    s = B.sattn_quant_query(n, n, n, 1)
    assert s.quant_workspace_bytes > L.sattn_noalloc_scratch_bytes()


def _ck(**kw):
    c = dict(acc=FAKE, s=FAKE, ld=64, m=None, d=None, alpha=None, p8=None, ro=None, nep=0, rcp=None)
    c.update(kw)
    return B.Checkpoints(*(c[n] for n, _ in B.Checkpoints._fields_))


def test_debug_scores_validation():
    """Row range, step, segment/head indices and checkpoint buffers are checked before any
    launch (dense and packed forms)."""
    L = B.lib()
    q = _quant_struct()
    d = L.sattn_debug_scores

    def call(cu=None, nseg=1, Lq=64, Lk=64, H=1, D=128, seg=0, head=0, q0=0, q1=64, step=1, ck=None, out=None):
        ck = _ck() if ck is None else ck
        return d(ctypes.byref(q), cu, cu, nseg, Lq, Lk, H, D, 0.1, seg, head, q0, q1, step, ctypes.byref(ck),
                 out or _out(), None)

    assert call(D=64) == B.SATTN_EUNSUPPORTED
    assert call(seg=1) == B.SATTN_EINVAL
    assert call(seg=-1) == B.SATTN_EINVAL
    assert call(head=1) == B.SATTN_EINVAL
    assert call(q0=-1) == B.SATTN_EINVAL
    assert call(q0=10, q1=10) == B.SATTN_EINVAL
    assert call(step=0) == B.SATTN_EINVAL
    assert call(ck=_ck(ld=0)) == B.SATTN_EINVAL            # scores asked for without a row length
    assert call(ck=_ck(m=FAKE, nep=0)) == B.SATTN_EINVAL   # per-epoch buffer without epochs
    assert call(ck=_ck(p8=FAKE, nep=0)) == B.SATTN_EINVAL
    assert call(ck=_ck(ro=FAKE, nep=-1)) == B.SATTN_EINVAL
    assert call(out=_out(ptr=MISALIGNED)) == B.SATTN_EINVAL
    assert d(ctypes.byref(q), None, None, 1, 64, 64, 1, 128, 0.1, 0, 0, 0, 64, 1, None, _out(), None) \
        == B.SATTN_EINVAL
    assert d(ctypes.byref(q), FAKE, None, 1, 64, 64, 1, 128, 0.1, 0, 0, 0, 64, 1, ctypes.byref(_ck()), _out(),
             None) == B.SATTN_EINVAL  # one cu_seqlens pointer without the other
    assert call(nseg=2, Lq=64, Lk=64 * 1000) == B.SATTN_ENOSPACE  # capacity of the quantized K buffers


def test_untile_layouts_are_permutations():
    import numpy as np
    idx = np.arange(8192).reshape(1, 8192)
    a = B.untile_qk(idx)
    b = B.untile_v(idx)
    assert sorted(a.ravel().tolist()) == list(range(8192)) == sorted(b.ravel().tolist())
    # spot-check the documented byte formulas
    t, u, g, i, s = 1, 2, 1, 5, 7
    assert a[32 * t + i, 64 * g + 16 * u + s] == ((t * 4 + u) * 64 + g * 32 + i) * 16 + s
    w, f, g, i, s = 3, 1, 0, 9, 13
    assert b[32 * f + 8 * (s // 4) + 4 * g + s % 4, 32 * w + i] == ((w * 2 + f) * 64 + g * 32 + i) * 16 + s
