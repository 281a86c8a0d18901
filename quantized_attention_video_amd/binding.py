"""ctypes binding of libsattn.so (include/sattn.h) — argument marshalling only.

Every function here has the name of the C entry point it wraps.  torch tensors supply
device memory and the current HIP stream; all computation happens in the library's
kernels.  If the library has not been built the calls raise; there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsattn.so")
D = 128

SATTN_OK, SATTN_EINVAL, SATTN_EUNSUPPORTED, SATTN_ENOSPACE, SATTN_EHIP = range(5)
EXPORTED = ("sattn_quant_query", "sattn_quantize_qkv", "sattn_fwd", "sattn_fwd_varlen", "sattn_debug_scores",
            "sattn_fwd_fused", "sattn_quantize_qkv_noalloc", "sattn_noalloc_scratch_bytes", "sattn_status_string")


class SattnError(RuntimeError):
    def __init__(self, status, name):
        super().__init__(f"{name} failed: {status_string(status)} (status {status})")
        self.status = status


class BF16In(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class BF16Out(ctypes.Structure):
    _fields_ = BF16In._fields_


class QKVQuant(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_mean", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("qblk_cap", ctypes.c_int64), ("kblk_cap", ctypes.c_int64),
                ("q_scale_rows", ctypes.c_int32)]


class Checkpoints(ctypes.Structure):
    _fields_ = [("acc", ctypes.c_void_p), ("s", ctypes.c_void_p), ("ld", ctypes.c_int64), ("m", ctypes.c_void_p),
                ("d", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("p8", ctypes.c_void_p), ("ro", ctypes.c_void_p),
                ("nep", ctypes.c_int64), ("rcp", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("qblk_cap", ctypes.c_int64), ("kblk_cap", ctypes.c_int64), ("q_bytes", ctypes.c_size_t),
                ("q_scale_bytes", ctypes.c_size_t), ("k_bytes", ctypes.c_size_t),
                ("k_scale_bytes", ctypes.c_size_t), ("k_mean_bytes", ctypes.c_size_t),
                ("v_bytes", ctypes.c_size_t), ("v_scale_bytes", ctypes.c_size_t),
                ("quant_workspace_bytes", ctypes.c_size_t), ("fwd_workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_attention_video_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.sattn_quant_query.argtypes = [i32, i64, i64, i32, i32, ctypes.POINTER(Sizes)]
        L.sattn_quantize_qkv.argtypes = [BF16In, BF16In, BF16In, i32, i32, i32, i64, i64, vp, vp,
                                         ctypes.POINTER(QKVQuant), vp, ctypes.c_size_t, vp]
        L.sattn_fwd.argtypes = [ctypes.POINTER(QKVQuant), i32, i32, i32, i32, i32, f32, BF16Out, vp, ctypes.c_size_t,
                                vp]
        L.sattn_fwd_varlen.argtypes = [ctypes.POINTER(QKVQuant), vp, vp, i32, i64, i64, i32, i32, f32, BF16Out, vp,
                                       ctypes.c_size_t, vp]
        L.sattn_debug_scores.argtypes = [ctypes.POINTER(QKVQuant), vp, vp, i32, i64, i64, i32, i32, f32, i32, i32, i64,
                                         i64, i64, ctypes.POINTER(Checkpoints), BF16Out, vp]
        L.sattn_fwd_fused.argtypes = [ctypes.POINTER(QKVQuant), BF16In, vp, vp, i32, i32, i64, i64, i32, f32,
                                      BF16Out, vp, ctypes.c_size_t, vp]
        L.sattn_quantize_qkv_noalloc.argtypes = [BF16In, BF16In, BF16In, i32, i32, i32, i64, i64, vp, vp,
                                                 ctypes.POINTER(QKVQuant), vp]
        L.sattn_noalloc_scratch_bytes.argtypes = []
        L.sattn_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.sattn_status_string.argtypes = [i32]
        L.sattn_status_string.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name not in ("sattn_status_string", "sattn_noalloc_scratch_bytes"):
                getattr(L, name).restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(status):
    return lib().sattn_status_string(int(status)).decode()


def _check(status, name):
    if status != SATTN_OK:
        raise SattnError(status, name)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _view(t, cls):
    """A [B, L, H, D] or [T, H, D] BF16 tensor view → its C struct (strides in elements)."""
    if t.dtype != torch.bfloat16 or t.shape[-1] != D or t.stride(-1) != 1:
        raise ValueError("expected a bfloat16 view with a contiguous last dimension of 128")
    if t.dim() == 4:
        return cls(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))
    if t.dim() == 3:
        return cls(t.data_ptr(), 0, t.stride(0), t.stride(1))
    raise ValueError("expected a 3-d [T, H, D] or 4-d [B, L, H, D] view")


def sattn_quant_query(nseg, total_q, total_k, H, D_=D):
    s = Sizes()
    _check(lib().sattn_quant_query(nseg, total_q, total_k, H, D_, ctypes.byref(s)), "sattn_quant_query")
    return s


@dataclass
class Quantized:
    """Device buffers of sattn_qkv_quant plus the quantization workspace."""
    q: torch.Tensor
    q_scale: torch.Tensor
    k: torch.Tensor
    k_scale: torch.Tensor
    k_mean: torch.Tensor
    v: torch.Tensor
    v_scale: torch.Tensor
    workspace: torch.Tensor
    qblk_cap: int
    kblk_cap: int
    nseg: int
    H: int
    sizes: Sizes
    q_scale_rows: int = 64  # query rows per Q scale: 64 or 32 (q_scale is [H, qblk_cap * 64 / rows])
    total_q: int = 0  # query and key tokens the buffers were sized for (packed: the views' lengths)
    total_k: int = 0

    def struct(self):
        return QKVQuant(_ptr(self.q), _ptr(self.q_scale), self.k.data_ptr(), self.k_scale.data_ptr(),
                        self.k_mean.data_ptr(), self.v.data_ptr(), self.v_scale.data_ptr(), self.qblk_cap,
                        self.kblk_cap, self.q_scale_rows)


def alloc_quantized(nseg, total_q, total_k, H, device="cuda", q_scale_rows=64, with_q=True):
    """Allocate (uninitialised) quantized buffers sized by sattn_quant_query.  with_q=False
    leaves out the INT8 Q buffers (K/V only, for sattn_fwd_fused)."""
    if q_scale_rows not in (32, 64):
        raise ValueError("q_scale_rows must be 32 or 64")
    s = sattn_quant_query(nseg, total_q, total_k, H)
    e = dict(device=device)
    return Quantized(
        q=torch.empty((H, s.qblk_cap, 8192), dtype=torch.int8, **e) if with_q else None,
        q_scale=torch.empty((H, s.qblk_cap * (64 // q_scale_rows)), dtype=torch.float32, **e) if with_q else None,
        k=torch.empty((H, s.kblk_cap, 8192), dtype=torch.int8, **e),
        k_scale=torch.empty((H, s.kblk_cap), dtype=torch.float32, **e),
        k_mean=torch.empty((nseg, H, D), dtype=torch.float32, **e),
        v=torch.empty((H, s.kblk_cap, 8192), dtype=torch.uint8, **e),
        v_scale=torch.empty((nseg, H, D), dtype=torch.float32, **e),
        workspace=torch.empty(max(s.quant_workspace_bytes, 16), dtype=torch.uint8, **e),
        qblk_cap=s.qblk_cap, kblk_cap=s.kblk_cap, nseg=nseg, H=H, sizes=s, q_scale_rows=q_scale_rows,
        total_q=total_q, total_k=total_k)


def sattn_quantize_qkv(q, k, v, cu_seqlens_q=None, cu_seqlens_k=None, out=None, stream=None, q_scale_rows=64):
    """Quantize BF16 Q/K/V views.  Dense: [B, L, H, D] views.  Varlen: packed [T, H, D]
    views plus device int32 cu_seqlens tensors of nseg+1 entries.  q_scale_rows: 64 (one
    Q scale per 64-token block) or 32 (one per 32 query rows); ignored when `out` is given
    (its own q_scale_rows applies)."""
    varlen = cu_seqlens_q is not None
    if varlen:
        nseg = cu_seqlens_q.numel() - 1
        H = q.shape[1]
        Lq, Lk = q.shape[0], k.shape[0]
        total_q, total_k = Lq, Lk
    else:
        nseg, Lq, H = q.shape[0], q.shape[1], q.shape[2]
        Lk = k.shape[1]
        total_q, total_k = nseg * Lq, nseg * Lk
    if out is None:
        with torch.cuda.stream(stream or torch.cuda.current_stream()):  # allocated on the stream that uses it
            out = alloc_quantized(nseg, total_q, total_k, H, device=q.device, q_scale_rows=q_scale_rows)
    st = out.struct()
    qv = _view(q, BF16In) if out.q is not None else BF16In(0, 0, 0, 0)
    _check(lib().sattn_quantize_qkv(qv, _view(k, BF16In), _view(v, BF16In), nseg, H, D, Lq, Lk,
                                    _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), ctypes.byref(st),
                                    out.workspace.data_ptr(), out.workspace.numel(), _stream(stream)),
           "sattn_quantize_qkv")
    return out


def _on(stream):
    """Allocate temporaries on the stream the library call runs on (the caching allocator
    then never hands their memory to other work while that stream still uses it)."""
    return torch.cuda.stream(stream or torch.cuda.current_stream())


def sattn_quantize_qkv_noalloc(q, k, v, out, cu_seqlens_q=None, cu_seqlens_k=None, stream=None):
    """sattn_quantize_qkv into caller-allocated buffers `out` (from alloc_quantized), with the
    library's per-device scratch array as its workspace: the call itself allocates nothing."""
    varlen = cu_seqlens_q is not None
    if varlen:
        nseg, H, Lq, Lk = cu_seqlens_q.numel() - 1, q.shape[1], q.shape[0], k.shape[0]
    else:
        nseg, Lq, H, Lk = q.shape[0], q.shape[1], q.shape[2], k.shape[1]
    st = out.struct()
    qv = _view(q, BF16In) if out.q is not None else BF16In(0, 0, 0, 0)
    _check(lib().sattn_quantize_qkv_noalloc(qv, _view(k, BF16In), _view(v, BF16In), nseg, H, D, Lq, Lk,
                                            _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), ctypes.byref(st),
                                            _stream(stream)), "sattn_quantize_qkv_noalloc")
    return out


def sattn_noalloc_scratch_bytes():
    return int(lib().sattn_noalloc_scratch_bytes())


def sattn_fwd(quant, B, H, Lq, Lk, sm_scale, out=None, stream=None, workspace=None):
    """Dense forward; returns (or fills) a BF16 [B, Lq, H, D] tensor (any strided view works).
    workspace: a zero-filled uint8 device tensor of fwd_workspace_bytes (split_workspace())
    lets problems too small to fill the GPU split their keys between two workgroups."""
    if out is None:
        with _on(stream):
            out = torch.empty((B, Lq, H, D), dtype=torch.bfloat16, device=quant.q.device)
    st = quant.struct()
    ws, wsb = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib().sattn_fwd(ctypes.byref(st), B, H, Lq, Lk, D, float(sm_scale), _view(out, BF16Out), ws, wsb,
                           _stream(stream)), "sattn_fwd")
    return out


def split_workspace(B, H, Lq, Lk, device="cuda"):
    """Zero-filled forward workspace for sattn_fwd's key split (kept zeroed by every call)."""
    s = sattn_quant_query(B, B * Lq, B * Lk, H)
    return torch.zeros(max(s.fwd_workspace_bytes, 16), dtype=torch.uint8, device=device)


def sattn_quantize_kv(q, k, v, cu_seqlens_q=None, cu_seqlens_k=None, stream=None, q_scale_rows=64):
    """K/V-only preparation for sattn_fwd_fused (Q buffers absent; the q view only gives
    the problem's query geometry and is not read)."""
    varlen = cu_seqlens_q is not None
    if varlen:
        nseg, H = cu_seqlens_q.numel() - 1, q.shape[1]
        total_q, total_k = q.shape[0], k.shape[0]
    else:
        nseg, H = q.shape[0], q.shape[2]
        total_q, total_k = nseg * q.shape[1], nseg * k.shape[1]
    with _on(stream):
        out = alloc_quantized(nseg, total_q, total_k, H, device=k.device, q_scale_rows=q_scale_rows, with_q=False)
    return sattn_quantize_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k, out=out, stream=stream)


def sattn_fwd_fused(kv, q, sm_scale, cu_seqlens_q=None, cu_seqlens_k=None, Lk=None, out=None, workspace=None,
                    stream=None):
    """Forward with the Q preparation in the attention launch.  Dense: q is a [B, Lq, H, D]
    view and Lk the keys per segment (an optional zero-filled `workspace`, see
    split_workspace, enables the key split of small grids as in sattn_fwd); varlen: q is
    packed [T, H, D] and Lk the packed key tokens.  Returns (or fills) the BF16 output
    shaped like q."""
    if Lk is None:
        raise ValueError("Lk (keys per segment, or packed key tokens) is required")
    varlen = cu_seqlens_q is not None
    if varlen:
        nseg, Lq, H = cu_seqlens_q.numel() - 1, q.shape[0], q.shape[1]
        if workspace is None:
            with _on(stream):
                workspace = fwd_workspace(nseg, device=q.device)
        ws, wsb = workspace.data_ptr(), workspace.numel()
    else:
        nseg, Lq, H = q.shape[0], q.shape[1], q.shape[2]
        ws, wsb = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    if out is None:
        with _on(stream):
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    st = kv.struct()
    _check(lib().sattn_fwd_fused(ctypes.byref(st), _view(q, BF16In), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseg, H,
                                 Lq, Lk, D, float(sm_scale), _view(out, BF16Out), ws, wsb, _stream(stream)),
           "sattn_fwd_fused")
    return out


def fwd_workspace(nseg, device="cuda"):
    s = sattn_quant_query(nseg, 0, 0, 1)
    return torch.empty(s.fwd_workspace_bytes, dtype=torch.uint8, device=device)


def sattn_fwd_varlen(quant, cu_seqlens_q, cu_seqlens_k, total_q, sm_scale, out=None, workspace=None, stream=None,
                     total_k=None):
    """Packed forward; returns (or fills) a BF16 [total_q, H, D] tensor.  total_k (the packed
    key tokens the K/V views held) defaults to what `quant` was sized for."""
    nseg = cu_seqlens_q.numel() - 1
    H = quant.H
    total_k = quant.total_k if total_k is None else total_k
    with _on(stream):
        if out is None:
            out = torch.empty((total_q, H, D), dtype=torch.bfloat16, device=quant.k.device)
        if workspace is None:
            workspace = fwd_workspace(nseg, device=quant.k.device)
    st = quant.struct()
    _check(lib().sattn_fwd_varlen(ctypes.byref(st), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseg, total_q, total_k, H,
                                  D, float(sm_scale), _view(out, BF16Out), workspace.data_ptr(), workspace.numel(),
                                  _stream(stream)), "sattn_fwd_varlen")
    return out


def sattn_debug_scores(quant, sm_scale, seg, head, q_begin, q_end, q_step=1, Lq=None, Lk=None, ld=None, nep=0,
                       cu_seqlens_q=None, cu_seqlens_k=None, out=None, scores=True, stream=None):
    """Checkpoints of the sampled query rows q_begin, q_begin + q_step, ... < q_end of one
    (segment, head).  Dense problems: Lq, Lk are the per-segment lengths (the segments are
    quant.nseg); packed: cu_seqlens tensors, and Lq, Lk the packed totals (default: what
    `quant` was sized for).  ld: keys per dumped score row (default Lk); nep: epochs of
    per-epoch checkpoints (0: none).  Returns a dict of device tensors: acc and s
    ([rows, ld], with scores=True), m, d, alpha ([rows, nep]), p8 ([rows, nep, 64]) and ro
    ([rows, nep, 128]) when nep > 0, rcp ([rows], the epilogue's 1 / (448 d)), and out, the
    forward output (the sampled rows of `head` only are written)."""
    dev = quant.k.device
    varlen = cu_seqlens_q is not None
    if varlen:
        Lq = quant.total_q if Lq is None else Lq
        Lk = quant.total_k if Lk is None else Lk
    ld = Lk if ld is None else ld
    rows = max(0, -(-(q_end - q_begin) // q_step))
    r = {}
    with _on(stream):
        if scores:
            r["acc"] = torch.zeros((rows, ld), dtype=torch.int32, device=dev)
            r["s"] = torch.zeros((rows, ld), dtype=torch.float32, device=dev)
        if nep:
            for n in ("m", "d", "alpha"):
                r[n] = torch.zeros((rows, nep), dtype=torch.float32, device=dev)
            r["p8"] = torch.zeros((rows, nep, 64), dtype=torch.uint8, device=dev)
            r["ro"] = torch.zeros((rows, nep, D), dtype=torch.float32, device=dev)
        r["rcp"] = torch.zeros((rows,), dtype=torch.float32, device=dev)
        if out is None:
            shape = (Lq, quant.H, D) if varlen else (quant.nseg, Lq, quant.H, D)
            out = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    r["out"] = out
    ck = Checkpoints(_ptr(r.get("acc")), _ptr(r.get("s")), ld if scores else 0, _ptr(r.get("m")), _ptr(r.get("d")),
                     _ptr(r.get("alpha")), _ptr(r.get("p8")), _ptr(r.get("ro")), nep, _ptr(r.get("rcp")))
    st = quant.struct()
    _check(lib().sattn_debug_scores(ctypes.byref(st), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), quant.nseg, Lq, Lk,
                                    quant.H, D, float(sm_scale), seg, head, q_begin, q_end, q_step, ctypes.byref(ck),
                                    _view(out, BF16Out), _stream(stream)), "sattn_debug_scores")
    return r


# ---------------------------------------------------------------- layout inspection
def untile_qk(tiles):
    """[nblk, 8192] INT8 operand tiles (one head) → [nblk*64, 128] token-major codes."""
    t = np.asarray(tiles).reshape(-1, 2, 4, 2, 32, 16)  # [blk, t, u, g, i, s]
    return t.transpose(0, 1, 4, 3, 2, 5).reshape(-1, 128)  # token = 32t + i, channel = 64g + 16u + s


def untile_v(tiles):
    """[nblk, 8192] E4M3 V tiles (one head) → [nblk*64, 128] token-major codes."""
    t = np.asarray(tiles).reshape(-1, 4, 2, 2, 32, 4, 4)  # [blk, w, f, g, i, q, r]
    # key = 32f + 8q + 4g + r, channel = 32w + i
    return t.transpose(0, 2, 5, 3, 6, 1, 4).reshape(-1, 128)


def segment_blocks(cu, dense_L=None):
    """First quantized block of every segment (dense: s*ceil(L/64); packed: cu[s]//64 + s)."""
    if dense_L is not None:
        nb = -(-dense_L // 64)
        return [s * nb for s in range(len(cu) - 1)]
    return [int(cu[s]) // 64 + s for s in range(len(cu) - 1)]
