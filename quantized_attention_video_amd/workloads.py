"""Seeded synthetic workloads shaped like the pages' attention problems.

This module only draws inputs; it holds none of the attention program's arithmetic and
is the single source of inputs for both the HIP path and the CPU oracle.

Shapes follow the pages' H3 workload ("H3 Performance Roadmap",
"Measured GB10 Baseline": 37,810 packed tokens of which 100 are text tokens; the
Phase 2B report's fixed B=1, H=1, Q=128, KV=192, D=128 shape with three K64 epochs).
The pages measure real block-24 activations, which are not available; these seeded
draws stand in for them.

Recipe (every workload):
  * one CPU torch.Generator seeded with 1000 + the workload number;
  * draw order: Q, K, V (each N(0, 1) in FP32, shape [B, L, H, D] or [T, H, D]), then the
    per-(head, channel) K bias (N(0, std), added to every token of K), then the Bernoulli
    row mask that scales Q rows by 8 (exact in BF16);
  * everything is rounded once to BF16 (round-to-nearest-even) at the end.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import torch

D = 128


@dataclass
class Workload:
    name: str
    number: int
    H: int
    # dense problems: B sequences of Lq queries and Lk keys
    B: int = 1
    Lq: int = 0
    Lk: int = 0
    # varlen problems: packed segment lengths (self-attention: queries = keys)
    seqlens: Optional[List[int]] = None
    k_bias_std: float = 0.0
    q_boost_frac: float = 0.0  # fraction of Q rows over (b, t, h) scaled by 8
    layout: str = "blhd"  # "bhld" | "blhd" | "fused_qkv" | "packed"
    sm_scale: float = D ** -0.5
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def varlen(self):
        return self.seqlens is not None

    def seqlens_q(self):
        return list(self.seqlens) if self.varlen else [self.Lq] * self.B

    def seqlens_k(self):
        return list(self.seqlens) if self.varlen else [self.Lk] * self.B

    def cu_q(self):
        return _prefix(self.seqlens_q())

    def cu_k(self):
        return _prefix(self.seqlens_k())

    def ops(self):
        """4 * Lq * Lk * D * H summed over segments: the operation count of the metric."""
        return sum(4 * a * b * D * self.H for a, b in zip(self.seqlens_q(), self.seqlens_k()))


def _prefix(lens):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return cu


WORKLOADS = {
    "fixed_q128_kv192": Workload("fixed_q128_kv192", 1, H=1, B=1, Lq=128, Lk=192, layout="bhld",
                                 notes="single head, fixed shape, three 64-key epochs"),
    "dense_h8_l4096": Workload("dense_h8_l4096", 2, H=8, B=1, Lq=4096, Lk=4096, k_bias_std=3.0,
                               layout="blhd", notes="per-channel K bias exercises K smoothing"),
    "ragged_b2_h16_l1000": Workload("ragged_b2_h16_l1000", 3, H=16, B=2, Lq=1000, Lk=1000,
                                    q_boost_frac=0.05, layout="blhd", notes="ragged tail of 40"),
    "ragged_b2_h16_l2049": Workload("ragged_b2_h16_l2049", 3, H=16, B=2, Lq=2049, Lk=2049,
                                    q_boost_frac=0.05, layout="blhd", notes="ragged tail of 1"),
    "h3_video_l37810": Workload("h3_video_l37810", 4, H=32, B=1, Lq=37810, Lk=37810, k_bias_std=2.0,
                                layout="fused_qkv",
                                notes="37,710 video + 100 text tokens; Q/K/V are slices of a fused "
                                      "[L, 3, H, D] projection output"),
    "varlen_h24_4seg": Workload("varlen_h24_4seg", 5, H=24, seqlens=[37810, 8192, 1536, 100], layout="packed",
                                notes="video, audio, short clip and text-only sequences, block-diagonal"),
    # The roadmap's larger size (243 frames at 1344x768, "74K tokens") with the head count
    # that its 7168-wide attention output implies at D=128 (56 heads).
    "h3_video_l74000_h56": Workload("h3_video_l74000_h56", 6, H=56, B=1, Lq=74000, Lk=74000, k_bias_std=2.0,
                                    layout="fused_qkv",
                                    notes="~74K packed tokens, 56 heads; fused [L, 3, H, D] projection output"),
}


def get(name):
    return WORKLOADS[name]


def make_inputs(w: Workload, seed: Optional[int] = None, scale_L: Optional[int] = None):
    """Draw the inputs of workload `w` on the CPU.

    Returns a dict with BF16 tensors q, k, v: dense workloads as [B, L, H, D] views (whose
    strides follow `w.layout`), varlen workloads as packed [T, H, D] tensors, plus
    cu_seqlens lists.  `scale_L` replaces the sequence length(s) of a dense workload
    (used to build small variants of a shape for tests).
    """
    g = torch.Generator().manual_seed(1000 + w.number if seed is None else seed)
    H = w.H
    if w.varlen:
        T = sum(w.seqlens)
        shapes = [(T, H, D)] * 3
    else:
        Lq = scale_L or w.Lq
        Lk = scale_L or w.Lk
        shapes = [(w.B, Lq, H, D), (w.B, Lk, H, D), (w.B, Lk, H, D)]
    q = torch.randn(shapes[0], generator=g, dtype=torch.float32)
    k = torch.randn(shapes[1], generator=g, dtype=torch.float32)
    v = torch.randn(shapes[2], generator=g, dtype=torch.float32)
    if w.k_bias_std:
        bias = torch.randn((H, D), generator=g, dtype=torch.float32) * w.k_bias_std
        k = k + bias
    if w.q_boost_frac:
        mask = torch.rand(q.shape[:-1], generator=g) < w.q_boost_frac
        q = torch.where(mask[..., None], q * 8.0, q)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    if w.layout == "bhld":  # contiguous [B, H, L, D] storage, viewed as [B, L, H, D]
        q, k, v = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    fused = None
    if w.layout == "fused_qkv":  # slices of one contiguous [B, L, 3, H, D] tensor
        fused = torch.stack([q, k, v], dim=2).contiguous()
        q, k, v = fused[:, :, 0], fused[:, :, 1], fused[:, :, 2]
    out = dict(q=q, k=k, v=v, workload=w, fused=fused)
    if w.varlen:
        out["cu_q"] = w.cu_q()
        out["cu_k"] = w.cu_k()
    else:
        Lq, Lk = shapes[0][1], shapes[1][1]
        out["cu_q"] = _prefix([Lq] * w.B)
        out["cu_k"] = _prefix([Lk] * w.B)
    return out


def to_device(inp, device="cuda"):
    """Copy q, k, v to `device` keeping their strides (the fused QKV storage moves whole)."""
    out = dict(inp)
    if inp.get("fused") is not None:
        f = inp["fused"].to(device)
        out.update(fused=f, q=f[:, :, 0], k=f[:, :, 1], v=f[:, :, 2])
    else:
        for n in ("q", "k", "v"):
            out[n] = inp[n].to(device)  # dense non-overlapping views keep their strides
    return out


def packed_float64(t):
    """[B, L, H, D] or [T, H, D] BF16 view → contiguous float64 NumPy [B*L or T, H, D]."""
    x = t.float()
    if x.dim() == 4:
        x = x.reshape(-1, x.shape[2], x.shape[3])
    return x.double().numpy()
