"""The C ABI without Python in the loop (needs an MI355X): tests/c_abi_driver, a C++ host
program that includes only include/sattn.h and the HIP runtime API, allocates every buffer
itself from sattn_quant_query and runs the quantizer and the forward on its own stream.
Its output must equal the Python binding's bit for bit (same library, same inputs) and
the oracle's within the tolerance."""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from oracle import sattn as O
from quantized_attention_video_amd import binding as B
from quantized_attention_video_amd import workloads as W

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver")
MAX_REL, MAE = 1e-2, 1e-3


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().astype(np.uint16).tobytes()


def _run_driver(tmp_path, header, cu, q, k, v, n_out):
    if not os.path.exists(DRIVER):
        pytest.fail("tests/c_abi_driver is not built: run __graft_entry__.build()")
    src, dst = tmp_path / "problem.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<5i", *header[:5]) + struct.pack("<f", header[5]))
        for c in cu:
            f.write(np.asarray(c, dtype="<i4").tobytes())
        for t in (q, k, v):
            f.write(_bits(t))
    p = subprocess.run([DRIVER, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    out = np.frombuffer(open(dst, "rb").read(), dtype=np.uint16)
    assert out.size == n_out
    return torch.from_numpy(out.astype(np.int16)).view(torch.bfloat16)


def _check(got, ref, label):
    H = ref.shape[1]
    for h in range(H):
        err = np.abs(got[:, h] - ref[:, h])
        scale = np.max(np.abs(ref[:, h]))
        assert np.max(err) <= MAX_REL * scale, f"{label} head {h}"
        assert np.mean(err) <= MAE, f"{label} head {h}"


def test_c_driver_dense(tmp_path):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    g = torch.Generator().manual_seed(23)
    nseg, H, Lq, Lk, sm = 2, 3, 150, 275, 0.0884
    q, k, v = (torch.randn((nseg, L, H, 128), generator=g).to(torch.bfloat16) for L in (Lq, Lk, Lk))
    out_c = _run_driver(tmp_path, (0, nseg, H, Lq, Lk, sm), [], q, k, v, nseg * Lq * H * 128)
    out_c = out_c.view(nseg, Lq, H, 128)
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda())
    out_py = B.sattn_fwd(quant, nseg, H, Lq, Lk, sm).cpu()
    assert torch.equal(out_c, out_py)
    cu_q, cu_k = [0, Lq, 2 * Lq], [0, Lk, 2 * Lk]
    ref = O.attention(O.quantize(*(W.packed_float64(t) for t in (q, k, v)), cu_q, cu_k), sm)
    _check(out_c.float().numpy().reshape(-1, H, 128).astype(np.float64), ref, "C driver, dense")


def test_c_driver_packed(tmp_path):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    g = torch.Generator().manual_seed(29)
    lens = [100, 0, 1, 257]
    H, sm = 2, 0.1
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    q, k, v = (torch.randn((T, H, 128), generator=g).to(torch.bfloat16) for _ in range(3))
    out_c = _run_driver(tmp_path, (1, len(lens), H, T, T, sm), [cu, cu], q, k, v, T * H * 128).view(T, H, 128)
    cq = torch.tensor(cu, dtype=torch.int32, device="cuda")
    quant = B.sattn_quantize_qkv(q.cuda(), k.cuda(), v.cuda(), cq, cq)
    out_py = B.sattn_fwd_varlen(quant, cq, cq, T, sm).cpu()
    assert torch.equal(out_c, out_py)
    ref = O.attention(O.quantize(*(W.packed_float64(t) for t in (q, k, v)), cu, cu), sm)
    _check(out_c.float().numpy().astype(np.float64), ref, "C driver, packed")
