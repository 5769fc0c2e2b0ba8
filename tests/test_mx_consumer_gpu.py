"""MXFP4 output read by an MI355X consumer: the MX-scaled FP4 GEMM of the
platform's BLAS library (hipBLASLt, reached through torch._scaled_mm with
float4_e2m1fn_x2 operands and float8_e8m0fnu block scales).

The library's MXFP4 encoding (page "A Fused Hadamard + NVFP4 Quantization
Kernel in Triton", section 1's contrast of NVFP4 with MXFP4 and its "Try this"
item 2; the E8M0 byte as the exponent 2^(byte - 127), page "Hopper kernel for
MXFP4", scale conversion) is fed to that GEMM as it is: codes [rows, cols/2]
with element 2k in the low nibble, scales [rows, cols/32] row-major.  The
product must equal the fp64 product of the library's own decode of the same
bytes, to one bf16 unit in the last place of the GEMM's output (2^-7
relative: its conversion to bf16 is not assumed to round to nearest) plus its
fp32 accumulation (K * 2^-24 of the sum of magnitudes).  So the nibble order, the
E2M1 values, the meaning of the scale byte and the scale layout agree with an
independent consumer on this hardware; a wrong scale byte must break it.

The NVFP4 layouts have no such consumer here: the same stack rejects E4M3
block scales on ROCm.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if not (hasattr(torch, "float4_e2m1fn_x2") and hasattr(torch, "float8_e8m0fnu")):
        pytest.skip("this PyTorch has no FP4 / E8M0 dtypes")
    import nvfp4_activation_amd as nv
    return nv


def spread_input(rows, cols, seed):
    """N(0,1) times a per-block log-normal gain (e^(2 N(0,1))), so that block
    scales differ widely and a misread scale shows."""
    z = synth.normal_f64(rows * cols, seed=seed, stream=1).reshape(rows, cols)
    gain = np.exp(2.0 * synth.normal_f64(rows * (cols // 32), seed=seed, stream=2)).reshape(rows, cols // 32)
    v = z * np.repeat(gain, 32, axis=1)
    return torch.from_numpy(synth.round_bf16(v.reshape(-1)).view(np.int16).reshape(rows, cols)).view(
        torch.bfloat16).to("cuda:0")


def consumer_gemm(qa, sa, qb, sb):
    """hipBLASLt's MX-FP4 GEMM: A [M, K] times B [N, K] transposed, bf16 out."""
    return torch._scaled_mm(qa.view(torch.float4_e2m1fn_x2), qb.view(torch.float4_e2m1fn_x2).t(),
                            sa.contiguous().view(torch.float8_e8m0fnu).flatten(),
                            sb.contiguous().view(torch.float8_e8m0fnu).flatten(), out_dtype=torch.bfloat16)


def within_bound(out, da, db, k):
    ref = da @ db.T
    slack = (da.abs() @ db.abs().T) * (k * 2.0 ** -24)
    err = (out.double() - ref).abs()
    return bool((err <= 2.0 ** -7 * ref.abs() + slack).all()), (err / (ref.abs() + slack)).max().item()


@pytest.mark.parametrize("m,n,k", [(256, 256, 512), (128, 384, 256), (384, 128, 1024)])
@pytest.mark.parametrize("rotate", [False, True])
def test_mxfp4_output_through_the_platform_gemm(nv, m, n, k, rotate):
    a = spread_input(m, k, seed=m + k)
    b = spread_input(n, k, seed=n + 3 * k)
    qa, sa = nv.mx_rotquant(a, rotate=rotate)
    qb, sb = nv.mx_rotquant(b, rotate=rotate)
    # the consumer multiplies the encoded values (in the rotated basis when
    # rotate: H is orthogonal, so that product approximates a b^T as well)
    da = nv.mx_dequant(qa, sa, rotate=False).double()
    db = nv.mx_dequant(qb, sb, rotate=False).double()
    try:
        out = consumer_gemm(qa, sa, qb, sb)
    except (RuntimeError, NotImplementedError, ValueError) as e:
        pytest.skip(f"MX-FP4 GEMM not available: {e}")
    torch.cuda.synchronize()
    ok, worst = within_bound(out, da, db, k)
    say(f"{m}x{n}x{k} rotate={rotate}: worst error / bound scale {worst:.3e}")
    assert ok, f"the platform GEMM disagrees with the decoded product (worst {worst:.3e})"
    if rotate:
        # rotating both operands leaves the product's meaning: close to a b^T
        exact = a.double() @ b.double().T
        rel = ((out.double() - exact).norm() / exact.norm()).item()
        say(f"  against a b^T: relative error {rel:.3f}")
        assert rel < 0.3
    # sensitivity: one scale byte one higher doubles one block of row 0
    sa2 = sa.clone()
    sa2[0, 0] += 1
    bad = consumer_gemm(qa, sa2, qb, sb)
    torch.cuda.synchronize()
    assert not within_bound(bad, da, db, k)[0] or not qa[0, :16].any(), "a changed scale went unnoticed"
