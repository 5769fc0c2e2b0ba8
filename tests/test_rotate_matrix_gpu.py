"""The general block rotation (the Hadamard replaced by a caller's 16 x 16
matrix, "Try this" item 3 of the page "A Fused Hadamard + NVFP4 Quantization
Kernel in Triton"): bit-exact against the oracle on ragged shapes and both
input dtypes, exact on matrices whose products are exact, and the random
orthogonal error study run through the library against an fp64 computation
from the oracle's decode."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x).to("cuda:0")


def make(rows: int, cols: int, dtype: str, seed: int) -> np.ndarray:
    n = rows * cols
    v = synth.normal_f64(n, seed=seed, stream=1) * np.exp(2.0 * synth.normal_f64(n, seed=seed, stream=2))
    return (synth.round_bf16(v) if dtype == "bf16" else v.astype(np.float32)).reshape(rows, cols)


def as_f32(x: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(x) if x.dtype == np.uint16 else x


SHAPES = [(1, 16), (3, 48), (127, 16), (300, 4112), (257, 8192), (1000, 1040)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_orthogonal_matches_oracle(nv, rows, cols, dtype):
    say(f"rotate_matrix {rows}x{cols} {dtype}")
    x = make(rows, cols, dtype, seed=rows * 7 + cols)
    r = synth.random_orthogonal16(rows + cols)
    y = nv.rotate_matrix(to_dev(x), torch.from_numpy(r).to("cuda:0")).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), oracle.rotate_matrix(x, r).view(np.uint32))


def test_dense_matrix_with_extreme_entries(nv):
    """A non-orthogonal matrix whose entries span many binades, with signed
    zeros and inputs that overflow to infinity in some partial sums: every
    rounding of the product and each fused step must still agree."""
    rng = np.random.default_rng(7)
    r = (rng.standard_normal((16, 16)) * np.exp2(rng.integers(-30, 30, (16, 16)))).astype(np.float32)
    r[3, :] = -0.0
    r[:, 5] = 0.0
    x = make(64, 1024, "f32", seed=9)
    x[0, :16] = np.float32(3e38)
    x[1, 16:32] = np.float32(-1e-40)          # subnormal inputs
    rd = torch.from_numpy(r).to("cuda:0")
    y = nv.rotate_matrix(to_dev(x), rd).cpu().numpy()
    want = oracle.rotate_matrix(x, r)
    same = (y.view(np.uint32) == want.view(np.uint32)) | (np.isnan(y) & np.isnan(want))
    assert same.all()


def test_exact_matrices(nv):
    """Identity and signed permutations give their inputs back exactly; the
    Sylvester matrix with entries +-1/4 agrees with the oracle's evaluation of
    the same product (not with the butterfly, whose rounding differs)."""
    x = make(97, 272, "bf16", seed=3)
    xd = to_dev(x)
    eye = torch.eye(16, dtype=torch.float32, device="cuda:0")
    assert np.array_equal(nv.rotate_matrix(xd, eye).cpu().numpy(), as_f32(x))
    rng = np.random.default_rng(11)
    perm = rng.permutation(16)
    sign = np.where(rng.random(16) < 0.5, -1.0, 1.0).astype(np.float32)
    p = np.zeros((16, 16), dtype=np.float32)
    p[perm, np.arange(16)] = sign                  # y_j = sign_j x_perm[j]
    want = (as_f32(x).reshape(-1, 16)[:, perm] * sign).reshape(x.shape)
    got = nv.rotate_matrix(xd, torch.from_numpy(p).to("cuda:0")).cpu().numpy()
    assert np.array_equal(got, want)
    h = np.ones((1, 1))
    for _ in range(4):
        h = np.block([[h, h], [h, -h]])
    h = (h / 4.0).astype(np.float32)
    got = nv.rotate_matrix(xd, torch.from_numpy(h).to("cuda:0")).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.rotate_matrix(x, h).view(np.uint32))


def test_empty_and_validation(nv):
    r = torch.from_numpy(synth.random_orthogonal16(1)).to("cuda:0")
    y = nv.rotate_matrix(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda:0"), r)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    x = torch.zeros(4, 64, dtype=torch.float32, device="cuda:0")
    with pytest.raises(TypeError):
        nv.rotate_matrix(x, r.double())
    with pytest.raises(ValueError):
        nv.rotate_matrix(x, r[:8])
    with pytest.raises(ValueError):
        nv.rotate_matrix(x, r.cpu())
    with pytest.raises(ValueError):
        nv.rotate_matrix(x, r.t())                 # not contiguous


def test_large_tensor_sampled_rows(nv):
    """16384 x 8192 bf16: rows are independent, so the oracle on a sample of
    rows gives those rows' exact expected values."""
    rows, cols = 16384, 8192
    x = synth.normal_bf16(rows * cols, seed=21, stream=0).reshape(rows, cols)
    r = synth.random_orthogonal16(21)
    y = nv.rotate_matrix(to_dev(x), torch.from_numpy(r).to("cuda:0"))
    pick = np.unique(np.concatenate([[0, 1, rows - 1], np.random.default_rng(5).integers(0, rows, 61)]))
    got = y[torch.from_numpy(pick).to("cuda:0")].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.rotate_matrix(x[pick], r).view(np.uint32))


def test_orthogonal_error_study_through_the_library(nv):
    """Rotate by R, quantize and decode without the built-in rotation, rotate
    back by R transposed: each stage equals the oracle (codes and scales byte
    for byte), and the relative error equals the one computed in fp64 from the
    oracle's decode and the exact product with R transposed."""
    from nvfp4_activation_amd import error_study as es
    r = synth.random_orthogonal16(0)
    x = make(256, 1024, "f32", seed=33)
    xd = to_dev(x)
    rd = torch.from_numpy(r).to("cuda:0")
    y = nv.rotate_matrix(xd, rd)
    yo = oracle.rotate_matrix(x, r)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))
    q, s, g, _ = nv.rotquant(y, rotate=False)
    oq, os_, og, _ = oracle.quantize(yo, False)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    e_gpu = es.nvfp4_orth_error(xd, rd)
    d = oracle.dequant_f64(oq, os_, og, False)
    back = (d.reshape(-1, 16) @ r.astype(np.float64).T).reshape(x.shape)
    e_ref = np.linalg.norm(back - x) / np.linalg.norm(x)
    say(f"orthogonal NVFP4 error {e_gpu:.6f} (fp64 {e_ref:.6f})")
    assert abs(e_gpu - e_ref) <= 1e-5 * e_ref

    mq, ms = nv.mx_rotquant(y, rotate=False)
    omq, oms = oracle.mx_quantize(yo, False)
    assert np.array_equal(mq.cpu().numpy(), omq) and np.array_equal(ms.cpu().numpy(), oms)
    e_gpu = es.mxfp4_orth_error(xd, rd)
    d = oracle.mx_dequant_f64(omq, oms, False)
    back = (d.reshape(-1, 16) @ r.astype(np.float64).T).reshape(x.shape)
    e_ref = np.linalg.norm(back - x) / np.linalg.norm(x)
    say(f"orthogonal MXFP4 error {e_gpu:.6f} (fp64 {e_ref:.6f})")
    assert abs(e_gpu - e_ref) <= 1e-5 * e_ref


def test_study_rows_carry_orthogonal_columns(nv):
    from nvfp4_activation_amd import error_study as es
    rows = es.study(es.section5_cases(), torch.from_numpy(synth.random_orthogonal16(0)).to("cuda:0"))
    for name, row in rows.items():
        for key in ("nvfp4_orth", "mxfp4_orth"):
            assert 0.0 < row[key] < 1.0, (name, key, row[key])
    say(es.table(rows))
