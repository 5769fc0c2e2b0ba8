"""Plain versus rotated round-trip error, NVFP4 and MXFP4, on the GPU path.

The question of section 5 of the page "A Fused Hadamard + NVFP4 Quantization
Kernel in Triton": does the 16-point rotation lower the relative L2 error
||dequant(quant(x)) - x|| / ||x||?  Asked here also under MXFP4 (the page's
"Try this" item 2: 32-element blocks, power-of-two scales) and with a random
orthogonal 16 x 16 matrix R in place of the Hadamard ("Try this" item 3:
rotate by R, quantize and decode with the built-in rotation off, rotate back
by R transposed).  Every rotation, encode and decode runs in the library's
kernels; only the two norms are taken with PyTorch, in fp64, on the device.

Inputs are arguments: a tensor (and optionally a column mask) per case, and R
as a float32 [16, 16] device tensor.  `section5_cases()` rebuilds the page's
four cases; `python bench.py --error-study` runs the study on them and on the
synthetic activation workloads and prints the table.
"""
from __future__ import annotations

import torch

import nvfp4_activation_amd as nv

# section 5: the outlier tensor has these three columns scaled by 20
OUTLIER_COLUMNS = (3, 17, 40)
OUTLIER_GAIN = 20.0


def section5_cases() -> dict:
    """The page's section-5 cases as {key: (float32 CPU tensor, column mask or
    None)}.  Its three 256 x 64 tensors come from PyTorch's CPU generator
    seeded with 0, drawn in the page's order: a normal tensor (which then gets
    the outlier columns), a second normal tensor, a Student-t sample with 3
    degrees of freedom.  The outlier tensor is scored twice: on every column
    and on the 61 columns without outliers."""
    gen_state = torch.random.get_rng_state()
    try:
        torch.manual_seed(0)
        draws = [torch.randn(256, 64), torch.randn(256, 64),
                 torch.distributions.StudentT(3.0).sample((256, 64))]
    finally:
        torch.random.set_rng_state(gen_state)
    outliers, gauss, t3 = draws
    cols = list(OUTLIER_COLUMNS)
    outliers[:, cols] *= OUTLIER_GAIN
    plain_cols = torch.ones(outliers.shape[1], dtype=torch.bool)
    plain_cols[cols] = False
    return {"outlier_all": (outliers, None), "outlier_normal": (outliers, plain_cols),
            "gaussian": (gauss, None), "student_t3": (t3, None)}


def relative_error(x: torch.Tensor, xr: torch.Tensor, cols: torch.Tensor | None = None) -> float:
    """||xr - x|| / ||x|| in fp64, over the columns `cols` selects (all when None)."""
    a, b = x.double(), xr.double()
    if cols is not None:
        keep = cols.to(a.device)
        a, b = a[:, keep], b[:, keep]
    return (torch.linalg.vector_norm(b - a) / torch.linalg.vector_norm(a)).item()


def nvfp4_error(x: torch.Tensor, rotate: bool, cols=None) -> float:
    q, s, g, _ = nv.rotquant(x, rotate=rotate)
    return relative_error(x, nv.dequant(q, s, g, rotate=rotate), cols)


def mxfp4_error(x: torch.Tensor, rotate: bool, cols=None) -> float:
    q, s = nv.mx_rotquant(x, rotate=rotate)
    return relative_error(x, nv.mx_dequant(q, s, rotate=rotate), cols)


def nvfp4_orth_error(x: torch.Tensor, r: torch.Tensor, cols=None) -> float:
    q, s, g, _ = nv.rotquant(nv.rotate_matrix(x, r), rotate=False)
    back = nv.rotate_matrix(nv.dequant(q, s, g, rotate=False), r.t().contiguous())
    return relative_error(x, back, cols)


def mxfp4_orth_error(x: torch.Tensor, r: torch.Tensor, cols=None) -> float:
    q, s = nv.mx_rotquant(nv.rotate_matrix(x, r), rotate=False)
    back = nv.rotate_matrix(nv.mx_dequant(q, s, rotate=False), r.t().contiguous())
    return relative_error(x, back, cols)


def study_row(x: torch.Tensor, r: torch.Tensor, cols=None) -> dict:
    """The six errors of one case: NVFP4 and MXFP4, each plain, with the
    built-in Hadamard rotation and with R."""
    return {"nvfp4_plain": nvfp4_error(x, False, cols), "nvfp4_rotated": nvfp4_error(x, True, cols),
            "nvfp4_orth": nvfp4_orth_error(x, r, cols),
            "mxfp4_plain": mxfp4_error(x, False, cols), "mxfp4_rotated": mxfp4_error(x, True, cols),
            "mxfp4_orth": mxfp4_orth_error(x, r, cols)}


def study(cases: dict, r: torch.Tensor) -> dict:
    """{key: study_row} for {key: (tensor, column mask or None)}; each tensor
    is moved to R's device."""
    return {k: study_row(t.to(r.device), r, cols) for k, (t, cols) in cases.items()}


def table(rows: dict) -> str:
    head = ("| case | NVFP4 plain | NVFP4 Hadamard | NVFP4 random orth. | MXFP4 plain | "
            "MXFP4 Hadamard | MXFP4 random orth. |\n|---|---|---|---|---|---|---|\n")
    return head + "".join(
        f"| {k} | {v['nvfp4_plain']:.4f} | {v['nvfp4_rotated']:.4f} | {v['nvfp4_orth']:.4f} | "
        f"{v['mxfp4_plain']:.4f} | {v['mxfp4_rotated']:.4f} | {v['mxfp4_orth']:.4f} |\n"
        for k, v in rows.items())
