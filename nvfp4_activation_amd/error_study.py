"""Plain versus rotated round-trip error, NVFP4 and MXFP4, on the GPU path.

The study of section 5 of the page "A Fused Hadamard + NVFP4 Quantization
Kernel in Triton" (does the 16-point rotation lower the relative L2 error
||dequant(quant(x)) - x|| / ||x||?), together with its "Try this" item 2 (the
same question under MXFP4: 32-element blocks, power-of-two scales) and item 3
(a random orthogonal 16 x 16 matrix in place of the Hadamard: rotate by R,
quantize and decode with the built-in rotation off, rotate back by R
transposed).  Every rotation, encode and decode runs in the library's kernels;
only the two norms are taken with PyTorch, in fp64, on the device.

Cases: the page's three 256 x 64 tensors, drawn with PyTorch's CPU generator
from seed 0 in the page's order (normal with columns 3, 17 and 40 scaled by
20, normal, Student-t with 3 degrees of freedom), the outlier tensor scored
on all columns and on the 61 normal ones; then the synthetic activation
workloads (seeded generators at the repository root).

    python -m nvfp4_activation_amd.error_study [--rows N]
"""
from __future__ import annotations

import argparse
import os
import sys

import torch

import nvfp4_activation_amd as nv

OUTLIER_COLS = (3, 17, 40)


def page_tensors() -> dict:
    """The section-5 tensors, as float32 CPU tensors."""
    torch.manual_seed(0)
    x = torch.randn(256, 64)
    x[:, list(OUTLIER_COLS)] *= 20.0
    gauss = torch.randn(256, 64)
    t3 = torch.distributions.StudentT(3.0).sample((256, 64))
    normal = torch.ones(64, dtype=torch.bool)
    normal[list(OUTLIER_COLS)] = False
    return {"outlier channels: all values": (x, None),
            "outlier channels: normal cols": (x, normal),
            "gaussian": (gauss, None),
            "student-t, 3 dof": (t3, None)}


def relative_error(x: torch.Tensor, xr: torch.Tensor, cols: torch.Tensor | None = None) -> float:
    x, xr = x.double(), xr.double()
    if cols is not None:
        cols = cols.to(x.device)
        x, xr = x[:, cols], xr[:, cols]
    return ((xr - x).norm() / x.norm()).item()


def nvfp4_error(x: torch.Tensor, rotate: bool, cols=None) -> float:
    q, s, g, _ = nv.rotquant(x, rotate=rotate)
    return relative_error(x, nv.dequant(q, s, g, rotate=rotate), cols)


def mxfp4_error(x: torch.Tensor, rotate: bool, cols=None) -> float:
    q, s = nv.mx_rotquant(x, rotate=rotate)
    return relative_error(x, nv.mx_dequant(q, s, rotate=rotate), cols)


def orthogonal(device, seed: int = 0) -> torch.Tensor:
    """The random orthogonal matrix (seeded Haar draw from the generators at
    the repository root), on the device."""
    _root_on_path()
    import synth
    return torch.from_numpy(synth.random_orthogonal16(seed)).to(device)


def nvfp4_orth_error(x: torch.Tensor, r: torch.Tensor, cols=None) -> float:
    q, s, g, _ = nv.rotquant(nv.rotate_matrix(x, r), rotate=False)
    back = nv.rotate_matrix(nv.dequant(q, s, g, rotate=False), r.t().contiguous())
    return relative_error(x, back, cols)


def mxfp4_orth_error(x: torch.Tensor, r: torch.Tensor, cols=None) -> float:
    q, s = nv.mx_rotquant(nv.rotate_matrix(x, r), rotate=False)
    back = nv.rotate_matrix(nv.mx_dequant(q, s, rotate=False), r.t().contiguous())
    return relative_error(x, back, cols)


def study_row(x: torch.Tensor, cols=None) -> dict:
    r = orthogonal(x.device)
    return {"nvfp4_plain": nvfp4_error(x, False, cols), "nvfp4_rotated": nvfp4_error(x, True, cols),
            "nvfp4_orth": nvfp4_orth_error(x, r, cols),
            "mxfp4_plain": mxfp4_error(x, False, cols), "mxfp4_rotated": mxfp4_error(x, True, cols),
            "mxfp4_orth": mxfp4_orth_error(x, r, cols)}


def page_study(device="cuda:0") -> dict:
    return {name: study_row(t.to(device), cols) for name, (t, cols) in page_tensors().items()}


def _root_on_path():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)


def workload_study(rows_cap: int, device="cuda:0") -> dict:
    _root_on_path()
    import numpy as np
    import synth
    out = {}
    for name, (rows, _, _, _) in synth.WORKLOADS.items():
        w = synth.make(name, rotate=True, rows=min(rows, rows_cap))
        if w.x.dtype == np.uint16:
            x = torch.from_numpy(w.x.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            x = torch.from_numpy(w.x).to(device)
        out[f"{name} ({x.shape[0]} rows)"] = study_row(x)
    return out


def table(rows: dict) -> str:
    head = ("| case | NVFP4 plain | NVFP4 Hadamard | NVFP4 random orth. | MXFP4 plain | "
            "MXFP4 Hadamard | MXFP4 random orth. |\n|---|---|---|---|---|---|---|\n")
    return head + "".join(
        f"| {k} | {v['nvfp4_plain']:.4f} | {v['nvfp4_rotated']:.4f} | {v['nvfp4_orth']:.4f} | "
        f"{v['mxfp4_plain']:.4f} | {v['mxfp4_rotated']:.4f} | {v['mxfp4_orth']:.4f} |\n"
        for k, v in rows.items())


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=4096, help="row cap for the synthetic workloads")
    args = ap.parse_args()
    rows = page_study()
    rows.update(workload_study(args.rows))
    print(table(rows), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
