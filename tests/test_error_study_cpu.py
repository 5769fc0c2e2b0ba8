"""The error study's section-5 cases (CPU): the case keys are the fixture's,
the tensors have the page's shape, the column mask drops exactly the three
outlier columns, and drawing them leaves PyTorch's global generator as it
was.  The printed errors themselves are checked through the GPU path in
test_unfused_gpu.py."""
from __future__ import annotations

import torch

from conftest import read_golden


def test_section5_cases_shape_and_keys():
    from nvfp4_activation_amd import error_study as es
    before = torch.random.get_rng_state()
    cases = es.section5_cases()
    assert torch.equal(before, torch.random.get_rng_state())
    assert sorted(cases) == sorted(r[0] for r in read_golden("error_table.txt"))
    for key, (t, cols) in cases.items():
        assert t.shape == (256, 64) and t.dtype == torch.float32, key
    mask = cases["outlier_normal"][1]
    assert mask.dtype == torch.bool and int(mask.sum()) == 61
    assert [c for c in range(64) if not mask[c]] == list(es.OUTLIER_COLUMNS)
    assert cases["outlier_all"][0] is cases["outlier_normal"][0]
    # the outlier columns carry the gain: their spread is far above the rest
    t = cases["outlier_all"][0]
    spread = t.std(dim=0)
    assert float(spread[mask].max()) * 5 < float(spread[~mask].min())
    # drawing twice gives the same tensors
    again = es.section5_cases()
    for key in cases:
        assert torch.equal(cases[key][0], again[key][0]), key
