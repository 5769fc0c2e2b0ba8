"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bar: packed codes, block-scale bytes, the global scale and the amax are
identical byte for byte (the method is a deterministic encoding: page "A Fused
Hadamard + NVFP4 Quantization Kernel in Triton", sections 2-3).  The
dequantized round-trip error agrees with the oracle's fp64 error within 1e-6
relative.
"""
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


def f32bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).reshape(-1)[0].view(np.uint32))


def compare(tag, x_np, rotate, got, ref=None):
    """Byte-for-byte comparison with the oracle; a readable report on failure."""
    q, s, g, a = [t.cpu().numpy() if torch.is_tensor(t) else t for t in got]
    if ref is None:
        ref = oracle.quantize(x_np, rotate)
    oq, os_, og, oa = ref
    msgs = []
    if f32bits(a) != f32bits(oa):
        msgs.append(f"amax {np.float32(a.reshape(-1)[0])!r} != oracle {oa!r}")
    if f32bits(g) != f32bits(og):
        msgs.append(f"gscale {np.float32(g.reshape(-1)[0])!r} != oracle {og!r}")
    if not np.array_equal(s, os_):
        bad = np.argwhere(s != os_)
        msgs.append(f"{len(bad)} scale bytes differ, first {bad[0].tolist()}: "
                    f"{s[tuple(bad[0])]:#04x} vs {os_[tuple(bad[0])]:#04x}")
    if not np.array_equal(q, oq):
        bad = np.argwhere(q != oq)
        msgs.append(f"{len(bad)} code bytes differ, first {bad[0].tolist()}: "
                    f"{q[tuple(bad[0])]:#04x} vs {oq[tuple(bad[0])]:#04x}")
    assert not msgs, f"{tag}: " + "; ".join(msgs)


# ---------------------------------------------------------------- small shapes

SHAPES = [(1, 16), (3, 48), (127, 16), (5, 1024), (300, 4112), (1000, 1040), (257, 8192),
          (65536, 16), (4099, 32), (1, 1048576), (3, 262160)]


def mixed_input(rows, cols, dtype, seed):
    """N(0,1) times a per-element log-normal spread of magnitudes, so sums in
    the butterfly round and scales cover a wide range."""
    n = rows * cols
    z = synth.normal_f64(n, seed=seed, stream=1)
    m = synth.normal_f64(n, seed=seed, stream=2)
    v = z * np.exp(2.0 * m)
    if dtype == "bf16":
        return synth.round_bf16(v).reshape(rows, cols)
    return v.astype(np.float32).reshape(rows, cols)


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [True, False])
def test_small_shapes(nv, rows, cols, dtype, rotate):
    x = mixed_input(rows, cols, dtype, seed=rows * 7919 + cols)
    got = nv.rotquant(to_dev(x), rotate=rotate)
    torch.cuda.synchronize()
    compare(f"{rows}x{cols} {dtype} rotate={rotate}", x, rotate, got)


# ---------------------------------------------------------------- the workloads

WORKLOAD_CASES = [(name, rot) for name, (_, _, _, rots) in synth.WORKLOADS.items() for rot in rots]


@pytest.mark.parametrize("name,rotate", WORKLOAD_CASES)
def test_workload_full_size(nv, name, rotate):
    say(f"[parity] {name} rotate={rotate}: generating")
    w = synth.make(name, rotate=rotate)
    say(f"[parity] {name}: gpu")
    xd = to_dev(w.x)
    got = nv.rotquant(xd, rotate=rotate)
    torch.cuda.synchronize()
    got = [t.cpu() for t in got]
    del xd
    say(f"[parity] {name}: oracle")
    ref = oracle.quantize(w.x, rotate)
    compare(f"{name} rotate={rotate}", w.x, rotate, got, ref)
    q, s, g, a = [t.numpy() for t in got]
    # structural facts the recipes plant
    assert s.max() == 0x7E
    if name.startswith("silu_ties"):
        assert g[0] == np.float32(1.0 / 16.0)
        flags = w.meta["tie_flags"].astype(bool)
        assert np.all(s.reshape(-1)[flags] == 0x58)      # E4M3 16.0
    if name.startswith("kv_heads"):
        kind = w.meta["block_kind"]
        sb = s.reshape(-1)
        assert np.all(sb[kind == 3] == 0x7E)
        assert np.all(sb[(kind == 1) | (kind == 2)] == 0)
        assert not q.reshape(-1, 8)[(kind == 1) | (kind == 2)].any()
    say(f"[parity] {name}: ok")


# ---------------------------------------------------------------- edge cases

def test_all_zero_and_negative_zero(nv):
    for dtype in ("bf16", "f32"):
        x = np.zeros((7, 64), dtype=np.uint16 if dtype == "bf16" else np.float32)
        if dtype == "bf16":
            x[2] = 0x8000
        else:
            x[2] = -0.0
        for rotate in (True, False):
            got = nv.rotquant(to_dev(x), rotate=rotate)
            torch.cuda.synchronize()
            compare(f"zeros {dtype} rotate={rotate}", x, rotate, got)
            assert got[2].item() == 1.0 and got[3].item() == 0.0


def test_negative_zero_blocks_among_values(nv):
    x = mixed_input(16, 256, "f32", seed=3)
    x[3, 16:32] = -0.0
    x[5, :] = -0.0
    x[7, 48:64] = 0.0
    for rotate in (True, False):
        got = nv.rotquant(to_dev(x), rotate=rotate)
        torch.cuda.synchronize()
        compare(f"-0 blocks rotate={rotate}", x, rotate, got)


def test_empty_tensors(nv):
    for shape in ((0, 64), (5, 0), (0, 0)):
        for dt in (torch.bfloat16, torch.float32):
            x = torch.empty(shape, dtype=dt, device="cuda:0")
            q, s, g, a = nv.rotquant(x, rotate=True)
            torch.cuda.synchronize()
            assert g.item() == 1.0 and a.item() == 0.0
            assert q.numel() == 0 and s.numel() == 0


def test_scale_rounds_to_zero_keeps_codes(nv):
    """Divisor 1.0 path (section 2's guard for a zero scale): a block far below
    the global amax gets scale 0 and codes of its raw values."""
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, 0] = 2.0 ** 20
    # (2 / 6) / g = 2 * 2688 / (6 * 2^20) < 2^-10, so the block scale rounds to 0
    x[1, :] = np.linspace(-2.0, 2.0, 64, dtype=np.float32)
    got = nv.rotquant(to_dev(x), rotate=False)
    torch.cuda.synchronize()
    compare("zero scale", x, False, got)
    ref = oracle.quantize(x, False)
    assert ref[1][1].max() == 0 and ref[0][1].any()


def test_e4m3_midpoint_scales(nv):
    """Global amax 2688 makes g = 1 exactly; block maxima 6 * m put the block
    value exactly on E4M3 midpoints m (ties to even)."""
    vals = []
    for e in range(-9, 9):
        for k in range(16):
            m = (8 + k + 0.5) * 2.0 ** (e - 3) if e >= -6 else (k + 0.5) * 2.0 ** -9
            if 6 * m < 2688:
                vals.append(6 * m)
    n = len(vals) + 1
    x = np.zeros((n, 16), dtype=np.float32)
    x[0, 0] = 2688.0
    for i, v in enumerate(vals):
        x[i + 1, 3] = -v
        x[i + 1, 7] = v / 3
    for rotate in (False,):
        got = nv.rotquant(to_dev(x), rotate=rotate)
        torch.cuda.synchronize()
        compare("e4m3 midpoints", x, rotate, got)


def test_extreme_magnitudes(nv):
    """Tiny (bf16 subnormal) and huge values; the contract allows |x| <= 2^123,
    so that no butterfly sum of 16 values overflows."""
    rng = np.random.default_rng(11)
    for lo, hi in ((-133, -120), (-40, 40), (100, 121), (-133, 121)):
        v = rng.standard_normal(64 * 128) * np.exp2(rng.integers(lo, hi, 64 * 128))
        v[::17] = 0.0
        for dtype in ("bf16", "f32"):
            x = (synth.round_bf16(v) if dtype == "bf16" else v.astype(np.float32)).reshape(64, 128)
            for rotate in (True, False):
                got = nv.rotquant(to_dev(x), rotate=rotate)
                torch.cuda.synchronize()
                compare(f"magnitudes 2^{lo}..2^{hi} {dtype} rotate={rotate}", x, rotate, got)


def test_quotients_near_e2m1_midpoints(nv):
    """fp32, rotate off, g = 1 (amax 2688): blocks whose scale is 1.0 (max 6),
    elements one ulp around each E2M1 midpoint and exactly on it."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    cand = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10)])
    cand = np.concatenate([cand, -cand])
    rows = (len(cand) + 14) // 15 + 1
    x = np.zeros((rows, 16), dtype=np.float32)
    x[0, 0] = 2688.0
    flat = list(cand)
    for r in range(1, rows):
        x[r, 0] = 6.0
        chunk = flat[(r - 1) * 15:(r - 1) * 15 + 15]
        x[r, 1:1 + len(chunk)] = chunk
    got = nv.rotquant(to_dev(x), rotate=False)
    torch.cuda.synchronize()
    compare("e2m1 midpoints", x, False, got)


# ---------------------------------------------------------------- paths and launch shapes

EXACT_CASES = [("gauss_outliers_128x1024", True), ("gauss_1pct_cols_4096x4096", False),
               ("silu_ties_32768x14336", True), ("silu_ties_32768x14336", False),
               ("t3_lognormal_16384x8192", True)]


@pytest.mark.parametrize("name,rotate", EXACT_CASES)
def test_exact_path_equals_oracle(nv, monkeypatch, name, rotate):
    """The all-IEEE-division path (taken outside the fast range, and forced
    here) gives the same bytes as the oracle and as the fast path."""
    w = synth.make(name, rotate=rotate, rows=min(synth.WORKLOADS[name][0], 512))
    xd = to_dev(w.x)
    fast = nv.rotquant(xd, rotate=rotate)
    monkeypatch.setenv("NVFP4RQ_EXACT_ONLY", "1")
    exact = nv.rotquant(xd, rotate=rotate)
    torch.cuda.synchronize()
    compare(f"{name} exact path", w.x, rotate, exact)
    for a, b in zip(fast, exact):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_launch_shape_invariance(nv, monkeypatch, dtype):
    """Outputs do not depend on the number of workgroups (the page's first
    "Try this": results must not depend on tiling)."""
    x = mixed_input(777, 2064, dtype, seed=99)
    xd = to_dev(x)
    ref = [t.clone() for t in nv.rotquant(xd, rotate=True)]
    torch.cuda.synchronize()
    compare(f"default shape {dtype}", x, True, ref)
    for a_wgs, q_wgs in ((1, 1), (3, 7), (64, 5), (1000, 4096), (2, 100000)):
        monkeypatch.setenv("NVFP4RQ_AMAX_WGS", str(a_wgs))
        monkeypatch.setenv("NVFP4RQ_QUANT_WGS", str(q_wgs))
        got = nv.rotquant(xd, rotate=True)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r, g), (a_wgs, q_wgs)


@pytest.mark.parametrize("target", [2.0 ** 15 * 0.999, 2.0 ** 15, 2.0 ** 15 * 1.01,
                                    2.0 ** -38, 2.0 ** -38 * 0.99, 2.0 ** -38 * 1.01])
def test_fast_range_edges(nv, target):
    """Tensors whose amax sits at either edge of the fast path's range."""
    base = mixed_input(64, 512, "f32", seed=7).astype(np.float64)
    for rotate in (True, False):
        v = base / np.abs(base).max() * target
        x = synth.round_bf16(v).reshape(64, 512)
        got = nv.rotquant(to_dev(x), rotate=rotate)
        torch.cuda.synchronize()
        compare(f"amax ~ {target!r} rotate={rotate}", x, rotate, got)


# ---------------------------------------------------------------- given global scale

GIVEN_CASES = [("gauss_outliers_128x1024", True), ("t3_lognormal_16384x8192", True),
               ("silu_ties_32768x14336", False), ("kv_heads_65536x8x128_f32", True)]


@pytest.mark.parametrize("name,rotate", GIVEN_CASES)
def test_given_scale_single_pass(nv, name, rotate):
    """Pass 2 with an amax from elsewhere (an earlier step): block values can
    exceed 448 (clamped) and quotients 6 (largest code).  Against the oracle's
    quantizer with the same global scale."""
    w = synth.make(name, rotate=rotate, rows=min(synth.WORKLOADS[name][0], 1024))
    xd = to_dev(w.x)
    true_amax = oracle.amax(w.x, rotate)
    for factor in (1e-6, 0.01, 0.3, 1.0, 2.0, 1e4):
        amax = np.float32(true_amax * factor)
        a = torch.tensor([amax], dtype=torch.float32, device="cuda:0")
        q, s, g = nv.quant_from_amax(xd, a, rotate=rotate)
        torch.cuda.synchronize()
        og = oracle.global_scale(amax)
        oq, os_ = oracle.quantize_given_scale(w.x, rotate, og)
        compare(f"{name} given amax x{factor}", w.x, rotate, (q, s, g, a), (oq, os_, og, amax))


def test_given_scale_huge_quotients(nv):
    """Values up to 2^100 with a global scale from amax 1: quotients far
    beyond binary32's reach of the corrected division take true divisions."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal(64 * 256) * np.exp2(rng.integers(-20, 101, 64 * 256))
    for dtype in ("bf16", "f32"):
        x = (synth.round_bf16(v) if dtype == "bf16" else v.astype(np.float32)).reshape(64, 256)
        xd = to_dev(x)
        for rotate in (True, False):
            for amax in (np.float32(1.0), np.float32(2.0 ** -30), np.float32(1000.0)):
                a = torch.tensor([amax], dtype=torch.float32, device="cuda:0")
                q, s, g = nv.quant_from_amax(xd, a, rotate=rotate)
                torch.cuda.synchronize()
                og = oracle.global_scale(amax)
                oq, os_ = oracle.quantize_given_scale(x, rotate, og)
                compare(f"huge {dtype} rotate={rotate} amax={amax}", x, rotate, (q, s, g, a),
                        (oq, os_, og, amax))


# ---------------------------------------------------------------- pass-level entry points

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_passes_equal_fused_call(nv, dtype):
    x = mixed_input(512, 2048, dtype, seed=21)
    xd = to_dev(x)
    for rotate in (True, False):
        amax = nv.rotamax(xd, rotate=rotate)
        q, s, g = nv.quant_from_amax(xd, amax, rotate=rotate)
        torch.cuda.synchronize()
        compare(f"two passes {dtype} rotate={rotate}", x, rotate, (q, s, g, amax))


def test_side_stream_and_repeat(nv):
    x = mixed_input(1024, 4096, "bf16", seed=5)
    xd = to_dev(x)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        r1 = nv.rotquant(xd, rotate=True)
        r2 = nv.rotquant(xd, rotate=True)
    st.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    compare("side stream", x, True, r1)


# ---------------------------------------------------------------- round trip

@pytest.mark.parametrize("name,rotate", WORKLOAD_CASES)
def test_dequant_round_trip(nv, name, rotate):
    w = synth.make(name, rotate=rotate, rows=min(synth.WORKLOADS[name][0], 2048))
    xd = to_dev(w.x)
    q, s, g, a = nv.rotquant(xd, rotate=rotate)
    y = nv.dequant(q, s, g, rotate=rotate)
    torch.cuda.synchronize()
    xf = xd.double()
    e_gpu = ((y.double() - xf).norm() / xf.norm()).item()
    oq, os_, og, oa = oracle.quantize(w.x, rotate)
    e_ora = oracle.roundtrip_error(w.x, rotate, oq, os_, og)
    assert abs(e_gpu - e_ora) <= 1e-6 * e_ora, (e_gpu, e_ora)
    # and element-wise against the oracle's fp64 decode
    yd = oracle.dequant_f64(oq, os_, og, rotate)
    scale = np.abs(yd).max()
    assert np.max(np.abs(y.cpu().numpy().astype(np.float64) - yd)) <= 1e-6 * scale


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("rotate", [True, False])
def test_dequant_small_shapes(nv, rows, cols, rotate):
    """Decode on shapes whose quarter-block count leaves a ragged last
    iteration, element by element against the oracle's fp64 decode."""
    x = mixed_input(rows, cols, "bf16", seed=rows * 13 + cols)
    q, s, g, a = nv.rotquant(to_dev(x), rotate=rotate)
    y = nv.dequant(q, s, g, rotate=rotate)
    torch.cuda.synchronize()
    compare(f"{rows}x{cols} rotate={rotate}", x, rotate, (q, s, g, a))
    yd = oracle.dequant_f64(q.cpu().numpy(), s.cpu().numpy(), float(g.cpu()[0]), rotate)
    tol = 1e-6 * np.abs(yd).reshape(-1, 16).max(1).repeat(16).reshape(yd.shape)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - yd) <= tol)


# ---------------------------------------------------------------- swizzled scales

SWZ_SHAPES = [(1, 16), (3, 48), (127, 16), (128, 64), (129, 80), (300, 4112), (257, 8192),
              (1000, 4096), (2000, 8192),   # these two: 16-chunk runs per XCD, ragged last tile
              (65536, 16), (4099, 256),     # one block per row; the head with a 3-row last row tile
              (1, 1048576)]                 # one row: 4096 one-row chunks


@pytest.mark.parametrize("rows,cols", SWZ_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swizzled_scales(nv, rows, cols, dtype):
    """Scales written in the tiled layout equal the oracle's row-major scales
    put through the oracle's layout map (zero padding included); codes, g and
    amax equal the row-major call's."""
    x = mixed_input(rows, cols, dtype, seed=rows * 3 + cols)
    xd = to_dev(x)
    q, s, g, a = nv.rotquant_swizzled(xd, rotate=True)
    torch.cuda.synchronize()
    oq, os_, og, oa = oracle.quantize(x, True)
    compare(f"swizzled {rows}x{cols} {dtype}", x, True, (q, os_, g, a), (oq, os_, og, oa))
    assert np.array_equal(s.cpu().numpy(), oracle.swizzle_scales(os_))


@pytest.mark.parametrize("name,rotate", WORKLOAD_CASES)
def test_swizzled_scales_full_size(nv, name, rotate):
    w = synth.make(name, rotate=rotate)
    xd = to_dev(w.x)
    q, s, g, a = nv.rotquant_swizzled(xd, rotate=rotate)
    rq, rs, rg, ra = nv.rotquant(xd, rotate=rotate)
    torch.cuda.synchronize()
    assert torch.equal(q, rq) and torch.equal(g, rg) and torch.equal(a, ra)
    assert np.array_equal(s.cpu().numpy(), oracle.swizzle_scales(rs.cpu().numpy()))


def test_swizzled_padding_is_rewritten_to_zero(nv):
    x = mixed_input(129, 80, "bf16", seed=4)
    xd = to_dev(x)
    q, s, g, a = nv.rotquant_swizzled(xd)
    s.fill_(0xAB)
    nv.rotquant_swizzled(xd, out=(q, s, g, a))
    torch.cuda.synchronize()
    oq, os_, og, oa = oracle.quantize(x, True)
    assert np.array_equal(s.cpu().numpy(), oracle.swizzle_scales(os_))


@pytest.mark.parametrize("rows,cols", [(129, 80), (257, 8192)])
def test_swizzled_dequant(nv, rows, cols):
    x = mixed_input(rows, cols, "bf16", seed=rows + 2 * cols)
    xd = to_dev(x)
    for rotate in (True, False):
        q, s, g, a = nv.rotquant_swizzled(xd, rotate=rotate)
        y = nv.dequant_swizzled(q, s, g, rotate=rotate)
        rq, rs, rg, ra = nv.rotquant(xd, rotate=rotate)
        y_ref = nv.dequant(rq, rs, rg, rotate=rotate)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swizzled_launch_shape_invariance(nv, monkeypatch, dtype):
    """Super-tile chunks handed out over any number of workgroups, of 256 or
    1024 threads, give the same bytes (ragged tile edges included), with the
    maxima at the head and through the zeroed word."""
    x = mixed_input(300, 4112, dtype, seed=8)
    xd = to_dev(x)
    ref = [t.clone() for t in nv.rotquant_swizzled(xd)]
    torch.cuda.synchronize()
    oq, os_, og, oa = oracle.quantize(x, True)
    assert np.array_equal(ref[1].cpu().numpy(), oracle.swizzle_scales(os_))
    for threads in (256, 1024):
        monkeypatch.setenv("NVFP4RQ_SWZ_THREADS", str(threads))
        for zeroed in (False, True):
            if zeroed:
                monkeypatch.setenv("NVFP4RQ_ZEROED_AMAX", "1")
            else:
                monkeypatch.delenv("NVFP4RQ_ZEROED_AMAX", raising=False)
            for wgs in (1, 3, 7, 64, 100000):
                monkeypatch.setenv("NVFP4RQ_QUANT_WGS", str(wgs))
                got = nv.rotquant_swizzled(xd)
                torch.cuda.synchronize()
                for r, g in zip(ref, got):
                    assert torch.equal(r, g), (threads, zeroed, wgs)


# ---------------------------------------------------------------- pass-1 partials in q_out

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partials_path_equals_zeroed_word_path(nv, monkeypatch, dtype):
    """The fused call keeps pass 1's per-workgroup maxima at the head of q_out
    (no zeroed word); forcing the zeroed-word path gives the same bytes, for
    every pass-2 grid size and for the swizzled layout too."""
    x = mixed_input(777, 2064, dtype, seed=31)
    xd = to_dev(x)
    for rotate in (True, False):
        a = [t.clone() for t in nv.rotquant(xd, rotate=rotate)]
        sa = [t.clone() for t in nv.rotquant_swizzled(xd, rotate=rotate)]
        torch.cuda.synchronize()
        compare(f"partials {dtype} rotate={rotate}", x, rotate, a)
        monkeypatch.setenv("NVFP4RQ_ZEROED_AMAX", "1")
        b = nv.rotquant(xd, rotate=rotate)
        sb = nv.rotquant_swizzled(xd, rotate=rotate)
        torch.cuda.synchronize()
        monkeypatch.delenv("NVFP4RQ_ZEROED_AMAX")
        for u, v in zip(a + sa, list(b) + list(sb)):
            assert torch.equal(u, v)
    for a_wgs, q_wgs in ((1, 1), (1000, 1), (3, 2048), (700, 5)):
        monkeypatch.setenv("NVFP4RQ_AMAX_WGS", str(a_wgs))
        monkeypatch.setenv("NVFP4RQ_QUANT_WGS", str(q_wgs))
        got = nv.rotquant(xd)
        torch.cuda.synchronize()
        compare(f"partials {dtype} grids {a_wgs}/{q_wgs}", x, True, got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,a_wgs", [(128, 1024, 0), (300, 4112, 0), (777, 2064, 3), (1000, 1040, 511)])
def test_head_ignores_stale_output_bytes(nv, monkeypatch, dtype, rows, cols, a_wgs):
    """The quantize pass reduces all 512 words of the head, so the words past
    pass 1's grid must be cleared by pass 1: with q_out and s_out filled with
    0xFF beforehand (stale words reading as 0xFFFFFFFF, above any amax), the
    row-major and swizzled calls still equal the oracle, for the default
    pass-1 grids (most words unused) and for forced grids of 3 and 511
    workgroups (509 words unused, and 1)."""
    if a_wgs:
        monkeypatch.setenv("NVFP4RQ_AMAX_WGS", str(a_wgs))
    x = mixed_input(rows, cols, dtype, seed=rows + cols + a_wgs)
    xd = to_dev(x)
    ref = oracle.quantize(x, True)
    q = torch.full((rows, cols // 2), 0xFF, dtype=torch.uint8, device="cuda:0")
    s = torch.full((rows, cols // 16), 0xFF, dtype=torch.uint8, device="cuda:0")
    g = torch.full((1,), float("nan"), device="cuda:0")
    a = torch.full((1,), float("nan"), device="cuda:0")
    nv.rotquant(xd, out=(q, s, g, a))
    torch.cuda.synchronize()
    compare(f"stale row-major {dtype} {rows}x{cols} grid {a_wgs}", x, True, (q, s, g, a), ref)
    qs, ss, gs, as_ = nv.rotquant_swizzled(xd)
    q.fill_(0xFF)
    ss.fill_(0xFF)
    nv.rotquant_swizzled(xd, out=(q, ss, gs, as_))
    torch.cuda.synchronize()
    assert np.array_equal(ss.cpu().numpy(), oracle.swizzle_scales(ref[1]))
    compare(f"stale swizzled {dtype} {rows}x{cols} grid {a_wgs}", x, True, (q, ref[1], gs, as_), ref)


def test_head_wait_with_tiny_time_limit(nv, monkeypatch):
    """A head-wait limit of one microsecond: the wait either completes in time
    (output equal to the oracle) or gives up and marks the call with a NaN
    global scale and a NaN amax; either way every workgroup exits.  Row-major
    codes and swizzled scales both carry the head."""
    monkeypatch.setenv("NVFP4RQ_HEAD_TIMEOUT_US", "1")
    x = mixed_input(1024, 4096, "bf16", seed=12)
    xd = to_dev(x)
    ref = oracle.quantize(x, True)
    for _ in range(3):
        for call in (nv.rotquant, nv.rotquant_swizzled):
            q, s, g, a = call(xd)
            torch.cuda.synchronize()
            gv, av = g.cpu().numpy()[0], a.cpu().numpy()[0]
            if np.isnan(gv):
                assert np.isnan(av), "a failed wait marks the amax too"
                continue
            if call is nv.rotquant:
                compare("tiny head-wait limit", x, True, (q, s, g, a), ref)
            else:
                assert np.array_equal(s.cpu().numpy(), oracle.swizzle_scales(ref[1]))
                assert np.array_equal(q.cpu().numpy(), ref[0])


def test_timed_entry_point(nv):
    """The measurement hook gives the fused call's bytes, reports the kernels
    it launched and leaves each kernel's duration in its event pair."""
    for rows, cols, want, dtype in ((2048, 4096, 2, "bf16"), (4, 64, 3, "bf16"),
                                    (2048, 4096, 2, "f32")):
        x = mixed_input(rows, cols, dtype, seed=rows)
        xd = to_dev(x)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in ev:
            e.record()
        torch.cuda.synchronize()
        q, s, g, a, nk = nv.rotquant_timed(xd, ev)
        torch.cuda.synchronize()
        assert nk == want
        compare(f"timed {rows}x{cols} {dtype}", x, True, (q, s, g, a))
        for k in range(nk):
            ms = ev[2 * k].elapsed_time(ev[2 * k + 1])
            assert 0.0 < ms < 100.0, (k, ms)


def test_large_input_path(nv):
    """From 512 MiB of input the fused call hands the amax over through a
    zeroed word (three kernels) and pass 2 runs a workgroup per chunk, the
    first workgroups taking the last chunks; just below that size it keeps
    the two-kernel path.  Both match the oracle byte for byte."""
    x = mixed_input(16384, 16384, "bf16", seed=77)
    for cols, want in ((16384, 3), (16368, 2)):
        xs = np.ascontiguousarray(x[:, :cols])
        xd = to_dev(xs)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in ev:
            e.record()
        torch.cuda.synchronize()
        q, s, g, a, nk = nv.rotquant_timed(xd, ev)
        torch.cuda.synchronize()
        assert nk == want, (cols, nk)
        compare(f"16384x{cols} bf16", xs, True, (q, s, g, a))
        del xd, q, s


# ---------------------------------------------------------------- beyond 2^31 elements

def test_beyond_two_to_the_31_elements(nv):
    """65536 x 32800 bf16 (2.15e9 elements, 4.3 GB): every index past 2^31
    must be formed in 64 bits.  The tensor repeats one 4096-row block of the
    Student-t recipe 16 times, with its last 64 rows drawn separately and the
    largest value in the last row, so the amax and the final blocks depend on
    data past 2^31; the fused call, the swizzled scales and MXFP4 all match the
    oracle byte for byte."""
    rows, cols = 65536, 32800
    assert rows * cols > 2 ** 31
    say("[max size] generating")
    x = np.tile(synth.t3_lognormal(4096, cols, seed=17), (rows // 4096, 1))
    x[-64:] = synth.t3_lognormal(64, cols, seed=18)
    x[-1, -7] = synth.round_bf16(np.array([3.0e6]))[0]
    say("[max size] gpu")
    xd = to_dev(x)
    got = [t.cpu() for t in nv.rotquant(xd)]
    sw = nv.rotquant_swizzled(xd)[1].cpu().numpy()
    mq, ms = [t.cpu().numpy() for t in nv.mx_rotquant(xd)]
    torch.cuda.synchronize()
    del xd
    say("[max size] oracle")
    ref = oracle.quantize(x, True)
    assert float(ref[3]) >= 0.24 * 3.0e6          # the planted value (bf16: 2998272) sets it
    compare("65536x32800", x, True, got, ref)
    assert np.array_equal(sw, oracle.swizzle_scales(ref[1]))
    del sw, got, ref
    oq, os_ = oracle.mx_quantize(x, True)
    assert np.array_equal(ms, os_) and np.array_equal(mq, oq)
    say("[max size] ok")


# ---------------------------------------------------------------- graph capture

def test_graph_capture_replays(nv):
    """The fused call captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed several times, with new input copied in and eager library calls
    in between: every replay gives the eager call's bytes for that input (the
    call allocates nothing and records no memset, so it can be captured)."""
    rows, cols = 2048, 4096
    inputs = [mixed_input(rows, cols, "bf16", seed=100 + i) for i in range(4)]
    xd = to_dev(inputs[0])
    out = (torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda:0"),
           torch.empty(rows, cols // 16, dtype=torch.uint8, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.rotquant(xd, out=out)              # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.rotquant(xd, out=out)
    for i, x in enumerate(inputs[1:] + inputs[:1]):
        xd.copy_(to_dev(x))
        eager = [t.clone() for t in nv.rotquant(xd)]   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), i
        compare(f"replay {i}", x, True, out)


# ---------------------------------------------------------------- full-size given-scale and decode

def test_given_scale_and_decode_at_bench_size(nv):
    """At 16384 x 8192, as the bench times them: the given-scale single pass
    with an amax kept from another tensor (codes and scales equal to the
    oracle's), and the decode of the fused call's output (round-trip error
    within 1e-6 relative of the oracle's fp64 one, every element within 1e-6
    of its block's largest decoded value)."""
    w = synth.make("t3_lognormal_16384x8192", rotate=True)
    xd = to_dev(w.x)
    other = synth.make("t3_lognormal_16384x8192", rotate=True, seed=9, rows=4096)
    kept = np.float32(oracle.amax(other.x, True))
    a = torch.tensor([kept], dtype=torch.float32, device="cuda:0")
    q, s, g = nv.quant_from_amax(xd, a, rotate=True)
    torch.cuda.synchronize()
    og = oracle.global_scale(kept)
    oq, os_ = oracle.quantize_given_scale(w.x, True, og)
    compare("given scale 16384x8192", w.x, True, (q, s, g, a), (oq, os_, og, kept))
    del q, s, oq, os_
    q, s, g, amax = nv.rotquant(xd, rotate=True)
    y = nv.dequant(q, s, g, rotate=True)
    torch.cuda.synchronize()
    xf = xd.double()
    e_gpu = ((y.double() - xf).norm() / xf.norm()).item()
    del xf
    qn, sn, gn = q.cpu().numpy(), s.cpu().numpy(), float(g.cpu()[0])
    e_ora = oracle.roundtrip_error(w.x, True, qn, sn, gn)
    assert abs(e_gpu - e_ora) <= 1e-6 * e_ora, (e_gpu, e_ora)
    yd = oracle.dequant_f64(qn, sn, gn, True)
    err = np.abs(y.cpu().numpy().astype(np.float64) - yd).reshape(-1, 16)
    assert np.all(err <= 1e-6 * np.abs(yd).reshape(-1, 16).max(1, keepdims=True))


@pytest.mark.parametrize("nb", [511, 512, 513, 767, 1040, 2047, 2048, 2049, 4101])
def test_partials_path_threshold(nv, monkeypatch, nb):
    """Around the size from which pass 1's maxima and counters fit at the head
    of q_out (512 blocks: chunks 0 and 1, written by chunk 0's workgroup alone),
    in one row and in one column of blocks, with the default grid and with
    pass-2 grids of 1 and 7 workgroups."""
    for rows, cols in ((1, 16 * nb), (nb, 16)):
        x = mixed_input(rows, cols, "bf16", seed=nb + rows)
        xd = to_dev(x)
        ref = oracle.quantize(x, True)
        for q_wgs in (None, 1, 7):
            if q_wgs is None:
                monkeypatch.delenv("NVFP4RQ_QUANT_WGS", raising=False)
            else:
                monkeypatch.setenv("NVFP4RQ_QUANT_WGS", str(q_wgs))
            got = nv.rotquant(xd)
            torch.cuda.synchronize()
            compare(f"nb={nb} {rows}x{cols} quant_wgs={q_wgs}", x, True, got, ref)
