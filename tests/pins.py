"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function takes an :class:`oracle.Oracle` handle and raises
``AssertionError`` when the oracle disagrees with a closed form, a brute
force enumeration, an independent library routine or a value worked by hand.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on builds with a planted mistake and requires each mistake to be
caught by at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from dfkv_workloads import GQA, MLA, Geometry, RopeSpec, bf16_bits, bits_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f(bits):
    return bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def _bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Distance between adjacent bf16 values around |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def pin_bf16_known_values(o):
    cases = [
        (1.0, 0x3F80),
        (-2.5, 0xC020),
        (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie -> even (mantissa 0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie -> even (mantissa 2)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie between 0 and 2^-133 -> even
        (3.0 * 2.0 ** -134, 0x0002),               # tie between 1 and 2 ulps -> even
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie with 2^128 -> rounds to +inf
        (float("inf"), 0x7F80),
        (-float("inf"), 0xFF80),
        (65536.0 + 128.0, 0x4780),                 # 2^16 + half spacing -> even
        (0.1, 0x3DCD),                             # 0.1 = 0x3DCCCCCD in fp32 -> 0x3DCD
    ]
    for x, want in cases:
        got = o.f64_to_bf16(x)
        assert got == want, f"bf16({x!r}) = {got:#06x}, want {want:#06x}"
    assert (o.f64_to_bf16(float("nan")) & 0x7F80) == 0x7F80 and (o.f64_to_bf16(float("nan")) & 0x7F) != 0


def pin_bf16_vs_torch(o):
    """torch's float32 -> bfloat16 conversion is round-to-nearest-even."""
    import torch
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0e38, 3.3e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.round_bf16(x.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} got {got[bad[0]]:#06x} want {ref[bad[0]]:#06x}"


# ---------------------------------------------------------------------------
# linear (fc and the stacked K/V GEMM)
# ---------------------------------------------------------------------------

def pin_linear_small_integers(o):
    """Small integers: every product and sum is exact, and |sum| <= 256 is a bf16 value."""
    rng = np.random.default_rng(11)
    n, k, m = 5, 16, 11
    xi = rng.integers(-2, 3, size=(n, k))
    wi = rng.integers(-2, 3, size=(m, k))
    got = _f(o.linear(bf16_bits(xi.astype(np.float32)), bf16_bits(wi.astype(np.float32))))
    want = (xi.astype(np.int64) @ wi.T.astype(np.int64)).astype(np.float64)
    assert np.array_equal(got, want), "integer GEMM mismatch"


def pin_linear_identity(o):
    rng = np.random.default_rng(12)
    x = bf16_bits(rng.standard_normal((3, 24)).astype(np.float32))
    eye = bf16_bits(np.eye(24, dtype=np.float32))
    assert np.array_equal(o.linear(x, eye), x)
    perm = rng.permutation(24)
    pm = bf16_bits(np.eye(24, dtype=np.float32)[perm])      # row j selects input column perm[j]
    assert np.array_equal(o.linear(x, pm), x[:, perm])


def pin_linear_vs_numpy(o):
    """numpy float64 matmul of the same bf16 values, then at most half a bf16 spacing apart."""
    rng = np.random.default_rng(13)
    for n, k, m in ((7, 96, 40), (1, 256, 3), (4, 33, 65)):
        x = bf16_bits(rng.standard_normal((n, k)).astype(np.float32))
        w = bf16_bits((rng.standard_normal((m, k)) / math.sqrt(k)).astype(np.float32))
        ref = _f(x) @ _f(w).T
        got = _f(o.linear(x, w))
        err = np.abs(got - ref)
        assert np.all(err <= 0.5 * _bf16_spacing(ref) * (1 + 1e-12)), f"max err {err.max()} for {(n, k, m)}"


def pin_linear_row_stride(o):
    """Rows read through a row stride larger than k: the padding (NaN) is never read."""
    rng = np.random.default_rng(14)
    x = bf16_bits(rng.standard_normal((6, 40)).astype(np.float32))
    pad = np.full((6, 56), 0x7FC0, dtype=np.uint16)
    pad[:, :40] = x
    w = bf16_bits(rng.standard_normal((9, 40)).astype(np.float32))
    assert np.array_equal(o.linear(pad, w), o.linear(x, w))


# ---------------------------------------------------------------------------
# RMSNorm (hidden_norm, k_norm, latent norm)
# ---------------------------------------------------------------------------

def pin_rmsnorm_unit_rms(o):
    """With weight 1 the output has RMS 1/sqrt(1 + eps/mean(x^2)) ~ 1 (up to bf16 rounding)."""
    rng = np.random.default_rng(21)
    for d, scale in ((128, 1.0), (512, 3.0), (4096, 0.05)):
        x = bf16_bits((rng.standard_normal((4, d)) * scale).astype(np.float32))
        y = _f(o.rmsnorm(x, bf16_bits(np.ones(d, np.float32)), 1e-6))
        xs = _f(x)
        rms = np.sqrt((y ** 2).mean(axis=1))
        want = 1.0 / np.sqrt(1.0 + 1e-6 / (xs ** 2).mean(axis=1))
        assert np.all(np.abs(rms - want) < 4e-3), (rms, want)


def pin_rmsnorm_scale_invariance(o):
    rng = np.random.default_rng(22)
    x = bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    w = bf16_bits((1 + 0.02 * rng.standard_normal(64)).astype(np.float32))
    x4 = bf16_bits(_f(x).astype(np.float32) * 4)             # exact: power-of-two scaling
    a, b = _f(o.rmsnorm(x, w, 0.0)), _f(o.rmsnorm(x4, w, 0.0))
    assert np.array_equal(a, b)


def pin_rmsnorm_constant(o):
    """A constant vector c maps to w*c/sqrt(c^2 + eps)."""
    for c in (0.5, -3.0, 1e-3):
        x = bf16_bits(np.full((1, 32), c, np.float32))
        w = bf16_bits(np.linspace(0.5, 1.5, 32).astype(np.float32))
        cb = _f(x)[0, 0]
        want = o.round_bf16(_f(w) * cb / math.sqrt(cb * cb + 1e-6))
        assert np.array_equal(o.rmsnorm(x, w, 1e-6)[0], want)


def pin_rmsnorm_vs_torch(o):
    """torch.nn.functional.rms_norm in float64 on the same values, within one bf16 spacing."""
    import torch
    rng = np.random.default_rng(23)
    x = bf16_bits(rng.standard_normal((6, 256)).astype(np.float32))
    w = bf16_bits((1 + 0.02 * rng.standard_normal(256)).astype(np.float32))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_f(x)), (256,), torch.from_numpy(_f(w)), eps=1e-6).numpy()
    got = _f(o.rmsnorm(x, w, 1e-6))
    assert np.all(np.abs(got - ref) <= 0.5 * _bf16_spacing(ref) * (1 + 1e-9))


# ---------------------------------------------------------------------------
# RoPE / YaRN cos/sin cache and the NeoX rotation
# ---------------------------------------------------------------------------

def pin_rope_inv_freq_closed_form(o):
    """theta=1e4, rot=8: inverse frequencies 1, 0.1, 0.01, 0.001."""
    inv, m = o.inv_freq(RopeSpec(theta=1e4, rot=8))
    assert np.allclose(inv, [1.0, 0.1, 0.01, 0.001], rtol=1e-14, atol=0) and m == 1.0


def pin_rope_cache_special_rows(o):
    rope = RopeSpec(theta=1e6, rot=64)
    cs = o.rope_cache(rope, 50)
    assert np.array_equal(cs[0, :32], np.ones(32, np.float32)) and np.array_equal(cs[0, 32:], np.zeros(32, np.float32))
    # dim 0 has inverse frequency 1: cos(p), sin(p) from the math library
    for p in (1, 7, 49):
        assert cs[p, 0] == np.float32(math.cos(p)) and cs[p, 32] == np.float32(math.sin(p))


def pin_rope_cache_long_positions(o):
    """Far into the context (positions 131071, 262144, 393216) every entry of the cache is
    m*cos(p*inv_i) / m*sin(p*inv_i) from an fp64 angle, rounded once to fp32: checked against Python's
    math.cos/math.sin of p*inv_i in fp64 (inv_i and m from inv_freq, which the YaRN pins fix), for plain
    RoPE and both YaRN specs of the workloads.  An angle formed in fp32 is off by up to half an fp32
    spacing of p*inv_i (about 4e-6 rad at 131 rad), hundreds of fp32 spacings of the value."""
    positions = (131071, 262144, 393216)
    for rope in (RopeSpec(theta=1e6, rot=128),
                 RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0),
                 RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0)):
        half = rope.rot // 2
        cs = o.rope_cache(rope, positions[-1] + 1)
        inv, m = o.inv_freq(rope)
        for p in positions:
            want = np.array([m * math.cos(p * f) for f in inv] + [m * math.sin(p * f) for f in inv],
                            dtype=np.float64)
            got = cs[p].astype(np.float64)
            tol = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
            bad = np.nonzero(np.abs(got - want) > tol)[0]
            assert bad.size == 0, (rope, p, int(bad[0]) % half, got[bad[0]], want[bad[0]])


def pin_rope_complex_rotation(o):
    """A NeoX pair (u_j, u_{j+h}) is the complex number u_j + i*u_{j+h}; RoPE multiplies it by exp(i*p*inv_j)."""
    rng = np.random.default_rng(31)
    rope = RopeSpec(theta=1e4, rot=16)
    cs = o.rope_cache(rope, 300)
    inv, _ = o.inv_freq(rope)
    u = bf16_bits(rng.standard_normal(16).astype(np.float32))
    for p in (0, 1, 5, 299):
        got = _f(o.rope_neox(u, cs[p]))
        z = (_f(u[:8]) + 1j * _f(u[8:])) * np.exp(1j * p * inv)
        ref = np.concatenate([z.real, z.imag])
        assert np.all(np.abs(got - ref) <= 0.5 * _bf16_spacing(ref) + 1e-6 * np.abs(ref) + 1e-7), (p, got, ref)


def pin_rope_norm_and_relative_position(o):
    """Rotation preserves norms and <R(p+d)q, R(k+d)k> = <R(p)q, R(k)k> (context and query rotate alike)."""
    rng = np.random.default_rng(32)
    rope = RopeSpec(theta=1e6, rot=128)
    cs = o.rope_cache(rope, 5000)
    q = bf16_bits(rng.standard_normal(128).astype(np.float32))
    k = bf16_bits(rng.standard_normal(128).astype(np.float32))
    nq = np.linalg.norm(_f(q))
    for p in (0, 3, 4000):
        assert abs(np.linalg.norm(_f(o.rope_neox(q, cs[p]))) - nq) < 1e-2 * nq
    base = _f(o.rope_neox(q, cs[10])) @ _f(o.rope_neox(k, cs[3]))
    for d in (1, 100, 4000):
        moved = _f(o.rope_neox(q, cs[10 + d])) @ _f(o.rope_neox(k, cs[3 + d]))
        assert abs(moved - base) < 0.05 * (1 + abs(base)), (d, moved, base)


def _recover_freq(cs_row1, half):
    """Angle of position 1 = the inverse frequency (valid while < pi)."""
    return np.arctan2(cs_row1[half:].astype(np.float64), cs_row1[:half].astype(np.float64))


def pin_yarn_factor_one_is_plain(o):
    plain = o.rope_cache(RopeSpec(theta=1e6, rot=64), 2000)
    yarn1 = o.rope_cache(RopeSpec(theta=1e6, rot=64, yarn=True, factor=1.0, orig_ctx=4096.0), 2000)
    d = np.abs(plain.view(np.int32).astype(np.int64) - yarn1.view(np.int32).astype(np.int64))
    assert d.max() <= 1


def pin_yarn_ramp_extremes(o):
    """Dims below the fast correction dim keep the original frequency, dims above the slow one are divided
    by the factor, dims in between lie strictly between (YaRN "NTK-by-parts")."""
    for rope in (RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0),
                 RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0)):
        half = rope.rot // 2
        plain, _ = o.inv_freq(RopeSpec(theta=rope.theta, rot=rope.rot))
        inv, _ = o.inv_freq(rope)
        ratio = inv / plain
        assert abs(ratio[0] - 1) < 1e-12 and abs(ratio[-1] - 1 / rope.factor) < 1e-12
        assert np.all(np.diff(ratio) <= 1e-15), "ramp must move monotonically from extrapolation to interpolation"
        inner = (ratio < 1 - 1e-12) & (ratio > 1 / rope.factor + 1e-12)
        assert inner.sum() >= 2
        # the cache holds the same frequencies: angle at position 1
        cs = o.rope_cache(rope, 2)
        _, m = o.inv_freq(rope)
        fr = _recover_freq(cs[1] / np.float32(m), half)
        assert np.allclose(fr, inv, rtol=1e-6, atol=1e-9)


def pin_yarn_correction_dims_meaning(o):
    """Recover lo/hi of the ramp from the interior dims; the dim at lo completes beta_fast turns over the
    original context, the dim at hi beta_slow turns (definition of the correction range)."""
    for rope in (RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0),
                 RopeSpec(theta=1e6, rot=128, yarn=True, factor=4.0, orig_ctx=32768.0)):
        plain, _ = o.inv_freq(RopeSpec(theta=rope.theta, rot=rope.rot))
        inv, _ = o.inv_freq(rope)
        ramp = (1 - inv / plain) / (1 - 1 / rope.factor)
        idx = np.nonzero((ramp > 1e-9) & (ramp < 1 - 1e-9))[0]
        i0, i1 = idx[0], idx[-1]
        slope = (ramp[i1] - ramp[i0]) / (i1 - i0)
        lo = i0 - ramp[i0] / slope
        hi = lo + 1 / slope
        turns = lambda dim: rope.orig_ctx * rope.theta ** (-2 * dim / rope.rot) / (2 * math.pi)
        assert abs(turns(lo) - rope.beta_fast) < 1e-6 * rope.beta_fast, (lo, turns(lo))
        assert abs(turns(hi) - rope.beta_slow) < 1e-6 * rope.beta_slow, (hi, turns(hi))


def pin_yarn_attention_factor(o):
    """Position 0: cos = m = 0.1*ln(s) + 1, sin = 0 (YaRN temperature)."""
    for s, want in ((40.0, 1.3688879454113936), (4.0, 1.1386294361119891)):
        cs = o.rope_cache(RopeSpec(theta=1e6, rot=64, yarn=True, factor=s, orig_ctx=4096.0), 1)
        assert np.all(cs[0, :32] == np.float32(want)) and np.all(cs[0, 32:] == 0)


def pin_yarn_truncate(o):
    """truncate=True floors/ceils the correction range: the recovered ramp ends are integers."""
    rope = RopeSpec(theta=1e6, rot=64, yarn=True, factor=40.0, orig_ctx=4096.0, truncate=True)
    plain, _ = o.inv_freq(RopeSpec(theta=1e6, rot=64))
    inv, _ = o.inv_freq(rope)
    ramp = (1 - inv / plain) / (1 - 1 / rope.factor)
    idx = np.nonzero((ramp > 1e-9) & (ramp < 1 - 1e-9))[0]
    slope = (ramp[idx[-1]] - ramp[idx[0]]) / (idx[-1] - idx[0])
    lo = idx[0] - ramp[idx[0]] / slope
    assert abs(lo - round(lo)) < 1e-9 and abs(1 / slope - round(1 / slope)) < 1e-9


# ---------------------------------------------------------------------------
# golden: a worked tiny RoPE example (tests/golden/rope_tiny.json)
# ---------------------------------------------------------------------------

def pin_golden_rope_tiny(o):
    with open(os.path.join(GOLDEN, "rope_tiny.json")) as fh:
        g = json.load(fh)
    rope = RopeSpec(theta=g["theta"], rot=g["rot"])
    cs = o.rope_cache(rope, g["pos"] + 1)
    u = bf16_bits(np.array(g["u"], np.float32))
    got = _f(o.rope_neox(u, cs[g["pos"]]))
    assert np.allclose(got, g["expected"], atol=g["atol"]), (got, g["expected"])


# ---------------------------------------------------------------------------
# k_norm + RoPE on the stacked projection, and the whole projection chain
# ---------------------------------------------------------------------------

def _tiny_geom(kind):
    if kind == GQA:
        return Geometry(kind=GQA, n_tgt=2, tgt_hidden=32, hidden=48, n_layers=2, n_kv_heads=2, head_dim=16,
                        latent_dim=0, rope_dim=16, eps=1e-6, page_size=4, width=3, block_size=4)
    return Geometry(kind=MLA, n_tgt=2, tgt_hidden=32, hidden=48, n_layers=2, n_kv_heads=1, head_dim=0,
                    latent_dim=32, rope_dim=8, eps=1e-6, page_size=4, width=3, block_size=4)


def _tiny_inputs(geom, seed):
    from dfkv_workloads import make_weights
    rng = np.random.default_rng(seed)
    B = 3
    N = B * geom.width
    x = bf16_bits(rng.standard_normal((N, geom.k_in)).astype(np.float32))
    w = make_weights(geom, rng)
    ctx = np.array([0, 5, 1000], np.int32)
    return x, w, ctx


def pin_norm_rope_structure(o):
    for kind in (GQA, MLA):
        geom = _tiny_geom(kind)
        rng = np.random.default_rng(41 + kind)
        N = 9
        y = bf16_bits(rng.standard_normal((N, geom.out_dim)).astype(np.float32))
        wk = bf16_bits((1 + 0.02 * rng.standard_normal((geom.n_layers, geom.knorm_dim))).astype(np.float32))
        ctx = np.array([0, 5, 1000], np.int32)
        rope = RopeSpec(theta=1e4, rot=geom.rope_dim)
        cs = o.rope_cache(rope, 600)                    # position 1000+ reads the last row (clamp)
        out = o.norm_rope(geom, y, wk, ctx, cs)
        for n in range(N):
            r, i = divmod(n, geom.width)
            p = min(int(ctx[r]) + i, cs.shape[0] - 1)
            for l in range(geom.n_layers):
                if kind == GQA:
                    base = l * geom.per_layer
                    hd, nkv = geom.head_dim, geom.n_kv_heads
                    v0 = base + nkv * hd
                    assert np.array_equal(out[n, v0:v0 + nkv * hd], y[n, v0:v0 + nkv * hd]), "V must be untouched"
                    for h in range(nkv):
                        seg = slice(base + h * hd, base + (h + 1) * hd)
                        u = o.rmsnorm(y[n:n + 1, seg], wk[l], geom.eps)[0]
                        assert np.array_equal(out[n, seg], o.rope_neox(u, cs[p]))
                        if p == 0:   # rotation at position 0 is the identity
                            assert np.array_equal(out[n, seg], u)
                else:
                    base = l * geom.per_layer
                    R = geom.latent_dim
                    lat = o.rmsnorm(y[n:n + 1, base:base + R], wk[l], geom.eps)[0]
                    assert np.array_equal(out[n, base:base + R], lat)
                    rp = y[n, base + R:base + R + geom.rope_dim]
                    assert np.array_equal(out[n, base + R:base + geom.per_layer], o.rope_neox(rp, cs[p]))


def pin_project_chain(o):
    """project() is fc -> hidden_norm -> stacked GEMM -> k_norm/RoPE, and rows are independent."""
    for kind in (GQA, MLA):
        geom = _tiny_geom(kind)
        x, w, ctx = _tiny_inputs(geom, 50 + kind)
        rope = RopeSpec(theta=1e4, rot=geom.rope_dim)
        cs = o.rope_cache(rope, 1100)
        res = o.project(geom, x, w["w_fc"], w["w_hnorm"], w["w_kv"], w["w_knorm"], ctx, cs)
        f = o.linear(x, w["w_fc"])
        g = o.rmsnorm(f, w["w_hnorm"], geom.eps)
        y = o.linear(g, w["w_kv"])
        kv = o.norm_rope(geom, y, w["w_knorm"], ctx, cs)
        for name, want in (("f", f), ("g", g), ("y", y), ("kv", kv)):
            assert np.array_equal(res[name], want), name
        sub = [7, 2, 4]
        part = o.project(geom, x, w["w_fc"], w["w_hnorm"], w["w_kv"], w["w_knorm"], ctx, cs, row_ids=sub)
        assert np.array_equal(part["kv"], kv[sub])


# ---------------------------------------------------------------------------
# bookkeeping: brute force against a position-first formulation
# ---------------------------------------------------------------------------

def _expected_writes_position_first(W, pg, ctx, n_acc, lim, dummy, row_valid, bt, num_pages):
    """Walk every pool slot (page, offset) and find the row, if any, that must land there."""
    B, cols = bt.shape
    want = {}
    for page in range(num_pages):
        for off in range(pg):
            for r in range(B):
                if dummy[r]:
                    continue
                for q in range(cols):
                    if bt[r, q] != page:
                        continue
                    p = q * pg + off
                    i = p - int(ctx[r])
                    if 0 <= i < W and i < n_acc[r] and 0 <= p < lim[r] and (row_valid is None or row_valid[r * W + i]):
                        assert (page * pg + off) not in want, "tables must be disjoint in the window"
                        want[page * pg + off] = r * W + i
    return want


def pin_bookkeeping_bruteforce(o):
    geom_base = dict(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8,
                     latent_dim=0, rope_dim=8, eps=1e-6)
    rng = np.random.default_rng(61)
    checked = 0
    for W, pg, cols in ((1, 1, 4), (2, 2, 3), (3, 4, 2), (4, 2, 4), (4, 4, 3)):
        geom = Geometry(page_size=pg, width=W, block_size=3, **geom_base)
        num_pages = 16
        for c, n, lim in itertools.product(range(0, 21, 3), range(0, W + 1), range(0, 17, 3)):
            for dummy in (0, 1):
                # one request under test plus a second one whose table is disjoint
                tbl = rng.permutation(num_pages)[:2 * cols].reshape(2, cols).astype(np.int32)
                neg = rng.random((2, cols)) < 0.25
                tbl[neg] = -1 - rng.integers(0, 3, size=int(neg.sum()))
                if rng.random() < 0.1:
                    tbl[0, :] = 99          # out-of-range pages
                rv = (rng.random(2 * W) < 0.8).astype(np.uint8) if rng.random() < 0.5 else None
                ctx = np.array([c, rng.integers(0, 12)], np.int32)
                na = np.array([n, rng.integers(0, W + 1)], np.int32)
                lm = np.array([lim, rng.integers(0, 16)], np.int32)
                dm = np.array([dummy, 0], np.uint8)
                acc = rng.integers(0, 1000, size=(2, W)).astype(np.int32)
                out = o.bookkeeping(geom, 2, ctx, na, lm, dm, rv, tbl, acc, W, 1, 777, num_pages)
                want = _expected_writes_position_first(W, pg, ctx, na, lm, dm, rv, tbl, num_pages)
                got = {int(out["slot"][row]): row for row in range(2 * W) if out["write_mask"][row]}
                assert got == want, (W, pg, c, n, lim, dummy, got, want)
                assert np.all(out["slot"][out["write_mask"] == 0] == -1)
                for r in range(2):
                    ctx_new = 0 if dm[r] else min(int(ctx[r]) + int(na[r]), int(lm[r]))
                    assert out["ctx_len"][r] == ctx_new
                    assert out["seq_len"][r] == ctx_new + 3
                    assert list(out["q_pos"][r]) == [ctx_new, ctx_new + 1, ctx_new + 2]
                    last = max(1, min(int(na[r]), W)) - 1
                    assert out["bonus"][r] == acc[r, last]
                    assert list(out["emb_ids"][r]) == [acc[r, last], 777, 777]
                    assert list(out["c_pos"][r]) == [int(ctx[r]) + i for i in range(W)]
                    if not dm[r] and rv is None and np.all((tbl[r] >= 0) & (tbl[r] < num_pages)):
                        span = min(int(na[r]), W, int(lm[r]) - int(ctx[r]), cols * pg - int(ctx[r]))
                        assert int(out["write_mask"][r * W:(r + 1) * W].sum()) == max(0, span)
                checked += 1
    assert checked > 1000


def pin_bookkeeping_strided_tokens(o):
    """The accepted-token tensor may be any strided view: transposed storage gives the same answers."""
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=4, width=4, block_size=5)
    rng = np.random.default_rng(62)
    B = 6
    tok = rng.integers(0, 5000, size=(B, 4)).astype(np.int32)
    ctx = rng.integers(0, 30, size=B).astype(np.int32)
    na = np.array([0, 1, 2, 3, 4, 4], np.int32)
    lim = np.full(B, 40, np.int32)
    dm = np.zeros(B, np.uint8)
    tbl = np.arange(B * 10, dtype=np.int32).reshape(B, 10)
    a = o.bookkeeping(geom, B, ctx, na, lim, dm, None, tbl, tok, 4, 1, 9, 64)
    b = o.bookkeeping(geom, B, ctx, na, lim, dm, None, tbl, np.ascontiguousarray(tok.T), 1, B, 9, 64)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert list(a["bonus"]) == [tok[0, 0], tok[1, 0], tok[2, 1], tok[3, 2], tok[4, 3], tok[5, 3]]


def pin_golden_bookkeeping(o):
    """A case worked by hand (tests/golden/bookkeeping_tiny.json)."""
    with open(os.path.join(GOLDEN, "bookkeeping_tiny.json")) as fh:
        g = json.load(fh)
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=g["page_size"], width=g["width"], block_size=g["block_size"])
    i = g["inputs"]
    rv = None if i["row_valid"] is None else np.array(i["row_valid"], np.uint8)
    out = o.bookkeeping(geom, len(i["ctx_len"]), np.array(i["ctx_len"], np.int32), np.array(i["n_acc"], np.int32),
                        np.array(i["alloc_limit"], np.int32), np.array(i["is_dummy"], np.uint8), rv,
                        np.array(i["block_table"], np.int32), np.array(i["accepted_tokens"], np.int32),
                        g["width"], 1, i["mask_token_id"], i["num_pages"])
    for k, v in g["expected"].items():
        assert np.array_equal(np.asarray(out[k]).reshape(-1), np.array(v).reshape(-1)), (k, out[k], v)


# ---------------------------------------------------------------------------
# block placement: the next draft block's own positions in the pages
# ---------------------------------------------------------------------------

def _expected_placement_position_first(bs, pg, ctx_new, lim, dummy, bt, num_pages):
    """Walk every table entry (column q, offset off) of each request and place the position it holds
    into the block when that position is one of ctx' .. ctx'+bs-1 inside the allocation."""
    B, cols = bt.shape
    want = np.full((B, bs), -1, np.int64)
    for r in range(B):
        if dummy[r]:
            continue
        for q in range(cols):
            page = int(bt[r, q])
            if not 0 <= page < num_pages:
                continue
            for off in range(pg):
                p = q * pg + off
                j = p - int(ctx_new[r])
                if 0 <= j < bs and p < lim[r]:
                    want[r, j] = page * pg + off
    return want


def pin_block_placement_bruteforce(o):
    geom_base = dict(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8,
                     latent_dim=0, rope_dim=8, eps=1e-6)
    rng = np.random.default_rng(63)
    checked = 0
    for W, pg, cols, bs in ((1, 1, 4, 1), (2, 2, 3, 3), (3, 4, 2, 5), (4, 2, 4, 2), (4, 4, 3, 7)):
        geom = Geometry(page_size=pg, width=W, block_size=bs, **geom_base)
        num_pages = 16
        for c, n, lim in itertools.product(range(0, 21, 3), range(0, W + 1), range(0, 17, 2)):
            for dummy in (0, 1):
                tbl = rng.permutation(num_pages)[:2 * cols].reshape(2, cols).astype(np.int32)
                neg = rng.random((2, cols)) < 0.25
                tbl[neg] = -1 - rng.integers(0, 3, size=int(neg.sum()))
                if rng.random() < 0.1:
                    tbl[0, :] = 99
                ctx = np.array([c, rng.integers(0, 12)], np.int32)
                na = np.array([n, rng.integers(0, W + 1)], np.int32)
                lm = np.array([lim, rng.integers(0, 16)], np.int32)
                dm = np.array([dummy, 0], np.uint8)
                acc = rng.integers(0, 1000, size=(2, W)).astype(np.int32)
                out = o.bookkeeping(geom, 2, ctx, na, lm, dm, None, tbl, acc, W, 1, 777, num_pages)
                want = _expected_placement_position_first(bs, pg, out["ctx_len"], lm, dm, tbl, num_pages)
                assert np.array_equal(out["block_slot"], want), (W, pg, c, n, lim, dummy, out["block_slot"], want)
                checked += 1
    assert checked > 1000


def pin_block_placement_matches_row_slots(o):
    """With nothing accepted the block starts at the pre-step context length, so its j-th position is the
    position of verify row j: when every row is accepted instead, row j's slot must equal the block's j-th
    placement (the row-slot formula is pinned by brute force above)."""
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=4, width=4, block_size=6)
    rng = np.random.default_rng(64)
    B, cols, P = 8, 6, 64
    for _ in range(40):
        tbl = rng.permutation(P)[:B * cols].reshape(B, cols).astype(np.int32)
        tbl[rng.random((B, cols)) < 0.2] = -1
        ctx = rng.integers(0, 20, size=B).astype(np.int32)
        lim = (ctx + rng.integers(0, 8, size=B)).astype(np.int32)
        dm = (rng.random(B) < 0.2).astype(np.uint8)
        acc = rng.integers(0, 1000, size=(B, 4)).astype(np.int32)
        none = o.bookkeeping(geom, B, ctx, np.zeros(B, np.int32), lim, dm, None, tbl, acc, 4, 1, 5, P)
        full = o.bookkeeping(geom, B, ctx, np.full(B, 4, np.int32), lim, dm, None, tbl, acc, 4, 1, 5, P)
        for r in range(B):
            for j in range(4):
                assert none["block_slot"][r, j] == full["slot"][r * 4 + j], (r, j)


def pin_golden_block_placement(o):
    """A case worked by hand (tests/golden/block_placement_tiny.json)."""
    with open(os.path.join(GOLDEN, "block_placement_tiny.json")) as fh:
        g = json.load(fh)
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=g["page_size"], width=g["width"], block_size=g["block_size"])
    i = g["inputs"]
    rv = None if i["row_valid"] is None else np.array(i["row_valid"], np.uint8)
    out = o.bookkeeping(geom, len(i["ctx_len"]), np.array(i["ctx_len"], np.int32), np.array(i["n_acc"], np.int32),
                        np.array(i["alloc_limit"], np.int32), np.array(i["is_dummy"], np.uint8), rv,
                        np.array(i["block_table"], np.int32), np.array(i["accepted_tokens"], np.int32),
                        g["width"], 1, i["mask_token_id"], i["num_pages"])
    assert np.array_equal(out["block_slot"], np.array(g["expected"]["block_slot"], np.int64)), out["block_slot"]


# ---------------------------------------------------------------------------
# draft-KV block-table decode
# ---------------------------------------------------------------------------

def pin_block_table_decode_position_walk(o):
    """Page counts from a walk over token positions (the distinct pages that positions 0..n-1 fall in,
    at most the table's width); each kept entry t is the page whose divisor-wide offset range holds the
    offset (t*d <= off < (t+1)*d); negative offsets and blocks past the count give -1."""
    rng = np.random.default_rng(65)
    for _ in range(300):
        B, mb = int(rng.integers(1, 6)), int(rng.integers(0, 7))
        pg, d = int(rng.integers(1, 9)), int(rng.integers(1, 5))
        off = rng.integers(-3, 40, size=(B, mb)).astype(np.int32)
        off[rng.random((B, mb)) < 0.3] = 0
        n_tok = rng.integers(-3, pg * (mb + 2) + 2, size=B).astype(np.int32)
        cnt, tbl = o.block_table_decode(off, mb, 1, B, mb, n_tok, pg, d)
        for r in range(B):
            walk = len({p // pg for p in range(max(0, int(n_tok[r])))})
            assert cnt[r] == min(walk, mb), (r, cnt[r], walk)
            for b in range(mb):
                t, v = int(tbl[r, b]), int(off[r, b])
                if b >= cnt[r] or v < 0:
                    assert t == -1, (r, b, t)
                else:
                    assert t >= 0 and t * d <= v < (t + 1) * d, (r, b, t, v, d)


def pin_block_table_decode_strided_views(o):
    """The offsets may be any strided view: row-major, transposed and every-other-column storage of one
    logical table decode identically."""
    rng = np.random.default_rng(66)
    B, mb = 7, 9
    off = rng.integers(-4, 50, size=(B, mb)).astype(np.int32)
    n_tok = rng.integers(0, 60, size=B).astype(np.int32)
    a = o.block_table_decode(off, mb, 1, B, mb, n_tok, 8, 3)
    b = o.block_table_decode(np.ascontiguousarray(off.T), 1, B, B, mb, n_tok, 8, 3)
    wide = np.full((B, 2 * mb), 12345, np.int32)
    wide[:, ::2] = off
    c = o.block_table_decode(wide, 2 * mb, 2, B, mb, n_tok, 8, 3)
    for x in (b, c):
        assert np.array_equal(a[0], x[0]) and np.array_equal(a[1], x[1])


def pin_golden_block_table_decode(o):
    """A case worked by hand (tests/golden/block_table_decode_tiny.json)."""
    with open(os.path.join(GOLDEN, "block_table_decode_tiny.json")) as fh:
        g = json.load(fh)
    i = g["inputs"]
    cnt, tbl = o.block_table_decode(np.array(i["offsets_storage"], np.int32), i["stride_req"], i["stride_blk"],
                                    g["n_reqs"], g["max_blocks"], np.array(i["n_tokens"], np.int32), g["page_size"],
                                    g["divisor"])
    assert np.array_equal(cnt, np.array(g["expected"]["page_count"])), cnt
    assert np.array_equal(tbl, np.array(g["expected"]["table"])), tbl


# ---------------------------------------------------------------------------
# strict acceptance of a uniform-width draft
# ---------------------------------------------------------------------------

def pin_strict_accept_prefix_search(o):
    """n_acc - 1 is the longest m such that the first m drafted tokens all equal the target's (found by trying
    every m from the longest down); the accepted tokens are the target's; 1 <= n_acc <= W."""
    rng = np.random.default_rng(67)
    for _ in range(400):
        B, W = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        tgt = rng.integers(0, 3, size=(B, W)).astype(np.int32)          # tiny vocabulary: many matches
        drf = rng.integers(0, 3, size=(B, max(W - 1, 0))).astype(np.int32)
        n_acc, acc = o.strict_accept(tgt, W, 1, drf, max(W - 1, 1), 1, B, W)
        assert np.array_equal(acc, tgt)
        for r in range(B):
            best = next(m for m in range(W - 1, -1, -1) if all(drf[r, i] == tgt[r, i] for i in range(m)))
            assert n_acc[r] == best + 1 and 1 <= n_acc[r] <= W, (r, n_acc[r], best)


def pin_golden_strict_accept(o):
    """A case worked by hand (tests/golden/strict_accept_tiny.json), target stored transposed."""
    with open(os.path.join(GOLDEN, "strict_accept_tiny.json")) as fh:
        g = json.load(fh)
    i, W, B = g["inputs"], g["width"], g["n_reqs"]
    n_acc, acc = o.strict_accept(np.array(i["target_storage"], np.int32), i["t_stride_req"], i["t_stride_tok"],
                                 np.array(i["draft"], np.int32), W - 1, 1, B, W)
    assert np.array_equal(n_acc, np.array(g["expected"]["n_acc"])), n_acc
    assert np.array_equal(acc, np.array(g["expected"]["accepted"])), acc


def pin_strict_accept_feeds_bookkeeping(o):
    """Acceptance then bookkeeping: the bonus token is the target's token after the last accepted draft
    token, i.e. target[r][n_acc - 1]."""
    rng = np.random.default_rng(68)
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=4, width=5, block_size=3)
    B, W = 9, 5
    tgt = rng.integers(0, 2, size=(B, W)).astype(np.int32)
    drf = np.where(rng.random((B, W - 1)) < 0.7, tgt[:, :W - 1], 1 - tgt[:, :W - 1]).astype(np.int32)
    n_acc, acc = o.strict_accept(tgt, W, 1, drf, W - 1, 1, B, W)
    tbl = np.arange(B * 4, dtype=np.int32).reshape(B, 4)
    out = o.bookkeeping(geom, B, np.zeros(B, np.int32), n_acc, np.full(B, 16, np.int32), np.zeros(B, np.uint8),
                        None, tbl, acc, W, 1, 77, 64)
    for r in range(B):
        first_miss = next((i for i in range(W - 1) if drf[r, i] != tgt[r, i]), W - 1)
        assert out["bonus"][r] == tgt[r, first_miss]
        assert out["ctx_len"][r] == n_acc[r]


# ---------------------------------------------------------------------------
# prefill-shaped (ragged) rows: destinations
# ---------------------------------------------------------------------------

def pin_row_slots_position_first(o):
    """Walk every table entry of every request and find the rows that must land in each of its slots."""
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=4, width=1, block_size=1)
    rng = np.random.default_rng(69)
    for _ in range(200):
        B, cols, P = int(rng.integers(1, 5)), int(rng.integers(1, 5)), 24
        tbl = rng.permutation(P)[:B * cols].reshape(B, cols).astype(np.int32)
        tbl[rng.random((B, cols)) < 0.2] = -1
        if rng.random() < 0.2:
            tbl[0, 0] = P                                  # one past the last page
        lim = rng.integers(0, cols * 4 + 3, size=B).astype(np.int32)
        n = int(rng.integers(1, 30))
        rq = rng.integers(-1, B + 1, size=n).astype(np.int32)
        rp = rng.integers(-2, cols * 4 + 4, size=n).astype(np.int32)
        slot, wm = o.row_slots(geom, rq, rp, B, lim, tbl, P)
        want = np.full(n, -1, np.int64)
        for r in range(B):
            for q in range(cols):
                page = int(tbl[r, q])
                if not 0 <= page < P:
                    continue
                for off in range(4):
                    p = q * 4 + off
                    if p >= lim[r]:
                        continue
                    for row in range(n):
                        if rq[row] == r and rp[row] == p:
                            want[row] = page * 4 + off
        assert np.array_equal(slot, want), (slot, want)
        assert np.array_equal(wm, (want >= 0).astype(np.uint8))


def pin_row_slots_match_uniform_bookkeeping(o):
    """A uniform batch with every row accepted, written row by row, gets the bookkeeping's slots."""
    geom = Geometry(kind=GQA, n_tgt=1, tgt_hidden=8, hidden=8, n_layers=1, n_kv_heads=1, head_dim=8, latent_dim=0,
                    rope_dim=8, eps=1e-6, page_size=4, width=3, block_size=2)
    rng = np.random.default_rng(70)
    B, W, P = 8, 3, 64
    tbl = rng.permutation(P)[:B * 5].reshape(B, 5).astype(np.int32)
    tbl[rng.random((B, 5)) < 0.2] = -1
    ctx = rng.integers(0, 18, size=B).astype(np.int32)
    lim = (ctx + rng.integers(0, 5, size=B)).astype(np.int32)
    acc = np.zeros((B, W), np.int32)
    bk = o.bookkeeping(geom, B, ctx, np.full(B, W, np.int32), lim, np.zeros(B, np.uint8), None, tbl, acc, W, 1, 1, P)
    rq = np.repeat(np.arange(B, dtype=np.int32), W)
    rp = (np.repeat(ctx, W) + np.tile(np.arange(W, dtype=np.int32), B)).astype(np.int32)
    slot, wm = o.row_slots(geom, rq, rp, B, lim, tbl, P)
    assert np.array_equal(slot, bk["slot"]) and np.array_equal(wm, bk["write_mask"])


# ---------------------------------------------------------------------------
# paged store
# ---------------------------------------------------------------------------

def pin_store_pool(o):
    """Random-byte pool: only destinations change; each holds the right row, layer, K/V half and head."""
    rng = np.random.default_rng(71)
    for kind in (GQA, MLA):
        geom = _tiny_geom(kind)
        L, pg = geom.n_layers, geom.page_size
        P = 10
        N = 9
        kv = rng.integers(0, 65536, size=(N, geom.out_dim)).astype(np.uint16)
        wm = (rng.random(N) < 0.6).astype(np.uint8)
        slots = rng.permutation(P * pg)[:N].astype(np.int64)
        slot = np.where(wm == 1, slots, -1)
        if kind == GQA:
            nkv, hd = geom.n_kv_heads, geom.head_dim
            shape = (P, pg, nkv, hd)
        else:
            shape = (P, pg, geom.per_layer)
        pk = [rng.integers(0, 65536, size=shape).astype(np.uint16) for _ in range(L)]
        pv = [rng.integers(0, 65536, size=shape).astype(np.uint16) for _ in range(L)] if kind == GQA else None
        before_k = [p.copy() for p in pk]
        before_v = [p.copy() for p in pv] if pv else None
        sp, ss = int(np.prod(shape[1:])), int(np.prod(shape[2:]))
        sh = geom.head_dim if kind == GQA else 0
        o.store(geom, kv, slot, wm, pk, pv, sp, ss, sh)
        touched = np.zeros((P, pg), bool)
        for row in np.nonzero(wm)[0]:
            page, off = divmod(int(slot[row]), pg)
            touched[page, off] = True
            for l in range(L):
                lay = kv[row].reshape(L, -1)[l]
                if kind == GQA:
                    k_part = lay.reshape(2, nkv, hd)[0]
                    v_part = lay.reshape(2, nkv, hd)[1]
                    assert np.array_equal(pk[l][page, off], k_part) and np.array_equal(pv[l][page, off], v_part)
                else:
                    assert np.array_equal(pk[l][page, off], lay)
        for l in range(L):
            assert np.array_equal(pk[l][~touched], before_k[l][~touched])
            if pv:
                assert np.array_equal(pv[l][~touched], before_v[l][~touched])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
