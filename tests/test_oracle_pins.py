"""Pins of the oracle's compressor, RoPE and RMSNorm against facts fixed by the
pages and by mathematics (no GPU).  The oracle is never compared with itself
here: each check is a printed value, a closed form, an invariant, an
independent formulation or a brute-force loop."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import csa
from tests.conftest import read_golden


def _floats(vals):
    return np.array([float(v) for v in vals], dtype=np.float64)


# ---------------------------------------------------------------------------
# The worked pooled scalar 7.4
# ---------------------------------------------------------------------------
def test_pooled_scalar_7_4_pool():
    g = read_golden("pooled_scalar.txt")
    gates = np.concatenate([_floats(g["prev_gates"]), _floats(g["cur_gates"])])[:, None]
    vals = np.concatenate([_floats(g["prev_values"]), _floats(g["cur_values"])])[:, None]
    got = oracle.pool(gates, vals)[0]
    assert got == pytest.approx(float(g["expected"][0]), abs=1e-12)
    assert f"{got:.6f}" == g["printed"][0]


def test_pooled_scalar_7_4_through_compress_entry():
    """Same value through the entry builder of entry 0 (the previous group of
    entry 0 does not exist, so no row before token 0 is ever read)."""
    g = read_golden("pooled_scalar.txt")
    r = int(g["ratio"][0])
    cur_g, cur_v = _floats(g["cur_gates"]), _floats(g["cur_values"])
    prev, cur = csa.entry_candidates(0, r, int(g["overlap"][0]))
    assert prev == [] and cur == [0, 1, 2, 3]
    # a second channel keeps the RMS of the pooled vector away from zero;
    # the pre-norm value of channel 0 is recovered from the normalised output
    kv = np.stack([cur_v, np.ones(r)], axis=1)
    gate = np.stack([cur_g, np.zeros(r)], axis=1)
    y = csa.compress_entry(0, kv, gate, kv, gate, np.ones(2), r, 1, 0, 10000.0, 0.0)
    pre = np.array([7.4, 1.0])
    assert np.allclose(y, pre / np.sqrt(np.mean(pre ** 2)), rtol=0, atol=1e-12)


def _entry_order_case():
    g = read_golden("entry_order.txt")
    D, r, e = int(g["D"][0]), int(g["ratio"][0]), int(g["entry"][0])
    gates1 = _floats(g["gates"])
    u, signs = _floats(g["u"]), _floats(g["signs"])
    kv = u[:, None] * signs[None, :]                  # token j: (u_j, u_j, -u_j, u_j)
    gate = np.repeat(gates1[:, None], D, axis=1)      # the same gates on every channel
    return g, D, r, e, kv, gate


def test_entry_pool_norm_gain_rope_order_hand_worked():
    """Pooling, then RMSNorm with a non-uniform gain (eps inside the root),
    then RoPE of the trailing pair at position e*r: a hand-worked entry whose
    rotated pair has unequal gains, so rotating before the gain-scaled norm
    (or at another position, or on the leading pair) gives other numbers."""
    g, D, r, e, kv, gate = _entry_order_case()
    gamma, eps = _floats(g["gamma"]), float(g["eps"][0])
    rd, base = int(g["rope_dim"][0]), float(g["rope_base"][0])
    want = _floats(g["expected"])
    prev, cur = csa.entry_candidates(e, r, int(g["overlap"][0]))
    assert prev == [0, 1] and cur == [2, 3]
    got = csa.compress_entry(e, kv, gate, kv, gate, gamma, r, 1, rd, base, eps)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    got2 = csa.entry_from_rows(e, r, gate, kv, gamma, rd, base, eps)
    assert np.allclose(got2, want, rtol=0, atol=1e-12)
    # the streaming compressor emits the same entry when token 3 completes group 1
    sc = csa.StreamingCompressor(gamma, r, 1, rd, base, eps)
    emitted = [sc.push(t, kv[t], gate[t]) for t in range(4)]
    assert emitted == [None, 0, None, 1]
    assert np.allclose(sc.cache[1], want, rtol=0, atol=1e-12)


def test_minus_inf_candidates_are_never_read():
    """A -inf gate excludes its value even when that value is NaN or inf."""
    gates = np.array([[-np.inf], [-np.inf], [0.0], [0.0]])
    vals = np.array([[np.nan], [np.inf], [2.0], [4.0]])
    assert oracle.pool(gates, vals)[0] == 3.0


def test_equal_gates_give_the_arithmetic_mean():
    """"Lab tổng hợp DeepSeek-V4.1-Flash", section "6 Thuật ngữ": a latent
    averages r consecutive tokens, the equal-gate case of softmax pooling."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((8, 5))
    g = np.full((8, 5), 0.37)
    assert np.allclose(oracle.pool(g, v), v.mean(axis=0), rtol=0, atol=1e-14)


def test_pool_is_per_channel_and_convex_and_shift_invariant():
    rng = np.random.default_rng(4)
    g = rng.standard_normal((8, 6)) * 3
    v = rng.standard_normal((8, 6))
    y = oracle.pool(g, v)
    assert np.all(y <= v.max(axis=0) + 1e-15) and np.all(y >= v.min(axis=0) - 1e-15)
    # a per-channel constant added to the gates changes nothing
    assert np.allclose(oracle.pool(g + rng.standard_normal(6), v), y, atol=1e-13)
    # channels do not interact: permuting channels permutes the result
    perm = rng.permutation(6)
    assert np.allclose(oracle.pool(g[:, perm], v[:, perm]), y[perm], atol=1e-15)
    # a dominant gate selects its value exactly
    g2 = g.copy()
    g2[5, :] = 1e4
    assert np.allclose(oracle.pool(g2, v), v[5], atol=1e-12)


def test_pool_matches_scalar_brute_force():
    rng = np.random.default_rng(5)
    g = rng.standard_normal((6, 3))
    v = rng.standard_normal((6, 3))
    g[:2, 1] = -np.inf
    for c in range(3):
        num = den = 0.0
        for j in range(6):
            if g[j, c] == -np.inf:
                continue
            e = math.exp(g[j, c])
            num += e * v[j, c]
            den += e
        assert oracle.pool(g, v)[c] == pytest.approx(num / den, abs=1e-14)


def test_overlap_candidate_lists():
    assert csa.entry_candidates(0, 4, 1) == ([], [0, 1, 2, 3])
    assert csa.entry_candidates(2, 4, 1) == ([4, 5, 6, 7], [8, 9, 10, 11])
    assert csa.entry_candidates(2, 4, 0) == ([], [8, 9, 10, 11])
    assert csa.entry_candidates(1, 128, 0) == ([], list(range(128, 256)))


# ---------------------------------------------------------------------------
# RMSNorm and RoPE
# ---------------------------------------------------------------------------
def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((4, 64)) * 7
    out = oracle.rms_norm(y, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(oracle.rms_norm(3.5 * y, np.ones(64), 0.0), out, atol=1e-14)
    gamma = rng.standard_normal(64)
    assert np.allclose(oracle.rms_norm(y, gamma, 0.0), out * gamma, atol=1e-14)
    # eps enters under the root: a zero row stays zero, a tiny row is damped
    assert np.all(oracle.rms_norm(np.zeros(8), np.ones(8), 1e-6) == 0)


def test_rope_matches_complex_rotation():
    """Independent formulation: pair (2i, 2i+1) as the complex number
    x_2i + j x_2i+1 multiplied by exp(j * pos * base^(-2i/rope_dim))."""
    rng = np.random.default_rng(7)
    d, rd, pos, base = 32, 8, 13, 10000.0
    x = rng.standard_normal(d)
    z = x[d - rd::2] + 1j * x[d - rd + 1::2]
    z = z * np.exp(1j * pos * base ** (-np.arange(rd // 2) * 2.0 / rd))
    want = x.copy()
    want[d - rd::2], want[d - rd + 1::2] = z.real, z.imag
    assert np.allclose(oracle.rope(x, pos, rd, base), want, atol=1e-14)


def test_rope_only_touches_the_trailing_slice_and_is_invertible():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 512))
    pos = np.array([0, 1, 1000, 65535, 1048575])
    y = oracle.rope(x, pos, 64)
    assert np.array_equal(y[:, :448], x[:, :448])
    assert np.array_equal(y[0], x[0])                       # position 0: identity
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    assert np.allclose(oracle.rope(y, pos, 64, inverse=True), x, atol=1e-12)
    assert np.array_equal(oracle.rope(x, pos, 0), x)


def test_rope_relative_position_property():
    rng = np.random.default_rng(9)
    a, b = rng.standard_normal(64), rng.standard_normal(64)
    d1 = oracle.rope(a, 1000, 64) @ oracle.rope(b, 990, 64)
    d2 = oracle.rope(a, 10, 64) @ oracle.rope(b, 0, 64)
    assert d1 == pytest.approx(d2, abs=1e-10)


def test_rope_large_position_angle_in_float64():
    """At p ~ 1e6 the angle of the fastest pair is reduced exactly in fp64:
    cos/sin of p * 1 rad, compared with math.cos/sin."""
    x = np.zeros(64)
    x[0] = 1.0
    y = oracle.rope(x, 1048575, 64)
    assert y[0] == pytest.approx(math.cos(1048575.0), abs=1e-12)
    assert y[1] == pytest.approx(math.sin(1048575.0), abs=1e-12)


# ---------------------------------------------------------------------------
# bfloat16 storage rounding
# ---------------------------------------------------------------------------
def test_round_bf16_known_values():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing in [1, 2)
    assert oracle.round_bf16(one) == one
    assert oracle.round_bf16(one + ulp / 2) == one                 # tie -> even (1.0)
    assert oracle.round_bf16(one + 3 * ulp / 2) == one + 2 * ulp   # tie -> even (1 + 2 ulp)
    assert oracle.round_bf16(one + ulp * 0.51) == one + ulp
    assert oracle.round_bf16(-3.0) == -3.0
    assert oracle.round_bf16(0.0) == 0.0


def test_round_bf16_matches_torch_conversion():
    """Library routine: torch's float32 -> bfloat16 conversion (nearest even)."""
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        np.float32(1.0) + np.arange(-300, 300) * np.float32(2.0 ** -16)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x), want)
