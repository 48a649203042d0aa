"""Pins of the tree-row append oracle against facts fixed by arithmetic, not by the oracle itself:
hand-worked bf16 roundings (ties to even, no double rounding), an independent bit-level rounding
of float32 values, RMSNorm closed forms and invariances, the rotation as a complex product, its
sign convention on unit vectors, inverse rotation, depths against an ancestor count, and
planted-mistake checks (mutants of the oracle, on the CPU, that the pins must catch)."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import append as A


def test_bf16_rounding_hand_values():
    cases = [
        (1.0, 0x3F80),
        (1 + 2 ** -8, 0x3F80),               # tie: to the even significand (1.0)
        (1 + 3 * 2 ** -8, 0x3F82),           # tie between 1 + 2^-7 and 1 + 2^-6: to the even one
        (1 + 2 ** -8 + 2 ** -30, 0x3F81),    # just above the tie; rounding to fp32 first gives 0x3F80
        (-1.5, 0xBFC0),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2 ** -130, 0x0008),                 # subnormal: 8 x 2^-133
        (3.4e38, 0x7F80),                    # past the largest bf16 + half a spacing: infinity
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),  # the largest finite bf16
        (3.38e38, 0x7F7E),                   # 1.98654 x 2^127: significand 126.28/128 -> 126
        (float("nan"), 0x7FC0),
    ]
    got = A.bf16_round_bits(np.array([v for v, _ in cases]))
    assert [int(g) for g in got] == [b for _, b in cases]


def test_bf16_rounding_matches_bit_trick_on_float32_values():
    """For values already in float32 there is one rounding either way: the oracle must agree with
    the integer round-to-nearest-even on the float32 bits (synth's independent implementation)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    # exact ties in float32: significand bit pattern ...1000 0000 0000 0000 below bf16 precision
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32) * np.float32(1.0)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(A.bf16_round_bits(x.astype(np.float64)), synth.f32_to_bf16_bits(x))


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(512)
    y = A.rms_norm(x, np.ones(512), 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-12                       # unit RMS
    assert np.allclose(A.rms_norm(7.5 * x, np.ones(512), 0.0), y, rtol=1e-13)  # scale invariant
    assert np.allclose(y, x / (np.linalg.norm(x) / math.sqrt(512)), rtol=1e-13)
    a, eps = 0.3, 1e-2                                             # constant row: a / sqrt(a^2 + eps)
    assert np.allclose(A.rms_norm(np.full(512, a), np.ones(512), eps), a / math.sqrt(a * a + eps), rtol=1e-14)
    w = np.zeros(512)
    w[17] = -2.0                                                   # the weight multiplies elementwise
    yw = A.rms_norm(x, w, 0.0)
    assert np.count_nonzero(yw) == 1 and yw[17] == pytest.approx(-2.0 * y[17], rel=1e-14)


def test_rope_unit_vectors_fix_pairing_and_signs():
    c = np.linspace(0.1, 0.9, 32)
    s = np.sqrt(1 - c * c)
    for j in (0, 5, 31):
        e = np.zeros(64)
        e[j] = 1.0
        out = A.rope_neox(e, c, s)
        expect = np.zeros(64)
        expect[j], expect[j + 32] = c[j], s[j]
        assert np.allclose(out, expect, atol=0)
        e = np.zeros(64)
        e[j + 32] = 1.0
        out = A.rope_neox(e, c, s)
        expect = np.zeros(64)
        expect[j], expect[j + 32] = -s[j], c[j]
        assert np.allclose(out, expect, atol=0)


def test_rope_is_a_complex_rotation_and_inverts():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(64)
    phi = rng.uniform(-math.pi, math.pi, 32)
    c, s = np.cos(phi), np.sin(phi)
    out = A.rope_neox(x, c, s)
    z = (x[:32] + 1j * x[32:]) * np.exp(1j * phi)
    assert np.allclose(out[:32], z.real, rtol=1e-13, atol=1e-15)
    assert np.allclose(out[32:], z.imag, rtol=1e-13, atol=1e-15)
    assert np.allclose(np.hypot(out[:32], out[32:]), np.hypot(x[:32], x[32:]), rtol=1e-13)
    assert np.allclose(A.rope_neox(out, c, -s), x, rtol=1e-12, atol=1e-14)


def test_depths_against_ancestor_count():
    assert list(A.tree_depths(np.arange(-1, 9))) == list(range(10))  # chain
    assert list(A.tree_depths(np.array([-1, 0, 0, 0]))) == [0, 1, 1, 1]  # star
    for seed in range(20):
        parents = synth.sample_parents(synth.rng_for(seed, 0, synth.TAG_PARENTS), 33)
        anc = oracle.ancestor_or_self(parents)
        assert np.array_equal(A.tree_depths(parents), anc.sum(axis=1) - 1)
    for bad in (np.array([0, 0]), np.array([-1, 1]), np.array([-1, 0, 3, 1])):
        with pytest.raises(ValueError):
            A.tree_depths(bad)


def rope_tables(rows, base=10000.0):
    inv = base ** (-np.arange(32) / 32.0)
    ang = np.arange(rows)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def test_append_writes_only_the_tree_block():
    rng = np.random.default_rng(6)
    s_count, q, rows = 3, 9, 40
    ckv = rng.integers(0, 65536, (s_count, rows, 512)).astype(np.uint16)
    kpe = rng.integers(0, 65536, (s_count, rows, 64)).astype(np.uint16)
    kv = rng.standard_normal((s_count, q, 576)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 512)
    cos, sin = rope_tables(64)
    parents = np.stack([synth.sample_parents(synth.rng_for(7, s, synth.TAG_PARENTS), q) for s in range(s_count)])
    prefixes = [0, 13, rows - q]
    nc, nk = A.append_tree_kv(ckv, kpe, kv, w, 1e-6, cos, sin, prefixes, parents)
    for s, p in enumerate(prefixes):
        keep = np.ones(rows, bool)
        keep[p:p + q] = False
        assert np.array_equal(nc[s, keep], ckv[s, keep]) and np.array_equal(nk[s, keep], kpe[s, keep])
        rc, rk = A.tree_rows(kv[s], w, 1e-6, cos, sin, p, parents[s])
        assert np.array_equal(nc[s, p:p + q], rc) and np.array_equal(nk[s, p:p + q], rk)
    with pytest.raises(ValueError):
        A.append_tree_kv(ckv, kpe, kv, w, 1e-6, cos, sin, [0, 0, rows - q + 1], parents)


def test_positions_follow_depth():
    """A table whose rotation angle encodes the position: the rotated unit vector reveals the
    position used for every node (P + depth), sibling nodes sharing one."""
    q, p = 6, 20
    parents = np.array([-1, 0, 0, 1, 3, 2])
    rows = 64
    ang = np.arange(rows) * 0.01
    cos = np.repeat(np.cos(ang)[:, None], 32, axis=1)
    sin = np.repeat(np.sin(ang)[:, None], 32, axis=1)
    kv = np.zeros((q, 576), np.float32)
    kv[:, :512] = 1.0
    kv[:, 512] = 1.0                                  # e_0 of the rotary part
    _, kpe = A.tree_rows(kv, np.ones(512), 0.0, cos, sin, p, parents)
    got = oracle.bf16_bits_to_f64(kpe)
    for i, d in enumerate([0, 1, 1, 2, 3, 2]):
        assert got[i, 0] == pytest.approx(math.cos((p + d) * 0.01), abs=4e-3)
        assert got[i, 32] == pytest.approx(math.sin((p + d) * 0.01), abs=2e-3)


def test_rows_are_rounded_results():
    """Each stored value is the bf16 rounding of the fp64 result: within half a bf16 spacing."""
    rng = np.random.default_rng(8)
    kv = rng.standard_normal((5, 576)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 512)
    cos, sin = rope_tables(32)
    parents = np.array([-1, 0, 1, 1, 0])
    ckv, kpe = A.tree_rows(kv, w, 1e-6, cos, sin, 3, parents)
    exact = np.stack([A.rms_norm(kv[i, :512], w, 1e-6) for i in range(5)])
    got = oracle.bf16_bits_to_f64(ckv)
    spacing = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert (np.abs(got - exact) <= spacing / 2 + 1e-300).all()


# --- planted mistakes: each mutant of the oracle must fail a pin above --------------------------

def mutant_rope_sign(x, c, s):
    x = np.asarray(x, dtype=np.float64)
    lo, hi = x[:32], x[32:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s])


def mutant_rope_interleaved(x, c, s):
    x = np.asarray(x, dtype=np.float64)
    ev, od = x[0::2], x[1::2]
    out = np.empty(64)
    out[0::2], out[1::2] = ev * c - od * s, od * c + ev * s
    return out


def mutant_rms_no_mean(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / math.sqrt(float(np.sum(x * x)) + eps) * w


def mutant_round_via_f32(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float64).astype(np.float32))


@pytest.mark.parametrize("name,mutant,pin", [
    ("rope_neox", mutant_rope_sign, test_rope_unit_vectors_fix_pairing_and_signs),
    ("rope_neox", mutant_rope_interleaved, test_rope_unit_vectors_fix_pairing_and_signs),
    ("rms_norm", mutant_rms_no_mean, test_rms_norm_closed_forms),
    ("bf16_round_bits", mutant_round_via_f32, test_bf16_rounding_hand_values),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant, pin):
    monkeypatch.setattr(A, name, mutant)
    with pytest.raises(AssertionError):
        pin()
