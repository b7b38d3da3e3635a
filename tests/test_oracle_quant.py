"""Pins of the oracle quantizer (CPU only).

What fixes it, independently of its own code:
* the tutorial's affine worked example (tests/golden/affine_example.txt);
* MinMax (gamma = beta = 1, the LWC equation's special case): the grid spans
  [min, max], no element is clipped, every element lands on its nearest grid
  point, both code endpoints are used;
* brute force over tiny rows: each code is the nearest admissible integer found
  by enumeration (ties to even), including constructed exact .5 ties;
* invariants: codes in [0, 2^N - 1], dequantized values on the grid
  {(k - z) h}, |x_hat - x| <= h / 2 inside the clipping range, sigma in (0, 1).
"""
import itertools
import os

import numpy as np
import pytest

from oracle import quant

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32


def _golden(name):
    d = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = [float(t) for t in v.split()]
    return d


def test_worked_affine_example():
    g = _golden("affine_example.txt")
    row = np.array([g["row"]], dtype=F32)
    nbits = int(g["nbits"][0])
    st = quant.quantize_rows(row, F32(1), F32(1), nbits)
    offset = -int(g["signed_qmin"][0])
    expect_codes = np.array(g["signed_codes"], dtype=np.int64) + offset
    assert st.codes[0].tolist() == expect_codes.tolist()
    # step h is the reciprocal of the tutorial's scale, z its zero point + offset
    assert st.h[0] == F32(1.0 / g["signed_scale"][0])
    assert st.z[0] == g["signed_zero_point"][0] + offset
    # the grid endpoints are exactly min and max, so dequantization is exact
    assert st.xhat[0].tolist() == g["row"]


def _nearest_code(u, z, Q):
    """Enumerate k in [0, Q]; nearest to u + z, ties to the even (k - z)."""
    best, bestd = None, None
    for k in range(int(Q) + 1):
        d = abs((k - z) - u)
        if bestd is None or d < bestd or (d == bestd and (k - z) % 2 == 0):
            best, bestd = k, d
    return best


@pytest.mark.parametrize("nbits", [2, 3, 4, 8])
def test_minmax_special_case(nbits):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 257)) * 0.02).astype(F32)
    one = quant.sigmoid32(np.full(64, 30.0, F32))
    assert np.all(one == F32(1.0))
    st = quant.quantize_rows(x, one, one, nbits)
    Q = 2 ** nbits - 1
    h = st.h.astype(np.float64)
    lo = (0 - st.z) * h
    hi = (Q - st.z) * h
    mn, mx = x.min(1).astype(np.float64), x.max(1).astype(np.float64)
    # grid endpoints within half a step (rounding of z) of min and max
    assert np.all(np.abs(lo - mn) <= h / 2 * (1 + 1e-6))
    assert np.all(np.abs(hi - mx) <= h / 2 * (1 + 1e-6))
    # both endpoints are used on rows with min < 0 < max
    assert np.all(st.codes.min(1) == 0) and np.all(st.codes.max(1) == Q)
    # no clipping: every element within half a step of its dequantized value
    err = np.abs(st.xhat.astype(np.float64) - x)
    assert np.all(err <= h[:, None] / 2 * (1 + 1e-5) + 1e-12)
    # every code is the nearest admissible grid point (sampled elements)
    for r, c in itertools.product(range(0, 64, 9), range(0, 257, 31)):
        assert st.codes[r, c] == _nearest_code(float(st.u[r, c]), float(st.z[r]), Q)


def test_brute_force_tiny_rows():
    vals = [-2.0, -1.0, -0.5, 0.0, 0.25, 0.5, 1.0, 1.5, 3.0]
    gb = [F32(1.0), F32(0.75), F32(0.5)]
    n = 0
    for nbits in (2, 3, 4):
        Q = 2 ** nbits - 1
        for L in (1, 2, 3, 4):
            for row in itertools.product(vals, repeat=L):
                if L == 4 and (row[0] > row[1] or n % 3):
                    n += 1
                    continue
                x = np.array([row], dtype=F32)
                for g_, b_ in itertools.product(gb, gb):
                    st = quant.quantize_rows(x, g_, b_, nbits)
                    # h and z from their definitions, in float32
                    M, m = F32(max(row)), F32(min(row))
                    h = (g_ * M - b_ * m) / F32(Q)
                    h = max(h, F32(1e-8))
                    assert st.h[0] == h
                    assert st.z[0] == -np.rint((b_ * m) / h)
                    for j in range(L):
                        u = F32(row[j]) / h
                        k = _nearest_code(float(u), float(st.z[0]), Q)
                        assert st.codes[0, j] == k, (row, nbits, g_, b_, j)
                        assert 0 <= k <= Q
                    n += 1
    assert n > 1000


def test_constructed_ties_round_to_even():
    # h = 1, z = 1 for [-1, ..., 2] at 2 bits: u = 0.5 -> 0, 1.5 -> 2 (even)
    x = np.array([[-1.0, 0.5, 1.5, 2.0]], dtype=F32)
    st = quant.quantize_rows(x, F32(1), F32(1), 2)
    assert st.h[0] == 1.0 and st.z[0] == 1.0
    assert st.codes[0].tolist() == [0, 1, 3, 3]
    # tie on z itself: beta*min/h = -2.5 -> rint -2 -> z = 2
    x = np.array([[-2.5, 0.0, 2.5]], dtype=F32)
    st = quant.quantize_rows(x, F32(1), F32(1), 1)  # Q = 1, h = 5
    assert st.h[0] == 5.0
    assert st.z[0] == 0.0   # rint(-0.5) = -0 -> z = 0


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_invariants_with_clipping(nbits):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((128, 300)) * 0.02).astype(F32)
    a = rng.uniform(-2, 6, size=128).astype(F32)
    b = rng.uniform(-2, 6, size=128).astype(F32)
    g_, b_ = quant.sigmoid32(a), quant.sigmoid32(b)
    assert np.all((g_ > 0) & (g_ < 1)) and np.all((b_ > 0) & (b_ < 1))
    st = quant.quantize_rows(x, g_, b_, nbits)
    Q = 2 ** nbits - 1
    assert st.codes.min() >= 0 and st.codes.max() <= Q
    h = st.h.astype(np.float64)[:, None]
    k = st.xhat.astype(np.float64) / h + st.z[:, None]
    assert np.allclose(k, np.rint(k), atol=1e-4)
    lo = (0 - st.z[:, None]) * h
    hi = (Q - st.z[:, None]) * h
    inside = (x >= lo) & (x <= hi)
    err = np.abs(st.xhat - x.astype(np.float64))
    assert np.all(err[inside] <= np.broadcast_to(h, x.shape)[inside] / 2 * (1 + 1e-5))
    # outside the range the value is the nearest endpoint
    below = x < lo - h / 2
    assert np.all(st.codes[below] == 0)
    above = x > hi + h / 2
    assert np.all(st.codes[above] == Q)


def test_sigmoid_values():
    s = quant.sigmoid32(np.array([0.0, 4.0, -4.0, 30.0], F32))
    assert s[0] == F32(0.5)
    assert abs(float(s[1]) - 0.9820137900379085) < 1e-7
    assert abs(float(s[1]) + float(s[2]) - 1.0) < 1e-7
    assert s[3] == F32(1.0)


def test_h_floor_on_constant_row():
    x = np.full((1, 8), 0.0, F32)
    st = quant.quantize_rows(x, F32(1), F32(1), 4)
    assert st.floor[0] and st.h[0] == F32(1e-8)
    assert np.all(st.xhat == 0)


def test_first_index_ties():
    x = np.array([[1.0, -1.0, 1.0, -1.0]], F32)
    st = quant.quantize_rows(x, F32(1), F32(1), 4)
    assert st.iM[0] == 0 and st.im[0] == 1


def test_let_identity_linear():
    """Quantizers off: X~ W~^T + B~ = X W^T + B within 1e-5 relative (fp32 LET)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((33, 70)).astype(F32) * 3
    W = (rng.standard_normal((20, 70)) * 0.02).astype(F32)
    B = rng.standard_normal(20).astype(F32)
    s = rng.uniform(0.3, 3.0, 70).astype(F32)
    d = rng.standard_normal(70).astype(F32)
    Xt = quant.let_act(X, s, d).astype(np.float64)
    Wt = quant.let_weight(W, s).astype(np.float64)
    Bt = quant.bias_fold(W, B, d)
    Y = X.astype(np.float64) @ W.astype(np.float64).T + B
    Y2 = Xt @ Wt.T + Bt
    assert np.linalg.norm(Y2 - Y) / np.linalg.norm(Y) < 1e-5


# --- group-wise LWC (the pages' g128 setting: clipping per group of input channels)

def test_group_lwc_full_width_is_per_channel():
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((12, 64)) * 0.02).astype(F32)
    ag = rng.uniform(1.0, 5.0, 12).astype(F32)
    ab = rng.uniform(1.0, 5.0, 12).astype(F32)
    s = rng.uniform(0.5, 2.0, 64).astype(F32)
    a = quant.lwc_fakequant(W, ag, ab, 3, s)
    b = quant.lwc_fakequant(W, ag, ab, 3, s, group=64)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.W_hat, b.W_hat)
    assert np.array_equal(a.h, b.h) and np.array_equal(a.z, b.z)


def test_group_lwc_slices_are_independent_quantizers():
    """Each (output channel, group) is the per-row quantizer of its own column slice
    with its own logits (logits stored output-channel major)."""
    rng = np.random.default_rng(22)
    C_out, C_in, g = 5, 48, 16
    G = C_in // g
    W = (rng.standard_normal((C_out, C_in)) * 0.02).astype(F32)
    ag = rng.uniform(1.0, 5.0, C_out * G).astype(F32)
    ab = rng.uniform(1.0, 5.0, C_out * G).astype(F32)
    r = quant.lwc_fakequant(W, ag, ab, 4, group=g)
    for o in range(C_out):
        for k in range(G):
            sl = W[o:o + 1, k * g:(k + 1) * g]
            one = quant.quantize_rows(sl, quant.sigmoid32(ag[o * G + k:o * G + k + 1]),
                                      quant.sigmoid32(ab[o * G + k:o * G + k + 1]), 4)
            assert np.array_equal(r.codes[o, k * g:(k + 1) * g], one.codes[0])
            assert np.array_equal(r.W_hat[o, k * g:(k + 1) * g], one.xhat[0])
            assert r.h[o * G + k] == one.h[0] and r.z[o * G + k] == one.z[0]


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_group_lwc_minmax(nbits):
    """gamma = beta = 1 (logits 30): every group of 128 is plain MinMax over its own
    range: grid ends within half a step of the group's min / max, no clipping."""
    rng = np.random.default_rng(23)
    C_out, C_in, g = 8, 512, 128
    W = (rng.standard_normal((C_out, C_in)) * 0.02).astype(F32)
    one = np.full(C_out * C_in // g, 30.0, F32)
    r = quant.lwc_fakequant(W, one, one, nbits, group=g)
    Q = 2 ** nbits - 1
    for o in range(C_out):
        for k in range(C_in // g):
            x = W[o, k * g:(k + 1) * g].astype(np.float64)
            j = o * (C_in // g) + k
            h, z = float(r.h[j]), float(r.z[j])
            assert abs((0 - z) * h - x.min()) <= h / 2 * (1 + 1e-6)
            assert abs((Q - z) * h - x.max()) <= h / 2 * (1 + 1e-6)
            assert np.all(np.abs(r.W_hat[o, k * g:(k + 1) * g] - x) <= h / 2 * (1 + 1e-5) + 1e-12)
            for c in range(0, g, 37):
                assert r.codes[o, k * g + c] == _nearest_code(float(x[c] / h), z, Q)


def test_code_product_brute_force_integers():
    """The code product against exact integer arithmetic on a tiny case: every entry
    is h_a h_b times an integer sum, formed here with Python ints, including rows
    whose zero point lies outside the code range (all-positive / all-negative rows)."""
    rng = np.random.default_rng(7)
    qa = rng.integers(0, 16, size=(3, 5))
    qb = rng.integers(0, 16, size=(4, 5))
    z_a = np.array([3.0, -21.0, 40.0])
    z_b = np.array([0.0, 15.0, -7.0, 8.0])
    h_a = np.array([0.5, 0.25, 2.0 ** -6])
    h_b = np.array([1.0, 0.125, 4.0, 2.0 ** -3])
    bias = np.array([1.0, -2.0, 0.5, 0.0])
    got = quant.code_product(qa, h_a, z_a, qb, h_b, z_b, bias)
    for m in range(3):
        for n in range(4):
            s = sum((int(qa[m, k]) - int(z_a[m])) * (int(qb[n, k]) - int(z_b[n]))
                    for k in range(5))
            assert got[m, n] == s * h_a[m] * h_b[n] + bias[n]   # powers of two: exact


def test_code_product_matches_fake_quant_product():
    """On the quantizers' own outputs the code product is X_hat W_hat^T: the
    fake-quantized operands are (q - z) h rounded once to float32."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((16, 64)).astype(np.float32)
    X[3] += 4.0                                   # an all-positive token row: z < 0
    W = rng.standard_normal((8, 64)).astype(np.float32)
    sx, Xh = quant.act_quant(X, 4)
    ref = quant.lwc_fakequant(W, np.full(8, 1.5, np.float32), np.full(8, 0.7, np.float32), 4)
    assert sx.z[3] < 0
    got = quant.code_product(sx.codes, sx.h, sx.z, ref.codes, ref.h, ref.z)
    want = Xh.astype(np.float64) @ ref.W_hat.astype(np.float64).T
    assert np.allclose(got, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
