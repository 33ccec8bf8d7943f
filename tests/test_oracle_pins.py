"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to mathematics (closed forms, exact
special cases, invertibility), to an independent brute force, or to the one
number the pages print.  Method: the technical summary of "SPHERICAL KV:
Angle-Domain Attention and Rate-Distortion Retention for Efficient
Long-Context Inference", section 2.1 (spherical parametrisation, quantised
radius, packed angle codes, logit estimator |q| * r~ * f_b(c_q, c_k) with f_b
a cosine similarity) and sections 2.2-2.3 (tier-homogeneous pages, paged store).
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle as O

PI = math.pi


# --- quantiser: predicates == floor(atan2 * 2^b / range) --------------------

@pytest.mark.parametrize("b", [2, 3, 4, 6, 8])
def test_polar_code_is_atan2_floor(b):
    rng = np.random.default_rng(1000 + b)
    n = 4000
    x = rng.standard_normal(n) * rng.choice([1e-3, 1.0, 1e3], n)
    S = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 1e3], n)) ** 2
    phi = np.arctan2(np.sqrt(S), x)
    ref = np.minimum(np.floor(phi * (1 << b) / PI), (1 << b) - 1).astype(int)
    frac = phi * (1 << b) / PI
    away = np.abs(frac - np.round(frac)) > 1e-9
    got = np.array([O.polar_code(x[i], S[i], b) for i in range(n)])
    assert away.sum() > 0.99 * n
    assert np.array_equal(got[away], ref[away])


@pytest.mark.parametrize("b", [2, 3, 4, 6, 8])
def test_azimuth_code_is_atan2_floor(b):
    rng = np.random.default_rng(2000 + b)
    n = 4000
    x = rng.standard_normal(n)
    y = rng.standard_normal(n)
    phi = np.mod(np.arctan2(y, x), 2 * PI)
    frac = phi * (1 << b) / (2 * PI)
    ref = np.minimum(np.floor(frac), (1 << b) - 1).astype(int)
    away = np.abs(frac - np.round(frac)) > 1e-9
    got = np.array([O.azimuth_code(x[i], y[i], b) for i in range(n)])
    assert np.array_equal(got[away], ref[away])


@pytest.mark.parametrize("b", [2, 3, 4, 6, 8])
def test_exact_edges_and_zero_vectors(b):
    n = 1 << b
    # phi = 0, pi/2 (an exact edge: upper bin), pi (clamped to the last bin)
    assert O.polar_code(1.0, 0.0, b) == 0
    assert O.polar_code(0.0, 1.0, b) == n // 2
    assert O.polar_code(-0.0, 1.0, b) == n // 2
    assert O.polar_code(-1.0, 0.0, b) == n - 1
    assert O.polar_code(0.0, 0.0, b) == 0
    # azimuth 0, pi/2, pi, 3pi/2 are edges for b >= 2
    assert O.azimuth_code(1.0, 0.0, b) == 0
    assert O.azimuth_code(1.0, -0.0, b) == 0
    assert O.azimuth_code(0.0, 1.0, b) == n // 4
    assert O.azimuth_code(-1.0, 0.0, b) == n // 2
    assert O.azimuth_code(-1.0, -0.0, b) == n // 2
    assert O.azimuth_code(0.0, -1.0, b) == 3 * n // 4
    assert O.azimuth_code(0.0, 0.0, b) == 0
    # every code is in range and the predicate count is monotone in phi
    phis = np.linspace(0, PI, 997)
    codes = [O.polar_code(math.cos(p), math.sin(p) ** 2, b) for p in phis]
    assert all(0 <= c < n for c in codes)
    assert all(c2 >= c1 for c1, c2 in zip(codes, codes[1:]))


@pytest.mark.parametrize("b", [2, 3, 4, 6])
def test_codes_nest_across_tiers(b):
    """The bins of every width are uniform over the same range, so each edge
    j*pi/2^b of a narrow tier is the edge (j*2^(8-b))*pi/2^8 of the 8-bit
    tier: the narrow code is the 8-bit code shifted right by 8 - b (the
    azimuth's half-plane offset shifts with it).  Checked on the edge tables
    (identical binary64 values), on random angles, and on inputs placed on
    8-bit edges, where the exact predicates decide."""
    k = 8 - b
    c2b, s2b = O.angle_thresholds(b)
    c28, s28 = O.angle_thresholds(8)
    j = np.arange(1, 1 << b)
    assert np.array_equal(c2b[j], c28[j << k]) and np.array_equal(s2b[j], s28[j << k])
    rng = np.random.default_rng(3000 + b)
    n = 3000
    x = rng.standard_normal(n) * rng.choice([1e-3, 1.0, 1e3], n)
    y = rng.standard_normal(n) * rng.choice([1e-3, 1.0, 1e3], n)
    # on (or within rounding of) 8-bit edges: cos and sin of j*pi/256
    je = rng.integers(1, 256, 400)
    xe = np.cos(je * PI / 256)
    ye = np.sin(je * PI / 256)
    for xi, yi in zip(np.r_[x, xe], np.r_[y, ye]):
        S = yi * yi
        assert O.polar_code(xi, S, b) == O.polar_code(xi, S, 8) >> k
        assert O.azimuth_code(xi, yi, b) == O.azimuth_code(xi, yi, 8) >> k
        assert O.azimuth_code(xi, -yi, b) == O.azimuth_code(xi, -yi, 8) >> k


def test_thresholds_are_squared_cos_sin_of_edges():
    for b in (2, 4, 8):
        c2, s2 = O.angle_thresholds(b)
        j = np.arange(1, 1 << b)
        np.testing.assert_allclose(c2[1:], np.cos(j * PI / (1 << b)) ** 2, rtol=0, atol=1e-15)
        np.testing.assert_allclose(s2[1:], np.sin(j * PI / (1 << b)) ** 2, rtol=0, atol=1e-15)


# --- Phi and its inverse ----------------------------------------------------

@pytest.mark.parametrize("d", [2, 3, 8, 64, 128])
def test_phi_is_invertible(d):
    rng = np.random.default_rng(d)
    for _ in range(20):
        x = (rng.standard_normal(d) * rng.lognormal(0, 0.5, d)).astype(np.float32)
        phi, T0 = O.angles(x)
        u = O.unit_from_angles(phi, d)
        ref = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64))
        assert np.abs(u - ref).max() <= 1e-14
        assert abs(T0 - float(np.dot(x.astype(np.float64), x.astype(np.float64)))) <= 1e-12 * T0
        assert np.all(phi[:-1] >= 0) and np.all(phi[:-1] <= PI)
        assert 0 <= phi[-1] < 2 * PI


@pytest.mark.parametrize("d,b", [(3, 3), (64, 4), (128, 2), (128, 8)])
def test_decoded_direction_is_unit(d, b):
    rng = np.random.default_rng(7 * d + b)
    for _ in range(20):
        c = rng.integers(0, 1 << b, d - 1)
        u = O.direction(c, d, b)
        assert abs(np.linalg.norm(u) - 1.0) < 1e-13


def test_codes_converge_to_the_direction_as_b_grows():
    """b -> infinity: the decoded direction tends to x/|x| (error halves per bit)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(8).astype(np.float32)
    ref = x / np.linalg.norm(x.astype(np.float64))
    errs = []
    for b in range(4, 15):
        c, _ = O.key_codes(x, b)
        errs.append(np.abs(O.direction(c, 8, b) - ref).max())
    assert errs[-1] < 1e-3
    assert all(e2 < e1 for e1, e2 in zip(errs[::2], errs[2::2]))


# --- hand examples (closed forms) -------------------------------------------

def test_d2_hand_example():
    """d=2: f = cos(phi_q - phi_k) of the bin centres."""
    cq, Tq = O.key_codes(np.array([1, 0], np.float32), 3)
    ck, Tk = O.key_codes(np.array([3, 4], np.float32), 3)
    assert list(cq) == [0] and list(ck) == [1] and Tk == 25.0
    f = O.direction(cq, 2, 3) @ O.direction(ck, 2, 3)
    assert abs(f - math.cos(PI / 4)) < 1e-15
    level, tau2 = O.radius_tables(O.UNIFORM, 0.0, 5.0)
    rc = O.radius_code(Tk, tau2)
    assert rc == 255 and level[rc] == 5.0
    # l = |q| * r~ * f with scale 1: 5 cos(pi/4) = 3.535534 (dense q.k = 3)
    assert abs(1.0 * level[rc] * f - 3.5355339059327378) < 1e-14


def test_d3_hand_example():
    """d=3: spherical law of cosines on the bin centres."""
    q = np.array([2, 1, 3], np.float32)
    k = np.array([1, 2, 3], np.float32)
    cq, _ = O.key_codes(q, 3)
    ck, _ = O.key_codes(k, 3)
    assert list(cq) == [2, 1] and list(ck) == [3, 1]
    f = O.direction(cq, 3, 3) @ O.direction(ck, 3, 3)
    a1, a2 = 2.5 * PI / 8, 3.5 * PI / 8
    law = math.cos(a1) * math.cos(a2) + math.sin(a1) * math.sin(a2) * math.cos(0.0)
    assert abs(f - law) < 1e-15
    assert abs(f - math.cos(PI / 8)) < 1e-15
    assert abs(14.0 * f - 12.934313) < 1e-6       # |q| r f with |q| = |k| = sqrt(14)


def test_near_zero_logit_example():
    """q.k = 0 exactly, yet the coded estimate is 0.0843 of the bound."""
    q = np.array([0.3, -1.2, 0.7], np.float32)
    k = np.array([1, 2, 3], np.float32)
    cq, _ = O.key_codes(q, 4)
    ck, _ = O.key_codes(k, 4)
    assert list(cq) == [6, 6] and list(ck) == [6, 2]
    f = O.direction(cq, 3, 4) @ O.direction(ck, 3, 4)
    # azimuth centres differ by pi/2, so f = cos^2(6.5 pi/16)
    assert abs(f - math.cos(6.5 * PI / 16) ** 2) < 1e-15


def test_logit_error_shrinks_monotonically_with_b():
    """RMS of (l_hat - q.k)/(|q||k|) at d=128 falls strictly with b, by at
    least a factor 0.75 per bit from b=4 on."""
    rng = np.random.default_rng(11)
    d, n = 128, 300
    chan = rng.lognormal(0, 0.5, d)
    K = (rng.standard_normal((n, d)) * chan).astype(np.float32)
    Q = rng.standard_normal((n, d)).astype(np.float32)
    rms = []
    for b in range(2, 11):
        e = []
        for i in range(n):
            cq, _ = O.key_codes(Q[i], b)
            ck, _ = O.key_codes(K[i], b)
            f = O.direction(cq, d, b) @ O.direction(ck, d, b)
            qd, kd = Q[i].astype(np.float64), K[i].astype(np.float64)
            e.append(f - qd @ kd / (np.linalg.norm(qd) * np.linalg.norm(kd)))
        rms.append(float(np.sqrt(np.mean(np.square(e)))))
    assert all(r2 < r1 for r1, r2 in zip(rms, rms[1:])), rms
    assert all(rms[i + 1] <= 0.75 * rms[i] for i in range(2, len(rms) - 1)), rms


# --- radius quantiser -------------------------------------------------------

def test_uniform_radius_rounds_half_up_and_hits_the_max():
    R = 7.25
    level, tau2 = O.radius_tables(O.UNIFORM, 0.0, R)
    assert level[0] == 0.0 and level[255] == R
    rng = np.random.default_rng(3)
    r = rng.uniform(0, R, 3000)
    frac = r * 255 / R
    away = np.abs(frac - np.floor(frac) - 0.5) > 1e-9
    ref = np.floor(frac + 0.5).astype(int)
    got = np.array([O.radius_code(x * x, tau2) for x in r])
    assert np.array_equal(got[away], ref[away])
    assert O.radius_code(R * R, tau2) == 255
    assert O.radius_code(4 * R * R, tau2) == 255
    assert O.radius_code(0.0, tau2) == 0


def test_log_radius_rounds_in_log_domain():
    lo, hi = 0.5, 40.0
    level, tau2 = O.radius_tables(O.LOG, lo, hi)
    assert abs(level[0] - lo) < 1e-15 and abs(level[255] - hi) < 1e-12
    rng = np.random.default_rng(4)
    r = np.exp(rng.uniform(np.log(lo), np.log(hi), 3000))
    frac = 255 * np.log(r / lo) / np.log(hi / lo)
    away = np.abs(frac - np.floor(frac) - 0.5) > 1e-7
    ref = np.floor(frac + 0.5).astype(int)
    got = np.array([O.radius_code(x * x, tau2) for x in r])
    assert np.array_equal(got[away], ref[away])
    assert O.radius_code(1e-6, tau2) == 0 and O.radius_code(1e6, tau2) == 255


def test_calibration_is_min_positive_and_max_norm():
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((50, 3, 16)).astype(np.float32)
    keys[7, 1] = 0.0
    rg = O.calibrate(keys)
    nrm = np.linalg.norm(keys.astype(np.float64), axis=2)
    for g in range(3):
        pos = nrm[:, g][nrm[:, g] > 0]
        assert abs(rg[g, 1] - nrm[:, g].max()) <= 1e-14 * rg[g, 1]
        assert abs(rg[g, 0] - pos.min()) <= 1e-14 * rg[g, 0]


# --- record layout ----------------------------------------------------------

@pytest.mark.parametrize("d,b", [(128, 2), (128, 3), (128, 4), (128, 6), (128, 8),
                                 (64, 2), (64, 4), (64, 8)])
def test_record_is_flat_lsb_first_bit_packing(d, b):
    """For these shapes the four-slice layout equals plain little-endian bit
    packing of the d-1 codes (numpy packbits), zero padded to KB bytes."""
    rng = np.random.default_rng(d * 10 + b)
    c = rng.integers(0, 1 << b, d - 1)
    rec = O.pack(c, d, b)
    assert len(rec) == 16 * math.ceil((d - 1) * b / 128)
    bits = ((c[:, None] >> np.arange(b)[None, :]) & 1).reshape(-1).astype(np.uint8)
    ref = np.packbits(bits, bitorder="little")
    assert np.array_equal(rec[: len(ref)], ref)
    assert not rec[len(ref):].any()
    assert np.array_equal(O.unpack(rec, d, b), c)


def test_d64_b3_slices_are_padded():
    d, b = 64, 3
    c = np.arange(d - 1) % 8
    rec = O.pack(c, d, b)
    assert len(rec) == 32
    for s in range(4):
        sl = rec[8 * s: 8 * s + 8]
        bits = np.unpackbits(sl, bitorder="little")
        na = min(16, d - 1 - 16 * s)
        got = [int("".join(map(str, bits[3 * i: 3 * i + 3][::-1])), 2) for i in range(na)]
        assert got == list(c[16 * s: 16 * s + na])
        assert not bits[3 * na:].any()
    assert np.array_equal(O.unpack(rec, d, b), c)


def test_resident_bytes_match_the_pages_range():
    """Bytes per (token, kv head) = KB(b) + 1 + 2d against dense bf16 K+V
    (4d); the pages' resident-byte reduction of 24-42 % (golden file) covers
    the tiers 3..8 at d=128."""
    path = os.path.join(os.path.dirname(__file__), "golden", "resident_bytes.txt")
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    lo, hi = vals["reduction_min_percent"], vals["reduction_max_percent"]
    d = 128
    red = {b: 100.0 * (1 - (O.kb(d, b) + 1 + 2 * d) / (4 * d)) for b in (2, 3, 4, 6, 8)}
    assert abs(red[4] - 37.3046875) < 1e-9
    for b in (3, 4, 6, 8):
        assert lo <= red[b] <= hi, (b, red[b])
