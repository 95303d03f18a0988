"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with its pin. They are run
against the built oracle (``test_oracle_pins.py``) and against deliberately
broken copies of it (``test_oracle_mutants.py``), which shows that each
plausible mistake is caught by at least one pin.

What each pin compares with:
* ``half_decode``      -- numpy's IEEE binary16 conversion, all 65,536 codes.
* ``golden``           -- hand-derived worked examples in ``tests/golden``.
* ``exact_rational``   -- exact ``fractions.Fraction`` sums on tiny shapes.
* ``library_matmul``   -- a dense f64 dequantization of the logical fields
                          multiplied by ``torch.matmul`` in float64.
* ``one_hot``          -- closed form: x = e_k gives y[n] = d * (q[n,k] - 8).
* ``zero_point``       -- all nibbles 8 give y = 0 and s = 0 exactly.
* ``extreme_nibbles``  -- q = 15 / q = 0 with x = 1 give 224 / -256 * sum d.
* ``subnormal_scale``  -- fp16 scale 2^-24 (and the largest subnormal).
* ``linear_in_d``      -- doubling every scale doubles y bitwise.
* ``integer_exact``    -- d = 1 and small integer x give an exact integer.
* ``q8_min``           -- q = -128 is honoured.
* ``permutations``     -- row permutation permutes y; a block permutation
                          along K of both W and x leaves y unchanged.
* ``special_values``   -- Inf / NaN scales propagate as IEEE arithmetic does.
* ``gelu_tanh_form``   -- the gate activation: gelu(0) = 0, the odd-part
                          identity gelu(g) - gelu(-g) = g, saturation,
                          distance <= 5e-4 to the exact GELU g * Phi(g)
                          (math.erf), and its curvature at 0, which must be
                          that of g * Phi(g): sqrt(2/pi) from math.pi.
* ``ffn_gate_up``      -- the gated FFN front half: its g and u equal the
                          pinned matmul, h vanishes with g or u, and two
                          rows with gates +g, -g over the same up row differ
                          by exactly g * u (the odd-part identity again).
* ``q4k_*``            -- Q4_K super-blocks: torch float64 matmul of a dense
                          dequantization of the logical fields, one-hot x,
                          zero nibbles and minimums give 0, scales 0 leave
                          -dmin * mn (closed form), d = dmin = 1 with integer
                          x is an exact integer, y(2d, 2dmin) = 2 y, row
                          permutations; the hand-worked golden super-block
                          (``golden``) pins the byte placement.

The logical fields (fp16 scales and integer codes) are placed into bytes by
``synth.pack_q4_0`` / ``synth.pack_q8_0``; the golden fixtures spell their
bytes out by hand, which pins that placement too.
"""

from __future__ import annotations

import math
import pathlib
from fractions import Fraction

import numpy as np

import synth

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"
EPS64 = 2.0 ** -53


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def pack(fmt, d, q):
    return synth.pack_q4_0(d, q) if fmt == "q4_0" else synth.pack_q8_0(d, q)


def centred(fmt, q):
    """Integer weight codes (q - 8 for Q4_0, q for Q8_0) as int64."""
    q = np.asarray(q).astype(np.int64)
    return q - 8 if fmt == "q4_0" else q


def dense_weights(fmt, d, q):
    """f64 dense W[N, K] from logical fields (test-side, for library pins)."""
    d64 = np.repeat(np.asarray(d, dtype=np.float64), 32, axis=1)
    return d64 * centred(fmt, q).astype(np.float64)


def random_fp16(rng, shape, allow_negative=True):
    """Finite fp16 values drawn over all exponents (incl. subnormals)."""
    bits = rng.integers(0, 0x7C00, size=shape, dtype=np.uint16)  # finite, >= 0
    if allow_negative:
        bits |= (rng.integers(0, 2, size=shape, dtype=np.uint16) << 15)
    return bits.view(np.float16)


def load_golden(path):
    spec = {}
    for line in pathlib.Path(path).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        spec[key] = rest.split()
    m, n, k = int(spec["M"][0]), int(spec["N"][0]), int(spec["K"][0])
    w = np.array([int(b, 16) for b in spec["w"]], dtype=np.uint8)
    x = np.array([float(Fraction(v)) for v in spec["x"]], dtype=np.float32).reshape(m, k)
    y = [Fraction(v) for v in spec["y"]]
    return dict(fmt=spec["fmt"][0], M=m, N=n, K=k, w=w, x=x, y=y)


def golden_cases():
    return sorted(GOLDEN.glob("*.txt"))


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def half_decode(o):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN codes disagree"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 decode disagrees with IEEE binary16"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "sign of zero"


def golden(o):
    for path in golden_cases():
        g = load_golden(path)
        y, s = o.matmul(g["fmt"], g["x"], g["w"], g["N"], g["K"])
        for i, want in enumerate(g["y"]):
            got = y.reshape(-1)[i]
            assert got == float(want), f"{path.name}[{i}]: {got!r} != {float(want)!r}"


def exact_rational(o, cases=200, seed=1234):
    rng = np.random.default_rng(seed)
    for case in range(cases):
        fmt = "q4_0" if case % 2 == 0 else "q8_0"
        m = int(rng.integers(1, 3))
        n = int(rng.integers(1, 5))
        k = int(rng.choice([32, 64, 256]))
        d = random_fp16(rng, (n, k // 32))
        if fmt == "q4_0":
            q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        else:
            q = rng.integers(-128, 128, (n, k), dtype=np.int8)
        scale = 2.0 ** rng.integers(-20, 20, size=(m, 1))
        x = (rng.standard_normal((m, k)) * scale).astype(np.float32)
        y, s = o.matmul(fmt, x, pack(fmt, d, q), n, k)
        c = centred(fmt, q)
        for mi in range(m):
            for ni in range(n):
                terms = [Fraction(float(d[ni, kk // 32])) * int(c[ni, kk]) * Fraction(float(x[mi, kk]))
                         for kk in range(k)]
                exact = sum(terms, Fraction(0))
                sabs = sum((abs(t) for t in terms), Fraction(0))
                bound = (k - 1) * EPS64 * float(sabs)
                assert abs(Fraction(y[mi, ni]) - exact) <= Fraction(bound), (
                    f"case {case} ({fmt}, m={mi}, n={ni}): y={y[mi, ni]!r} exact={float(exact)!r}")
                assert abs(Fraction(s[mi, ni]) - sabs) <= Fraction(bound), (
                    f"case {case}: s={s[mi, ni]!r} exact={float(sabs)!r}")
                # the terms are exact f64 values, so fsum of them is the exact
                # sum correctly rounded, and the oracle must be within its bound
                fs = math.fsum(float(t) for t in terms)
                assert fs == float(exact)


def library_matmul(o, shapes=((1, 256, 512), (3, 1000, 2048), (2, 64, 8192))):
    import torch

    for fmt in ("q4_0", "q8_0"):
        for (m, n, k) in shapes:
            if fmt == "q4_0":
                d, q = synth.q4_0_fields(n, k, seed=7)
            else:
                d, q = synth.q8_0_fields(n, k, seed=7)
            x = synth.activations(m, k, seed=7)
            y, s = o.matmul(fmt, x, pack(fmt, d, q), n, k)
            wd = torch.from_numpy(dense_weights(fmt, d, q))
            xd = torch.from_numpy(x.astype(np.float64))
            ref = (xd @ wd.T).numpy()
            sref = (xd.abs() @ wd.abs().T).numpy()
            tol = 2 * k * EPS64 * sref
            assert np.all(np.abs(y - ref) <= tol), f"{fmt} {m}x{n}x{k}: max err {np.abs(y - ref).max()}"
            assert np.all(np.abs(s - sref) <= tol), f"{fmt} {m}x{n}x{k}: s disagrees"


def one_hot(o, n=16, k=256, seed=3):
    rng = np.random.default_rng(seed)
    for fmt in ("q4_0", "q8_0"):
        d = random_fp16(rng, (n, k // 32))
        if fmt == "q4_0":
            q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        else:
            q = rng.integers(-128, 128, (n, k), dtype=np.int8)
        w = pack(fmt, d, q)
        c = centred(fmt, q)
        ks = list(range(64)) + [int(v) for v in rng.integers(64, k, 16)]
        x = np.zeros((len(ks), k), dtype=np.float32)
        x[np.arange(len(ks)), ks] = 1.0
        y, _ = o.matmul(fmt, x, w, n, k)
        want = d.astype(np.float64)[:, np.array(ks) // 32].T * c[:, ks].T
        assert np.array_equal(y, want), f"{fmt}: one-hot x does not select w[n, k]"


def zero_point(o, n=8, k=512, seed=4):
    rng = np.random.default_rng(seed)
    d = random_fp16(rng, (n, k // 32))
    q = np.full((n, k), 8, dtype=np.uint8)
    x = (rng.standard_normal((3, k)) * 1e3).astype(np.float32)
    y, s = o.matmul("q4_0", x, synth.pack_q4_0(d, q), n, k)
    assert np.all(y == 0.0) and np.all(s == 0.0), "all-8 nibbles must give exactly 0"


def extreme_nibbles(o, n=4, k=2048, seed=5):
    rng = np.random.default_rng(seed)
    d = (2.0 ** rng.integers(-14, 4, (n, k // 32))).astype(np.float16)
    x = np.ones((1, k), dtype=np.float32)
    dsum = d.astype(np.float64).sum(axis=1)  # powers of two: exact
    for nib, factor in ((15, 224), (0, -256)):
        q = np.full((n, k), nib, dtype=np.uint8)
        y, _ = o.matmul("q4_0", x, synth.pack_q4_0(d, q), n, k)
        assert np.array_equal(y[0], factor * dsum), f"nibble {nib}: {y[0]} != {factor * dsum}"


def subnormal_scale(o):
    for bits in (0x0001, 0x03FF, 0x8001):
        d = np.array([[bits]], dtype=np.uint16).view(np.float16)
        q = np.full((1, 32), 15, dtype=np.uint8)
        y, _ = o.matmul("q4_0", np.ones((1, 32), np.float32), synth.pack_q4_0(d, q), 1, 32)
        f = bits & 0x3FF
        want = (-1.0 if bits & 0x8000 else 1.0) * 224 * f * 2.0 ** -24
        assert y[0, 0] == want, f"subnormal d 0x{bits:04x}: {y[0, 0]!r} != {want!r}"


def linear_in_d(o, n=64, k=1024, seed=6):
    for fmt in ("q4_0", "q8_0"):
        if fmt == "q4_0":
            d, q = synth.q4_0_fields(n, k, seed=seed)
        else:
            d, q = synth.q8_0_fields(n, k, seed=seed)
        d2 = (d.astype(np.float64) * 2).astype(np.float16)
        assert np.array_equal(d2.astype(np.float64), 2 * d.astype(np.float64))
        x = synth.activations(2, k, seed=seed)
        y1, s1 = o.matmul(fmt, x, pack(fmt, d, q), n, k)
        y2, s2 = o.matmul(fmt, x, pack(fmt, d2, q), n, k)
        assert np.array_equal(y2, 2 * y1) and np.array_equal(s2, 2 * s1), f"{fmt}: y(2d) != 2 y(d)"


def integer_exact(o, n=32, k=2048, seed=8):
    rng = np.random.default_rng(seed)
    d = np.ones((n, k // 32), dtype=np.float16)
    x = rng.integers(-8, 9, (2, k)).astype(np.float32)
    xi = x.astype(np.int64)
    for fmt in ("q4_0", "q8_0"):
        if fmt == "q4_0":
            q = rng.integers(0, 16, (n, k), dtype=np.uint8)
        else:
            q = rng.integers(-128, 128, (n, k), dtype=np.int8)
        y, _ = o.matmul(fmt, x, pack(fmt, d, q), n, k)
        want = xi @ centred(fmt, q).T  # Python/numpy integers, exact
        assert np.array_equal(y, want.astype(np.float64)), f"{fmt}: integer case not exact"


def q8_min(o):
    d = np.ones((1, 1), dtype=np.float16)
    q = np.full((1, 32), -128, dtype=np.int8)
    y, _ = o.matmul("q8_0", np.ones((1, 32), np.float32), synth.pack_q8_0(d, q), 1, 32)
    assert y[0, 0] == -4096.0, f"q = -128 gives {y[0, 0]}"


def permutations(o, n=48, k=1024, seed=9):
    rng = np.random.default_rng(seed)
    for fmt in ("q4_0", "q8_0"):
        if fmt == "q4_0":
            d, q = synth.q4_0_fields(n, k, seed=seed)
        else:
            d, q = synth.q8_0_fields(n, k, seed=seed)
        x = synth.activations(3, k, seed=seed)
        y, s = o.matmul(fmt, x, pack(fmt, d, q), n, k)
        rp = rng.permutation(n)
        yr, _ = o.matmul(fmt, x, pack(fmt, d[rp], q[rp]), n, k)
        assert np.array_equal(yr, y[:, rp]), f"{fmt}: row permutation"
        bp = rng.permutation(k // 32)
        kp = (bp[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
        yb, sb = o.matmul(fmt, x[:, kp], pack(fmt, d[:, bp], q[:, kp]), n, k)
        tol = 2 * k * EPS64 * s
        assert np.all(np.abs(yb - y) <= tol), f"{fmt}: block permutation along K"


def special_values(o):
    q = np.full((1, 32), 9, dtype=np.uint8)  # w = +d everywhere
    x = np.ones((1, 32), np.float32)
    for bits, want in ((0x7C00, math.inf), (0xFC00, -math.inf)):
        d = np.array([[bits]], dtype=np.uint16).view(np.float16)
        y, _ = o.matmul("q4_0", x, synth.pack_q4_0(d, q), 1, 32)
        assert y[0, 0] == want
    d = np.array([[0x7E00]], dtype=np.uint16).view(np.float16)  # NaN
    y, _ = o.matmul("q4_0", x, synth.pack_q4_0(d, q), 1, 32)
    assert math.isnan(y[0, 0])


def gelu_tanh_form(o):
    assert o.gelu_tanh(0.0) == 0.0
    for g in np.linspace(-7.0, 7.0, 141):
        g = float(g)
        a, b = o.gelu_tanh(g), o.gelu_tanh(-g)
        # g/2 (1 + t) - (-g/2)(1 - t) = g for any odd argument of tanh
        assert abs((a - b) - g) <= 4 * EPS64 * max(1.0, abs(g)), f"odd part at {g}"
        exact = 0.5 * g * (1.0 + math.erf(g / math.sqrt(2.0)))
        # the tanh form's own largest distance to g * Phi(g) over [-7, 7] is
        # 4.73e-4 (at |g| ~ 2.2); a constant off by 0.3 % (0.797 for
        # sqrt(2/pi)) or a cubic coefficient off by 10 % already exceeds 5e-4
        assert abs(a - exact) <= 5e-4, f"far from g * Phi(g) at {g}: {a} vs {exact}"
    # Curvature at 0, independent of the form's constants as written: any
    # gelu(g) = g/2 (1 + t(g)) with t odd has (gelu(h) + gelu(-h)) / h^2 =
    # t(h) / h -> t'(0), and the exact GELU g * Phi(g) has second derivative
    # 2 phi(0) = sqrt(2/pi) at 0, so t'(0) must be sqrt(2/pi) (the h^2 term
    # moves the quotient by ~1e-9 at h = 1e-4).
    c = math.sqrt(2.0 / math.pi)
    h = 1e-4
    curv = (o.gelu_tanh(h) + o.gelu_tanh(-h)) / (h * h)
    assert abs(curv - c) <= 1e-7 * c, f"curvature at 0: {curv} vs sqrt(2/pi) = {c}"
    assert o.gelu_tanh(12.0) == 12.0 and abs(o.gelu_tanh(-12.0)) < 1e-30
    assert 0.0 < o.gelu_tanh(0.5) < 0.5 and o.gelu_tanh(-0.5) < 0.0


def ffn_gate_up(o, n=24, k=512, seed=10):
    rng = np.random.default_rng(seed)
    # rows 2i and 2i+1: gate codes mirrored around 8 (gates +g and -g under
    # x = e_k0), up codes equal; d = 1, so g = q - 8 and u = q_up - 8 exactly
    half = n // 2
    qg = rng.integers(0, 16, (half, k), dtype=np.uint8)
    qg = np.repeat(qg, 2, axis=0)
    qg[1::2] = (16 - qg[1::2].astype(np.int64)).clip(0, 15).astype(np.uint8)
    qu = np.repeat(rng.integers(0, 16, (half, k), dtype=np.uint8), 2, axis=0)
    d = np.ones((n, k // 32), dtype=np.float16)
    wg, wu = synth.pack_q4_0(d, qg), synth.pack_q4_0(d, qu)
    k0 = int(rng.integers(0, k))
    x = np.zeros((1, k), np.float32)
    x[0, k0] = 1.0
    h, g, u, sg, su = o.ffn_gate_up(x, wg, wu, n, k)
    yg, syg = o.matmul("q4_0", x, wg, n, k)
    yu, syu = o.matmul("q4_0", x, wu, n, k)
    assert np.array_equal(g, yg) and np.array_equal(u, yu), "g, u are not the matmul"
    assert np.array_equal(sg, syg) and np.array_equal(su, syu)
    assert np.array_equal(g[0], qg[:, k0].astype(np.float64) - 8)
    for i in range(half):
        a, b = 2 * i, 2 * i + 1
        if g[0, a] == -g[0, b]:               # mirrored (q = 0 has no mirror)
            want = g[0, a] * u[0, a]
            assert abs((h[0, a] - h[0, b]) - want) <= 8 * EPS64 * max(1.0, abs(want))
        if g[0, a] == 0 or u[0, a] == 0:
            assert h[0, a] == 0.0
    # random operands: h is gelu(g) u with g, u the pinned sums
    dg, qg2 = synth.q4_0_fields(n, k, seed=seed)
    du, qu2 = synth.q4_0_fields(n, k, seed=seed + 1)
    xr = synth.activations(3, k, seed=seed)
    h2, g2, u2, _, _ = o.ffn_gate_up(xr, synth.pack_q4_0(dg, qg2), synth.pack_q4_0(du, qu2), n, k)
    assert np.array_equal(g2, o.matmul("q4_0", xr, synth.pack_q4_0(dg, qg2), n, k)[0])
    assert np.all(np.sign(h2[g2 > 0]) == np.sign(u2[g2 > 0]))   # gelu(g) > 0 for g > 0


# ----------------------------------------------------------------------------
# Q4_K super-blocks (256 weights: d, dmin, 6-bit sub-block scales and
# minimums, nibbles); the golden fixture pins the byte placement
# ----------------------------------------------------------------------------

def q4k_dense(d, dmin, sc, mn, q):
    """f64 dense W[N, K] from logical Q4_K fields (test-side): weight e of a
    super-block is d * sc[e // 32] * q[e] - dmin * mn[e // 32]."""
    n, k = q.shape
    ns = k // 256
    dsc = d.astype(np.float64)[:, :, None] * sc.astype(np.float64)
    dmn = dmin.astype(np.float64)[:, :, None] * mn.astype(np.float64)
    dsc = np.repeat(dsc.reshape(n, ns * 8), 32, axis=1)
    dmn = np.repeat(dmn.reshape(n, ns * 8), 32, axis=1)
    return dsc * q.astype(np.float64) - dmn


def q4k_random_fields(rng, n, k, fp16_any=True):
    ns = k // 256
    if fp16_any:
        d = random_fp16(rng, (n, ns), allow_negative=True)
        dmin = random_fp16(rng, (n, ns), allow_negative=True)
    else:
        d = (2.0 ** rng.integers(-10, 3, (n, ns))).astype(np.float16)
        dmin = (2.0 ** rng.integers(-10, 3, (n, ns))).astype(np.float16)
    sc = rng.integers(0, 64, (n, ns, 8), dtype=np.uint8)
    mn = rng.integers(0, 64, (n, ns, 8), dtype=np.uint8)
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    return d, dmin, sc, mn, q


def q4k_library_matmul(o, shapes=((1, 64, 256), (3, 300, 2048), (2, 40, 8192))):
    import torch

    for (m, n, k) in shapes:
        f = synth.q4_k_fields(n, k, seed=11)
        x = synth.activations(m, k, seed=11)
        y, s = o.matmul("q4_k", x, synth.pack_q4_k(*f), n, k)
        wd = torch.from_numpy(q4k_dense(*f))
        xd = torch.from_numpy(x.astype(np.float64))
        ref = (xd @ wd.T).numpy()
        sref = (xd.abs() @ wd.abs().T).numpy()
        tol = 4 * k * EPS64 * sref
        assert np.all(np.abs(y - ref) <= tol), f"q4_k {m}x{n}x{k}: max err {np.abs(y - ref).max()}"
        assert np.all(np.abs(s - sref) <= tol), f"q4_k {m}x{n}x{k}: s disagrees"


def q4k_one_hot(o, n=12, k=512, seed=12):
    rng = np.random.default_rng(seed)
    f = q4k_random_fields(rng, n, k)
    w = synth.pack_q4_k(*f)
    ks = list(range(0, 256, 3)) + [int(v) for v in rng.integers(256, k, 24)]
    x = np.zeros((len(ks), k), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    y, _ = o.matmul("q4_k", x, w, n, k)
    want = q4k_dense(*f)[:, ks].T
    assert np.array_equal(y, want), "q4_k: one-hot x does not select w[n, k]"


def q4k_zero(o, n=6, k=512, seed=13):
    rng = np.random.default_rng(seed)
    d, dmin, sc, _, _ = q4k_random_fields(rng, n, k)
    mn = np.zeros_like(sc)
    q = np.zeros((n, k), dtype=np.uint8)
    x = (rng.standard_normal((2, k)) * 1e3).astype(np.float32)
    y, s = o.matmul("q4_k", x, synth.pack_q4_k(d, dmin, sc, mn, q), n, k)
    assert np.all(y == 0.0) and np.all(s == 0.0), "q4_k: zero nibbles and minimums must give 0"


def q4k_mins_only(o, n=5, k=1024, seed=14):
    rng = np.random.default_rng(seed)
    d, dmin, _, mn, q = q4k_random_fields(rng, n, k, fp16_any=False)
    sc = np.zeros_like(mn)
    x = np.ones((1, k), dtype=np.float32)
    y, _ = o.matmul("q4_k", x, synth.pack_q4_k(d, dmin, sc, mn, q), n, k)
    want = -(32 * dmin.astype(np.float64) * mn.astype(np.float64).sum(axis=2)).sum(axis=1)
    assert np.array_equal(y[0], want), f"q4_k minimums: {y[0]} != {want}"


def q4k_integer_exact(o, n=16, k=2048, seed=15):
    rng = np.random.default_rng(seed)
    _, _, sc, mn, q = q4k_random_fields(rng, n, k)
    ones = np.ones((n, k // 256), dtype=np.float16)
    x = rng.integers(-8, 9, (2, k)).astype(np.float32)
    y, _ = o.matmul("q4_k", x, synth.pack_q4_k(ones, ones, sc, mn, q), n, k)
    sub_sc = np.repeat(sc.reshape(n, -1).astype(np.int64), 32, axis=1)
    sub_mn = np.repeat(mn.reshape(n, -1).astype(np.int64), 32, axis=1)
    want = x.astype(np.int64) @ (sub_sc * q.astype(np.int64) - sub_mn).T
    assert np.array_equal(y, want.astype(np.float64)), "q4_k: integer case not exact"


def q4k_linear_and_rows(o, n=40, k=1024, seed=16):
    rng = np.random.default_rng(seed)
    d, dmin, sc, mn, q = synth.q4_k_fields(n, k, seed=seed)
    x = synth.activations(2, k, seed=seed)
    y, s = o.matmul("q4_k", x, synth.pack_q4_k(d, dmin, sc, mn, q), n, k)
    d2 = (d.astype(np.float64) * 2).astype(np.float16)
    m2 = (dmin.astype(np.float64) * 2).astype(np.float16)
    y2, s2 = o.matmul("q4_k", x, synth.pack_q4_k(d2, m2, sc, mn, q), n, k)
    assert np.array_equal(y2, 2 * y) and np.array_equal(s2, 2 * s), "q4_k: y(2d, 2dmin) != 2y"
    rp = rng.permutation(n)
    yr, _ = o.matmul("q4_k", x, synth.pack_q4_k(d[rp], dmin[rp], sc[rp], mn[rp], q[rp]), n, k)
    assert np.array_equal(yr, y[:, rp]), "q4_k: row permutation"


ALL = [half_decode, golden, exact_rational, library_matmul, one_hot, zero_point,
       extreme_nibbles, subnormal_scale, linear_in_d, integer_exact, q8_min,
       permutations, special_values, gelu_tanh_form, ffn_gate_up,
       q4k_library_matmul, q4k_one_hot, q4k_zero, q4k_mins_only, q4k_integer_exact,
       q4k_linear_and_rows]


def failures(o, quick=True):
    """Names of the pins ``o`` fails (quick: fewer rational cases)."""
    failed = []
    for pin in ALL:
        try:
            if pin is exact_rational and quick:
                pin(o, cases=24)
            elif pin is library_matmul and quick:
                pin(o, shapes=((2, 40, 256),))
            elif pin is q4k_library_matmul and quick:
                pin(o, shapes=((2, 40, 512),))
            else:
                pin(o)
        except Exception:  # an assertion, or a value no pin can even read
            failed.append(pin.__name__)
    return failed
