"""Pins of the CPU oracle against what the pages and plain mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, hand derivations from the pages' formulas, exact rational
arithmetic (``fractions``), brute force over all codes on tiny inputs, closed
forms and invariants.  Several tests plant a plausible mistake in a copy of an
oracle step and check that the pin catches it.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
from oracle import gq_oracle as O
import synth


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def _f16_values():
    """All finite non-negative fp16 values, as Fractions, ascending."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits, [Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64)]


def _nearest_even(x: Fraction, grid_bits, grid):
    """Nearest grid value to x >= 0 (ties to the even bit pattern); exact."""
    import bisect
    i = bisect.bisect_left(grid, x)
    if i < len(grid) and grid[i] == x:
        return int(grid_bits[i])
    if i == 0:
        return int(grid_bits[0])
    if i == len(grid):
        return None
    a, b = grid[i - 1], grid[i]
    if x - a < b - x:
        return int(grid_bits[i - 1])
    if x - a > b - x:
        return int(grid_bits[i])
    return int(grid_bits[i - 1]) if grid_bits[i - 1] % 2 == 0 else int(grid_bits[i])


def test_f16_cast_is_single_rounding():
    grid_bits, grid = _f16_values()
    rng = np.random.default_rng(5)
    vals = list(np.exp(rng.uniform(np.log(1e-7), np.log(6e4), 3000)))
    # midpoints +- tiny: a float32 detour would round these twice
    for h in (1.0, 0.0078125, 3.0, 0.260009765625, 1000.0, 2.0 ** -20):
        ulp = float(np.spacing(np.float16(h)))
        for d in (2.0 ** -40, -(2.0 ** -40), 0.0):
            vals.append(h + ulp / 2 + d * h)
    for v in vals:
        got = int(O.f64_to_f16_bits(np.array([v]))[0])
        want = _nearest_even(Fraction(v), grid_bits, grid)
        assert got == want, (v, got, want)


def test_bf16_rounding_matches_exact_nearest():
    # bf16 grid around 1: spacing 2^-7
    for num in range(0, 1 << 10):
        v = 1.0 + num * 2.0 ** -16                       # exact in float32
        got = int(O.f32_exact_to_bf16_bits(np.array([v]))[0])
        frac = Fraction(v) - 1
        steps = frac / Fraction(1, 128)
        lo = math.floor(steps)
        rem = steps - lo
        k = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else 0)
        assert got == 0x3F80 + k, (v, hex(got))


# ---------------------------------------------------------------------------
# page-printed worked examples
# ---------------------------------------------------------------------------

def test_p3_worked_example_printed_step_and_bound():
    g = read_golden("p3_worked_example.txt")
    x = np.array([[float(v) for v in g["input"].split()]])
    codes, s, z = O.quantize_groups(x, int(g["bits"]), x.shape[1], symmetric=False)
    S = float(s[0, 0])
    printed = f"INT4 step {S:.2f}, error <= {S / 2:.2f}"
    assert printed == g["printed"]
    assert S == float(g["scale_fp16"])
    assert int(z[0, 0]) == int(g["zero"])
    assert codes[0].tolist() == [int(c) for c in g["codes"].split()]
    xhat = O.dequantize_codes(codes, s, z, x.shape[1])
    assert np.all(np.abs(x - xhat) <= S / 2)          # bound of the same page


def test_p1_worked_example_hand_derived():
    g = read_golden("p1_worked_example.txt")
    x = np.array([[float(v) for v in g["input"].split()]])
    for key, G, nmeta in (("tensor", 8, 1), ("group4", 4, 2)):
        codes, s, z = O.quantize_groups(x, 4, G, symmetric=False, fp16_scale=False)
        assert s.shape[1] == nmeta                      # the listing's asserts
        assert codes[0].tolist() == [int(c) for c in g[f"{key}_codes"].split()]
        meta = [float(v) for v in g[f"{key}_meta"].split()]
        for gi in range(nmeta):
            assert s[0, gi] == pytest.approx(meta[2 * gi], rel=1e-15)
            assert z[0, gi] == meta[2 * gi + 1]
        mae = np.abs(x - O.dequantize_codes(codes, s, z, G)).mean()
        assert mae == pytest.approx(float(g[f"{key}_mae"]), rel=1e-12)
    # the page's remark: per-group is not guaranteed to have lower error
    assert float(g["group4_mae"]) > float(g["tensor_mae"])


def test_p1_byte_counts():
    g = read_golden("p1_byte_counts.txt")
    for n, G, payload, meta, total in (map(int, r) for r in g["_rows"]):
        qb, sb, zb = O.packed_sizes(1, n, G, symmetric=False)
        assert (qb, sb + zb, qb + sb + zb) == (payload, meta, total)


def test_effective_bits():
    g = read_golden("p2_effective_bits.txt")
    for scheme, G, sym, meta, bpw in g["_rows"]:
        G, meta, bpw = int(G), int(meta), float(bpw)
        if scheme == "superblock":
            assert O.Q4K_BYTES * 8 / O.Q4K_BLOCK == bpw
            assert O.Q4K_BYTES == 128 + meta
        else:
            qb, sb, zb = O.packed_sizes(1, G * 64, G, symmetric=bool(int(sym)))
            assert sb / 64 == meta and zb == 0
            assert (qb + sb + zb) * 8 / (G * 64) == bpw


# ---------------------------------------------------------------------------
# exact arithmetic / brute force
# ---------------------------------------------------------------------------

def _fp16_grid():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


F16_GRID = _fp16_grid()


def _exact_scale(lo, hi, qrange):
    """Nearest fp16 to the exact rational (hi-lo)/qrange, by search."""
    t = (Fraction(hi) - Fraction(lo)) / qrange
    i = int(np.searchsorted(F16_GRID, float(t)))
    cands = [F16_GRID[j] for j in (i - 1, i, i + 1) if 0 <= j < len(F16_GRID)]
    best = min(cands, key=lambda c: (abs(Fraction(c) - t),
                                     int(np.float16(c).view(np.uint16)) % 2))
    return best


def _bf16_values(rng, n, std):
    return O.bf16_to_f64(synth.f32_to_bf16_bits(rng.normal(0, std, n).astype(np.float32)))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("symmetric", [False, True])
def test_brute_force_codes_and_scale(bits, symmetric):
    rng = np.random.default_rng(100 + bits + 10 * symmetric)
    qmin, qmax = O.code_range(bits, symmetric)
    for trial in range(300):
        n = int(rng.integers(2, 9))
        g = _bf16_values(rng, n, float(rng.choice([0.01, 1.0, 30.0])))
        if trial % 7 == 0:
            g = np.abs(g)                               # all-positive group
        if trial % 11 == 0:
            g[int(rng.integers(n))] = 0.0
        codes, s, z = O.quantize_groups(g[None, :], bits, n, symmetric)
        S = s[0, 0]
        # the scale is the nearest fp16 to the exact min-max / max-abs quotient
        if symmetric:
            want = _exact_scale(0.0, np.abs(g).max(), qmax) if np.abs(g).max() > 0 else 1.0
        else:
            lo, hi = min(g.min(), 0.0), max(g.max(), 0.0)
            want = _exact_scale(lo, hi, qmax - qmin) if hi != lo else 1.0
        assert S == want
        zz = 0 if symmetric else int(z[0, 0])
        if not symmetric:
            # zero point: nearest integer to -lo/S (exactly), clamped
            t = -Fraction(min(g.min(), 0.0)) / Fraction(S)
            zr = math.floor(t + Fraction(1, 2))
            if t + Fraction(1, 2) == zr and zr % 2:        # exact tie -> even
                zr -= 1
            assert zz == min(max(zr, qmin), qmax)
        # each code minimises |x - S (q - z)| over every admissible code
        for xv, q in zip(g, codes[0]):
            errs = [abs(Fraction(xv) - Fraction(S) * (c - zz)) for c in range(qmin, qmax + 1)]
            best = min(errs)
            assert errs[q - qmin] == best, (xv, q, S, zz)
            ties = [c for c in range(qmin, qmax + 1) if errs[c - qmin] == best]
            if len(ties) > 1:
                assert (q - zz) % 2 == 0                # round half to even


def test_error_bound_and_exact_zero():
    rng = np.random.default_rng(7)
    for symmetric in (False, True):
        for G in (32, 128):
            w = _bf16_values(rng, 64 * 512, 0.02).reshape(64, 512)
            w[:, ::37] = 0.0
            w[3] = np.abs(w[3])                          # all-positive row
            codes, s, z = O.quantize_groups(w, 4, G, symmetric)
            xh = O.dequantize_codes(codes, s, z, G)
            qmin, qmax = O.code_range(4, symmetric)
            S = np.repeat(s, G, axis=1)
            Z = 0.0 if symmetric else np.repeat(z, G, axis=1)
            inr = (w >= S * (qmin - Z)) & (w <= S * (qmax - Z))
            assert inr.mean() > 0.9
            assert np.all(np.abs(w - xh)[inr] <= S[inr] / 2)
            assert np.all(xh[w == 0] == 0.0)             # exact zero
            if symmetric:
                assert codes.min() >= -7                 # -8 never produced
            else:
                assert np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= 15


def test_degenerate_and_saturating_scales():
    w = np.zeros((1, 32))
    c, s, z = O.quantize_groups(w, 4, 32, False)
    assert s[0, 0] == 1.0 and z[0, 0] == 0 and np.all(c == 0)
    c, s, _ = O.quantize_groups(w, 4, 32, True)
    assert s[0, 0] == 1.0 and np.all(c == 0)
    w = np.full((1, 32), 0.5)
    c, s, z = O.quantize_groups(w, 4, 32, False)       # range [0, 0.5]
    assert z[0, 0] == 0 and np.all(c == 15) and s[0, 0] == float(np.float16(0.5 / 15))
    w = np.array([[-1e9] + [1e9] * 31])                  # beyond fp16 range
    c, s, z = O.quantize_groups(w, 4, 32, False)
    assert s[0, 0] == 65504.0
    w = np.array([[1e-9] * 32])                          # underflows fp16
    c, s, z = O.quantize_groups(w, 4, 32, False)
    assert s[0, 0] == 2.0 ** -24


# ---------------------------------------------------------------------------
# packing and dequantization
# ---------------------------------------------------------------------------

def test_pack_nibble_order_and_roundtrip():
    codes = np.array([[1, 2, 15, 0, 7, 8]])
    qw = O.pack_int4(codes, symmetric=False)
    assert qw.tolist() == [[0x21, 0x0F, 0x87]]          # low nibble = even k
    sym = np.array([[-8, 7, 0, -1]])
    assert O.pack_int4(sym, symmetric=True).tolist() == [[0xF0, 0x78]]
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, size=(5, 64))
    assert np.array_equal(O.unpack_int4(O.pack_int4(c, False), False), c)
    c = rng.integers(-8, 8, size=(5, 64))
    assert np.array_equal(O.unpack_int4(O.pack_int4(c, True), True), c)


def test_dequant_closed_form():
    rng = np.random.default_rng(11)
    w = synth.weights(8, 256, seed=1)[0]
    for symmetric in (False, True):
        codes, sb, zb = O.quantize_to_storage(w, 4, 64, symmetric)
        qw = O.pack_int4(codes, symmetric)
        xh = O.dequantize_packed(qw, sb, zb, 64, symmetric)
        for _ in range(200):
            n, k = int(rng.integers(8)), int(rng.integers(256))
            byte = int(qw[n, k // 2])
            nib = (byte >> (4 * (k % 2))) & 15
            S = Fraction(float(np.uint16(sb[n, k // 64]).view(np.float16)))
            zz = 8 if symmetric else int(float(np.uint16(zb[n, k // 64]).view(np.float16)))
            assert Fraction(xh[n, k]) == S * (nib - zz)


# ---------------------------------------------------------------------------
# matmul
# ---------------------------------------------------------------------------

def test_matmul_brute_force_tiny():
    rng = np.random.default_rng(21)
    for M, N, K, G in ((1, 3, 64, 32), (2, 8, 64, 16), (2, 5, 48, 48)):
        x = _bf16_values(rng, M * K, 1.0).reshape(M, K)
        w = _bf16_values(rng, N * K, 0.02).reshape(N, K)
        codes, s, z = O.quantize_groups(w, 4, G, False)
        wh = O.dequantize_codes(codes, s, z, G)
        y = O.matmul_groupwise(x, wh, G)
        for m in range(M):
            for n in range(N):
                exact = sum(Fraction(x[m, k]) * Fraction(wh[n, k]) for k in range(K))
                assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)


def test_matmul_special_cases_and_second_route():
    rng = np.random.default_rng(22)
    N, K, G = 16, 256, 64
    w = synth.weights(N, K, seed=3)[0]
    codes, sb, zb = O.quantize_to_storage(w, 4, G, False)
    qw = O.pack_int4(codes, False)
    wh = O.dequantize_packed(qw, sb, zb, G, False)
    # one-hot activation picks out a column of W^
    for k in (0, 1, 77, 255):
        e = np.zeros((1, K)); e[0, k] = 1.0
        assert np.array_equal(O.matmul_groupwise(e, wh, G)[0], wh[:, k])
    # codes equal to the zero point give exactly zero
    zc = np.repeat(O.f16_to_f64(zb), G, axis=1).astype(np.int64)
    qz = O.pack_int4(zc, False)
    x = _bf16_values(rng, 3 * K, 1.0).reshape(3, K)
    assert np.all(O.w4a16_reference(synth.f32_to_bf16_bits(x.astype(np.float32)), qz, sb, zb, G, False) == 0.0)
    # single-group == textbook product; group loop agrees with one BLAS call
    y1 = O.matmul_groupwise(x, wh, K)
    y2 = O.matmul_groupwise(x, wh, G)
    ref = np.einsum("mk,nk->mn", x, wh)
    assert np.allclose(y1, ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(y2, ref, rtol=1e-12, atol=1e-14)
    # linearity in x
    x2 = _bf16_values(rng, 3 * K, 1.0).reshape(3, K)
    assert np.allclose(O.matmul_groupwise(x + x2, wh, G),
                       O.matmul_groupwise(x, wh, G) + O.matmul_groupwise(x2, wh, G), rtol=1e-12, atol=1e-13)


def test_tolerance_bar_accepts_bf16_rounding_and_rejects_mistakes():
    """The parity bar passes bf16 RNE of the exact product and fails planted
    mistakes of the kind a kernel could make (dropped zero point, swapped
    nibbles, scale from the wrong group, bf16-rounded dequantized weights)."""
    w, x = synth.decode_case("o")
    w, x = w[:512], x
    G = 128
    codes, sb, zb = O.quantize_to_storage(w, 4, G, False)
    qw = O.pack_int4(codes, False)
    ref = O.w4a16_reference(x, qw, sb, zb, G, False)
    wh = O.dequantize_packed(qw, sb, zb, G, False)
    x64 = O.bf16_to_f64(x)

    def passes(y):
        ok, _, _ = O.within_parity(y, ref, x64, wh)
        return ok

    y_rne = O.bf16_to_f64(O.f32_exact_to_bf16_bits(ref.astype(np.float32).astype(np.float64)))
    assert passes(y_rne)
    # planted: zero point dropped
    wz = O.dequantize_codes(codes, O.f16_to_f64(sb), None, G)
    assert not passes(O.matmul_groupwise(x64, wz, G))
    # planted: nibbles swapped within each byte
    sw = ((qw & 15) << 4) | (qw >> 4)
    assert not passes(O.w4a16_reference(x, sw.astype(np.uint8), sb, zb, G, False))
    # planted: scale of the neighbouring group
    sb2 = np.roll(sb, 1, axis=1)
    assert not passes(O.w4a16_reference(x, qw, sb2, zb, G, False))


def test_planted_half_away_rounding_is_caught():
    """Round-half-away-from-zero instead of half-to-even must fail the tie pin."""
    def bad_quant(g, S):
        return np.sign(g / S) * np.floor(np.abs(g / S) + 0.5)
    S = 0.5
    g = np.array([0.25, 0.75, -0.25])                   # exact ties 0.5, 1.5, -0.5
    good = np.rint(g / S)
    assert not np.array_equal(bad_quant(g, S), good)
    codes, s, _ = O.quantize_groups(np.array([[0.25, 0.75, -0.25, 3.5]]), 4, 4, True)
    # S = 3.5/7 = 0.5 exactly; ties go to even codes: 0, 2, 0, 7
    assert s[0, 0] == 0.5 and codes[0].tolist() == [0, 2, 0, 7]


# ---------------------------------------------------------------------------
# outlier behaviour stated by the pages (direction only)
# ---------------------------------------------------------------------------

def test_outlier_blowup_with_whole_row_scale():
    """Page 2 ("核心思路" and the widget notes): one scale over a range that holds
    outlier channels collapses ordinary weights onto two or three codes, and
    small groups confine the damage to the outlier's own group."""
    w, _ = synth.tiny_reference()
    wf = O.bf16_to_f64(w)
    ok = np.ones(512, bool); ok[[7, 300]] = False
    c128, s128, z128 = O.quantize_groups(wf, 4, 128, False)
    c512, s512, z512 = O.quantize_groups(wf, 4, 512, False)
    wh128 = O.dequantize_codes(c128, s128, z128, 128)
    wh512 = O.dequantize_codes(c512, s512, z512, 512)
    assert O.snr_db(wf, wh128) > O.snr_db(wf, wh512) + 3
    ordinary_codes_512 = [len(np.unique(c512[r, ok])) for r in range(256)]
    assert np.median(ordinary_codes_512) <= 4
    # group 1 (k=128..255) holds no outlier: its codes use most of the 16 levels
    assert np.median([len(np.unique(c128[r, 128:256])) for r in range(256)]) >= 12
    # on ordinary weights the grouped error is far smaller
    e128 = np.abs(wf - wh128)[:, 128:256].mean()
    e512 = np.abs(wf - wh512)[:, 128:256].mean()
    assert e512 > 3 * e128


# ---------------------------------------------------------------------------
# super-block format
# ---------------------------------------------------------------------------

def test_q4k_fields_codes_and_bytes():
    rng = np.random.default_rng(31)
    w = synth.weights(4, 1024, seed=9)[0]
    wf = O.bf16_to_f64(w)
    wf[1, 256:512] = 0.0                                 # an all-zero block
    wf[2, 32:64] = 0.0                                   # an all-zero sub-block
    f = O.q4k_quantize(wf)
    blocks = O.q4k_encode(f)
    assert blocks.shape == (4, 4, 144)
    g = O.q4k_decode(blocks)
    for key in ("d", "dmin", "sc", "mn", "q"):
        assert np.array_equal(np.asarray(f[key]), np.asarray(g[key])), key
    wh = O.q4k_dequantize_fields(f)
    assert np.all(wh[1, 256:512] == 0.0) and np.all(wh[2, 32:64] == 0.0)
    sub = wf.reshape(4, 4, 8, 32)
    for n in range(4):
        for b in range(4):
            s = np.array([(max(v.max(), 0) - min(v.min(), 0)) / 15 for v in sub[n, b]])
            m = np.array([-min(v.min(), 0) for v in sub[n, b]])
            d, dmin = f["d"][n, b], f["dmin"][n, b]
            if s.max() > 0:
                # d is the nearest fp16 to the exact max_j (hi_j - lo_j) / (15 * 63)
                j = int(np.argmax(s))
                v = sub[n, b, j]
                assert d == _exact_scale(min(v.min(), 0), max(v.max(), 0), 15 * 63)
                for j in range(8):
                    errs = [abs(Fraction(s[j]) - Fraction(d) * c) for c in range(64)]
                    assert errs[f["sc"][n, b, j]] == min(errs)
            if m.max() > 0:
                for j in range(8):
                    errs = [abs(Fraction(m[j]) - Fraction(dmin) * c) for c in range(64)]
                    assert errs[f["mn"][n, b, j]] == min(errs)
            for j in range(8):
                S = Fraction(d) * int(f["sc"][n, b, j])
                Mn = Fraction(dmin) * int(f["mn"][n, b, j])
                for t in range(0, 32, 3):
                    k = b * 256 + j * 32 + t
                    q = int(f["q"][n, k])
                    xv = Fraction(wf[n, k])
                    errs = [abs(xv - (S * c - Mn)) for c in range(16)]
                    assert errs[q] == min(errs)
                    if S > 0 and -Mn <= xv <= S * 15 - Mn:
                        assert errs[q] <= S / 2
    # bytes: 144 per 256 weights, d/dmin at offsets 0/2 as fp16
    assert blocks[0, 0, 0:2].view(np.uint16)[0] == np.float16(f["d"][0, 0]).view(np.uint16)


def test_q4k_reference_matches_dense_product():
    w = synth.weights(8, 512, seed=12)[0]
    x, _ = synth.activations(2, 512, seed=13)
    blocks = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(w)))
    wh = O.q4k_dequantize_fields(O.q4k_decode(blocks))
    y = O.q4k_reference(x, blocks)
    ref = O.bf16_to_f64(x) @ wh.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    assert O.snr_db(O.bf16_to_f64(w), wh) > 15


def test_bf16_half_ulp_closed_form():
    # bf16 keeps 8 significant bits: spacing 2^(e-7) in [2^e, 2^(e+1))
    for v, want in ((1.0, 2.0 ** -8), (1.99, 2.0 ** -8), (2.0, 2.0 ** -7), (10.0, 2.0 ** -5),
                    (-0.3, 2.0 ** -10), (0.0, 2.0 ** -134)):
        assert float(O.bf16_half_ulp(np.array([v]))[0]) == want
    # a value and its bf16 rounding differ by at most half an ulp
    rng = np.random.default_rng(2)
    v = rng.normal(0, 10, 5000).astype(np.float32).astype(np.float64)
    r = O.bf16_to_f64(O.f32_exact_to_bf16_bits(v))
    assert np.all(np.abs(r - v) <= O.bf16_half_ulp(v))


def test_group_major_ingest_preserves_the_product():
    """The chapter's layout (codes [n_groups, group, N], scales [n_groups, N]) and
    its group-by-group product out += x[:, g] @ (q[g] * s[g]) must give, after
    ingest into [N, K/2] + [N, K/G], exactly the canonical oracle product; a
    transposed slab or a swapped nibble would not."""
    rng = np.random.default_rng(11)
    ng, g, n, m = 5, 32, 24, 3
    codes = rng.integers(-8, 8, size=(ng, g, n))
    scales = O.f64_to_f16_bits(rng.uniform(0.001, 0.05, size=(ng, n)))
    x = O.f32_exact_to_bf16_bits(rng.normal(size=(m, ng * g)).astype(np.float32).astype(np.float64))
    xf = O.bf16_to_f64(x)
    s = O.f16_to_f64(scales)
    page = np.zeros((m, n))
    for gi in range(ng):   # the page's fused form, written independently of the oracle
        page += xf[:, gi * g:(gi + 1) * g] @ (codes[gi].astype(np.float64) * s[gi])
    qw, sc = O.ingest_group_major(codes, scales)
    assert qw.shape == (n, ng * g // 2) and sc.shape == (n, ng)
    assert np.array_equal(O.unpack_int4(qw, True)[3, 32:64], codes[1, :, 3])
    canon = O.w4a16_reference(x, qw, sc, None, g, True)
    assert np.allclose(canon, page, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the element-wise half of the parity bar
# ---------------------------------------------------------------------------

def test_max_err_bound_closed_form():
    """1e-2 * max|x| * max|w^| * sqrt(K) / 64 with max|x| = 2, max|w^| = 3 and
    K = 4096 is 1e-2 * 2 * 3 * 64 / 64 = 0.06; the maxima are of absolute values
    and K is the reduction length (the number of columns of x)."""
    x = np.zeros((2, 4096)); x[1, 17] = -2.0; x[0, 3] = 1.5
    w = np.zeros((5, 4096)); w[4, 100] = -3.0; w[2, 7] = 2.9
    assert abs(O.max_err_bound(x, w) - 0.06) < 1e-15
    # K from x's columns: a quarter of the length halves the bound
    assert abs(O.max_err_bound(x[:, :1024], w[:, :1024]) - 0.03) < 1e-15


def test_f16_half_ulp_closed_form():
    # binary16 keeps 11 significant bits: spacing 2^(e-10) in [2^e, 2^(e+1)),
    # subnormal spacing 2^-24 below 2^-14
    for v, want in ((1.0, 2.0 ** -11), (1.99, 2.0 ** -11), (2.0, 2.0 ** -10), (10.0, 2.0 ** -8),
                    (-0.3, 2.0 ** -13), (2.0 ** -14, 2.0 ** -25), (1e-6, 2.0 ** -25),
                    (0.0, 2.0 ** -25)):
        assert float(O.f16_half_ulp(np.array([v]))[0]) == want
    rng = np.random.default_rng(4)
    v = rng.normal(0, 10, 5000)
    r = v.astype(np.float16).astype(np.float64)
    assert np.all(np.abs(r - v) <= O.f16_half_ulp(v))


def test_element_bound_rejects_what_frobenius_accepts():
    """An error on a single output that the relative Frobenius half cannot see
    (20000 outputs of 10) must still be rejected once it exceeds the element
    bound 0.06 plus half an output ulp, and accepted just below it; the bound of
    fp16 outputs uses fp16's half ulp (2^-8 at 10), bf16's uses 2^-5."""
    x = np.zeros((1, 4096)); x[0, 9] = 2.0
    w = np.zeros((3, 4096)); w[1, 11] = -3.0
    ref = np.full((1, 20000), 10.0)
    for out, half in (("bf16", 2.0 ** -5), ("f16", 2.0 ** -8)):
        allow = 0.06 + half
        y = ref.copy(); y[0, 123] += 1.04 * allow
        ok, rel, ratio = O.within_parity(y, ref, x, w, out=out)
        assert rel < 2e-3 and not ok and 1.0 < ratio < 1.05, (out, rel, ratio)
        y = ref.copy(); y[0, 123] -= 0.96 * allow
        ok, rel, ratio = O.within_parity(y, ref, x, w, out=out)
        assert ok and 0.95 < ratio < 1.0, (out, rel, ratio)
    # the Frobenius half on its own: a uniform relative error of 3e-3 fails
    y = ref * (1 + 3e-3)
    ok, rel, _ = O.within_parity(y, ref, x * 1e3, w, out="bf16")
    assert not ok and abs(rel - 3e-3) < 1e-9


# ---------------------------------------------------------------------------
# super-block format: scale-of-mins, byte layout, signed zero
# ---------------------------------------------------------------------------

def test_q4k_dmin_is_nearest_fp16_of_max_min_over_63():
    """dmin is the fp16 nearest to the exact max_j(0 - lo_j) / 63, as d is the
    fp16 nearest to max_j (hi_j - lo_j) / (15 * 63)."""
    w = synth.weights(6, 1024, seed=21)[0]
    wf = O.bf16_to_f64(w)
    f = O.q4k_quantize(wf)
    sub = wf.reshape(6, 4, 8, 32)
    checked = 0
    for n in range(6):
        for b in range(4):
            m = np.array([-min(v.min(), 0.0) for v in sub[n, b]])
            assert m.max() > 0
            j = int(np.argmax(m))
            want = _exact_scale(min(sub[n, b, j].min(), 0.0), 0.0, 63)
            assert f["dmin"][n, b] == want, (n, b)
            checked += 1
    assert checked == 24


def test_q4k_hand_built_block_bytes():
    """Encode and decode of a block whose fields were chosen by hand, against
    the literal bytes derived in the fixture (d, dmin, sc, mn at offsets 0, 2,
    4, 10; nibbles from 16)."""
    gd = read_golden("q4k_block_layout.txt")
    f = {"d": np.array([[float(gd["d"])]]), "dmin": np.array([[float(gd["dmin"])]]),
         "sc": np.array([[[int(v) for v in gd["sc"].split()]]]),
         "mn": np.array([[[int(v) for v in gd["mn"].split()]]]),
         "q": (np.arange(256) % 16)[None, :].astype(np.int64)}
    want = np.array([int(v, 16) for v in gd["header_hex"].split()]
                    + [int(v, 16) for v in gd["nibble_hex"].split()] * 16, dtype=np.uint8)
    assert want.size == 144
    blk = O.q4k_encode(f)
    assert blk.shape == (1, 1, 144)
    assert np.array_equal(blk[0, 0], want)
    g = O.q4k_decode(want.reshape(1, 1, 144))
    for key in ("d", "dmin", "sc", "mn", "q"):
        assert np.array_equal(np.asarray(g[key]), np.asarray(f[key])), key
    wh = O.q4k_dequantize_fields(g)
    assert wh[0, 5] == float(gd["xhat_k5"]) and wh[0, 255] == float(gd["xhat_k255"])


def test_q4k_zero_min_is_positive_zero():
    """A block with no negative weight has every sub-block min 0 - 0 = +0, so
    dmin is stored as +0 (0x0000) and every mn field is 0; an all-zero block
    stores d = +0 as well."""
    w = np.abs(O.bf16_to_f64(synth.weights(2, 512, seed=5)[0]))
    w[1, 256:] = 0.0
    blocks = O.q4k_encode(O.q4k_quantize(w))
    hdr = blocks[..., 0:4].copy().view(np.uint16)       # [N, nb, 2]: d, dmin
    assert np.all(hdr[..., 1] == 0x0000)                 # dmin = +0, not 0x8000
    assert np.all(blocks[..., 10:16] == 0)               # mn fields
    assert hdr[1, 1, 0] == 0x0000 and hdr[0, 0, 0] != 0
