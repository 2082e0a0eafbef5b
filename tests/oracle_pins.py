"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Each ``pin_*`` takes an oracle module ``o`` so that the same checks can be run
against deliberately broken copies of the oracle (tests/test_oracle_mutations.py):
every planted mistake must make at least one pin fail.

Independent means: bf16 values are decoded here with ``struct`` (not the
oracle's numpy bit view), nibbles are read here with Python integer ops,
brute-force sums use exact rationals (``fractions.Fraction``), and expected
values come either from the pages' printed constants (tests/golden/), from a
closed form, or from an invariant of the definition.
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers

def bf16_value(bits: int) -> float:
    """Decode one bf16 bit pattern with struct (independent of the oracle)."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def f32_round(v: float) -> float:
    """Round a Python float (binary64) to binary32 via struct (the C library's
    conversion, round to nearest even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def nibble(p_row: np.ndarray, k: int) -> int:
    b = int(p_row[k // 2])
    return (b >> 4) & 0xF if k % 2 else b & 0xF


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def rand_case(M, N, K, seed, G=None, m_sizes=None, group=128):
    from synth import make_inputs
    return make_inputs(M, N, K, seed, G=G, m_sizes=m_sizes, group=group)


def bf16_scale_samples():
    """bf16 bit patterns for the sample scales: 0.005, 0.02, 2^-7, 2^-6, the
    smallest bf16 >= 0.005 and the largest bf16 < 0.02, plus 256 draws from
    the workload's scale distribution."""
    out = set()
    for v in (0.005, 0.02, 2.0 ** -7, 2.0 ** -6):
        b = f32_bits(f32_round(v)) >> 16
        out.update([b, b + 1, b - 1])
    lo = next(b for b in range(0x3B00, 0x3D00) if bf16_value(b) >= 0.005)
    hi = max(b for b in range(0x3B00, 0x3D00) if bf16_value(b) < 0.02)
    out.update([lo, hi])
    rng = np.random.default_rng(123)
    for v in rng.uniform(0.005, 0.02, 256):
        out.add(f32_bits(f32_round(float(v))) >> 16)
    return sorted(out)


# ------------------------------------------------------------------ bf16

def pin_bf16_decode_page_constants(o):
    """The page's magic constants decode to the values it states."""
    for name, hexbits, val in read_golden("magic_dequant_constants.txt"):
        bits = int(hexbits, 16)
        got = float(o.bf16_to_f64(np.array([bits], dtype=np.uint16))[0])
        assert got == float(val), (name, hexbits, got, val)
        assert got == bf16_value(bits)


def pin_bf16_decode_exhaustive(o):
    """All 65536 bf16 patterns decode like struct's float32 decode."""
    bits = np.arange(65536, dtype=np.uint32)
    got = o.bf16_to_f64(bits.astype(np.uint16))
    ref = np.array([bf16_value(int(b)) for b in bits], dtype=np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert bool(np.all(same))


def pin_rne_known_values(o):
    """Hand-derived round-to-nearest-even cases, built from bit patterns."""
    cases = [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # 1 + 2^-8: tie, kept LSB even -> stays
        (0x3F818000, 0x3F82),  # 1 + 3*2^-8: tie, kept LSB odd -> up
        (0x3F808001, 0x3F81),  # just above the tie -> up
        (0x3F807FFF, 0x3F80),  # just below the tie -> down
        (0xBF818000, 0xBF82),  # negative tie, odd -> away from zero
        (0x80000000, 0x8000),  # -0.0
        (0x7F800000, 0x7F80),  # +inf
        (0xFF800000, 0xFF80),  # -inf
        (0x7F7FFFFF, 0x7F80),  # FLT_MAX rounds to +inf
        (0x00008000, 0x0000),  # subnormal tie at zero -> even (0)
        (0x00018000, 0x0002),  # subnormal tie, odd -> up
        (0x43088000, 0x4308),  # 136.5 -> 136 (tie to even)
    ]
    a = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = o.f32_to_bf16_rne(a)
    for (src, want), g in zip(cases, got):
        assert int(g) == want, (hex(src), hex(int(g)), hex(want))
    nan = o.f32_to_bf16_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_value(int(nan[0])))


def pin_rne_roundtrip_and_monotone(o):
    """Every finite bf16 value converts back to itself; rounding any float32
    lands on one of its two bf16 neighbours, the nearer one."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    fin = np.isfinite(f)
    back = o.f32_to_bf16_rne(f[fin])
    assert np.array_equal(back.astype(np.uint32), bits[fin])
    rng = np.random.default_rng(7)
    u = rng.integers(0, 0x7F7F0000, 4000, dtype=np.uint32)
    u |= rng.integers(0, 2, 4000, dtype=np.uint32) << 31
    x = u.view(np.float32)
    r = o.f32_to_bf16_rne(x)
    for xi, ri, ui in zip(x, r, u):
        down = int(ui) >> 16
        cand = [down, down + 1]
        assert int(ri) in cand
        err = abs(bf16_value(int(ri)) - float(xi))
        other = cand[1] if int(ri) == cand[0] else cand[0]
        assert err <= abs(bf16_value(other) - float(xi))


# ------------------------------------------------------------------ packing

def pin_pack_page_byte_order(o):
    for qe, qo, hexb in read_golden("nibble_order.txt"):
        q = np.array([[int(qe), int(qo)]], dtype=np.uint8)
        assert int(o.pack_int4(q)[0, 0]) == int(hexb, 16)
        back = o.unpack_int4(np.array([[int(hexb, 16)]], dtype=np.uint8))
        assert back.tolist() == [[int(qe), int(qo)]]


def pin_pack_unpack_exhaustive(o):
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = o.unpack_int4(b)
    for j in range(256):
        assert int(q[0, 2 * j]) == j & 0xF and int(q[0, 2 * j + 1]) == j >> 4
    assert np.array_equal(o.pack_int4(q), b)
    hi_bits = (q | np.uint8(0xF0)).astype(np.uint8)   # high bits are ignored
    assert np.array_equal(o.pack_int4(hi_bits), b)


# ------------------------------------------------------------------ dequant

def pin_dequant_magic_identity(o):
    """For every nibble n and every sample scale s, the oracle's dequantised
    weight equals the page's route s*bf16(0x4300|n) + s*bf16(0xC308), in
    exact rationals."""
    golden = {r[0]: (int(r[1], 16), float(r[2]))
              for r in read_golden("magic_dequant_constants.txt")}
    neg = Fraction(bf16_value(golden["pair"][0]))
    scales = bf16_scale_samples()
    K = 16 * 128   # 16 groups, nibble n fills group n
    q = np.repeat(np.arange(16, dtype=np.uint8), 128).reshape(1, K)
    p = o.pack_int4(q)
    for sb in scales:
        s = np.full((1, 16), sb, dtype=np.uint16)
        wd = o.dequant(p, s)
        sv = Fraction(bf16_value(sb))
        for n in range(16):
            magic = Fraction(bf16_value(golden["base"][0] | n))
            want = sv * magic + sv * neg
            got = wd[0, n * 128: (n + 1) * 128]
            assert np.all(got == float(want)), (hex(sb), n, got[0], float(want))


def pin_one_hot_rows(o):
    """X = e_k gives Y[i, n] = S[n, k // 128] * (nibble(P[n], k) - 8): pins
    the nibble order, the scale index and the operand orientation."""
    c = rand_case(1, 7, 384, seed=11)
    p = o.pack_int4(c.q)
    ks = [0, 1, 2, 127, 128, 129, 255, 256, 383]
    x = np.zeros((len(ks), 384), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80   # 1.0
    y = o.gemm(x, p, c.s)
    assert y.shape == (len(ks), 7)
    for i, k in enumerate(ks):
        for n in range(7):
            want = bf16_value(int(c.s[n, k // 128])) * (nibble(p[n], k) - 8)
            assert y[i, n] == want, (k, n, y[i, n], want)


def _brute(x_bits, p, s_bits, group=128):
    M, K = x_bits.shape
    N = p.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    mag = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            am = Fraction(0)
            for k in range(K):
                xv = Fraction(bf16_value(int(x_bits[m, k])))
                wv = Fraction(bf16_value(int(s_bits[n, k // group]))) * (nibble(p[n], k) - 8)
                acc += xv * wv
                am += abs(xv * wv)
            y[m][n] = acc
            mag[m][n] = am
    return y, mag


def pin_brute_force_tiny(o):
    """Exact rational triple loop vs the vectorised oracle on tiny shapes,
    random plus extreme inputs; bound 1e-12 * sum|x*w|."""
    shapes = [(1, 1, 128), (1, 3, 256), (2, 5, 128), (3, 4, 384)]
    for idx, (M, N, K) in enumerate(shapes):
        c = rand_case(M, N, K, seed=100 + idx)
        variants = [(c.x, c.q)]
        variants.append((c.x, np.zeros_like(c.q)))
        variants.append((c.x, np.full_like(c.q, 15)))
        xmax = int(c.x.ravel()[np.argmax(np.abs(o.bf16_to_f64(c.x)).ravel())]) & 0x7FFF
        xe = c.x.copy()
        xe[:, ::2] = xmax
        xe[:, 1::2] = xmax | 0x8000
        variants.append((xe, c.q))
        for xb, q in variants:
            p = o.pack_int4(q)
            y = o.gemm(xb, p, c.s)
            ref, mag = _brute(xb, p, c.s)
            for m in range(M):
                for n in range(N):
                    bound = 1e-12 * float(mag[m][n]) + 1e-300
                    assert abs(y[m, n] - float(ref[m][n])) <= bound, (M, N, K, m, n)


def pin_even_odd_identity(o):
    """[x_even | x_odd] . [w_lo | w_hi]^T == x_even.w_lo^T + x_odd.w_hi^T ==
    X.Wd^T (the concatenation identity of the fused A-operand dot), within
    float64 reassociation; and invariance under the permutation
    (0,4,1,5,2,6,3,7) of each 8-k chunk applied to both operands."""
    c = rand_case(5, 9, 512, seed=21)
    p = o.pack_int4(c.q)
    x = o.bf16_to_f64(c.x)
    wd = o.dequant(p, c.s)
    y = o.gemm(c.x, p, c.s)
    xe, xo = x[:, 0::2], x[:, 1::2]
    wlo, whi = wd[:, 0::2], wd[:, 1::2]
    cat = np.concatenate([xe, xo], 1) @ np.concatenate([wlo, whi], 1).T
    two = xe @ wlo.T + xo @ whi.T
    bound = 512 * 2.0 ** -52 * (np.abs(x) @ np.abs(wd).T) + 1e-300
    assert np.all(np.abs(cat - y) <= bound)
    assert np.all(np.abs(two - y) <= bound)
    perm = np.concatenate([8 * j + np.array([0, 4, 1, 5, 2, 6, 3, 7])
                           for j in range(512 // 8)])
    yp = x[:, perm] @ wd[:, perm].T
    assert np.all(np.abs(yp - y) <= bound)


def pin_zero_and_linearity(o):
    """q == 8 everywhere gives Y == 0 exactly; doubling every scale doubles
    Y exactly; negating X negates Y exactly."""
    c = rand_case(4, 6, 256, seed=31)
    p8 = o.pack_int4(np.full_like(c.q, 8))
    assert np.all(o.gemm(c.x, p8, c.s) == 0.0)
    p = o.pack_int4(c.q)
    y = o.gemm(c.x, p, c.s)
    s2 = (c.s.astype(np.uint32) + (1 << 7)).astype(np.uint16)   # exponent + 1
    assert np.all(o.gemm(c.x, p, s2) == 2.0 * y)
    xn = (c.x ^ np.uint16(0x8000)).astype(np.uint16)
    assert np.all(o.gemm(xn, p, c.s) == -y)


def pin_closed_form_ones(o):
    """X = all ones and a constant nibble c_g per (row, group) give the closed
    form Y[0, n] = sum_g 128 * s[n, g] * (c_g - 8)."""
    N, K = 5, 640
    rng = np.random.default_rng(41)
    cg = rng.integers(0, 16, (N, K // 128), dtype=np.uint8)
    q = np.repeat(cg, 128, axis=1)
    s = np.array([[f32_bits(f32_round(v)) >> 16 for v in row]
                  for row in rng.uniform(0.005, 0.02, (N, K // 128))],
                 dtype=np.uint16)
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    y = o.gemm(x, o.pack_int4(q), s)
    for n in range(N):
        want = sum(Fraction(128) * Fraction(bf16_value(int(s[n, g]))) * (int(cg[n, g]) - 8)
                   for g in range(K // 128))
        assert y[0, n] == float(want)


def pin_gemm_entries(o):
    c = rand_case(3, 11, 384, seed=51)
    p = o.pack_int4(c.q)
    rows = np.array([0, 2, 1, 2, 0])
    cols = np.array([10, 0, 5, 5, 3])
    e = o.gemm_entries(c.x, p, c.s, rows, cols)
    ref, mag = _brute(c.x[:, :], p, c.s)
    for i in range(5):
        assert abs(e[i] - float(ref[rows[i]][cols[i]])) <= 1e-12 * float(mag[rows[i]][cols[i]])


# ------------------------------------------------------------------ group 32
# The first page's kernel quantises with one scale per 32 k (its per-GEMM
# table, section "Results"); the definition is the same with k // 32.

def pin_group32_one_hot_rows(o):
    """X = e_k at group 32 gives S[n, k // 32] * (nibble - 8): pins the scale
    index at every 32-group boundary of a 128-k stage."""
    c = rand_case(1, 5, 256, seed=61, group=32)
    assert c.s.shape == (5, 8)
    p = o.pack_int4(c.q)
    ks = [0, 31, 32, 33, 63, 64, 95, 96, 127, 128, 160, 255]
    x = np.zeros((len(ks), 256), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80
    y = o.gemm(x, p, c.s, 32)
    e = o.gemm_entries(x, p, c.s, np.arange(len(ks)), np.full(len(ks), 3), 32)
    for i, k in enumerate(ks):
        for n in range(5):
            want = bf16_value(int(c.s[n, k // 32])) * (nibble(p[n], k) - 8)
            assert y[i, n] == want, (k, n, y[i, n], want)
        assert e[i] == y[i, 3]


def pin_group32_brute_force(o):
    """Exact rational triple loop at group 32 (random and all-15 weights) vs
    the oracle's gemm and gemm_entries; bound 1e-12 * sum|x*w|."""
    for idx, (M, N, K) in enumerate([(1, 3, 128), (2, 4, 256), (3, 2, 384)]):
        c = rand_case(M, N, K, seed=200 + idx, group=32)
        for q in (c.q, np.full_like(c.q, 15)):
            p = o.pack_int4(q)
            y = o.gemm(c.x, p, c.s, 32)
            ref, mag = _brute(c.x, p, c.s, 32)
            rows = np.repeat(np.arange(M), N)
            cols = np.tile(np.arange(N), M)
            e = o.gemm_entries(c.x, p, c.s, rows, cols, 32)
            for i, (m, n) in enumerate(zip(rows, cols)):
                bound = 1e-12 * float(mag[m][n]) + 1e-300
                assert abs(y[m, n] - float(ref[m][n])) <= bound, (M, N, K, m, n)
                assert abs(e[i] - float(ref[m][n])) <= bound, (M, N, K, m, n)


def pin_group32_closed_form_ones(o):
    """X = all ones and a constant nibble c_g per (row, 32-group):
    Y[0, n] = sum_g 32 * s[n, g] * (c_g - 8), exactly."""
    N, K = 4, 384
    rng = np.random.default_rng(71)
    cg = rng.integers(0, 16, (N, K // 32), dtype=np.uint8)
    q = np.repeat(cg, 32, axis=1)
    s = np.array([[f32_bits(f32_round(v)) >> 16 for v in row]
                  for row in rng.uniform(0.005, 0.02, (N, K // 32))],
                 dtype=np.uint16)
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    y = o.gemm(x, o.pack_int4(q), s, 32)
    for n in range(N):
        want = sum(Fraction(32) * Fraction(bf16_value(int(s[n, g]))) * (int(cg[n, g]) - 8)
                   for g in range(K // 32))
        assert y[0, n] == float(want)


def pin_group32_refines_128(o):
    """Scales equal over each run of four 32-groups give exactly the group-128
    result with those scales (the dequantised weights are the same)."""
    c = rand_case(3, 6, 512, seed=81)
    s32 = np.repeat(c.s, 4, axis=1)
    p = o.pack_int4(c.q)
    assert np.array_equal(o.dequant(p, s32, 32), o.dequant(p, c.s, 128))
    assert np.array_equal(o.gemm(c.x, p, s32, 32), o.gemm(c.x, p, c.s, 128))


def pin_group32_grouped_and_batched_one_hot(o):
    """Grouped and batched at group 32 with one-hot rows: row i of group g
    (problem b) gives S_g[n, k_i // 32] * (nibble(P_g[n], k_i) - 8) with that
    group's own weights and scales; empty groups contribute no rows."""
    K, N = 256, 3
    ks = [0, 31, 32, 63, 64, 100, 127, 128, 159, 160, 200, 255]
    ms = [2, 0, 3, 4]
    c = rand_case(sum(ms), N, K, seed=91, G=len(ms), m_sizes=ms, group=32)
    p = o.pack_int4(c.q)
    x = np.zeros((sum(ms), K), dtype=np.uint16)
    row_k = [ks[(3 * i + 1) % len(ks)] for i in range(sum(ms))]
    for i, k in enumerate(row_k):
        x[i, k] = 0x3F80
    y = o.gemm_grouped(x, p, c.s, ms, 32)
    r = 0
    for g, m in enumerate(ms):
        for _ in range(m):
            k = row_k[r]
            for n in range(N):
                want = bf16_value(int(c.s[g, n, k // 32])) * (nibble(p[g, n], k) - 8)
                assert y[r, n] == want, (g, r, n, k)
            r += 1
    B, M = 3, 4
    cb = rand_case(B * M, N, K, seed=92, G=B, m_sizes=[M] * B, group=32)
    pb = o.pack_int4(cb.q)
    xb = np.zeros((B, M, K), dtype=np.uint16)
    for b in range(B):
        for i in range(M):
            xb[b, i, ks[(5 * b + 2 * i) % len(ks)]] = 0x3F80
    yb = o.gemm_batched(xb, pb, cb.s, 32)
    for b in range(B):
        for i in range(M):
            k = ks[(5 * b + 2 * i) % len(ks)]
            for n in range(N):
                want = bf16_value(int(cb.s[b, n, k // 32])) * (nibble(pb[b, n], k) - 8)
                assert yb[b, i, n] == want, (b, i, n, k)


# ------------------------------------------------------------------ split-K

def pin_splitk_ranges(o):
    assert o.splitk_group_ranges(3, 2) == [(0, 2), (2, 3)]
    assert o.splitk_group_ranges(3, 4) == [(0, 1), (1, 2), (2, 3), (3, 3)]
    assert o.splitk_group_ranges(64, 8) == [(8 * i, 8 * i + 8) for i in range(8)]
    assert o.splitk_group_ranges(40, 1) == [(0, 40)]
    for G in range(1, 70):
        for sk in (1, 2, 3, 4, 8, 16):
            r = o.splitk_group_ranges(G, sk)
            assert len(r) == sk and r[0][0] == 0 and r[-1][1] == G
            for (a0, a1), (b0, b1) in zip(r, r[1:]):
                assert a1 == b0 and a0 <= a1
            assert max(b - a for a, b in r) == -(-G // sk)


def pin_splitk_invariance(o):
    """sum_s Y_s == Y within float64 reassociation, including a K that the
    split does not divide (3 groups) and an empty trailing slice."""
    for (M, N, K) in [(2, 5, 384), (3, 4, 1024)]:
        c = rand_case(M, N, K, seed=61 + K)
        p = o.pack_int4(c.q)
        y = o.gemm(c.x, p, c.s)
        x = o.bf16_to_f64(c.x)
        wd = o.dequant(p, c.s)
        bound = K * 2.0 ** -52 * (np.abs(x) @ np.abs(wd).T) * 4 + 1e-300
        for sk in (1, 2, 4, 8):
            part = o.gemm_splitk_partials(c.x, p, c.s, sk)
            assert part.shape == (sk, M, N)
            assert np.all(np.abs(part.sum(0) - y) <= bound)
            for s, (g0, g1) in enumerate(o.splitk_group_ranges(K // 128, sk)):
                k0, k1 = g0 * 128, g1 * 128
                ref = x[:, k0:k1] @ wd[:, k0:k1].T if k1 > k0 else np.zeros((M, N))
                assert np.all(np.abs(part[s] - ref) <= bound)


def pin_splitk_reduce(o):
    """The reduce is a float32 sum in slice order then RNE to bf16; checked
    with struct-based float32 rounding and bf16 decode, including exact ties."""
    from synth import make_workspace
    for sk in (1, 2, 3, 8):
        ws = make_workspace(sk, 3, 37, seed=70 + sk)
        got = o.splitk_reduce_bf16(ws)
        assert got.shape == (3, 37) and got.dtype == np.uint16
        for m in range(3):
            for n in range(37):
                acc = float(ws[0, m, n])
                for s in range(1, sk):
                    acc = f32_round(acc + float(ws[s, m, n]))
                b = int(got[m, n])
                lo_b = f32_bits(acc) >> 16
                # the result is one of the two bf16 neighbours, the nearer,
                # and on an exact tie the even one
                assert b in (lo_b, lo_b + 1)
                d = abs(bf16_value(b) - acc)
                other = lo_b + 1 if b == lo_b else lo_b
                do = abs(bf16_value(other) - acc)
                assert d <= do
                if d == do:
                    assert b % 2 == 0


# ------------------------------------------------------------------ grouped

def pin_group_starts(o):
    assert list(o.group_starts([3, 0, 5, 2])) == [0, 3, 3, 8]
    assert list(o.group_starts([0, 0])) == [0, 0]
    assert list(o.group_starts([7])) == [0]


def pin_grouped_matches_plain(o):
    """G = 1 equals the plain GEMM; G > 1 equals the per-group plain GEMMs
    stacked in group order, empty groups included."""
    c1 = rand_case(6, 5, 256, seed=81, G=1, m_sizes=[6])
    p1 = o.pack_int4(c1.q)
    assert np.array_equal(o.gemm_grouped(c1.x, p1, c1.s, c1.m_sizes),
                          o.gemm(c1.x, p1[0], c1.s[0]))
    ms = [3, 0, 4, 0, 1]
    c = rand_case(sum(ms), 6, 384, seed=82, G=5, m_sizes=ms)
    p = o.pack_int4(c.q)
    y = o.gemm_grouped(c.x, p, c.s, c.m_sizes)
    r = 0
    for g, mg in enumerate(ms):
        if mg:
            assert np.array_equal(y[r:r + mg], o.gemm(c.x[r:r + mg], p[g], c.s[g]))
            # and the row does NOT match another group's weights
            other = (g + 1) % 5
            assert not np.array_equal(y[r:r + mg], o.gemm(c.x[r:r + mg], p[other], c.s[other]))
        r += mg


# ------------------------------------------------------------------ batched

def pin_batched_matches_plain(o):
    """B = 1 equals the plain GEMM; B > 1 equals the per-problem plain GEMMs,
    each problem with its own weights (not a neighbour's), and equals the
    grouped GEMM with equal group sizes on the flattened rows; permuting the
    problems permutes the outputs."""
    c1 = rand_case(5, 7, 256, seed=93, G=1, m_sizes=[5])
    p1 = o.pack_int4(c1.q)
    x1 = c1.x.reshape(1, 5, 256)
    assert np.array_equal(o.gemm_batched(x1, p1, c1.s)[0], o.gemm(c1.x, p1[0], c1.s[0]))
    B, M, N, K = 3, 4, 6, 384
    c = rand_case(B * M, N, K, seed=94, G=B, m_sizes=[M] * B)
    p = o.pack_int4(c.q)
    xb = c.x.reshape(B, M, K)
    y = o.gemm_batched(xb, p, c.s)
    assert y.shape == (B, M, N)
    for b in range(B):
        assert np.array_equal(y[b], o.gemm(xb[b], p[b], c.s[b]))
        other = (b + 1) % B
        assert not np.array_equal(y[b], o.gemm(xb[b], p[other], c.s[other]))
    assert np.array_equal(y.reshape(B * M, N), o.gemm_grouped(c.x, p, c.s, [M] * B))
    perm = [2, 0, 1]
    assert np.array_equal(o.gemm_batched(xb[perm], p[perm], c.s[perm]), y[perm])


# ------------------------------------------------------------------ gate

def pin_gate(o):
    rng = np.random.default_rng(91)
    ref = rng.standard_normal((4, 50)) * 5
    bits = o.f32_to_bf16_rne(ref.astype(np.float32))
    g = o.gate(bits, ref)
    assert g["ok"] and g["max_err"] <= 2.0 ** -8 * np.max(np.abs(ref))
    tol = 4e-3 * np.max(np.abs(ref)) + 1e-3
    for sign in (1.0, -1.0):
        bad = ref.copy()
        bad[1, 7] += sign * 3 * tol
        assert not o.gate(o.f32_to_bf16_rne(bad.astype(np.float32)), ref)["ok"]
    nanb = bits.copy()
    nanb[0, 0] = 0x7FC0
    assert not o.gate(nanb, ref)["ok"]
    neg = (bits ^ np.uint16(0x8000)).astype(np.uint16)
    r = o.gate(neg, ref)
    assert not r["ok"] and r["cos"] < 0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
