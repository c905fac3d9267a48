"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle library handle ``L`` and raises
``AssertionError`` when the oracle disagrees with an independent fact:

* fp16 conversion against numpy's IEEE conversions (a library routine) and
  against values worked out by hand;
* the rotate-half examples printed in sglang rope_cache.py
  (``tests/golden/rotate_half_page2.txt``);
* the rotation against three independent formulations: the page's own
  sign-mask-and-flip description (_get_neox_rotated_x / _get_gptj_rotated_x /
  _unit_rope), complex multiplication ``(x_u + i x_v) * e^{i theta}``, and an
  explicit D x D block-rotation matrix;
* invariants: angle 0 is the identity, each pair keeps its norm, q.k after
  rotation depends only on the position difference, rotating back undoes the
  rotation, GPT-J is NeoX under the pair permutation;
* layout and indexing by brute-force decoding: V payloads that encode
  (b, s, h) are located by scanning the whole cache;
* bit-exact copies of all 65,536 fp16 patterns, untouched-slot sentinels,
  cross-call reductions, skip rules case by case, the capacity truth table
  (``tests/golden/capacity_check.txt``);
* the fp8 (E4M3) cache variants: the codec against torch's float8_e4m3fn
  conversions, against brute-force nearest-even search over the 256 codes and
  against hand-worked values of the OCP format
  (``tests/golden/e4m3_values.txt``); cache bytes against the exact rational
  rotation (an explicit matrix in ``fractions.Fraction``) times the fp32
  reciprocal scale, encoded by brute force; layout and skip rules against the
  fp16 variant's.

``tests/test_oracle_pins.py`` runs every pin against the oracle;
``tests/test_oracle_mutations.py`` plants mistakes into a copy of the oracle
source and checks that some pin fails for each.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEOX, GPTJ = W.NEOX, W.GPTJ


def f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def val(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _row(R, angles):
    half = R // 2
    row = np.empty(R, dtype=np.float32)
    row[:half] = np.cos(angles)
    row[half:] = np.sin(angles)
    return row


def _rand_angles(r, half):
    return r.uniform(-40.0, 40.0, size=half)


# ------------------------------------------------------------------ fp16 --

def pin_half_to_double_all_patterns(L):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b), L) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_double_to_half_round_trip(L):
    for b in range(1 << 16):
        e = (b >> 10) & 0x1F
        if e == 31 and (b & 0x3FF):
            got = oracle.double_to_half(oracle.half_to_double(b, L), L)
            assert (got & 0x7C00) == 0x7C00 and (got & 0x3FF), hex(b)
            continue
        got = oracle.double_to_half(val(b).item(), L)
        assert got == b, (hex(b), hex(got))


def pin_double_to_half_vs_numpy(L):
    r = np.random.default_rng(7)
    xs = [r.standard_normal(20000) * 10.0 ** r.uniform(-9, 5, 20000)]
    # exact midpoints between neighbouring fp16 values and points just off them
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16)
    lo, hi = val(h), val(h + 1)
    mid = (lo + hi) / 2.0
    xs += [mid, -mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    xs.append(np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e300, 2.0 ** -24, 2.0 ** -25,
                        2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                        2.0 ** -14 - 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0, -0.0,
                        1e-300, -1e-300]))
    x = np.concatenate(xs)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half(float(v), L) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_double_to_half_hand_values(L):
    # values worked out from the binary16 definition
    cases = {1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF, 65520.0: 0x7C00, 2.0 ** -24: 0x0001,
             2.0 ** -14: 0x0400, 1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02,
             2.0 ** -25: 0x0000, 3 * 2.0 ** -25: 0x0002, 0.333251953125: 0x3555}
    for x, b in cases.items():
        assert oracle.double_to_half(x, L) == b, (x, hex(oracle.double_to_half(x, L)), hex(b))


# ---------------------------------------------------------------- rotate --

def pin_golden_rotate_half(L):
    path = os.path.join(GOLDEN, "rotate_half_page2.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].split()
        if not line:
            continue
        style = NEOX if line[0] == "neox" else GPTJ
        c, s = float(line[1]), float(line[2])
        x = [float(v) for v in line[3:7]]
        want = [float(v) for v in line[7:11]]
        row = np.array([c, c, s, s], dtype=np.float32)
        y = oracle.rotate_row(f16(x), row, 4, style, L)
        assert np.array_equal(val(y), np.array(want)), (line, val(y))
        n += 1
    assert n >= 8


def _page2_rotate(x_bits, row, R, style):
    """The page's formulation: y = x*cos + rotate(x)*sin, with rotate built
    by a sign mask and flips, cos/sin expanded per element from the
    half-width table; evaluated in float64 and rounded by numpy."""
    x = val(x_bits)
    D = x.size
    xr = x[:R]
    d = np.arange(R)
    if style == NEOX:
        mask = d < R // 2
        t = np.where(mask, xr, -xr).reshape(2, R // 2)[:, ::-1].reshape(R)[::-1]
        dc = np.where(d >= R // 2, d - R // 2, d)
    else:
        mask = d % 2 == 0
        t = np.where(mask, xr, -xr).reshape(R // 2, 2)[:, ::-1].reshape(R)
        dc = d // 2
    cos = row[dc].astype(np.float64)
    sin = row[dc + R // 2].astype(np.float64)
    y = np.concatenate([xr * cos + t * sin, x[R:]]) if R < D else xr * cos + t * sin
    out = f16(y)
    out[R:] = x_bits[R:]
    return out


def pin_page2_formulation(L):
    r = np.random.default_rng(11)
    for D, R in [(64, 64), (128, 128), (128, 64), (256, 96), (16, 8), (4, 4)]:
        for style in (NEOX, GPTJ):
            for _ in range(20):
                x = W.normal_f16(r, (D,))
                row = _row(R, _rand_angles(r, R // 2))
                got = oracle.rotate_row(x, row, R, style, L)
                want = _page2_rotate(x, row, R, style)
                assert np.array_equal(got, want), (D, R, style)


def pin_complex_multiplication(L):
    r = np.random.default_rng(12)
    for D, R in [(128, 128), (64, 32)]:
        for style in (NEOX, GPTJ):
            x = W.normal_f16(r, (D,))
            row = _row(R, _rand_angles(r, R // 2))
            half = R // 2
            xv = val(x)
            if style == NEOX:
                re, im = xv[:half], xv[half:R]
            else:
                re, im = xv[0:R:2], xv[1:R:2]
            w = (re + 1j * im) * (row[:half].astype(np.float64) + 1j * row[half:].astype(np.float64))
            got = val(oracle.rotate_row(x, row, R, style, L))
            if style == NEOX:
                g_re, g_im = got[:half], got[half:R]
            else:
                g_re, g_im = got[0:R:2], got[1:R:2]
            assert np.array_equal(f16(w.real), f16(g_re))
            assert np.array_equal(f16(w.imag), f16(g_im))
            assert np.array_equal(oracle.rotate_row(x, row, R, style, L)[R:], x[R:])


def _rotation_matrix(row, D, R, style):
    half = R // 2
    M = np.eye(D)
    for i in range(half):
        u, v = (i, i + half) if style == NEOX else (2 * i, 2 * i + 1)
        c, s = float(row[i]), float(row[half + i])
        M[u, u], M[u, v], M[v, u], M[v, v] = c, -s, s, c
    return M


def pin_brute_force_matrix(L):
    """Two tokens at two positions, rotated by an explicit D x D matrix."""
    r = np.random.default_rng(13)
    D = 64
    for R in (64, 48):
        for style in (NEOX, GPTJ):
            table = W.rope_table(1, 64, R, 10000.0)[0]
            for pos in (5, 63):
                x = W.normal_f16(r, (D,))
                M = _rotation_matrix(table[pos], D, R, style)
                want = f16(M @ val(x))
                got = oracle.rotate_row(x, table[pos], R, style, L)
                assert np.array_equal(got, want), (R, style, pos)


def pin_identity_at_position_zero(L):
    r = np.random.default_rng(14)
    table = W.rope_table(1, 4, 128, 10000.0)[0]
    for style in (NEOX, GPTJ):
        x = W.normal_f16(r, (128,))
        y = oracle.rotate_row(x, table[0], 128, style, L)
        assert np.array_equal(val(y), val(x))   # value equality: -0 may become +0


def pin_pair_norm(L):
    r = np.random.default_rng(15)
    R = 128
    table = W.rope_table(1, 4096, R, 10000.0)[0]
    for style in (NEOX, GPTJ):
        for pos in (1, 17, 1000, 4095):
            x = W.normal_f16(r, (R,))
            y = oracle.rotate_row(x, table[pos], R, style, L)
            xv, yv = val(x), val(y)
            if style == NEOX:
                nx = xv[:64] ** 2 + xv[64:] ** 2
                ny = yv[:64] ** 2 + yv[64:] ** 2
            else:
                nx = xv[0::2] ** 2 + xv[1::2] ** 2
                ny = yv[0::2] ** 2 + yv[1::2] ** 2
            assert np.all(np.abs(ny - nx) <= 2.0 ** -9 * nx + 2.0 ** -22), (style, pos)


def pin_relative_position(L):
    r = np.random.default_rng(16)
    R = 128
    table = W.rope_table(1, 8192, R, 10000.0)[0]
    for style in (NEOX, GPTJ):
        for m, n, delta in [(5, 3, 100), (700, 20, 3000), (4000, 4000, 17), (1, 900, 6000)]:
            q = W.normal_f16(r, (R,))
            k = W.normal_f16(r, (R,))
            a = val(oracle.rotate_row(q, table[m], R, style, L)) @ \
                val(oracle.rotate_row(k, table[n], R, style, L))
            b = val(oracle.rotate_row(q, table[m + delta], R, style, L)) @ \
                val(oracle.rotate_row(k, table[n + delta], R, style, L))
            bound = 4 * 2.0 ** -11 * np.linalg.norm(val(q)) * np.linalg.norm(val(k))
            assert abs(a - b) <= bound, (style, m, n, delta, a, b)


def pin_inverse_rotation(L):
    r = np.random.default_rng(17)
    R = 64
    for style in (NEOX, GPTJ):
        row = _row(R, _rand_angles(r, R // 2))
        back = row.copy()
        back[R // 2:] = -back[R // 2:]
        x = W.normal_f16(r, (R,))
        z = oracle.rotate_row(oracle.rotate_row(x, row, R, style, L), back, R, style, L)
        xv, zv = val(x), val(z)
        # each rounding errs by at most half an fp16 ulp of a pair member,
        # whose size is bounded by the pair's norm
        partner = (np.arange(R) + R // 2) % R if style == NEOX else np.arange(R) ^ 1
        pair = np.hypot(xv, xv[partner])
        assert np.all(np.abs(zv - xv) <= 2.0 ** -9 * pair + 2.0 ** -23), style


def pin_gptj_is_permuted_neox(L):
    r = np.random.default_rng(18)
    for D, R in [(128, 128), (128, 64)]:
        row = _row(R, _rand_angles(r, R // 2))
        x = W.normal_f16(r, (D,))
        half = R // 2
        perm = np.arange(D)
        perm[:half] = np.arange(0, R, 2)          # NeoX slot i <- GPT-J slot 2i
        perm[half:R] = np.arange(1, R, 2)         # NeoX slot i+R/2 <- GPT-J slot 2i+1
        y_neox = oracle.rotate_row(x[perm], row, R, NEOX, L)
        y = np.empty_like(y_neox)
        y[perm] = y_neox
        assert np.array_equal(y, oracle.rotate_row(x, row, R, GPTJ, L)), (D, R)


def pin_passthrough_bits(L):
    """Dims >= R keep every one of the 65,536 bit patterns."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    D, R = 128, 64
    rows = allbits.reshape(-1, D - R)
    r = np.random.default_rng(19)
    row = _row(R, _rand_angles(r, R // 2))
    for style in (NEOX, GPTJ):
        for k in range(0, rows.shape[0], 37):
            x = np.concatenate([W.normal_f16(r, (R,)), rows[k]])
            y = oracle.rotate_row(x, row, R, style, L)
            assert np.array_equal(y[R:], rows[k])


# ----------------------------------------------------------------- calls --

def _code_rows(n, D):
    """n distinct finite positive fp16 payload rows (all D elements equal)."""
    codes = (0x0400 + np.arange(n)).astype(np.uint16)
    assert codes.max() < 0x7C00
    return np.repeat(codes[:, None], D, axis=1), codes


def pin_v_copy_all_patterns(L):
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    B, S, Hq, Hkv, D = 1, 64, 1, 16, 64     # 64 tokens x 16 V heads x 64 dims
    qkv = np.zeros((B, S, Hq + 2 * Hkv, D), dtype=np.uint16)
    qkv[0, :, Hq + Hkv:, :] = allbits.reshape(S, Hkv, D)
    table = W.rope_table(1, S, D, 10000.0)
    cache = W.sentinel_f16((B, 2, Hkv, S, D))
    q2, c2 = oracle.packed_qkv(table, qkv, cache, NEOX, L)
    assert np.array_equal(c2[0, 1].transpose(1, 0, 2), allbits.reshape(S, Hkv, D))
    assert np.array_equal(q2[0, :, Hq + Hkv:], qkv[0, :, Hq + Hkv:])   # V unchanged in place


def pin_layout_packed(L):
    """Call 1 with R = 0 (no rotation): decode where every K and V row landed."""
    B, S, Hq, Hkv, D, cap = 2, 5, 3, 2, 16, 8
    H = Hq + 2 * Hkv
    rows, codes = _code_rows(B * S * H, D)
    qkv = rows.reshape(B, S, H, D).copy()
    table = np.zeros((1, cap, 0), dtype=np.float32)
    cache = W.sentinel_f16((B, 2, Hkv, cap, D))
    q2, c2 = oracle.packed_qkv(table, qkv, cache, NEOX, L)
    assert np.array_equal(q2, qkv)
    seen = set()
    for b in range(B):
        for plane in range(2):
            for h in range(Hkv):
                for slot in range(cap):
                    v = c2[b, plane, h, slot]
                    if slot >= S:
                        assert np.all(v == W.SENTINEL), (b, plane, h, slot)
                        continue
                    assert np.all(v == v[0])
                    idx = int(v[0]) - 0x0400
                    bb, rest = divmod(idx, S * H)
                    ss, hh = divmod(rest, H)
                    assert (bb, ss) == (b, slot), (b, plane, h, slot, bb, ss)
                    assert hh == Hq + plane * Hkv + h, (hh, plane, h)
                    seen.add(idx)
    assert len(seen) == B * S * 2 * Hkv


def pin_layout_continuous_and_tree(L):
    B, S, Hq, Hkv, D, cap = 3, 4, 2, 2, 16, 12
    H = Hq + 2 * Hkv
    rows, _ = _code_rows(B * S * H, D)
    qkv = rows.reshape(B, S, H, D).copy()
    end = np.array([4, 12, 7], dtype=np.int32)
    table = np.zeros((1, cap, 0), dtype=np.float32)
    for call in ("continuous", "tree"):
        cache = W.sentinel_f16((B, 2, Hkv, cap, D))
        q_out = W.sentinel_f16((B, S, Hq, D))
        if call == "continuous":
            c2, qo = oracle.continuous(table, end, qkv, cache, q_out, NEOX, L)
        else:
            pos = np.tile(np.array([0, 1, 1, 2], dtype=np.int32), (B, 1))
            c2, qo = oracle.tree(table, end, pos, qkv, cache, q_out, GPTJ, L)
        assert np.array_equal(qo, qkv[:, :, :Hq])
        for b in range(B):
            for plane in range(2):
                for h in range(Hkv):
                    for slot in range(cap):
                        v = c2[b, plane, h, slot]
                        if not (end[b] - S <= slot < end[b]):
                            assert np.all(v == W.SENTINEL), (call, b, plane, h, slot)
                            continue
                        idx = int(v[0]) - 0x0400
                        bb, rest = divmod(idx, S * H)
                        ss, hh = divmod(rest, H)
                        assert (bb, ss + end[b] - S) == (b, slot), (call, b, slot, bb, ss)
                        assert hh == Hq + plane * Hkv + h


def pin_layout_paged(L):
    N, batch, Hkv, D, P, M = 6, 3, 2, 16, 5, 3
    rows, _ = _code_rows(N * Hkv, D)
    v_delta = rows.reshape(N, Hkv, D).copy()
    k_delta = rows.reshape(N, Hkv, D).copy() + np.uint16(0x1000)
    pos = np.array([0, 63, 64, 130, 5, 191], dtype=np.int32)
    seq = np.array([0, 0, 1, 1, 2, 2], dtype=np.int32)
    pt = np.empty((batch, 2, M), dtype=np.int32)
    pt[:, 0, :] = np.array([[4, 0, 1], [2, 3, 0], [1, 2, 3]])
    pt[:, 1, :] = P + np.array([[1, 2, 3], [0, 4, 2], [3, 1, 0]])
    pool = W.sentinel_f16((2, P, 64, Hkv, D))
    cs = np.zeros((N, 0), dtype=np.float32)
    out = oracle.paged_delta(k_delta, v_delta, pool, cs, pos, seq, pt, batch, NEOX, L)
    flat = out.reshape(2 * P, 64, Hkv, D)
    written = 0
    for pid in range(2 * P):
        for off in range(64):
            for h in range(Hkv):
                v = flat[pid, off, h]
                if np.all(v == W.SENTINEL):
                    continue
                written += 1
                code = int(v[0])
                is_k = code >= 0x1400
                i, hh = divmod(code - (0x1400 if is_k else 0x0400), Hkv)
                plane = 0 if is_k else 1
                assert hh == h
                assert pid == pt[seq[i], plane, pos[i] // 64], (i, plane, pid)
                assert off == pos[i] % 64
    assert written == 2 * N * Hkv


def pin_untouched_and_in_place_k(L):
    w = W.packed(2, 7, 3, 2, 64, 64, 16, GPTJ, 99, table_batch=2, table_len=9,
                 offsets=np.array([0, 3]))
    q2, c2 = oracle.packed_qkv(w.cos_sin, w.qkv, w.cache, w.style, L)
    assert np.all(c2[:, :, :, w.S:] == W.SENTINEL)
    # K in place == K in the cache, bitwise
    k_inplace = q2[:, :, w.Hq:w.Hq + w.Hkv].transpose(0, 2, 1, 3)
    assert np.array_equal(k_inplace, c2[:, 0, :, :w.S])
    # Q and K changed, V not
    assert not np.array_equal(q2[:, :, :w.Hq + w.Hkv], w.qkv[:, :, :w.Hq + w.Hkv])
    assert np.array_equal(q2[:, :, w.Hq + w.Hkv:], w.qkv[:, :, w.Hq + w.Hkv:])
    # each head row equals the row rotation at (table batch b, position s)
    for b in range(w.B):
        for s in range(w.S):
            for h in range(w.Hq + w.Hkv):
                want = oracle.rotate_row(w.qkv[b, s, h], w.cos_sin[b, s], w.R, w.style, L)
                assert np.array_equal(q2[b, s, h], want), (b, s, h)


def pin_cross_call_reductions(L):
    r = np.random.default_rng(20)
    B, S, Hq, Hkv, D, cap = 2, 6, 4, 2, 64, 10
    for style in (NEOX, GPTJ):
        qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
        table = W.rope_table(1, cap, D, 10000.0)
        cache = W.sentinel_f16((B, 2, Hkv, cap, D))
        q1, c1 = oracle.packed_qkv(table, qkv, cache, style, L)
        end = np.full(B, S, dtype=np.int32)
        c2, qo2 = oracle.continuous(table, end, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                                    style, L)
        assert np.array_equal(c1, c2)
        assert np.array_equal(q1[:, :, :Hq], qo2)
        # a linear chain of tree positions is the continuous write
        end = np.array([7, 10], dtype=np.int32)
        c2, qo2 = oracle.continuous(table, end, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                                    style, L)
        pos = (end[:, None] - S + np.arange(S)[None, :]).astype(np.int32)
        c3, qo3 = oracle.tree(table, end, pos, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                              style, L)
        assert np.array_equal(c2, c3) and np.array_equal(qo2, qo3)
        # the paged update through an identity page table is the continuous K/V write
        TPP = 64
        M = 1
        P = B
        pt = np.empty((B, 2, M), dtype=np.int32)
        pt[:, 0, 0] = np.arange(B)
        pt[:, 1, 0] = P + np.arange(B)
        N = B * S
        k_delta = qkv[:, :, Hq:Hq + Hkv].reshape(N, Hkv, D)
        v_delta = qkv[:, :, Hq + Hkv:].reshape(N, Hkv, D)
        posd = pos.reshape(-1).astype(np.int32)
        seqd = np.repeat(np.arange(B), S).astype(np.int32)
        rows = table[0][posd]
        pool = W.sentinel_f16((2, P, TPP, Hkv, D))
        pool = oracle.paged_delta(k_delta, v_delta, pool, rows, posd, seqd, pt, B, style, L)
        for b in range(B):
            for plane in range(2):
                got = pool[plane, b, :cap].transpose(1, 0, 2)     # [Hkv, cap, D]
                assert np.array_equal(got, c2[b, plane]), (style, b, plane)


def pin_skip_rules_contiguous(L):
    """Calls 2 and 3: a token whose slot or position is out of range writes
    nothing; its neighbours still write."""
    r = np.random.default_rng(21)
    B, S, Hq, Hkv, D, cap, tlen = 4, 3, 2, 1, 16, 6, 5
    qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    table = W.rope_table(1, tlen, D, 10000.0)
    end = np.array([2, 7, 6, 3], dtype=np.int32)   # slots: [-1,0,1] [4,5,6] [3,4,5] [0,1,2]
    cache = W.sentinel_f16((B, 2, Hkv, cap, D))
    qo0 = W.sentinel_f16((B, S, Hq, D))
    c2, qo = oracle.continuous(table, end, qkv, cache, qo0, NEOX, L)
    wrote = ~np.all(qo == W.SENTINEL, axis=(2, 3))
    # call 2 requires slot in [0, cap) and position (= slot) in [0, tlen)
    want = np.array([[0, 1, 1], [1, 0, 0], [1, 1, 0], [1, 1, 1]], dtype=bool)
    assert np.array_equal(wrote, want), wrote
    for b in range(B):
        for s in range(S):
            slot = end[b] - S + s
            if 0 <= slot < cap:
                assert np.all(c2[b, :, :, slot] == W.SENTINEL) != want[b, s]
    pos = np.array([[0, 4, 5], [-1, 0, 1], [2, 2, 9], [4, 4, 4]], dtype=np.int32)
    c3, qo = oracle.tree(table, end, pos, qkv, cache, qo0, NEOX, L)
    wrote = ~np.all(qo == W.SENTINEL, axis=(2, 3))
    # call 3 requires slot in [0, cap) and position in [0, tlen)
    want = np.array([[0, 1, 0], [0, 1, 0], [1, 1, 0], [1, 1, 1]], dtype=bool)
    assert np.array_equal(wrote, want), wrote


def pin_skip_rules_paged(L):
    """Call 4, one row at a time through every skip reason."""
    batch, Hkv, D, P, M, R = 2, 1, 16, 4, 2, 16
    r = np.random.default_rng(22)
    k = W.normal_f16(r, (1, Hkv, D))
    v = W.normal_f16(r, (1, Hkv, D))
    cs = W.rope_rows([70], R, 10000.0)
    pool0 = W.sentinel_f16((2, P, 64, Hkv, D))

    def run(pos, seq, kid, vid):
        # the table has a row for one sequence beyond the active batch (the
        # page's pageTable is [B, ...] while batchSize is the active count),
        # holding valid ids, so that a row of an inactive sequence that were
        # kept would write somewhere
        pt = np.zeros((batch + 1, 2, M), dtype=np.int32)
        pt[:, 0, :] = 1
        pt[:, 1, :] = P + 1
        if 0 <= seq <= batch and 0 <= pos < M * 64:
            pt[seq, 0, pos // 64] = kid
            pt[seq, 1, pos // 64] = vid
        out = oracle.paged_delta(k, v, pool0, cs, np.array([pos], np.int32),
                                 np.array([seq], np.int32), pt, batch, NEOX, L)
        flat = out.reshape(2 * P, 64, Hkv, D)
        changed = np.argwhere(~np.all(flat == pool0.reshape(2 * P, 64, Hkv, D), axis=(2, 3)))
        return {(int(a), int(b)) for a, b in changed}

    ok_k, ok_v = 2, P + 3
    assert run(70, 1, ok_k, ok_v) == {(ok_k, 6), (ok_v, 6)}
    assert run(-1, 1, ok_k, ok_v) == set()             # padding position
    assert run(70, -1, ok_k, ok_v) == set()            # padding sequence
    assert run(-5, -5, ok_k, ok_v) == set()
    assert run(70, 2, ok_k, ok_v) == set()             # sequence beyond the active batch
    assert run(128, 1, ok_k, ok_v) == set()            # position beyond maxPagesPerSeq pages
    assert run(127, 1, ok_k, ok_v) == {(ok_k, 63), (ok_v, 63)}   # last writable position
    assert run(70, 1, -1, ok_v) == {(ok_v, 6)}         # unmapped K page
    assert run(70, 1, P, ok_v) == {(ok_v, 6)}          # K entry in the V plane
    assert run(70, 1, 2 * P, ok_v) == {(ok_v, 6)}      # beyond both planes
    assert run(70, 1, ok_k, -1) == {(ok_k, 6)}         # unmapped V page
    assert run(70, 1, ok_k, P - 1) == {(ok_k, 6)}      # V entry in the K plane
    assert run(70, 1, ok_k, 2 * P) == {(ok_k, 6)}      # beyond both planes
    assert run(70, 1, 0, P) == {(0, 6), (P, 6)}        # lowest valid id of each plane
    assert run(70, 1, P - 1, 2 * P - 1) == {(P - 1, 6), (2 * P - 1, 6)}   # highest
    assert run(70, 1, -1, -1) == set()
    # position == maxPagesPerSeq * 64 for sequence 0: the int32 entries that
    # follow its last logical page in memory hold ids that are valid for the
    # plane being read, so any read past the page row would show as a write
    pt = np.zeros((batch, 2, M), dtype=np.int32)
    pt[:, 0, :] = 1
    pt[:, 1, :] = P + 1
    pt[0, 1, 0] = 2          # read by K at logical page M of sequence 0
    pt[1, 0, 0] = P + 2      # read by V at logical page M of sequence 0
    out = oracle.paged_delta(k, v, pool0, cs, np.array([M * 64], np.int32),
                             np.array([0], np.int32), pt, batch, NEOX, L)
    assert np.array_equal(out, pool0)


def pin_paged_values(L):
    """A written K page row is the rotated delta row with its own table row;
    a written V page row is the delta row, bit for bit."""
    w = W.paged(64, 4, 2, 64, 32, 16, 4, GPTJ, 23, width=16, pool_fill="sentinel")
    out = oracle.paged_delta(w.k_delta, w.v_delta, w.pool, w.cos_sin, w.positions, w.seq,
                             w.page_table, w.batch, w.style, L)
    flat = out.reshape(2 * w.num_pages, 64, w.Hkv, w.D)
    n_k = n_v = 0
    for i in range(w.N):
        p, q = int(w.positions[i]), int(w.seq[i])
        if p < 0 or q < 0:
            continue
        kid = int(w.page_table[q, 0, p // 64])
        vid = int(w.page_table[q, 1, p // 64])
        if 0 <= kid < w.num_pages:
            n_k += 1
            for h in range(w.Hkv):
                want = oracle.rotate_row(w.k_delta[i, h], w.cos_sin[i], w.R, w.style, L)
                assert np.array_equal(flat[kid, p % 64, h], want)
        if w.num_pages <= vid < 2 * w.num_pages:
            n_v += 1
            assert np.array_equal(flat[vid, p % 64], w.v_delta[i])
    assert n_k > 10 and n_v > 10


def pin_capacity_truth_table(L):
    n = 0
    for line in open(os.path.join(GOLDEN, "capacity_check.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        a, b, want = int(line[0]), int(line[1]), line[2]
        rc = oracle.check_rope_capacity(a, b, L)
        assert (rc == 0) == (want == "ok"), (a, b, rc)
        n += 1
    assert n >= 10


def pin_argument_errors(L):
    t = W.rope_table(1, 8, 16, 10000.0)
    qkv = np.zeros((1, 4, 4, 16), np.uint16)
    cache = np.zeros((1, 2, 1, 8, 16), np.uint16)
    # S > capacity or S > table length: capacity error
    try:
        oracle.packed_qkv(t, qkv, np.zeros((1, 2, 1, 3, 16), np.uint16), NEOX, L)
        raise AssertionError("S > cap accepted")
    except oracle.OracleError as e:
        assert e.code == oracle.ERR_CAPACITY
    try:
        oracle.packed_qkv(W.rope_table(1, 3, 16, 1e4), qkv, cache, NEOX, L)
        raise AssertionError("S > table length accepted")
    except oracle.OracleError as e:
        assert e.code == oracle.ERR_CAPACITY
    for bad in [dict(t=W.rope_table(2, 8, 16, 1e4)), dict(style=2), dict(t=np.zeros((1, 8, 15), np.float32)),
                dict(t=np.zeros((1, 8, 18), np.float32))]:
        try:
            oracle.packed_qkv(bad.get("t", t), qkv, cache, bad.get("style", NEOX), L)
            raise AssertionError(f"accepted {bad}")
        except oracle.OracleError as e:
            assert e.code == oracle.ERR_ARG


def pin_gather_delta_rope(L):
    """The gather picks table[state(seq)][pos] row by row; rows without one
    (padding, inactive sequence, missing state, position past the table)
    come back as NaN."""
    r = np.random.default_rng(24)
    states, rows, R, batch = 3, 40, 16, 4
    rope = r.standard_normal((states, rows, R)).astype(np.float32)
    pos = np.array([0, 39, 40, -1, 5, 7, 7, 12, 3], dtype=np.int32)
    seq = np.array([0, 1, 2, 0, -1, 4, 3, 3, 2], dtype=np.int32)
    si = np.array([2, 0, 1, 7], dtype=np.int32)          # sequence 3 maps to a missing state
    got = oracle.gather_delta_rope(rope, si, pos, seq, batch, L)
    for i in range(pos.size):
        p, q = int(pos[i]), int(seq[i])
        ok = p >= 0 and 0 <= q < batch and 0 <= si[q] < states and p < rows
        if ok:
            assert np.array_equal(got[i], rope[si[q], p]), i
        else:
            assert np.all(np.isnan(got[i])), i
    # without state indices: sequence q uses state q (or 0 for a one-state table)
    got = oracle.gather_delta_rope(rope, None, np.array([4, 4, 4], np.int32),
                                   np.array([0, 1, 2], np.int32), 3, L)
    assert np.array_equal(got, rope[[0, 1, 2], 4])
    got = oracle.gather_delta_rope(rope[:1], None, np.array([4, 9], np.int32),
                                   np.array([1, 2], np.int32), 3, L)
    assert np.array_equal(got, rope[[0, 0], [4, 9]])


def pin_fused_gather_is_gather_then_update(L):
    """With every live row covered by the table, the fused call equals the
    gather followed by the paged update, bit for bit; a row without a rope
    row leaves its K slot untouched but still writes V."""
    for style in (NEOX, GPTJ):
        w = W.paged(128, 4, 2, 64, 64, 16, 4, style, 25 + style, width=32, pool_fill="sentinel")
        rope = W.rope_table(4, 256, w.R, 10000.0, offsets=np.array([0, 3, 9, 27]))
        si = np.array([3, 1, 0, 2], dtype=np.int32)
        rows = oracle.gather_delta_rope(rope, si, w.positions, w.seq, w.batch, L)
        want = oracle.paged_delta(w.k_delta, w.v_delta, w.pool, rows, w.positions, w.seq,
                                  w.page_table, w.batch, style, L)
        got = oracle.paged_delta_gather(w.k_delta, w.v_delta, w.pool, rope, si, w.positions,
                                        w.seq, w.page_table, w.batch, style, L)
        assert np.array_equal(got, want), style
    # a table too short for one live row
    w = W.paged(8, 1, 1, 64, 64, 4, 2, NEOX, 27, width=8, pad_frac=0.0, bad_frac=0.0,
                pool_fill="sentinel")
    p_max = int(w.positions.max())
    rope = W.rope_table(1, p_max, 64, 10000.0)            # rows 0 .. p_max-1
    got = oracle.paged_delta_gather(w.k_delta, w.v_delta, w.pool, rope, None, w.positions, w.seq,
                                    w.page_table, 1, NEOX, L)
    i = int(np.argmax(w.positions))
    kid = int(w.page_table[0, 0, p_max // 64])
    vid = int(w.page_table[0, 1, p_max // 64])
    flat = got.reshape(2 * w.num_pages, 64, w.Hkv, w.D)
    assert np.all(flat[kid, p_max % 64] == W.SENTINEL)
    assert np.array_equal(flat[vid, p_max % 64], w.v_delta[i])


# ------------------------------------------------------------------- fp8 --

def _e4m3_values():
    """The 256 E4M3 codes decoded by torch (a library routine)."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_positive():
    """(magnitudes, codes) of the finite non-negative codes 0x00..0x7e, ascending."""
    v = _e4m3_values()[:0x7F]
    assert np.all(np.diff(v) > 0)
    return v, np.arange(0x7F)


def _nearest_e4m3(x) -> np.ndarray:
    """Brute force: the code nearest to each double, ties to the even code,
    magnitudes past 448 saturated, NaN kept (sign bit copied)."""
    x = np.asarray(x, dtype=np.float64)
    mags, codes = _e4m3_positive()
    a = np.abs(x)
    d = np.abs(a[..., None] - mags)                     # [..., 127]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    out = codes[pick].astype(np.uint8)
    out = np.where(a >= 448.0, np.uint8(0x7E), out)
    out = np.where(np.isnan(x), np.uint8(0x7F), out)
    return np.where(np.signbit(x), out | np.uint8(0x80), out).astype(np.uint8)


def _nearest_e4m3_exact(fr: Fraction) -> int:
    """Brute force on an exact rational: nearest code, ties to even, saturating."""
    mags, codes = _e4m3_positive()
    a = abs(fr)
    sign = 0x80 if fr < 0 else 0
    if a >= 448:
        return sign | 0x7E
    i = int(np.searchsorted(mags, float(a)))
    best, best_d = None, None
    for j in (i - 2, i - 1, i, i + 1):
        if 0 <= j < mags.size:
            dj = abs(a - Fraction(float(mags[j])))
            if best is None or dj < best_d or (dj == best_d and codes[j] % 2 == 0):
                best, best_d = j, dj
    return sign | int(codes[best])


def _rcp(scale) -> float:
    """fp32 reciprocal of an fp32 scale (numpy's IEEE division)."""
    if scale is None:
        return 1.0
    return float(np.float32(1.0) / np.float32(scale))


def pin_e4m3_decode_all_codes(L):
    want = _e4m3_values()
    got = np.array([oracle.e4m3_to_double(b, L) for b in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_e4m3_encode_vs_torch(L):
    """fp32 inputs below the saturation point round exactly as torch rounds
    float32 -> float8_e4m3fn (nearest even); every midpoint between adjacent
    codes and its two fp32 neighbours is included."""
    import torch
    mags, _ = _e4m3_positive()
    mids = (mags[:-1] + mags[1:]) / 2
    base = np.concatenate([mags, mids]).astype(np.float32)
    xs = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                         np.nextafter(base, np.float32(0))])
    r = np.random.default_rng(40)
    xs = np.concatenate([xs, r.uniform(0, 447.9, 3000).astype(np.float32),
                         np.exp2(r.uniform(-14, 8.8, 3000)).astype(np.float32)])
    xs = xs[xs < 448]
    xs = np.concatenate([xs, -xs])
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.double_to_e4m3(float(x), L) for x in xs], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_e4m3_encode_brute_force(L):
    """Doubles over the whole range, saturation, infinities, NaN and signed
    zero, against a nearest-even search over all codes."""
    r = np.random.default_rng(41)
    xs = np.concatenate([np.exp2(r.uniform(-16, 12, 4000)), r.uniform(0, 500, 2000),
                         [0.0, 447.9999, 448.0, 464.0, 480.0, 1e300, np.inf, np.nan,
                          2.0 ** -10, 2.0 ** -10 * 1.0000001, 3 * 2.0 ** -10]])
    xs = np.concatenate([xs, -xs])
    got = np.array([oracle.double_to_e4m3(float(x), L) for x in xs], dtype=np.uint8)
    want = _nearest_e4m3(xs)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def pin_e4m3_hand_values(L):
    """Values worked out from the OCP E4M3 definition (the golden file)."""
    path = os.path.join(GOLDEN, "e4m3_values.txt")
    n = 0
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        x, code = line.split()
        x = float.fromhex(x) if "0x" in x.lower() and "p" in x.lower() else float(x)
        assert oracle.double_to_e4m3(x, L) == int(code, 16), (x, code)
        n += 1
    assert n >= 20


def pin_fp8_v_all_patterns(L):
    """The V rows of every fp16 bit pattern reach the fp8 pool as the nearest
    E4M3 code of v * (1/v_scale), for a missing scale (1) and for 2 and 0.0109."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    N, Hkv, D = 64, 16, 64
    v_delta = allbits.reshape(N, Hkv, D)
    k_delta = np.zeros_like(v_delta)
    pos = np.arange(N, dtype=np.int32)
    seq = np.zeros(N, dtype=np.int32)
    pt = np.array([[[0], [1]]], dtype=np.int32)
    cs = np.zeros((N, 0), dtype=np.float32)
    for vs in (None, 2.0, 0.0109):
        pool = np.full((2, 1, 64, Hkv, D), W.SENTINEL8, dtype=np.uint8)
        out = oracle.paged_delta_fp8(k_delta, v_delta, pool, cs, pos, seq, pt, 1, None, vs,
                                     NEOX, L)
        with np.errstate(invalid="ignore"):
            want = _nearest_e4m3(val(allbits) * _rcp(vs)).reshape(N, Hkv, D)
        assert np.array_equal(out[1, 0], want), vs
        assert np.all(out[0, 0] == 0)       # K of zeros is +0


def pin_fp8_k_exact_rational(L):
    """K cache bytes are the exact rotation (an explicit rotation matrix in
    rational arithmetic) times the fp32 reciprocal scale, rounded once to the
    nearest E4M3 code; the fp16 result never enters."""
    r = np.random.default_rng(42)
    B, S, Hq, Hkv, D, cap = 2, 16, 1, 4, 128, 16
    for style, R, ks, n_tok in [(NEOX, 128, 0.0123, 32), (GPTJ, 96, None, 4),
                                (NEOX, 64, 0.25, 4)]:
        qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
        table = W.rope_table(2, cap, R, 10000.0, offsets=np.array([3, 1000]))
        cache = np.full((B, 2, Hkv, cap, D), W.SENTINEL8, dtype=np.uint8)
        _, c8 = oracle.packed_qkv_fp8(table, qkv, cache, ks, 1.0, style, L)
        rcp = Fraction(_rcp(ks))
        for t in range(n_tok):
            b, s = divmod(t, S)
            M = _rotation_matrix(table[b, s], D, R, style)
            terms = [[(j, Fraction(float(M[i, j]))) for j in np.nonzero(M[i])[0]]
                     for i in range(D)]
            for h in range(Hkv):
                x = [Fraction(float(v)) for v in val(qkv[b, s, Hq + h])]
                want = [_nearest_e4m3_exact(sum(m * x[j] for j, m in terms[i]) * rcp)
                        for i in range(D)]
                assert c8[b, 0, h, s].tolist() == want, (style, R, b, s, h)


def pin_fp8_layout_and_skips_match_fp16(L):
    """Every call with an fp8 cache writes exactly the slots the fp16 variant
    writes (sentinel-filled caches on both sides), leaves Q (and the in-place
    K of call 1) as the fp16 variant leaves them, and its V bytes are the
    nearest codes of the fp16 V values times 1/v_scale."""
    ks, vs = 0.0123, 0.0109
    rv = _rcp(vs)
    for style in (NEOX, GPTJ):
        # call 1
        w = W.packed(2, 7, 3, 2, 64, 48, 9, style, 50 + style, table_batch=2, table_len=9)
        q16, c16 = oracle.packed_qkv(w.cos_sin, w.qkv, w.cache, style, L)
        c8 = np.full(w.cache.shape, W.SENTINEL8, dtype=np.uint8)
        q8, c8 = oracle.packed_qkv_fp8(w.cos_sin, w.qkv, c8, ks, vs, style, L)
        assert np.array_equal(q8, q16)
        assert np.array_equal(c8 == W.SENTINEL8, c16 == W.SENTINEL)
        assert np.array_equal(c8[:, 1, :, :w.S], _nearest_e4m3(val(c16[:, 1, :, :w.S]) * rv))
        # calls 2 and 3 with out-of-range tokens
        B, S, Hq, Hkv, D, cap = 3, 6, 2, 2, 64, 12
        r = np.random.default_rng(60 + style)
        qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
        table = W.rope_table(1, 10, D, 10000.0)
        end = np.array([3, 12, 8], dtype=np.int32)
        pos = np.array([[-1, 0, 1, 2, 9, 10]] * B, dtype=np.int32)
        for call in ("continuous", "tree"):
            cache16 = W.sentinel_f16((B, 2, Hkv, cap, D))
            cache8 = np.full(cache16.shape, W.SENTINEL8, dtype=np.uint8)
            qo = W.sentinel_f16((B, S, Hq, D))
            if call == "continuous":
                c16, q16 = oracle.continuous(table, end, qkv, cache16, qo, style, L)
                c8, q8 = oracle.continuous_fp8(table, end, qkv, cache8, qo, ks, vs, style, L)
            else:
                c16, q16 = oracle.tree(table, end, pos, qkv, cache16, qo, style, L)
                c8, q8 = oracle.tree_fp8(table, end, pos, qkv, cache8, qo, ks, vs, style, L)
            assert np.array_equal(q8, q16), call
            written = c16 != W.SENTINEL
            assert np.array_equal(c8 != W.SENTINEL8, written), call
            assert written.any() and not written.all()
            v16 = c16[:, 1][written[:, 1]]
            assert np.array_equal(c8[:, 1][written[:, 1]], _nearest_e4m3(val(v16) * rv)), call
        # call 4, plain and with the gather fused in
        w = W.paged(96, 4, 2, 64, 64, 12, 3, style, 70 + style, width=24, pool_fill="sentinel")
        p16 = oracle.paged_delta(w.k_delta, w.v_delta, w.pool, w.cos_sin, w.positions, w.seq,
                                 w.page_table, w.batch, style, L)
        p8 = oracle.paged_delta_fp8(w.k_delta, w.v_delta,
                                    np.full(w.pool.shape, W.SENTINEL8, np.uint8), w.cos_sin,
                                    w.positions, w.seq, w.page_table, w.batch, ks, vs, style, L)
        written = p16 != W.SENTINEL
        assert np.array_equal(p8 != W.SENTINEL8, written)
        assert np.array_equal(p8[1][written[1]], _nearest_e4m3(val(p16[1][written[1]]) * rv))
        rope = W.rope_table(4, 200, 64, 10000.0, offsets=np.array([0, 3, 9, 27]))
        si = np.array([3, 1, 0, 2], dtype=np.int32)
        g16 = oracle.paged_delta_gather(w.k_delta, w.v_delta, w.pool, rope, si, w.positions,
                                        w.seq, w.page_table, w.batch, style, L)
        g8 = oracle.paged_delta_gather_fp8(w.k_delta, w.v_delta,
                                           np.full(w.pool.shape, W.SENTINEL8, np.uint8), rope,
                                           si, w.positions, w.seq, w.page_table, w.batch, ks, vs,
                                           style, L)
        gw = g16 != W.SENTINEL
        assert np.array_equal(g8 != W.SENTINEL8, gw)
        # K through the gather: the rotation with the gathered row
        rows = oracle.gather_delta_rope(rope, si, w.positions, w.seq, w.batch, L)
        k8 = oracle.paged_delta_fp8(w.k_delta, w.v_delta,
                                    np.full(w.pool.shape, W.SENTINEL8, np.uint8), rows,
                                    w.positions, w.seq, w.page_table, w.batch, ks, vs, style, L)
        assert np.array_equal(g8[0], k8[0])


def pin_fp8_k_near_fp16(L):
    """Scale 1: each K byte decodes to within half an E4M3 quantum (plus the
    fp16 rounding) of the fp16 variant's K."""
    w = W.packed(1, 32, 2, 4, 128, 128, 32, NEOX, 80)
    _, c16 = oracle.packed_qkv(w.cos_sin, w.qkv, w.cache, NEOX, L)
    c8 = np.full(w.cache.shape, W.SENTINEL8, dtype=np.uint8)
    _, c8 = oracle.packed_qkv_fp8(w.cos_sin, w.qkv, c8, None, None, NEOX, L)
    k16 = val(c16[:, 0])
    k8 = _e4m3_values()[c8[:, 0].astype(np.int64)]
    a = np.abs(k16)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    quantum = 2.0 ** (e - 3)
    assert np.all(np.abs(k8 - k16) <= quantum / 2 + 2.0 ** -11 * a + 2.0 ** -25)


def pin_fp8_cross_call_reductions(L):
    """The fp8 cache of call 2 from an empty cache equals call 1's (whose K
    bytes are pinned exactly above), a linear-chain tree equals call 2, and the
    paged update through an identity page table equals call 2's K and V."""
    r = np.random.default_rng(90)
    B, S, Hq, Hkv, D, cap = 2, 6, 2, 2, 64, 10
    ks, vs = 0.0123, 0.0109
    for style in (NEOX, GPTJ):
        qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
        table = W.rope_table(1, cap, D, 10000.0)
        cache = np.full((B, 2, Hkv, cap, D), W.SENTINEL8, dtype=np.uint8)
        _, c1 = oracle.packed_qkv_fp8(table, qkv, cache, ks, vs, style, L)
        end = np.full(B, S, dtype=np.int32)
        c2, _ = oracle.continuous_fp8(table, end, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                                      ks, vs, style, L)
        assert np.array_equal(c1, c2), style
        end = np.array([7, 10], dtype=np.int32)
        c2, _ = oracle.continuous_fp8(table, end, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                                      ks, vs, style, L)
        pos = (end[:, None] - S + np.arange(S)[None, :]).astype(np.int32)
        c3, _ = oracle.tree_fp8(table, end, pos, qkv, cache, W.sentinel_f16((B, S, Hq, D)),
                                ks, vs, style, L)
        assert np.array_equal(c2, c3), style
        P = B
        pt = np.empty((B, 2, 1), dtype=np.int32)
        pt[:, 0, 0] = np.arange(B)
        pt[:, 1, 0] = P + np.arange(B)
        N = B * S
        k_delta = qkv[:, :, Hq:Hq + Hkv].reshape(N, Hkv, D)
        v_delta = qkv[:, :, Hq + Hkv:].reshape(N, Hkv, D)
        posd = pos.reshape(-1).astype(np.int32)
        seqd = np.repeat(np.arange(B), S).astype(np.int32)
        pool = np.full((2, P, 64, Hkv, D), W.SENTINEL8, dtype=np.uint8)
        pool = oracle.paged_delta_fp8(k_delta, v_delta, pool, table[0][posd], posd, seqd, pt, B,
                                      ks, vs, style, L)
        for b in range(B):
            for plane in range(2):
                got = pool[plane, b, :cap].transpose(1, 0, 2)
                assert np.array_equal(got, c2[b, plane]), (style, b, plane)


# ------------------------------------------------------------ Q/K norm --

def _exact_mean_square(bits) -> float:
    """Python integers: each fp16 value times 2^24 is an integer; the mean
    of squares as an exact fraction, converted once (float(Fraction) rounds
    correctly)."""
    v = val(bits)
    if np.isnan(v).any():
        return float("nan")
    if np.isinf(v).any():
        return float("inf")
    total = sum(int(round(abs(float(a)) * 2 ** 24)) ** 2 for a in v)
    return float(Fraction(total, 2 ** 48 * len(v)))


def pin_mean_square_exact(L):
    r = np.random.default_rng(100)
    rows = [W.normal_f16(r, (128,)), W.normal_f16(r, (64,)), W.normal_f16(r, (256,)),
            f16(r.uniform(-6e4, 6e4, 128)), f16(np.exp2(r.uniform(-24, 15, 128)))]
    # one large square and many small ones: a running binary64 sum would drop
    # the small ones, the exact mean keeps them
    big = np.full(256, 2.0 ** -12)
    big[0] = 2.0 ** 15
    rows.append(f16(big))
    rows.append(np.arange(1, 129, dtype=np.uint16))            # subnormals only
    rows.append(np.zeros(64, dtype=np.uint16))
    tiny = np.zeros(64, dtype=np.uint16)
    tiny[9] = 0x8001                                           # one -2^-24: the sum is 2^-48
    rows.append(tiny)
    for x in rows:
        assert oracle.mean_square(x, L) == _exact_mean_square(x), x[:4]
    x = W.normal_f16(r, (64,))
    x[5] = 0x7C00
    assert np.isinf(oracle.mean_square(x, L))
    x[6] = 0x7E00
    assert np.isnan(oracle.mean_square(x, L))


def pin_rms_norm_closed_forms(L):
    r = np.random.default_rng(101)
    wt = (0.5 + r.random(128)).astype(np.float32)
    # a row of +-2^k: mean square 2^2k, so with eps = 0 the row becomes +-w exactly
    for k in (-20, -3, 0, 7, 15):
        signs = r.choice([-1.0, 1.0], 128)
        n = oracle.rms_normalize(f16(signs * 2.0 ** k), wt, 0.0, L)
        assert np.array_equal(n, signs * wt.astype(np.float64)), k
    # scale invariance by powers of two (exact) with eps = 0
    x = W.normal_f16(r, (128,))
    for j in (-4, 3):
        xs = f16(val(x) * 2.0 ** j)
        assert np.array_equal(oracle.rms_normalize(xs, wt, 0.0, L),
                              oracle.rms_normalize(x, wt, 0.0, L)), j
    # with unit weights the normalised row has mean square 1
    n = oracle.rms_normalize(x, np.ones(128, np.float32), 0.0, L)
    assert abs(np.mean(n ** 2) - 1.0) < 1e-14
    # a dominant epsilon: n = x * w / sqrt(ms + eps)
    eps = 1e6
    n = oracle.rms_normalize(x, wt, eps, L)
    ms = np.mean(val(x) ** 2)
    assert np.allclose(n, val(x) * wt / np.sqrt(ms + eps), rtol=1e-14, atol=0)
    # a zero row with eps = 0 is 0/0
    assert np.isnan(oracle.rms_normalize(np.zeros(64, np.uint16), wt[:64], 0.0, L)).all()


def _numpy_qknorm_packed(cos_sin, qkv, Hq, Hkv, qw, kw, eps, style):
    """Independent float64 model of call 1 with Q/K norm: r = sqrt(D)/||x||
    (np.linalg.norm, pairwise summation), then the rotation as a complex
    multiplication, rounded to fp16 by numpy."""
    B, S, H, D = qkv.shape
    R = cos_sin.shape[2]
    half = R // 2
    out = qkv.copy()
    for b in range(B):
        t = 0 if cos_sin.shape[0] == 1 else b
        for s in range(S):
            c = cos_sin[t, s, :half].astype(np.float64)
            sn = cos_sin[t, s, half:].astype(np.float64)
            for h in range(Hq + Hkv):
                wt = qw if h < Hq else kw
                x = val(qkv[b, s, h])
                if wt is not None:
                    nrm = np.linalg.norm(x) / np.sqrt(D)
                    x = x * wt.astype(np.float64) / np.sqrt(nrm ** 2 + eps)
                y = x.copy()
                if style == NEOX:
                    z = (x[:half] + 1j * x[half:R]) * (c + 1j * sn)
                    y[:half], y[half:R] = z.real, z.imag
                else:
                    z = (x[0:R:2] + 1j * x[1:R:2]) * (c + 1j * sn)
                    y[0:R:2], y[1:R:2] = z.real, z.imag
                out[b, s, h] = f16(y) if (wt is not None or R == D) else \
                    np.concatenate([f16(y[:R]), qkv[b, s, h, R:]])
    return out


def pin_qknorm_against_numpy(L):
    """Whole call 1 with Q/K norm against the independent numpy model: at
    most one fp16 ulp apart (the two binary64 evaluations differ in the last
    bits) and equal almost everywhere."""
    for style, D, R, eps in [(NEOX, 128, 128, 1e-6), (GPTJ, 64, 32, 1e-5), (NEOX, 128, 64, 0.0)]:
        w = W.with_qk_norm(W.packed(2, 6, 3, 2, D, R, 8, style, 110 + D + R), 111 + R, eps=eps,
                           scale=7.0)
        n = w.extra["qknorm"]
        got, _ = oracle.packed_qkv_qknorm(w.cos_sin, w.qkv, w.cache, n["q_weight"],
                                          n["k_weight"], n["eps"], style, L=L)
        want = _numpy_qknorm_packed(w.cos_sin, w.qkv, w.Hq, w.Hkv, n["q_weight"], n["k_weight"],
                                    n["eps"], style)
        g = got.view(np.float16).astype(np.float64)
        e = want.view(np.float16).astype(np.float64)
        diff = got != want
        assert diff.mean() < 1e-3, (style, D, R, diff.mean())
        ulp = np.spacing(np.abs(want.view(np.float16))).astype(np.float64)
        assert np.all(np.abs(g - e) <= ulp), (style, D, R)


def pin_qknorm_weight_roles(L):
    """Q heads use the Q weight, K heads the K weight, V is untouched; a
    side without a weight is the plain call's output for that side."""
    r = np.random.default_rng(120)
    B, S, Hq, Hkv, D, cap = 1, 4, 2, 2, 64, 4
    qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    qkv[:, :, Hq:Hq + Hkv] = qkv[:, :, :Hkv]                  # K heads copy Q heads 0..Hkv-1
    table = np.zeros((1, cap, 0), dtype=np.float32)            # R = 0: no rotation
    ones = np.ones(D, np.float32)
    cache = W.sentinel_f16((B, 2, Hkv, cap, D))
    q2, c2 = oracle.packed_qkv_qknorm(table, qkv, cache, ones, 2 * ones, 1e-6, NEOX, L=L)
    assert np.array_equal(val(q2[:, :, Hq:Hq + Hkv]), 2 * val(q2[:, :, :Hkv]))
    assert np.array_equal(q2[:, :, Hq + Hkv:], qkv[:, :, Hq + Hkv:])
    assert np.array_equal(c2[0, 1].transpose(1, 0, 2), qkv[0, :, Hq + Hkv:])
    assert np.array_equal(c2[0, 0].transpose(1, 0, 2), q2[0, :, Hq:Hq + Hkv])
    # no Q weight: Q rows as the plain call leaves them (here unrotated, R = 0)
    q3, _ = oracle.packed_qkv_qknorm(table, qkv, cache, None, ones, 1e-6, NEOX, L=L)
    assert np.array_equal(q3[:, :, :Hq], qkv[:, :, :Hq])
    assert np.array_equal(q3[:, :, Hq:Hq + Hkv], q2[:, :, :Hkv])


def pin_qknorm_without_weights_is_the_plain_call(L):
    for w in (W.packed(2, 5, 3, 2, 64, 48, 8, GPTJ, 130),
              W.continuous(2, 5, 3, 2, 64, 64, 12, NEOX, 131, 3, 12),
              W.tree(2, 5, 3, 2, 128, 64, 16, NEOX, 132, 5, 16)):
        plain = oracle.run(w, L=L)
        w.extra["qknorm"] = {"q_weight": None, "k_weight": None, "eps": 1e-6}
        normed = oracle.run(w, L=L)
        for k in plain:
            assert np.array_equal(plain[k], normed[k]), (w.call, k)
        W.with_fp8_cache(w, 133, fill="sentinel")
        normed = oracle.run(w, L=L)
        del w.extra["qknorm"]
        plain = oracle.run(w, L=L)
        for k in plain:
            assert np.array_equal(plain[k], normed[k]), (w.call, k, "fp8")


def pin_qknorm_fp8_and_calls_agree(L):
    """With norm, the E4M3 cache is written where the fp16 cache is, its V
    bytes are the nearest codes of V/v_scale, its K bytes decode to within
    half a quantum (plus the fp16 rounding) of the fp16 K times 1/k_scale;
    call 2 from an empty cache equals call 1, a linear tree equals call 2."""
    for style in (NEOX, GPTJ):
        w = W.with_qk_norm(W.packed(2, 6, 3, 2, 128, 96, 10, style, 140 + style), 141, scale=3.0)
        n = w.extra["qknorm"]
        q16, c16 = oracle.run(w, L=L)["qkv"], oracle.run(w, L=L)["cache"]
        c8 = np.full(w.cache.shape, W.SENTINEL8, np.uint8)
        q8, c8 = oracle.packed_qkv_qknorm(w.cos_sin, w.qkv, c8, n["q_weight"], n["k_weight"],
                                          n["eps"], style, 1.0, 0.5, L=L)
        assert np.array_equal(q8, q16)
        written = c16 != W.SENTINEL
        assert np.array_equal(c8 != W.SENTINEL8, written)
        assert np.array_equal(c8[:, 1][written[:, 1]], _nearest_e4m3(val(c16[:, 1][written[:, 1]]) * 2))
        k16 = val(c16[:, 0][written[:, 0]])
        k8 = _e4m3_values()[c8[:, 0][written[:, 0]].astype(np.int64)]
        a = np.abs(k16)
        quantum = 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)
        assert np.all(np.abs(k8 - k16) <= quantum / 2 + 2.0 ** -11 * a + 2.0 ** -25)
        # call 2 with end = S from an empty cache is call 1
        end = np.full(w.B, w.S, np.int32)
        c2, qo = oracle.continuous_qknorm(w.cos_sin, end, w.qkv, w.cache,
                                          W.sentinel_f16((w.B, w.S, w.Hq, w.D)), n["q_weight"],
                                          n["k_weight"], n["eps"], style, L=L)
        assert np.array_equal(c2, c16) and np.array_equal(qo, q16[:, :, :w.Hq])
        pos = np.tile(np.arange(w.S, dtype=np.int32), (w.B, 1))
        c3, qo3 = oracle.tree_qknorm(w.cos_sin, end, pos, w.qkv, w.cache,
                                     W.sentinel_f16((w.B, w.S, w.Hq, w.D)), n["q_weight"],
                                     n["k_weight"], n["eps"], style, L=L)
        assert np.array_equal(c3, c2) and np.array_equal(qo3, qo)


def pin_qknorm_argument_errors(L):
    w = W.packed(1, 2, 1, 1, 64, 64, 4, NEOX, 150)
    ones = np.ones(64, np.float32)
    for eps in (-1e-6, float("inf"), float("nan")):
        try:
            oracle.packed_qkv_qknorm(w.cos_sin, w.qkv, w.cache, ones, ones, eps, NEOX, L=L)
        except oracle.OracleError as e:
            assert e.code == oracle.ERR_ARG
        else:
            raise AssertionError(f"eps {eps} accepted")


# ------------------------------------------------------------ metadata --

def pin_delta_metadata_golden(L):
    n = 0
    for line in open(os.path.join(GOLDEN, "delta_metadata.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        width, old, dl, pos, seq = [f.split() for f in line.split("|")]
        got_p, got_s = oracle.prepare_delta_metadata(np.array(old, np.int32),
                                                     np.array(dl, np.int32), int(width[0]), L)
        assert got_p.tolist() == [int(v) for v in pos], (line, got_p)
        assert got_s.tolist() == [int(v) for v in seq], (line, got_s)
        n += 1
    assert n == 3


def pin_delta_metadata_invariants(L):
    """Each sequence owns a prefix of its block of width rows, of length
    clamp(deltaLength, 0, width), at consecutive positions from its old
    length; every other row is padding in both arrays."""
    r = np.random.default_rng(160)
    B, width = 37, 24
    old = r.integers(0, 100000, B).astype(np.int32)
    dl = r.integers(-3, width + 5, B).astype(np.int32)
    pos, seq = oracle.prepare_delta_metadata(old, dl, width, L)
    pos, seq = pos.reshape(B, width), seq.reshape(B, width)
    for b in range(B):
        k = min(max(int(dl[b]), 0), width)
        assert np.array_equal(pos[b, :k], old[b] + np.arange(k)), b
        assert np.all(seq[b, :k] == b) and np.all(pos[b, k:] == -1) and np.all(seq[b, k:] == -1)


def pin_linear_tree_metadata(L):
    """Node 0 is the root; each later node's parent is the previous node;
    each depth is the number of parent steps to the root (walked here)."""
    par, dep = oracle.linear_tree_metadata(3, 9, L)
    for b in range(3):
        assert par[b, 0] == -1
        for i in range(1, 9):
            assert par[b, i] == i - 1
        for i in range(9):
            steps, node = 0, i
            while par[b, node] != -1:
                node, steps = par[b, node], steps + 1
            assert dep[b, i] == steps
    p0, d0 = oracle.linear_tree_metadata(0, 5, L)
    assert p0.size == 0 and d0.size == 0


def pin_metadata_feeds_the_writes(L):
    """The builders' outputs drive calls 3 and 4 exactly like the direct
    positions: call 3 with tokenPosIds = end - S + linear depth equals call
    2; call 4 fed by the delta metadata through an identity page table
    writes what call 2 writes for the same tokens."""
    r = np.random.default_rng(170)
    B, S, Hq, Hkv, D = 3, 6, 2, 2, 64
    qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    table = W.rope_table(1, 64, D, 10000.0)
    end = np.array([6, 40, 17], np.int32)
    cache = W.sentinel_f16((B, 2, Hkv, 64, D))
    c2, q2 = oracle.continuous(table, end, qkv, cache, W.sentinel_f16((B, S, Hq, D)), NEOX, L)
    _, dep = oracle.linear_tree_metadata(B, S, L)
    c3, q3 = oracle.tree(table, end, (end[:, None] - S + dep).astype(np.int32), qkv, cache,
                         W.sentinel_f16((B, S, Hq, D)), NEOX, L)
    assert np.array_equal(c2, c3) and np.array_equal(q2, q3)
    old = (end - S).astype(np.int32)
    pos, seq = oracle.prepare_delta_metadata(old, np.full(B, S, np.int32), S, L)
    pt = np.empty((B, 2, 1), np.int32)
    pt[:, 0, 0] = np.arange(B)
    pt[:, 1, 0] = B + np.arange(B)
    rows = table[0][np.maximum(pos, 0)]
    pool = oracle.paged_delta(qkv[:, :, Hq:Hq + Hkv].reshape(B * S, Hkv, D),
                              qkv[:, :, Hq + Hkv:].reshape(B * S, Hkv, D),
                              W.sentinel_f16((2, B, 64, Hkv, D)), rows, pos, seq, pt, B, NEOX, L)
    for b in range(B):
        for plane in range(2):
            assert np.array_equal(pool[plane, b].transpose(1, 0, 2), c2[b, plane]), (b, plane)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
