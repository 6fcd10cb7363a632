"""Pins of the CPU oracle to facts outside itself (no GPU needed).

The oracle computes C = A*B + sum(peers) in fp64 and rounds once (GEMM +
AllReduce row of Table 3, thelatestinai.com page). Each pin below checks it
against something it does not share code with:
  - integer-valued inputs: an exact int64 evaluation (numpy integer matmul);
  - tiny shapes: exact rational arithmetic (fractions.Fraction) with a
    rounding routine written here;
  - peer permutation: bitwise invariance of the result;
  - bfloat16 rounding: hand-derived cases in tests/golden/bf16_rne_cases.txt;
  - the exact peer summation: math.fsum (correctly rounded) on adversarial data;
  - hand-worked GEMM+AllReduce cases in tests/golden/hand_cases.json;
  - row selection: rows computed alone equal the same rows of a full run;
  - the GEMM+ReduceScatter share: over a simulated K-split group, ReduceScatter
    followed by AllGather gives numpy's exact int64 product.
The last test builds planted-mistake variants of the oracle and checks that
every one of them fails at least one pin.
"""
import json
import math
import os
import random
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import build as oracle_build
from tests.compare import check_exact, check_tolerance, tolerance_stats

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# --------------------------------------------------------------------------- helpers

def bf16_bits_of(values):
    """bfloat16 bit patterns of values that are exactly representable in bfloat16."""
    f = np.asarray(values, dtype=np.float64).astype(np.float32)
    assert np.all(f.astype(np.float64) == np.asarray(values, dtype=np.float64))
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bfloat16"
    return (u >> 16).astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def frac_rne(q, p, emin, emax):
    """Round the rational q to a binary format with p significant bits, minimum normal
    exponent emin and maximum exponent emax, ties to even. Returns a Fraction or +-inf."""
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    m = a / quantum
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** (emax + 1):
        return s * math.inf
    return s * v


def frac_to_bf16_bits(q):
    v = frac_rne(q, 8, -126, 127)
    if isinstance(v, float):
        return 0x7F80 if v > 0 else 0xFF80
    f = np.float32(float(v))
    u = int(np.array([f]).view(np.uint32)[0])
    if v == 0 and q < 0:
        u = 0x80000000
    assert u & 0xFFFF == 0
    return u >> 16


def frac_to_f32(q):
    v = frac_rne(q, 24, -126, 127)
    if isinstance(v, float):
        return np.float32(v)
    return np.float32(float(v))


def random_bf16(rng, shape, spread=0):
    """Random bfloat16 values; spread > 0 scales each by 2^U(-spread, spread)."""
    x = rng.standard_normal(shape).astype(np.float32)
    if spread:
        x = x * np.exp2(rng.integers(-spread, spread + 1, size=shape)).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_f32(rng, shape, spread=0):
    x = rng.standard_normal(shape).astype(np.float32)
    if spread:
        x = x * np.exp2(rng.integers(-spread, spread + 1, size=shape)).astype(np.float32)
    return x


def peer_values_f64(peers):
    if peers is None or len(peers) == 0:
        return None
    if peers.dtype == np.uint16:
        return bits_to_f64(peers)
    return peers.astype(np.float64)


# --------------------------------------------------------------------------- pins

def pin_integer_exact(orc, seed=0):
    """Integer inputs in [-4,4]: C64 equals the int64 result exactly, and C_out equals
    its rounding by torch's float32->bfloat16 conversion (integers below 2^24 are exact
    in float32, so that conversion rounds once)."""
    rng = np.random.default_rng(seed)
    shapes = [(37, 24, 40, 3), (130, 136, 72, 15), (1, 8, 8, 0), (16, 16, 0, 2), (5, 16, 8, 1),
              (64, 40, 264, 7)]
    for (M, N, K, npeer) in shapes:
        A = rng.integers(-4, 5, size=(M, K))
        B = rng.integers(-4, 5, size=(K, N))
        P = rng.integers(-4, 5, size=(npeer, M, N))
        want = A.astype(np.int64) @ B.astype(np.int64) + P.sum(axis=0).astype(np.int64)
        for peer_dt in ("bf16", "f32"):
            peers = bf16_bits_of(P) if peer_dt == "bf16" else P.astype(np.float32)
            for c_dt in ("bf16", "f32"):
                C64, Cout = orc.gemm_ar(bf16_bits_of(A), bf16_bits_of(B), peers, c_dt)
                assert np.array_equal(C64, want.astype(np.float64)), (M, N, K, npeer)
                w32 = torch.from_numpy(want.astype(np.float32))
                if c_dt == "bf16":
                    wbits = w32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                    check_exact(Cout, wbits, f"int {M}x{N}x{K} P-1={npeer} {peer_dt}")
                else:
                    check_exact(Cout, w32.numpy(), f"int {M}x{N}x{K} P-1={npeer} {peer_dt}")


def pin_bruteforce_fraction(orc, n_cases=200, seed=1):
    """Tiny random shapes against exact rational arithmetic.

    The oracle's C64 must lie within the recursive-summation error bound of the exact
    value: |C64 - C| <= gamma_{K} sum|a b| + u |S| + u |G + S|, u = 2^-53 (peer sum S
    exact then rounded once, ascending-k sum G, one final addition). C_out must equal
    the exact value rounded once, unless the exact value is within that bound of a
    rounding boundary (then either neighbour is acceptable)."""
    rng = np.random.default_rng(seed)
    u = 2.0 ** -53
    for case in range(n_cases):
        M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        K = int(rng.integers(0, 9))
        npeer = int(rng.integers(0, 5))
        spread = int(rng.choice([0, 0, 8, 40, 60]))
        A = random_bf16(rng, (M, K), spread)
        B = random_bf16(rng, (K, N), spread)
        peer_dt = "f32" if case % 2 else "bf16"
        if npeer:
            peers = random_f32(rng, (npeer, M, N), spread) if peer_dt == "f32" else random_bf16(
                rng, (npeer, M, N), spread)
        else:
            peers = None
        c_dt = "bf16" if case % 3 else "f32"
        C64, Cout = orc.gemm_ar(A, B, peers, c_dt)
        Af, Bf, Pf = bits_to_f64(A), bits_to_f64(B), peer_values_f64(peers)
        for i in range(M):
            for j in range(N):
                prods = [Fraction(Af[i, k]) * Fraction(Bf[k, j]) for k in range(K)]
                pv = [Fraction(Pf[p, i, j]) for p in range(npeer)] if npeer else []
                exact = sum(prods, Fraction(0)) + sum(pv, Fraction(0))
                sabs = float(sum((abs(x) for x in prods), Fraction(0)))
                s_exact = float(abs(sum(pv, Fraction(0))))
                gk = K * u / (1 - K * u)
                bound = 1.01 * (gk * sabs + u * s_exact + u * (abs(float(exact)) + gk * sabs))
                err = abs(Fraction(C64[i, j]) - exact)
                assert err <= Fraction(bound) + Fraction(2.0 ** -1074), (case, i, j, float(err),
                                                                          bound)
                lo, hi = exact - Fraction(bound), exact + Fraction(bound)
                if c_dt == "bf16":
                    a, b = frac_to_bf16_bits(lo), frac_to_bf16_bits(hi)
                    if a == b:
                        assert int(Cout[i, j]) == frac_to_bf16_bits(exact), (case, i, j)
                else:
                    a, b = frac_to_f32(lo), frac_to_f32(hi)
                    if a == b:
                        want = frac_to_f32(exact)
                        assert Cout[i, j].view(np.uint32) == np.float32(want).view(np.uint32), (
                            case, i, j)


def pin_peer_permutation(orc, seed=2):
    """Reordering the peers leaves C64 and C_out bitwise unchanged, including peers whose
    magnitudes span far more than a double's 53 bits (where naive left-to-right
    summation would depend on the order)."""
    rng = np.random.default_rng(seed)
    for (M, N, K, npeer, spread) in [(7, 16, 24, 15, 0), (5, 8, 8, 7, 60), (3, 8, 16, 5, 90)]:
        A = random_bf16(rng, (M, K))
        B = random_bf16(rng, (K, N))
        for peer_dt in ("bf16", "f32"):
            if peer_dt == "bf16":
                peers = random_bf16(rng, (npeer, M, N), spread)
            else:
                peers = random_f32(rng, (npeer, M, N), spread)
            # plant exact cancellations across peers
            peers[0, 0, 0], peers[1, 0, 0] = peers[2, 0, 0], peers[2, 0, 0]
            if peer_dt == "f32":
                peers[1, 0, 0] = -peers[1, 0, 0]
                peers[0, 0, 1], peers[1, 0, 1], peers[2, 0, 1] = np.float32(2.0 ** 60), np.float32(
                    1.0), np.float32(-(2.0 ** 60))
            else:
                peers[1, 0, 0] ^= np.uint16(0x8000)
                peers[0, 0, 1], peers[1, 0, 1], peers[2, 0, 1] = 0x5D80, 0x3F80, 0xDD80
            ref64, refout = orc.gemm_ar(A, B, peers, "f32")
            _, refout16 = orc.gemm_ar(A, B, peers, "bf16")
            for _ in range(6):
                perm = rng.permutation(npeer)
                c64, cout = orc.gemm_ar(A, B, np.ascontiguousarray(peers[perm]), "f32")
                _, cout16 = orc.gemm_ar(A, B, np.ascontiguousarray(peers[perm]), "bf16")
                assert np.array_equal(c64.view(np.uint64), ref64.view(np.uint64))
                check_exact(cout, refout, "perm f32")
                check_exact(cout16, refout16, "perm bf16")


def read_rne_cases():
    cases = []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            x, want = line.split()[:2]
            cases.append((float.fromhex(x), int(want, 16)))
    return cases


def pin_bf16_rounding(orc, seed=3):
    """Hand-derived rounding cases, then random doubles against the rational rounding
    routine above, then float32-representable values against torch's conversion."""
    cases = read_rne_cases()
    xs = np.array([c[0] for c in cases], dtype=np.float64)
    got = orc.f64_to_bf16(xs)
    for (x, want), g in zip(cases, got):
        assert int(g) == want, f"bf16 RNE of {x!r}: got {int(g):#06x} want {want:#06x}"
    nan = orc.f64_to_bf16(np.array([np.nan]))[0]
    assert (int(nan) & 0x7F80) == 0x7F80 and (int(nan) & 0x7F) != 0
    rng = np.random.default_rng(seed)
    xs = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, size=3000))
    got = orc.f64_to_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == frac_to_bf16_bits(Fraction(float(x))), x
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, size=20000))).astype(
        np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    check_exact(orc.f64_to_bf16(f.astype(np.float64)), want, "bf16 vs torch")
    # widening is exact and inverse to rounding on representable values
    allbits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = (allbits & 0x7F80) != 0x7F80
    w = orc.bf16_to_f64(allbits[finite])
    assert np.array_equal(w, (allbits[finite].astype(np.uint32) << 16).view(np.float32).astype(
        np.float64))
    back = orc.f64_to_bf16(w)
    zero = w == 0
    check_exact(back[~zero], allbits[finite][~zero], "bf16 round trip")


def pin_exact_sum(orc, seed=4):
    """The exact peer summation equals math.fsum (a correctly rounded sum)."""
    rng = np.random.default_rng(seed)
    lists = [[1e-16, 1.0, 1e16], [1.0, 1e100, 1.0, -1e100], [2.0 ** 53, 1.0, -(2.0 ** 53)],
             [2.0 ** 53, 1.0, 1.0 / 2 ** 30], [1.0, 2.0 ** -53, 2.0 ** -106],
             [1.0, -(2.0 ** -54), -(2.0 ** -120)], [0.1] * 10, []]
    # 64 values (the most peers), each in its own binade: 64 non-overlapping partials
    lists.append([(-1.0) ** i * 2.0 ** (16 * i) for i in range(-32, 32)])
    lists.append(list(rng.standard_normal(64) * np.exp2(rng.integers(-300, 300, size=64))))
    for _ in range(3000):
        n = int(rng.integers(1, 20))
        v = rng.standard_normal(n) * np.exp2(rng.integers(-80, 80, size=n))
        if rng.random() < 0.3:
            v = np.concatenate([v, -v[: n // 2]])
        lists.append(list(rng.permutation(v)))
    for L in lists:
        got = orc.exact_sum(np.array(L, dtype=np.float64))
        want = math.fsum(L)
        assert got == want, (L, got, want)


def pin_hand_cases(orc):
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        A = np.array(case["A"], dtype=np.float64)
        if A.size == 0:
            A = A.reshape(len(case["A"]), 0)
        N = case.get("N") or len(case["C"][0])
        K = A.shape[1]
        B = np.array(case["B"], dtype=np.float64).reshape(K, N)
        M = A.shape[0]
        P = np.array(case["peers"], dtype=np.float64).reshape(-1, M, N)
        peers = P.astype(np.float32) if len(P) else None
        C64, Cf = orc.gemm_ar(bf16_bits_of(A), bf16_bits_of(B), peers, "f32")
        assert np.array_equal(C64, np.array(case["C"], dtype=np.float64)), case["name"]
        _, Cb = orc.gemm_ar(bf16_bits_of(A), bf16_bits_of(B),
                            bf16_bits_of(P) if len(P) else None, "bf16")
        want = np.array([int(b, 16) for b in case["C_bf16_bits"]], dtype=np.uint16).reshape(M, N)
        check_exact(Cb, want, case["name"])


def pin_row_selection(orc, seed=5):
    rng = np.random.default_rng(seed)
    M, N, K, npeer = 33, 24, 40, 3
    A, B = random_bf16(rng, (M, K)), random_bf16(rng, (K, N))
    peers = random_bf16(rng, (npeer, M, N))
    full64, full = orc.gemm_ar(A, B, peers, "bf16")
    rows = [32, 0, 17, 17, 5]
    c64, c = orc.gemm_ar(A, B, peers, "bf16", rows=rows)
    assert np.array_equal(c64, full64[rows])
    check_exact(c, full[rows], "row selection")


def pin_reduce_scatter_group(orc, seed=13):
    """GEMM+ReduceScatter share ("GEMM + ReduceScatter (TP)" row of Table 3): over a
    simulated group of P GPUs that split K, every GPU publishes its partial of the rows
    it does not own, each owner reduces its rows with the others' published rows as
    peers, and the owned slices put together are the whole product (ReduceScatter
    followed by AllGather is an AllReduce). Integer inputs keep everything exact, so
    the result is compared bit for bit with numpy's int64 matmul, rounded here."""
    rng = np.random.default_rng(seed)
    P, M, N, Kc = 4, 22, 16, 6
    A = rng.integers(-4, 5, (M, P * Kc))
    B = rng.integers(-4, 5, (P * Kc, N))
    full = A @ B
    bounds = [0, 5, 11, 11, 22]  # uneven slices, one of them empty
    Ab = [bf16_bits_of(A[:, r * Kc:(r + 1) * Kc]) for r in range(P)]
    Bb = [bf16_bits_of(B[r * Kc:(r + 1) * Kc]) for r in range(P)]
    sends = []
    for r in range(P):
        o0, o1 = bounds[r], bounds[r + 1]
        no_peers = np.zeros((0, o1 - o0, N), np.uint16)
        (owned, _, _), (other, _, s_out) = orc.gemm_rs(Ab[r], Bb[r], no_peers, o0, o1, "bf16",
                                                        "bf16")
        assert sorted(owned) == list(range(o0, o1)) and len(other) == M - (o1 - o0)
        send = np.zeros((M, N), np.uint16)
        send[other] = s_out
        # a published row is this GPU's own partial (|value| <= 96: exact in bfloat16)
        part = A[:, r * Kc:(r + 1) * Kc] @ B[r * Kc:(r + 1) * Kc]
        check_exact(send[other], bf16_bits_of(part[other]), f"send of GPU {r}")
        sends.append(send)
    C = np.zeros((M, N), np.uint16)
    for r in range(P):
        o0, o1 = bounds[r], bounds[r + 1]
        peers = np.stack([sends[q][o0:o1] for q in range(P) if q != r])
        (owned, c64, c_out), _ = orc.gemm_rs(Ab[r], Bb[r], peers, o0, o1, "bf16", "bf16")
        assert np.array_equal(c64, full[o0:o1].astype(np.float64))
        C[owned] = c_out
    want = np.array([[frac_to_bf16_bits(Fraction(int(v))) for v in row] for row in full],
                    dtype=np.uint16)
    check_exact(C, want, "ReduceScatter then AllGather")


def pin_allgather_group(orc, seed=17):
    """AllGather+GEMM share ("AllGather + GEMM (TP)" row of Table 3): over a simulated
    group of P GPUs, GPU r holds row shard r of the activation matrix X and column
    shard r of the weight W. After the gather every GPU holds all of X in rank order,
    and the GPUs' outputs side by side are X times W. The test builds X and W whole
    and slices them, so the shard order is fixed by the slicing, not by the oracle.
    Integer inputs keep the products exact: compared bit for bit with numpy's int64
    matmul, rounded here."""
    rng = np.random.default_rng(seed)
    P, Ms, K, Nc = 4, 3, 10, 5
    X = rng.integers(-4, 5, (P * Ms, K))
    W = rng.integers(-4, 5, (K, P * Nc))
    Xb = bf16_bits_of(X)
    outs = []
    for r in range(P):
        peers_A = np.stack([Xb[q * Ms:(q + 1) * Ms] for q in range(P) if q != r])
        A_full, c64, c_out = orc.gemm_ag(Xb[r * Ms:(r + 1) * Ms], peers_A, r,
                                         bf16_bits_of(W[:, r * Nc:(r + 1) * Nc]), "bf16")
        check_exact(A_full, Xb, f"gathered activations of GPU {r}")
        assert np.array_equal(c64, (X @ W[:, r * Nc:(r + 1) * Nc]).astype(np.float64))
        outs.append(c_out)
        # a row selection returns those rows of the whole result
        _, c64s, c_outs = orc.gemm_ag(Xb[r * Ms:(r + 1) * Ms], peers_A, r,
                                      bf16_bits_of(W[:, r * Nc:(r + 1) * Nc]), "bf16",
                                      rows=[P * Ms - 1, r * Ms, 0])
        check_exact(c_outs, c_out[[P * Ms - 1, r * Ms, 0]], f"selected rows of GPU {r}")
    full = X @ W
    want = np.array([[frac_to_bf16_bits(Fraction(int(v))) for v in row] for row in full],
                    dtype=np.uint16)
    check_exact(np.concatenate(outs, axis=1), want, "AllGather then column-parallel GEMM")


PINS = [pin_integer_exact, pin_bruteforce_fraction, pin_peer_permutation, pin_bf16_rounding,
        pin_exact_sum, pin_hand_cases, pin_row_selection, pin_reduce_scatter_group,
        pin_allgather_group]


# --------------------------------------------------------------------------- tests

@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_comparator_rejects_one_flipped_bit():
    rng = np.random.default_rng(6)
    A, B = random_bf16(rng, (16, 32)), random_bf16(rng, (32, 16))
    peers = random_bf16(rng, (3, 16, 16))
    C64, Cb = oracle.gemm_ar(A, B, peers, "bf16")
    check_exact(Cb, Cb.copy())
    check_tolerance(Cb, C64, "bf16")
    for bit in (0, 6, 9, 14):
        bad = Cb.copy()
        bad[3, 5] ^= np.uint16(1 << bit)
        with pytest.raises(AssertionError):
            check_exact(bad, Cb)
        if bit >= 6:
            assert not tolerance_stats(bad, C64, "bf16")["ok"]
    C64f, Cf = oracle.gemm_ar(A, B, peers, "f32")
    check_tolerance(Cf, C64f, "f32")
    bad = Cf.copy()
    bad.view(np.uint32)[2, 2] ^= np.uint32(1 << 22)
    assert not tolerance_stats(bad, C64f, "f32")["ok"]


def test_oracle_rejects_bad_arguments():
    A = np.zeros((4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_ar(A, np.zeros((7, 8), np.uint16), None)
    with pytest.raises(ValueError):
        oracle.gemm_ar(A, np.zeros((8, 8), np.uint16), None, rows=[4])
    with pytest.raises(ValueError):  # more peers than the library accepts (64)
        oracle.gemm_ar(A, np.zeros((8, 8), np.uint16), np.zeros((65, 4, 8), np.uint16))


def test_oracle_sums_the_most_peers_exactly():
    """64 peers spanning many binades: the peer sum equals math.fsum of them, and the
    result with A = 0 is its correct rounding."""
    rng = np.random.default_rng(9)
    vals = (rng.standard_normal((64, 2, 8)) * np.exp2(rng.integers(-60, 60, (64, 2, 8))))
    peers = vals.astype(np.float32)
    A = np.zeros((2, 8), np.uint16)
    B = np.zeros((8, 8), np.uint16)
    C64, C32 = oracle.gemm_ar(A, B, peers, "f32")
    for i in range(2):
        for j in range(8):
            want = math.fsum(float(v) for v in peers[:, i, j])
            assert C64[i, j] == want
            assert C32[i, j] == np.float32(want)


MUTANTS = {1: "drops the last peer", 2: "reads a mirrored column of B", 3: "subtracts the peers",
           4: "skips the last k", 5: "rounds bfloat16 ties away from zero",
           6: "adds peers left to right after the product sum", 7: "computes the wrong row",
           8: "drops a fraction bit when widening bfloat16",
           9: "omits the tie correction of the exact sum",
           10: "rounds the product sum and the peer sum separately to float32"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_reject_planted_mistake(mutant, tmp_path):
    lib = oracle_build.build(mutant=mutant, out=str(tmp_path / f"libmut{mutant}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the oracle that {MUTANTS[mutant]}"


class _BrokenRS(oracle.Oracle):
    """The ReduceScatter composition with one planted mistake."""

    def __init__(self, lib, mistake):
        super().__init__(lib)
        self.mistake = mistake

    def gemm_rs(self, A_bits, B_bits, peers_own, own_m0, own_m1, c_dtype="bf16",
                peer_dtype="bf16", rows=None, threads=0):
        M = A_bits.shape[0]
        rows = np.arange(M)
        mine = (rows >= own_m0) & (rows < own_m1)
        owned, other = rows[mine], rows[~mine]
        if self.mistake == "owned rows not shifted to the slice":
            sel = np.minimum(owned, own_m1 - own_m0 - 1) if own_m1 > own_m0 else owned - own_m0
            C64, C_out = self.gemm_ar(A_bits[own_m0:own_m1], B_bits, peers_own, c_dtype, rows=sel)
        elif self.mistake == "local partial left out of owned rows":
            C64, C_out = self.gemm_ar(np.zeros_like(A_bits[own_m0:own_m1]), B_bits, peers_own,
                                      c_dtype, rows=owned - own_m0)
        else:
            C64, C_out = self.gemm_ar(A_bits[own_m0:own_m1], B_bits, peers_own, c_dtype,
                                      rows=owned - own_m0)
        if self.mistake == "published rows taken from the owned slice":
            S64, S_out = self.gemm_ar(A_bits, B_bits, None, peer_dtype,
                                      rows=np.where(other < own_m0, other, other - 1))
        elif self.mistake == "publishes every row":
            S64, S_out = self.gemm_ar(A_bits, B_bits, None, peer_dtype, rows=rows)
            other = rows
        else:
            S64, S_out = self.gemm_ar(A_bits, B_bits, None, peer_dtype, rows=other)
        return (owned, C64, C_out), (other, S64, S_out)


@pytest.mark.parametrize("mistake", ["owned rows not shifted to the slice",
                                     "local partial left out of owned rows",
                                     "published rows taken from the owned slice",
                                     "publishes every row"])
def test_reduce_scatter_pin_rejects_planted_mistake(mistake):
    orc = _BrokenRS(oracle.default().path, mistake)
    with pytest.raises(AssertionError):
        pin_reduce_scatter_group(orc)


class _BrokenAG(oracle.Oracle):
    """The AllGather composition with one planted mistake."""

    def __init__(self, lib, mistake):
        super().__init__(lib)
        self.mistake = mistake

    def gemm_ag(self, A_local, peers_A, rank, B_bits, c_dtype="bf16", rows=None, threads=0):
        shards = [peers_A[q] for q in range(peers_A.shape[0])]
        if self.mistake == "local shard first":
            shards.insert(0, A_local)
        elif self.mistake == "local shard last":
            shards.append(A_local)
        elif self.mistake == "peers in reverse order":
            shards = shards[::-1]
            shards.insert(rank, A_local)
        else:  # "rank off by one"
            shards.insert(min(rank + 1, len(shards)), A_local)
        A_full = np.concatenate(shards, axis=0)
        C64, C_out = self.gemm_ar(A_full, B_bits, None, c_dtype, rows=rows, threads=threads)
        return A_full, C64, C_out


@pytest.mark.parametrize("mistake", ["local shard first", "local shard last",
                                     "peers in reverse order", "rank off by one"])
def test_allgather_pin_rejects_planted_mistake(mistake):
    orc = _BrokenAG(oracle.default().path, mistake)
    with pytest.raises(AssertionError):
        pin_allgather_group(orc)
