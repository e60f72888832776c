"""The rounding bound behind the many-token router's candidate test, checked
on the CPU against exact arithmetic.

With bf16 x and W_r the router scores experts approximately with fp32
accumulation of the H products x_h w_h (each product is exact in fp32), and
treats every expert whose exact score could reach the k-th largest as a
candidate. The test needs: for any order in which fp32 additions combine the
products (sequential, in blocks of 32 as one matrix-core step then into the
accumulator, split in two halves added at the end),

    |fp32 sum - exact sum| <= B = 2^-23 * 1.125 * H * |x| * |w|,

and for the norms, summed in fp32 from squares two at a time (each two-term
step rounding at most twice), the exact |v|^2 stays below
q * (1 + n 2^-21) + n 2^-120 for n >= H terms, including squares flushed to
zero below fp32's normal range.  Exact values: math.fsum of the fp64
products (bf16 x bf16 fits in 16 significant bits)."""
import math

import numpy as np
import pytest

F32 = np.float32


def bf16(a):
    """Round fp32 to bf16 (nearest even), returned as fp32 values."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def exact_dot(x, w):
    return math.fsum((x.astype(np.float64) * w.astype(np.float64)).tolist())


def f32_sequential(p):
    s = F32(0)
    for v in p:
        s = F32(s + v)
    return float(s)


def f32_blocks(p, blk=32):
    """Each block of 32 products summed by a pairwise tree, then added to
    the accumulator (one matrix-core step per block)."""
    acc = F32(0)
    for i in range(0, len(p), blk):
        b = list(p[i:i + blk])
        while len(b) > 1:
            b = [F32(b[j] + b[j + 1]) if j + 1 < len(b) else b[j] for j in range(0, len(b), 2)]
        acc = F32(acc + b[0])
    return float(acc)


def f32_halves(p):
    h = len(p) // 2
    return float(F32(F32(f32_blocks(p[:h])) + F32(f32_blocks(p[h:]))))


def bound(x, w):
    H = len(x)
    nx = math.sqrt(math.fsum((x.astype(np.float64) ** 2).tolist()))
    nw = math.sqrt(math.fsum((w.astype(np.float64) ** 2).tolist()))
    return 2.0 ** -23 * 1.125 * H * nx * nw


def inputs(kind, H, rng):
    if kind == "normal":
        x, w = rng.standard_normal(H), 0.02 * rng.standard_normal(H)
    elif kind == "wide":  # magnitudes spread over 2^-30 .. 2^30
        x = rng.standard_normal(H) * np.exp2(rng.uniform(-30, 30, H))
        w = rng.standard_normal(H) * np.exp2(rng.uniform(-30, 30, H))
    else:  # "cancel": products of alternating sign and equal size, plus a small remainder
        base = np.exp2(rng.uniform(0, 20, H // 2))
        x = np.repeat(base, 2)
        w = np.tile([1.0, -1.0], H // 2) * (1 + 2.0 ** -7 * rng.standard_normal(H))
    return bf16(x), bf16(w)


@pytest.mark.parametrize("H", [64, 256, 4096])
@pytest.mark.parametrize("kind", ["normal", "wide", "cancel"])
def test_fp32_score_within_bound(kind, H):
    rng = np.random.default_rng(H + len(kind))
    for _ in range(3 if H == 4096 else 8):
        x, w = inputs(kind, H, rng)
        p = (x * w).astype(np.float32)  # exact: 8-bit x 8-bit significands
        assert np.array_equal(p.astype(np.float64), x.astype(np.float64) * w.astype(np.float64))
        ex, B = exact_dot(x, w), bound(x, w)
        perm = rng.permutation(H)
        for approx in (f32_sequential(p), f32_sequential(p[::-1]), f32_sequential(p[perm]), f32_blocks(p),
                       f32_halves(p)):
            assert abs(approx - ex) <= B, (kind, H, approx, ex, B)


def f32_round_up(p):
    """Sequential fp32 sum with every inexact addition rounded up: a faithful
    rounding, and the slowest-converging one the bound must still cover."""
    s = F32(0)
    for v in p:
        t = F32(s + v)
        if float(t) < float(s) + float(v):  # fp32 + fp32 is exact in fp64 here
            t = np.nextafter(t, F32(np.inf))
        s = t
    return float(s)


def test_directed_rounding_stays_within_and_near_the_bound():
    """Positive products with low-order bits below the running sum's ulp, all
    rounded the same way: the error grows linearly with H and reaches about
    a tenth of B at H = 4096, so a bound short by a factor of ten fails here."""
    rng = np.random.default_rng(3)
    H = 4096
    x = bf16(1.0 + rng.uniform(0, 0.99, H))
    w = bf16(1.0 + rng.uniform(0, 0.99, H))
    p = (x * w).astype(np.float32)
    err = f32_round_up(p) - exact_dot(x, w)
    B = bound(x, w)
    assert 0.05 * B <= err <= B


def test_bound_is_tight_enough_to_prune():
    """For the prefill workload's statistics (x ~ N(0,1), W_r ~ N(0, 0.02),
    H = 4096) the bound is a few per cent of the spread of the scores, so
    only experts near the k-th score are recomputed."""
    rng = np.random.default_rng(7)
    x = bf16(rng.standard_normal(4096))
    W = bf16(0.02 * rng.standard_normal((64, 4096)))
    scores = W.astype(np.float64) @ x.astype(np.float64)
    B = max(bound(x, W[e]) for e in range(64))
    assert B < 0.05 * scores.std()


def norm_upper(q, n):
    return math.sqrt(float(q) * (1.0 + n * 2.0 ** -21) + n * 2.0 ** -120) * (1.0 + 2.0 ** -50)


def sq_pairs_f32(v, flush):
    """fp32 sum of squares two at a time: s = (a^2 + b^2) + s, two roundings per step."""
    s = F32(0)
    for i in range(0, len(v), 2):
        a2, b2 = F32(v[i]) * F32(v[i]), F32(v[i + 1]) * F32(v[i + 1])
        if flush:
            a2 = F32(0) if abs(a2) < 2.0 ** -126 else a2
            b2 = F32(0) if abs(b2) < 2.0 ** -126 else b2
        s = F32(F32(a2 + b2) + s)
    return s


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny"])
def test_norm_upper_bounds_exact_norm(kind):
    rng = np.random.default_rng(11 + len(kind))
    H = 4096
    for _ in range(4):
        if kind == "normal":
            v = rng.standard_normal(H)
        elif kind == "wide":
            v = rng.standard_normal(H) * np.exp2(rng.uniform(-40, 40, H))
        else:  # squares below fp32's normal range, flushed
            v = rng.standard_normal(H) * 2.0 ** -70
        v = bf16(v)
        exact = math.sqrt(math.fsum((v.astype(np.float64) ** 2).tolist()))
        for flush in (False, True):
            q = sq_pairs_f32(v, flush)
            assert norm_upper(q, H + 8) >= exact
