"""The error of the split-fp16 products that the matrix-core forms use,
checked on the host with numpy's fp16 rounding (round to nearest even, as
gfx950's v_cvt_pk_f16_f32): x_hi = fp16(x), x_lo = fp16(x - x_hi), and the
product a b formed as a_hi b_hi + a_hi b_lo + a_lo b_hi. The header states
each such product within 2^-21 of the exact one (the dropped a_lo b_lo is
at most 2^-22 |ab|, each operand's remainder at most 2^-23 of it) and about
2^-24 on average; the bf16 split (the opt-in) is far coarser."""
import numpy as np


def split16(x, dtype):
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        hi = x.astype(np.float16).astype(np.float64)
        lo = (x.astype(np.float64) - hi).astype(np.float16).astype(np.float64)
    else:   # bf16: keep the top 16 bits, round to nearest even
        def to_bf16(v):
            u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
            r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
            return r.astype(np.uint32).view(np.float32).astype(np.float64)
        hi = to_bf16(x)
        lo = to_bf16((x.astype(np.float64) - hi).astype(np.float32))
    return hi, lo


def operands(n, lo_exp, hi_exp, seed):
    rng = np.random.default_rng(seed)
    e = rng.uniform(lo_exp, hi_exp, n)
    return (rng.choice([-1.0, 1.0], n) * 2.0 ** e).astype(np.float32)


def product_errors(dtype, n=1_000_000):
    # unit-magnitude phasors against amplitudes scaled into [2^0, 2^15)
    a = operands(n, -2, 0, 1)
    b = operands(n, 0, 15, 2)
    ah, al = split16(a, dtype)
    bh, bl = split16(b, dtype)
    exact = a.astype(np.float64) * b.astype(np.float64)
    got = ah * bh + ah * bl + al * bh
    return np.abs(got - exact) / np.abs(exact)


def test_f16_split_products_within_the_stated_bound():
    rel = product_errors("f16")
    assert rel.max() <= 2.0 ** -21
    assert rel.mean() <= 2.0 ** -23.5
    a = operands(200_000, -2, 15, 3)
    h, l = split16(a, "f16")
    assert np.max(np.abs(a - (h + l)) / np.abs(a)) <= 2.0 ** -23


def test_bf16_split_is_coarser():
    f16, bf16 = product_errors("f16", 200_000), product_errors("bf16", 200_000)
    assert bf16.mean() > 8 * f16.mean()
    assert bf16.max() <= 2.0 ** -14
