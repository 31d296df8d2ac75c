"""Error of the three-term bf16 product used for the logits of bf16 models, on the CPU.

Each float32 operand x is split as x = hi + lo + r with hi = bf16(x) and lo = bf16(x - hi),
both rounded to nearest even, and a product taken as hi*hi + hi*lo + lo*hi.  bf16 keeps 8
significant bits, so |x - hi| <= 2^-8 |x| and |r| <= 2^-8 |x - hi| <= 2^-16 |x|; the dropped
lo*lo and the two products with a residual leave at most (3 * 2^-16 + 2^-30) |a b| per
product.  Checked against float64, and on hidden vectors and codebook weights of the synthetic
workloads' scale a 2048-term logit lands within 1e-4 of the exact one, a tenth of the decode's
1e-3 log-prob bound."""
import numpy as np


def bf16_rne(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def split(x):
    x = np.asarray(x, dtype=np.float32)
    hi = bf16_rne(x)
    lo = bf16_rne(x - hi)          # x - hi is exact in float32
    return hi, lo


def test_residual_of_the_split():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-20, 20, 200_000))).astype(np.float32)
    hi, lo = split(x)
    r = x.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64)
    assert np.all(np.abs(r) <= np.exp2(-16) * np.abs(x.astype(np.float64)))


def test_three_term_products():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(100_000).astype(np.float32)
    b = rng.standard_normal(100_000).astype(np.float32)
    ah, al = split(a)
    bh, bl = split(b)
    f = lambda v: v.astype(np.float64)
    got = f(ah) * f(bh) + f(ah) * f(bl) + f(al) * f(bh)
    exact = f(a) * f(b)
    assert np.all(np.abs(got - exact) <= (3 * np.exp2(-16) + np.exp2(-30)) * np.abs(exact))


def test_logits_of_workload_scale():
    rng = np.random.default_rng(3)
    H, V, R = 2048, 256, 128
    h = (rng.standard_normal((R, H)) * 0.3).astype(np.float32)
    w = (rng.standard_normal((H, V)) / np.sqrt(H)).astype(np.float32)
    hh, hl = split(h)
    wh, wl = split(w)
    f = lambda v: v.astype(np.float64)
    got = f(hh) @ f(wh) + f(hh) @ f(wl) + f(hl) @ f(wh)
    exact = f(h) @ f(w)
    bound = (3 * np.exp2(-16) + np.exp2(-30)) * (np.abs(f(h)) @ np.abs(f(w)))
    assert np.all(np.abs(got - exact) <= bound)
    assert float(np.max(np.abs(got - exact))) < 1e-4
