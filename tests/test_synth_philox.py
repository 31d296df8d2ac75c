"""The counter stream behind the bf16 inputs, written out from its definition and checked
against numpy's Philox bit generator (a library routine).

Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011, the Philox section): four 64-bit counter words, two key words; each of ten rounds
multiplies words 0 and 2 by two fixed constants, takes high and low product halves,
mixes the high halves with words 1 and 3 and the key, and the key grows by two Weyl
constants between rounds.  numpy's bit generator advances the counter by one before each
block, so block b of a fresh generator is the bijection applied to counter b + 1; a
generator's ``bytes`` read the 64-bit words little-endian.  The device generator of the
bf16 inputs follows exactly this definition; its GPU test compares it with the host
generator element by element."""
import numpy as np

from synth import get_config
from synth.gen import _T_CTX_K, _bf16_normal, _key, _philox, BF16_NORMAL_TABLE

M0, M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
W0, W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
MASK32 = np.uint64(0xFFFFFFFF)


def mulhilo(a, b):
    """(high, low) 64-bit halves of the 128-bit product of uint64 arrays, by 32-bit pieces."""
    s32 = np.uint64(32)
    al, ah = a & MASK32, a >> s32
    bl, bh = b & MASK32, b >> s32
    t = al * bl
    u = ah * bl + (t >> s32)
    v = al * bh + (u & MASK32)
    return ah * bh + (u >> s32) + (v >> s32), a * b


def philox4x64_10(counters, key):
    """Blocks of four words for counters [n] (low word; the other three zero)."""
    x0 = np.asarray(counters, dtype=np.uint64).copy()
    x1 = np.zeros_like(x0)
    x2 = np.zeros_like(x0)
    x3 = np.zeros_like(x0)
    k0, k1 = np.uint64(key & 0xFFFFFFFFFFFFFFFF), np.uint64(key >> 64)
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0, k1 = k0 + W0, k1 + W1
            hi0, lo0 = mulhilo(M0, x0)
            hi1, lo1 = mulhilo(M1, x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=1)


def test_mulhilo_against_python_integers():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2**64, size=200, dtype=np.uint64)
    b = rng.integers(0, 2**64, size=200, dtype=np.uint64)
    with np.errstate(over="ignore"):
        hi, lo = mulhilo(a, b)
    for x, y, h, l in zip(a.tolist(), b.tolist(), hi.tolist(), lo.tolist()):
        p = x * y
        assert h == p >> 64 and l == p & (2**64 - 1)


def test_definition_matches_numpy_bit_generator():
    cfg = get_config("ctx5k_beam256_r8")
    for tensor, a, b in [(1, 0, 0), (_T_CTX_K, 5, 27), (3, 2**31 - 1, 7)]:
        key = _key(cfg, tensor, a, b)
        raw = np.random.Philox(key=key).random_raw(4 * 64)
        mine = philox4x64_10(np.arange(1, 65), key).reshape(-1)
        assert np.array_equal(raw, mine), tensor


def test_bf16_values_are_table_lookups_of_the_word_stream():
    """Value i of a block = table[16-bit piece i of the little-endian word stream]."""
    cfg = get_config("ragged_r128")
    key = _key(cfg, _T_CTX_K, 17, 3)
    n = 1000 * 16 + 8                                 # ends inside a block
    got = _bf16_normal(_philox(cfg, _T_CTX_K, 17, 3), (n,))
    words = philox4x64_10(np.arange(1, (n + 15) // 16 + 1), key).reshape(-1)
    idx = ((words[:, None] >> (np.arange(4, dtype=np.uint64) * np.uint64(16))[None, :]) & np.uint64(0xFFFF))
    want = BF16_NORMAL_TABLE[idx.reshape(-1)[:n].astype(np.int64)]
    assert np.array_equal(got, want)
