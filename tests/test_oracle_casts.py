"""Pins for the oracle's casts (CPU only).

The oracle's round-to-nearest-even narrowing and exact widening are checked
against library casts over every f32 bit pattern (torch's CPU casts for
bf16 and fp16, numpy's float16 as a second library for fp16), and against
the IEEE definition itself (nearest representable value, ties to the even
one) on a structured set that covers every exponent, both tie directions,
subnormals, overflow and NaN.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

F16, BF16 = 1, 2
_TDT = {F16: torch.float16, BF16: torch.bfloat16}
CHUNK = 1 << 24


def _nan16(b, dtype):
    b = b.astype(np.int64)
    if dtype == F16:
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def _check_chunk(oracle_mod, first, n, dtype):
    got = oracle_mod.round_bits_range(first, n, dtype)
    x = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    want = torch.from_numpy(x).to(_TDT[dtype]).view(torch.int16).numpy().view(np.uint16)
    xnan = np.isnan(x)
    # NaN in -> NaN out (a quiet NaN; payload and sign are not part of the contract)
    assert _nan16(got[xnan], dtype).all()
    ok = ~xnan
    bad = ok & (got != want)
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"f32 bits {first + i:#010x}: oracle {got[i]:#06x} torch {want[i]:#06x}")
    return int(ok.sum())


@pytest.mark.slow
@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
def test_round_exhaustive_vs_torch(oracle_mod, dtype):
    """All 2^32 f32 inputs: the oracle's narrowing equals torch's CPU cast."""
    starts = range(0, 1 << 32, CHUNK)
    workers = min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(workers) as ex:
        total = sum(ex.map(lambda s: _check_chunk(oracle_mod, s, CHUNK, dtype), starts))
    assert total > (1 << 32) - (1 << 25)  # everything except the NaN patterns


def test_round_f16_vs_numpy_sample(oracle_mod):
    """fp16 against numpy's own float16 conversion (an independent library)."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    # add every exponent's boundary patterns
    e = np.arange(256, dtype=np.uint32) << 23
    low = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3FFF, 0x7FFFFF], dtype=np.uint32)
    bits = np.concatenate([bits, (e[:, None] | low[None, :]).ravel(),
                           (e[:, None] | low[None, :] | 0x80000000).ravel()])
    x = bits.view(np.float32)
    got = oracle_mod.round_to(x, F16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    ok = ~np.isnan(x)
    assert np.array_equal(got[ok], want[ok])
    assert _nan16(got[~ok], F16).all()


def _decode(bits, dtype):
    b = np.asarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(_TDT[dtype]).double().numpy()


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
def test_round_matches_ieee_definition(oracle_mod, dtype):
    """Nearest representable value, ties to even mantissa, overflow to inf.

    Checked with float64 arithmetic on the decoded candidates: the result r
    and its two neighbours r-, r+ (next patterns by magnitude) must satisfy
    |x - r| <= |x - r-| and |x - r| <= |x - r+|, with equality only when r's
    last mantissa bit is 0."""
    exps = np.arange(1, 255, dtype=np.uint32)
    mants = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x10000, 0x18000,
                      0x0FFF, 0x1000, 0x1001, 0x2000, 0x3000, 0x7FFFFF, 0x400000,
                      0x7F8000, 0x7FC000, 0x7FE000], dtype=np.uint32)
    pos = (exps[:, None] << 23 | mants[None, :]).ravel()
    sub = np.arange(0, 1 << 23, 997, dtype=np.uint32)  # f32 subnormals
    tiny = np.array([0x00008000, 0x00018000, 0x00010000, 0x00007FFF], dtype=np.uint32)
    bits = np.concatenate([pos, sub, tiny])
    bits = np.concatenate([bits, bits | 0x80000000])
    x = bits.view(np.float32)
    r_bits = oracle_mod.round_to(x, dtype)
    r = _decode(r_bits, dtype)
    xd = x.astype(np.float64)
    mag = r_bits.astype(np.int64) & 0x7FFF
    sign = r_bits.astype(np.int64) & 0x8000
    fin_max = 0x7F7F if dtype == BF16 else 0x7BFF
    finite = mag <= fin_max
    # overflow: the result is inf exactly when |x| >= max + half an ulp of max
    maxv = float(_decode(np.array([fin_max], dtype=np.uint16), dtype)[0])
    below = float(_decode(np.array([fin_max - 1], dtype=np.uint16), dtype)[0])
    half = (maxv - below) / 2
    assert np.array_equal(~finite, np.abs(xd) >= maxv + half)
    up = _decode(((np.minimum(mag + 1, fin_max)) | sign).astype(np.uint16), dtype)
    dn = _decode(((np.maximum(mag - 1, 0)) | sign).astype(np.uint16), dtype)
    f = finite
    dr = np.abs(xd - r)[f]
    assert (dr <= np.abs(xd - up)[f]).all()
    assert (dr <= np.abs(xd - dn)[f]).all()
    tie = ((dr == np.abs(xd - up)[f]) & (up[f] != r[f])) | ((dr == np.abs(xd - dn)[f]) & (dn[f] != r[f]))
    assert ((mag[f][tie] & 1) == 0).all(), "a tie went to the odd neighbour"
    # sign is kept (including signed zero)
    assert np.array_equal(sign != 0, np.signbit(x))


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
def test_widen_exhaustive(oracle_mod, dtype):
    """All 65536 16-bit patterns widen exactly (torch and, for fp16, numpy agree)."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.widen(h, dtype)
    want = torch.from_numpy(h.view(np.int16)).view(_TDT[dtype]).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    if dtype == F16:
        assert np.array_equal(got[~nan], h.view(np.float16)[~nan].astype(np.float32))
    # a widened value narrows back to itself
    assert np.array_equal(oracle_mod.round_to(got[~nan], dtype), h[~nan])


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
def test_round_special_values(oracle_mod, dtype):
    """NaN stays NaN (any payload, either sign), infinities and signed zeros
    are kept, and the largest finite inputs overflow exactly as IEEE says."""
    nans = np.array([0x7FC00000, 0x7F800001, 0x7FFFFFFF, 0xFFC00000, 0xFF800001, 0x7FA00000],
                    dtype=np.uint32).view(np.float32)
    got = oracle_mod.round_to(nans, dtype)
    assert _nan16(got, dtype).all()
    inf_bits = 0x7F80 if dtype == BF16 else 0x7C00
    sp = np.array([np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)
    assert oracle_mod.round_to(sp, dtype).tolist() == [inf_bits, inf_bits | 0x8000, 0, 0x8000]
    big = np.array([3.4e38, 65504.0, 65519.0, 65520.0], dtype=np.float32)
    got = oracle_mod.round_to(big, dtype)
    if dtype == F16:
        assert got.tolist() == [0x7C00, 0x7BFF, 0x7BFF, 0x7C00]
