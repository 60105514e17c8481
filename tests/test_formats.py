"""Pins for the oracle's format decoders (exhaustive tables) and the pages' sizes."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import generator as gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _same(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_matches_ocp_value_table():
    # OCP MX v1.0 lists the E2M1 magnitudes for codes 0..7 as 0, 0.5, 1, 1.5, 2, 3, 4, 6;
    # codes 8..15 are their negatives.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    table = mags + [-m for m in mags]
    for c in range(16):
        assert _same(oracle.e2m1_value(c), table[c]), c
        assert _same(float(oracle.E2M1[c]), table[c]), c


def test_e8m0_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().tolist()
    for u in range(256):
        assert _same(oracle.e8m0_value(u), ref[u]), u
        assert _same(float(oracle.E8M0[u]), ref[u]), u
    assert oracle.E8M0[127] == 1.0 and oracle.E8M0[0] == 2.0 ** -127 and math.isnan(oracle.E8M0[255])


def test_e4m3fn_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().tolist()
    for c in range(256):
        assert _same(oracle.e4m3fn_value(c), ref[c]), c
    assert oracle.e4m3fn_value(0x7E) == 448.0


def test_bf16_matches_torch_decoder():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_value(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_fp4_times_scale_exhaustive_exact():
    # Every (E2M1 code, E8M0 code) product against exact rationals: 16 x 255 cases.
    for u in range(255):
        sc = Fraction(2) ** (u - 127)
        for c in range(16):
            mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
                   Fraction(4), Fraction(6)][c & 7]
            v = (-mag if c & 8 else mag) * sc
            rec = np.zeros((1, 68), dtype=np.uint8)
            rec[0, 0] = c
            rec[0, 64] = u
            got = oracle.dequant_idx(rec)[0, 0]
            assert Fraction(got) == v, (c, u)


def test_record_layout_golden():
    g = json.load(open(os.path.join(GOLD, "fp4_fp8_records.json")))
    idx = np.zeros((1, 68), dtype=np.uint8)
    for k, v in g["indexer_record"]["bytes_set"].items():
        idx[0, int(k)] = v
    exp = np.zeros(128)
    for k, v in g["indexer_record"]["expected_nonzero"].items():
        exp[int(k)] = v
    assert np.array_equal(oracle.dequant_idx(idx)[0], exp)

    main = np.zeros((1, 288), dtype=np.uint8)
    main[0, 256:] = g["main_record"]["other_scale_byte"]
    for k, v in g["main_record"]["bytes_set"].items():
        main[0, int(k)] = v
    exp = np.zeros(512)
    for k, v in g["main_record"]["expected_nonzero"].items():
        exp[int(k)] = v
    assert np.array_equal(oracle.dequant_main(main)[0], exp)

    t = g["e4m3_tokens"]
    codes = np.array([t["codes"]], dtype=np.uint8)
    got = oracle.dequant_swa(np.pad(codes, ((0, 0), (0, 512 - codes.shape[1]))), np.array([t["scale"]],
                             dtype=np.float32))[0, :codes.shape[1]]
    for a, b in zip(got, t["expected"]):
        assert _same(float(a), float(b)), (a, b)


def test_page_sizes_identity():
    g = json.load(open(os.path.join(GOLD, "page_sizes.json")))
    # The entry sizes follow from the layouts ...
    assert oracle.MAIN_BYTES == 512 // 2 + 512 // 16 == g["main_entry_bytes"]
    assert oracle.IDX_BYTES == 128 // 2 + 128 // 32 == g["indexer_entry_bytes"]
    assert gen.MAIN_BYTES == g["main_entry_bytes"] and gen.IDX_BYTES == g["indexer_entry_bytes"]
    # ... and reproduce the pages' 890 logical bytes per original token: three caches
    # pooled two tokens per entry plus one cache with one entry per token.
    per_entry = g["main_entry_bytes"] + g["indexer_entry_bytes"]
    pooled = g["pooled_caches"] * Fraction(per_entry, g["pool_stride"])
    unpooled = (g["global_caches"] - g["pooled_caches"]) * per_entry
    assert pooled + unpooled == g["logical_bytes_per_token"]


def test_generator_encoders_roundtrip_through_oracle():
    # Values already on the FP4 grid survive encode -> oracle decode exactly, which pins
    # the encoder and the decoder to the same layout (nibble order, scale position).
    rng = np.random.default_rng(7)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    for dim, block, dec in ((512, 16, oracle.dequant_main), (128, 32, oracle.dequant_idx)):
        n = 64
        v = mags[rng.integers(0, 8, size=(n, dim))] * rng.choice([-1, 1], size=(n, dim))
        v[:, ::block] = 6.0                       # make each block's amax exactly 6
        e = rng.integers(-20, 20, size=(n, dim // block))
        x = (v * np.repeat(np.ldexp(1.0, e), block, axis=1)).astype(np.float32)
        rec = gen.encode_fp4_blocks(x, block)
        assert np.array_equal(dec(rec), x.astype(np.float64))
    # E4M3: codes decoded by the oracle times the scale reproduce inputs already on the grid.
    grid = oracle.E4M3[np.isfinite(oracle.E4M3)]
    x = rng.choice(grid, size=(8, 512)).astype(np.float32)
    x[:, 0] = 448.0
    codes, scale = gen.encode_e4m3_tokens(x)
    assert np.all(scale == 1.0)
    assert np.array_equal(oracle.dequant_swa(codes, scale), x.astype(np.float64))


@pytest.mark.parametrize("block", [16, 32])
def test_generator_fp4_rounding_is_nearest(block):
    # Encoded values are a nearest grid point of x / 2**e for the block's shared exponent.
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 128 if block == 32 else 512)).astype(np.float32)
    rec = gen.encode_fp4_blocks(x, block)
    dec = oracle.dequant_idx(rec) if block == 32 else oracle.dequant_main(rec)
    d = x.shape[1]
    scale = np.repeat(oracle.E8M0[rec[:, d // 2:]], block, axis=1)
    y = x / scale
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    best = np.abs(np.abs(y)[..., None] - grid).min(axis=-1)
    got = np.abs(np.abs(dec / scale) - np.abs(y))
    assert np.all(got <= best + 1e-12)
