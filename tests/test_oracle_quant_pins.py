"""Pins of the write-path oracle (oracle/quant_ref.py) to facts outside itself.

The encoders are checked against torch's float8_e4m3fn cast (a library's nearest-even
rounding), the OCP E2M1 table, midpoints worked out by hand from "ties to even", an
independently written encoder (the input generator's bucketize quantiser), and closed-form
properties of the scales (the largest value of a group always lands on +-6, every value
is within half a grid step).  A swapped nibble, a wrong tie rule, a scale computed from
the wrong group or a dropped sign fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats
from _util import read_golden


def bf16(x):
    """f32 array -> bf16 bit patterns (uint16) by torch's nearest-even cast."""
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3_encode_matches_torch_cast():
    vals = formats.e4m3_decode(np.arange(0x7F))                # finite non-negative values
    mids = (vals[:-1] + vals[1:]) / 2                            # exact ties
    rng = np.random.default_rng(11)
    probe = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                            rng.uniform(0, 448, 20000), rng.uniform(0, 2 ** -5, 5000)])
    probe = probe.astype(np.float32).astype(np.float64)          # values the kernels see
    probe = np.concatenate([probe, -probe])
    want = torch.tensor(probe, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(probe), want)


def test_e4m3_encode_roundtrip_and_saturation():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(oracle.e4m3_encode(formats.e4m3_decode(codes)), codes)
    big = np.array([449.0, 463.9, 464.0, 480.0, 1e6, 1e30, 3e38, -500.0])
    assert list(oracle.e4m3_encode(big)) == [0x7E] * 7 + [0xFE]


def test_e2m1_encode_table_ties_and_saturation():
    rows = read_golden("e2m1_ocp_mx.txt")
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows], dtype=np.float32)
    assert np.array_equal(oracle.e2m1_encode(vals), codes)
    # midpoints between neighbouring magnitudes go to the code with mantissa bit 0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert list(oracle.e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.e2m1_encode(-mids)) == [8, 10, 10, 12, 12, 14, 14]
    assert list(oracle.e2m1_encode(np.array([6.5, 100.0, -7.0, 1e30, -3e38], np.float32))) == [7, 7, 15, 7, 15]
    assert list(oracle.e2m1_encode(np.array([-0.0, -1e-30, 0.2499], np.float32))) == [8, 8, 0]


def test_e2m1_encode_matches_generator_encoder():
    # synth's encoder is written independently (bucketize on the midpoints)
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.normal(0, 3, 50000),
                        np.repeat([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], 2) * np.tile([1, -1], 7)])
    v = v.astype(np.float32)
    want = synth.e2m1_encode(torch.tensor(v)).numpy()
    assert np.array_equal(oracle.e2m1_encode(v), want)


def test_pack_nibbles_order():
    assert list(oracle.quant_ref.pack_nibbles(np.array([1, 2, 15, 0]))) == [0x21, 0x0F]


def _dequant_index(codes, scale):
    return formats.e2m1_decode(formats.unpack_nibbles(codes)) * scale[:, None]


def _half_step(mag):
    """Half the E2M1 grid spacing around a magnitude (in units of the scale)."""
    return np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0))


def test_quantize_index_entry_properties():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, (300, 128)) * rng.uniform(1e-3, 1e3, (300, 1))
    bits = bf16(x)
    xv = formats.bf16_decode(bits)
    codes, scale = oracle.quantize_index_entry(bits)
    amax = np.abs(xv).max(axis=1)
    assert np.array_equal(scale, (amax.astype(np.float32) / np.float32(6)).astype(np.float32))
    c = formats.unpack_nibbles(codes)
    am = np.abs(xv).argmax(axis=1)
    assert np.all((c[np.arange(300), am] & 7) == 7)                # the largest value is +-6
    assert np.array_equal(c >> 3, np.signbit(xv).astype(np.uint8))  # sign bits
    deq = _dequant_index(codes, scale.astype(np.float64))
    assert np.all(np.abs(deq - xv) <= _half_step(np.abs(xv) / scale[:, None]) * scale[:, None] * (1 + 1e-6))


def test_quantize_main_entry_properties():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1, (200, 512)) * rng.uniform(1e-2, 1e2, (200, 32)).repeat(16, axis=1)
    bits = bf16(x)
    xv = formats.bf16_decode(bits).reshape(200, 32, 16)
    codes, sbytes = oracle.quantize_main_entry(bits)
    amax = np.abs(xv).max(axis=2)
    want_s = torch.tensor((amax.astype(np.float32) / np.float32(6))).to(torch.float8_e4m3fn)
    assert np.array_equal(sbytes, want_s.view(torch.uint8).numpy())  # no zero codes at these sizes
    s = formats.e4m3_decode(sbytes)
    c = formats.unpack_nibbles(codes).reshape(200, 32, 16)
    am = np.abs(xv).argmax(axis=2)
    top = np.take_along_axis(c, am[..., None], axis=2)[..., 0]
    assert np.all((top & 7) == 7)
    deq = formats.e2m1_decode(c) * s[..., None]
    ratio = np.abs(xv) / s[..., None]
    assert np.all(np.abs(deq - xv) <= np.maximum(_half_step(ratio), (ratio - 6) * (ratio > 6)) * s[..., None] * (1 + 1e-6))


def test_quantizers_match_generator_quantizers():
    # the input generator's quantisers are an independently written reading of the same
    # encoders; on bf16-representable N(0,1) inputs they must agree byte for byte
    g = torch.Generator().manual_seed(3)
    x_idx = torch.randn(500, 128, generator=g).to(torch.bfloat16).float()
    x_kv = torch.randn(500, 512, generator=g).to(torch.bfloat16).float()
    sc, ss, _ = synth.quantize_index_keys(x_idx)
    kc, ks, _ = synth.quantize_main_kv(x_kv)
    oc, os_ = oracle.quantize_index_entry(x_idx.to(torch.bfloat16).view(torch.int16).numpy())
    mc, ms = oracle.quantize_main_entry(x_kv.to(torch.bfloat16).view(torch.int16).numpy())
    assert np.array_equal(oc, sc.numpy()) and np.array_equal(os_, ss.numpy())
    assert np.array_equal(mc, kc.numpy()) and np.array_equal(ms, ks.numpy())


def test_degenerate_scales():
    # all-zero rows: indexer scale 1, main scales code 1 (2^-9), codes keep the sign
    z = np.zeros((1, 128), np.float32)
    z[0, 3] = -0.0
    codes, scale = oracle.quantize_index_entry(bf16(z))
    assert scale[0] == 1.0 and codes[0, 1] == 0x80 and np.count_nonzero(codes) == 1
    codes, sb = oracle.quantize_main_entry(bf16(np.zeros((1, 512))))
    assert np.all(sb == 1) and np.all(codes == 0)
    # a group whose amax/6 is far above 448 saturates its scale and its codes
    x = np.ones((1, 512), np.float32)
    x[0, :16] = 3e4
    codes, sb = oracle.quantize_main_entry(bf16(x))
    assert sb[0, 0] == 0x7E and np.all(formats.unpack_nibbles(codes)[0, :16] == 7)


def test_kv_append_scatter_and_swa_ring():
    rng = np.random.default_rng(2)
    cap = 50
    planes = (np.zeros((cap, 64), np.uint8), np.zeros(cap, np.float32),
              np.zeros((cap, 256), np.uint8), np.zeros((cap, 32), np.uint8))
    xi, xk = bf16(rng.normal(size=(6, 128))), bf16(rng.normal(size=(6, 512)))
    dst = np.array([7, 49, -1, 0, 50, 20])
    ic, isc, kc, ksc, bad = oracle.kv_append(*planes, xi, xk, dst)
    assert bad == 2
    for i, d in enumerate(dst):
        if 0 <= d < cap:
            a, b = oracle.quantize_index_entry(xi[i:i + 1])
            c, e = oracle.quantize_main_entry(xk[i:i + 1])
            assert np.array_equal(ic[d], a[0]) and isc[d] == b[0]
            assert np.array_equal(kc[d], c[0]) and np.array_equal(ksc[d], e[0])
    untouched = np.setdiff1d(np.arange(cap), dst)
    assert not ic[untouched].any() and not kc[untouched].any() and not isc[untouched].any()
    # ring: after positions 0..200 of one sequence the slots hold positions 73..200
    swa = np.zeros((1, 128, 512), np.uint8)
    rows = bf16(rng.normal(size=(201, 512)))
    for p in range(201):
        swa = oracle.swa_append(swa, rows[p:p + 1], np.array([p]))
    for p in range(73, 201):
        assert np.array_equal(swa[0, p % 128], oracle.swa_encode(rows[p]))
    want = torch.tensor(formats.bf16_decode(rows[200]), dtype=torch.float32).to(torch.float8_e4m3fn)
    assert np.array_equal(swa[0, 200 % 128], want.view(torch.uint8).numpy())
