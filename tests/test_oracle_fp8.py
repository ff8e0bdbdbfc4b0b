"""Pins of the FP8 (OCP E4M3) codec and the fp8-pool oracle (CPU)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import fp8
from oracle.build import build_pool
from oracle.numerics import to_f64
from tests.test_oracle_pins import torch_sdpa_seq


def torch_codes():
    return torch.arange(0, 256, dtype=torch.uint8).view(torch.float8_e4m3fn)


def test_decode_table_matches_torch_float8_e4m3fn():
    ref = torch_codes().double().numpy()
    ours = fp8.e4m3_decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~np.isnan(ref)], ours[~np.isnan(ours)])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(7)
    vals = torch_codes().double().numpy()
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([
        np.clip(rng.standard_normal(50000).astype(np.float32) * 60, -448, 448),
        rng.standard_normal(5000).astype(np.float32) * 2e-3,     # subnormal range and underflow
        mids, -mids, fin.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0]),
        np.float32([448.00003, -448.00003, 455.9, 456.0, 460.0, 464.0, -464.0]),   # round down to 448
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_quantize_rows_properties():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((300, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, (300, 1)).astype(np.float32)
    x[5] = 0.0
    codes, scales = fp8.quantize_rows(x)
    assert codes[5].max() == 0 and scales[5] == 1.0
    # every scale is a power of two, the smallest one with amax / scale <= 448
    frac, _ = np.frexp(scales.astype(np.float64))
    assert (frac == 0.5).all()
    live = np.arange(300) != 5
    amax = np.abs(x).max(axis=1).astype(np.float64)
    ratio = amax[live] / scales[live]
    assert (ratio <= 448.0 * (1 + 2.0 ** -23)).all() and (ratio > 224.0 * (1 - 2.0 ** -23)).all()
    # so the largest magnitude of each row takes one of the codes for (224, 448]
    amax_idx = np.abs(x).argmax(axis=1)
    top = codes[np.arange(300), amax_idx] & 0x7F
    assert ((top[live] >= 0x76) & (top[live] <= 0x7E)).all()
    deq = fp8.dequantize(codes, scales)
    # within half a unit in the last place: 2^-4 relative for normals, 2^-10 * scale near zero
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert (np.abs(deq - x) <= bound * (1 + 1e-12)).all()
    assert not np.array_equal(deq, x)


def test_pow2_ceil_is_the_smallest_power_of_two_not_below():
    rng = np.random.default_rng(9)
    # normal and subnormal fp32 values, exact powers of two and their neighbours
    s = np.concatenate([
        (rng.uniform(0.5, 1.0, 4000) * 2.0 ** rng.integers(-140, 100, 4000)).astype(np.float32),
        np.float32(2.0) ** np.arange(-149, 100, dtype=np.float64).astype(np.float32),
        np.nextafter(np.float32(2.0) ** np.arange(-148, 100).astype(np.float32), np.float32(np.inf)),
        np.nextafter(np.float32(2.0) ** np.arange(-148, 100).astype(np.float32), np.float32(0)),
    ]).astype(np.float32)
    s = s[s > 0]
    got = fp8.pow2_ceil(s).astype(np.float64)
    # brute force: the first of 2^-149, 2^-148, ... that is >= s
    powers = 2.0 ** np.arange(-149, 128, dtype=np.float64)
    want = powers[np.searchsorted(powers, s.astype(np.float64), side="left")]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name,kw", [
    ("llama3_70b_decode_fp8", dict(batch=2, len_const=300)),
    ("llama3_70b_decode_fp8", dict(batch=3, len_const=0, lens=(1, 33, 64))),
])
def test_fp8_pool_attention_vs_torch_sdpa(name, kw):
    w = workloads.generate(workloads.config(name, **kw))
    cfg = w.cfg
    pool, _, tables, _ = build_pool(w)
    got = oatt.attention_paged(w.q_all(), pool, tables, w.lens, cfg.q_len, cfg.scale)
    for b in range(cfg.batch):
        k, v = w.logical_kv(b)
        # dequantise with torch's own float8 decode and the oracle-independent scales
        kq = torch.from_numpy(to_f64(k, "bf16").astype(np.float32))
        vq = torch.from_numpy(to_f64(v, "bf16").astype(np.float32))
        # scales: the power of two 2^ceil(log2(amax / 448)), the quotient in fp32, the log in fp64
        ks = torch.exp2(torch.ceil(torch.log2((kq.abs().amax(-1, keepdim=True) / 448.0).double()))).float()
        vs = torch.exp2(torch.ceil(torch.log2((vq.abs().amax(-1, keepdim=True) / 448.0).double()))).float()
        kd = (kq / ks).to(torch.float8_e4m3fn).double() * ks.double()
        vd = (vq / vs).to(torch.float8_e4m3fn).double() * vs.double()
        ref = torch_sdpa_seq(w.seqs[b].q, kd.numpy(), vd.numpy(), cfg.q_len, cfg.group, cfg.scale, "bf16",
                             kv_dtype="f64")
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)


def test_fp8_pool_bytes_and_scales_layout():
    w = workloads.generate(workloads.config("llama3_70b_decode_fp8", batch=2, len_const=70))
    pool, _, tables, _ = build_pool(w)
    k, v = w.logical_kv(1)
    t = 37
    blk, off = tables[1][t // 32], t % 32
    kc, ks = fp8.quantize_rows(to_f64(k[t], "bf16").astype(np.float32))
    assert np.array_equal(pool.k[blk, :, :, off, :].reshape(8, 128), kc)
    assert np.array_equal(pool.k_scale[blk, :, off], ks)
    vc, vs = fp8.quantize_rows(to_f64(v[t], "bf16").astype(np.float32))
    assert np.array_equal(pool.v[blk, :, :, off], vc) and np.array_equal(pool.v_scale[blk, :, off], vs)
    # unwritten slots (tokens 70..95 of the last block) keep the NaN code and NaN scales
    last = tables[1][70 // 32]
    assert (pool.k[last, :, :, 70 % 32:, :] == 0x7F).all() and np.isnan(pool.k_scale[last, :, 70 % 32:]).all()
