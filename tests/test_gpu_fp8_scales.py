"""The device's FP8 quantiser at the edges of its scale rule (MI355X): rows
whose amax / 448 is exactly a power of two, just above one, far below 1,
below the smallest normal fp32 (a subnormal quotient) and in the bf16
subnormal range, plus an all-zero row, written through pa_write_kv and
compared bit for bit with the oracle's quantiser on the same bf16 rows."""
import numpy as np
import pytest

from oracle import fp8
from oracle.numerics import to_f64
from workloads.gen import bf16_bits_from_f32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BS, HKV, D = 16, 2, 128


def edge_rows(rng):
    """[BS][HKV][D] float32 rows; row (t, h) has its own magnitude."""
    amax = [448.0, 224.0, 450.0, 1.0, 3.0, 2.0 ** -100, 2.0 ** -120, 1e-36, 4e-37, 1e-38, 1e-40,
            0.0, 1e3, 1e-3, 7.0, 0.1]
    rows = np.empty((BS, HKV, D), dtype=np.float32)
    for t in range(BS):
        for h in range(HKV):
            x = rng.standard_normal(D).astype(np.float32)
            x /= np.abs(x).max()
            a = amax[(t + 5 * h) % len(amax)]
            rows[t, h] = x * np.float32(a)
            rows[t, h, (t * 7 + h) % D] = np.float32(a) * (1 if h == 0 else -1)  # the row's amax exactly
    return rows


def test_fp8_quantiser_edges_bit_exact():
    import paged_kv_cache_218_amd as pa
    from paged_kv_cache_218_amd.cache import PagedKVCache
    rng = np.random.default_rng(218)
    k_bits = bf16_bits_from_f32(edge_rows(rng))
    v_bits = bf16_bits_from_f32(edge_rows(rng) * np.float32(0.5))
    cache = PagedKVCache(4, BS, HKV, D, torch.bfloat16, 1, 2, kv_fp8=True)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    print(f"fp8 quantiser edges: {BS} tokens x {HKV} heads x {D}", flush=True)
    cache.write(0, 0, dev(k_bits), dev(v_bits))
    torch.cuda.synchronize()
    blk = int(cache.tables[0, 0])
    codes = 4 * HKV * BS * D
    kb, vb = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    k_codes = kb[:codes].reshape(4, HKV, D // 64, BS, 64)[blk]
    v_codes = vb[:codes].reshape(4, HKV, D, BS)[blk]
    k_scales = kb[codes:].view(np.float32).reshape(4, HKV, BS)[blk]
    v_scales = vb[codes:].view(np.float32).reshape(4, HKV, BS)[blk]
    for t in range(BS):
        for h in range(HKV):
            kc, ks = fp8.quantize_rows(to_f64(k_bits[t, h], "bf16").astype(np.float32))
            vc, vs = fp8.quantize_rows(to_f64(v_bits[t, h], "bf16").astype(np.float32))
            got_k = k_codes[h, :, t, :].reshape(-1)
            assert np.array_equal(got_k, kc), (t, h)
            assert np.array_equal(v_codes[h, :, t], vc), (t, h)
            assert k_scales[h, t].view(np.uint32) == np.float32(ks).view(np.uint32), (t, h, k_scales[h, t], ks)
            assert v_scales[h, t].view(np.uint32) == np.float32(vs).view(np.uint32), (t, h, v_scales[h, t], vs)
    # the edges are really there: exact powers of two, subnormal quotients, a zero row
    assert pa is not None
    assert np.any(k_scales == np.float32(1.0)) and np.any(k_scales < np.float32(2.0 ** -126))
    assert np.all(np.frexp(k_scales.astype(np.float64))[0] == 0.5)
