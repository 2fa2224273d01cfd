"""Pins of the oracle's cache write (CPU only)."""
import numpy as np

from oracle import cache as CW
from oracle import formats as F
from oracle import plan as PL


def _rows(rng, T):
    kv = (rng.standard_normal((T, 512)) * 2).astype(np.float32)
    pe = (rng.standard_normal((T, 64)) * 2).astype(np.float32)
    bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    return bits(kv), bits(pe)


def test_bf16_rows_come_back_through_the_page_expansion():
    rng = np.random.default_rng(0)
    ps, pages, L = 16, 8, 70
    bt = rng.permutation(pages)[:5].astype(np.int32)           # one request, 5 pages
    kv, pe = _rows(rng, L)
    slots = np.array([bt[j // ps] * ps + j % ps for j in range(L)], np.int64)
    cache = np.zeros((pages, ps, 576), np.uint16)
    out = CW.concat_and_cache(kv, pe, slots, cache, "bf16")
    rows = PL.gather_rows_all([bt], [L], ps)
    flat = out.reshape(-1, 576)
    assert np.array_equal(flat[rows, :512], kv) and np.array_equal(flat[rows, 512:], pe)
    # every other row is untouched
    mask = np.ones(len(flat), bool)
    mask[rows] = False
    assert not flat[mask].any()


def test_padding_and_out_of_range_slots_write_nothing():
    rng = np.random.default_rng(1)
    kv, pe = _rows(rng, 4)
    cache = np.full((2, 4, 576), 7, np.uint16)
    out = CW.concat_and_cache(kv, pe, np.array([-1, 8, 100, 3], np.int64), cache, "bf16")
    assert np.array_equal(out[0, 3], np.concatenate([kv[3], pe[3]]))
    out[0, 3] = 7
    assert (out == 7).all()


def test_fp8_rows_are_the_quantised_values():
    rng = np.random.default_rng(2)
    kv, pe = _rows(rng, 6)
    k_scale = 0.0137
    cache = np.zeros((3, 2, 576), np.uint8)
    out = CW.concat_and_cache(kv, pe, np.arange(6, dtype=np.int64)[::-1], cache, "fp8", k_scale)
    for i in range(6):
        s = 5 - i
        x = (np.concatenate([kv[i], pe[i]]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        v = F.E4M3FN_TABLE[out[s // 2, s % 2]] * k_scale
        inside = np.abs(x) < 440 * k_scale
        e = np.floor(np.log2(np.maximum(np.abs(v[inside] / k_scale), 2.0 ** -6)))
        step = 2.0 ** (e - 3) * k_scale
        assert np.all(np.abs(v[inside] - x[inside]) <= step / 2 * (1 + 1e-6) + 1e-9)
