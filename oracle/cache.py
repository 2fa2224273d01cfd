"""Write of new latent rows into the paged cache (oracle; test infrastructure only).

Source: vLLM ``v1/attention/backends/mla/common.py``, ``MLACommonImpl`` forward: "write
the latent and rope to kv cache" with ``concat_and_cache_mla(k_c_normed, k_pe, kv_cache,
slot_mapping, kv_cache_dtype, scale=k_scale)``; the ``MLAAttention`` layer of the
mla_attention page does the same through ``do_kv_cache_update``.

Token i with slot s = slot_mapping[i] writes cache row (s // page_size, s % page_size) =
[kv_c[i] | k_pe[i]].  An fp8 cache stores ``quant.quantize(x, k_scale)`` (the static
per-tensor quantisation, read as for the query).  Readings (the pages do not print the
kernel): a negative slot marks a padding token and writes nothing; a slot past the cache
is skipped too.
"""
import numpy as np

from oracle import quant as Q


def concat_and_cache(kv_c_bits, k_pe_bits, slot_mapping, cache, kv_dtype: str, k_scale: float = 1.0):
    """Returns a copy of ``cache`` ([num_pages, page_size, 576] uint16 bf16 bits or uint8
    e4m3fn codes) with the rows of the tokens written."""
    out = np.array(cache, copy=True)
    num_pages, ps, _ = out.shape
    kv_c_bits = np.asarray(kv_c_bits, np.uint16)
    k_pe_bits = np.asarray(k_pe_bits, np.uint16)
    for i, s in enumerate(np.asarray(slot_mapping, np.int64)):
        if s < 0 or s >= num_pages * ps:
            continue
        row = np.concatenate([kv_c_bits[i], k_pe_bits[i]])
        if kv_dtype == "bf16":
            out[s // ps, s % ps] = row
        elif kv_dtype == "fp8":
            x = (row.astype(np.uint32) << np.uint32(16)).view(np.float32)
            out[s // ps, s % ps] = Q.quantize(x, k_scale)
        else:
            raise ValueError(kv_dtype)
    return out
