"""CPU fp64 oracle for MLA paged decode (absorbed, latent-MQA form).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The library in ``mla_paged_decode_03_amd`` never calls it, and this
package imports nothing from the library (it shares no kernels, helpers,
tables or constants with it).  Inputs come from the seeded generators in
``mla_paged_decode_03_amd.inputs`` (which hold no attention arithmetic) or from
the tests themselves.

What it computes is the plain definition, written out in float64 with no
tiling and no reordering beyond what the definitions state:

* ``formats``   bit-exact decoding of bfloat16 and OCP float8 e4m3fn.
* ``attention`` W_UK absorption, latent attention over a paged cache (with the
  causal window of multi-token verify), W_UV up-projection, the LSE merge, and
  the compute-friendly MHA path used to cross-check the absorbed one.
* ``bmm8``      the fp8 W_UK / W_UV batched GEMMs: per-tensor weight quantisation,
  per-token group-of-128 activation quantisation, the scaled product.
* ``plan``      an independent re-derivation of the split-KV work plan and of
  the page -> physical row expansion, for bit-exact comparison.

Sources are the four pages on vLLM's MLA backends: the module docstring of
``vllm/v1/attention/backends/mla/common.py`` (sections "Compute Friendly
Approach", "Data-Movement Friendly Approach", "Chunked Prefill"), the layer
``vllm.model_executor.layers.attention.mla_attention`` (``forward_impl``,
``process_weights_after_loading``, ``_v_up_proj``), the ROCm backend
``vllm.v1.attention.backends.mla.rocm_aiter_mla`` (``AiterMLAImpl.forward_mqa``,
``AiterMLAHelper``, ``AiterMLAMetadataBuilder._build_decode``) and the generic
``vllm.v1.attention.backends.flashinfer`` backend (LSE base conventions).

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (brute force, closed forms, the two-path
equivalence, merge exactness, head independence, causal flattening, paging
invariance, format tables against torch's casts).  The split plan is a rule of
this library, not of the pages; it is pinned by its invariants.
"""
