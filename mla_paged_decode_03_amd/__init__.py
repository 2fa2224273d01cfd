"""MI355X-native MLA paged decode (absorbed latent-MQA form).

The compute path lives in the HIP library ``libmla_decode.so`` (built from
``csrc/``) behind a C ABI declared in ``include/mla_decode.h``; ``api`` is a thin
ctypes binding with the same entry-point names.  Importing this package does not
load the library; ``api`` does, and fails loudly if it is missing.
"""
__all__ = ["api", "inputs"]
