"""Query-union sparse-attention prefill over a paged FP8 KV cache, for MI355X.

* ``query_union_paged_amd.pageweaver`` -- the ctypes binding of
  ``libpageweaver.so`` (pw_group, pw_union_attention, pw_dense_union_ref).
  Importing it raises ImportError when the library is not built.
* ``query_union_paged_amd.synth`` -- the seeded synthetic inputs.
* ``query_union_paged_amd.build`` -- hipcc build of the library (gfx950).
"""
