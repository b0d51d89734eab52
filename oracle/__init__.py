"""CPU oracle for paged KV-cache decode.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product path: the two share no code, tables or constants.

Everything here is plain numpy in float64 (integers for allocator state,
uint8 codes for fp8, int8 codes for int8).  Each function cites the web page and section it
follows:

* ``allocator.OracleAllocator``  block manager: FIFO free queue, reference
  counts, per-sequence block tables, copy-on-write on append.
* ``kvstore.OracleKVStore``      the block-pooled K/V store and the
  reshape-and-cache write (fp16 copy, fp8 e4m3 or int8 scale + zero point
  quantise).
* ``attention.decode``           exact softmax(q K^T / sqrt(d)) V per query head
  over the K/V rebuilt contiguously from each block table.
* ``attention.multi_token``      causal attention for several new query tokens
  per sequence (prefill chunks mixed with decode tokens) through the tables.
* ``attention.split_partials`` / ``attention.lse_merge``  per-chunk
  (max, sum, normalised output) and their log-sum-exp merge.
* ``fp8``                        OCP E4M3FN decode / saturating RNE encode.
* ``int8``                       affine int8 codes: (c - z) * s, RNE encode
  with saturation.
* ``formulas``                   the pages' closed forms (KV bytes, waste bound,
  prefix savings, ...).

Pins (tests/test_oracle_*.py, all ``-m "not gpu"``): page-printed numbers under
tests/golden/, torch's float8_e4m3fn tables, torch's per-tensor qint8
quantiser, torch scaled_dot_product_attention
in float64 on contiguous K/V, closed-form special cases, the LSE identity and
the allocator invariants.  No function in this package is "parity unpinned".
"""
