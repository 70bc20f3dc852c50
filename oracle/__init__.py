"""CPU fp64 oracle for tiled attention over a grouped-quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU library never imports, links or calls it, and it shares no code with the
GPU library: it is written from the method's definition, not from the kernels.

What it computes (every function cites the passage it follows):

* ``quant``     - grouped asymmetric quantisation of K/V (group of 32 adjacent
                  channels of one token, one fp16 scale and one zero-point per
                  group), dequantisation, and the byte layouts of the cache.
* ``exact``     - the same quantiser for single groups in exact rational
                  arithmetic, and a division-free brute-force code search;
                  both serve as pins of ``quant``.
* ``attention`` - causal scaled-dot-product attention with GQA head sharing,
                  KV-tile skip mask and ragged lengths, as whole rows in fp64.
* ``brute``     - the same attention as explicit pure-Python loops on tiny
                  shapes (``math.exp`` / ``math.fsum``), a pin of ``attention``.

Pins of every function are listed in each module header; none of them is
"parity unpinned".
"""
