"""CPU oracle for the CSA2 decode hot path (FP4 main-KV cache + sparse indexer).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, tables or helpers); the two meet only through
the seeded input generators, which hold none of the method's arithmetic.

The oracle is plain NumPy, float64 for every floating-point step unless a
decision (a quantised code, a rounded scale) has to be taken in the precision
the kernel takes it in, in which case that is stated at the step.  It is slow
and written to be checked by eye against the pages.

Citation keys used in this package (the pages are web articles; sections are
the pages' own headings):

* ``[0539edu §N]``  -- http://www.0539edu.com/news/5732216/ , section N
  (§1 the three multiplicative compression dimensions, §3 the inference
  configuration in JSON/TOML form and the explanation that follows it).
* ``[nxbn §N.M]``   -- http://m.nxbn.cn/news/78290 , section N.M
  (§2.1 the worked KV-size example, §3.1 FP4 E2M1, §4.2 the main key
  compressor).
* ``[ai-feeds Method]`` -- https://ai-feeds.com/i/paper/2609.19969 , the
  "Method" and "Key findings" sections.
* ``[daiw table X]`` -- https://daiw.net/manual/deepseek-v4-flash/million-token-cost ,
  the chapter "百万 token 的成本账": its "four factors" table (cache-size
  factors), its "four generations" table (per-token global KV) and the
  "decode reads" section.

Parity status: every public function here is exercised by a pin in
``tests/test_oracle_*.py`` -- closed forms, exhaustive format tables, an
independent library routine or brute force.  ``tests/test_oracle_coverage.py``
checks that each of them is called by at least one of those pins, so a helper
added without a pin fails the CPU suite; none is "parity unpinned".
"""

from . import formats, csa2, accounting  # noqa: F401
