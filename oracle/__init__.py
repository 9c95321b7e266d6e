"""Float64 CPU oracle for BeaconKV's KV-cache eviction step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct definition that the HIP library is checked against.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it;
the library and its Python binding never do, and this package imports
nothing from them.  The two sides share only the seeded input generators
(the ``synth`` package), which hold none of the method's arithmetic.

Sources (cited by page title and section throughout):

* "BeaconKV: Key-Value Cache Compression Guided by Beacon Queries for
  Efficient Large Reasoning Model Inference" -- the paper's own text
  (signal-papers reader page), cited as *paper text* with its section
  (§2.1, §2.2, §4.2, §4.3, §5.1, App. D.1 = Algorithm 1, App. D.2 =
  Algorithm 2).  Its displayed equations were lost in extraction.
* "BeaconKV：信标查询引导的大型推理模型KV缓存压缩" -- structured summary
  (paper.rainbus.top), cited as *summary*; its section "方法步骤详情"
  restates Algorithm 2 as steps (1)-(6) with the formulas.
* the jaehun.me review of the same paper, cited as *review*, with its
  section headings (§4.2, §4.3, "작동 원리 ①").

Floating point is float64 throughout except the one rounding the method's
precision contract names: the RoPE-aligned observation queries are rounded
to bfloat16 (via float32, round-to-nearest-even both times) before they
meet the keys, because the cache holds bfloat16 and the kernel feeds its
matrix cores bfloat16 operands.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, brute force, library routines, the pages'
worked example).  One composite is NOT separately pinned:

* ``evict.evict_unit`` as a whole -- parity unpinned beyond its pinned
  parts (RoPE, bf16 rounding, score, select, compact, FPS): the pages print
  no worked eviction with numbers.
"""

from . import bf16, rope, fps, score, select, compact, evict, stream, decode  # noqa: F401
