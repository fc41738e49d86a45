"""CPU oracle for decode attention over hybrid compressed KV caches.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: it exists so that the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` can check the HIP library against
a plain, slow, obviously correct implementation.  It shares no code with the
HIP path and imports nothing from it.

Everything here is fp64 NumPy unless a format fixes the precision (the fp8 /
fp4 / bf16 codecs take their rounding decisions in fp32, as the stored formats
demand).  Each function names the passage of the source pages it follows; the
pages are:

* "DeepSeek-V4 Serving ... vLLM" (wmrh.cn news 47220), cited as [V4-vLLM]
  with its section numbers (2.1 shared K/V and c4a/c128a compression,
  2.2 indexer KV, 2.3 sliding window, 3.1.1 single logical block size,
  3.1.2 compressor state as a sliding window, 3.1.3 unified page sizes,
  3.2.1 kernel fusion);
* "vLLM 0.7.2 ... DeepSeek-V4" (lpnh.cn news 995630), cited as [vLLM-0.7.2]
  (2.1 PagedAttention v2 block tables, 2.2 fp8_e4m3 KV, 2.3 window-aware block
  skipping, 4.3 RoPE base 1e6).

Where the pages leave a step open, the plainest reading is taken; every such
reading is listed in the design notes of the repository and restated at the
function that adopts it.

Parity status: every public function here is pinned by a ``-m "not gpu"``
test against something other than itself (closed forms, brute force, library
routines, the pages' worked numbers).  The real model's learned compressor and
indexer parameters are not available; the oracle pins the method as stated,
with synthetic parameters.
"""

from . import codecs, rope, norm, compressor, paging, indexer, attention, pipeline  # noqa: F401
