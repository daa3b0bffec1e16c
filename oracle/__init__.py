"""CPU oracle for NVFP4-compressed sparse MLA decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library and
its Python binding never import, link or call it, and it imports nothing
from them: the two share no code, headers, tables or helpers.

Everything here is plain, slow and written to be checked by eye against
the format definitions and the attention formula:

* ``codec``      -- E2M1 / E4M3 element codecs, the 352-byte NVFP4 row,
                    the 576-byte FP8 row and the staged FP8 re-encoding,
                    in numpy FP64 with exact comparisons.
* ``attention``  -- sparse MLA decode over the selected rows, dense softmax
                    in FP64.
* ``indexer``    -- the sparse indexer's exact scores and per-token top-k
                    position lists.

Sources: the Prime Inference write-up ("Prime Inference: Fast, Reliable
Serving for Frontier Open Models", sections "Making room for low-latency
decode" and "A native NVFP4 sparse-MLA decode kernel") and its two
re-tellings (mo.ai.kr, section on the KV cache and data transfer;
wireai.ir, section on 4-bit caches).  Where those pages leave a step
open, the reading taken is stated at the function that takes it.
"""

from . import codec, attention, indexer  # noqa: F401
