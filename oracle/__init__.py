"""Plain, slow, float64 CPU oracle for the Cactus Quants (CQ) matrix product.

TEST INFRASTRUCTURE ONLY.  The only code allowed to import, call or execute
anything in this package is ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path
(``hadamard_rotated_codebook_amd``: the HIP kernels, the C-ABI library and its
Python binding) never imports it, and this package never imports the product
path: the two share no code, no tables and no constant generators.

Every function follows a passage of the public pages that describe the
format.  Citations use these page names:

* *cact-format post*  -- Cactus blog, "cact-format" (sections "Five regions",
  "Cactus Quants", "How the kernel reads it", "Versions").
* *needle.js tutorial* -- "The .cact archive and Cactus Quants" (sections
  "Shared codebooks", "Anatomy of a CQ matrix", "2-bit", "4-bit", "3-bit",
  "Reconstructing one group", "Keep the quantized views").
* *porting post* -- Cactus blog, "Porting Needle 3" (section 1, "Test against
  float32 with quantisation simulated").
* *OpenNeedle reference* -- OpenNeedle ``docs/reference.md`` (written in
  Chinese, no headings; cited by topic: "CQ quantisation steps", "codebook
  generation", "file layout", "byte accounting table", "idempotence note",
  "rotated-activation identity", "Cactus 2-bit kernel", "activation
  fake-quant note", "numeric-paths note", "attention note").

Readings taken where the pages are silent or garbled are stated next to the
code they affect (each is also listed in the design notes of the repository).

Parity status of each public function is pinned by ``tests/test_oracle_*.py``
(run with ``-m "not gpu"``); nothing here is "parity unpinned" except the
official CQ3/CQ4 codebook values, which no page prints (the codebook is an
input of every product call, so this affects no parity claim).
"""

from .cq import *  # noqa: F401,F403
from .w2a8 import *  # noqa: F401,F403
from .kv import *  # noqa: F401,F403
from . import cq as _cq, w2a8 as _w2a8, kv as _kv

__all__ = list(_cq.__all__) + list(_w2a8.__all__) + list(_kv.__all__)
