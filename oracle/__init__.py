"""CPU oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  Only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The product path (``paged_kv_attention_29_amd``) never imports, calls or
links anything here, and this package imports nothing from the product.

Everything is computed in float64 with plain PyTorch CPU ops; fp16/bf16
inputs are widened exactly before any arithmetic.  Parity pins (tests under
``tests/`` marked "not gpu") tie every function to the pages and to
mathematics independent of this code:

* ``scatter``        — bit-exact against numpy fancy-index assignment.
* ``attend``         — pure-Python brute force on tiny shapes; torch SDPA
                        (float64) with hand-built masks; closed forms.
* ``decode_splits``  — split-then-merge equals the unsplit result.
* ``merge``          — closed forms (identical states, -inf parts).
* ``cascade``        — equals plain causal ``attend`` (itself pinned above)
                        on batches that share a block-aligned prefix.
* ``fp8``            — e4m3 code table and quantiser against torch's
                        float8_e4m3fn type, closed-form codes, the rounding
                        error bound.  An fp8 cache is attended by passing
                        its dequantised float64 copy to ``attend``; an fp8
                        query (``scaled_fp8_quant``) likewise through
                        ``dequantize_query``.

Readings the pages leave open (softcap/ALiBi order, ALiBi slope index,
window edge) are fixed by the readings documented with each function; they
are locked by the brute-force tests but no page value pins them
("parity unpinned by the pages" for those three points only).
"""
from .paged_attention import (
    scatter,
    gather_sequence,
    attend,
    decode,
    split_bounds,
    decode_splits,
    merge,
    cascade,
)
from . import fp8

__all__ = [
    "scatter",
    "gather_sequence",
    "attend",
    "decode",
    "split_bounds",
    "decode_splits",
    "merge",
    "cascade",
    "fp8",
]
