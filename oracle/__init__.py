"""Plain, slow CPU oracle of PackKV's compressed KV cache and its two decode GEMVs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP library never calls it, and the two share no code: the only
module both sides use is ``kvsynth`` (seeded random inputs, no arithmetic of
the method).

Source: "PackKV: Reducing KV Cache Memory Footprint through LLM-Aware Lossy
Compression" (arXiv 2512.24449): its abstract, its TL;DR and the captions of
its Figures 1-5, plus the visual-explainer page on the same paper.  The pages
give the method's steps in prose only (quantise -> reorder tokens -> lossless
channel-direction bit-packing -> decompression fused into the attention
matrix-vector products); every point they leave open is fixed by a reading
that is named where it is used.  All floating point here is fp64 (exact where
noted); integer work is exact.

Modules
-------
fp16bits   fp16 bit helpers, independent of the GPU code
quant      asymmetric min-max quantiser (K per channel per block, V per token)
perm       greedy token grouping inside a block (the "rearrange" step)
record     run widths, header and bit-packed record bytes (encoder)
unpack     record bytes -> quantised ints (a second, independent decoder)
attention  dequantisation, K GEMV, softmax, V GEMV (plain fp64 definitions)
cr         exact compression-ratio accounting
stream     per-stream cache: bulk compress, single-token append, arena layout
"""

from .config import Config  # noqa: F401
from . import fp16bits, quant, perm, record, unpack, attention, cr, stream  # noqa: F401
