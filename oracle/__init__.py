"""CPU oracle for decode attention over a KIVI / WindowQuant low-bit KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call anything here; the product
package never does, and this package imports nothing from it.  It shares no
code, table or helper with the HIP path: the pack layout is implemented here a
second time, independently, from its written definition in ``include/kvq.h``.

Precision: the quantizer runs in IEEE fp32 with round-half-even, on fp16
inputs, exactly as the written specification fixes it (so that codes, scales
and zero-points can be compared bit for bit); dequantization and attention
run in float64.

Modules
-------
quant      group quantizer (KIVI quick-read formula; WindowQuant Sec. 3.3.3)
pack       byte layout of codes and (scale, zero) pairs (defined by kvq.h)
kivi       KIVI prefill / decoding state machine (KIVI note, Algorithm 1)
windows    WindowQuant window reorder and per-window quantization (Sec. 3.3)
search     WindowQuant window-level quantization search (Sec. 3.2), float64
attention  single-query softmax attention over the cache, float64
pq         PQCache decode-time PQ search: approximate scores and Top-k, float64
vq         decode attention over a vector-quantized (codebook) cache, float64

Parity pins: every function is checked by ``tests/test_oracle_*.py`` against
closed forms, hand-derived fixtures in ``tests/golden/``, brute force on tiny
inputs and a library routine (torch scaled_dot_product_attention, CPU fp64).
The byte layout in ``pack`` is pinned by the header's written definition and
hand-derived bytes, not by the pages (the pages define no layout).
"""
from . import quant, pack, kivi, windows, search, attention, pq, vq  # noqa: F401
