"""CPU oracle for block-quantized batch-1 decode GEMV.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
product path (the C-ABI library and its Python binding) never imports,
links or runs this package, and this package never imports the product.

The oracle is a plain, slow, obviously-correct restatement of what the pages
define, in numpy:

* ``formats``   -- the block formats (Q8_0, Q4_0, Q4_1, Q4_K on the handbook
                   page; Q2_K, ternary-in-2-bit and 1-bit from the low-bit
                   pages), their quantizers, dequantizers and the byte layout.
* ``page_sample`` -- the handbook page's weight sample (the torch draw its
                   error table is printed for); the table is reproduced by
                   the quantizers' page-literal mode (fp32 scales).
* ``gemv``      -- y = W x in float64 and the acceptance bound.
* ``moe``       -- the routed expert layer (softmax top-K, SwiGLU, gated
                   combine + residual) and its propagated error bound.
* ``norm``      -- RMS normalisation (two passes) feeding the GEMV, and
                   its bound.
* ``decode_bound`` -- the handbook page's decode speed bound
                   (bandwidth x efficiency / weight bytes).

Parity status per function is stated in each module's header.  Q2_K's layout
is not printed on any page: its definition is a reading (the handbook's Q4_K
construction with 2-bit codes) and it is pinned only by round trips, brute
force and closed forms, not by a printed value.  The ternary and 1-bit
"quantizers" are exact packers of given codes, pinned by round trips.
"""
