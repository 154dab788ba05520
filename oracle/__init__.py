"""CPU oracle of the LowRAM decode step — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what one decode step computes, written
from the LowRAM pages:

  * LowRAM review (agihunt.info), key paragraph: keys are factorised with a
    cross-layer low-rank basis shared by adjacent layers, after undoing RoPE;
    at decode the prefix is cut into chunks whose mean key is a landmark, and
    only the top-k chunks for the current query are rebuilt.
  * LowRAM explainer (cctest.ai), "How the method works": low-rank keys,
    amortised values through a small per-head key-to-value predictor,
    residuals kept only for the worst-predicted tokens, and selective
    reconstruction at each decoding step.
  * LowRAM abstract: values predicted from keys by a lightweight per-head
    predictor, residuals for the worst tokens, a selected subset of KV pairs
    rebuilt per step.

Only the test suite, the package's smoke check and the CPU-baseline leg of
the benchmark may import this package.  The GPU library never does, and this
package imports nothing from it: the two share no code.  Both read their
inputs from the seeded generators in ``synth``.

Modules
  codecs    bf16 / fp16 / int4-group-32 storage codecs (pinned by golden bytes)
  steps     the per-step definitions: RoPE, GELU, value MLP, landmark score,
            top-k selection, reconstruction, softmax attention
  decode    one decode step over a batch, and the dense-attention baseline
  compress  the prefill side that writes the compressed cache (projection,
            landmarks, values, residual selection, window, eviction)
"""
