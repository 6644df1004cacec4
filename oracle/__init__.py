"""CPU oracle for the canvas denoise step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct fp64 implementations of what one denoise step
computes, written from the DiffusionGemma explainer (ai.google.dev,
"DiffusionGemma explained"; Italian/Vietnamese/Turkish renderings of the same
page).  Sections cited by their Italian headings:

  "Il problema con i modelli autoregressivi"  the 256-token random canvas
  "Diffusione dello stato uniforme"           renoise below a threshold
  "Architettura: il prefill incrementale e il denoising"
                                              causal prefill writes the KV cache;
                                              denoise attends bidirectionally
  "Autocondizionamento"                       probabilities times the embedding table
  "Campionamento multi-canvas (diffusione a blocchi)"
                                              append a finished block to the cache
  "Diffusione mascherata"                     the masked sampler: unmask where
                                              confident, committed tokens locked

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP path, and the
HIP path never imports it.

Modules:
  philox   Philox4x64-10 (Salmon et al., SC'11) and the uniform token draw
  numerics rounding of API-visible tensors to their storage precision
  step     numpy fp64 step (assemble, projections, attention, vocab head,
           self-conditioning, renoise, causal append; the masked sampler's
           unmask-and-lock)
  brute    the same step in scalar pure-Python loops with math.fsum, for
           canvases of at most 16 tokens
"""
