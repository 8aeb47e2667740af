"""Plain, slow CPU oracle for microscaled FP4 quantization.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it. It shares no code, tables or helpers with the
HIP path under ``mxfp4_microscaling_quantization_amd/``.

Everything is numpy on the host. Values are carried in float64, which holds every
bf16, fp32, E4M3 and E2M1 value and every power-of-two product used here exactly;
where a quotient is involved (NVFP4) each function states why a float64 result
decides the rounding exactly as exact real arithmetic would.

Sources (cited by title and section in every module):
  [HOPPER-FR]  "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
               French summary page, "Résumé technique" (sections 1-5).
  [HOPPER-ES]  the same paper, Spanish summary page, "Resumen técnico".
  [MXFP4-MI355X] "Pretraining large language models with MXFP4 on Native FP4
               Hardware", news article, sections "Qu'est-ce que le MXFP4 ?" and
               "Expérience d'investigation".
  [NVFP4]      "Pretraining Large Language Models with NVFP4", French summary page,
               "Résumé technique" section 2 (A. format, B. methodology).

Readings of points the pages leave open are listed in each function's docstring.

Parity status per function (what pins it is in tests/test_oracle_*.py):
  formats.*            pinned (brute force, torch casts, closed-form tables)
  mx.*                 pinned (invariants, brute force, hand-worked golden blocks)
  fp8.*                pinned (torch E4M3 casts, exhaustive code x shift sweep;
                       the rows-to-columns conversion also by a Fraction brute
                       force over ragged expert segments)
  rht.*                pinned (scipy Hadamard, orthogonality, inverse, norms)
  nvfp4.*              pinned (Fraction brute force, torch E4M3 cast, invariants)
  philox.philox4x32_10 pinned against the published known-answer vectors of
                       Philox4x32-10 (tests/golden/philox_kat.json) and against
                       rocRAND's independent Philox4x32-10 header when hipcc is
                       present (skipped otherwise); statistical tests
  philox.element_r16_halves  pinned against rocRAND's word stream (half n mod 2 of
                       word n/2), a hand-worked vector from the known-answer words,
                       and uniformity / unbiased-rounding statistics
  rht.sign_mask_from_seed  the seed-to-signs mapping is a definition made here
                       (the pages only say "random signs"); pinned by the published
                       word of seed 0 (mask 0xE8D5) and rocRAND's engine
"""
