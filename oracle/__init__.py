"""Plain, slow, float64 CPU oracle for TurboQuant-style KV-cache compression.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product
library never calls it, and it imports nothing from the product package.

The pages this oracle follows (cited by tag in every module):

  [P1] "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
       Cuantizaciones de Cache KV Inspiradas en TurboQuant"
       (gist.science/es/paper/2605.08114)
  [P2] "Resumo Técnico: Ablação, Inferência Estatística e Validação para
       Compressão de KV-Cache" (gist.science/pt/paper/2607.09683)
  [P3] "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
       Espaço de Pontuação para Quantização de KV-Cache"
       (gist.science/pt/paper/2605.03562)

Everything is numpy float64 with dense matrices and no blocking.  The read
side is computed by its plain definition: every key and value is
dequantised densely in the original domain, then textbook softmax attention
is applied.

Parity status of each part (what pins it is listed in the tests):
  codebook, rotation, quantiser, QJL estimator, attention, metrics: pinned.
  SpectralQuant with uniform allocation (spectral.py): pinned (Gaussian
      codebook against Max's table, calibration, hand-worked case,
      equivariance, distortion, the pages' orderings).
  A^2-weighted value policy (value_policy.py): pinned (weights in closed
      form for equal and dominant keys and their bounds, the selection by
      brute force, uniform chosen for equal weights by the convexity of the
      distortion in the bit width, the expected surrogate by Monte Carlo,
      the pages' ordering against uniform values at 2 bits).
  HeadQ side quantiser Q_q: parity unpinned (the pages give no form; the
      per-token symmetric absmax 4-bit reading is our own).
  RNG streams for the sign vector and the Gaussian sketch: a reading (the
      pages fix only the distributions, which are pinned statistically).
"""
from . import codebook, rng, rotation, quantizer, attention, metrics, headq, schemes, spectral, value_policy  # noqa: F401
