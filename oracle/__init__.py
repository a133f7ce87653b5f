"""Plain, slow CPU reference for the block-diffusion denoise step (test infrastructure only).

This package is the oracle that the HIP library is checked against. It is NOT part of the
product path: only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it, and the library never calls into it. It shares no code, tables or
helpers with ``two_tower_cross_amd``; the only module both sides use is ``synth`` (seeded inputs,
no method arithmetic).

Everything is computed in float64 with NumPy from the definitions on the pages:

* ``attention.block_attention`` -- the denoiser's attention at one layer: the block queries attend,
  under one softmax, to the context tower's same-layer KV cache and to the block's own KV
  (Nemotron-TwoTower explainer, gist.science, sections "Architektur" and "Generierungsprozess";
  the Chinese version of the same page, same sections; "NVIDIA loest den zentralen Kompromiss
  moderner LLMs", gotburnout.io, section "2. Denoiser Tower"; dgnews.ru report on Nemotron-Labs-
  TwoTower, architecture section).
* ``unmask.confidence_unmask`` -- confidence unmasking: predict all masked positions, commit those
  whose confidence exceeds the threshold, keep the rest masked (explainer, section "Training und
  Konditionierung", sampling paragraph; dgnews.ru, test-results section for the threshold 0.8).
* ``step`` -- one denoise step of a synthetic attention-only denoiser and the T-step loop around
  it (explainer, section "Generierungsprozess").
* ``bruteforce`` -- pure-Python loops with an explicit softmax, for tiny shapes only.

Every function here is pinned by ``tests/test_oracle.py`` against closed forms, invariants,
brute force and independent library routines.
"""
from . import attention, unmask, step, bruteforce  # noqa: F401
