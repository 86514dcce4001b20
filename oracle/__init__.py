"""CPU oracle for RACE Attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything in this package.  The
GPU library never routes through it and shares no code with it.

Two implementations of the same computation, both in float64:

* ``dense``  — NumPy, one (batch, head) at a time, for small N.
* ``stream`` — plain C with OpenMP over (batch, head), a per-token recurrence
  over the sequence, for any N; inputs may be float32, bf16 bits or float64.

Sources (pages on arXiv 2510.04008, "RACE Attention: A Strictly Linear-Time
Attention for Long-Sequence Training"):
  * gist.science (Japanese), technical overview, section 2.1 (kernel,
    soft bucketing, aggregation, reconstruction), section 2.2 (temperature,
    causal prefix sums, complexity), section 3 (P plays the role of gamma);
  * gist.science (Italian), "Sommario tecnico", section 2 Metodologia
    (tanh + softmax over hypercube vertices; mass and value sums; L tables;
    normalised weighted average);
  * gist.science (Korean), "기술 요약", section 2 방법론 (L tables, P random
    hyperplanes each, R = 2^P buckets);
  * fugumt.com, English abstract (forward-backward pass; randomized
    projections and soft LSH).

Readings where the pages are silent are listed in the module docstrings of
``dense`` and ``race_oracle.c``.
"""
