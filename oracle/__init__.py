"""CPU oracle for the sparse Mixture-of-Experts layer forward — TEST INFRASTRUCTURE.

A plain, slow, obviously correct float64 NumPy implementation of what the layer
computes, written from the pages' definitions.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; the HIP product path never
does, and this package imports nothing from it.

Modules
    numerics  bf16 widening, fp8 e4m3fn decode/encode (round to nearest even)
    moe       the layer's steps: logits, group limit, top-k, sparse softmax,
              load statistics, dispatch plan, dispatch values, expert FFNs,
              combine, and the whole forward
    compare   the comparison procedure (tie-band adoption) used by parity tests
    brute     pure-Python brute force for tiny inputs (an independent check)

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` (brute force, closed forms, the pages' printed
numbers, invariants).  Parity unpinned: none of the functions; the full-size
expert outputs are pinned only through the same code at small sizes.
"""
