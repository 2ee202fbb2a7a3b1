"""CPU oracle for the QAM-W weight codec -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the codec computes, written from
the description of QAM-W ("QAM-W: Joint 2D Codebook Quantization for LLM
Weights via Hadamard Rotation and Activation-Aware Scaling", gist.science
explainer of paper 2605.26339; cited below as "QAM-W, <section>").

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(``vector_codebook_codec_amd``) never imports it, and this package imports
nothing from the product: the two share no code.  Inputs come from the
``workloads`` module, which holds none of the codec's arithmetic.

Modules
  qamw_ref  -- the codec: sign mask, rotation, calibration, nearest-centroid
               search, bit packing, decode; output-error identity.
  lloyd     -- the 2D Lloyd-Max codebook trainer (offline, CPU).

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against closed forms, textbook or library routines,
published test vectors or brute force.  Agreement with the paper authors' own
implementation is unpinned: the pages print no codebook, sigma values, test
vectors or code, so the readings this oracle takes where the pages are
silent (sign generator, Hadamard order, bit layout, sigma estimator, ...)
cannot be checked against them.
"""
