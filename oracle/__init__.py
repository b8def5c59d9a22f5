"""CPU oracle for exact attention forward (test infrastructure only).

This package is the independent reference that the HIP path is checked
against. It is plain, slow, obviously correct numpy code in float64 (the
FP8 quantiser is the one exception: it works in float32 on purpose, because
a quantised code must be decided in the same precision on both sides).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (the HIP library and its Python
binding) never imports, links or calls anything here, and shares no code with
it: the two meet only through the seeded inputs in ``synth_inputs``.

Contents
--------
attention   plain definition O = softmax(alpha Q K^T) V with LSE, the online
            (m, l, O~) recurrence, the block-combine rule, sampled rows.
attention_bwd  gradients dQ, dK, dV of the plain definition.
fp8         Sylvester Hadamard matrix, fast Walsh-Hadamard transform, the
            splitmix64 sign generator, OCP e4m3 encode/decode, block
            quantisation, and the fp8-emulating reference.
variants    grouped/multi-query heads, N_q != N_k, packed variable-length
            batches, split-KV partial states and their merge.

Every function names the passage of the pages it follows. Pins (tests that
check the oracle against something other than itself) live in
``tests/test_oracle.py``, ``tests/test_oracle_bwd.py``,
``tests/test_oracle_fp8.py`` and ``tests/test_oracle_variants.py``.
"""
from . import attention, attention_bwd, fp8, variants  # noqa: F401
