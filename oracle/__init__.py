"""CPU reference ("oracle") for the rolling-window attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers); the only thing both sides consume is
the seeded input generator, which holds none of the method's arithmetic.

Everything here is plain, slow and written to be checked by eye against the
source pages ("A kernel-centric path to real-time video generation on
Trainium" and its digests):

* ``bf16``      -- exact float64 <-> bfloat16 conversion (round to nearest even).
* ``rope3d``    -- 3D rotary embedding over (time, row, column) token positions,
                   exact float64 and the bit-exact bf16 specification.
* ``ring``      -- the rolling frame-window KV cache as a model of frames/slots.
* ``attention`` -- non-causal softmax attention of query tokens over the
                   window's context frames, float64.
* ``qkv``       -- the layer's QKV projection and what it leaves in the cache
                   (q, rotated k, v as bf16), float64.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
closed forms, invariants, library routines or brute force.
"""

from . import bf16, rope3d, ring, attention, qkv  # noqa: F401
