"""CPU oracle for the W4A16 NVFP4 routed-expert MLP.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may use it. It shares no code with the HIP library (no
kernels, headers, helpers, tables or constant generators); the two meet only
through the seeded inputs from ``synth``.

What it computes, and from which passage:

* ``formats``  - bf16 widening/narrowing, the e2m1 and e4m3 number formats
  (decode from their closed forms, round-to-nearest-even encode).
* ``nvfp4``    - the load-time BF16 -> NVFP4 pack and the dequantization of
  stored weights (TensorFold issue #308, section "The checkpoint": e2m1 codes,
  one e4m3 scale per 16 inputs, one fp32 weight_scale_2 per tensor; section
  "What the branch does": at load, ModelOpt's recipe quantizes the MTP layer's
  BF16 experts one projection after another).
* ``mlp``      - the dense Fp4Linear (separate gate and up projections, each with
  its own tensor scale), the expert permutation, and the routed expert MLP
  (grouped gate/up, SiLU(gate)*up, grouped down, routing-weighted sum).
* ``block``    - the steps either side of the routed experts: the BF16 router
  with top-k softmax selection, the shared-expert BF16 MLP, and the MoE block
  (routed + shared).
* ``brute``    - float64 pure-Python loops on tiny shapes, used only to pin the
  vectorised oracle.

Precision: the pack runs in float32, because the quantized codes and scale
bytes are decided by float32 arithmetic on both sides. Every contraction runs
in float64 and represents the exact real-number result of the dequantized
weights applied to the bf16 inputs.

Pins (tests marked ``not gpu``) tie every function to something other than
itself: torch's float8/bfloat16 casts, closed forms and value sets of the
formats, hand-derived golden bytes, invariants of the pack, brute force,
exact integer arithmetic, and library sorts. No function here is
"parity unpinned".
"""
from . import formats, nvfp4, mlp, block, brute  # noqa: F401
