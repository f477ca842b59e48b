"""CPU oracle for the scaled FP8 linear layer: TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct definition of what the GPU
path computes. It exists so that the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` can check the HIP kernels against it. The
product path (``scaled_fp8_linear_amd``) never imports, links or calls anything
in here, and nothing in here imports the product path. The two share no code.

Sources (the web pages this method is taken from):

* AstrAI, ``astrai/extension/fp8_state.py``: the constant E4M3_MAX = 448, the
  GEMM layout comment ``D = A_SCALE * B_SCALE * A * B``, ``FP8TensorMeta``
  (``record``, ``refresh``), ``FP8State.step``, ``_update_delayed_scale``,
  ``fp8_linear_forward`` / ``fp8_linear_backward``.
* SpecForge PR 2, "Add training.fp8_linear: torchao Float8Linear with float8
  all-gather", Conclusion (Constraints bullet) and Modifications: the token
  count of an fp8 GEMM must be a multiple of 16; current (dynamic tensorwise)
  scaling.
* NeMo PR 15754, "Add FP8 support for SALMAutomodel", review thread on BSHD
  padding: ``pad = (-T) % seq_multiple``; TE's block recipe.
* The OCP 8-bit floating point specification (OFP8, E4M3 variant), which the
  name "e4m3" and the maximum 448 identify; its E5M2 variant for the hybrid
  format's gradients.

Modules:

* ``e4m3``      -- the E4M3 code table and two independent encoders.
* ``e5m2``      -- the same for E5M2, the gradient format of the hybrid recipe.
* ``quantize``  -- tensorwise quantize with amax, and the transposed copy.
* ``scaling``   -- scale from amax, the weight amax-history ring, and the
                   per-step delayed-scaling schedule of one linear layer.
* ``gemm``      -- the exact scaled GEMM in float64 and its error bound.
* ``bias``      -- the bias added to the forward output, and the bias gradient
                   (column sums of the output gradient), with their tolerances.
* ``padding``   -- token-count padding to a multiple.
* ``block``     -- the block-scaled recipe (1x128 / 128x128 tiles).

Every function works on numpy arrays: bf16 tensors travel as ``uint16`` bit
patterns, e4m3 tensors as ``uint8`` codes, scales as ``float32``.
"""
