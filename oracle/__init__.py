"""CPU oracle for the layer-streamed decoder training step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything under ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  The oracle shares no code with the HIP library in
``layer_streaming_amd/``; the two meet only through the seeded input
generators in ``layer_streaming_amd/synth.py``, which hold none of the
method's arithmetic.

What it computes.  The pages describe a memory-centric trainer whose
streaming changes where bytes live and when they move, never the result:
standard BF16/FP32 mixed-precision full-parameter training with Adam, with
no quantisation and no approximation (lilting.ch article "MegaTrain ...
120B ... full precision", section on accuracy verification; MegaTrain review
on dimensionstp.github.io, section 5-1 accuracy table).  The oracle is
therefore the plain definition of one training step of a pre-norm decoder
LM, written out in float64 with numpy:

* ``oracle.bf16``  -- round-to-nearest-even float32 -> bfloat16.
* ``oracle.block`` -- RMSNorm, linear maps, RoPE, causal GQA attention,
  SwiGLU, cross-entropy; forward and hand-written backward of each.
* ``oracle.step``  -- the decoder layer, the LM head, the whole-model loss
  and gradients (monolithic and layer-streamed forms), and the host Adam.

Pins (``tests/test_oracle_*.py``, all ``-m "not gpu"``): finite differences
of every parameter element on tiny shapes, closed forms (CE with a zero head
equals ln V, attention special cases, RoPE identities, RMSNorm of a constant
row, Adam's first steps), float64 autograd of torch at the tiny-LM shape,
torch's scaled-dot-product attention, brute force, and an exhaustive check
of the bf16 rounding against its IEEE definition.  No function here is
"parity unpinned".
"""
