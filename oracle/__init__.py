"""CPU oracle for the NVFP4 weight-only linear layer with LoRA and AQN.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct definition that the HIP library is checked against.  It may be
imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``.  The product path never calls it and
shares no code with it: the HIP side and this side each implement the
number formats, the quantizer, the noise generator and the linear layer on
their own.  The only thing both sides use is the seeded input generator
package ``workloads``, which holds none of the method's arithmetic.

Sources are cited by page and section; the pages are
  * "QeRL: Beyond Efficiency -- Quantization-enhanced Reinforcement
    Learning for LLMs", the long summary page (paper-graph-ui), cited as
    [QeRL summary, <section>, <Eq./Table/Fig.>];
  * the arXiv abstract on the mlsanity.com page, cited as [QeRL abstract].
Facts that are not on the pages (the OCP FP8 E4M3 encoding, the Philox
counter-based generator, the Box-Muller transform) cite their own
published definition.

Modules
  formats  E2M1 / E4M3 / bf16 / fp32 value tables and exact rounding.
  nvfp4    quantize (bf16 -> E2M1 codes + E4M3 block scales + FP32 scale)
           and dequantize (Eq. 6).
  aqn      the exponential sigma schedule (Eq. 8) and the noise vector
           (Eq. 7) drawn from Philox4x64-10 + Box-Muller.
  linear   y = (x * (1 + z)) W^T + s (x * (1 + z)) A^T B^T in fp64.
  rmsnorm  the noisy RMSNorm producer (w + z) * x / rms(x) (Eq. 10).
  swiglu   SiLU(gate) * up between the gate/up and down layers.
  mxfp4    the MXFP4 variant (E8M0 scale per 32) and its NVFP4-layout form.

Parity pins (tests/test_oracle_*.py): every function here is checked
against something other than itself: values printed on the pages
(tests/golden/), brute force in exact rational arithmetic, numpy's own
Philox bit generator, closed forms and invariants.  No function here is
"parity unpinned".
"""
