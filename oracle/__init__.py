"""CPU oracle for the unmerged-LoRA linear over a frozen 4-bit base.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The GPU library never links, imports or calls it, and this package
never imports the GPU library: the two share no code, tables or constants.

The oracle is plain and slow on purpose. Every function follows a passage of
the source pages, cited by page title and section:

* "Quantized weights, full precision: The math behind 75% cheaper
  fine-tuning" (the Crusoe post): the unmerged forward ``Y = Y^base + Y^LoRA``,
  the gradients dX, dA, dB and no dW (sections "LoRA operations and
  quantization", "Backward pass and optimizer step in training"); 4-bit
  storage dequantized in flight to bf16 ("Forward pass in training").
* "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ": the LoRA math and the
  alpha/r scale (section 2, "The math", "Initialization matters"), NF4,
  blockwise absmax and double quantization (section 3, "The three QLoRA
  tricks"), the memory table (section 3).
* "Fine-Tuning 4-Bit Models: Adapting a Base That Only Ships Quantized":
  MXFP4 with a 32-element E8M0 block scale (section "Case 2").
* "Fine-Tuning 4-Bit Models", section "Case 2: An NVFP4 deployment
  checkpoint is what you were handed": NVFP4, E2M1 with an FP8 scale per
  16-element micro-block (see ``nvfp4`` for the readings).
* "Training LLMs on a Budget", section 4: LoftQ, alternating quantization
  and a rank-r SVD of the residual (see ``loftq``).
* The Crusoe post, "Forward pass in inference": the MXFP4-native base
  product (activations as MXFP8, a reading; see ``mxfp8``).

Floating-point products are evaluated in float64 on exactly representable
bf16 inputs. Encodings (bf16 rounding, NF4, E4M3, E2M1, E8M0) are written out
step by step from their definitions.

Parity status per function (what pins it is listed in ``tests/``):

* codecs.*           pinned (torch's own dtype conversions, exhaustive).
* nf4.codebook       pinned by invariants and two independent inverse-CDF
                     routines; the exact offset delta and the 7/8 asymmetry
                     are a reading of the pages, and parity against an
                     outside NF4 implementation is unpinned.
* nf4.* quantize/dq  pinned by brute force on tiny inputs, tie tables, round
                     trips and the pages' bits-per-weight figures.
* mxfp4.*            pinned by the OCP E2M1 value table, exhaustive code x
                     scale products and brute force.
* nvfp4.*            pinned by torch's float8_e4m3fn rounding of amax / 6,
                     brute-force nearest elements, exact tie midpoints, on-grid
                     round trips, exact dequant and the page's finer-than-MXFP4
                     claim on Gaussian weights.
* mxfp8.*            pinned by torch's float8_e4m3fn conversion, the scale
                     property, round trips of on-grid blocks, the zero and
                     subnormal blocks, the plain forward on on-grid X and the
                     E4M3 error bound.
* loftq.*            pinned by the page's 3 x 3 worked example, the
                     non-increasing error of the rounding loop (the page's
                     256 x 256 rank-8 setup), Eckart-Young on known singular
                     values and NF4 LoftQ against plain NF4.
* lora.*             pinned by finite differences, pure-Python loops, the
                     merge identity and the B = 0 / A = 0 special cases.
"""

from . import codecs, nf4, mxfp4, nvfp4, lora, mxfp8, loftq  # noqa: F401

__all__ = ["codecs", "nf4", "mxfp4", "nvfp4", "lora", "mxfp8", "loftq"]
