"""CPU oracle for the NF4 + LoRA layer-streamed hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code, table or constant with the HIP
library under ``nf4_layer_streamed_amd/``; the two meet only in the seeded
input generators of ``synth.py``, which hold no arithmetic of the method.

Everything here is plain NumPy in float64, written from the definitions:

* ``nf4``    - the 4-bit NormalFloat codebook, the block-wise quantiser,
               the packing of two codes per byte, and the dequantiser.
* ``linear`` - the frozen NF4 linear with its LoRA adapter, forward and
               backward (no gradient for the frozen weight).
* ``stack``  - the attention-free decoder-layer stand-in (RMSNorm, q/k/v/o,
               SwiGLU) stacked over layers, forward and backward, plus the
               per-layer store sizes.

Sources: the Soup pages (GitHub README "Citing Soup"; the themenonlab blog
post "Soup: Fine-Tune an 8B LLM on a 4 GB Laptop GPU From One YAML File";
the soup-cli 0.72.0 -> 0.72.2 diff, CHANGELOG [0.72.2] and the docs section
"NF4 streaming (quantization: 4bit)") say what is computed; they are silent
on the NF4 codebook, block size, scale format and rounding, for which the
QLoRA paper (Dettmers et al., 2023, section 3, "4-bit NormalFloat") is the
published method followed here.

Parity status per function is stated in each module header.
"""

from . import nf4, linear, stack  # noqa: F401
