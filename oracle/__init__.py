"""CPU oracle for the fused W4A16 mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code in float64 that states what the layer
computes, so that the HIP library can be checked against it. Only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the HIP library and imports nothing from it.

What it follows (FlashInfer PR 4255, "feat(moe): sync SM12x W4A16 fused MoE
family to b12x HEAD"; and the OCP Microscaling v1.0 / OCP FP8 specifications
for the code formats, which the page names but does not define):

* ``formats``    -- E2M1 / E4M3FN / E8M0 code tables, round-to-nearest-even
                    quantisers, MXFP4 (E8M0 per 32) and NVFP4 (E4M3 per 16 +
                    fp32 global) quantise / dequantise, MXFP8 (E4M3 per element,
                    E8M0 per 32) for the W4A8 variant's FC2 operand, nibble
                    packing, bf16 rounding. Page: Description (NVFP4 weights; the new
                    fp4_e8m0_k32 source with scale tails), Review round 1
                    (power-of-two-ceiling UE8M0 scale helper).
* ``route_pack`` -- grouping of token x expert routes by expert into a padded,
                    power-of-two-capacity workspace with expert_map remapping
                    and dropping of invalid ids. Page: Description
                    (shape-stable route packing), Tests (expert_map, invalid
                    ids, capacity contract), Review round 1 (capacity helper,
                    minimum-one clamps).
* ``moe``        -- FC1 -> SiLU-SwiGLU or relu2 -> FC2 and the router-weighted
                    top-k sum. Page: Description (fused FC1/FC2 kernel, top-k
                    sum folded into the FC2 store epilogue), Performance
                    (relu2 and silu activations); the W4A8 variant (review: the
                    grouped MXFP8 quantisation of the SiLU-mul output, with an
                    exact-silu reference) quantises the activation output to
                    MXFP8 before FC2.

Every function is pinned by tests under ``tests/`` against specification
tables, closed forms, hand-computed cases, library decoders and brute force.
Nothing here is parity-unpinned.
"""

from . import formats, route_pack, moe  # noqa: F401
