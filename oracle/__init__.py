"""CPU oracle for one decode step of a mixture-of-experts transformer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

The pages on the decode megakernel present it as a change to how a serving
system schedules work, not a new model: it is assembled from plain tiled
matrix products and paged attention and loses no accuracy ("Cohere Publishes
One-Kernel Server for North Mini Code, Claims 1.58x vLLM Speedup", opening
section and section "A hand-built approach to a specialized server"). So the
oracle is the plain sequential definition of a decode step, one sequence at a
time, in float32 over BF16 weights (float64 on request), with rotary angles
in float64.

Parity status of each function is stated in its docstring; every function
here is pinned by a test under tests/ (invariant, closed form, library
special case or brute force). Nothing is "parity unpinned".
"""

from .decode import (  # noqa: F401
    bf16_to_f32,
    f32_to_bf16_rne,
    rms_norm,
    rope_rotate,
    rope_cos_sin,
    gather_pages,
    attention_decode,
    route_topk,
    route_weights,
    swiglu_expert,
    attention_block,
    moe_block,
    final_logits,
    moe_combine,
    DenseModel,
    PagedKV,
    decode_step,
    decode_sequence,
    prefill,
)
