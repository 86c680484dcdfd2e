"""CPU oracle for the DiffusionGemma canvas denoising step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
shares no code with that path: the two meet only in the seeded input
generators of ``synth``.

The oracle is plain and slow on purpose: numpy in float64 for every floating
point step (weights and logits are widened from their storage types), library
primitives (matmul, sort, cumsum) as single steps, no blocking or fusion.
Each function cites the passage of the pages it follows. Sources:

* [MC-zh] DiffusionGemma model card, Traditional Chinese edition
  (gemma.gh.miniasp.com): intro list, "模型總覽" (model overview), the spec
  table, "核心能力" (capabilities) and best practice 1, "擴散取樣設定"
  (diffusion sampling settings).
* [MC-ko] DiffusionGemma model card, Korean edition (ai.google.dev):
  "모델 개요" (overview) and recommendation 1 (diffusion sampling settings).
* [AIT] aitrends.kr summary of diffusiongemma-26B-A4B-it, sections
  "알아두면 좋은 것" (good to know) and "기술적 특징" (technical features).
* [GATE] gate.com news post, section on how the model generates without a
  sequential order.
* [BLOG] charlie27.com digest, section on DiffusionGemma (its remark that
  outputs are corrected over the iterations).

Where the pages are silent the plainest reading is taken; every such reading
is listed in the design notes of the repository.
"""
from . import fp8, sampler, model, generate  # noqa: F401
