"""CPU oracle of the SenseNova-U1 gen-tower denoise step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never calls it and shares no code with
it; the two meet only in the seeded inputs of ``workloads``.

Plain numpy, no fusion, no online softmax, no blocking: every function writes
out the definition of one step of the method.  Arithmetic runs in the dtype
of the inputs: float32 for parity runs (the "plain fp32 CPU implementation"
the GPU path is judged against) and float64 for the pins in
``tests/test_oracle_pins.py``.

Sources, cited by page title and section:
  [U1-recipe]    vllm-omni recipe "SenseNova-U1" (A3B (MoE) variant; Measured
                 (1x H20 96GB, BF16) with its kernel table; TP=2 notes)
  [U1.5-recipe]  vllm-omni recipe "SenseNova-U1.5" (Text-to-Image command;
                 8-step distilled LoRA)
  [DiffSynth]    DiffSynth-Studio model page "SenseNova-U1" (模型推理 inference
                 parameters; 快速推理 8-step LoRA; 架构说明 architecture notes;
                 模型训练 LoRA targets)
  [SETUP]        sensenova-u1-lora-trainer "Setup notes" (Why bf16 base on CPU
                 + tower offload?)
  [lilting]      lilting.ch "SenseNova U1 8BのLoRA trainerは32GB GPUのbf16学習を
                 前提にする" (default.yaml section: x0 loss, uniform timestep)
Where the pages leave a step open, the reading taken is stated at the function.

``backward.py`` holds the gradients of LoRA training with the x0 loss (the
derivative of each forward step, the block and the tower walked in reverse).

Parity status: every function here is pinned by a CPU test against a closed
form, a brute-force computation, a library routine or an invariant, except the
composition of the full tower, which is pinned only through its pinned parts
(the pages print no intermediate or output values): full tower parity
unpinned beyond composition.
"""
from .ref import *  # noqa: F401,F403
from .backward import *  # noqa: F401,F403
