"""CPU oracle for the blockwise-FP8 ZeRO-1 shard-local optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or constants with the HIP library, and it imports nothing from it.

It is a plain, slow, obviously correct numpy restatement of what the step
computes, written from these pages (cited by title and section):

* [FP8-ZeRO1] "面向 Blockwise FP8 量化的 ZeRO 优化器设计" (A ZeRO optimizer
  design for blockwise FP8 quantization), beipo.top/blog/fp8-zero1 -- the
  authority on the method: 128x128 blockwise weight quantization
  (section "Blockwise 量化"), the param-wise and block-wise shard splits
  (sections "参数粒度切分", "块粒度切分"), fold/unfold (section
  "参数布局变换") and the step order (section "总结").
* [DS-ZeRO] "DeepSpeed ZeRO 优化" (gitcode.csdn.net) -- the optimizer step
  order (section 3.2), dynamic loss scaling (section 6), global-norm gradient
  clipping (section 7) and the overflow check (section 9, Q6).
* [FSDP] "FSDP-Zero123分片简介" (solus-sano.com) -- the AdamW state set
  (section "参数组成").
* [FP8-Ling] "FP8训练技术与万亿参数模型优化实践" -- E4M3 as the training
  format (section 1.1) and the amax/qmax scale pattern (section 1.2).

Floating point: the pages fix the master weights, the moments and the
gradients at FP32 and the weights at FP8 E4M3; the oracle therefore does the
elementwise update in float32 numpy (one IEEE rounding per operation, no
fused multiply-add) and every scalar (norms, bias corrections, step size) in
float64, rounded once to float32.  Where the pages leave a step open the
reading taken is written beside the code that takes it.

Parity status per function (how each is pinned is in tests/test_oracle_*.py):
  e4m3.encode/decode   pinned (exhaustive vs torch's E4M3FN cast, OCP closed forms)
  table.*              pinned (ownership/padding invariants, hand-derived golden table,
                               independent LPT, brute-force optimum on tiny inputs)
  layout.fold/unfold   pinned (the printed view/permute formula run in torch,
                               round trip, index-tensor closed form)
  optim.*              pinned (float64 brute force, closed forms at t=1,
                               torch.optim.AdamW, fsum, hand-computed loss-scale runs)
  quant.requant_block  pinned (amax code is 0x7E, half-ULP error bound, zero block)
  step.*               pinned (sharded == unsharded over all ranks, skip/poison invariants)
The whole-method scale rule (s = amax/448, quantize by division) is a reading
of silent pages; no page prints a worked numeric example, so that rule is
"parity unpinned" beyond the invariants listed above.
"""

from . import e4m3, layout, optim, quant, step, table  # noqa: F401
