"""CPU oracle for the KV-chunk quantizer and the attention over its packed cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It is a plain, slow, deliberately unoptimised restatement of
what the method computes, written from the pages (sources below), in NumPy, with
fp64 arithmetic wherever the pages leave the precision open and the stated
rounding steps (fp32, bf16) wherever a reading fixes them.

Sources (cited by page title and section):
  * "Quant VideoGen: Auto-Regressive Long Video Generation via 2-Bit KV-Cache
    Quantization" (paper notes page, ICML 2026) -- called *QVG notes* below.
  * "AI生成视频时为什么会悄然记错画面？一个被忽视2比特量化陷阱" (QuantWM summary
    page) -- called *QuantWM summary* below.
  * "视频生成中的2比特量化陷阱：画面为何悄悄失真" (explainer article) -- called
    *2-bit trap explainer* below.
  * "视频世界模型KV Cache时序稳定2-bit压缩方案实战" (practitioner blog) -- called
    *practitioner blog* below.

Modules:
  numerics   -- bf16 round-to-nearest-even, exact (correctly rounded) group sums
  kmeans     -- Lloyd k-means with the fixed protocol (strided init, 10 iterations)
  quant      -- per-group symmetric quantizer, channel classes, bit packing
  pipeline   -- one chunk through all stages (smoothing, quantization, progressive
                residual stages, PSAC encode) and dequantization
  psac       -- query statistics: QSAC channel weights, principal subspace, ranking
  attention  -- softmax attention over the dequantized cache with the PSAC term

Every function's parity status is stated in its docstring; functions without an
independent pin say "parity unpinned".
"""
