"""CPU oracle for confidence-scheduled, flattened speculative verification.

TEST INFRASTRUCTURE. This package is the slow, plain reference that the HIP
library is checked against. Only the test suite, the smoke check of the entry
script and the CPU-baseline leg of the benchmark may import it; the product
path never does.

It is written from the DSpark pages, cited by title and section:

  [P1] "刚融完500亿创始人亲自下场写代码DeepSeek不卷参数专治AI“嘴慢”"
       (mooersco.com news article), sections "1. 半自回归生成",
       "2. 置信度调度验证" and the engineering table under
       "不止是算法更是“工业级”的系统魔改".
  [P2] "DSpark 的 661% 提速，是真突破还是数字游戏？" (new-universe.cn),
       sections 一 (why decoding is slow; speculative decoding),
       3.1 (生成侧：半自回归架构), 3.2 (验证侧：置信度调度的动态决策).
  [P3] "DeepSeek服务器不再卡顿！DSpark加速60% - 80%，推理成本降40%"
       (qwbw.cn), section "DSpark的神奇之处".
  [P4] aibuzzwire.news article "deepseek-dspark-speculative-decoding-85-percent-
       faster-llm-inference", sections "置信度计划、负载感知验证" and the opening
       paragraphs on speculative decoding.

Arithmetic is float64 throughout; bf16 and fp32 inputs are decoded exactly.
Loops run in index order; numpy primitives (exp, sum, argmax, cumsum, matmul)
serve as single steps with no blocking or reordering beyond what the
definitions state. Nothing here is shared with the HIP sources.

Modules
  numerics  decoding, bf16 rounding, softmax, argmax, inverse-CDF draw
  philox    the counter-based generator (Philox4x64-10) behind every uniform
  rule      the acceptance rule for one request, in any exact or float arithmetic
  verify    the rule over a flattened batch, float64, vectorised over requests
  schedule  calibration, survival, the hardware-aware prefix scheduler, flatten
  markov    the Markov head of the semi-autoregressive drafter
  rnn       the RNN head (recurrent state over the block's prefix)
  attention tag-masked attention of the flattened rows over a paged KV cache
"""

from . import numerics, philox, rule, verify, schedule, markov, rnn, attention  # noqa: F401
