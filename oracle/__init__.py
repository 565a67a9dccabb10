"""fp64 CPU oracle for Falcon fast-weight attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP path and never imports it.

Sources (cited by page title and section throughout):
  [P1] zhouql-dev.github.io, "把状态更新写成一条学习规则：Falcon 家族重新对齐
       fast-weight 记忆" -- sections 本质 (essence), Falcon家族 (the family),
       三种等价形式 (three equivalent forms), Figures 1-4.
  [P2] 59188saintaubert.com, "给记忆装一个“及时纠错”的开关：Falcon让循环模型学会
       边写边改" -- sections 一个被忽略的时间差 (the time gap), 把记忆更新变成一次
       梯度下降 (one gradient step), 六个变体 (six variants), 正衰减钳制 (positive
       decay clamp), 三种视角 (three views).
  [P3] chooseai.io news brief on "Fast Weight Attention for Continual Learning"
       -- section 核心方法 (core method).

The pages lost the update equation in extraction; the oracle follows the
explicit statement of the method (residual-driven, prefix-aligned NLMS write
with a clamped positive decay) whose readings are listed in the module
docstring of :mod:`oracle.falcon_oracle`.

Pinning status: every public function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute-force masked-parallel equivalence, closed
forms, reductions and invariants).  The absolute values of the constants
eps_phi, eps_eta, the zero first key of a fresh sequence and the window divisor
at the start of a sequence are readings, not values the pages fix: for them the
parity is unpinned by the pages and fixed only by the readings.
"""

from .falcon_oracle import (VARIANTS, recurrent, masked_parallel, chunked,
                            decode_step, phi, recurrent_backward)

__all__ = ["VARIANTS", "recurrent", "masked_parallel", "chunked", "decode_step", "phi",
           "recurrent_backward"]
