"""Plain CPU oracle for one Muon optimizer step and the AdamW elementwise step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``muon_step_amd``) and imports nothing from it.

Sources (the pages this oracle is written from):

* "Muon 优化器完全拆解：矩阵级正交化更新如何撑起万亿 MoE 训练" (the Muon
  deep-dive page), sections "V4 的完整更新公式，逐行拆解", "系数怎么调出来的",
  "更新尺度", "为什么嵌入层、输出头、bias、RMSNorm 还在用 AdamW",
  "收益与代价".
* "Ch 06 · Muon — 矩阵参数的指南针" (DeepSeek-V4 book, chapter 6), sections
  3 (Newton–Schulz), 4 (hybrid two-stage 10 steps) and 5 (the expanded
  Algorithm 1 with the explicit Frobenius normalisation).

Precision: the Newton–Schulz iteration, normalisation and rescale run in
float64.  The elementwise bookkeeping (momentum, Nesterov input, the final
decay + update, AdamW) runs in numpy float32 with one IEEE round-to-nearest
per operation and no fused multiply-add, because that bookkeeping is required
to be reproduced bit for bit.

Pins: every public function is pinned by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, a Jacobi-SVD polar factor, the
singular-value map, torch's own SGD/AdamW and brute force.  No function here
is "parity unpinned".
"""

from .muon import (  # noqa: F401
    DEEPSEEK_V4_SCHEDULE,
    QUINTIC5_SCHEDULE,
    nesterov_momentum_f32,
    newton_schulz,
    orthogonalized_update,
    muon_scalars_f32,
    unit_rms_factor,
    update_scale,
    apply_update_f32,
    muon_step,
    ns_flops_algorithmic,
    ns_flops_dense,
)
from .adamw import adamw_scalars_f32, adamw_step_f32  # noqa: F401
from .bf16 import bf16_round_f32, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
from .jacobi import jacobi_svd, polar_factor  # noqa: F401
