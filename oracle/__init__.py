"""CPU oracle for the hybrid MuonAdamW optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code, constants or helpers with
the HIP library; the two meet only through seeded inputs and compared outputs.

The method is described on the OpenDM training-stack page ("VLA训练栈深度揭秘：
OpenDM的MuonAdamW优化器、FSDP分布式训练与混合精度策略"), in its sections on the
Muon/AdamW hybrid optimizer (parameter routing, Newton-Schulz orthogonalisation,
the hyperparameter table with the shape-dependent learning-rate factor) and in
its defaults table (gradient clipping).  Every function in `muon_adamw` names
the part of that page it follows.
"""

from .muon_adamw import *  # noqa: F401,F403
from .muon_adamw import __all__  # noqa: F401
