"""Plain float64 CPU oracle of one Muon optimizer step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it. It shares no code with the HIP library and imports nothing from it.

Sources (the pages are cited by title and section):

* [P3] "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (reposource.net),
  section "Muon优化器：动量正交化技术", subsections "核心算法" (the optimizer's
  constructor defaults and the three phases of ``step``) and "Newton-Schulz正交化"
  (the quintic iteration and its coefficients).
* [P1] "Muon优化器与FP8混合精度：AI训练能效革命与绿色计算新范式" (bxzpzcl.cn), section
  "Muon优化器的能效突破" (Muon = momentum orthogonalised by Newton-Schulz).
* [P4] the RecursiveFromBest record analysis (lqnn.cn/news/184262), section 3.2 "NorMuon
  中的退火行 RMS 缩放 Langevin/SGLD 探索噪声", which names Frobenius normalisation as the
  step in front of the quintic maps of the Muon family; and section 3.3 "bigram 与
  value-embedding 银行上的 C-Optim / 谨慎 Adam" (cautious Adam for the embedding-like
  parameters, oracle/cautious_adam.py); section 3.2 also names NorMuon's per-lane energy
  equaliser after the orthogonalisation (oracle/row_equalizer.py).

Readings where the pages are silent are listed in the headers of muon.py,
cautious_adam.py and row_equalizer.py.
"""
from .muon import (  # noqa: F401
    DEFAULT_ABC,
    momentum_update,
    frobenius_normalize,
    newton_schulz,
    orthogonalize,
    muon_step,
    muon_run,
)
from .cautious_adam import (  # noqa: F401
    adam_moments,
    adam_direction,
    cautious_decay,
    cautious_adam_step,
    cautious_adam_run,
)
from .row_equalizer import (  # noqa: F401
    row_second_moment,
    row_equalize,
    muon_step_equalized,
    muon_run_equalized,
)
