"""MI355X-native Muon optimizer step: a C-ABI HIP library (libmuon.so, include/muon.h)
with a thin PyTorch binding.

    from orthogonalized_momentum_optimizer_amd import Muon
    opt = Muon(model_matrices, lr=0.02, momentum=0.95, nesterov=True, ns_steps=5)
    adam = CautiousAdam(other_params, lr=1e-3, betas=(0.9, 0.999), weight_decay=0.01)

The library must be built first (``python -m orthogonalized_momentum_optimizer_amd.build``);
importing the optimizer never falls back to another implementation.
"""
from ._lib import MuonError  # noqa: F401
from .optim import (  # noqa: F401
    CautiousAdam,
    Muon,
    MuonPlan,
    cautious_adam_step,
    make_adam_config,
    make_config,
    zeropower_via_newtonschulz5,
)
