"""CPU oracle of the TensorGRaD step. TEST INFRASTRUCTURE ONLY: imported solely by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg; never by the library."""
from .tgrad_oracle import *  # noqa: F401,F403
from .tgrad_oracle import TGradOracle, topk_keys, select_omega, gather, residual, gram, \
    hosvd_factor, project, reconstruct, mode_product, unfold, adam, adam_consts, decode, \
    encode, real_view, canonicalize_columns, lowrank_param_count, dense_adam_reference  # noqa: F401
