"""libmuon: the Muon update (momentum, Newton-Schulz orthogonalisation, apply)
as hand-written HIP kernels for AMD Instinct MI355X (gfx950).

The Python surface is a thin ctypes binding of the C ABI in include/muon.h;
see binding.py.  Build the library with `python -m spectral_optimizer_ssm_amd.build`.
"""
from .binding import (MUON_BF16, MUON_F32, MUON_NS_ACCUMULATE, MUON_NS_AUTO, MUON_NS_ITERATE,  # noqa: F401
                      AdamwTensors, MuonError, MuonGroup, lib, make_cfg, muon_adamw, muon_ns_batched_small,
                      muon_ns_factored, muon_ssm_momentum, muon_ns_orthogonalize, muon_ns_orthogonalize_noalloc, muon_query_flags,
                      muon_spectral_diag,
                      muon_ns_workspace_size, muon_step, muon_step_phases, muon_step_workspace_size,
                      muon_version, status_string)
