"""MI355X (gfx950) Muon optimizer step: momentum, batched Newton-Schulz
orthogonalisation and decoupled weight decay, in hand-written HIP kernels
behind a C ABI (include/muon.h).

Importing the package loads nothing; the HIP library is loaded on first use
and its absence is an error (there is no fallback path).
"""
from .binding import (MUON_BF16, MUON_F32, MuonError, MuonLibraryMissing, MuonPlan,  # noqa: F401
                      AdamWGroup, adamw_step, load_library, poll_timeout, shard_update)

__all__ = ["MuonPlan", "MuonError", "MuonLibraryMissing", "load_library", "shard_update", "adamw_step", "AdamWGroup",
           "poll_timeout"]
