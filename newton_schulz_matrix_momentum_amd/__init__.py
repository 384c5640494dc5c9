"""libmuon: the Muon / MONA optimizer step on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmuon.so`` (hand-written HIP
kernels); this package is its Python binding.  PyTorch provides device memory
and streams only.
"""
from ._lib import MuonError, load, version, last_error, EXPORTS  # noqa: F401
from .api import muon_step, muon_step_static, muon_workspace_size, adamw_step, Workspace  # noqa: F401
from .optim import Muon  # noqa: F401

__all__ = ["muon_step", "muon_step_static", "muon_workspace_size", "adamw_step", "Workspace", "Muon", "MuonError", "load", "version"]
