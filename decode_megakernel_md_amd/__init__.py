"""MI355X decode megakernel: C-ABI library (libmd.so) plus a thin binding.

The hot path -- one persistent gfx950 kernel per decode step -- lives in
csrc/; this package only marshals arguments and owns device buffers through
PyTorch.  There is no CPU fallback: without libmd.so every entry raises."""
from ._lib import MdConfig, MdError, check, config_from, lib, weight_inventory  # noqa: F401
