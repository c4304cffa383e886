"""MI355X (gfx950) staged single-token decode: a C-ABI library (liblps) of
hand-written HIP kernels, with a thin ctypes binding and a decode driver that
uses PyTorch only for device memory and streams."""
from . import _lib as lps  # noqa: F401
