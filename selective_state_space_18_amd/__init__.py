"""libssmscan for AMD Instinct MI355X: selective state-space scan and decode step.

The compute path is the HIP library ``libssmscan.so`` (C ABI in
``include/ssmscan.h``); ``ssmscan`` is its Python binding.  Importing the
binding does not load the library; the first call does, and fails loudly if
the library has not been built.
"""
from . import ssmscan  # noqa: F401
from .ssmscan import scan_fwd, step, SSMError  # noqa: F401

__version__ = "1.0.0"
