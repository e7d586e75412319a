"""CPU oracle for one block-diffusion drafting step (test infrastructure).

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
the oracle imports nothing from the product path.

See ``oracle.dflash_ref`` for the definitions and the passages they follow.
"""
from .dflash_ref import *  # noqa: F401,F403
