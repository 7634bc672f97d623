"""MI355X-native DSA lightning-indexer hot path.

The work runs in hand-written HIP kernels for gfx950 behind a C-ABI shared
library (``include/dsa_indexer.h``); ``dsa_lightning_indexer_amd.binding``
marshals torch tensors into that ABI.  Importing this package does not load
the library; the binding loads it on first use and raises if it is missing.
"""

__all__ = ["binding", "synth"]
