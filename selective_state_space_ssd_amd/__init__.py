"""MI355X (gfx950) HIP library for the Mamba-2 SSD hot path.

Two operations behind a C ABI (``include/ssd_mi355x.h``):

* ``ssd_chunk_scan_fwd`` -- the SSD chunked selective scan (four-step block
  decomposition of the semiseparable sequence map).
* ``ssd_verify_step`` -- the K-token recurrent update a target model runs when it
  verifies speculative-decoding drafts, keeping the state at the accepted
  position (and optionally at every position).

The Python binding (``selective_state_space_ssd_amd.binding``) only marshals
torch tensors into the C calls; every step runs in the HIP kernels.  Importing
this package loads nothing; the shared library is opened on first use and a
missing library is an error, never a fallback.
"""

__version__ = "0.1.0"
