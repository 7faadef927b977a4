"""ReplaySSM decode hot path for AMD MI355X (gfx950).

The SSM state of every (sequence, head) is kept as a read-only fp32 checkpoint plus a ring of
the last W tokens' inputs; decode tokens replay the ring against the checkpoint, a full ring is
folded into a new checkpoint, and speculative drafts are committed or rolled back by moving a
pointer. The kernels live in librssm.so (C ABI: include/rssm.h); this package is its ctypes
binding.
"""
from .binding import (Context, RssmError, load_library, make_config, make_inputs, step_baseline,
                      RSSM_MAMBA2, RSSM_GDN, RSSM_F_BF16_READ, RSSM_F_STORE_C,
                      RSSM_DEV_COMMIT_RANGE, RSSM_DEV_ROLLBACK_RANGE, EXPORTS)

__all__ = ["Context", "RssmError", "load_library", "make_config", "make_inputs", "step_baseline",
           "RSSM_MAMBA2", "RSSM_GDN", "RSSM_F_BF16_READ", "RSSM_F_STORE_C",
           "RSSM_DEV_COMMIT_RANGE", "RSSM_DEV_ROLLBACK_RANGE", "EXPORTS"]
