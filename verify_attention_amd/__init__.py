"""verify_attention_amd: block-query draft/verify attention over a paged KV
cache plus the speculative accept epilogue, as hand-written HIP for MI355X
(gfx950) behind a C ABI (include/specattn.h). This package is the thin Python
binding (argument marshalling only) and the seeded input generator."""
from .binding import *  # noqa: F401,F403
from .binding import load, lib_path  # noqa: F401
