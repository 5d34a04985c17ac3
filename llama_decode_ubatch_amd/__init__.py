"""MI355X (gfx950) implementation of one llama_decode step over ubatches with
a KV cache.  The compute runs in libubd.so (HIP kernels + C++ runtime, C ABI
in include/ubd.h); this package only binds it."""
from .binding import (Model, Context, Planner, Sampler, load_library, last_error,  # noqa: F401
                      UBD_OK, UBD_NO_KV_SLOT, UBD_ABORTED, UBD_INVALID,
                      UBD_ALLOC_FAILED, UBD_COMPUTE_FAILED, UBD_MAX_SEQ, LIB_PATH)
