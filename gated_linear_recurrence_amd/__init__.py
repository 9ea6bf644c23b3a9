"""MI355X-native (gfx950) RG-LRU recurrent-block path: prefill, decode and conv-state update.

The compute runs in librglru.so (hand-written HIP, see ``csrc/``); ``binding`` is a thin
ctypes layer with the same names as the C ABI in ``include/rglru.h``.  ``synth`` draws the
seeded synthetic inputs.
"""
from .binding import (Params, RglruError, Workspace, conv1d_state_update, load_library,  # noqa: F401
                      make_decode_workspace, make_workspace, rglru_decode_step,
                      rglru_decode_workspace_bytes, rglru_prefill, rglru_prefill_workspace_bytes,
                      rglru_prefill_workspace_init)
