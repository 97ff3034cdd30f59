"""MI355X (gfx950) hybrid attention of Hybrid Forcing: HIP kernels behind a C ABI.

``binding`` exposes the C entry points of include/hf.h under the same names;
``HybridAttentionState`` wraps them for PyTorch tensors. Importing this package
loads libhf.so and fails loudly if it has not been built.
"""

from .binding import (  # noqa: F401
    HF_BF16, HF_F32, HF_OK, HF_ERR_INVALID_ARG, HF_ERR_UNSUPPORTED, HF_ERR_STATE, HF_ERR_HIP,
    HfError, hf_config, hf_workspace_bytes, hf_state_init, hf_absorb_evicted, hf_attend_chunk,
    hf_absorb_and_attend, hf_attend_chunk_cached, hf_absorb_and_attend_cached,
    hf_absorb_and_attend_ahead, hf_absorb_flush, hf_pending_ev, hf_key_cache_reset,
    hf_window_attach, hf_window_begin_chunk, hf_window_attend, hf_window_range,
    hf_block_scores, hf_backward_workspace_bytes, hf_attend_backward, hf_absorb_backward,
    hf_attend_ragged, hf_rope, hf_rope_workspace_bytes, hf_set_rope, hf_attend_chunk_noalloc, hf_profile_start, hf_profile_stop, hf_next_ev_index,
    hf_state_destroy, hf_status_string, library_path)
from .state import HybridAttentionState, window_frames  # noqa: F401
