"""MI355X-native hot path of speculative decoding: a verify forward pass over
K+1 positions with weights streamed from HBM once, the exact accept/reject
rule, and a graph-captured draft loop, behind the C ABI of libspec.so."""
from .binding import (  # noqa: F401
    Ctx, Mat, SpecError, SPEC_OK, SPEC_ERR_ARG, SPEC_ERR_CAPACITY, SPEC_ERR_STATE, SPEC_ERR_OOM,
    SPEC_ERR_HIP, SPEC_K_MAX, SPEC_AR_K_MAX, EXPORTED, LIBPATH,
    spec_init, spec_draft, spec_draft_ngram, spec_heads_init, spec_draft_heads, spec_verify, spec_commit, spec_destroy, spec_last_error, spec_sync,
    spec_stream, spec_get_state, spec_get_history, spec_kernel_times, spec_set_profiling, spec_head_time,
    spec_accept_reject, spec_accept_reject_noalloc, spec_expected_tokens, spec_alpha_from_tokens,
    spec_choose_k,
    spec_mat_create, spec_mat_mul, spec_mat_destroy, spec_read_ceiling,
    Batch, SPEC_BATCH_MAX_SEQ, spec_batch_init, spec_batch_draft_ngram, spec_batch_verify,
    spec_batch_commit, spec_batch_sync, spec_batch_get_state, spec_batch_get_history,
    spec_batch_last_error, spec_batch_destroy,
)
