"""DSpark draft -> schedule -> verify hot path on MI355X (gfx950).

The compute lives in libdspark.so (hand-written HIP kernels behind the C ABI
declared in include/dspark.h).  This package is a thin ctypes binding with the
same names as the C entry points; PyTorch only provides device memory and the
stream.  ``workloads`` holds the seeded synthetic input generators.

The binding is loaded on first use and raises if the library is not built:
there is no fallback path.
"""

_BINDING_NAMES = {
    "dspark_markov_draft", "dspark_markov_draft_with_confidence",
    "dspark_schedule", "dspark_schedule_async", "dspark_schedule_noalloc", "dspark_verify",
    "dspark_markov_draft_workspace_bytes", "dspark_schedule_workspace_bytes", "dspark_verify_workspace_bytes",
    "dspark_acceptance_label", "dspark_acceptance_label_workspace_bytes",
    "dspark_confidence_head", "dspark_sts_fit", "dspark_sts_fit_workspace_bytes",
    "dspark_rnn_draft", "dspark_rnn_draft_workspace_bytes", "dspark_rnn_verify", "dspark_rnn_acceptance_label",
    "dspark_rnn_verify_workspace_bytes", "dspark_rnn_acceptance_label_workspace_bytes",
    "dspark_status_string", "dspark_version", "dspark_build_id", "dspark_uniforms",
    "dspark_markov_prepare_w2", "dspark_markov_w2_frag_bytes", "dspark_rnn_prepare_w2", "dspark_rnn_w2_f16_bytes",
    "dspark_profiler_enable", "dspark_profiler_reset", "dspark_profiler_read",
    "DSparkError", "load_library", "library_path",
    "DSPARK_F32", "DSPARK_BF16",
    "DSPARK_SCHED_EARLY_STOP", "DSPARK_SCHED_GLOBAL", "DSPARK_SCHED_TOPK",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = sorted(_BINDING_NAMES)
