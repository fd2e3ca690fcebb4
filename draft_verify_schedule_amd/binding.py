"""ctypes binding of libdspark (argument marshalling only).

Each function takes torch tensors on the GPU, checks dtype / shape /
contiguity, allocates the outputs and the workspace if the caller passes
none, and calls the C entry point of the same name on the current torch
stream.  Every step of the method runs in the library's HIP kernels.
"""
import ctypes
import os

import torch

from ._build import lib_path as _lib_path

DSPARK_F32 = 0
DSPARK_BF16 = 1
DSPARK_SCHED_EARLY_STOP = 0
DSPARK_SCHED_GLOBAL = 1
DSPARK_SCHED_TOPK = 2

_lib = None


class DSparkError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.dspark_status_string(status).decode() if _lib is not None else str(status)
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


def library_path():
    return _lib_path()


def load_library():
    """Load libdspark.so from the package's lib/ folder (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_path()
    if not os.path.exists(path):
        raise RuntimeError("libdspark.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    c_int, c_size, c_u64, vp, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_float
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_status_string.argtypes = [c_int]
    lib.dspark_version.restype = c_int
    lib.dspark_build_id.restype = ctypes.c_char_p
    lib.dspark_markov_draft_workspace_bytes.restype = c_size
    lib.dspark_markov_draft_workspace_bytes.argtypes = [c_int] * 4
    lib.dspark_markov_draft.restype = c_int
    lib.dspark_markov_draft.argtypes = [c_int, c_int, c_int, c_int, c_float, vp, c_int, vp, vp, vp, vp,
                                        c_u64, c_u64, vp, vp, vp, vp, c_size, vp]
    lib.dspark_markov_draft_with_confidence.restype = c_int
    lib.dspark_markov_draft_with_confidence.argtypes = [c_int, c_int, c_int, c_int, c_float, vp, c_int, vp, vp, vp,
                                                        vp, c_u64, c_u64, vp, vp, vp, c_int, vp, c_int, vp, vp,
                                                        c_float, vp, vp, vp, vp, c_size, vp]
    lib.dspark_markov_w2_frag_bytes.restype = c_size
    lib.dspark_markov_w2_frag_bytes.argtypes = [c_int, c_int]
    lib.dspark_markov_prepare_w2.restype = c_int
    lib.dspark_markov_prepare_w2.argtypes = [c_int, c_int, vp, vp, c_size, vp]
    lib.dspark_rnn_w2_f16_bytes.restype = c_size
    lib.dspark_rnn_w2_f16_bytes.argtypes = [c_int, c_int]
    lib.dspark_rnn_prepare_w2.restype = c_int
    lib.dspark_rnn_prepare_w2.argtypes = [c_int, c_int, vp, vp, c_size, vp]
    lib.dspark_schedule.restype = c_int
    lib.dspark_schedule_workspace_bytes.restype = c_size
    lib.dspark_schedule_workspace_bytes.argtypes = [c_int] * 2
    lib.dspark_schedule.argtypes = [c_int, c_int, vp, vp, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, c_size, vp]
    lib.dspark_schedule_noalloc.restype = c_int
    lib.dspark_schedule_noalloc.argtypes = [c_int, c_int, vp, vp, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp]
    lib.dspark_schedule_async.restype = c_int
    lib.dspark_schedule_async.argtypes = [c_int, c_int, vp, vp, c_int, vp, vp, vp, vp, vp, vp, vp, c_size, vp]
    lib.dspark_verify_workspace_bytes.restype = c_size
    lib.dspark_verify_workspace_bytes.argtypes = [c_int] * 5
    lib.dspark_verify.restype = c_int
    lib.dspark_verify.argtypes = [c_int, c_int, c_int, c_float, vp, c_int, c_int, vp, vp, c_int, vp, vp, vp,
                                  c_int, vp, vp, vp, vp, c_u64, c_u64, vp, vp, vp, vp, c_size, vp]
    lib.dspark_acceptance_label_workspace_bytes.restype = c_size
    lib.dspark_acceptance_label_workspace_bytes.argtypes = [c_int] * 4
    lib.dspark_acceptance_label.restype = c_int
    lib.dspark_acceptance_label.argtypes = [c_int, c_int, c_int, c_float, vp, c_int, vp, c_int, vp, vp, vp, c_int,
                                            vp, vp, vp, vp, vp, c_size, vp]
    lib.dspark_rnn_draft_workspace_bytes.restype = c_size
    lib.dspark_rnn_draft_workspace_bytes.argtypes = [c_int] * 5
    lib.dspark_rnn_draft.restype = c_int
    lib.dspark_rnn_draft.argtypes = [c_int, c_int, c_int, c_int, c_int, c_float, vp, c_int, vp, c_int, vp, vp, vp,
                                     vp, vp, c_u64, c_u64, vp, vp, vp, vp, vp, c_size, vp]
    lib.dspark_rnn_verify_workspace_bytes.restype = c_size
    lib.dspark_rnn_verify_workspace_bytes.argtypes = [c_int] * 5
    lib.dspark_rnn_acceptance_label_workspace_bytes.restype = c_size
    lib.dspark_rnn_acceptance_label_workspace_bytes.argtypes = [c_int] * 4
    lib.dspark_rnn_verify.restype = c_int
    lib.dspark_rnn_verify.argtypes = [c_int, c_int, c_int, c_float, vp, c_int, c_int, vp, vp, c_int, vp, vp, vp,
                                      c_int, vp, vp, vp, vp, c_u64, c_u64, vp, vp, vp, vp, c_size, vp]
    lib.dspark_rnn_acceptance_label.restype = c_int
    lib.dspark_rnn_acceptance_label.argtypes = [c_int, c_int, c_int, c_float, vp, c_int, vp, c_int, vp, vp, vp,
                                                c_int, vp, vp, vp, vp, vp, c_size, vp]
    lib.dspark_confidence_head.restype = c_int
    lib.dspark_confidence_head.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, c_int, vp, vp, c_float, vp, vp, vp,
                                           vp, vp, vp, vp]
    lib.dspark_sts_fit_workspace_bytes.restype = c_size
    lib.dspark_sts_fit_workspace_bytes.argtypes = [c_int] * 3
    lib.dspark_sts_fit.restype = c_int
    lib.dspark_sts_fit.argtypes = [c_int, c_int, vp, vp, c_int, vp, c_int, vp, vp, vp, c_size, vp]
    lib.dspark_uniforms.restype = c_int
    lib.dspark_uniforms.argtypes = [c_u64, c_u64, c_int, c_int, c_int, vp, vp]
    lib.dspark_profiler_enable.restype = c_int
    lib.dspark_profiler_enable.argtypes = [c_int]
    lib.dspark_profiler_reset.restype = c_int
    lib.dspark_profiler_read.restype = c_int
    lib.dspark_profiler_read.argtypes = [c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    _lib = lib
    return lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DSPARK_F32
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    raise TypeError("logits must be float32 or bfloat16, got %s" % t.dtype)


def _check(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _workspace(nbytes, device):
    # torch's caching allocator returns 256-byte aligned blocks on ROCm
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dspark_status_string(status):
    return load_library().dspark_status_string(int(status)).decode()


def dspark_version():
    return load_library().dspark_version()


def dspark_build_id():
    """Hash of the sources the loaded library was built from."""
    return load_library().dspark_build_id().decode()


def dspark_markov_draft_workspace_bytes(B, K, V, r):
    return load_library().dspark_markov_draft_workspace_bytes(B, K, V, r)


def dspark_verify_workspace_bytes(R, K, V, r, N):
    return load_library().dspark_verify_workspace_bytes(R, K, V, r, N)


def dspark_markov_w2_frag_bytes(V, r):
    return load_library().dspark_markov_w2_frag_bytes(V, r)


def dspark_markov_prepare_w2(W2, out=None):
    """The fragment-ordered copy of W2 ([V, r] bf16, column-major r x V) that
    the bias MFMAs read, made once per weight load; pass it as w2f to the
    draft, verify and label calls.  Returns a uint8 GPU tensor."""
    lib = load_library()
    V, r = W2.shape
    _check(W2, "W2", torch.bfloat16)
    nbytes = lib.dspark_markov_w2_frag_bytes(V, r)
    if out is None:
        out = _workspace(nbytes, W2.device)
    st = lib.dspark_markov_prepare_w2(V, r, _ptr(W2), _ptr(out), out.numel() * out.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_markov_prepare_w2", st)
    return out


def dspark_rnn_w2_f16_bytes(V, r):
    return load_library().dspark_rnn_w2_f16_bytes(V, r)


def dspark_rnn_prepare_w2(W2, out=None):
    """The RNN head's fp16 fragment-ordered copy of W2 ([V, r] bf16), made once;
    pass it as w2h to the RNN calls.  Returns a uint8 GPU tensor."""
    lib = load_library()
    V, r = W2.shape
    _check(W2, "W2", torch.bfloat16)
    nbytes = lib.dspark_rnn_w2_f16_bytes(V, r)
    if out is None:
        out = _workspace(nbytes, W2.device)
    st = lib.dspark_rnn_prepare_w2(V, r, _ptr(W2), _ptr(out), out.numel() * out.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_rnn_prepare_w2", st)
    return out


def dspark_markov_draft(U, W1, W2, x0, temperature, seed, step, out=None, workspace=None, w2f=None):
    """Sequential Markov-head draft.

    U [B, K, V] f32/bf16; W1 [V, r] bf16; W2 the r x V factor in column-major
    storage, i.e. a [V, r] bf16 tensor whose row v produces logit v; x0 [B]
    int32.  W1 = W2 = None means no Markov head (r = 0).  w2f: the copy made
    by dspark_markov_prepare_w2 (else the call makes one in its workspace).
    Returns (x [B, K] int32, q_tok [B, K] f32, lse [B, K] f32).
    """
    lib = load_library()
    B, K, V = U.shape
    _check(U, "U")
    r = 0
    if W1 is not None or W2 is not None:
        r = W1.shape[1]
        _check(W1, "W1", torch.bfloat16, (V, r))
        _check(W2, "W2", torch.bfloat16, (V, r))
    _check(x0, "x0", torch.int32, (B,))
    dev = U.device
    if out is None:
        out = (torch.empty((B, K), dtype=torch.int32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev))
    x, q, lse = out
    need = lib.dspark_markov_draft_workspace_bytes(B, K, V, r)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_markov_draft(B, K, V, r, float(temperature), _ptr(U), _dtype_code(U), _ptr(W1), _ptr(W2),
                                 _ptr(w2f), _ptr(x0), int(seed), int(step), _ptr(x), _ptr(q), _ptr(lse),
                                 _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_markov_draft", st)
    return x, q, lse


def dspark_markov_draft_with_confidence(U, W1, W2, x0, temperature, seed, step, H, w_h, w_e, bias,
                                        sts_temperature=None, out=None, workspace=None, w2f=None, logits_out=False):
    """dspark_markov_draft plus the confidence head of every position,
    evaluated inside the draft.  Arguments as for dspark_markov_draft, then
    H [B, K, d] f32/bf16, w_h [d] f32, w_e [r] f32 (or None when W1 is None),
    bias, sts_temperature [K] f32 or None.
    Returns (x, q_tok, lse, c) [B, K], and the head's logits when logits_out
    (True, or a [B, K] f32 tensor to write them into).
    """
    lib = load_library()
    B, K, V = U.shape
    _check(U, "U")
    r = 0
    if W1 is not None or W2 is not None:
        r = W1.shape[1]
        _check(W1, "W1", torch.bfloat16, (V, r))
        _check(W2, "W2", torch.bfloat16, (V, r))
        _check(w_e, "w_e", torch.float32, (r,))
    _check(x0, "x0", torch.int32, (B,))
    _check(H, "H")
    d = H.shape[2]
    _check(H, "H", None, (B, K, d))
    _check(w_h, "w_h", torch.float32, (d,))
    if sts_temperature is not None:
        _check(sts_temperature, "sts_temperature", torch.float32, (K,))
    dev = U.device
    if out is None:
        out = (torch.empty((B, K), dtype=torch.int32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev))
    x, q, lse, c = out
    if isinstance(logits_out, torch.Tensor):
        _check(logits_out, "logits_out", torch.float32, (B, K))
        z = logits_out
    else:
        z = torch.empty((B, K), dtype=torch.float32, device=dev) if logits_out else None
    need = lib.dspark_markov_draft_workspace_bytes(B, K, V, r)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_markov_draft_with_confidence(
        B, K, V, r, float(temperature), _ptr(U), _dtype_code(U), _ptr(W1), _ptr(W2), _ptr(w2f), _ptr(x0),
        int(seed), int(step), _ptr(x), _ptr(q), _ptr(lse), d, _ptr(H), _dtype_code(H), _ptr(w_h),
        _ptr(w_e if r > 0 else None), float(bias), _ptr(sts_temperature), _ptr(c), _ptr(z), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_markov_draft_with_confidence", st)
    return (x, q, lse, c, z) if z is not None else (x, q, lse, c)


def dspark_schedule_workspace_bytes(R, K):
    return load_library().dspark_schedule_workspace_bytes(R, K)


def dspark_schedule(c, sps, mode=DSPARK_SCHED_EARLY_STOP, capacity=0, out=None, workspace=None):
    """Algorithm 1 on confidences c [R, K] f32 and the SPS table sps [L] f64.

    Returns dict with a [R, K] f32, ell [R] int32, cu_seqlens [R+1] int32,
    n_admitted [1] int32 and theta [1] f64 (all on the GPU).
    """
    lib = load_library()
    R, K = c.shape
    _check(c, "c", torch.float32)
    _check(sps, "sps", torch.float64)
    dev = c.device
    if out is None:
        out = {"a": torch.empty((R, K), dtype=torch.float32, device=dev),
               "ell": torch.empty(R, dtype=torch.int32, device=dev),
               "cu_seqlens": torch.empty(R + 1, dtype=torch.int32, device=dev),
               "n_admitted": torch.empty(1, dtype=torch.int32, device=dev),
               "theta": torch.empty(1, dtype=torch.float64, device=dev)}
    need = lib.dspark_schedule_workspace_bytes(R, K)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_schedule(R, K, _ptr(c), _ptr(sps), sps.numel(), int(mode), int(capacity), _ptr(out["a"]),
                             _ptr(out["ell"]), _ptr(out["cu_seqlens"]), _ptr(out["n_admitted"]),
                             _ptr(out["theta"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream())
    if st != 0:
        raise DSparkError("dspark_schedule", st)
    return out


def dspark_schedule_noalloc(c, sps, mode=DSPARK_SCHED_EARLY_STOP, capacity=0, out=None):
    """dspark_schedule with the sorted keys in the library's own device array
    (no workspace, nothing allocated by the library; pass `out` to allocate
    nothing here either).  Same results as dspark_schedule; calls that
    overlap on one GPU race on the shared array."""
    lib = load_library()
    R, K = c.shape
    _check(c, "c", torch.float32)
    _check(sps, "sps", torch.float64)
    dev = c.device
    if out is None:
        out = {"a": torch.empty((R, K), dtype=torch.float32, device=dev),
               "ell": torch.empty(R, dtype=torch.int32, device=dev),
               "cu_seqlens": torch.empty(R + 1, dtype=torch.int32, device=dev),
               "n_admitted": torch.empty(1, dtype=torch.int32, device=dev),
               "theta": torch.empty(1, dtype=torch.float64, device=dev)}
    st = lib.dspark_schedule_noalloc(R, K, _ptr(c), _ptr(sps), sps.numel(), int(mode), int(capacity), _ptr(out["a"]),
                                     _ptr(out["ell"]), _ptr(out["cu_seqlens"]), _ptr(out["n_admitted"]),
                                     _ptr(out["theta"]), _stream())
    if st != 0:
        raise DSparkError("dspark_schedule_noalloc", st)
    return out


def dspark_schedule_async(c, sps, capacity, out=None, workspace=None):
    """Top-capacity admission of c [R, K] with the capacity read on the device
    (capacity: int32 tensor of one element, e.g. the n_admitted of an earlier
    GLOBAL schedule).  Returns the same dict as dspark_schedule."""
    lib = load_library()
    R, K = c.shape
    _check(c, "c", torch.float32)
    _check(sps, "sps", torch.float64)
    _check(capacity, "capacity", torch.int32)
    if capacity.numel() < 1:
        raise ValueError("capacity: one int32 element expected")
    dev = c.device
    if out is None:
        out = {"a": torch.empty((R, K), dtype=torch.float32, device=dev),
               "ell": torch.empty(R, dtype=torch.int32, device=dev),
               "cu_seqlens": torch.empty(R + 1, dtype=torch.int32, device=dev),
               "n_admitted": torch.empty(1, dtype=torch.int32, device=dev),
               "theta": torch.empty(1, dtype=torch.float64, device=dev)}
    need = lib.dspark_schedule_workspace_bytes(R, K)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_schedule_async(R, K, _ptr(c), _ptr(sps), sps.numel(), _ptr(capacity), _ptr(out["a"]),
                                   _ptr(out["ell"]), _ptr(out["cu_seqlens"]), _ptr(out["n_admitted"]),
                                   _ptr(out["theta"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream())
    if st != 0:
        raise DSparkError("dspark_schedule_async", st)
    return out


def _margin_out(min_margin, R, dev):
    if min_margin is None or min_margin is False:
        return None
    if min_margin is True:
        return torch.empty(R, dtype=torch.float32, device=dev)
    _check(min_margin, "min_margin", torch.float32, (R,))
    return min_margin


def dspark_verify(P, cu_seqlens, D, W1, W2, x0, x, q_tok, lse_d, temperature, seed, step, out=None,
                  workspace=None, w2f=None, min_margin=None):
    """Rejection-sampling verification over the flat batch.

    P [N, V] target logits; cu_seqlens [R+1] int32; D [R, K, V] draft base
    logits; W1 / W2 as for dspark_markov_draft (or None); x0 [R]; x [R, K]
    the drafted tokens; q_tok, lse_d [R, K] from the draft, or None (then
    recomputed from D and the bias); w2f as for dspark_markov_draft.
    min_margin: True (or an [R] f32 tensor) to also get each request's
    smallest decision margin.
    Returns (n_acc [R] int32, tok [R] int32), plus the margins when asked.
    """
    lib = load_library()
    N, V = P.shape
    R, K, V2 = D.shape
    if V2 != V:
        raise ValueError("P and D disagree on V")
    _check(P, "P")
    _check(D, "D")
    _check(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,))
    _check(x0, "x0", torch.int32, (R,))
    _check(x, "x", torch.int32, (R, K))
    r = 0
    if W1 is not None or W2 is not None:
        r = W1.shape[1]
        _check(W1, "W1", torch.bfloat16, (V, r))
        _check(W2, "W2", torch.bfloat16, (V, r))
    if q_tok is not None:
        _check(q_tok, "q_tok", torch.float32, (R, K))
    if lse_d is not None:
        _check(lse_d, "lse_d", torch.float32, (R, K))
    dev = P.device
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev))
    n_acc, tok = out
    mm = _margin_out(min_margin, R, dev)
    need = lib.dspark_verify_workspace_bytes(R, K, V, r, N)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_verify(R, K, V, float(temperature), _ptr(P), _dtype_code(P), N, _ptr(cu_seqlens), _ptr(D),
                           _dtype_code(D), _ptr(W1), _ptr(W2), _ptr(w2f), r, _ptr(x0), _ptr(x), _ptr(q_tok),
                           _ptr(lse_d), int(seed), int(step), _ptr(n_acc), _ptr(tok), _ptr(mm), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_verify", st)
    return (n_acc, tok) if mm is None else (n_acc, tok, mm)


def dspark_acceptance_label_workspace_bytes(B, K, V, r):
    return load_library().dspark_acceptance_label_workspace_bytes(B, K, V, r)


def dspark_acceptance_label(P, D, W1, W2, x0, x, lse_d, temperature, out=None, workspace=None, w2f=None):
    """Analytic acceptance probability c*[r, k] = 1 - TV(q_{r,k}, p_{r,k}).

    P [B, K, V] target logits (row (r, k) judges draft position k+1); D
    [B, K, V] draft base logits; W1 / W2 as for dspark_markov_draft (or None);
    x0 [B]; x, lse_d [B, K] from dspark_markov_draft.  Returns c [B, K] f32.
    """
    lib = load_library()
    B, K, V = D.shape
    _check(P, "P", shape=(B, K, V))
    _check(D, "D")
    r = 0
    if W1 is not None or W2 is not None:
        r = W1.shape[1]
        _check(W1, "W1", torch.bfloat16, (V, r))
        _check(W2, "W2", torch.bfloat16, (V, r))
    _check(x0, "x0", torch.int32, (B,))
    _check(x, "x", torch.int32, (B, K))
    _check(lse_d, "lse_d", torch.float32, (B, K))
    dev = D.device
    if out is None:
        out = torch.empty((B, K), dtype=torch.float32, device=dev)
    need = lib.dspark_acceptance_label_workspace_bytes(B, K, V, r)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_acceptance_label(B, K, V, float(temperature), _ptr(P), _dtype_code(P), _ptr(D), _dtype_code(D),
                                     _ptr(W1), _ptr(W2), _ptr(w2f), r, _ptr(x0), _ptr(x), _ptr(lse_d), _ptr(out),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_acceptance_label", st)
    return out


def dspark_rnn_draft_workspace_bytes(B, K, V, r, d):
    return load_library().dspark_rnn_draft_workspace_bytes(B, K, V, r, d)


def dspark_rnn_draft(U, H, W, W1, W2, x0, temperature, seed, step, out=None, workspace=None, w2h=None):
    """Sequential RNN-head draft.

    U [B, K, V] f32/bf16 base logits; H [B, K, d] bf16 hidden states; W
    [3r, 2r + d] bf16 (gate, candidate, output rows); W1 [V, r] bf16; W2 the
    r x V factor column-major ([V, r] bf16); x0 [B] int32.
    Returns (x [B, K] int32, q_tok [B, K] f32, lse [B, K] f32, O [B, K, r] f32).
    """
    lib = load_library()
    B, K, V = U.shape
    _check(U, "U")
    r = W1.shape[1]
    d = H.shape[2]
    _check(H, "H", torch.bfloat16, (B, K, d))
    _check(W, "W", torch.bfloat16, (3 * r, 2 * r + d))
    _check(W1, "W1", torch.bfloat16, (V, r))
    _check(W2, "W2", torch.bfloat16, (V, r))
    _check(x0, "x0", torch.int32, (B,))
    dev = U.device
    if out is None:
        out = (torch.empty((B, K), dtype=torch.int32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K, r), dtype=torch.float32, device=dev))
    x, q, lse, O = out
    need = lib.dspark_rnn_draft_workspace_bytes(B, K, V, r, d)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_rnn_draft(B, K, V, r, d, float(temperature), _ptr(U), _dtype_code(U), _ptr(H), DSPARK_BF16,
                              _ptr(W), _ptr(W1), _ptr(W2), _ptr(w2h), _ptr(x0), int(seed), int(step), _ptr(x), _ptr(q),
                              _ptr(lse), _ptr(O), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream())
    if st != 0:
        raise DSparkError("dspark_rnn_draft", st)
    return x, q, lse, O


def dspark_rnn_verify_workspace_bytes(R, K, V, r, N):
    return load_library().dspark_rnn_verify_workspace_bytes(R, K, V, r, N)


def dspark_rnn_acceptance_label_workspace_bytes(B, K, V, r):
    return load_library().dspark_rnn_acceptance_label_workspace_bytes(B, K, V, r)


def dspark_rnn_verify(P, cu_seqlens, D, O, W2, x0, x, q_tok, lse_d, temperature, seed, step, out=None,
                      workspace=None, w2h=None, min_margin=None):
    """Verification of RNN-head drafts: as dspark_verify, with the draft rows'
    bias rebuilt from the output parts O [R, K, r] f32 returned by
    dspark_rnn_draft.  Returns (n_acc [R] int32, tok [R] int32)."""
    lib = load_library()
    N, V = P.shape
    R, K, V2 = D.shape
    if V2 != V:
        raise ValueError("P and D disagree on V")
    r = O.shape[2]
    _check(P, "P")
    _check(D, "D")
    _check(O, "O", torch.float32, (R, K, r))
    _check(W2, "W2", torch.bfloat16, (V, r))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,))
    _check(x0, "x0", torch.int32, (R,))
    _check(x, "x", torch.int32, (R, K))
    if q_tok is not None:
        _check(q_tok, "q_tok", torch.float32, (R, K))
    if lse_d is not None:
        _check(lse_d, "lse_d", torch.float32, (R, K))
    dev = P.device
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev))
    n_acc, tok = out
    need = lib.dspark_rnn_verify_workspace_bytes(R, K, V, r, N)
    if workspace is None:
        workspace = _workspace(need, dev)
    mm = _margin_out(min_margin, R, dev)
    st = lib.dspark_rnn_verify(R, K, V, float(temperature), _ptr(P), _dtype_code(P), N, _ptr(cu_seqlens), _ptr(D),
                               _dtype_code(D), _ptr(O), _ptr(W2), _ptr(w2h), r, _ptr(x0), _ptr(x), _ptr(q_tok),
                               _ptr(lse_d), int(seed), int(step), _ptr(n_acc), _ptr(tok), _ptr(mm), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_rnn_verify", st)
    return (n_acc, tok) if mm is None else (n_acc, tok, mm)


def dspark_rnn_acceptance_label(P, D, O, W2, x0, x, lse_d, temperature, out=None, workspace=None, w2h=None):
    """Acceptance label of RNN-head drafts: as dspark_acceptance_label, with
    the output parts O [B, K, r] f32 in place of the Markov embeddings."""
    lib = load_library()
    B, K, V = D.shape
    r = O.shape[2]
    _check(P, "P", shape=(B, K, V))
    _check(D, "D")
    _check(O, "O", torch.float32, (B, K, r))
    _check(W2, "W2", torch.bfloat16, (V, r))
    _check(x0, "x0", torch.int32, (B,))
    _check(x, "x", torch.int32, (B, K))
    _check(lse_d, "lse_d", torch.float32, (B, K))
    dev = D.device
    if out is None:
        out = torch.empty((B, K), dtype=torch.float32, device=dev)
    need = lib.dspark_rnn_acceptance_label_workspace_bytes(B, K, V, r)
    if workspace is None:
        workspace = _workspace(need, dev)
    st = lib.dspark_rnn_acceptance_label(B, K, V, float(temperature), _ptr(P), _dtype_code(P), _ptr(D),
                                         _dtype_code(D), _ptr(O), _ptr(W2), _ptr(w2h), r, _ptr(x0), _ptr(x),
                                         _ptr(lse_d),
                                         _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream())
    if st != 0:
        raise DSparkError("dspark_rnn_acceptance_label", st)
    return out


def dspark_confidence_head(H, w_h, w_e, bias, W1, x0, x, V, sts_temperature=None, out=None, logits_out=False):
    """Confidence head c[r, k] = sigmoid((w_h . H[r, k] + w_e . W1[x_{k-1}] + bias) / T_k).

    H [B, K, d] f32/bf16; w_h [d] f32; w_e [r] f32 and W1 [V, r] bf16 (or
    None); x0 [B], x [B, K] int32; sts_temperature [K] f32 or None.
    Returns c [B, K] f32, and the logits [B, K] when logits_out is set.
    """
    lib = load_library()
    B, K, d = H.shape
    _check(H, "H")
    _check(w_h, "w_h", torch.float32, (d,))
    r = 0
    if W1 is not None:
        r = W1.shape[1]
        _check(W1, "W1", torch.bfloat16, (V, r))
        _check(w_e, "w_e", torch.float32, (r,))
    _check(x0, "x0", torch.int32, (B,))
    _check(x, "x", torch.int32, (B, K))
    if sts_temperature is not None:
        _check(sts_temperature, "sts_temperature", torch.float32, (K,))
    c = torch.empty((B, K), dtype=torch.float32, device=H.device) if out is None else out
    z = torch.empty((B, K), dtype=torch.float32, device=H.device) if logits_out else None
    st = lib.dspark_confidence_head(B, K, int(V), d, r, _ptr(H), _dtype_code(H), _ptr(w_h), _ptr(w_e),
                                    float(bias), _ptr(W1), _ptr(x0), _ptr(x), _ptr(sts_temperature), _ptr(c),
                                    _ptr(z), _stream())
    if st != 0:
        raise DSparkError("dspark_confidence_head", st)
    return (c, z) if logits_out else c


def dspark_sts_fit_workspace_bytes(N, K, n_grid):
    return load_library().dspark_sts_fit_workspace_bytes(N, K, n_grid)


def dspark_sts_fit(logits, survived, grid, n_bins=10, workspace=None):
    """Sequential Temperature Scaling on held-out logits [N, K] f32 and
    prefix-survival labels [N, K] uint8 over the candidate temperatures
    grid [G] f32.  Returns (T [K] f32, ece [K] f32) on the GPU."""
    lib = load_library()
    N, K = logits.shape
    _check(logits, "logits", torch.float32)
    _check(survived, "survived", torch.uint8, (N, K))
    _check(grid, "grid", torch.float32)
    G = grid.numel()
    T = torch.empty(K, dtype=torch.float32, device=logits.device)
    ece = torch.empty(K, dtype=torch.float32, device=logits.device)
    need = lib.dspark_sts_fit_workspace_bytes(N, K, G)
    if workspace is None:
        workspace = _workspace(need, logits.device)
    st = lib.dspark_sts_fit(N, K, _ptr(logits), _ptr(survived), G, _ptr(grid), int(n_bins), _ptr(T), _ptr(ece),
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st != 0:
        raise DSparkError("dspark_sts_fit", st)
    return T, ece


def dspark_uniforms(seed, step, n, position, purpose, out=None):
    """u(seed, step, request i, position, purpose) for i in [0, n), float32 on the GPU."""
    lib = load_library()
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    st = lib.dspark_uniforms(int(seed), int(step), int(n), int(position), int(purpose), _ptr(out), _stream())
    if st != 0:
        raise DSparkError("dspark_uniforms", st)
    return out


def dspark_profiler_enable(on=True):
    return load_library().dspark_profiler_enable(1 if on else 0)


def dspark_profiler_reset():
    return load_library().dspark_profiler_reset()


def dspark_profiler_read():
    """{kernel name: (launches, total ms)} for the events recorded so far."""
    lib = load_library()
    n = lib.dspark_profiler_read(0, None, None, None)
    res = {}
    for i in range(n):
        name = ctypes.c_char_p()
        launches = ctypes.c_int64()
        ms = ctypes.c_double()
        if lib.dspark_profiler_read(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms)) == 0:
            res[name.value.decode()] = (launches.value, ms.value)
    return res
