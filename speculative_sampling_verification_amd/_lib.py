"""ctypes binding to libspecverify.so.

Argument marshalling only: tensors are checked for device, dtype and layout, and their
``data_ptr()`` values and torch's current HIP stream are passed to the C ABI.  Every step of
the computation runs in the library's kernels.  There is no fallback: if the library is
missing the import fails.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that the library binds to torch's HIP runtime

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libspecverify.so")

SV_OK = 0
SV_ERR_SCRATCH_TOO_SMALL = 5
NOALLOC_SCRATCH_BYTES = 64 << 20  # SPEC_VERIFY_NOALLOC_SCRATCH_BYTES
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1


class SVSampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("lenience", ctypes.c_float),
                ("mentor_kl", ctypes.c_float)]


EXPORTS = [
    "spec_verify_workspace_size", "spec_verify", "spec_verify_profiled",
    "spec_sample_workspace_size", "spec_sample",
    "spec_verify_tree_workspace_size", "spec_verify_tree", "spec_verify_tree_profiled",
    "spec_build_tree", "spec_philox_uniform", "spec_acceptance_rate", "spec_verify_rates",
    "spec_verify_presampled", "spec_verify_noalloc",
    "spec_expected_tokens",
    "spec_walltime_speedup", "spec_ops_factor", "spec_optimal_gamma",
    "spec_verify_status_string",
]


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with speculative_sampling_verification_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    psamp = ctypes.POINTER(SVSampling)
    lib.spec_verify_workspace_size.argtypes = [i32, i32, i32, i32, psamp]
    lib.spec_verify_workspace_size.restype = sz
    lib.spec_verify.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, psamp, vp, vp, vp, vp, vp,
                                vp, sz, vp]
    lib.spec_verify.restype = i32
    lib.spec_verify_profiled.argtypes = lib.spec_verify.argtypes + [vp, i32]
    lib.spec_verify_profiled.restype = i32
    lib.spec_verify_rates.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, psamp, vp, vp, vp,
                                      vp, vp, vp, vp, sz, vp]
    lib.spec_verify_rates.restype = i32
    lib.spec_verify_presampled.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, psamp, vp, vp, vp,
                                           vp, vp, vp, sz, vp, sz, vp]
    lib.spec_verify_presampled.restype = i32
    lib.spec_verify_noalloc.argtypes = lib.spec_verify.argtypes[:15] + [vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_sample_workspace_size.argtypes = [i32, i32, i32, psamp]
    lib.spec_sample_workspace_size.restype = sz
    lib.spec_sample.argtypes = [vp, i32, i32, i32, vp, psamp, vp, vp, sz, vp]
    lib.spec_sample.restype = i32
    lib.spec_verify_tree_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_tree_workspace_size.restype = sz
    lib.spec_verify_tree.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_tree.restype = i32
    lib.spec_verify_tree_profiled.argtypes = lib.spec_verify_tree.argtypes + [vp, i32]
    lib.spec_verify_tree_profiled.restype = i32
    lib.spec_build_tree.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.spec_build_tree.restype = i32
    u64 = ctypes.c_uint64
    lib.spec_philox_uniform.argtypes = [u64, u64, u64, ctypes.c_int64, vp, vp]
    lib.spec_philox_uniform.restype = i32
    lib.spec_acceptance_rate.argtypes = [vp, vp, i32, i32, i32, i32, i32, psamp, vp, vp, sz, vp]
    lib.spec_acceptance_rate.restype = i32
    dbl = ctypes.c_double
    lib.spec_expected_tokens.argtypes = [dbl, i32]
    lib.spec_expected_tokens.restype = dbl
    lib.spec_walltime_speedup.argtypes = [dbl, i32, dbl]
    lib.spec_walltime_speedup.restype = dbl
    lib.spec_ops_factor.argtypes = [dbl, i32, dbl]
    lib.spec_ops_factor.restype = dbl
    lib.spec_optimal_gamma.argtypes = [dbl, dbl, i32]
    lib.spec_optimal_gamma.restype = i32
    lib.spec_verify_status_string.argtypes = [i32]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    return lib


_lib = load()


def lib():
    return _lib


def status_string(code):
    return _lib.spec_verify_status_string(int(code)).decode()


class SpecVerifyError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} (status {code})")
        self.code = code


def _check(fn, code):
    if code != SV_OK:
        raise SpecVerifyError(fn, code)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def sampling(temperature=1.0, top_k=0, top_p=1.0, lenience=1.0, mentor_kl=0.0):
    return SVSampling(float(temperature), int(top_k), float(top_p), float(lenience),
                      float(mentor_kl))


_workspaces = {}
_outgrown = []  # replaced workspaces, kept alive: a captured HIP graph may still use them


def workspace(device, nbytes, stream=None):
    """A cached uint8 device buffer of at least nbytes, one per (device, stream): calls that
    share a workspace must be ordered on one stream.  Grown on demand; a buffer it replaces is
    never freed, so work already captured in a HIP graph keeps valid memory."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device.type, device.index, s.cuda_stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _outgrown.append(buf)
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


def release_workspaces(device=None):
    """Frees the cached workspaces (of one device, or of all) and the outgrown ones kept for
    captured graphs, after the device has finished the work queued on them.  A HIP graph
    captured over calls of this binding must not be replayed afterwards; the next call
    allocates afresh.  Returns the number of bytes released."""
    freed = 0
    devs = {d for (_, d, _) in _workspaces} | {b.device.index for b in _outgrown}
    for d in devs:
        if device is None or torch.device(device).index in (None, d):
            torch.cuda.synchronize(d)
    keep = {}
    for key, buf in _workspaces.items():
        if device is None or torch.device(device).index in (None, key[1]):
            freed += buf.numel()
        else:
            keep[key] = buf
    _workspaces.clear()
    _workspaces.update(keep)
    rest = []
    for buf in _outgrown:
        if device is None or torch.device(device).index in (None, buf.device.index):
            freed += buf.numel()
        else:
            rest.append(buf)
    _outgrown[:] = rest
    return freed


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def spec_verify(target_logits, draft_logits, draft_tokens, uniforms, *, temperature=1.0, top_k=0,
                top_p=1.0, lenience=1.0, mentor_kl=0.0, out=None, want_probs=True,
                want_rates=False, presampled=None, stream=None, events=None):
    """Verify-and-resample for a batch (see include/spec_verify.h).

    target_logits [B, K+1, V], draft_logits [B, K or K+1, V] (bf16 or fp32, same dtype),
    draft_tokens [B, K] int32, uniforms [B, K+1] float32, all on one GPU.
    Returns a dict: tokens [B, K+1], num_accepted [B], and if want_probs accept_prob / q_draft /
    p_draft [B, K].  ``out`` may hold preallocated tensors under the same keys.
    ``mentor_kl`` > 0 selects mentored decoding with that KL bound (needs lenience 1 and, for
    temperature > 0, top_k in 1..256).
    ``want_rates``: also return rate [B, K], the acceptance rate sum_x min(p, q/l) of each
    position (spec_verify_rates: the same results plus the rates, one pass over the logits).
    ``presampled``: the ``summary`` buffer of a spec_sample call on draft_logits viewed as
    [B*K, V] with the same sampling parameters (spec_verify_presampled: the draft rows are not
    streamed again; same results).
    ``events``: optional list of >= 2 hipEvent_t handles (ints) for per-phase timing.
    """
    dev = target_logits.device
    B, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    if K > 0:
        _need(draft_logits, "draft_logits", dev, target_logits.dtype)
        if draft_logits.dim() != 3 or draft_logits.shape[0] != B or draft_logits.shape[2] != V:
            raise ValueError("draft_logits must be [B, K or K+1, V]")
        draft_rows = draft_logits.shape[1]
        _need(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    else:
        draft_rows = 0
    _need(uniforms, "uniforms", dev, torch.float32, (B, K + 1))
    out = dict(out or {})
    if "tokens" not in out:
        out["tokens"] = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if "num_accepted" not in out:
        out["num_accepted"] = torch.empty((B,), dtype=torch.int32, device=dev)
    if want_probs:
        for k in ("accept_prob", "q_draft", "p_draft"):
            if k not in out:
                out[k] = torch.empty((B, K), dtype=torch.float32, device=dev)
    _need(out["tokens"], "out tokens", dev, torch.int32, (B, K + 1))
    _need(out["num_accepted"], "out num_accepted", dev, torch.int32, (B,))
    for k in ("accept_prob", "q_draft", "p_draft"):
        if k in out:
            _need(out[k], f"out {k}", dev, torch.float32, (B, K))
    if want_rates:
        if events is not None:
            raise ValueError("want_rates and events cannot be combined")
        if "rate" not in out:
            out["rate"] = torch.empty((B, K), dtype=torch.float32, device=dev)
        _need(out["rate"], "out rate", dev, torch.float32, (B, K))
    samp = sampling(temperature, top_k, top_p, lenience, mentor_kl)
    need = _lib.spec_verify_workspace_size(B, K, V, dt, ctypes.byref(samp))
    if need == 0:
        raise SpecVerifyError("spec_verify_workspace_size", 1)
    ws = workspace(dev, need, stream)
    args = [_ptr(target_logits), _ptr(draft_logits) if K > 0 else None, dt, B, K, V, draft_rows,
            _ptr(draft_tokens) if K > 0 else None, _ptr(uniforms), ctypes.byref(samp),
            _ptr(out["tokens"]), _ptr(out["num_accepted"]), _ptr(out.get("accept_prob")),
            _ptr(out.get("q_draft")), _ptr(out.get("p_draft")), _ptr(ws), ws.numel(),
            _stream(dev, stream)]
    if presampled is not None:
        if want_rates or events is not None:
            raise ValueError("presampled cannot be combined with want_rates or events")
        if draft_rows != K:
            raise ValueError("presampled needs draft_logits [B, K, V]")
        _need(presampled, "presampled", dev, torch.uint8)
        _check("spec_verify_presampled", _lib.spec_verify_presampled(
            args[0], args[1], dt, B, K, V, *args[7:15], _ptr(presampled), presampled.numel(),
            *args[15:]))
    elif want_rates:
        _check("spec_verify_rates", _lib.spec_verify_rates(*args[:15], _ptr(out["rate"]),
                                                           *args[15:]))
    elif events is None:
        _check("spec_verify", _lib.spec_verify(*args))
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check("spec_verify_profiled", _lib.spec_verify_profiled(*args, arr, len(events)))
    return out


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, uniforms, out, *,
                        temperature=1.0, top_k=0, top_p=1.0, lenience=1.0, mentor_kl=0.0,
                        stream=None):
    """spec_verify through the entry point that takes no workspace (the library's own scratch
    buffer, one per GPU; see include/spec_verify.h), for callers that cannot allocate.  ``out``
    must hold the output tensors (tokens, num_accepted and optionally accept_prob, q_draft,
    p_draft), so that this call allocates nothing.  Raises SpecVerifyError with status 5 when
    the problem needs more scratch than the buffer holds."""
    dev = target_logits.device
    B, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    if K > 0:
        _need(draft_logits, "draft_logits", dev, target_logits.dtype)
        if draft_logits.dim() != 3 or draft_logits.shape[0] != B or draft_logits.shape[2] != V:
            raise ValueError("draft_logits must be [B, K or K+1, V]")
        draft_rows = draft_logits.shape[1]
        _need(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    else:
        draft_rows = 0
    _need(uniforms, "uniforms", dev, torch.float32, (B, K + 1))
    _need(out["tokens"], "out tokens", dev, torch.int32, (B, K + 1))
    _need(out["num_accepted"], "out num_accepted", dev, torch.int32, (B,))
    for k in ("accept_prob", "q_draft", "p_draft"):
        if k in out:
            _need(out[k], f"out {k}", dev, torch.float32, (B, K))
    samp = sampling(temperature, top_k, top_p, lenience, mentor_kl)
    _check("spec_verify_noalloc", _lib.spec_verify_noalloc(
        _ptr(target_logits), _ptr(draft_logits) if K > 0 else None, dt, B, K, V, draft_rows,
        _ptr(draft_tokens) if K > 0 else None, _ptr(uniforms), ctypes.byref(samp),
        _ptr(out["tokens"]), _ptr(out["num_accepted"]), _ptr(out.get("accept_prob")),
        _ptr(out.get("q_draft")), _ptr(out.get("p_draft")), _stream(dev, stream)))
    return out


def sample_summary(R, V, dtype, *, temperature=1.0, top_k=0, top_p=1.0, device=None):
    """A device buffer for spec_sample(summary=...) over R rows of V logits of torch dtype
    ``dtype``: it keeps the rows' summaries for spec_verify(presampled=...)."""
    dt = _dtype_code(torch.empty(0, dtype=dtype))
    samp = sampling(temperature, top_k, top_p, 1.0)
    need = _lib.spec_sample_workspace_size(R, V, dt, ctypes.byref(samp))
    if need == 0:
        raise SpecVerifyError("spec_sample_workspace_size", 1)
    return torch.empty(need, dtype=torch.uint8,
                       device=device if device is not None else torch.device("cuda"))


def spec_sample(logits, uniforms, *, temperature=1.0, top_k=0, top_p=1.0, out=None,
                summary=None, stream=None):
    """One token per row of logits [R, V] from its processed distribution; uniforms [R].
    ``summary``: a buffer from sample_summary; the rows' summaries are kept there (instead of
    the stream's shared workspace) for a later spec_verify(presampled=summary)."""
    dev = logits.device
    R, V = logits.shape
    _need(logits, "logits", dev)
    dt = _dtype_code(logits)
    _need(uniforms, "uniforms", dev, torch.float32, (R,))
    if out is None:
        out = torch.empty((R,), dtype=torch.int32, device=dev)
    _need(out, "out", dev, torch.int32, (R,))
    samp = sampling(temperature, top_k, top_p, 1.0)
    need = _lib.spec_sample_workspace_size(R, V, dt, ctypes.byref(samp))
    if need == 0:
        raise SpecVerifyError("spec_sample_workspace_size", 1)
    if summary is not None:
        _need(summary, "summary", dev, torch.uint8)
        ws = summary
    else:
        ws = workspace(dev, need, stream)
    _check("spec_sample", _lib.spec_sample(_ptr(logits), dt, R, V, _ptr(uniforms),
                                           ctypes.byref(samp), _ptr(out), _ptr(ws), ws.numel(),
                                           _stream(dev, stream)))
    return out


def spec_verify_tree(target_logits, parent, node_tokens, max_depth, *, out=None, stream=None,
                     events=None):
    """Greedy tree verification: target_logits [B, N, V], parent / node_tokens [B, N] int32.

    ``events``: optional list of >= 2 hipEvent_t handles (ints) for per-phase timing.
    """
    dev = target_logits.device
    B, N, V = target_logits.shape
    _need(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    _need(parent, "parent", dev, torch.int32, (B, N))
    _need(node_tokens, "node_tokens", dev, torch.int32, (B, N))
    out = dict(out or {})
    out.setdefault("tokens", torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev))
    out.setdefault("num_accepted", torch.empty((B,), dtype=torch.int32, device=dev))
    out.setdefault("last_node", torch.empty((B,), dtype=torch.int32, device=dev))
    _need(out["tokens"], "out tokens", dev, torch.int32, (B, max_depth + 1))
    _need(out["num_accepted"], "out num_accepted", dev, torch.int32, (B,))
    _need(out["last_node"], "out last_node", dev, torch.int32, (B,))
    need = _lib.spec_verify_tree_workspace_size(B, N, V, dt)
    if need == 0:
        raise SpecVerifyError("spec_verify_tree_workspace_size", 1)
    ws = workspace(dev, need, stream)
    args = (_ptr(target_logits), dt, B, N, V, _ptr(parent), _ptr(node_tokens), int(max_depth),
            _ptr(out["tokens"]), _ptr(out["num_accepted"]), _ptr(out["last_node"]), _ptr(ws),
            ws.numel(), _stream(dev, stream))
    if events is None:
        _check("spec_verify_tree", _lib.spec_verify_tree(*args))
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check("spec_verify_tree_profiled",
               _lib.spec_verify_tree_profiled(*args, arr, len(events)))
    return out


def spec_build_tree(candidates, N, *, want_mask=True, out=None, stream=None):
    """REST draft tree from candidates [B, M, L] int32 (a candidate ends at its first negative
    entry): returns parent, tokens, depth, weight [B, N], num_nodes [B] and, if want_mask,
    mask [B, N, N] uint8 (see include/spec_verify.h)."""
    dev = candidates.device
    _need(candidates, "candidates", dev, torch.int32)
    if candidates.dim() != 3:
        raise ValueError("candidates must be [B, M, L]")
    B, M, L = candidates.shape
    out = dict(out or {})
    for k in ("parent", "tokens", "depth", "weight"):
        out.setdefault(k, torch.empty((B, N), dtype=torch.int32, device=dev))
        _need(out[k], f"out {k}", dev, torch.int32, (B, N))
    out.setdefault("num_nodes", torch.empty((B,), dtype=torch.int32, device=dev))
    _need(out["num_nodes"], "out num_nodes", dev, torch.int32, (B,))
    if want_mask:
        out.setdefault("mask", torch.empty((B, N, N), dtype=torch.uint8, device=dev))
        _need(out["mask"], "out mask", dev, torch.uint8, (B, N, N))
    _check("spec_build_tree", _lib.spec_build_tree(
        _ptr(candidates), B, M, L, int(N), _ptr(out["parent"]), _ptr(out["tokens"]),
        _ptr(out["num_nodes"]), _ptr(out["depth"]), _ptr(out["weight"]), _ptr(out.get("mask")),
        _stream(dev, stream)))
    return out


def spec_philox_uniform(key, counter, n, *, device=None, out=None, stream=None):
    """n float32 uniforms of the Philox4x64-10 stream (key = (k0, k1), 64-bit start counter)
    generated on the GPU (see include/spec_verify.h)."""
    if out is None:
        out = torch.empty((int(n),), dtype=torch.float32, device=device or "cuda")
    dev = out.device
    _need(out, "out", dev, torch.float32)
    if out.numel() < n:
        raise ValueError("out is too small")
    k0, k1 = (int(k) & (2**64 - 1) for k in key)
    _check("spec_philox_uniform", _lib.spec_philox_uniform(
        k0, k1, int(counter) & (2**64 - 1), int(n), _ptr(out) if n else None,
        _stream(dev, stream)))
    return out


def spec_acceptance_rate(target_logits, draft_logits, *, temperature=1.0, top_k=0, top_p=1.0,
                         lenience=1.0, out=None, stream=None):
    """beta [B, K] = sum_x min(p(x), q(x) / l) per draft position (see include/spec_verify.h)."""
    dev = target_logits.device
    B, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits", dev)
    dt = _dtype_code(target_logits)
    _need(draft_logits, "draft_logits", dev, target_logits.dtype)
    if draft_logits.dim() != 3 or draft_logits.shape[0] != B or draft_logits.shape[2] != V:
        raise ValueError("draft_logits must be [B, K or K+1, V]")
    if out is None:
        out = torch.empty((B, K), dtype=torch.float32, device=dev)
    _need(out, "out", dev, torch.float32, (B, K))
    samp = sampling(temperature, top_k, top_p, lenience)
    need = _lib.spec_verify_workspace_size(B, K, V, dt, ctypes.byref(samp))
    if need == 0:
        raise SpecVerifyError("spec_verify_workspace_size", 1)
    ws = workspace(dev, need, stream)
    _check("spec_acceptance_rate", _lib.spec_acceptance_rate(
        _ptr(target_logits), _ptr(draft_logits), dt, B, K, V, draft_logits.shape[1],
        ctypes.byref(samp), _ptr(out), _ptr(ws), ws.numel(), _stream(dev, stream)))
    return out


def expected_tokens(alpha, gamma):
    return _lib.spec_expected_tokens(float(alpha), int(gamma))


def walltime_speedup(alpha, gamma, c):
    return _lib.spec_walltime_speedup(float(alpha), int(gamma), float(c))


def ops_factor(alpha, gamma, c_hat):
    return _lib.spec_ops_factor(float(alpha), int(gamma), float(c_hat))


def optimal_gamma(alpha, c, max_gamma):
    return _lib.spec_optimal_gamma(float(alpha), float(c), int(max_gamma))
