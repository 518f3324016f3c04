"""Python binding of libdflash.so: argument marshalling only.

Every function here checks tensor placement, dtype and contiguity, turns
tensors into raw device pointers and calls the C ABI of the same name
(``include/dflash.h``) on the current HIP stream.  All arithmetic of the path
runs in the library's HIP kernels.  Importing this package fails if the
library has not been built (``python block_draft_select_amd/build.py``).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

F32 = 0
BF16 = 1
K_MAX, L_MAX, R_MAX, V_MAX, CHUNK = 16, 16, 256, 2097152, 4096
STATIC_SCRATCH_BYTES = 8 << 20

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4

KERNELS = ("topk", "gate", "scores", "trace", "stats", "finalize", "cycle_stream", "cycle_scores",
           "cycle_finalize", "conv2tap", "trace_viterbi", "topk_merge", "shard_stats", "shard_finalize")


class dflash_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "L", "V", "K", "r", "hidden", "logit_dtype", "param_dtype")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class DFlashError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_draft_select_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    D = ctypes.POINTER(dflash_dims)
    sig = {
        "dflash_abi_version": (I32, []),
        "dflash_status_string": (ctypes.c_char_p, [I32]),
        "dflash_last_error": (ctypes.c_char_p, []),
        "dflash_workspace_bytes": (I32, [D, ctypes.POINTER(SZ)]),
        "dflash_workspace_init": (I32, [P, SZ, P]),
        "dflash_topk": (I32, [D, P, P, P, P, SZ, P]),
        "dflash_pair_scores": (I32, [D, P, P, P, P, P, P, P, P, SZ, P]),
        "dflash_trace": (I32, [D, P, P, P, P, U64, P, P, P, P]),
        "dflash_verify": (I32, [D, P, P, P, P, P, P, U64, P, P, P, SZ, P]),
        "dflash_cycle": (I32, [D, P, P, P, P, P, P, P, P, U64, P, P, P, P, P, P, P, P, P, SZ, P]),
        "dflash_cycle_maxsum": (I32, [D, P, P, P, P, P, P, P, P, U64, P, P, P, P, P, P, P, P, P, SZ, P]),
        "dflash_cycle_static": (I32, [D, P, P, P, P, P, P, P, P, U64, P, P, P, P, P, P, P, P, P]),
        "dflash_conv2tap": (I32, [D, P, P, P, P, P]),
        "dflash_trace_viterbi": (I32, [D, P, P, P, P, P, P]),
        "dflash_topk_merge": (I32, [D, I32, ctypes.POINTER(I32), P, P, P, P, P]),
        "dflash_shard_stats_bytes": (I32, [D, I32, ctypes.POINTER(I32), ctypes.POINTER(SZ)]),
        "dflash_shard_stats": (I32, [D, I32, ctypes.POINTER(I32), I32, P, P, P, P]),
        "dflash_verify_shards": (I32, [D, I32, ctypes.POINTER(I32), ctypes.POINTER(P), P, P, P, P, P, P, U64, P, P,
                                       P]),
        "dflash_read_probe": (I32, [P, SZ, P, P]),
        "dflash_copy_probe": (I32, [P, P, SZ, P]),
        "dflash_kernel_name": (ctypes.c_char_p, [I32]),
        "dflash_profile_enable": (I32, [I32]),
        "dflash_profile_collect": (I32, [I32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status):
    if status != OK:
        raise DFlashError(status, lib.dflash_last_error().decode())


# ------------------------------------------------------------------ helpers

def dims(B, L, V, K, r, hidden, logit_dtype, param_dtype):
    """A ``dflash_dims`` value (dtypes: F32 / BF16 or the strings 'f32'/'bf16')."""
    conv = {"f32": F32, "bf16": BF16, F32: F32, BF16: BF16}
    return dflash_dims(int(B), int(L), int(V), int(K), int(r), int(hidden),
                       conv[logit_dtype], conv[param_dtype])


def workspace_bytes(d):
    n = ctypes.c_size_t(0)
    _check(lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def workspace(d, device="cuda"):
    """A zero-filled workspace tensor large enough for every entry point."""
    return torch.zeros(max(workspace_bytes(d), 16), dtype=torch.uint8, device=device)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_LOGIT = {F32: torch.float32, BF16: torch.bfloat16}


def _ptr(t, name, dtype=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ entry points

def dflash_topk(d, U, cand_idx, cand_logit, ws, stream=None):
    R = d.B * d.L
    _check(lib.dflash_topk(ctypes.byref(d), _ptr(U, "U", _TORCH_LOGIT[d.logit_dtype], R * d.V),
                           _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                           _ptr(cand_logit, "cand_logit", torch.float32, R * d.K),
                           _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def dflash_pair_scores(d, x0, cand_idx, cand_logit, E, W_g, h, S, ws, stream=None):
    R, pt = d.B * d.L, _TORCH_LOGIT[d.param_dtype]
    _check(lib.dflash_pair_scores(ctypes.byref(d), _ptr(x0, "x0", torch.int32, d.B),
                                  _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                                  _ptr(cand_logit, "cand_logit", torch.float32, R * d.K),
                                  _ptr(E, "E", pt, d.V * d.r), _ptr(W_g, "W_g", pt, d.hidden * d.r),
                                  _ptr(h, "h", pt, R * d.hidden), _ptr(S, "S", torch.float32, R * d.K * d.K),
                                  _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def dflash_trace(d, S, cand_idx, T, seed, cycle, path_rank, draft_tok, q, stream=None):
    R = d.B * d.L
    _check(lib.dflash_trace(ctypes.byref(d), _ptr(S, "S", torch.float32, R * d.K * d.K),
                            _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                            _ptr(T, "T", torch.float32, d.B), _ptr(seed, "seed", torch.int64, d.B),
                            ctypes.c_uint64(int(cycle) & 0xFFFFFFFFFFFFFFFF),
                            _ptr(path_rank, "path_rank", torch.int32, R),
                            _ptr(draft_tok, "draft_tok", torch.int32, R),
                            _ptr(q, "q", torch.float32, R * d.K), _stream(stream)))


def dflash_verify(d, Z, cand_idx, path_rank, q, T, seed, cycle, accept_len, out_tok, ws, stream=None):
    R = d.B * d.L
    _check(lib.dflash_verify(ctypes.byref(d),
                             _ptr(Z, "Z", _TORCH_LOGIT[d.logit_dtype], d.B * (d.L + 1) * d.V),
                             _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                             _ptr(path_rank, "path_rank", torch.int32, R),
                             _ptr(q, "q", torch.float32, R * d.K),
                             _ptr(T, "T", torch.float32, d.B), _ptr(seed, "seed", torch.int64, d.B),
                             ctypes.c_uint64(int(cycle) & 0xFFFFFFFFFFFFFFFF),
                             _ptr(accept_len, "accept_len", torch.int32, d.B),
                             _ptr(out_tok, "out_tok", torch.int32, d.B * (d.L + 1)),
                             _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def _cycle_call(fn, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, ws,
                cand_idx, cand_logit, S, path_rank, draft_tok, q, stream):
    R, lt, pt = d.B * d.L, _TORCH_LOGIT[d.logit_dtype], _TORCH_LOGIT[d.param_dtype]
    _check(fn(
        ctypes.byref(d), _ptr(U, "U", lt, R * d.V), _ptr(Z, "Z", lt, d.B * (d.L + 1) * d.V),
        _ptr(x0, "x0", torch.int32, d.B), _ptr(E, "E", pt, d.V * d.r),
        _ptr(W_g, "W_g", pt, d.hidden * d.r), _ptr(h, "h", pt, R * d.hidden),
        _ptr(T, "T", torch.float32, d.B), _ptr(seed, "seed", torch.int64, d.B),
        ctypes.c_uint64(int(cycle) & 0xFFFFFFFFFFFFFFFF),
        _ptr(accept_len, "accept_len", torch.int32, d.B),
        _ptr(out_tok, "out_tok", torch.int32, d.B * (d.L + 1)),
        _ptr(cand_idx, "cand_idx", torch.int32, R * d.K, optional=True),
        _ptr(cand_logit, "cand_logit", torch.float32, R * d.K, optional=True),
        _ptr(S, "S", torch.float32, R * d.K * d.K, optional=True),
        _ptr(path_rank, "path_rank", torch.int32, R, optional=True),
        _ptr(draft_tok, "draft_tok", torch.int32, R, optional=True),
        _ptr(q, "q", torch.float32, R * d.K, optional=True),
        _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def dflash_cycle(d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, ws,
                 cand_idx=None, cand_logit=None, S=None, path_rank=None, draft_tok=None, q=None,
                 stream=None):
    _cycle_call(lib.dflash_cycle, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, ws,
                cand_idx, cand_logit, S, path_rank, draft_tok, q, stream)


def dflash_cycle_maxsum(d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, ws,
                        cand_idx=None, cand_logit=None, S=None, path_rank=None, draft_tok=None, q=None,
                        stream=None):
    _cycle_call(lib.dflash_cycle_maxsum, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, ws,
                cand_idx, cand_logit, S, path_rank, draft_tok, q, stream)


def dflash_cycle_static(d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok,
                        cand_idx=None, cand_logit=None, S=None, path_rank=None, draft_tok=None, q=None,
                        stream=None):
    """dflash_cycle on the library's own static scratch (no workspace argument)."""
    R, lt, pt = d.B * d.L, _TORCH_LOGIT[d.logit_dtype], _TORCH_LOGIT[d.param_dtype]
    _check(lib.dflash_cycle_static(
        ctypes.byref(d), _ptr(U, "U", lt, R * d.V), _ptr(Z, "Z", lt, d.B * (d.L + 1) * d.V),
        _ptr(x0, "x0", torch.int32, d.B), _ptr(E, "E", pt, d.V * d.r),
        _ptr(W_g, "W_g", pt, d.hidden * d.r), _ptr(h, "h", pt, R * d.hidden),
        _ptr(T, "T", torch.float32, d.B), _ptr(seed, "seed", torch.int64, d.B),
        ctypes.c_uint64(int(cycle) & 0xFFFFFFFFFFFFFFFF),
        _ptr(accept_len, "accept_len", torch.int32, d.B),
        _ptr(out_tok, "out_tok", torch.int32, d.B * (d.L + 1)),
        _ptr(cand_idx, "cand_idx", torch.int32, R * d.K, optional=True),
        _ptr(cand_logit, "cand_logit", torch.float32, R * d.K, optional=True),
        _ptr(S, "S", torch.float32, R * d.K * d.K, optional=True),
        _ptr(path_rank, "path_rank", torch.int32, R, optional=True),
        _ptr(draft_tok, "draft_tok", torch.int32, R, optional=True),
        _ptr(q, "q", torch.float32, R * d.K, optional=True), _stream(stream)))


def dflash_topk_merge(d, shard_begin, cand_idx_parts, cand_logit_parts, cand_idx, cand_logit, stream=None):
    """``shard_begin``: a Python sequence of the shards' first token indices."""
    R, n = d.B * d.L, len(shard_begin)
    begins = (ctypes.c_int32 * n)(*[int(v) for v in shard_begin])
    _check(lib.dflash_topk_merge(ctypes.byref(d), n, begins,
                                 _ptr(cand_idx_parts, "cand_idx_parts", torch.int32, n * R * d.K),
                                 _ptr(cand_logit_parts, "cand_logit_parts", torch.float32, n * R * d.K),
                                 _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                                 _ptr(cand_logit, "cand_logit", torch.float32, R * d.K), _stream(stream)))


def _begins(shard_begin):
    n = len(shard_begin)
    return n, (ctypes.c_int32 * n)(*[int(v) for v in shard_begin])


def shard_stats_bytes(d, shard_begin):
    n, begins = _begins(shard_begin)
    out = ctypes.c_size_t(0)
    _check(lib.dflash_shard_stats_bytes(ctypes.byref(d), n, begins, ctypes.byref(out)))
    return out.value


def dflash_shard_stats(d, shard_begin, shard, Z_shard, T, stats, stream=None):
    """Statistics of shard ``shard`` (its rows ``Z_shard`` [B, L+1, width])
    into its columns of ``stats`` (a uint8 tensor of shard_stats_bytes)."""
    n, begins = _begins(shard_begin)
    hi = shard_begin[shard + 1] if shard + 1 < n else d.V
    width = int(hi) - int(shard_begin[shard])
    _check(lib.dflash_shard_stats(ctypes.byref(d), n, begins, int(shard),
                                  _ptr(Z_shard, "Z_shard", _TORCH_LOGIT[d.logit_dtype], d.B * (d.L + 1) * width),
                                  _ptr(T, "T", torch.float32, d.B), _ptr(stats, "stats", torch.uint8),
                                  _stream(stream)))


def dflash_verify_shards(d, shard_begin, Z_shards, stats, cand_idx, path_rank, q, T, seed, cycle, accept_len,
                         out_tok, stream=None):
    """``Z_shards``: one [B, L+1, width] tensor per shard."""
    n, begins = _begins(shard_begin)
    R = d.B * d.L
    zp = (ctypes.c_void_p * n)(*[_ptr(z, "Z_shards[]", _TORCH_LOGIT[d.logit_dtype]).value for z in Z_shards])
    _check(lib.dflash_verify_shards(ctypes.byref(d), n, begins, zp, _ptr(stats, "stats", torch.uint8),
                                    _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                                    _ptr(path_rank, "path_rank", torch.int32, R),
                                    _ptr(q, "q", torch.float32, R * d.K),
                                    _ptr(T, "T", torch.float32, d.B), _ptr(seed, "seed", torch.int64, d.B),
                                    ctypes.c_uint64(int(cycle) & 0xFFFFFFFFFFFFFFFF),
                                    _ptr(accept_len, "accept_len", torch.int32, d.B),
                                    _ptr(out_tok, "out_tok", torch.int32, d.B * (d.L + 1)), _stream(stream)))


def dflash_trace_viterbi(d, S, cand_idx, path_rank, draft_tok, q, stream=None):
    R = d.B * d.L
    _check(lib.dflash_trace_viterbi(ctypes.byref(d), _ptr(S, "S", torch.float32, R * d.K * d.K),
                                    _ptr(cand_idx, "cand_idx", torch.int32, R * d.K),
                                    _ptr(path_rank, "path_rank", torch.int32, R),
                                    _ptr(draft_tok, "draft_tok", torch.int32, R),
                                    _ptr(q, "q", torch.float32, R * d.K), _stream(stream)))


def dflash_conv2tap(d, x, x0, Wt, y, stream=None):
    R, pt = d.B * d.L, _TORCH_LOGIT[d.param_dtype]
    _check(lib.dflash_conv2tap(ctypes.byref(d), _ptr(x, "x", pt, R * d.hidden), _ptr(x0, "x0", pt, d.B * d.hidden),
                               _ptr(Wt, "Wt", pt, 2 * d.hidden * d.hidden),
                               _ptr(y, "y", torch.float32, R * d.hidden), _stream(stream)))


def dflash_workspace_init(ws, stream=None):
    _check(lib.dflash_workspace_init(_ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def dflash_read_probe(buf, sink, stream=None):
    _check(lib.dflash_read_probe(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                 _ptr(sink, "sink", torch.int32), _stream(stream)))


def dflash_copy_probe(dst, src, stream=None):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _check(lib.dflash_copy_probe(_ptr(dst, "dst"), _ptr(src, "src"), n, _stream(stream)))


def dflash_profile_enable(on):
    _check(lib.dflash_profile_enable(1 if on else 0))


def dflash_profile_collect(kernel):
    """(launches, total_ms) of the recorded launches of a kernel (name or id)."""
    kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib.dflash_profile_collect(kid, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
