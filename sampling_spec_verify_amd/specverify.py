"""Python binding of libspecverify (ctypes; argument marshalling only).

Every function has the name of its C entry point without the ``sv_`` prefix.
Tensors are torch tensors on the GPU; the binding checks shapes and dtypes,
allocates outputs and the workspace with torch, and passes raw device pointers
and ``torch.cuda.current_stream()``.  All computation happens in the HIP
kernels of ``libspecverify.so``; if that library is missing the binding raises,
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB names another build of the same library (the host-sanitizer
# build of the ABI tests); the binding raises if the file is missing.
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(HERE, "libspecverify.so")

SV_OK, SV_EINVAL, SV_ENULL, SV_EALIGN, SV_EWORKSPACE, SV_EDTYPE, SV_EHIP, SV_ETOOBIG = range(8)
SV_NOALLOC_SCRATCH_BYTES = 16 << 20
SV_BF16, SV_F32 = 0, 1
SV_MIX_PROB, SV_MIX_LOGIT = 0, 1
MIX_SPACES = {"prob": SV_MIX_PROB, "logit": SV_MIX_LOGIT}
SV_MAX_POSITIONS = 64
SV_MAX_TREE_NODES = 1024
SV_MAX_VOCAB_BF16 = 1 << 21
SV_MAX_VOCAB_F32 = 1 << 20
SV_MAX_BLOCKS_PER_TREE = 32
DATA_FLAGS = {
    0x01: "BAD_TOKEN", 0x02: "BAD_ROW", 0x04: "ZERO_Q", 0x08: "BAD_LENGTH",
    0x10: "BAD_TREE", 0x20: "FALLBACK", 0x40: "DEPTH", 0x80: "SYNC",
}

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t

_CHAIN_ARGS = [_P, _L, _P, _L, _I, _I, _I, _I, _P, _P, _P, _P, _F, _F, _P, _P, _P, _P, _P, _S, _P]
_GREEDY_ARGS = [_P, _L, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _S, _P]
_PATH_ARGS = [_P, _L, _P, _L, _I, _I, _I, _I, _P, _P, _I, _P, _P, _F, _F, _P, _P, _P, _P, _P, _S,
              _P]
_MULTI_ARGS = [_P, _L, _P, _L, _I, _I, _I, _I, _P, _P, _P, _P, _F, _F, _I, _P, _P, _P, _P, _I, _P,
               _P, _S, _P]

SIGNATURES = {
    "sv_status_string": ([_I], ctypes.c_char_p),
    "sv_chain_workspace_bytes": ([_I, _I, _I], _S),
    "sv_chain_verify": (_CHAIN_ARGS, _I),
    "sv_chain_verify_noalloc": (_CHAIN_ARGS[:18] + [_P], _I),
    "sv_chain_row_stats": (_CHAIN_ARGS, _I),
    "sv_chain_accept_resample": (_CHAIN_ARGS, _I),
    "sv_chain_row_stats_timed": (_CHAIN_ARGS + [_P, _P], _I),
    "sv_chain_verify_ex": (_CHAIN_ARGS + [_I, _I, _P, _P], _I),
    "sv_chain_acceptance_workspace_bytes": ([_I, _I, _I], _S),
    "sv_chain_acceptance_rate": ([_P, _L, _P, _L, _I, _I, _I, _I, _P, _F, _F, _I, _P, _P, _P, _S,
                                  _P], _I),
    "sv_tree_workspace_bytes": ([_I, _I, _I], _S),
    "sv_tree_verify_greedy": (_GREEDY_ARGS, _I),
    "sv_tree_row_argmax": (_GREEDY_ARGS, _I),
    "sv_tree_greedy_walk": (_GREEDY_ARGS, _I),
    "sv_tree_row_argmax_timed": (_GREEDY_ARGS + [_P, _P], _I),
    "sv_tree_verify_greedy_timed": (_GREEDY_ARGS + [_P, _P], _I),
    "sv_tree_attention_mask": ([_P, _I, _I, _P, _I, _P, _P, _P], _I),
    "sv_tree_attention_mask_timed": ([_P, _I, _I, _P, _I, _P, _P, _P, _P, _P], _I),
    "sv_tree_multi_workspace_bytes": ([_I, _I, _I], _S),
    "sv_tree_verify_multi": (_MULTI_ARGS, _I),
    "sv_tree_verify_multi_ex": (_MULTI_ARGS + [_I], _I),
    "sv_tree_verify_path": (_PATH_ARGS, _I),
    "sv_tree_verify_path_ex": (_PATH_ARGS + [_I], _I),
    "sv_read_stream": ([_P, _S, _P, _P, _P, _P], _I),
}

_lib = None


class SpecVerifyError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with sampling_spec_verify_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


class KernelTimer:
    """``n`` pairs of HIP events for the ``*_timed`` calls.

    A timed call attaches pair ``i`` to its kernel launch, so that
    ``elapsed_ms(i)`` is that kernel's own duration (dispatch begin to end).
    """

    def __init__(self, n: int):
        _torch().cuda.init()
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(_F), _P, _P]
        self._hip.hipEventDestroy.argtypes = [_P]
        self.start, self.stop = [], []
        for _ in range(n):
            for lst in (self.start, self.stop):
                ev = _P()
                if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise SpecVerifyError("hipEventCreate failed")
                lst.append(ev)

    def pair(self, i: int):
        return self.start[i], self.stop[i]

    def elapsed_ms(self, i: int) -> float:
        ms = _F()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
            raise SpecVerifyError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for ev in self.start + self.stop:
            self._hip.hipEventDestroy(ev)
        self.start, self.stop = [], []


def read_stream(buf, nbytes: int, sink, events=None, stream=None):
    """sv_read_stream over the first ``nbytes`` bytes of the GPU tensor ``buf``
    (a calibration read, not a step of the method); ``sink`` is a device int32
    tensor of at least one element, ``events`` an optional (start, stop) pair."""
    if not buf.is_cuda or not sink.is_cuda:
        raise ValueError("buf and sink must be GPU tensors")
    if nbytes > buf.numel() * buf.element_size() or sink.numel() < 1:
        raise ValueError("nbytes exceeds buf, or sink is empty")
    ev = (None, None) if events is None else events
    _check(lib().sv_read_stream(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream), *ev),
           "sv_read_stream")


def status_string(code: int) -> str:
    return lib().sv_status_string(int(code)).decode()


def decode_flags(word: int):
    return [name for bit, name in DATA_FLAGS.items() if word & bit]


def _check(code: int, what: str):
    if code != SV_OK:
        raise SpecVerifyError(f"{what}: {status_string(code)}")


def chain_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(lib().sv_chain_workspace_bytes(B, K, V))


def tree_workspace_bytes(B: int, N: int, V: int) -> int:
    return int(lib().sv_tree_workspace_bytes(B, N, V))


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _rows(t, B: int, R: int, V: int, name: str) -> int:
    """Check a [B, R, V] logits tensor with unit last stride; returns its row stride."""
    if t.dim() != 3 or t.shape[0] != B or t.shape[1] != R or t.shape[2] != V:
        raise ValueError(f"{name} must be [{B}, {R}, {V}], got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    ld = t.stride(1)
    if t.stride(2) != 1 or ld < V or (B > 1 and t.stride(0) != R * ld):
        raise ValueError(f"{name} must be a [B, R, V] view of a contiguous [B, R, ld] buffer")
    return int(ld)


def _i32(t, shape, name):
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor of shape {tuple(shape)}")
    return t


def _f32(t, shape, name):
    torch = _torch()
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor of shape {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class ChainOut(NamedTuple):
    accepted: object        # [B] int32
    out_tokens: object      # [B, K+1] int32
    accept_prob: object     # [B, K] float32
    status: object          # [1] int32 (device word of SV_DATA_* bits)


class ChainCall:
    """A chain-verify call with its outputs and workspace bound once.

    ``run()`` launches both kernels; ``row_stats()`` / ``accept_resample()``
    launch one each (the pair equals ``run()``).  Rebinding inputs with
    ``set_inputs`` keeps the outputs and workspace.  The stream (default: the
    current torch stream) is bound when the inputs are.  ``space`` is "prob"
    (the mixture equation) or "logit" (the pseudocode's mixed logits).
    """

    def __init__(self, target, draft, tokens, u_accept, u_sample, lam=0.0, temperature=1.0,
                 draft_len=None, stream=None, workspace=None, space: str = "prob"):
        torch = _torch()
        if space not in MIX_SPACES:
            raise ValueError(f"space must be one of {sorted(MIX_SPACES)}, got {space!r}")
        self.space = MIX_SPACES[space]
        B, K1, V = target.shape
        K = K1 - 1
        dev = target.device
        self.B, self.K, self.V = B, K, V
        self.lam, self.temperature = float(lam), float(temperature)
        self.stream = stream
        self.out = ChainOut(torch.empty(B, dtype=torch.int32, device=dev),
                            torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                            torch.empty(B, K, dtype=torch.float32, device=dev),
                            torch.empty(1, dtype=torch.int32, device=dev))
        nbytes = chain_workspace_bytes(B, K, V)
        if nbytes == 0 and B > 0:
            raise SpecVerifyError("invalid chain sizes")
        self.workspace = workspace if workspace is not None else torch.empty(
            max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.set_inputs(target, draft, tokens, u_accept, u_sample, draft_len)

    def set_inputs(self, target, draft, tokens, u_accept, u_sample, draft_len=None):
        B, K, V = self.B, self.K, self.V
        self.dtype = _dtype_code(target)
        if draft.dtype != target.dtype:
            raise TypeError("target and draft logits must share a dtype")
        self.ld_t = _rows(target, B, K + 1, V, "target")
        self.ld_q = _rows(draft, B, K, V, "draft") if K > 0 else V
        self.inputs = (target, draft, _i32(tokens, (B, K), "tokens"),
                       _i32(draft_len, (B,), "draft_len"),
                       _f32(u_accept, (B, K), "u_accept"), _f32(u_sample, (B,), "u_sample"))
        self._cached = self._args()

    def _args(self):
        t, d, tok, dl, ua, us = self.inputs
        o = self.out
        return (_ptr(t), self.ld_t, _ptr(d), self.ld_q, self.dtype, self.B, self.K, self.V,
                _ptr(tok), _ptr(dl), _ptr(ua), _ptr(us), self.lam, self.temperature,
                _ptr(o.accepted), _ptr(o.out_tokens), _ptr(o.accept_prob), _ptr(o.status),
                _ptr(self.workspace), self.workspace.numel(), _stream(self.stream))

    def _ex(self, stages: int, events=None):
        ev = (None, None) if events is None else events
        _check(lib().sv_chain_verify_ex(*self._cached, self.space, stages, *ev),
               "sv_chain_verify_ex")

    def run(self) -> ChainOut:
        if self.space == SV_MIX_PROB:
            _check(lib().sv_chain_verify(*self._cached), "sv_chain_verify")
        else:
            self._ex(3)
        return self.out

    def row_stats(self, events=None):
        """Launch the row-statistics kernel; ``events`` = (start, stop) times it."""
        if self.space != SV_MIX_PROB:
            self._ex(1, events)
        elif events is None:
            _check(lib().sv_chain_row_stats(*self._cached), "sv_chain_row_stats")
        else:
            _check(lib().sv_chain_row_stats_timed(*self._cached, *events),
                   "sv_chain_row_stats_timed")

    def accept_resample(self, events=None) -> ChainOut:
        """Launch the accept / resample kernel; ``events`` = (start, stop) times it."""
        if self.space != SV_MIX_PROB or events is not None:
            self._ex(2, events)
        else:
            _check(lib().sv_chain_accept_resample(*self._cached), "sv_chain_accept_resample")
        return self.out


def chain_verify_noalloc(call: "ChainCall") -> ChainOut:
    """sv_chain_verify_noalloc on the inputs and outputs bound to ``call`` (its
    workspace is not used: the library's own per-GPU scratch array is)."""
    if call.space != SV_MIX_PROB:
        raise ValueError("sv_chain_verify_noalloc mixes in probability space")
    args = call._cached
    _check(lib().sv_chain_verify_noalloc(*args[:18], args[20]), "sv_chain_verify_noalloc")
    return call.out


def chain_verify(target, draft, tokens, u_accept, u_sample, lam: float = 0.0,
                 temperature: float = 1.0, draft_len=None, stream=None,
                 space: str = "prob") -> ChainOut:
    """sv_chain_verify on torch tensors: target [B,K+1,V], draft [B,K,V] (bf16 or fp32)."""
    return ChainCall(target, draft, tokens, u_accept, u_sample, lam, temperature, draft_len,
                     stream, space=space).run()


class AcceptanceRateCall:
    """sv_chain_acceptance_rate with its output and workspace bound once:
    alpha[b, i] = sum_v min(p~(v), q(v)) for every drafted position."""

    def __init__(self, target, draft, lam=0.0, temperature=1.0, draft_len=None, stream=None,
                 workspace=None, space: str = "prob"):
        torch = _torch()
        if space not in MIX_SPACES:
            raise ValueError(f"space must be one of {sorted(MIX_SPACES)}, got {space!r}")
        B, K1, V = target.shape
        K = K1 - 1
        if draft.dtype != target.dtype:
            raise TypeError("target and draft logits must share a dtype")
        ld_t = _rows(target, B, K + 1, V, "target")
        ld_q = _rows(draft, B, K, V, "draft") if K > 0 else V
        _i32(draft_len, (B,), "draft_len")
        dev = target.device
        self.alpha = torch.empty(B, K, dtype=torch.float32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        nbytes = int(lib().sv_chain_acceptance_workspace_bytes(B, K, V))
        if nbytes == 0 and B > 0:
            raise SpecVerifyError("invalid sizes")
        self.workspace = workspace if workspace is not None else torch.empty(
            max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.inputs = (target, draft, draft_len)
        self._cached = (_ptr(target), ld_t, _ptr(draft), ld_q, _dtype_code(target), B, K, V,
                        _ptr(draft_len), float(lam), float(temperature), MIX_SPACES[space],
                        _ptr(self.alpha), _ptr(self.status), _ptr(self.workspace),
                        self.workspace.numel(), _stream(stream))

    def run(self):
        _check(lib().sv_chain_acceptance_rate(*self._cached), "sv_chain_acceptance_rate")
        return self.alpha, self.status


def chain_acceptance_rate(target, draft, lam: float = 0.0, temperature: float = 1.0,
                          draft_len=None, stream=None, space: str = "prob"):
    """alpha [B, K] (and the status word) for target [B,K+1,V], draft [B,K,V]."""
    return AcceptanceRateCall(target, draft, lam, temperature, draft_len, stream,
                              space=space).run()


class TreeGreedyOut(NamedTuple):
    accepted: object        # [B]
    out_tokens: object      # [B, Dmax+1]
    accepted_nodes: object  # [B, Dmax]
    status: object          # [1]


class TreeGreedyCall:
    """A greedy tree-verify call with outputs and workspace bound once (see ChainCall)."""

    def __init__(self, target, parent, node_token, Dmax: int, stream=None, workspace=None):
        torch = _torch()
        B, N1, V = target.shape
        N = N1 - 1
        ld = _rows(target, B, N + 1, V, "target")
        _i32(parent, (B, N), "parent")
        _i32(node_token, (B, N), "node_token")
        dev = target.device
        self.out = TreeGreedyOut(torch.empty(B, dtype=torch.int32, device=dev),
                                 torch.empty(B, Dmax + 1, dtype=torch.int32, device=dev),
                                 torch.empty(B, max(Dmax, 0), dtype=torch.int32, device=dev),
                                 torch.empty(1, dtype=torch.int32, device=dev))
        self.workspace = workspace if workspace is not None else torch.empty(
            max(tree_workspace_bytes(B, N, V), 16), dtype=torch.uint8, device=dev)
        self.inputs = (target, parent, node_token)
        o = self.out
        self._cached = (_ptr(target), ld, _dtype_code(target), B, N, V, _ptr(parent),
                        _ptr(node_token), _ptr(o.accepted), _ptr(o.out_tokens),
                        _ptr(o.accepted_nodes), int(Dmax), _ptr(o.status), _ptr(self.workspace),
                        self.workspace.numel(), _stream(stream))

    def run(self, events=None) -> TreeGreedyOut:
        """The whole call; ``events`` = (start, stop) times its first launch."""
        if events is None:
            _check(lib().sv_tree_verify_greedy(*self._cached), "sv_tree_verify_greedy")
        else:
            _check(lib().sv_tree_verify_greedy_timed(*self._cached, *events),
                   "sv_tree_verify_greedy_timed")
        return self.out

    def row_argmax(self, events=None):
        """Launch the row-argmax kernel; ``events`` = (start, stop) times it."""
        if events is None:
            _check(lib().sv_tree_row_argmax(*self._cached), "sv_tree_row_argmax")
        else:
            _check(lib().sv_tree_row_argmax_timed(*self._cached, *events),
                   "sv_tree_row_argmax_timed")

    def walk(self) -> TreeGreedyOut:
        _check(lib().sv_tree_greedy_walk(*self._cached), "sv_tree_greedy_walk")
        return self.out


def tree_verify_greedy(target, parent, node_token, Dmax: int, stream=None,
                       workspace=None) -> TreeGreedyOut:
    """sv_tree_verify_greedy: target [B, N+1, V], parent / node_token [B, N] int32."""
    return TreeGreedyCall(target, parent, node_token, Dmax, stream, workspace).run()


class TreeMaskOut(NamedTuple):
    mask: object            # [B, N+1, W] int32 words (bit patterns of the uint32 mask)
    depth: object           # [B, N+1] int32
    status: object          # [1] int32


class TreeMaskCall:
    """A tree-attention-mask call with its outputs bound once.

    The mask tensor is int32 (torch has no uint32 arithmetic); its bits are the
    uint32 words the C call writes.  ``status`` (a [1] int32 tensor) is OR-ed
    into, not cleared; a fresh zeroed one is made when omitted.
    """

    def __init__(self, parent, N: Optional[int] = None, mask_words: Optional[int] = None,
                 stream=None, status=None):
        torch = _torch()
        B = parent.shape[0]
        N = parent.shape[1] if N is None else N
        _i32(parent, (B, N), "parent")
        W = (N + 32) // 32 if mask_words is None else int(mask_words)
        dev = parent.device
        self.out = TreeMaskOut(torch.empty(B, N + 1, W, dtype=torch.int32, device=dev),
                               torch.empty(B, N + 1, dtype=torch.int32, device=dev),
                               torch.zeros(1, dtype=torch.int32, device=dev) if status is None
                               else status)
        o = self.out
        self.inputs = (parent,)
        self._cached = (_ptr(parent), B, N, _ptr(o.mask), W, _ptr(o.depth), _ptr(o.status),
                        _stream(stream))

    def run(self, events=None) -> TreeMaskOut:
        """Launch the mask kernel; ``events`` = (start, stop) times it."""
        if events is None:
            _check(lib().sv_tree_attention_mask(*self._cached), "sv_tree_attention_mask")
        else:
            _check(lib().sv_tree_attention_mask_timed(*self._cached, *events),
                   "sv_tree_attention_mask_timed")
        return self.out


def tree_attention_mask(parent, N: Optional[int] = None, mask_words: Optional[int] = None,
                        stream=None, status=None) -> TreeMaskOut:
    """sv_tree_attention_mask: parent [B, N] int32 -> ancestor mask words and depths."""
    return TreeMaskCall(parent, N, mask_words, stream, status).run()


class TreePathCall:
    """A path-mode call (chain acceptance along one root->leaf path of each
    tree) with its outputs and workspace bound once (see ChainCall)."""

    def __init__(self, target, draft, node_token, path, u_accept, u_sample, lam: float = 0.0,
                 temperature: float = 1.0, stream=None, workspace=None, space: str = "prob"):
        torch = _torch()
        B, N1, V = target.shape
        N = N1 - 1
        Dmax = path.shape[1]
        ld_t = _rows(target, B, N + 1, V, "target")
        ld_q = _rows(draft, B, N + 1, V, "draft")
        if draft.dtype != target.dtype:
            raise TypeError("target and draft logits must share a dtype")
        _i32(node_token, (B, N), "node_token")
        _i32(path, (B, Dmax), "path")
        _f32(u_accept, (B, Dmax), "u_accept")
        _f32(u_sample, (B,), "u_sample")
        if space not in MIX_SPACES:
            raise ValueError(f"space must be one of {sorted(MIX_SPACES)}, got {space!r}")
        self.space = space
        dev = target.device
        self.out = ChainOut(torch.empty(B, dtype=torch.int32, device=dev),
                            torch.empty(B, Dmax + 1, dtype=torch.int32, device=dev),
                            torch.empty(B, Dmax, dtype=torch.float32, device=dev),
                            torch.empty(1, dtype=torch.int32, device=dev))
        self.workspace = workspace if workspace is not None else torch.empty(
            max(tree_workspace_bytes(B, N, V), 16), dtype=torch.uint8, device=dev)
        self.inputs = (target, draft, node_token, path, u_accept, u_sample)
        o = self.out
        self._cached = (_ptr(target), ld_t, _ptr(draft), ld_q, _dtype_code(target), B, N, V,
                        _ptr(node_token), _ptr(path), Dmax, _ptr(u_accept), _ptr(u_sample),
                        float(lam), float(temperature), _ptr(o.accepted), _ptr(o.out_tokens),
                        _ptr(o.accept_prob), _ptr(o.status), _ptr(self.workspace),
                        self.workspace.numel(), _stream(stream))

    def run(self) -> ChainOut:
        if self.space == "prob":
            _check(lib().sv_tree_verify_path(*self._cached), "sv_tree_verify_path")
        else:
            _check(lib().sv_tree_verify_path_ex(*self._cached, MIX_SPACES[self.space]),
                   "sv_tree_verify_path_ex")
        return self.out


def tree_verify_path(target, draft, node_token, path, u_accept, u_sample, lam: float = 0.0,
                     temperature: float = 1.0, stream=None, workspace=None,
                     space: str = "prob") -> ChainOut:
    """sv_tree_verify_path: target / draft [B, N+1, V], path [B, Dmax] (-1 terminated)."""
    return TreePathCall(target, draft, node_token, path, u_accept, u_sample, lam, temperature,
                        stream, workspace, space).run()


class TreeMultiOut(NamedTuple):
    accepted: object        # [B]
    out_tokens: object      # [B, Dmax+1]
    accepted_nodes: object  # [B, Dmax]
    accept_prob: object     # [B, N], -1 for untested nodes
    status: object          # [1]


def tree_verify_multi(target, draft, parent, node_token, u_accept, u_sample, Dmax: int,
                      lam: float = 0.0, temperature: float = 1.0, space: str = "prob",
                      stream=None, workspace=None, blocks_per_tree: int = 0) -> TreeMultiOut:
    """sv_tree_verify_multi: target / draft [B, N+1, V], parent / node_token [B, N],
    u_accept [B, N] (one per node), u_sample [B].  blocks_per_tree other than 0
    calls sv_tree_verify_multi_ex with it."""
    torch = _torch()
    if space not in MIX_SPACES:
        raise ValueError(f"space must be one of {sorted(MIX_SPACES)}, got {space!r}")
    B, N1, V = target.shape
    N = N1 - 1
    ld_t = _rows(target, B, N + 1, V, "target")
    ld_q = _rows(draft, B, N + 1, V, "draft")
    if draft.dtype != target.dtype:
        raise TypeError("target and draft logits must share a dtype")
    _i32(parent, (B, N), "parent")
    _i32(node_token, (B, N), "node_token")
    _f32(u_accept, (B, N), "u_accept")
    _f32(u_sample, (B,), "u_sample")
    dev = target.device
    out = TreeMultiOut(torch.empty(B, dtype=torch.int32, device=dev),
                       torch.empty(B, Dmax + 1, dtype=torch.int32, device=dev),
                       torch.empty(B, max(Dmax, 0), dtype=torch.int32, device=dev),
                       torch.empty(B, N, dtype=torch.float32, device=dev),
                       torch.empty(1, dtype=torch.int32, device=dev))
    ws = workspace if workspace is not None else torch.empty(
        max(int(lib().sv_tree_multi_workspace_bytes(B, N, V)), 16), dtype=torch.uint8, device=dev)
    args = [_ptr(target), ld_t, _ptr(draft), ld_q, _dtype_code(target), B, N, V, _ptr(parent),
            _ptr(node_token), _ptr(u_accept), _ptr(u_sample), float(lam), float(temperature),
            MIX_SPACES[space], _ptr(out.accepted), _ptr(out.out_tokens), _ptr(out.accepted_nodes),
            _ptr(out.accept_prob), int(Dmax), _ptr(out.status), _ptr(ws), ws.numel(), _stream(stream)]
    if blocks_per_tree:
        _check(lib().sv_tree_verify_multi_ex(*args, int(blocks_per_tree)), "sv_tree_verify_multi_ex")
    else:
        _check(lib().sv_tree_verify_multi(*args), "sv_tree_verify_multi")
    return out

