"""ctypes binding of the C ABI in include/gqa_decode.h (marshalling only)."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_decode.so")
if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is not built; build it with `python -m decode_attention_08_amd.build` "
        "(or __graft_entry__.build()). There is no non-HIP fallback.")

lib = ctypes.CDLL(library_path)

GQA_F16 = 0
GQA_BF16 = 1

EXPORTED_SYMBOLS = ("gqa_policy_default", "gqa_policy_pages", "gqa_decode_workspace_size",
                    "gqa_decode", "gqa_decode_xsplit", "gqa_decode_contiguous",
                    "gqa_status_string")
X = 8   # elements per 16-byte vector of the x-split K layout


class Policy(ctypes.Structure):
    """gqa_policy_t: partition_size, v1_max_ctx, phases (0/3 both, 1 partition, 2 merge)."""
    _fields_ = [("partition_size", ctypes.c_int32), ("v1_max_ctx", ctypes.c_int32),
                ("phases", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def __repr__(self):
        return (f"Policy(partition_size={self.partition_size}, v1_max_ctx={self.v1_max_ctx}, "
                f"phases={self.phases})")


_P = ctypes.c_void_p
_I = ctypes.c_int
lib.gqa_policy_default.argtypes = [ctypes.POINTER(Policy)]
lib.gqa_policy_default.restype = None
lib.gqa_policy_pages.argtypes = [ctypes.POINTER(Policy)]
lib.gqa_policy_pages.restype = None
lib.gqa_decode_workspace_size.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(Policy)]
lib.gqa_decode_workspace_size.restype = ctypes.c_size_t
lib.gqa_decode.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                           _P, ctypes.c_size_t, ctypes.POINTER(Policy), _P]
lib.gqa_decode.restype = _I
lib.gqa_decode_xsplit.argtypes = lib.gqa_decode.argtypes
lib.gqa_decode_xsplit.restype = _I
lib.gqa_decode_contiguous.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                      _P, ctypes.c_size_t, ctypes.POINTER(Policy), _P]
lib.gqa_decode_contiguous.restype = _I
lib.gqa_status_string.argtypes = [_I]
lib.gqa_status_string.restype = ctypes.c_char_p


class GqaError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(status_string(status))


def status_string(status: int) -> str:
    return lib.gqa_status_string(int(status)).decode()


def policy_default(**overrides) -> Policy:
    p = Policy()
    lib.gqa_policy_default(ctypes.byref(p))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def policy_pages(**overrides) -> Policy:
    p = Policy()
    lib.gqa_policy_pages(ctypes.byref(p))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def _pref(policy: Optional[Policy]):
    return None if policy is None else ctypes.byref(policy)


def workspace_size(num_seqs: int, h_q: int, h_kv: int, d_head: int, max_ctx: int,
                   policy: Optional[Policy] = None) -> int:
    return int(lib.gqa_decode_workspace_size(num_seqs, h_q, h_kv, d_head, max_ctx, _pref(policy)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return GQA_F16
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; fp16 or bf16 expected")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _common(q, tensors, out):
    for name, t in tensors.items():
        _require(t.is_cuda, f"{name} must be a GPU tensor")
        _require(t.is_contiguous(), f"{name} must be contiguous")
        _require(t.device == q.device, f"{name} is on {t.device}, q on {q.device}")
    _require(q.dim() == 3, "q must be [num_seqs, h_q, d_head]")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
             and out.device == q.device, "out must match q")
    return out


def _workspace(workspace, need, device):
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _require(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous GPU tensor")
    return workspace, workspace.numel() * workspace.element_size()


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_table: torch.Tensor, ctx_lens: torch.Tensor, *, scale: Optional[float] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           policy: Optional[Policy] = None, stream=None) -> torch.Tensor:
    """Paged GQA decode: q [B, h_q, d], k/v [num_blocks, bs, h_kv, d],
    block_table [B, max_blocks] int32, ctx_lens [B] int32 -> out [B, h_q, d]."""
    out = _common(q, {"q": q, "k_cache": k_cache, "v_cache": v_cache,
                      "block_table": block_table, "ctx_lens": ctx_lens}, out)
    _, bs, h_kv = _paged_shapes(q, k_cache, v_cache, block_table, ctx_lens, False)
    B, h_q, d = q.shape
    max_blocks = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = workspace_size(B, h_q, h_kv, d, max_blocks * bs, policy)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    st = lib.gqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens),
                        _ptr(out), B, max_blocks, h_q, h_kv, d, bs, scale, _dtype_code(q),
                        _ptr(workspace), ws_bytes, _pref(policy), _stream(stream, q.device))
    if st != 0:
        raise GqaError(st)
    return out


def _paged_shapes(q, k_cache, v_cache, block_table, ctx_lens, xsplit: bool):
    """(num_blocks, block_size, h_kv) of a paged cache pair, checked."""
    _require(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q, k, v must share a dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2, "block_table: int32 [B, max_blocks]")
    _require(ctx_lens.dtype == torch.int32 and ctx_lens.dim() == 1, "ctx_lens: int32 [B]")
    B, h_q, d = q.shape
    if xsplit:
        _require(k_cache.dim() == 5 and v_cache.dim() == 4,
                 "x-split k must be [num_blocks, h_kv, d/8, bs, 8] and v [num_blocks, h_kv, d, bs]")
        nb, h_kv, dx, bs, x = k_cache.shape
        _require(x == X and dx * X == d, "x-split k: last dims must be (d/8, bs, 8)")
        _require(tuple(v_cache.shape) == (nb, h_kv, d, bs), "x-split v must be [num_blocks, h_kv, d, bs]")
    else:
        _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "k/v must be [num_blocks, bs, h_kv, d]")
        nb, bs, h_kv, dk = k_cache.shape
        _require(dk == d, "head dims differ")
    _require(block_table.shape[0] == B and ctx_lens.shape[0] == B, "batch sizes differ")
    return nb, bs, h_kv


def decode_xsplit(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_table: torch.Tensor, ctx_lens: torch.Tensor, *,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, policy: Optional[Policy] = None,
                  stream=None) -> torch.Tensor:
    """Paged GQA decode over the x-split layout: k [num_blocks, h_kv, d/8, bs, 8],
    v [num_blocks, h_kv, d, bs]; otherwise as decode()."""
    out = _common(q, {"q": q, "k_cache": k_cache, "v_cache": v_cache,
                      "block_table": block_table, "ctx_lens": ctx_lens}, out)
    _, bs, h_kv = _paged_shapes(q, k_cache, v_cache, block_table, ctx_lens, True)
    B, h_q, d = q.shape
    max_blocks = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = workspace_size(B, h_q, h_kv, d, max_blocks * bs, policy)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    st = lib.gqa_decode_xsplit(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                               _ptr(ctx_lens), _ptr(out), B, max_blocks, h_q, h_kv, d, bs, scale,
                               _dtype_code(q), _ptr(workspace), ws_bytes, _pref(policy),
                               _stream(stream, q.device))
    if st != 0:
        raise GqaError(st)
    return out


def decode_contiguous(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, policy: Optional[Policy] = None,
                      stream=None) -> torch.Tensor:
    """Contiguous GQA decode: q [B, h_q, d], k/v [B, S, h_kv, d] -> out [B, h_q, d]."""
    out = _common(q, {"q": q, "k": k, "v": v}, out)
    _require(k.dim() == 4 and k.shape == v.shape, "k/v must be [B, S, h_kv, d]")
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    B, h_q, d = q.shape
    Bk, S, h_kv, dk = k.shape
    _require(Bk == B and dk == d, "k/v shape does not match q")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = workspace_size(B, h_q, h_kv, d, S, policy)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    st = lib.gqa_decode_contiguous(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, h_q, h_kv, d,
                                   scale, _dtype_code(q), _ptr(workspace), ws_bytes,
                                   _pref(policy), _stream(stream, q.device))
    if st != 0:
        raise GqaError(st)
    return out


class PreparedCall:
    """A decode call with its arguments marshalled once, for tight loops.

    ``call(k=None, v=None, phases=None)`` invokes the C entry point again with
    the same buffers, optionally another K/V pair of identical shape and
    dtype, and optionally a different ``phases`` value.  The caller keeps
    every tensor alive.
    """

    def __init__(self, fn, args, k_index, policy: Policy, keep):
        self._fn = fn
        self._args = list(args)
        self._k_index = k_index
        self._policy = Policy(policy.partition_size, policy.v1_max_ctx, policy.phases, 0)
        self._pol_index = len(args) - 2
        self._args[self._pol_index] = ctypes.byref(self._policy)
        self._keep = keep

    def __call__(self, k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                 phases: Optional[int] = None) -> None:
        args = self._args
        if k is not None:
            args = list(args)
            args[self._k_index] = k.data_ptr()
            args[self._k_index + 1] = v.data_ptr()
        if phases is not None:
            self._policy.phases = phases
        st = self._fn(*args)
        if st != 0:
            raise GqaError(st)


def prepare(q, k, v, *, block_table=None, ctx_lens=None, scale=None, out=None,
            workspace=None, policy: Optional[Policy] = None, stream=None,
            xsplit: bool = False) -> PreparedCall:
    """Validate once (same checks as decode / decode_xsplit / decode_contiguous)
    and return a PreparedCall.  Paged when block_table is given (x-split layout
    with xsplit=True), contiguous otherwise."""
    policy = policy_default() if policy is None else policy
    if block_table is not None:
        out = _common(q, {"q": q, "k_cache": k, "v_cache": v, "block_table": block_table,
                          "ctx_lens": ctx_lens}, out)
        _, bs, h_kv = _paged_shapes(q, k, v, block_table, ctx_lens, xsplit)
        B, h_q, d = q.shape
        max_blocks = block_table.shape[1]
        need = workspace_size(B, h_q, h_kv, d, max_blocks * bs, policy)
        workspace, ws_bytes = _workspace(workspace, need, q.device)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(block_table), _ptr(ctx_lens), _ptr(out), B,
                max_blocks, h_q, h_kv, d, bs, scale, _dtype_code(q), _ptr(workspace), ws_bytes,
                None, _stream(stream, q.device))
        fn = lib.gqa_decode_xsplit if xsplit else lib.gqa_decode
        return PreparedCall(fn, args, 1, policy, (q, k, v, block_table, ctx_lens, out, workspace))
    _require(not xsplit, "the x-split layout is a paged layout (block_table required)")
    out = _common(q, {"q": q, "k": k, "v": v}, out)
    B, h_q, d = q.shape
    _, S, h_kv, _ = k.shape
    need = workspace_size(B, h_q, h_kv, d, S, policy)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, h_q, h_kv, d, scale, _dtype_code(q),
            _ptr(workspace), ws_bytes, None, _stream(stream, q.device))
    return PreparedCall(lib.gqa_decode_contiguous, args, 1, policy, (q, k, v, out, workspace))
