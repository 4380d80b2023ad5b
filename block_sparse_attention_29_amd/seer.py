"""Thin Python binding of libseer (ctypes).

Argument marshalling only: every step of the computation runs in the gfx950
kernels behind the C-ABI declared in include/seer.h.  PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: if the library is
missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first so that libseer binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libseer.so")

SEER_OK = 0
SEER_ERR_INVALID_ARG = 1
SEER_ERR_UNSUPPORTED = 2
SEER_ERR_WORKSPACE = 3
SEER_ERR_HIP = 4

SEER_F32 = 0
SEER_BF16 = 1

# Every symbol include/seer.h declares.
EXPORTS = (
    "seer_block_pool_keys",
    "seer_gate_scores_topk",
    "seer_gate_select",
    "seer_learned_gate_select",
    "seer_learned_gated_sparse_decode",
    "seer_sparse_decode_workspace_size",
    "seer_sparse_decode",
    "seer_sparse_decode_partial",
    "seer_sparse_decode_combine",
    "seer_sparse_decode_combine_mode",
    "seer_gated_sparse_decode",
    "seer_gated_sparse_decode_partial",
    "seer_gated_decode_is_fused",
    "seer_gated_sparse_decode_no_alloc",
    "seer_gated_sparse_decode_append",
    "seer_multi_gate_select",
    "seer_multi_sparse_decode_workspace_size",
    "seer_multi_sparse_decode",
    "seer_multi_sparse_decode_partial",
    "seer_multi_sparse_decode_combine",
    "seer_multi_gated_sparse_decode",
    "seer_multi_gated_sparse_decode_partial",
    "seer_keep_blocks",
    "seer_status_str",
    "seer_last_error",
)


SEER_SELECT_TOPK, SEER_SELECT_THRESHOLD = 0, 1


class Select(ctypes.Structure):
    """seer_select: the selection rule (include/seer.h)."""
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("top_k", ctypes.c_void_p),
        ("keep_num", ctypes.c_int32),
        ("keep_den", ctypes.c_int32),
        ("threshold", ctypes.c_double),
        ("force_first", ctypes.c_int32),
        ("force_last", ctypes.c_int32),
        ("unified", ctypes.c_int32),
        ("fuse", ctypes.c_int32),
    ]


SEER_FUSE_AUTO, SEER_FUSE_ALWAYS, SEER_FUSE_NEVER = 0, 1, 2
SEER_COMBINE_AUTO, SEER_COMBINE_PER_UNIT, SEER_COMBINE_PER_HEAD = 0, 1, 2
_FUSE = {None: SEER_FUSE_AUTO, "auto": SEER_FUSE_AUTO, True: SEER_FUSE_ALWAYS,
         "always": SEER_FUSE_ALWAYS, False: SEER_FUSE_NEVER, "never": SEER_FUSE_NEVER}


def make_select(*, top_k: Optional[torch.Tensor] = None, keep=None, threshold=None,
                force_first=False, force_last=False, unified=False, fuse=None) -> Select:
    """seer_select; ``fuse`` None/"auto" (the library's choice), True/"always"
    or False/"never" (whether the gated calls select inside the attention
    kernel)."""
    num, den = keep if keep is not None else (1, 1)
    mode = SEER_SELECT_THRESHOLD if threshold is not None else SEER_SELECT_TOPK
    return Select(mode, None if top_k is None else top_k.data_ptr(), num, den,
                  0.0 if threshold is None else float(threshold), int(force_first),
                  int(force_last), int(unified), _FUSE[fuse])


class GateWeightsC(ctypes.Structure):
    """seer_gate_weights: the learned gate's weights (include/seer.h)."""
    _fields_ = [
        ("w1", ctypes.c_void_p),
        ("w1_scale", ctypes.c_void_p),
        ("b1", ctypes.c_void_p),
        ("wq", ctypes.c_void_p),
        ("hidden", ctypes.c_int32),
    ]


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class KV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
    ]


class SeerError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def _status_name(st: int) -> str:
    if _lib is None:
        return str(st)
    return _lib.seer_status_str(st).decode()


def load(path: str = LIB_PATH):
    """Loads libseer.so (built by ``python -m block_sparse_attention_29_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_29_amd.build`")
    lib = ctypes.CDLL(path)
    SP = ctypes.POINTER(Shape)
    KP = ctypes.POINTER(KV)
    lib.seer_block_pool_keys.argtypes = [SP, KP, _P, _P, _P, _P, _P]
    lib.seer_gate_scores_topk.argtypes = [SP, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P]
    lib.seer_sparse_decode_workspace_size.argtypes = [SP, ctypes.POINTER(ctypes.c_size_t)]
    lib.seer_sparse_decode.argtypes = [SP, _P, KP, _P, _P, _P, _I32, ctypes.c_float, _P, _P, _P,
                                       ctypes.c_size_t, _P]
    lib.seer_sparse_decode_partial.argtypes = [SP, _P, KP, _P, _P, _P, _I32, ctypes.c_float, _P,
                                               ctypes.c_size_t, _P]
    lib.seer_sparse_decode_combine.argtypes = [SP, _P, _P, _P, ctypes.c_size_t, _P]
    lib.seer_sparse_decode_combine_mode.argtypes = [SP, _I32, _P, _P, _P, ctypes.c_size_t, _P]
    RP = ctypes.POINTER(Select)
    lib.seer_gate_select.argtypes = [SP, _P, _P, _P, RP, _I32, _P, _P, _P, _P]
    lib.seer_learned_gate_select.argtypes = [SP, _P, _P, _P, ctypes.POINTER(GateWeightsC), RP,
                                             _I32, _P, _P, _P, _P]
    lib.seer_learned_gated_sparse_decode.argtypes = [SP, _P, KP, _P, _P,
                                                     ctypes.POINTER(GateWeightsC), RP, _I32,
                                                     ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                                     ctypes.c_size_t, _P]
    lib.seer_multi_gate_select.argtypes = [SP, _I32, _P, _P, _P, RP, _I32, _P, _P, _P, _P]
    lib.seer_multi_sparse_decode_workspace_size.argtypes = [SP, _I32,
                                                            ctypes.POINTER(ctypes.c_size_t)]
    lib.seer_multi_sparse_decode.argtypes = [SP, _I32, _P, KP, _P, _P, _P, _I32, ctypes.c_float,
                                             _P, _P, _P, ctypes.c_size_t, _P]
    lib.seer_multi_sparse_decode_partial.argtypes = [SP, _I32, _P, KP, _P, _P, _P, _I32,
                                                     ctypes.c_float, _P, ctypes.c_size_t, _P]
    lib.seer_multi_sparse_decode_combine.argtypes = [SP, _I32, _P, _P, _P, ctypes.c_size_t, _P]
    lib.seer_gated_sparse_decode.argtypes = [SP, _P, KP, _P, _P, RP, _I32, ctypes.c_float, _P,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.seer_gated_sparse_decode_partial.argtypes = [SP, _P, KP, _P, _P, RP, _I32,
                                                     ctypes.c_float, _P, _P, _P, _P,
                                                     ctypes.c_size_t, _P]
    lib.seer_gated_sparse_decode_no_alloc.argtypes = [SP, _P, KP, _P, _P, RP, _I32,
                                                      ctypes.c_float, _P, _P, _P, _P, _P, _P]
    lib.seer_gated_sparse_decode_append.argtypes = [SP, _P, KP, _P, _P, _P, _P, RP, _I32,
                                                    ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                                    ctypes.c_size_t, _P]
    lib.seer_gated_decode_is_fused.argtypes = [SP, _I32, RP, _I32, ctypes.POINTER(ctypes.c_int32)]
    lib.seer_multi_gated_sparse_decode.argtypes = [SP, _I32, _P, KP, _P, _P, RP, _I32,
                                                   ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_size_t, _P]
    lib.seer_multi_gated_sparse_decode_partial.argtypes = [SP, _I32, _P, KP, _P, _P, RP, _I32,
                                                           ctypes.c_float, _P, _P, _P, _P,
                                                           ctypes.c_size_t, _P]
    lib.seer_keep_blocks.argtypes = [_I32, _I32, _I32]
    lib.seer_keep_blocks.restype = _I32
    lib.seer_status_str.argtypes = [_I32]
    lib.seer_status_str.restype = ctypes.c_char_p
    lib.seer_last_error.argtypes = []
    lib.seer_last_error.restype = ctypes.c_char_p
    for name in ("seer_block_pool_keys", "seer_gate_scores_topk", "seer_gate_select",
                 "seer_learned_gate_select", "seer_learned_gated_sparse_decode",
                 "seer_multi_gate_select",
                 "seer_multi_sparse_decode_workspace_size", "seer_multi_sparse_decode",
                 "seer_sparse_decode_workspace_size", "seer_sparse_decode",
                 "seer_sparse_decode_partial", "seer_sparse_decode_combine",
                 "seer_sparse_decode_combine_mode",
                 "seer_gated_sparse_decode", "seer_gated_sparse_decode_partial",
                 "seer_gated_sparse_decode_no_alloc", "seer_gated_sparse_decode_append"):
        getattr(lib, name).restype = _I32
    _lib = lib
    return lib


def _check(st: int):
    if st != SEER_OK:
        raise SeerError(st, _lib.seer_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, dtype) -> Shape:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: SEER_F32, torch.bfloat16: SEER_BF16}[dtype]
    return Shape(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, dtype)


def make_kv(k: torch.Tensor, v: torch.Tensor, page_table: Optional[torch.Tensor] = None) -> KV:
    return KV(k.data_ptr(), v.data_ptr(), None if page_table is None else page_table.data_ptr(),
              0 if page_table is None else k.shape[0])


def _need(t: torch.Tensor, dtype, numel: int, name: str):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name}: want a contiguous {dtype} device tensor of >= {numel} "
                         f"elements, got {t.dtype} {tuple(t.shape)} on {t.device}")


def _need_q(shape: Shape, q: Optional[torch.Tensor], tokens: int = 1):
    """q must hold exactly [B][tokens][Hq][d] elements of the shape's dtype (a
    NULL q is left to the library, which rejects it)."""
    if q is None:
        return
    want = {SEER_F32: torch.float32, SEER_BF16: torch.bfloat16}.get(shape.dtype)
    n = shape.batch * tokens * shape.num_q_heads * shape.head_dim
    if not q.is_cuda or q.dtype != want or not q.is_contiguous() or q.numel() != n:
        raise ValueError(f"q: want a contiguous {want} device tensor of {n} elements "
                         f"([B][{tokens}][Hq][d]), got {q.dtype} {tuple(q.shape)} on {q.device}")


# ------------------------------------------------------------------ calls

def keep_blocks(n_blocks: int, keep_num: int, keep_den: int) -> int:
    return int(load().seer_keep_blocks(n_blocks, keep_num, keep_den))


def block_pool_keys(shape: Shape, kv: KV, lens_old: Optional[torch.Tensor],
                    lens_new: torch.Tensor, pooled: torch.Tensor, open_sum: torch.Tensor):
    lib = load()
    U = shape.batch * shape.num_kv_heads
    _need(lens_new, torch.int32, shape.batch, "lens_new")
    if lens_old is not None:
        _need(lens_old, torch.int32, shape.batch, "lens_old")
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(open_sum, torch.float64, U * shape.head_dim, "open_sum")
    _check(lib.seer_block_pool_keys(ctypes.byref(shape), ctypes.byref(kv), _ptr(lens_old),
                                    _ptr(lens_new), _ptr(pooled), _ptr(open_sum), _stream()))


def gate_scores_topk(shape: Shape, q: torch.Tensor, pooled: torch.Tensor, lens: torch.Tensor,
                     top_k: Optional[torch.Tensor], keep_num: int, keep_den: int, k_max: int,
                     scores: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor):
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    if top_k is not None:
        _need(top_k, torch.int32, shape.batch, "top_k")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _check(lib.seer_gate_scores_topk(ctypes.byref(shape), _ptr(q), _ptr(pooled), _ptr(lens),
                                     _ptr(top_k), keep_num, keep_den, k_max, _ptr(scores),
                                     _ptr(sel_idx), _ptr(sel_cnt), _stream()))


def gate_select(shape: Shape, q: torch.Tensor, pooled: torch.Tensor, lens: torch.Tensor,
                rule: Select, k_max: int, scores: torch.Tensor, sel_idx: torch.Tensor,
                sel_cnt: torch.Tensor):
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _check(lib.seer_gate_select(ctypes.byref(shape), _ptr(q), _ptr(pooled), _ptr(lens),
                                ctypes.byref(rule), k_max, _ptr(scores), _ptr(sel_idx),
                                _ptr(sel_cnt), _stream()))


def learned_gate_select(shape: Shape, q: torch.Tensor, pooled: torch.Tensor,
                        lens: torch.Tensor, weights, rule: Select, k_max: int,
                        scores: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor):
    """seer_learned_gate_select; ``weights`` has device tensors w1 (int8), w1_scale,
    b1, wq (float32) in the layouts of include/seer.h."""
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    H = int(weights.w1.shape[-2])
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _need(weights.w1, torch.int8, shape.num_kv_heads * H * shape.head_dim, "w1")
    _need(weights.w1_scale, torch.float32, shape.num_kv_heads * H, "w1_scale")
    _need(weights.b1, torch.float32, shape.num_kv_heads * H, "b1")
    _need(weights.wq, torch.float32, shape.num_kv_heads * H * shape.head_dim, "wq")
    w = GateWeightsC(_ptr(weights.w1), _ptr(weights.w1_scale), _ptr(weights.b1),
                     _ptr(weights.wq), H)
    _check(lib.seer_learned_gate_select(ctypes.byref(shape), _ptr(q), _ptr(pooled), _ptr(lens),
                                        ctypes.byref(w), ctypes.byref(rule), k_max,
                                        _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt), _stream()))


def _gate_weights_c(shape: Shape, weights) -> GateWeightsC:
    H = int(weights.w1.shape[-2])
    _need(weights.w1, torch.int8, shape.num_kv_heads * H * shape.head_dim, "w1")
    _need(weights.w1_scale, torch.float32, shape.num_kv_heads * H, "w1_scale")
    _need(weights.b1, torch.float32, shape.num_kv_heads * H, "b1")
    _need(weights.wq, torch.float32, shape.num_kv_heads * H * shape.head_dim, "wq")
    return GateWeightsC(_ptr(weights.w1), _ptr(weights.w1_scale), _ptr(weights.b1),
                        _ptr(weights.wq), H)


def learned_gated_sparse_decode(shape: Shape, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                                pooled: torch.Tensor, weights, rule: Select, k_max: int,
                                scores: torch.Tensor, sel_idx: torch.Tensor,
                                sel_cnt: torch.Tensor, out: Optional[torch.Tensor],
                                lse: Optional[torch.Tensor], workspace: torch.Tensor,
                                softmax_scale: float = 0.0):
    """seer_learned_gated_sparse_decode: the learned gate's step (gate, selection,
    sparse decode, merge; out=None stops before the merge)."""
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    if out is not None:
        _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    w = _gate_weights_c(shape, weights)
    _check(lib.seer_learned_gated_sparse_decode(
        ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
        ctypes.byref(w), ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx),
        _ptr(sel_cnt), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))


def sparse_decode_workspace_size(shape: Shape) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.seer_sparse_decode_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def alloc_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    return torch.empty(sparse_decode_workspace_size(shape), dtype=torch.uint8, device=device)


def sparse_decode(shape: Shape, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                  sel_idx: Optional[torch.Tensor], sel_cnt: Optional[torch.Tensor], k_max: int,
                  out: torch.Tensor, lse: Optional[torch.Tensor], workspace: torch.Tensor,
                  softmax_scale: float = 0.0):
    lib = load()
    _need_q(shape, q)
    _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    _check(lib.seer_sparse_decode(ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens),
                                  _ptr(sel_idx), _ptr(sel_cnt), k_max, softmax_scale, _ptr(out),
                                  _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))


def multi_gate_select(shape: Shape, tokens: int, q: torch.Tensor, pooled: torch.Tensor,
                      lens: torch.Tensor, rule: Select, k_max: int, scores: torch.Tensor,
                      sel_idx: torch.Tensor, sel_cnt: torch.Tensor):
    """seer_multi_gate_select: q is [B][tokens][Hq][d]."""
    lib = load()
    _need_q(shape, q, tokens)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _check(lib.seer_multi_gate_select(ctypes.byref(shape), tokens, _ptr(q), _ptr(pooled),
                                      _ptr(lens), ctypes.byref(rule), k_max, _ptr(scores),
                                      _ptr(sel_idx), _ptr(sel_cnt), _stream()))


def multi_decode_workspace_size(shape: Shape, tokens: int) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.seer_multi_sparse_decode_workspace_size(ctypes.byref(shape), tokens,
                                                       ctypes.byref(n)))
    return int(n.value)


def multi_sparse_decode(shape: Shape, tokens: int, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                        sel_idx: Optional[torch.Tensor], sel_cnt: Optional[torch.Tensor],
                        k_max: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                        workspace: torch.Tensor, softmax_scale: float = 0.0):
    """seer_multi_sparse_decode: q [B][tokens][Hq][d]; out [B][tokens][Hq][d]; lse [B][tokens][Hq]."""
    lib = load()
    _need_q(shape, q, tokens)
    rows = shape.batch * tokens * shape.num_q_heads
    _need(out, torch.float32, rows * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, rows, "lse")
    _check(lib.seer_multi_sparse_decode(ctypes.byref(shape), tokens, _ptr(q), ctypes.byref(kv),
                                        _ptr(lens), _ptr(sel_idx), _ptr(sel_cnt), k_max,
                                        softmax_scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel(), _stream()))


def multi_sparse_decode_partial(shape: Shape, tokens: int, q: torch.Tensor, kv: KV,
                                lens: torch.Tensor, sel_idx: Optional[torch.Tensor],
                                sel_cnt: Optional[torch.Tensor], k_max: int,
                                workspace: torch.Tensor, softmax_scale: float = 0.0):
    """seer_multi_sparse_decode_partial: the partial records of the T tokens."""
    lib = load()
    _need_q(shape, q, tokens)
    _check(lib.seer_multi_sparse_decode_partial(
        ctypes.byref(shape), tokens, _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(sel_idx),
        _ptr(sel_cnt), k_max, softmax_scale, _ptr(workspace), workspace.numel(), _stream()))


def multi_sparse_decode_combine(shape: Shape, tokens: int, out: torch.Tensor,
                                lse: Optional[torch.Tensor], workspace: torch.Tensor):
    """seer_multi_sparse_decode_combine: out [B][tokens][Hq][d], lse [B][tokens][Hq]."""
    lib = load()
    rows = shape.batch * tokens * shape.num_q_heads
    _need(out, torch.float32, rows * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, rows, "lse")
    _check(lib.seer_multi_sparse_decode_combine(ctypes.byref(shape), tokens, _ptr(out), _ptr(lse),
                                                _ptr(workspace), workspace.numel(), _stream()))


def sparse_decode_partial(shape: Shape, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                          sel_idx: Optional[torch.Tensor], sel_cnt: Optional[torch.Tensor],
                          k_max: int, workspace: torch.Tensor, softmax_scale: float = 0.0):
    lib = load()
    _need_q(shape, q)
    _check(lib.seer_sparse_decode_partial(ctypes.byref(shape), _ptr(q), ctypes.byref(kv),
                                          _ptr(lens), _ptr(sel_idx), _ptr(sel_cnt), k_max,
                                          softmax_scale, _ptr(workspace), workspace.numel(),
                                          _stream()))


def sparse_decode_combine(shape: Shape, out: torch.Tensor, lse: Optional[torch.Tensor],
                          workspace: torch.Tensor, mode: int = SEER_COMBINE_AUTO):
    """seer_sparse_decode_combine, or seer_sparse_decode_combine_mode with an
    explicit mode (SEER_COMBINE_PER_UNIT / SEER_COMBINE_PER_HEAD)."""
    lib = load()
    _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    if mode == SEER_COMBINE_AUTO:
        _check(lib.seer_sparse_decode_combine(ctypes.byref(shape), _ptr(out), _ptr(lse),
                                              _ptr(workspace), workspace.numel(), _stream()))
    else:
        _check(lib.seer_sparse_decode_combine_mode(ctypes.byref(shape), mode, _ptr(out),
                                                   _ptr(lse), _ptr(workspace),
                                                   workspace.numel(), _stream()))


def gated_decode_path(shape: Shape, rule: Select, k_max: int, tokens: int = 1) -> int:
    """seer_gated_decode_is_fused's value: 1 if gated_sparse_decode (tokens = 1)
    or multi_gated_sparse_decode scores and selects inside the attention
    kernel for this shape and rule on the current device, 2 if the score
    kernel scores first and the attention kernel selects, 0 if the gate
    kernel(s) run first."""
    lib = load()
    f = ctypes.c_int32(0)
    _check(lib.seer_gated_decode_is_fused(ctypes.byref(shape), tokens, ctypes.byref(rule), k_max,
                                          ctypes.byref(f)))
    return int(f.value)


def gated_decode_is_fused(shape: Shape, rule: Select, k_max: int, tokens: int = 1) -> bool:
    """Whether gated_sparse_decode (tokens = 1) or multi_gated_sparse_decode
    selects inside the attention kernel for this shape and rule on the
    current device (gated_decode_path nonzero)."""
    return gated_decode_path(shape, rule, k_max, tokens) != 0


def multi_gated_sparse_decode(shape: Shape, tokens: int, q: torch.Tensor, kv: KV,
                              lens: torch.Tensor, pooled: torch.Tensor, rule: Select, k_max: int,
                              scores: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                              out: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                              workspace: torch.Tensor, softmax_scale: float = 0.0):
    """seer_multi_gated_sparse_decode (out None: the _partial entry alone)."""
    lib = load()
    _need_q(shape, q, tokens)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    if out is None:
        _check(lib.seer_multi_gated_sparse_decode_partial(
            ctypes.byref(shape), tokens, _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
            ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
            _ptr(workspace), workspace.numel(), _stream()))
        return
    rows = shape.batch * tokens * shape.num_q_heads
    _need(out, torch.float32, rows * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, rows, "lse")
    _check(lib.seer_multi_gated_sparse_decode(
        ctypes.byref(shape), tokens, _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
        ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))


def gated_sparse_decode(shape: Shape, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                        pooled: torch.Tensor, rule: Select, k_max: int, scores: torch.Tensor,
                        sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                        out: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                        workspace: torch.Tensor, softmax_scale: float = 0.0):
    """Gate, selection and sparse decode in two launches; out=None stops after
    the first (the partial results stay in the workspace for
    sparse_decode_combine)."""
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    if out is None:
        _check(lib.seer_gated_sparse_decode_partial(
            ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
            ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
            _ptr(workspace), workspace.numel(), _stream()))
        return
    _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    _check(lib.seer_gated_sparse_decode(
        ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
        ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))


def gated_sparse_decode_no_alloc(shape: Shape, q: torch.Tensor, kv: KV, lens: torch.Tensor,
                                 pooled: torch.Tensor, rule: Select, k_max: int,
                                 scores: torch.Tensor, sel_idx: torch.Tensor,
                                 sel_cnt: torch.Tensor, out: torch.Tensor,
                                 lse: Optional[torch.Tensor], softmax_scale: float = 0.0):
    """seer_gated_sparse_decode_no_alloc: the gated decode step with the
    library's static device scratch instead of a workspace."""
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    _check(lib.seer_gated_sparse_decode_no_alloc(
        ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens), _ptr(pooled),
        ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(out), _ptr(lse), _stream()))


def gated_sparse_decode_append(shape: Shape, q: torch.Tensor, kv: KV, lens_old: torch.Tensor,
                               lens: torch.Tensor, pooled: torch.Tensor, open_sum: torch.Tensor,
                               rule: Select, k_max: int, scores: torch.Tensor,
                               sel_idx: torch.Tensor, sel_cnt: torch.Tensor, out: torch.Tensor,
                               lse: Optional[torch.Tensor], workspace: torch.Tensor,
                               softmax_scale: float = 0.0):
    """seer_gated_sparse_decode_append: pool the tokens lens_old .. lens - 1,
    then the gated decode step at lens."""
    lib = load()
    _need_q(shape, q)
    U = shape.batch * shape.num_kv_heads
    _need(lens_old, torch.int32, shape.batch, "lens_old")
    _need(lens, torch.int32, shape.batch, "lens")
    _need(pooled, torch.float32, U * shape.head_dim * shape.max_blocks, "pooled")
    _need(open_sum, torch.float64, U * shape.head_dim, "open_sum")
    _need(scores, torch.float64, U * shape.max_blocks, "scores")
    _need(sel_idx, torch.int32, U * k_max, "sel_idx")
    _need(sel_cnt, torch.int32, U, "sel_cnt")
    _need(out, torch.float32, shape.batch * shape.num_q_heads * shape.head_dim, "out")
    if lse is not None:
        _need(lse, torch.float32, shape.batch * shape.num_q_heads, "lse")
    _check(lib.seer_gated_sparse_decode_append(
        ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(lens_old), _ptr(lens), _ptr(pooled),
        _ptr(open_sum), ctypes.byref(rule), k_max, softmax_scale, _ptr(scores), _ptr(sel_idx),
        _ptr(sel_cnt), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
