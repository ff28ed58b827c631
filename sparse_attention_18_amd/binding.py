"""ctypes binding of libdsa.so (see include/dsa.h): argument marshalling only.

Every entry point takes torch tensors that already live on the GPU, checks
their dtype / shape / contiguity, and passes raw device pointers and the
current HIP stream to the C ABI.  All compute happens in the library's HIP
kernels; there is no fallback.  If libdsa.so is missing or fails to load, the
first call raises ``DsaLibraryError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")
_lock = threading.Lock()
_lib = None

DSA_OK = 0
DSA_ERR_INVALID_ARGUMENT = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_WORKSPACE = 3
DSA_ERR_HIP = 4
WS_TOPK, WS_ATTN, WS_FORWARD, WS_INDEXER_BWD, WS_FORWARD_FUSED, WS_ATTN_PREFILL = 0, 1, 2, 3, 4, 5

EXPORTED = ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_forward",
            "dsa_indexer_scores_paged", "dsa_sparse_attn_paged", "dsa_forward_paged",
            "dsa_indexer_align_loss", "dsa_indexer_backward", "dsa_workspace_bytes", "dsa_last_error", "dsa_version",
            "dsa_forward_noalloc", "dsa_forward_fused", "dsa_sparse_attn_prefill")
NOALLOC_SCRATCH_BYTES = 256 << 20      # DSA_NOALLOC_SCRATCH_BYTES in include/dsa.h


class DsaLibraryError(RuntimeError):
    """libdsa.so is missing or could not be loaded."""


class DsaError(RuntimeError):
    """A libdsa call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libdsa status {status}: {message}")
        self.status = status


class DsaProblem(ctypes.Structure):
    """Mirror of ``dsa_problem`` in include/dsa.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("max_q_len", ctypes.c_int64),
        ("max_kv_len", ctypes.c_int64),
        ("q_offsets", ctypes.c_void_p),
        ("kv_offsets", ctypes.c_void_p),
        ("q_pos0", ctypes.c_void_p),
    ]


class DsaPagedKV(ctypes.Structure):
    """Mirror of ``dsa_paged_kv`` in include/dsa.h."""

    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
    ]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdsa.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(_LIB_PATH)
        return _lib


def open_library(path: str):
    """Load a build of the library at `path` (libdsa.so or one of its
    variants, e.g. libdsa_debug.so) and declare its signatures."""
    if not os.path.exists(path):
        raise DsaLibraryError(f"{path} is missing: build it with `python -m sparse_attention_18_amd.build`")
    try:
        lib = ctypes.CDLL(path)
    except OSError as e:
        raise DsaLibraryError(f"cannot load {path}: {e}") from e
    P = ctypes.POINTER(DsaProblem)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.dsa_indexer_scores.argtypes = [P, vp, vp, vp, vp, vp, vp, i64, vp]
    lib.dsa_topk.argtypes = [P, vp, i64, vp, vp, sz, vp]
    lib.dsa_sparse_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    G = ctypes.POINTER(DsaPagedKV)
    lib.dsa_indexer_scores_paged.argtypes = [P, G, vp, vp, vp, vp, vp, vp, i64, vp]
    lib.dsa_sparse_attn_paged.argtypes = [P, G, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_forward_paged.argtypes = [P, G, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_indexer_align_loss.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, i64, vp]
    lib.dsa_indexer_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.dsa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dsa_forward_fused.argtypes = [P, G, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_sparse_attn_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    for name in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_forward",
                 "dsa_indexer_scores_paged", "dsa_sparse_attn_paged", "dsa_forward_paged",
                 "dsa_indexer_align_loss", "dsa_indexer_backward", "dsa_forward_noalloc",
                 "dsa_forward_fused", "dsa_sparse_attn_prefill"):
        getattr(lib, name).restype = ctypes.c_int
    lib.dsa_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.dsa_workspace_bytes.restype = sz
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_version.argtypes = []
    lib.dsa_version.restype = ctypes.c_char_p
    return lib


def _check(status: int):
    if status != DSA_OK:
        msg = load_library().dsa_last_error().decode(errors="replace")
        raise DsaError(status, msg)


def _ptr(t: torch.Tensor | None, dtype, name: str, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Problem:
    """A ``dsa_problem`` with its device offset arrays kept alive.

    ``q_offsets`` / ``kv_offsets`` (length B+1) and ``q_pos0`` (length B) are
    Python lists; they are copied to ``device`` as int32 tensors.
    """

    def __init__(self, *, q_offsets, kv_offsets, q_pos0, idx_heads, idx_dim, heads,
                 d_latent, d_rope, topk, softmax_scale, device="cuda"):
        B = len(q_pos0)
        if len(q_offsets) != B + 1 or len(kv_offsets) != B + 1:
            raise ValueError("q_offsets and kv_offsets need batch + 1 entries")
        self.q_offsets_list = [int(x) for x in q_offsets]
        self.kv_offsets_list = [int(x) for x in kv_offsets]
        self.q_pos0_list = [int(x) for x in q_pos0]
        self._q_off = torch.tensor(self.q_offsets_list, dtype=torch.int32, device=device)
        self._kv_off = torch.tensor(self.kv_offsets_list, dtype=torch.int32, device=device)
        self._pos0 = torch.tensor(self.q_pos0_list, dtype=torch.int32, device=device)
        q_lens = [self.q_offsets_list[i + 1] - self.q_offsets_list[i] for i in range(B)]
        kv_lens = [self.kv_offsets_list[i + 1] - self.kv_offsets_list[i] for i in range(B)]
        self.c = DsaProblem(
            batch=B, idx_heads=idx_heads, idx_dim=idx_dim, heads=heads, d_latent=d_latent,
            d_rope=d_rope, topk=topk, softmax_scale=softmax_scale,
            total_q=self.q_offsets_list[-1], total_kv=self.kv_offsets_list[-1],
            max_q_len=max(q_lens) if q_lens else 0, max_kv_len=max(kv_lens) if kv_lens else 0,
            q_offsets=self._q_off.data_ptr(), kv_offsets=self._kv_off.data_ptr(),
            q_pos0=self._pos0.data_ptr())

    @classmethod
    def from_workload(cls, wl, inputs: dict, device="cuda", q_rows=None, q_pos0=None):
        """Problem for a workload's generated inputs, optionally restricted to
        the query rows ``q_rows`` (a slice) of a single sequence starting at
        position ``q_pos0`` (chunked prefill)."""
        if q_rows is None:
            q_off, pos0 = inputs["q_offsets"], inputs["q_pos0"]
        else:
            q_off, pos0 = [0, q_rows.stop - q_rows.start], [q_pos0]
        kv_off = inputs["kv_offsets"]
        if q_rows is not None:
            kv_off = [0, q_rows.stop]     # the causal prefix of the chunk
        return cls(q_offsets=q_off, kv_offsets=kv_off, q_pos0=pos0, idx_heads=wl.idx_heads,
                   idx_dim=wl.idx_dim, heads=wl.heads, d_latent=wl.d_latent, d_rope=wl.d_rope,
                   topk=wl.topk, softmax_scale=wl.softmax_scale, device=device)

    @property
    def total_q(self):
        return self.c.total_q

    @property
    def total_kv(self):
        return self.c.total_kv

    @property
    def max_kv_len(self):
        return self.c.max_kv_len

    def ld_scores(self) -> int:
        """Smallest valid leading dimension for a scores matrix (multiple of 64)."""
        return max(64, (self.max_kv_len + 63) // 64 * 64)


def version() -> str:
    return load_library().dsa_version().decode()


def workspace_bytes(prob: Problem, which: int) -> int:
    n = load_library().dsa_workspace_bytes(ctypes.byref(prob.c), which)
    if n == ctypes.c_size_t(-1).value:
        _check(DSA_ERR_INVALID_ARGUMENT)
    return int(n)


def indexer_scores(prob: Problem, q_fp8, q_scale, w, k_fp8, k_scale, scores, ld=None, stream=None):
    """Stage 1 (dsa_indexer_scores): writes scores[r, s] for s <= pos(r)."""
    c = prob.c
    ld = prob.ld_scores() if ld is None else int(ld)
    args = (_ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
            _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
            _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
            _ptr(k_fp8, torch.uint8, "k_fp8", (c.total_kv, c.idx_dim)),
            _ptr(k_scale, torch.float32, "k_scale", (c.total_kv,)),
            _ptr(scores, torch.float32, "scores", (c.total_q, ld)))
    _check(load_library().dsa_indexer_scores(ctypes.byref(c), *args, ld, _stream(stream)))


def topk(prob: Problem, scores, idx, ld=None, workspace=None, stream=None):
    """Stage 2 (dsa_topk): ascending top-k positions per query row, -1 padded."""
    c = prob.c
    ld = prob.ld_scores() if ld is None else int(ld)
    ws_ptr = _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_n = workspace.numel() if workspace is not None else 0
    _check(load_library().dsa_topk(
        ctypes.byref(c), _ptr(scores, torch.float32, "scores", (c.total_q, ld)), ld,
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)), ws_ptr, ws_n, _stream(stream)))


def sparse_attn(prob: Problem, q, kv, idx, out, lse=None, workspace=None, stream=None):
    """Stage 3 (dsa_sparse_attn): attention of every head over its token's selected rows."""
    c = prob.c
    D = c.d_latent + c.d_rope
    ws_ptr = _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_n = workspace.numel() if workspace is not None else 0
    _check(load_library().dsa_sparse_attn(
        ctypes.byref(c), _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv, torch.bfloat16, "kv", (c.total_kv, D)),
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)), ws_ptr, ws_n, _stream(stream)))


MHA_NOPE, MHA_ROPE, MHA_V = 128, 64, 128   # per-head widths of the prefill form


def sparse_attn_prefill(prob: Problem, q, k_nope, k_rope, v, idx, out, lse=None, workspace=None,
                        stream=None):
    """Stage 3 in prefill mode (dsa_sparse_attn_prefill): per-head keys and values,
    the selection applied as a mask.  ``workspace`` is a uint8 GPU tensor of at least
    ``workspace_bytes(prob, WS_ATTN_PREFILL)`` bytes."""
    c = prob.c
    if workspace is None:
        raise ValueError("sparse_attn_prefill needs a workspace tensor")
    _check(load_library().dsa_sparse_attn_prefill(
        ctypes.byref(c), _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, MHA_NOPE + MHA_ROPE)),
        _ptr(k_nope, torch.bfloat16, "k_nope", (c.total_kv, c.heads, MHA_NOPE)),
        _ptr(k_rope, torch.bfloat16, "k_rope", (c.total_kv, MHA_ROPE)),
        _ptr(v, torch.bfloat16, "v", (c.total_kv, c.heads, MHA_V)),
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, MHA_V)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def forward(prob: Problem, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse=None,
            idx_out=None, workspace=None, stream=None):
    """The three stages in order (dsa_forward); ``workspace`` is a uint8 GPU tensor
    of at least ``workspace_bytes(prob, WS_FORWARD)`` bytes."""
    c = prob.c
    D = c.d_latent + c.d_rope
    if workspace is None:
        raise ValueError("forward needs a workspace tensor")
    _check(load_library().dsa_forward(
        ctypes.byref(c),
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_fp8, torch.uint8, "k_fp8", (c.total_kv, c.idx_dim)),
        _ptr(k_scale, torch.float32, "k_scale", (c.total_kv,)),
        _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv, torch.bfloat16, "kv", (c.total_kv, D)),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(idx_out, torch.int32, "idx_out", (c.total_q, c.topk)),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def forward_noalloc(prob: Problem, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse=None,
                    idx_out=None, stream=None):
    """dsa_forward_noalloc: dsa_forward with the library's own device scratch as
    its workspace (no allocation in the call; problems whose forward
    workspace exceeds NOALLOC_SCRATCH_BYTES are refused)."""
    c = prob.c
    D = c.d_latent + c.d_rope
    _check(load_library().dsa_forward_noalloc(
        ctypes.byref(c),
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_fp8, torch.uint8, "k_fp8", (c.total_kv, c.idx_dim)),
        _ptr(k_scale, torch.float32, "k_scale", (c.total_kv,)),
        _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv, torch.bfloat16, "kv", (c.total_kv, D)),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(idx_out, torch.int32, "idx_out", (c.total_q, c.topk)), _stream(stream)))


def forward_fused(prob: Problem, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse=None,
                  idx_out=None, workspace=None, pg: "PagedKV" = None, stream=None):
    """dsa_forward_fused: the forward with the indexer and the selector fused
    (decode-shaped problems); ``workspace`` holds at least
    ``workspace_bytes(prob, WS_FORWARD_FUSED)`` bytes.  With ``pg`` the key and
    KV arguments are the paged caches."""
    c = prob.c
    D = c.d_latent + c.d_rope
    if workspace is None:
        raise ValueError("forward_fused needs a workspace tensor")
    if pg is None:
        ksh, ssh, vsh = (c.total_kv, c.idx_dim), (c.total_kv,), (c.total_kv, D)
    else:
        ksh, ssh, vsh = _cache_shapes(c, pg)
    _check(load_library().dsa_forward_fused(
        ctypes.byref(c), ctypes.byref(pg.c) if pg is not None else None,
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_fp8, torch.uint8, "k_fp8", ksh),
        _ptr(k_scale, torch.float32, "k_scale", ssh),
        _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv, torch.bfloat16, "kv", vsh),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(idx_out, torch.int32, "idx_out", (c.total_q, c.topk)),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def indexer_align_loss(prob: Problem, q, kv, lse, scores, loss, grad, idx=None, ld=None,
                       stream=None):
    """dsa_indexer_align_loss: per-row KL(attention target || indexer softmax) into
    ``loss`` [total_q] and its gradient with respect to the scores into ``grad``.

    Sparse form (``idx`` given): grad is [total_q, k], entry i for idx[:, i].
    Dense warm-up form (``idx`` None): grad is [total_q, ld_grad] by position,
    with ld_grad = grad.shape[1] >= max_kv_len."""
    c = prob.c
    D = c.d_latent + c.d_rope
    ld = prob.ld_scores() if ld is None else int(ld)
    if not isinstance(grad, torch.Tensor) or grad.dim() != 2:
        raise ValueError("grad must be a 2-D tensor")
    ld_grad = int(grad.shape[1])
    _check(load_library().dsa_indexer_align_loss(
        ctypes.byref(c), _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv, torch.bfloat16, "kv", (c.total_kv, D)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(scores, torch.float32, "scores", (c.total_q, ld)), ld,
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)),
        _ptr(loss, torch.float32, "loss", (c.total_q,)),
        _ptr(grad, torch.float32, "grad", (c.total_q, ld_grad)), ld_grad, _stream(stream)))


def indexer_backward(prob: Problem, q_fp8, q_scale, w, k_fp8, k_scale, grad, dq, dw, dk, idx=None,
                     workspace=None, stream=None):
    """dsa_indexer_backward: the score gradient ``grad`` carried to dq [total_q, H_I,
    d_I], dw [total_q, H_I] (both overwritten) and dk [total_kv, d_I] (added to).

    Sparse form (``idx`` given): grad is aligned with idx; dense form (``idx``
    None): grad is by position, grad.shape[1] >= max_kv_len.  ``workspace`` (a
    uint8 tensor of at least ``workspace_bytes(prob, WS_INDEXER_BWD)`` bytes)
    selects the two-pass dk of the sparse form; None: dk by atomics."""
    c = prob.c
    if not isinstance(grad, torch.Tensor) or grad.dim() != 2:
        raise ValueError("grad must be a 2-D tensor")
    ld_grad = int(grad.shape[1])
    _check(load_library().dsa_indexer_backward(
        ctypes.byref(c),
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_fp8, torch.uint8, "k_fp8", (c.total_kv, c.idx_dim)),
        _ptr(k_scale, torch.float32, "k_scale", (c.total_kv,)),
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)),
        _ptr(grad, torch.float32, "grad", (c.total_q, ld_grad)), ld_grad,
        _ptr(dq, torch.float32, "dq", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(dw, torch.float32, "dw", (c.total_q, c.idx_heads)),
        _ptr(dk, torch.float32, "dk", (c.total_kv, c.idx_dim)),
        _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream(stream)))


class PagedKV:
    """A ``dsa_paged_kv`` with its device block table kept alive.

    ``block_table`` is a [batch, max_blocks] int32 tensor (any device; copied to
    ``device``); ``num_blocks`` is the number of physical blocks in the caches."""

    def __init__(self, block_table, block_size: int, num_blocks: int, device="cuda"):
        bt = torch.as_tensor(block_table, dtype=torch.int32)
        if bt.dim() != 2:
            raise ValueError("block_table must be [batch, max_blocks]")
        self.table = bt.to(device).contiguous()
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        self.c = DsaPagedKV(block_table=self.table.data_ptr(), block_size=self.block_size,
                            max_blocks=int(bt.shape[1]), num_blocks=self.num_blocks)


def _cache_shapes(c, pg: PagedKV):
    nb, bs = pg.num_blocks, pg.block_size
    return (nb, bs, c.idx_dim), (nb, bs), (nb, bs, c.d_latent + c.d_rope)


def indexer_scores_paged(prob: Problem, pg: PagedKV, q_fp8, q_scale, w, k_cache, ks_cache, scores,
                         ld=None, stream=None):
    """dsa_indexer_scores_paged: the indexer with keys read through the block table."""
    c = prob.c
    ld = prob.ld_scores() if ld is None else int(ld)
    ksh, ssh, _ = _cache_shapes(c, pg)
    _check(load_library().dsa_indexer_scores_paged(
        ctypes.byref(c), ctypes.byref(pg.c),
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_cache, torch.uint8, "k_cache", ksh),
        _ptr(ks_cache, torch.float32, "ks_cache", ssh),
        _ptr(scores, torch.float32, "scores", (c.total_q, ld)), ld, _stream(stream)))


def sparse_attn_paged(prob: Problem, pg: PagedKV, q, kv_cache, idx, out, lse=None, workspace=None,
                      stream=None):
    """dsa_sparse_attn_paged: attention over latent rows read through the block table."""
    c = prob.c
    D = c.d_latent + c.d_rope
    _, _, vsh = _cache_shapes(c, pg)
    ws_ptr = _ptr(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_n = workspace.numel() if workspace is not None else 0
    _check(load_library().dsa_sparse_attn_paged(
        ctypes.byref(c), ctypes.byref(pg.c), _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv_cache, torch.bfloat16, "kv_cache", vsh),
        _ptr(idx, torch.int32, "idx", (c.total_q, c.topk)),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)), ws_ptr, ws_n, _stream(stream)))


def forward_paged(prob: Problem, pg: PagedKV, q_fp8, q_scale, w, k_cache, ks_cache, q, kv_cache, out,
                  lse=None, idx_out=None, workspace=None, stream=None):
    """dsa_forward_paged: the three stages over paged caches."""
    c = prob.c
    D = c.d_latent + c.d_rope
    if workspace is None:
        raise ValueError("forward_paged needs a workspace tensor")
    ksh, ssh, vsh = _cache_shapes(c, pg)
    _check(load_library().dsa_forward_paged(
        ctypes.byref(c), ctypes.byref(pg.c),
        _ptr(q_fp8, torch.uint8, "q_fp8", (c.total_q, c.idx_heads, c.idx_dim)),
        _ptr(q_scale, torch.float32, "q_scale", (c.total_q,)),
        _ptr(w, torch.float32, "w", (c.total_q, c.idx_heads)),
        _ptr(k_cache, torch.uint8, "k_cache", ksh),
        _ptr(ks_cache, torch.float32, "ks_cache", ssh),
        _ptr(q, torch.bfloat16, "q", (c.total_q, c.heads, D)),
        _ptr(kv_cache, torch.bfloat16, "kv_cache", vsh),
        _ptr(out, torch.bfloat16, "out", (c.total_q, c.heads, c.d_latent)),
        _ptr(lse, torch.float32, "lse", (c.total_q, c.heads)),
        _ptr(idx_out, torch.int32, "idx_out", (c.total_q, c.topk)),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
