"""Python binding of libgdn_tree.so (ctypes): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
dtype / contiguity / device / shape, and passes raw device pointers plus
torch's current HIP stream to the C ABI declared in ``include/gdn_tree.h``.
All arithmetic happens in the library's gfx950 kernels; there is no fallback
path, and a missing library raises at import of the first call.

Tensor formats (row-major, on one GPU):
  S0, S_out   float32 [n_slots, Hv, 128, 128]  (state stored transposed)
  q, k        bfloat16 [T, Hk, 128];  v bfloat16 [T, Hv, 128]
  g, beta     float32 [T, Hv]
  node_offset int32 [B+1];  parent int32 [T] (request-local, -1 = S0)
  out, U      float32 [T, Hv, 128];  anc_mask int64 [T] (uint64 bit patterns)
  path        int32 [B, max_nodes];  path_len, accept_node, status int32 [B]
  node_state  float32 [T, Hv, 128, 128]
Tree-bias attention:
  q           bfloat16 [T, Hq, 128];  k_ctx, v_ctx bfloat16 [C, Hkv, 128]
  k_node, v_node bfloat16 [T, Hkv, 128];  ctx_offset int32 [B+1]
  out         float32 [T, Hq, 128];  lse float32 [T, Hq]
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn_tree.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gdn_tree.h")

HEAD_DIM = 128
MAX_NODES = 64
STATIC_SCRATCH_BYTES = 64 << 20   # GDN_TREE_STATIC_SCRATCH_BYTES

# status codes (include/gdn_tree.h)
(S_OK, S_BAD_OFFSETS, S_TOO_MANY, S_BAD_PARENT, S_BAD_PATH, S_BAD_ACCEPT, S_BAD_SLOT, S_BAD_CONTEXT,
 S_BAD_MASK) = range(9)


class GdnTreeError(RuntimeError):
    """A negative return code from the C ABI (nothing was enqueued)."""

    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {strerror(code)} (code {code})")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hv", "Hk", "d_k", "d_v", "T", "max_nodes", "n_slots")]


class AttnDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "Hq", "Hkv", "head_dim", "T", "C", "max_nodes", "max_ctx",
                                               "split")]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "gdn_tree_verify": [ctypes.POINTER(Dims)] + [_P] * 14,
    "gdn_tree_commit": [ctypes.POINTER(Dims)] + [_P] * 12,
    "gdn_tree_accepted_path": [ctypes.POINTER(Dims)] + [_P] * 7,
    "gdn_tree_verify_storeall": [ctypes.POINTER(Dims)] + [_P] * 13,
    "gdn_tree_commit_storeall": [ctypes.POINTER(Dims)] + [_P] * 9,
    "gdn_tree_accept_greedy": [ctypes.POINTER(Dims)] + [_P] * 10,
    "gdn_tree_accept_commit": [ctypes.POINTER(Dims)] + [_P] * 16,
    "gdn_tree_commit_node": [ctypes.POINTER(Dims)] + [_P] * 13,
    "gdn_tree_commit_verify": [ctypes.POINTER(Dims), ctypes.POINTER(Dims)] + [_P] * 24,
    "gdn_tree_accept_commit_verify": [ctypes.POINTER(Dims), ctypes.POINTER(Dims)] + [_P] * 27,
    "gdn_tree_commit_replay": [ctypes.POINTER(Dims)] + [_P] * 13,
    "gdn_tree_budget_select": [ctypes.POINTER(Dims), _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                               _P, _P, _P, _P, _P],
    "gdn_tree_ancestry": [ctypes.POINTER(Dims)] + [_P] * 5,
    "gdn_tree_attention": [ctypes.POINTER(AttnDims)] + [_P] * 8 + [ctypes.c_float, _P, _P, _P, ctypes.c_size_t,
                                                                   _P, _P],
    "gdn_tree_attention_static": [ctypes.POINTER(AttnDims)] + [_P] * 8 + [ctypes.c_float, _P, _P, _P, _P],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn_tree.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m speculative_decoding_tree_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _I
        L.gdn_tree_state_bytes.argtypes = [ctypes.POINTER(Dims), _I]
        L.gdn_tree_state_bytes.restype = ctypes.c_size_t
        L.gdn_tree_attention_workspace_bytes.argtypes = [ctypes.POINTER(AttnDims)]
        L.gdn_tree_attention_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_tree_strerror.argtypes = [_I]
        L.gdn_tree_strerror.restype = ctypes.c_char_p
        L.gdn_tree_abi_version.argtypes = []
        L.gdn_tree_abi_version.restype = _I
        _lib = L
    return _lib


def declared_symbols():
    """Names of the functions include/gdn_tree.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gdn_tree_[a-z_]+)\s*\(", text)))


def strerror(code: int) -> str:
    return lib().gdn_tree_strerror(int(code)).decode()


def abi_version() -> int:
    return lib().gdn_tree_abi_version()


def make_dims(B, Hv, Hk, T, max_nodes, n_slots, d_k=HEAD_DIM, d_v=HEAD_DIM) -> Dims:
    return Dims(int(B), int(Hv), int(Hk), int(d_k), int(d_v), int(T), int(max_nodes), int(n_slots))


def state_bytes(dims: Dims, storeall: bool) -> int:
    return int(lib().gdn_tree_state_bytes(ctypes.byref(dims), int(bool(storeall))))


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], name: str, dtypes, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


_F32 = (torch.float32,)
_I32 = (torch.int32,)
_B16 = (torch.bfloat16, torch.int16, torch.uint16)
_U64 = (torch.int64, torch.uint64)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise GdnTreeError(fn, rc)


def _geometry(S0, q, v, node_offset, parent, max_nodes):
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    Hk = int(q.shape[1]) if q.dim() == 3 else 1
    return B, Hv, Hk, T, n_slots


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def verify(S0, q, k, v, g, beta, node_offset, parent, max_nodes: int, state_slot=None,
           out=None, U=None, anc_mask=None, status=None, stream=None):
    """gdn_tree_verify.  Returns (out, U, anc_mask, status); outputs not given are allocated."""
    B, Hv, Hk, T, n_slots = _geometry(S0, q, v, node_offset, parent, max_nodes)
    dev = S0.device
    out = out if out is not None else torch.empty((T, Hv, HEAD_DIM), dtype=torch.float32, device=dev)
    U = U if U is not None else torch.empty((T, Hv, HEAD_DIM), dtype=torch.float32, device=dev)
    anc_mask = anc_mask if anc_mask is not None else torch.empty((T,), dtype=torch.int64, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_verify(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(q, "q", _B16, (T, Hk, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
        _ptr(v, "v", _B16, (T, Hv, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)), _ptr(beta, "beta", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(out, "out", _F32, (T, Hv, HEAD_DIM)), _ptr(U, "U", _F32, (T, Hv, HEAD_DIM)),
        _ptr(anc_mask, "anc_mask", _U64, (T,)), _ptr(status, "status", _I32, (B,)),
        _stream(stream))
    _check("gdn_tree_verify", rc)
    return out, U, anc_mask, status


def commit(S0, U, k, g, node_offset, parent, path, path_len, max_nodes: int, S_out=None,
           state_slot=None, status=None, stream=None):
    """gdn_tree_commit.  S_out defaults to a new buffer shaped like S0 (pass S0 for in-place)."""
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    Hk = int(k.shape[1])
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=S0.device)
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_commit(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(U, "U", _F32, (T, Hv, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(path, "path", _I32, (B, max_nodes)), _ptr(path_len, "path_len", _I32, (B,)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_commit", rc)
    return S_out, status


def accepted_path(node_offset, parent, accept_node, max_nodes: int, path=None, path_len=None,
                  status=None, stream=None):
    """gdn_tree_accepted_path.  Returns (path, path_len, status)."""
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    dev = node_offset.device
    path = path if path is not None else torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    path_len = path_len if path_len is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    dims = make_dims(B, 1, 1, T, max_nodes, 1)
    rc = lib().gdn_tree_accepted_path(
        ctypes.byref(dims),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(accept_node, "accept_node", _I32, (B,)),
        _ptr(path, "path", _I32, (B, max_nodes)), _ptr(path_len, "path_len", _I32, (B,)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_accepted_path", rc)
    return path, path_len, status


def verify_storeall(S0, q, k, v, g, beta, node_offset, parent, max_nodes: int, state_slot=None,
                    out=None, node_state=None, status=None, stream=None):
    """gdn_tree_verify_storeall.  Returns (out, node_state, status)."""
    B, Hv, Hk, T, n_slots = _geometry(S0, q, v, node_offset, parent, max_nodes)
    dev = S0.device
    out = out if out is not None else torch.empty((T, Hv, HEAD_DIM), dtype=torch.float32, device=dev)
    node_state = node_state if node_state is not None else torch.empty(
        (T, Hv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_verify_storeall(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(q, "q", _B16, (T, Hk, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
        _ptr(v, "v", _B16, (T, Hv, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)), _ptr(beta, "beta", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(out, "out", _F32, (T, Hv, HEAD_DIM)),
        _ptr(node_state, "node_state", _F32, (T, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_verify_storeall", rc)
    return out, node_state, status


def commit_storeall(S0, node_state, node_offset, parent, accept_node, max_nodes: int, S_out=None,
                    state_slot=None, status=None, stream=None):
    """gdn_tree_commit_storeall.  Returns (S_out, status)."""
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=S0.device)
    dims = make_dims(B, Hv, 1, T, max_nodes, n_slots)
    rc = lib().gdn_tree_commit_storeall(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(node_state, "node_state", _F32, (T, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(accept_node, "accept_node", _I32, (B,)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_commit_storeall", rc)
    return S_out, status


def accept_greedy(node_offset, parent, draft_token, target_token, root_token, max_nodes: int,
                  accept_node=None, path=None, path_len=None, status=None, stream=None):
    """gdn_tree_accept_greedy.  Returns (accept_node, path, path_len, status)."""
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    dev = node_offset.device
    mk = lambda shape: torch.empty(shape, dtype=torch.int32, device=dev)
    accept_node = accept_node if accept_node is not None else mk((B,))
    path = path if path is not None else mk((B, max_nodes))
    path_len = path_len if path_len is not None else mk((B,))
    status = status if status is not None else mk((B,))
    dims = make_dims(B, 1, 1, T, max_nodes, 1)
    rc = lib().gdn_tree_accept_greedy(
        ctypes.byref(dims),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(draft_token, "draft_token", _I32, (T,)), _ptr(target_token, "target_token", _I32, (T,)),
        _ptr(root_token, "root_token", _I32, (B,)),
        _ptr(accept_node, "accept_node", _I32, (B,)), _ptr(path, "path", _I32, (B, max_nodes)),
        _ptr(path_len, "path_len", _I32, (B,)), _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_accept_greedy", rc)
    return accept_node, path, path_len, status


def accept_commit(S0, U, k, g, node_offset, parent, draft_token, target_token, root_token, max_nodes: int,
                  S_out=None, state_slot=None, accept_node=None, path=None, path_len=None, status=None,
                  stream=None):
    """gdn_tree_accept_commit (greedy acceptance fused with the commit).
    Returns (S_out, accept_node, path, path_len, status); the optional outputs are
    allocated unless given."""
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    Hk = int(k.shape[1])
    dev = S0.device
    mk = lambda shape: torch.empty(shape, dtype=torch.int32, device=dev)
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    accept_node = accept_node if accept_node is not None else mk((B,))
    path = path if path is not None else mk((B, max_nodes))
    path_len = path_len if path_len is not None else mk((B,))
    status = status if status is not None else mk((B,))
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_accept_commit(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(U, "U", _F32, (T, Hv, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(draft_token, "draft_token", _I32, (T,)), _ptr(target_token, "target_token", _I32, (T,)),
        _ptr(root_token, "root_token", _I32, (B,)),
        _ptr(accept_node, "accept_node", _I32, (B,)), _ptr(path, "path", _I32, (B, max_nodes)),
        _ptr(path_len, "path_len", _I32, (B,)), _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_accept_commit", rc)
    return S_out, accept_node, path, path_len, status


def commit_node(S0, U, k, g, node_offset, parent, accept_node, max_nodes: int, S_out=None, state_slot=None,
                path=None, path_len=None, status=None, stream=None):
    """gdn_tree_commit_node (the accepted node's path and the commit in one launch).
    Returns (S_out, path, path_len, status); the outputs are allocated unless given."""
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    Hk = int(k.shape[1])
    dev = S0.device
    mk = lambda shape: torch.empty(shape, dtype=torch.int32, device=dev)
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    path = path if path is not None else mk((B, max_nodes))
    path_len = path_len if path_len is not None else mk((B,))
    status = status if status is not None else mk((B,))
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_commit_node(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(U, "U", _F32, (T, Hv, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(accept_node, "accept_node", _I32, (B,)),
        _ptr(path, "path", _I32, (B, max_nodes)), _ptr(path_len, "path_len", _I32, (B,)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_commit_node", rc)
    return S_out, path, path_len, status


def commit_verify(S0, prev, accept_node, q, k, v, g, beta, node_offset, parent, max_nodes: int, S_out=None,
                  state_slot=None, out=None, U=None, anc_mask=None, status=None, commit_status=None,
                  stream=None, greedy=None, path=None, path_len=None):
    """gdn_tree_commit_verify: commit the previous tree's accepted node into S_out, then verify the
    next tree from that state, in one launch.  ``prev`` is a dict with the previous tree's
    ``U``, ``k``, ``g``, ``node_offset``, ``parent`` and ``max_nodes``.
    With ``greedy`` = dict(draft_token, target_token, root_token) the accepted node comes from the
    device-side greedy walk instead (gdn_tree_accept_commit_verify) and ``accept_node`` is an
    optional output.  ``path`` [B][prev max_nodes] and ``path_len`` [B] are optional outputs
    (the accepted root-first path; not written when None).
    Returns (S_out, out, U, anc_mask, status, commit_status[, accept_node])."""
    B, Hv, Hk, T, n_slots = _geometry(S0, q, v, node_offset, parent, max_nodes)
    U_p, k_p, g_p, off_p, par_p = prev["U"], prev["k"], prev["g"], prev["node_offset"], prev["parent"]
    T_p = int(par_p.numel())
    dev = S0.device
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    out = out if out is not None else torch.empty((T, Hv, HEAD_DIM), dtype=torch.float32, device=dev)
    U = U if U is not None else torch.empty((T, Hv, HEAD_DIM), dtype=torch.float32, device=dev)
    anc_mask = anc_mask if anc_mask is not None else torch.empty((T,), dtype=torch.int64, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    commit_status = (commit_status if commit_status is not None
                     else torch.empty((B,), dtype=torch.int32, device=dev))
    pdims = make_dims(int(off_p.numel()) - 1, Hv, Hk, T_p, prev["max_nodes"], n_slots)
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    head = [ctypes.byref(pdims), ctypes.byref(dims),
            _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
            _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
            _ptr(state_slot, "state_slot", _I32, (B,)),
            _ptr(U_p, "prev U", _F32, (T_p, Hv, HEAD_DIM)), _ptr(k_p, "prev k", _B16, (T_p, Hk, HEAD_DIM)),
            _ptr(g_p, "prev g", _F32, (T_p, Hv)),
            _ptr(off_p, "prev node_offset", _I32, (B + 1,)), _ptr(par_p, "prev parent", _I32, (T_p,))]
    tail = [_ptr(q, "q", _B16, (T, Hk, HEAD_DIM)), _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)),
            _ptr(v, "v", _B16, (T, Hv, HEAD_DIM)),
            _ptr(g, "g", _F32, (T, Hv)), _ptr(beta, "beta", _F32, (T, Hv)),
            _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
            _ptr(out, "out", _F32, (T, Hv, HEAD_DIM)), _ptr(U, "U", _F32, (T, Hv, HEAD_DIM)),
            _ptr(anc_mask, "anc_mask", _U64, (T,)), _ptr(status, "status", _I32, (B,)),
            _stream(stream)]
    mnp = int(prev["max_nodes"])
    pth = [_ptr(path, "path", _I32, (B, mnp)), _ptr(path_len, "path_len", _I32, (B,))]
    if greedy is None:
        rc = lib().gdn_tree_commit_verify(
            *head, _ptr(accept_node, "accept_node", _I32, (B,)), *pth,
            _ptr(commit_status, "commit_status", _I32, (B,)), *tail)
        _check("gdn_tree_commit_verify", rc)
        return S_out, out, U, anc_mask, status, commit_status
    accept_node = accept_node if accept_node is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    rc = lib().gdn_tree_accept_commit_verify(
        *head, _ptr(greedy["draft_token"], "draft_token", _I32, (T_p,)),
        _ptr(greedy["target_token"], "target_token", _I32, (T_p,)),
        _ptr(greedy["root_token"], "root_token", _I32, (B,)), _ptr(accept_node, "accept_node", _I32, (B,)),
        *pth, _ptr(commit_status, "commit_status", _I32, (B,)), *tail)
    _check("gdn_tree_accept_commit_verify", rc)
    return S_out, out, U, anc_mask, status, commit_status, accept_node


def commit_replay(S0, k, v, g, beta, node_offset, parent, path, path_len, max_nodes: int, S_out=None,
                  state_slot=None, status=None, stream=None):
    """gdn_tree_commit_replay (sequential replay of the accepted path, no U)."""
    n_slots, Hv = int(S0.shape[0]), int(S0.shape[1])
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    Hk = int(k.shape[1])
    S_out = S_out if S_out is not None else torch.empty_like(S0)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=S0.device)
    dims = make_dims(B, Hv, Hk, T, max_nodes, n_slots)
    rc = lib().gdn_tree_commit_replay(
        ctypes.byref(dims),
        _ptr(S0, "S0", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(S_out, "S_out", _F32, (n_slots, Hv, HEAD_DIM, HEAD_DIM)),
        _ptr(state_slot, "state_slot", _I32, (B,)),
        _ptr(k, "k", _B16, (T, Hk, HEAD_DIM)), _ptr(v, "v", _B16, (T, Hv, HEAD_DIM)),
        _ptr(g, "g", _F32, (T, Hv)), _ptr(beta, "beta", _F32, (T, Hv)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(path, "path", _I32, (B, max_nodes)), _ptr(path_len, "path_len", _I32, (B,)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_commit_replay", rc)
    return S_out, status


def budget_select(node_offset, parent, accept_prob, budget: int, threshold: float, max_nodes: int,
                  survival=None, keep=None, kept=None, status=None, stream=None):
    """gdn_tree_budget_select.  Returns (survival, keep (uint8), kept, status)."""
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    dev = node_offset.device
    survival = survival if survival is not None else torch.empty((T,), dtype=torch.float32, device=dev)
    keep = keep if keep is not None else torch.empty((T,), dtype=torch.uint8, device=dev)
    kept = kept if kept is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    dims = make_dims(B, 1, 1, T, max_nodes, 1)
    rc = lib().gdn_tree_budget_select(
        ctypes.byref(dims),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(accept_prob, "accept_prob", _F32, (T,)), int(budget), float(threshold),
        _ptr(survival, "survival", _F32, (T,)), _ptr(keep, "keep", (torch.uint8,), (T,)),
        _ptr(kept, "kept", _I32, (B,)), _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_budget_select", rc)
    return survival, keep, kept, status


def ancestry(node_offset, parent, max_nodes: int, anc_mask=None, status=None, stream=None):
    """gdn_tree_ancestry.  Returns (anc_mask int64 [T], status)."""
    B = int(node_offset.numel()) - 1
    T = int(parent.numel())
    dev = node_offset.device
    anc_mask = anc_mask if anc_mask is not None else torch.empty((T,), dtype=torch.int64, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    dims = make_dims(B, 1, 1, T, max_nodes, 1)
    rc = lib().gdn_tree_ancestry(
        ctypes.byref(dims),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(parent, "parent", _I32, (T,)),
        _ptr(anc_mask, "anc_mask", _U64, (T,)), _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_ancestry", rc)
    return anc_mask, status


def make_attn_dims(B, Hq, Hkv, T, C, max_nodes, max_ctx, split=None, head_dim=HEAD_DIM) -> AttnDims:
    split = max(1, int(max_ctx)) if split is None else int(split)
    return AttnDims(int(B), int(Hq), int(Hkv), int(head_dim), int(T), int(C), int(max_nodes), int(max_ctx), split)


def attention_workspace_bytes(dims: AttnDims) -> int:
    return int(lib().gdn_tree_attention_workspace_bytes(ctypes.byref(dims)))


def attention(q, k_ctx, v_ctx, ctx_offset, k_node, v_node, node_offset, anc_mask, scale: float,
              max_nodes: int, max_ctx: int, split: Optional[int] = None, out=None, lse=None, workspace=None,
              status=None, stream=None):
    """gdn_tree_attention.  Returns (out, lse, status).  split=None runs one
    pass; split=0 lets the library choose the context part size.  A workspace
    of attention_workspace_bytes(dims) is allocated when none is given (work
    distribution counters, plus partial results when the context is split)."""
    B = int(node_offset.numel()) - 1
    T, Hq = int(q.shape[0]), int(q.shape[1])
    C, Hkv = int(k_ctx.shape[0]), int(k_ctx.shape[1])
    dev = q.device
    dims = make_attn_dims(B, Hq, Hkv, T, C, max_nodes, max_ctx, split)
    out = out if out is not None else torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((T, Hq), dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    need = attention_workspace_bytes(dims)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    rc = lib().gdn_tree_attention(
        ctypes.byref(dims),
        _ptr(q, "q", _B16, (T, Hq, HEAD_DIM)),
        _ptr(k_ctx, "k_ctx", _B16, (C, Hkv, HEAD_DIM)), _ptr(v_ctx, "v_ctx", _B16, (C, Hkv, HEAD_DIM)),
        _ptr(ctx_offset, "ctx_offset", _I32, (B + 1,)),
        _ptr(k_node, "k_node", _B16, (T, Hkv, HEAD_DIM)), _ptr(v_node, "v_node", _B16, (T, Hkv, HEAD_DIM)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(anc_mask, "anc_mask", _U64, (T,)),
        ctypes.c_float(scale),
        _ptr(out, "out", _F32, (T, Hq, HEAD_DIM)), _ptr(lse, "lse", _F32, (T, Hq)),
        ws_ptr, ctypes.c_size_t(ws_bytes), _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_attention", rc)
    return out, lse, status


def attention_static(q, k_ctx, v_ctx, ctx_offset, k_node, v_node, node_offset, anc_mask, scale: float,
                     max_nodes: int, max_ctx: int, split: Optional[int] = None, out=None, lse=None, status=None,
                     stream=None):
    """gdn_tree_attention_static: gdn_tree_attention with the library's static per-device
    scratch instead of a workspace (no allocation by the library).  Returns (out, lse, status);
    out, lse and status are allocated here unless given (pass them to allocate nothing)."""
    B = int(node_offset.numel()) - 1
    T, Hq = int(q.shape[0]), int(q.shape[1])
    C, Hkv = int(k_ctx.shape[0]), int(k_ctx.shape[1])
    dev = q.device
    dims = make_attn_dims(B, Hq, Hkv, T, C, max_nodes, max_ctx, split)
    out = out if out is not None else torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    lse = lse if lse is not None else torch.empty((T, Hq), dtype=torch.float32, device=dev)
    status = status if status is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    rc = lib().gdn_tree_attention_static(
        ctypes.byref(dims),
        _ptr(q, "q", _B16, (T, Hq, HEAD_DIM)),
        _ptr(k_ctx, "k_ctx", _B16, (C, Hkv, HEAD_DIM)), _ptr(v_ctx, "v_ctx", _B16, (C, Hkv, HEAD_DIM)),
        _ptr(ctx_offset, "ctx_offset", _I32, (B + 1,)),
        _ptr(k_node, "k_node", _B16, (T, Hkv, HEAD_DIM)), _ptr(v_node, "v_node", _B16, (T, Hkv, HEAD_DIM)),
        _ptr(node_offset, "node_offset", _I32, (B + 1,)), _ptr(anc_mask, "anc_mask", _U64, (T,)),
        ctypes.c_float(scale),
        _ptr(out, "out", _F32, (T, Hq, HEAD_DIM)), _ptr(lse, "lse", _F32, (T, Hq)),
        _ptr(status, "status", _I32, (B,)), _stream(stream))
    _check("gdn_tree_attention_static", rc)
    return out, lse, status
