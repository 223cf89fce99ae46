"""Thin ctypes binding over libbole.so, using the C function names of include/bole.h.

Only argument marshalling happens here: dtype, device and shape checks, building the
dims descriptor, and passing data pointers plus torch's current HIP stream. Every step
of verify, commit and prepare runs in the library's HIP kernels. If the library is
missing, importing this module fails: there is no fallback path.
"""
import ctypes
import os

import torch  # must be imported before libbole.so: the two share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbole.so")

BOLE_OK, BOLE_ERR_INVALID_VALUE, BOLE_ERR_UNSUPPORTED, BOLE_ERR_HIP, BOLE_ERR_BAD_TREE = 0, 1, 2, 3, 4
BOLE_TREE_OK, BOLE_TREE_BAD_SIZE, BOLE_TREE_BAD_PARENT, BOLE_TREE_BAD_PATH = 0, 1, 2, 3
BOLE_TREE_BAD_TOKEN, BOLE_TREE_BAD_GATE = 4, 5
BOLE_DTYPE_BF16, BOLE_DTYPE_F32 = 0, 1
BOLE_GATE_SCALAR, BOLE_GATE_VECTOR = 0, 1
BOLE_FLAG_FORCE_GENERIC = 1
BOLE_FLAG_TREES_LE_32 = 2
BOLE_FLAG_VALIDATE_GATES = 4
MAX_TREE_NODES = 64

EXPORTED = ("bole_max_tree_nodes", "bole_status_string", "bole_check_dims",
            "bole_workspace_bytes", "bole_read_status", "bole_tree_verify",
            "bole_tree_verify_lazy_commit", "bole_tree_verify_layers", "bole_commit_path_layers",
            "bole_tree_verify_lazy_commit_layers", "bole_tree_verify_naive", "bole_commit_path",
            "bole_tree_prepare", "bole_build_tree_workspace_size", "bole_build_tree",
            "bole_build_tree_noalloc",
            "bole_tree_accept")
BOLE_ACCEPT_GREEDY, BOLE_ACCEPT_SAMPLE = 0, 1
BOLE_BUILD_FIXED_BUDGET = 1


class bole_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("total_nodes", ctypes.c_int32),
                ("max_path", ctypes.c_int32), ("factor_dtype", ctypes.c_int32),
                ("gate_kind", ctypes.c_int32), ("flags", ctypes.c_int32)]


class bole_factors_t(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("parent", ctypes.c_void_p), ("node_offsets", ctypes.c_void_p)]


class bole_layer_t(ctypes.Structure):
    _fields_ = [("H0", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("prev_k", ctypes.c_void_p), ("prev_v", ctypes.c_void_p),
                ("prev_gate", ctypes.c_void_p)]


class bole_build_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("depth", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_max", ctypes.c_int32), ("flags", ctypes.c_int32)]


class bole_accept_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_nodes", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_path", ctypes.c_int32), ("mode", ctypes.c_int32)]


class BoleError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(hipcc, gfx950) before using the HIP path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    D = ctypes.POINTER(bole_dims_t)
    lib.bole_max_tree_nodes.restype = I32
    lib.bole_max_tree_nodes.argtypes = []
    lib.bole_status_string.restype = ctypes.c_char_p
    lib.bole_status_string.argtypes = [ctypes.c_int]
    lib.bole_check_dims.restype = ctypes.c_int
    lib.bole_check_dims.argtypes = [D, I32]
    lib.bole_workspace_bytes.restype = ctypes.c_size_t
    lib.bole_workspace_bytes.argtypes = [D]
    lib.bole_read_status.restype = ctypes.c_int
    lib.bole_read_status.argtypes = [P, I32, P, P]
    lib.bole_tree_verify.restype = ctypes.c_int
    lib.bole_tree_verify.argtypes = [P, P, P, P, P, P, P, P, D, P, P]
    lib.bole_tree_verify_lazy_commit.restype = ctypes.c_int
    lib.bole_tree_verify_lazy_commit.argtypes = [P, ctypes.POINTER(bole_factors_t), P, P, D, P, P,
                                                 P, P, P, P, P, P, P, D, P, P]
    LP = ctypes.POINTER(bole_layer_t)
    lib.bole_tree_verify_layers.restype = ctypes.c_int
    lib.bole_tree_verify_layers.argtypes = [LP, I32, P, P, D, P, P]
    lib.bole_commit_path_layers.restype = ctypes.c_int
    lib.bole_commit_path_layers.argtypes = [LP, I32, P, P, P, P, D, P, P, P]
    lib.bole_tree_verify_lazy_commit_layers.restype = ctypes.c_int
    lib.bole_tree_verify_lazy_commit_layers.argtypes = [LP, I32, P, P, P, P, D, P, P, P, P, D, P, P]
    BD = ctypes.POINTER(bole_build_dims_t)
    lib.bole_build_tree_workspace_size.restype = ctypes.c_size_t
    lib.bole_build_tree_workspace_size.argtypes = [BD]
    lib.bole_build_tree.restype = ctypes.c_int
    lib.bole_build_tree.argtypes = [P, P, ctypes.c_float, P, ctypes.c_size_t, BD, P, P, P, P, P, P]
    lib.bole_build_tree_noalloc.restype = ctypes.c_int
    lib.bole_build_tree_noalloc.argtypes = [P, P, ctypes.c_float, BD, P, P, P, P, P, P]
    AD = ctypes.POINTER(bole_accept_dims_t)
    lib.bole_tree_accept.restype = ctypes.c_int
    lib.bole_tree_accept.argtypes = [P, P, P, P, P, P, P, P, P, AD, P, P, P, P, P]
    lib.bole_tree_verify_naive.restype = ctypes.c_int
    lib.bole_tree_verify_naive.argtypes = [P, P, P, P, P, P, P, P, P, D, P, P]
    lib.bole_commit_path.restype = ctypes.c_int
    lib.bole_commit_path.argtypes = [P, ctypes.POINTER(bole_factors_t), P, P, D, P, P, P]
    lib.bole_tree_prepare.restype = ctypes.c_int
    lib.bole_tree_prepare.argtypes = [P, P, P, D, P, P, P, P, P]
    return lib


lib = _load()


def _check(status: int, what: str):
    if status != BOLE_OK:
        raise BoleError(f"{what}: {lib.bole_status_string(status).decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def make_dims(batch, heads, d_k, d_v, total_nodes, factor_dtype, vector_gate, max_path=0,
              force_generic=False, trees_le_32=False, validate_gates=False) -> bole_dims_t:
    fd = {torch.bfloat16: BOLE_DTYPE_BF16, torch.float32: BOLE_DTYPE_F32}.get(factor_dtype)
    if fd is None:
        raise TypeError(f"factor dtype must be bfloat16 or float32, got {factor_dtype}")
    flags = (BOLE_FLAG_FORCE_GENERIC if force_generic else 0) | \
        (BOLE_FLAG_TREES_LE_32 if trees_le_32 else 0) | \
        (BOLE_FLAG_VALIDATE_GATES if validate_gates else 0)
    return bole_dims_t(batch, heads, d_k, d_v, total_nodes, max_path, fd,
                       BOLE_GATE_VECTOR if vector_gate else BOLE_GATE_SCALAR, flags)


def _factor_dims(H0, q_or_k, v, gate, parent, node_offsets):
    dev = H0.device
    _need(H0, "H0", torch.float32)
    if H0.dim() != 4:
        raise ValueError("H0 must be [B, H, d_k, d_v]")
    B, Hh, d_k, d_v = H0.shape
    _need(q_or_k, "k", device=dev)
    _need(v, "v", q_or_k.dtype, dev)
    _need(gate, "gate", torch.float32, dev)
    _need(parent, "parent", torch.int32, dev)
    _need(node_offsets, "node_offsets", torch.int32, dev)
    T = q_or_k.shape[0]
    if tuple(q_or_k.shape) != (T, Hh, d_k) or tuple(v.shape) != (T, Hh, d_v):
        raise ValueError("factor shapes must be [T, H, d_k] and [T, H, d_v]")
    if tuple(parent.shape) != (T,) or tuple(node_offsets.shape) != (B + 1,):
        raise ValueError("parent must be [T] and node_offsets [B + 1]")
    if tuple(gate.shape) == (T, Hh):
        vector_gate = False
    elif tuple(gate.shape) == (T, Hh, d_k):
        vector_gate = True
    else:
        raise ValueError("gate must be [T, H] (scalar) or [T, H, d_k] (vector)")
    return B, Hh, d_k, d_v, T, vector_gate


def bole_tree_verify(H0, q, k, v, gate, parent, node_offsets, out=None, tree_status=None,
                     stream=None, force_generic=False, trees_le_32=False, validate_gates=False):
    """out[T, H, d_v] (fp32) = H_i^T q_i for every node, by the parallel closed form.
    trees_le_32: the caller's tree budget is at most 32 nodes (larger trees are reported
    BOLE_TREE_BAD_SIZE and left untouched). validate_gates: BOLE_FLAG_VALIDATE_GATES
    (needs tree_status)."""
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    _need(q, "q", k.dtype, H0.device)
    if tuple(q.shape) != tuple(k.shape):
        raise ValueError("q must have the shape of k")
    if out is None:
        out = torch.empty((T, Hh, d_v), dtype=torch.float32, device=H0.device)
    _need(out, "out", torch.float32, H0.device)
    if tuple(out.shape) != (T, Hh, d_v):
        raise ValueError("out must be [T, H, d_v]")
    if tree_status is not None:
        _need(tree_status, "tree_status", torch.int32, H0.device)
        if tree_status.numel() < B:
            raise ValueError("tree_status needs B entries")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, 0, force_generic, trees_le_32,
                     validate_gates)
    _check(lib.bole_tree_verify(_ptr(H0), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(parent),
                                _ptr(node_offsets), _ptr(out), ctypes.byref(dims),
                                _ptr(tree_status), _stream(stream)), "bole_tree_verify")
    return out


def bole_tree_verify_naive(H0, q, k, v, gate, parent, node_offsets, out=None, states=None,
                           tree_status=None, stream=None, trees_le_32=False):
    """Baseline serial walk: out[T, H, d_v] as bole_tree_verify, with every node's state
    written to states[T, H, d_k, d_v] (fp32, allocated here when None). Returns
    (out, states)."""
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    _need(q, "q", k.dtype, H0.device)
    if tuple(q.shape) != tuple(k.shape):
        raise ValueError("q must have the shape of k")
    if out is None:
        out = torch.empty((T, Hh, d_v), dtype=torch.float32, device=H0.device)
    if states is None:
        states = torch.empty((T, Hh, d_k, d_v), dtype=torch.float32, device=H0.device)
    _need(out, "out", torch.float32, H0.device)
    _need(states, "states", torch.float32, H0.device)
    if tuple(out.shape) != (T, Hh, d_v) or tuple(states.shape) != (T, Hh, d_k, d_v):
        raise ValueError("out must be [T, H, d_v] and states [T, H, d_k, d_v]")
    if tree_status is not None:
        _need(tree_status, "tree_status", torch.int32, H0.device)
        if tree_status.numel() < B:
            raise ValueError("tree_status needs B entries")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, 0, trees_le_32=trees_le_32)
    _check(lib.bole_tree_verify_naive(_ptr(H0), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                      _ptr(parent), _ptr(node_offsets), _ptr(out), _ptr(states),
                                      ctypes.byref(dims), _ptr(tree_status), _stream(stream)),
           "bole_tree_verify_naive")
    return out, states


def _lazy_args(H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate, parent,
               node_offsets, out, prev_path_nodes, prev_tree_status, tree_status, stream,
               trees_le_32, prev_trees_le_32, validate_gates=False):
    pk, pv, pgate, pparent, poffs = prev
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    pB, pH, pdk, pdv, pT, pvec = _factor_dims(H0, pk, pv, pgate, pparent, poffs)
    if pk.dtype != k.dtype or pvec != vec:
        raise ValueError("the previous step's factors must match this step's dtype and gate kind")
    _need(q, "q", k.dtype, H0.device)
    if tuple(q.shape) != tuple(k.shape):
        raise ValueError("q must have the shape of k")
    _need(prev_accepted_idx, "prev_accepted_idx", torch.int32, H0.device)
    _need(prev_accepted_len, "prev_accepted_len", torch.int32, H0.device)
    if (prev_accepted_idx.dim() != 2 or prev_accepted_idx.shape[0] != B
            or tuple(prev_accepted_len.shape) != (B,)):
        raise ValueError("prev_accepted_idx must be [B, max_path] and prev_accepted_len [B]")
    max_path = prev_accepted_idx.shape[1]
    if out is None:
        out = torch.empty((T, Hh, d_v), dtype=torch.float32, device=H0.device)
    _need(out, "out", torch.float32, H0.device)
    if tuple(out.shape) != (T, Hh, d_v):
        raise ValueError("out must be [T, H, d_v]")
    for t, name in ((prev_path_nodes, "prev_path_nodes"), (prev_tree_status, "prev_tree_status"),
                    (tree_status, "tree_status")):
        if t is not None:
            _need(t, name, torch.int32, H0.device)
    if prev_path_nodes is not None and tuple(prev_path_nodes.shape) != (B, max_path):
        raise ValueError("prev_path_nodes must be [B, max_path]")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, 0, trees_le_32=trees_le_32,
                     validate_gates=validate_gates)
    pdims = make_dims(B, Hh, d_k, d_v, pT, k.dtype, vec, max_path, trees_le_32=prev_trees_le_32,
                      validate_gates=validate_gates)
    f = bole_factors_t(pk.data_ptr(), pv.data_ptr(), pgate.data_ptr(), pparent.data_ptr(),
                       poffs.data_ptr())
    args = (_ptr(H0), ctypes.byref(f), _ptr(prev_accepted_idx), _ptr(prev_accepted_len),
            ctypes.byref(pdims), _ptr(prev_path_nodes), _ptr(prev_tree_status), _ptr(q), _ptr(k),
            _ptr(v), _ptr(gate), _ptr(parent), _ptr(node_offsets), _ptr(out), ctypes.byref(dims),
            _ptr(tree_status), _stream(stream))
    keep = (H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate, parent, node_offsets,
            out, prev_path_nodes, prev_tree_status, tree_status, dims, pdims, f)
    return out, args, keep


def bole_tree_verify_lazy_commit(H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate,
                                 parent, node_offsets, out=None, prev_path_nodes=None,
                                 prev_tree_status=None, tree_status=None, stream=None,
                                 trees_le_32=False, prev_trees_le_32=False, validate_gates=False):
    """Commits the previous step's accepted path into H0 and verifies this step's tree
    against the result, in one pass over H0. prev = (k, v, gate, parent, node_offsets)
    of the previous step. Same result as bole_commit_path(previous step) followed by
    bole_tree_verify(this step), to fp32 rounding; returns out. validate_gates sets
    BOLE_FLAG_VALIDATE_GATES for both steps."""
    out, args, _ = _lazy_args(H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate,
                              parent, node_offsets, out, prev_path_nodes, prev_tree_status,
                              tree_status, stream, trees_le_32, prev_trees_le_32, validate_gates)
    _check(lib.bole_tree_verify_lazy_commit(*args), "bole_tree_verify_lazy_commit")
    return out


class _Bound:
    """A launch whose arguments were checked and marshalled once; calling it enqueues the
    same C call again (the tensors are kept alive by the object)."""

    def __init__(self, fn, what, args, keep):
        self._fn, self._what, self._args, self._keep = fn, what, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != BOLE_OK:
            _check(st, self._what)


def bind_tree_verify(H0, q, k, v, gate, parent, node_offsets, out, tree_status=None,
                     stream=None, force_generic=False, trees_le_32=False, validate_gates=False):
    """Same checks as bole_tree_verify, done once; returns a callable that launches the
    verify on these buffers each time it is called (for tight launch loops)."""
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    _need(q, "q", k.dtype, H0.device)
    _need(out, "out", torch.float32, H0.device)
    if tuple(q.shape) != tuple(k.shape) or tuple(out.shape) != (T, Hh, d_v):
        raise ValueError("q must have the shape of k and out must be [T, H, d_v]")
    if tree_status is not None:
        _need(tree_status, "tree_status", torch.int32, H0.device)
        if tree_status.numel() < B:
            raise ValueError("tree_status needs B entries")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, 0, force_generic, trees_le_32,
                     validate_gates)
    args = (_ptr(H0), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(parent), _ptr(node_offsets),
            _ptr(out), ctypes.byref(dims), _ptr(tree_status), _stream(stream))
    return _Bound(lib.bole_tree_verify, "bole_tree_verify", args,
                  (H0, q, k, v, gate, parent, node_offsets, out, tree_status, dims))


def bind_commit_path(H0, k, v, gate, parent, node_offsets, accepted_idx, accepted_len,
                     path_nodes=None, tree_status=None, stream=None, trees_le_32=False,
                     validate_gates=False):
    """Same checks as bole_commit_path, done once; returns a callable that commits into
    H0 in place each time it is called."""
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    _need(accepted_idx, "accepted_idx", torch.int32, H0.device)
    _need(accepted_len, "accepted_len", torch.int32, H0.device)
    if accepted_idx.dim() != 2 or accepted_idx.shape[0] != B or tuple(accepted_len.shape) != (B,):
        raise ValueError("accepted_idx must be [B, max_path] and accepted_len [B]")
    max_path = accepted_idx.shape[1]
    for t, name in ((path_nodes, "path_nodes"), (tree_status, "tree_status")):
        if t is not None:
            _need(t, name, torch.int32, H0.device)
    if path_nodes is not None and tuple(path_nodes.shape) != (B, max_path):
        raise ValueError("path_nodes must be [B, max_path]")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, max_path, trees_le_32=trees_le_32,
                     validate_gates=validate_gates)
    f = bole_factors_t(k.data_ptr(), v.data_ptr(), gate.data_ptr(), parent.data_ptr(),
                       node_offsets.data_ptr())
    args = (_ptr(H0), ctypes.byref(f), _ptr(accepted_idx), _ptr(accepted_len),
            ctypes.byref(dims), _ptr(path_nodes), _ptr(tree_status), _stream(stream))
    return _Bound(lib.bole_commit_path, "bole_commit_path", args,
                  (H0, k, v, gate, parent, node_offsets, accepted_idx, accepted_len, path_nodes,
                   tree_status, dims, f))


def bind_tree_verify_lazy_commit(H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate,
                                 parent, node_offsets, out, prev_path_nodes=None,
                                 prev_tree_status=None, tree_status=None, stream=None,
                                 trees_le_32=False, prev_trees_le_32=False, validate_gates=False):
    """Same checks as bole_tree_verify_lazy_commit, done once; returns a callable that
    launches it on these buffers each time it is called."""
    _, args, keep = _lazy_args(H0, prev, prev_accepted_idx, prev_accepted_len, q, k, v, gate,
                               parent, node_offsets, out, prev_path_nodes, prev_tree_status,
                               tree_status, stream, trees_le_32, prev_trees_le_32, validate_gates)
    return _Bound(lib.bole_tree_verify_lazy_commit, "bole_tree_verify_lazy_commit", args, keep)


def bole_commit_path(H0, k, v, gate, parent, node_offsets, accepted_idx, accepted_len,
                     path_nodes=None, tree_status=None, stream=None, trees_le_32=False,
                     validate_gates=False):
    """Commits each tree's accepted path into H0 in place; returns H0."""
    B, Hh, d_k, d_v, T, vec = _factor_dims(H0, k, v, gate, parent, node_offsets)
    _need(accepted_idx, "accepted_idx", torch.int32, H0.device)
    _need(accepted_len, "accepted_len", torch.int32, H0.device)
    if accepted_idx.dim() != 2 or accepted_idx.shape[0] != B or tuple(accepted_len.shape) != (B,):
        raise ValueError("accepted_idx must be [B, max_path] and accepted_len [B]")
    max_path = accepted_idx.shape[1]
    for t, name in ((path_nodes, "path_nodes"), (tree_status, "tree_status")):
        if t is not None:
            _need(t, name, torch.int32, H0.device)
    if path_nodes is not None and tuple(path_nodes.shape) != (B, max_path):
        raise ValueError("path_nodes must be [B, max_path]")
    dims = make_dims(B, Hh, d_k, d_v, T, k.dtype, vec, max_path, trees_le_32=trees_le_32,
                     validate_gates=validate_gates)
    f = bole_factors_t(k.data_ptr(), v.data_ptr(), gate.data_ptr(), parent.data_ptr(),
                       node_offsets.data_ptr())
    _check(lib.bole_commit_path(_ptr(H0), ctypes.byref(f), _ptr(accepted_idx),
                                _ptr(accepted_len), ctypes.byref(dims), _ptr(path_nodes),
                                _ptr(tree_status), _stream(stream)), "bole_commit_path")
    return H0


# ---- layer stacks: a layer is a dict with H0, q, k, v, gate, and as needed out (verify;
# allocated when missing) and prev_k, prev_v, prev_gate (lazy commit). All layers share
# the shapes of the first and the trees passed beside them.

def _layers_args(layers, parent, node_offsets, verify, prev_parent=None, prev_node_offsets=None):
    if len(layers) < 1:
        raise ValueError("need at least one layer")
    y0 = layers[0]
    dims = _factor_dims(y0["H0"], y0["k"], y0["v"], y0["gate"], parent, node_offsets)
    B, Hh, d_k, d_v, T, vec = dims
    pT = None
    arr = (bole_layer_t * len(layers))()
    keep = [layers, arr]
    for i, y in enumerate(layers):
        H0, k, v, gate = y["H0"], y["k"], y["v"], y["gate"]
        if _factor_dims(H0, k, v, gate, parent, node_offsets) != dims or k.dtype != y0["k"].dtype:
            raise ValueError(f"layer {i} does not match layer 0's shapes and dtypes")
        e = arr[i]
        e.H0, e.k, e.v, e.gate = H0.data_ptr(), k.data_ptr(), v.data_ptr(), gate.data_ptr()
        if verify:
            q = y["q"]
            _need(q, "q", k.dtype, H0.device)
            if tuple(q.shape) != tuple(k.shape):
                raise ValueError("q must have the shape of k")
            if y.get("out") is None:
                y["out"] = torch.empty((T, Hh, d_v), dtype=torch.float32, device=H0.device)
            _need(y["out"], "out", torch.float32, H0.device)
            if tuple(y["out"].shape) != (T, Hh, d_v):
                raise ValueError("out must be [T, H, d_v]")
            e.q, e.out = q.data_ptr(), y["out"].data_ptr()
        if prev_parent is not None:
            pk, pv, pg = y["prev_k"], y["prev_v"], y["prev_gate"]
            pd = _factor_dims(H0, pk, pv, pg, prev_parent, prev_node_offsets)
            if pk.dtype != k.dtype or pd[5] != vec:
                raise ValueError("the previous step's factors must match this step's dtype "
                                 "and gate kind")
            pT = pd[4]
            e.prev_k, e.prev_v, e.prev_gate = pk.data_ptr(), pv.data_ptr(), pg.data_ptr()
    return arr, dims, pT, keep


def _status_arg(t, name, B, dev):
    if t is not None:
        _need(t, name, torch.int32, dev)
        if t.numel() < B:
            raise ValueError(f"{name} needs B entries")
    return _ptr(t)


def _path_args(accepted_idx, accepted_len, path_nodes, B, dev, what=""):
    _need(accepted_idx, what + "accepted_idx", torch.int32, dev)
    _need(accepted_len, what + "accepted_len", torch.int32, dev)
    if accepted_idx.dim() != 2 or accepted_idx.shape[0] != B or tuple(accepted_len.shape) != (B,):
        raise ValueError(f"{what}accepted_idx must be [B, max_path] and {what}accepted_len [B]")
    max_path = accepted_idx.shape[1]
    if path_nodes is not None:
        _need(path_nodes, what + "path_nodes", torch.int32, dev)
        if tuple(path_nodes.shape) != (B, max_path):
            raise ValueError(f"{what}path_nodes must be [B, max_path]")
    return max_path


def _verify_layers_call(layers, parent, node_offsets, tree_status, stream, force_generic,
                        trees_le_32, validate_gates=False):
    arr, (B, Hh, d_k, d_v, T, vec), _, keep = _layers_args(layers, parent, node_offsets, True)
    dev = layers[0]["H0"].device
    dims = make_dims(B, Hh, d_k, d_v, T, layers[0]["k"].dtype, vec, 0, force_generic, trees_le_32,
                     validate_gates)
    args = (arr, len(layers), _ptr(parent), _ptr(node_offsets), ctypes.byref(dims),
            _status_arg(tree_status, "tree_status", B, dev), _stream(stream))
    return args, keep + [parent, node_offsets, tree_status, dims]


def bole_tree_verify_layers(layers, parent, node_offsets, tree_status=None, stream=None,
                            force_generic=False, trees_le_32=False, validate_gates=False):
    """bole_tree_verify on every layer of a stack that shares the trees, in as few
    launches as the kernels allow; returns the list of outs."""
    args, _ = _verify_layers_call(layers, parent, node_offsets, tree_status, stream,
                                  force_generic, trees_le_32, validate_gates)
    _check(lib.bole_tree_verify_layers(*args), "bole_tree_verify_layers")
    return [y["out"] for y in layers]


def bind_tree_verify_layers(layers, parent, node_offsets, tree_status=None, stream=None,
                            force_generic=False, trees_le_32=False, validate_gates=False):
    args, keep = _verify_layers_call(layers, parent, node_offsets, tree_status, stream,
                                     force_generic, trees_le_32, validate_gates)
    return _Bound(lib.bole_tree_verify_layers, "bole_tree_verify_layers", args, keep)


def _commit_layers_call(layers, parent, node_offsets, accepted_idx, accepted_len, path_nodes,
                        tree_status, stream, trees_le_32, validate_gates=False):
    arr, (B, Hh, d_k, d_v, T, vec), _, keep = _layers_args(layers, parent, node_offsets, False)
    dev = layers[0]["H0"].device
    max_path = _path_args(accepted_idx, accepted_len, path_nodes, B, dev)
    dims = make_dims(B, Hh, d_k, d_v, T, layers[0]["k"].dtype, vec, max_path,
                     trees_le_32=trees_le_32, validate_gates=validate_gates)
    args = (arr, len(layers), _ptr(parent), _ptr(node_offsets), _ptr(accepted_idx),
            _ptr(accepted_len), ctypes.byref(dims), _ptr(path_nodes),
            _status_arg(tree_status, "tree_status", B, dev), _stream(stream))
    return args, keep + [parent, node_offsets, accepted_idx, accepted_len, path_nodes,
                         tree_status, dims]


def bole_commit_path_layers(layers, parent, node_offsets, accepted_idx, accepted_len,
                            path_nodes=None, tree_status=None, stream=None, trees_le_32=False,
                            validate_gates=False):
    """bole_commit_path of each layer's k, v, gate along the shared accepted paths."""
    args, _ = _commit_layers_call(layers, parent, node_offsets, accepted_idx, accepted_len,
                                  path_nodes, tree_status, stream, trees_le_32, validate_gates)
    _check(lib.bole_commit_path_layers(*args), "bole_commit_path_layers")


def bind_commit_path_layers(layers, parent, node_offsets, accepted_idx, accepted_len,
                            path_nodes=None, tree_status=None, stream=None, trees_le_32=False,
                            validate_gates=False):
    args, keep = _commit_layers_call(layers, parent, node_offsets, accepted_idx, accepted_len,
                                     path_nodes, tree_status, stream, trees_le_32, validate_gates)
    return _Bound(lib.bole_commit_path_layers, "bole_commit_path_layers", args, keep)


def _lazy_layers_call(layers, prev_parent, prev_node_offsets, prev_accepted_idx,
                      prev_accepted_len, parent, node_offsets, prev_path_nodes, prev_tree_status,
                      tree_status, stream, trees_le_32, prev_trees_le_32, validate_gates=False):
    arr, (B, Hh, d_k, d_v, T, vec), pT, keep = _layers_args(
        layers, parent, node_offsets, True, prev_parent, prev_node_offsets)
    dev = layers[0]["H0"].device
    max_path = _path_args(prev_accepted_idx, prev_accepted_len, prev_path_nodes, B, dev, "prev_")
    fd = layers[0]["k"].dtype
    dims = make_dims(B, Hh, d_k, d_v, T, fd, vec, 0, trees_le_32=trees_le_32,
                     validate_gates=validate_gates)
    pdims = make_dims(B, Hh, d_k, d_v, pT, fd, vec, max_path, trees_le_32=prev_trees_le_32,
                      validate_gates=validate_gates)
    args = (arr, len(layers), _ptr(prev_parent), _ptr(prev_node_offsets), _ptr(prev_accepted_idx),
            _ptr(prev_accepted_len), ctypes.byref(pdims), _ptr(prev_path_nodes),
            _status_arg(prev_tree_status, "prev_tree_status", B, dev), _ptr(parent),
            _ptr(node_offsets), ctypes.byref(dims), _status_arg(tree_status, "tree_status", B, dev),
            _stream(stream))
    return args, keep + [prev_parent, prev_node_offsets, prev_accepted_idx, prev_accepted_len,
                         parent, node_offsets, prev_path_nodes, prev_tree_status, tree_status,
                         dims, pdims]


def bole_tree_verify_lazy_commit_layers(layers, prev_parent, prev_node_offsets,
                                        prev_accepted_idx, prev_accepted_len, parent,
                                        node_offsets, prev_path_nodes=None, prev_tree_status=None,
                                        tree_status=None, stream=None, trees_le_32=False,
                                        prev_trees_le_32=False, validate_gates=False):
    """bole_tree_verify_lazy_commit on every layer of a stack (each layer's prev_k,
    prev_v, prev_gate along the shared previous path, then its verify); returns the outs.
    validate_gates sets BOLE_FLAG_VALIDATE_GATES for both steps."""
    args, _ = _lazy_layers_call(layers, prev_parent, prev_node_offsets, prev_accepted_idx,
                                prev_accepted_len, parent, node_offsets, prev_path_nodes,
                                prev_tree_status, tree_status, stream, trees_le_32,
                                prev_trees_le_32, validate_gates)
    _check(lib.bole_tree_verify_lazy_commit_layers(*args), "bole_tree_verify_lazy_commit_layers")
    return [y["out"] for y in layers]


def bind_tree_verify_lazy_commit_layers(layers, prev_parent, prev_node_offsets,
                                        prev_accepted_idx, prev_accepted_len, parent,
                                        node_offsets, prev_path_nodes=None, prev_tree_status=None,
                                        tree_status=None, stream=None, trees_le_32=False,
                                        prev_trees_le_32=False, validate_gates=False):
    args, keep = _lazy_layers_call(layers, prev_parent, prev_node_offsets, prev_accepted_idx,
                                   prev_accepted_len, parent, node_offsets, prev_path_nodes,
                                   prev_tree_status, tree_status, stream, trees_le_32,
                                   prev_trees_le_32, validate_gates)
    return _Bound(lib.bole_tree_verify_lazy_commit_layers, "bole_tree_verify_lazy_commit_layers",
                  args, keep)


# ---- draft-tree construction (best-first expansion and budget controller)

def _build_call(marginals, cost, l_ar, n_max, fixed, workspace, out, stream):
    _need(marginals, "marginals", torch.float32)
    dev = marginals.device
    if marginals.dim() != 3:
        raise ValueError("marginals must be [B, depth, vocab]")
    B, D, V = marginals.shape
    if cost is not None:
        _need(cost, "cost", torch.float32, dev)
        if cost.numel() < n_max:
            raise ValueError("cost needs n_max entries")
    dims = bole_build_dims_t(B, D, V, n_max, BOLE_BUILD_FIXED_BUDGET if fixed else 0)
    need = lib.bole_build_tree_workspace_size(ctypes.byref(dims))
    if need == 0:
        raise ValueError("unsupported tree-build dims (depth 1..32, n_max 1..64, vocab >= 1)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    if out is None:
        cap = max(B * n_max, 1)
        out = {"node_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
               "parent": torch.empty(cap, dtype=torch.int32, device=dev),
               "token": torch.empty(cap, dtype=torch.int32, device=dev),
               "rho": torch.empty(cap, dtype=torch.float32, device=dev),
               "speedup": torch.empty(max(B, 1), dtype=torch.float32, device=dev) if cost is not None else None}
    args = (_ptr(marginals), _ptr(cost), ctypes.c_float(l_ar), _ptr(workspace),
            workspace.numel() * workspace.element_size(), ctypes.byref(dims),
            _ptr(out["node_offsets"]), _ptr(out["parent"]), _ptr(out["token"]), _ptr(out.get("rho")),
            _ptr(out.get("speedup")), _stream(stream))
    return args, out, (marginals, cost, workspace, out, dims)


def bole_build_tree(marginals, cost, l_ar=1.0, n_max=64, fixed=False, workspace=None, out=None,
                    stream=None):
    """Best-first draft trees from position-wise marginals [B, depth, vocab] (fp32
    probabilities) with the budget controller over cost[n_max] (C(N) at N - 1) and L_AR.
    Returns a dict of device tensors: node_offsets [B + 1], and parent, token, rho (packed,
    capacity B * n_max; node_offsets[B] of them are written), speedup [B]."""
    args, out, _ = _build_call(marginals, cost, l_ar, n_max, fixed, workspace, out, stream)
    _check(lib.bole_build_tree(*args), "bole_build_tree")
    return out


BUILD_NOALLOC_MAX_BYTES = 4 << 20


def bole_build_tree_noalloc(marginals, cost, l_ar=1.0, n_max=64, fixed=False, out=None,
                            stream=None):
    """bole_build_tree with the library's own scratch array instead of a workspace: the
    call allocates no device memory (pass `out` to allocate nothing at all). Dims whose
    workspace would exceed BUILD_NOALLOC_MAX_BYTES raise BoleError (BOLE_ERR_UNSUPPORTED).
    Calls that overlap on one GPU race on the shared array."""
    _need(marginals, "marginals", torch.float32)
    dev = marginals.device
    if marginals.dim() != 3:
        raise ValueError("marginals must be [B, depth, vocab]")
    B, D, V = marginals.shape
    if cost is not None:
        _need(cost, "cost", torch.float32, dev)
        if cost.numel() < n_max:
            raise ValueError("cost needs n_max entries")
    dims = bole_build_dims_t(B, D, V, n_max, BOLE_BUILD_FIXED_BUDGET if fixed else 0)
    if out is None:
        cap = max(B * n_max, 1)
        out = {"node_offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
               "parent": torch.empty(cap, dtype=torch.int32, device=dev),
               "token": torch.empty(cap, dtype=torch.int32, device=dev),
               "rho": torch.empty(cap, dtype=torch.float32, device=dev),
               "speedup": torch.empty(max(B, 1), dtype=torch.float32, device=dev) if cost is not None else None}
    _check(lib.bole_build_tree_noalloc(_ptr(marginals), _ptr(cost), ctypes.c_float(l_ar),
                                       ctypes.byref(dims), _ptr(out["node_offsets"]),
                                       _ptr(out["parent"]), _ptr(out["token"]),
                                       _ptr(out.get("rho")), _ptr(out.get("speedup")),
                                       _stream(stream)), "bole_build_tree_noalloc")
    return out


def bind_build_tree(marginals, cost, l_ar=1.0, n_max=64, fixed=False, workspace=None, out=None,
                    stream=None):
    args, out, keep = _build_call(marginals, cost, l_ar, n_max, fixed, workspace, out, stream)
    bound = _Bound(lib.bole_build_tree, "bole_build_tree", args, keep)
    bound.out = out
    return bound


# ---- tree acceptance

def _accept_call(p_ctx, p_node, parent, token, node_offsets, max_path, sample, q_ctx, q_node,
                 u_node, u_bonus, out, stream):
    _need(p_ctx, "p_ctx", torch.float32)
    dev = p_ctx.device
    if p_ctx.dim() != 2:
        raise ValueError("p_ctx must be [B, V]")
    B, V = p_ctx.shape
    _need(p_node, "p_node", torch.float32, dev)
    _need(parent, "parent", torch.int32, dev)
    _need(token, "token", torch.int32, dev)
    _need(node_offsets, "node_offsets", torch.int32, dev)
    T = parent.shape[0]
    if tuple(p_node.shape) != (T, V) or tuple(token.shape) != (T,) or \
            tuple(node_offsets.shape) != (B + 1,):
        raise ValueError("p_node must be [T, V], token [T] and node_offsets [B + 1]")
    if sample:
        for t, name, shape in ((q_ctx, "q_ctx", (B, V)), (q_node, "q_node", (T, V)),
                               (u_node, "u_node", (T,)), (u_bonus, "u_bonus", (B,))):
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {list(shape)}")
    dims = bole_accept_dims_t(B, T, V, max_path, BOLE_ACCEPT_SAMPLE if sample else BOLE_ACCEPT_GREEDY)
    if out is None:
        out = {"accepted_idx": torch.empty((max(B, 1), max_path), dtype=torch.int32, device=dev),
               "accepted_len": torch.empty(max(B, 1), dtype=torch.int32, device=dev),
               "bonus": torch.empty(max(B, 1), dtype=torch.int32, device=dev),
               "status": torch.empty(max(B, 1), dtype=torch.int32, device=dev)}
    args = (_ptr(p_ctx), _ptr(p_node), _ptr(q_ctx), _ptr(q_node), _ptr(parent), _ptr(token),
            _ptr(node_offsets), _ptr(u_node), _ptr(u_bonus), ctypes.byref(dims), _ptr(out["accepted_idx"]), _ptr(out["accepted_len"]),
            _ptr(out["bonus"]), _ptr(out["status"]), _stream(stream))
    keep = (p_ctx, p_node, parent, token, node_offsets, q_ctx, q_node, u_node, u_bonus, out,
            dims)
    return args, out, keep


def bole_tree_accept(p_ctx, p_node, parent, token, node_offsets, max_path, sample=False,
                     q_ctx=None, q_node=None, u_node=None, u_bonus=None, out=None, stream=None):
    """Accepted path and bonus token per tree: greedy longest match against the target's
    argmax, or (sample=True) min(1, p/q) acceptance with residual resampling. Returns a
    dict of device tensors accepted_idx [B, max_path], accepted_len [B], bonus [B],
    status [B]."""
    args, out, _ = _accept_call(p_ctx, p_node, parent, token, node_offsets, max_path, sample,
                                q_ctx, q_node, u_node, u_bonus, out, stream)
    _check(lib.bole_tree_accept(*args), "bole_tree_accept")
    return out


def bind_tree_accept(p_ctx, p_node, parent, token, node_offsets, max_path, sample=False,
                     q_ctx=None, q_node=None, u_node=None, u_bonus=None, out=None, stream=None):
    args, out, keep = _accept_call(p_ctx, p_node, parent, token, node_offsets, max_path, sample,
                                   q_ctx, q_node, u_node, u_bonus, out, stream)
    bound = _Bound(lib.bole_tree_accept, "bole_tree_accept", args, keep)
    bound.out = out
    return bound


def bole_tree_prepare(parent, node_offsets, heads=1, d_k=1, gate=None, want_cumlog=False,
                      tree_status=None, stream=None, validate_gates=False):
    """Topology export: (depth int32[T], mask int64[T] holding the uint64 bits,
    cumlog float32 [T, H] / [T, H, d_k] or None)."""
    _need(parent, "parent", torch.int32)
    dev = parent.device
    _need(node_offsets, "node_offsets", torch.int32, dev)
    T, B = parent.shape[0], node_offsets.shape[0] - 1
    vec = gate is not None and gate.dim() == 3
    if want_cumlog:
        _need(gate, "gate", torch.float32, dev)
        heads = gate.shape[1]
        d_k = gate.shape[2] if vec else d_k
    depth = torch.zeros(T, dtype=torch.int32, device=dev)
    mask = torch.zeros(T, dtype=torch.int64, device=dev)
    cum = None
    if want_cumlog:
        cum = torch.zeros(tuple(gate.shape), dtype=torch.float32, device=dev)
    if tree_status is not None:
        _need(tree_status, "tree_status", torch.int32, dev)
    if validate_gates:
        _need(gate, "gate", torch.float32, dev)
        heads = gate.shape[1]
        d_k = gate.shape[2] if vec else d_k
    dims = make_dims(B, heads, d_k, 1, T, torch.float32, vec, validate_gates=validate_gates)
    _check(lib.bole_tree_prepare(_ptr(parent), _ptr(node_offsets), _ptr(gate), ctypes.byref(dims),
                                 _ptr(depth), _ptr(mask), _ptr(cum), _ptr(tree_status),
                                 _stream(None)), "bole_tree_prepare")
    return depth, mask, cum


# ---- boundary helpers

def bole_workspace_bytes(dims=None) -> int:
    """Scratch bytes verify, commit and prepare need (always 0)."""
    return int(lib.bole_workspace_bytes(None if dims is None else ctypes.byref(dims)))


def bole_read_status(tree_status, batch=None, stream=None):
    """Blocks until `stream`'s work is done and returns (host int32 numpy array of the
    first `batch` statuses, C status: BOLE_OK or BOLE_ERR_BAD_TREE)."""
    import numpy as np
    _need(tree_status, "tree_status", torch.int32)
    B = tree_status.numel() if batch is None else int(batch)
    host = np.zeros(max(B, 0), np.int32)
    st = lib.bole_read_status(_ptr(tree_status), B, host.ctypes.data_as(ctypes.c_void_p),
                              _stream(stream))
    if st not in (BOLE_OK, BOLE_ERR_BAD_TREE):
        _check(st, "bole_read_status")
    return host, st
