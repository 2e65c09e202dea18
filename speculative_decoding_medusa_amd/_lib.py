"""ctypes binding of libmedusa: argument marshalling only.

Every function here has the name of the C entry point it calls, checks the
tensors it is handed (device, dtype, contiguity, shape), allocates missing
outputs and workspaces with torch, passes raw pointers and torch's current
HIP stream, and raises MedusaError on a negative status.  All computation
happens in the library's HIP kernels; there is no other code path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa.so")

MEDUSA_F32 = 0
MEDUSA_BF16 = 1
_ERR_SHAPE = -2   # MEDUSA_ERR_SHAPE

SPEC_STATUS = {0: "ok", 1: "padding", 2: "empty", 3: "rank", 4: "duplicate", 5: "prefix",
               6: "too_many_paths"}


class MedusaError(RuntimeError):
    def __init__(self, code, fn, msg):
        super().__init__("%s failed with status %d: %s" % (fn, code, msg))
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libmedusa.so is not built (expected at %s); run "
            "`python speculative_decoding_medusa_amd/build.py`" % LIB_PATH)
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "medusa_heads_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "medusa_resblock": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "medusa_lm_head_topk": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "medusa_heads": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "medusa_lm_head_topk_tree": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _sz, _vp]),
    "medusa_heads_tree": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _sz, _vp]),
    "medusa_heads_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "medusa_lm_head_topk_packed": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "medusa_heads_packed_bytes": (_sz, [_i, _i, _i]),
    "medusa_tree_candidates": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "medusa_linear_workspace": (_sz, [_i, _i, _i]),
    "medusa_linear": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "medusa_heads_packed": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "medusa_heads_pack": (_i, [_i, _i, _i, _i, _vp, _vp, _vp]),
    "medusa_build_tree": (_i, [_i, _i, _i, _i] + [_vp] * 12 + [_i, _vp, _vp]),
    "medusa_tree_attention_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "medusa_tree_attention": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _sz, _vp]),
    "medusa_posterior_workspace": (_sz, [_i, _i, _i]),
    "medusa_evaluate_posterior": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _f, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "medusa_commit_kv": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp]),
    "medusa_base_lm_head_packed_bytes": (_sz, [_i, _i]),
    "medusa_base_lm_head_pack": (_i, [_i, _i, _i, _vp, _vp, _vp]),
    "medusa_base_lm_head": (_i, [_i, _i, _i, _i, _vp, _vp, _i, _vp, _vp]),
    "medusa_base_posterior_workspace": (_sz, [_i, _i, _i, _i]),
    "medusa_base_posterior": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _vp, _f, _f, _f, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "medusa_posterior_nucleus_workspace": (_sz, [_i, _i]),
    "medusa_evaluate_posterior_nucleus": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _sz, _vp]),
    "medusa_philox_uniforms": (_i, [ctypes.c_uint64, ctypes.c_uint64, _i, _i, _i, _vp, _vp]),
    "medusa_sample_typical": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _f, ctypes.c_uint64,
                                   ctypes.c_uint64, _vp, _vp]),
    "medusa_embed": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp]),
    "medusa_add_rmsnorm": (_i, [_i, _i, _vp, _vp, _vp, _f, _vp, _vp]),
    "medusa_rope_qkv": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp]),
    "medusa_silu_mul": (_i, [_i, _i, _vp, _vp, _vp]),
    "medusa_status_string": (ctypes.c_char_p, [_i]),
    "medusa_last_error": (ctypes.c_char_p, []),
    "medusa_abi_version": (_i, []),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(rc, fn):
    if rc != 0:
        raise MedusaError(rc, fn, "%s (%s)" % (lib.medusa_status_string(rc).decode(),
                                               lib.medusa_last_error().decode()))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MEDUSA_BF16
    if t.dtype == torch.float32:
        return MEDUSA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


_WS = {}


def workspace(kind, device, nbytes):
    """A cached workspace of at least ``nbytes`` bytes, one per kind, device
    and stream: calls that share a workspace must not overlap, and calls on
    different streams may, so each stream gets its own.  (Two threads
    issuing calls on the same stream still share one; pass ``ws`` to keep
    them apart.)"""
    dev = torch.device(device)
    key = (kind, dev.index, torch.cuda.current_stream(dev).cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def medusa_heads_workspace(dtype, B, H, V, K, topk):
    return int(lib.medusa_heads_workspace(dtype, B, H, V, K, topk))


def medusa_resblock(hidden, w1, b1, r=None):
    dt = _dtype_code(hidden)
    B, H = hidden.shape
    K = w1.shape[0]
    dev = hidden.device
    if r is None:
        r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
    rc = lib.medusa_resblock(dt, B, H, K, _ptr(hidden, "hidden"), _ptr(w1, "w1", hidden.dtype, (K, H, H)),
                             _ptr(b1, "b1", hidden.dtype, (K, H)), _ptr(r, "r", torch.float32, (B, K, H)),
                             _stream(dev))
    _check(rc, "medusa_resblock")
    return r


def medusa_lm_head_topk(r, w_lm, topk, keep_logits=False, out=None, ws=None):
    dt = _dtype_code(w_lm)
    B, K, H = r.shape
    V = w_lm.shape[1]
    dev = r.device
    out = out or {}
    ids = out.get("topk_ids")
    vals = out.get("topk_logits")
    logits = out.get("logits")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    if keep_logits and logits is None:
        logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    need = medusa_heads_workspace(dt, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_lm_head_topk(dt, B, H, V, K, topk, _ptr(r, "r", torch.float32),
                                 _ptr(w_lm, "w_lm", None, (K, V, H)),
                                 _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                                 _ptr(vals, "topk_logits", torch.float32, (B, K, topk)),
                                 _ptr(logits, "logits", torch.float32, (B, K, V)),
                                 _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_lm_head_topk")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits)


def _check_packed(t, name, K, H, V):
    need = int(lib.medusa_heads_packed_bytes(K, H, V))
    if t.dtype != torch.uint8 or t.numel() < need:
        raise MedusaError(_ERR_SHAPE, name, "expected >= %d packed bytes (uint8), got %s of %d elements"
                          % (need, t.dtype, t.numel()))


def medusa_heads_pack(w_lm):
    """bf16 [K][V][H] head weights -> the packed layout (uint8 tensor)."""
    K, V, H = w_lm.shape
    nbytes = int(lib.medusa_heads_packed_bytes(K, H, V))
    if nbytes == 0:
        raise MedusaError(_ERR_SHAPE, "medusa_heads_pack", "unsupported shape K=%d H=%d V=%d" % (K, H, V))
    out = torch.empty(nbytes, dtype=torch.uint8, device=w_lm.device)
    rc = lib.medusa_heads_pack(MEDUSA_BF16, K, H, V, _ptr(w_lm, "w_lm", torch.bfloat16), _ptr(out, "w_packed"),
                               _stream(w_lm.device))
    _check(rc, "medusa_heads_pack")
    return out


def medusa_lm_head_topk_packed(r, w_packed, V, topk, keep_logits=False, out=None, ws=None):
    """lm_head + top-k on packed head weights (medusa_heads_pack); r float32 [B][K][H]."""
    B, K, H = r.shape
    dev = r.device
    out = out or {}
    ids = out.get("topk_ids")
    vals = out.get("topk_logits")
    logits = out.get("logits")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    if keep_logits and logits is None:
        logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    _check_packed(w_packed, "w_packed", K, H, V)
    need = medusa_heads_workspace(MEDUSA_BF16, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_lm_head_topk_packed(MEDUSA_BF16, B, H, V, K, topk, _ptr(r, "r", torch.float32, (B, K, H)),
                                        _ptr(w_packed, "w_packed", torch.uint8),
                                        _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                                        _ptr(vals, "topk_logits", torch.float32, (B, K, topk)),
                                        _ptr(logits, "logits", torch.float32, (B, K, V)),
                                        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_lm_head_topk_packed")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits)


def medusa_heads_packed(hidden, w1_packed, b1, w_lm_packed, V, topk, keep_logits=False, keep_r=False, out=None,
                        ws=None):
    """Both head stages on packed weights (medusa_heads_pack of W1 with V = H
    and of w_lm); hidden bf16 [B][H], b1 bf16 [K][H]."""
    B, H = hidden.shape
    K = b1.shape[0]
    dev = hidden.device
    out = out or {}
    ids = out.get("topk_ids")
    vals = out.get("topk_logits")
    logits = out.get("logits")
    r = out.get("r")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    if keep_logits and logits is None:
        logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    if keep_r and r is None:
        r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
    _check_packed(w1_packed, "w1_packed", K, H, H)
    _check_packed(w_lm_packed, "w_lm_packed", K, H, V)
    need = medusa_heads_workspace(MEDUSA_BF16, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_heads_packed(MEDUSA_BF16, B, H, V, K, topk, _ptr(hidden, "hidden", torch.bfloat16, (B, H)),
                                 _ptr(w1_packed, "w1_packed", torch.uint8), _ptr(b1, "b1", torch.bfloat16, (K, H)),
                                 _ptr(w_lm_packed, "w_lm_packed", torch.uint8),
                                 _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                                 _ptr(vals, "topk_logits", torch.float32, (B, K, topk)),
                                 _ptr(logits, "logits", torch.float32, (B, K, V)),
                                 _ptr(r, "r", torch.float32, (B, K, H)),
                                 _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_heads_packed")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits, r=r)


def medusa_heads(hidden, w1, b1, w_lm, topk, keep_logits=False, keep_r=False, ws=None):
    dt = _dtype_code(hidden)
    B, H = hidden.shape
    K, V = w_lm.shape[0], w_lm.shape[1]
    dev = hidden.device
    ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    logits = torch.empty((B, K, V), dtype=torch.float32, device=dev) if keep_logits else None
    r = torch.empty((B, K, H), dtype=torch.float32, device=dev) if keep_r else None
    need = medusa_heads_workspace(dt, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_heads(dt, B, H, V, K, topk, _ptr(hidden, "hidden"),
                          _ptr(w1, "w1", hidden.dtype, (K, H, H)), _ptr(b1, "b1", hidden.dtype, (K, H)),
                          _ptr(w_lm, "w_lm", hidden.dtype, (K, V, H)), _ptr(ids, "topk_ids"),
                          _ptr(vals, "topk_logits"), _ptr(logits, "logits"), _ptr(r, "r"),
                          _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_heads")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits, r=r)


def medusa_heads_tree(hidden, w1, b1, w_lm, topk, tree_indices, depth, root_token, prefix_len, keep_logits=False,
                      keep_r=False, out=None, ws=None):
    """medusa_heads, then the tree gather of medusa_tree_candidates on its
    top-k, in one call (the gather runs inside the lm_head kernel where its
    top-k merge does)."""
    dt = _dtype_code(hidden)
    B, H = hidden.shape
    K, V = w_lm.shape[0], w_lm.shape[1]
    T = tree_indices.shape[0]
    dev = hidden.device
    o = out or {}
    ids = o.get("topk_ids")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    vals = o.get("topk_logits")
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    cand = o.get("tree_candidates")
    if cand is None:
        cand = torch.empty((B, T), dtype=torch.int32, device=dev)
    pos = o.get("position_ids")
    if pos is None:
        pos = torch.empty((B, T), dtype=torch.int32, device=dev)
    logits = torch.empty((B, K, V), dtype=torch.float32, device=dev) if keep_logits else None
    r = torch.empty((B, K, H), dtype=torch.float32, device=dev) if keep_r else None
    need = medusa_heads_workspace(dt, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_heads_tree(dt, B, H, V, K, topk, _ptr(hidden, "hidden"),
                               _ptr(w1, "w1", hidden.dtype, (K, H, H)), _ptr(b1, "b1", hidden.dtype, (K, H)),
                               _ptr(w_lm, "w_lm", hidden.dtype, (K, V, H)),
                               _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                               _ptr(vals, "topk_logits", torch.float32, (B, K, topk)), _ptr(logits, "logits"),
                               _ptr(r, "r"), T, _ptr(tree_indices, "tree_indices", torch.int32, (T,)),
                               _ptr(depth, "depth", torch.int32, (T,)),
                               _ptr(root_token, "root_token", torch.int32, (B,)),
                               _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                               _ptr(cand, "tree_candidates", torch.int32, (B, T)),
                               _ptr(pos, "position_ids", torch.int32, (B, T)),
                               _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_heads_tree")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits, r=r, tree_candidates=cand, position_ids=pos)


def medusa_lm_head_topk_tree(r, w_lm, topk, tree_indices, depth, root_token, prefix_len, keep_logits=False,
                             out=None, ws=None):
    """medusa_lm_head_topk on r [B][K][H], then the tree gather of
    medusa_tree_candidates on its top-k, in one call."""
    dt = _dtype_code(w_lm)
    B, K, H = r.shape
    V = w_lm.shape[1]
    T = tree_indices.shape[0]
    dev = r.device
    o = out or {}
    ids = o.get("topk_ids")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    vals = o.get("topk_logits")
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    cand = o.get("tree_candidates")
    if cand is None:
        cand = torch.empty((B, T), dtype=torch.int32, device=dev)
    pos = o.get("position_ids")
    if pos is None:
        pos = torch.empty((B, T), dtype=torch.int32, device=dev)
    logits = torch.empty((B, K, V), dtype=torch.float32, device=dev) if keep_logits else None
    need = medusa_heads_workspace(dt, B, H, V, K, topk)
    if ws is None:
        ws = workspace("heads", dev, need)
    rc = lib.medusa_lm_head_topk_tree(dt, B, H, V, K, topk, _ptr(r, "r", torch.float32, (B, K, H)),
                                      _ptr(w_lm, "w_lm", None, (K, V, H)),
                                      _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                                      _ptr(vals, "topk_logits", torch.float32, (B, K, topk)),
                                      _ptr(logits, "logits"), T,
                                      _ptr(tree_indices, "tree_indices", torch.int32, (T,)),
                                      _ptr(depth, "depth", torch.int32, (T,)),
                                      _ptr(root_token, "root_token", torch.int32, (B,)),
                                      _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                                      _ptr(cand, "tree_candidates", torch.int32, (B, T)),
                                      _ptr(pos, "position_ids", torch.int32, (B, T)),
                                      _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_lm_head_topk_tree")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits, tree_candidates=cand, position_ids=pos)


PURPOSE_NUCLEUS = 0
PURPOSE_NEXT_TOKEN = 1


def medusa_philox_uniforms(seed, step, purpose, B, T, device="cuda", out=None):
    """float32 [B][T] counter-based uniforms of (seed, step, sequence, node,
    purpose)."""
    if out is None:
        out = torch.empty((B, T), dtype=torch.float32, device=device)
    dev = out.device
    rc = lib.medusa_philox_uniforms(int(seed) & ((1 << 64) - 1), int(step) & ((1 << 64) - 1), int(purpose), B, T,
                                    _ptr(out, "out", torch.float32, (B, T)), _stream(dev))
    _check(rc, "medusa_philox_uniforms")
    return out


def medusa_sample_typical(logits, retrieve, best_path, accept_len, temperature, eps, delta, seed, step,
                          out=None):
    """Typical-mode next token per sequence, drawn at the last accepted node."""
    B, T, V = logits.shape
    p_max, D = retrieve.shape
    dev = logits.device
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=dev)
    rc = lib.medusa_sample_typical(B, T, V, p_max, D, _ptr(logits, "logits", torch.float32),
                                   _ptr(retrieve, "retrieve", torch.int32),
                                   _ptr(best_path, "best_path", torch.int32, (B,)),
                                   _ptr(accept_len, "accept_len", torch.int32, (B,)), float(temperature), float(eps),
                                   float(delta), int(seed) & ((1 << 64) - 1), int(step) & ((1 << 64) - 1),
                                   _ptr(out, "next_token", torch.int32, (B,)), _stream(dev))
    _check(rc, "medusa_sample_typical")
    return out


def medusa_heads_noalloc(hidden, w1, b1, w_lm, topk, keep_logits=False, keep_r=False, out=None):
    """medusa_heads on the library's per-GPU scratch (no workspace).  Outputs
    come from ``out`` (topk_ids, topk_logits and optionally logits, r) or are
    allocated here; the C call itself allocates nothing."""
    dt = _dtype_code(hidden)
    B, H = hidden.shape
    K, V = w_lm.shape[0], w_lm.shape[1]
    dev = hidden.device
    o = out or {}
    ids = o.get("topk_ids")
    vals = o.get("topk_logits")
    logits = o.get("logits")
    r = o.get("r")
    if ids is None:
        ids = torch.empty((B, K, topk), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, K, topk), dtype=torch.float32, device=dev)
    if logits is None and keep_logits:
        logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    if r is None and keep_r:
        r = torch.empty((B, K, H), dtype=torch.float32, device=dev)
    rc = lib.medusa_heads_noalloc(dt, B, H, V, K, topk, _ptr(hidden, "hidden"),
                                  _ptr(w1, "w1", hidden.dtype, (K, H, H)), _ptr(b1, "b1", hidden.dtype, (K, H)),
                                  _ptr(w_lm, "w_lm", hidden.dtype, (K, V, H)),
                                  _ptr(ids, "topk_ids", torch.int32, (B, K, topk)),
                                  _ptr(vals, "topk_logits", torch.float32, (B, K, topk)),
                                  _ptr(logits, "logits", torch.float32, (B, K, V)),
                                  _ptr(r, "r", torch.float32, (B, K, H)), _stream(dev))
    _check(rc, "medusa_heads_noalloc")
    return dict(topk_ids=ids, topk_logits=vals, logits=logits, r=r)


def medusa_build_tree(choices, topk_ids, root_token, prefix_len, p_max=None, out=None):
    """choices int32 [N][K] (device), topk_ids int32 [B][K][topk], root_token / prefix_len int32 [B]."""
    B, K, topk = topk_ids.shape
    N = choices.shape[0]
    T = N + 1
    dev = topk_ids.device
    if p_max is None:
        p_max = T
    o = out or {}

    def get(name, shape, dtype=torch.int32):
        t = o.get(name)
        return t if t is not None else torch.empty(shape, dtype=dtype, device=dev)

    res = dict(tree_candidates=get("tree_candidates", (B, T)), tree_indices=get("tree_indices", (T,)),
               parent=get("parent", (T,)), depth=get("depth", (T,)),
               position_ids=get("position_ids", (B, T)),
               tree_mask=get("tree_mask", (T, T), torch.uint8),
               retrieve=get("retrieve", (p_max, K + 1)), num_paths=get("num_paths", (1,)),
               status=get("status", (2,)))
    if N > 0:
        cptr = _ptr(choices, "choices", torch.int32, (N, K))
    else:
        cptr = None
    rc = lib.medusa_build_tree(B, K, topk, N, cptr, _ptr(topk_ids, "topk_ids", torch.int32),
                               _ptr(root_token, "root_token", torch.int32, (B,)),
                               _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                               _ptr(res["tree_candidates"], "tree_candidates", torch.int32, (B, T)),
                               _ptr(res["tree_indices"], "tree_indices", torch.int32, (T,)),
                               _ptr(res["parent"], "parent", torch.int32, (T,)),
                               _ptr(res["depth"], "depth", torch.int32, (T,)),
                               _ptr(res["position_ids"], "position_ids", torch.int32, (B, T)),
                               _ptr(res["tree_mask"], "tree_mask", torch.uint8, (T, T)),
                               _ptr(res["retrieve"], "retrieve", torch.int32, (p_max, K + 1)),
                               _ptr(res["num_paths"], "num_paths", torch.int32, (1,)), p_max,
                               _ptr(res["status"], "status", torch.int32, (2,)), _stream(dev))
    _check(rc, "medusa_build_tree")
    return res


def medusa_tree_candidates(tree_indices, depth, topk_ids, root_token, prefix_len, out=None):
    """Per-step gather on a tree built by medusa_build_tree: tree_candidates and
    position_ids [B][T] for new topk_ids [B][K][topk], root_token, prefix_len [B]."""
    B, K, topk = topk_ids.shape
    T = tree_indices.shape[0]
    dev = topk_ids.device
    o = out or {}
    cand = o.get("tree_candidates")
    pos = o.get("position_ids")
    if cand is None:
        cand = torch.empty((B, T), dtype=torch.int32, device=dev)
    if pos is None:
        pos = torch.empty((B, T), dtype=torch.int32, device=dev)
    rc = lib.medusa_tree_candidates(B, T, K, topk, _ptr(tree_indices, "tree_indices", torch.int32, (T,)),
                                    _ptr(depth, "depth", torch.int32, (T,)),
                                    _ptr(topk_ids, "topk_ids", torch.int32, (B, K, topk)),
                                    _ptr(root_token, "root_token", torch.int32, (B,)),
                                    _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                                    _ptr(cand, "tree_candidates", torch.int32, (B, T)),
                                    _ptr(pos, "position_ids", torch.int32, (B, T)), _stream(dev))
    _check(rc, "medusa_tree_candidates")
    return dict(tree_candidates=cand, position_ids=pos)


def medusa_tree_attention_workspace(dtype, B, T, Hq, d, max_slots):
    return int(lib.medusa_tree_attention_workspace(dtype, B, T, Hq, d, max_slots))


def medusa_tree_attention(q, k_cache, v_cache, prefix_len, tree_mask, scale, out=None, ws=None):
    """q [B][T][Hq][d]; k_cache, v_cache [B][Hq][max_slots][d] (one layer)."""
    dt = _dtype_code(q)
    B, T, Hq, d = q.shape
    max_slots = k_cache.shape[2]
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    need = medusa_tree_attention_workspace(dt, B, T, Hq, d, max_slots)
    if ws is None:
        ws = workspace("attention", dev, need)
    rc = lib.medusa_tree_attention(dt, B, T, Hq, d, max_slots, _ptr(q, "q"),
                                   _ptr(k_cache, "k_cache", q.dtype, (B, Hq, max_slots, d)),
                                   _ptr(v_cache, "v_cache", q.dtype, (B, Hq, max_slots, d)),
                                   _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                                   _ptr(tree_mask, "tree_mask", torch.uint8, (T, T)), float(scale),
                                   _ptr(out, "out", q.dtype, (B, T, Hq, d)), _ptr(ws, "ws"),
                                   ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_tree_attention")
    return out


def medusa_posterior_workspace(B, T, V):
    return int(lib.medusa_posterior_workspace(B, T, V))


def medusa_evaluate_posterior(logits, tree_candidates, retrieve, num_paths, temperature, eps, delta,
                              out=None, ws=None):
    B, T, V = logits.shape
    p_max, D = retrieve.shape
    dev = logits.device
    o = out or {}
    best = o.get("best_path")
    acc = o.get("accept_len")
    nxt = o.get("next_token")
    if best is None:
        best = torch.empty(B, dtype=torch.int32, device=dev)
    if acc is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
    if nxt is None:
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
    need = medusa_posterior_workspace(B, T, V)
    if ws is None:
        ws = workspace("posterior", dev, need)
    rc = lib.medusa_evaluate_posterior(B, T, V, p_max, D, _ptr(logits, "logits", torch.float32),
                                       _ptr(tree_candidates, "tree_candidates", torch.int32, (B, T)),
                                       _ptr(retrieve, "retrieve", torch.int32),
                                       _ptr(num_paths, "num_paths", torch.int32),
                                       float(temperature), float(eps), float(delta),
                                       _ptr(best, "best_path", torch.int32, (B,)),
                                       _ptr(acc, "accept_len", torch.int32, (B,)),
                                       _ptr(nxt, "next_token", torch.int32, (B,)), _ptr(ws, "ws"),
                                       ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_evaluate_posterior")
    return dict(best_path=best, accept_len=acc, next_token=nxt)


def medusa_posterior_nucleus_workspace(B, T):
    return int(lib.medusa_posterior_nucleus_workspace(B, T))


def medusa_evaluate_posterior_nucleus(logits, tree_candidates, retrieve, num_paths, temperature, top_p, uniforms,
                                      out=None, ws=None, keep_samples=False):
    """Nucleus (top-p) acceptance: logits float32 [B][T][V], uniforms
    float32 [B][T] (one random number per node)."""
    B, T, V = logits.shape
    p_max, D = retrieve.shape
    dev = logits.device
    o = out or {}
    res = {}
    for name in ("best_path", "accept_len", "next_token"):
        t = o.get(name)
        res[name] = t if t is not None else torch.empty(B, dtype=torch.int32, device=dev)
    samples = o.get("samples")
    if samples is None and keep_samples:
        samples = torch.empty((B, T), dtype=torch.int32, device=dev)
    need = medusa_posterior_nucleus_workspace(B, T)
    if ws is None:
        ws = workspace("posterior_nucleus", dev, need)
    rc = lib.medusa_evaluate_posterior_nucleus(
        B, T, V, p_max, D, _ptr(logits, "logits", torch.float32),
        _ptr(tree_candidates, "tree_candidates", torch.int32, (B, T)), _ptr(retrieve, "retrieve", torch.int32),
        _ptr(num_paths, "num_paths", torch.int32), float(temperature), float(top_p),
        _ptr(uniforms, "uniforms", torch.float32, (B, T)), _ptr(res["best_path"], "best_path", torch.int32, (B,)),
        _ptr(res["accept_len"], "accept_len", torch.int32, (B,)),
        _ptr(res["next_token"], "next_token", torch.int32, (B,)),
        _ptr(samples, "samples", torch.int32, (B, T)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(dev))
    _check(rc, "medusa_evaluate_posterior_nucleus")
    res["samples"] = samples
    return res


def medusa_commit_kv(k_cache, v_cache, prefix_len, retrieve, best_path, accept_len, new_prefix_len=None):
    """k_cache, v_cache [n_layers][B][H][max_slots][d], updated in place."""
    dt = _dtype_code(k_cache)
    nl, B, H, S, d = k_cache.shape
    p_max, D = retrieve.shape
    dev = k_cache.device
    if new_prefix_len is None:
        new_prefix_len = torch.empty(B, dtype=torch.int32, device=dev)
    rc = lib.medusa_commit_kv(dt, B, nl, H, d, S, _ptr(k_cache, "k_cache"),
                              _ptr(v_cache, "v_cache", k_cache.dtype, tuple(k_cache.shape)),
                              _ptr(prefix_len, "prefix_len", torch.int32, (B,)),
                              _ptr(retrieve, "retrieve", torch.int32), p_max, D,
                              _ptr(best_path, "best_path", torch.int32, (B,)),
                              _ptr(accept_len, "accept_len", torch.int32, (B,)),
                              _ptr(new_prefix_len, "new_prefix_len", torch.int32, (B,)), _stream(dev))
    _check(rc, "medusa_commit_kv")
    return new_prefix_len


def medusa_base_lm_head_pack(w_base):
    """bf16 [V][H] row-major base lm_head -> its packed layout (uint8 tensor)."""
    V, H = w_base.shape
    nbytes = int(lib.medusa_base_lm_head_packed_bytes(H, V))
    if nbytes == 0:
        raise MedusaError(_ERR_SHAPE, "medusa_base_lm_head_pack", "unsupported shape V=%d H=%d" % (V, H))
    packed = torch.empty(nbytes, dtype=torch.uint8, device=w_base.device)
    rc = lib.medusa_base_lm_head_pack(_dtype_code(w_base), H, V, _ptr(w_base, "w_base"), _ptr(packed, "w_packed"),
                                      _stream(w_base.device))
    _check(rc, "medusa_base_lm_head_pack")
    return packed


def medusa_linear_workspace(M, H, V):
    return int(lib.medusa_linear_workspace(M, H, V))


def medusa_linear(x, w_packed, V, out=None, ws=None):
    """x bf16 [..][H] -> float32 [..][V] on packed weights (medusa_base_lm_head_pack),
    the reduction split into slices when the output is narrow."""
    shape = x.shape
    H = shape[-1]
    M = 1
    for s_ in shape[:-1]:
        M *= s_
    need = int(lib.medusa_base_lm_head_packed_bytes(H, V))
    if w_packed.dtype != torch.uint8 or w_packed.numel() != need:
        raise MedusaError(_ERR_SHAPE, "medusa_linear", "packed weights: expected %d uint8 bytes for H=%d V=%d"
                          % (need, H, V))
    dev = x.device
    if out is None:
        out = torch.empty(tuple(shape[:-1]) + (V,), dtype=torch.float32, device=dev)
    nb = medusa_linear_workspace(M, H, V)
    if ws is None:
        ws = workspace("linear", dev, nb)
    rc = lib.medusa_linear(MEDUSA_BF16, M, H, V, _ptr(x, "x", torch.bfloat16), _ptr(w_packed, "w_packed"),
                           _ptr(out, "y", torch.float32), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                           _stream(dev))
    _check(rc, "medusa_linear")
    return out


def medusa_base_lm_head(hidden, w_base, logits=None, V=None):
    """hidden bf16 [M][H] (or [B][T][H]) -> logits float32 [M][V] (or [B][T][V]).

    w_base: bf16 [V][H] row-major, or the uint8 tensor from
    medusa_base_lm_head_pack (then V must be given)."""
    shape = hidden.shape
    H = shape[-1]
    M = 1
    for x in shape[:-1]:
        M *= x
    packed = w_base.dtype == torch.uint8
    if packed:
        if V is None:
            raise ValueError("V is required with packed weights")
        if w_base.numel() != int(lib.medusa_base_lm_head_packed_bytes(H, V)):
            raise ValueError("packed weights have %d bytes, expected %d for H=%d V=%d"
                             % (w_base.numel(), lib.medusa_base_lm_head_packed_bytes(H, V), H, V))
        wptr = _ptr(w_base, "w_base")
    else:
        V = w_base.shape[0]
        wptr = _ptr(w_base, "w_base", hidden.dtype, (V, H))
    dev = hidden.device
    if logits is None:
        logits = torch.empty(tuple(shape[:-1]) + (V,), dtype=torch.float32, device=dev)
    rc = lib.medusa_base_lm_head(_dtype_code(hidden), M, H, V, _ptr(hidden, "hidden"), wptr, 1 if packed else 0,
                                 _ptr(logits, "logits", torch.float32, tuple(shape[:-1]) + (V,)), _stream(dev))
    _check(rc, "medusa_base_lm_head")
    return logits


def medusa_base_posterior_workspace(B, T, H, V):
    return int(lib.medusa_base_posterior_workspace(B, T, H, V))


def medusa_base_posterior(hidden, w_base, tree_candidates, retrieve, num_paths, temperature, eps, delta,
                          V=None, out=None, ws=None):
    """The acceptance test on the base logits of every tree node, fused:
    hidden bf16 [B][T][H]; w_base bf16 [V][H] or packed (uint8, V given)."""
    B, T, H = hidden.shape
    packed = w_base.dtype == torch.uint8
    if packed:
        if V is None:
            raise ValueError("V is required with packed weights")
        wptr = _ptr(w_base, "w_base")
    else:
        V = w_base.shape[0]
        wptr = _ptr(w_base, "w_base", hidden.dtype, (V, H))
    p_max, D = retrieve.shape
    dev = hidden.device
    o = out or {}
    best = o.get("best_path")
    acc = o.get("accept_len")
    nxt = o.get("next_token")
    if best is None:
        best = torch.empty(B, dtype=torch.int32, device=dev)
    if acc is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
    if nxt is None:
        nxt = torch.empty(B, dtype=torch.int32, device=dev)
    need = medusa_base_posterior_workspace(B, T, H, V)
    if need == 0:
        raise MedusaError(_ERR_SHAPE, "medusa_base_posterior", "unsupported shape B=%d T=%d H=%d V=%d" % (B, T, H, V))
    if ws is None:
        ws = workspace("base_posterior", dev, need)
    rc = lib.medusa_base_posterior(B, T, H, V, p_max, D, _ptr(hidden, "hidden"), wptr, 1 if packed else 0,
                                   _ptr(tree_candidates, "tree_candidates", torch.int32, (B, T)),
                                   _ptr(retrieve, "retrieve", torch.int32), _ptr(num_paths, "num_paths", torch.int32),
                                   float(temperature), float(eps), float(delta),
                                   _ptr(best, "best_path", torch.int32, (B,)), _ptr(acc, "accept_len", torch.int32, (B,)),
                                   _ptr(nxt, "next_token", torch.int32, (B,)), _ptr(ws, "ws"),
                                   ws.numel() * ws.element_size(), _stream(dev))
    _check(rc, "medusa_base_posterior")
    return dict(best_path=best, accept_len=acc, next_token=nxt)


def medusa_embed(tokens, embed, x=None):
    """tokens int32 [M] (or [B][T]) -> x float32 [M][H] (or [B][T][H])."""
    V, H = embed.shape
    M = tokens.numel()
    if x is None:
        x = torch.empty(tuple(tokens.shape) + (H,), dtype=torch.float32, device=tokens.device)
    rc = lib.medusa_embed(M, H, V, _ptr(tokens, "tokens", torch.int32), _ptr(embed, "embed", torch.bfloat16),
                          _ptr(x, "x", torch.float32), _stream(tokens.device))
    _check(rc, "medusa_embed")
    return x


def medusa_add_rmsnorm(x, gain, eps, y=None, out=None):
    """x float32 [..][H] (updated in place: x += y), out = bf16 rmsnorm(x) * gain."""
    H = x.shape[-1]
    M = x.numel() // H
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    rc = lib.medusa_add_rmsnorm(M, H, _ptr(x, "x", torch.float32), _ptr(y, "y", torch.float32, tuple(x.shape)),
                                _ptr(gain, "gain", torch.bfloat16, (H,)), float(eps),
                                _ptr(out, "out", torch.bfloat16, tuple(x.shape)), _stream(x.device))
    _check(rc, "medusa_add_rmsnorm")
    return out


def medusa_rope_qkv(qkv, positions, prefix_len, theta, k_cache, v_cache, q=None):
    """qkv float32 [B][T][3][heads][d]; k_cache, v_cache bf16 [B][heads][S][d]
    (one layer): returns q bf16 [B][T][heads][d]; k, v written to slots
    prefix_len[b] + t."""
    B, T, three, heads, d = qkv.shape
    S = k_cache.shape[2]
    if q is None:
        q = torch.empty((B, T, heads, d), dtype=torch.bfloat16, device=qkv.device)
    rc = lib.medusa_rope_qkv(B, T, heads, d, S, _ptr(qkv, "qkv", torch.float32),
                             _ptr(positions, "positions", torch.int32, (B, T)),
                             _ptr(prefix_len, "prefix_len", torch.int32, (B,)), float(theta),
                             _ptr(q, "q", torch.bfloat16, (B, T, heads, d)),
                             _ptr(k_cache, "k_cache", torch.bfloat16, (B, heads, S, d)),
                             _ptr(v_cache, "v_cache", torch.bfloat16, (B, heads, S, d)), _stream(qkv.device))
    _check(rc, "medusa_rope_qkv")
    return q


def medusa_silu_mul(gate_up, out=None):
    """gate_up float32 [..][2I] -> bf16 [..][I] = silu(gate) * up."""
    I2 = gate_up.shape[-1]
    M = gate_up.numel() // I2
    if out is None:
        out = torch.empty(tuple(gate_up.shape[:-1]) + (I2 // 2,), dtype=torch.bfloat16, device=gate_up.device)
    rc = lib.medusa_silu_mul(M, I2 // 2, _ptr(gate_up, "gate_up", torch.float32), _ptr(out, "out", torch.bfloat16),
                             _stream(gate_up.device))
    _check(rc, "medusa_silu_mul")
    return out
