"""ctypes binding over librcgqa.so (the C ABI in include/rcgqa.h).

Argument marshalling only: shapes and device pointers are read off torch
tensors and handed to the library (the attention scale is always the
caller's: no default is computed here), which runs every step in its own HIP
kernels on the caller's current stream.  There is no fallback: if the library
is missing or a tensor is not a CUDA (HIP) tensor, the call raises.
"""
import ctypes
import os

LIB_NAME = "librcgqa.so"
_HERE = os.path.dirname(os.path.abspath(__file__))

OK, EINVAL, EUNSUPPORTED, EHIP, ENOSPACE = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1

_lib = None


class RcgqaError(RuntimeError):
    """A non-OK status from the library (EHIP or unexpected)."""


def lib_path():
    return os.path.join(_HERE, LIB_NAME)


def lib():
    """Load librcgqa.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RcgqaError(f"{path} is not built; run `python -m rope_causal_gqa_amd.build` "
                         "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.rope_apply.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, i32, vp]
    L.rope_apply.restype = i32
    L.rope_apply_interleaved.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, i32, vp]
    L.rope_apply_interleaved.restype = i32
    L.attn_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_prefill.restype = i32
    L.attn_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.attn_prefill_workspace_bytes.restype = sz
    L.attn_prefill_ws.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    L.attn_prefill_ws.restype = i32
    L.attn_prefill_masked.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_prefill_masked.restype = i32
    L.attn_prefill_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_prefill_cache.restype = i32
    L.attn_prefill_cache_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.attn_prefill_cache_workspace_bytes.restype = sz
    L.attn_prefill_cache_ws.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz,
                                        vp]
    L.attn_prefill_cache_ws.restype = i32
    L.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    L.attn_decode.restype = i32
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    L.attn_decode_noalloc.restype = i32
    L.kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.kv_append.restype = i32
    L.rope_attn_prefill_workspace_bytes.argtypes = [i32, i32, i32]
    L.rope_attn_prefill_workspace_bytes.restype = sz
    L.rope_attn_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, vp, sz,
                                    vp]
    L.rope_attn_prefill.restype = i32
    L.rope_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.rope_attn_decode_workspace_bytes.restype = sz
    L.rope_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, f32, i32, vp,
                                   sz, vp]
    L.rope_attn_decode.restype = i32
    L.rope_ntk_theta.argtypes = [f32, i32, f32, ctypes.POINTER(ctypes.c_float)]
    L.rope_ntk_theta.restype = i32
    L.rope_dynamic_ntk_theta.argtypes = [f32, i32, f32, i32, i32, ctypes.POINTER(ctypes.c_float)]
    L.rope_dynamic_ntk_theta.restype = i32
    L.rcgqa_status_string.argtypes = [i32]
    L.rcgqa_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status, what):
    if status == OK:
        return
    msg = lib().rcgqa_status_string(status).decode()
    if status in (EINVAL, ENOSPACE):
        raise ValueError(f"{what}: {msg}")
    if status == EUNSUPPORTED:
        raise NotImplementedError(f"{what}: {msg}")
    raise RcgqaError(f"{what}: {msg}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name, dt=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if dt is not None and _dtype_code(t) != dt:
        raise ValueError(f"{name} has dtype {t.dtype}, expected the run dtype")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name, n):
    import torch
    if t.dtype != torch.int32 or t.numel() != n:
        raise ValueError(f"{name} must be int32 with {n} elements")
    return _dev(t, name)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rope(name, q, k, position_ids, theta, linear_factor):
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    pos = ctypes.c_void_p(0) if position_ids is None else _i32(position_ids, "position_ids", B * S)
    st = getattr(lib(), name)(_dev(q, "q", dt, 4), _dev(k, "k", dt, 4), pos, B, S, Hq, Hkv, D,
                              float(theta), float(linear_factor), dt, _stream(q))
    _check(st, name)
    return q, k


def rope_ntk_theta(theta, head_dim, alpha):
    """RoPE base for NTK-aware scaling by alpha (see rcgqa.h); pass it to rope_apply."""
    out = ctypes.c_float()
    _check(lib().rope_ntk_theta(float(theta), int(head_dim), float(alpha), ctypes.byref(out)), "rope_ntk_theta")
    return out.value


def rope_dynamic_ntk_theta(theta, head_dim, factor, seq_len, max_position):
    """RoPE base of the dynamic NTK form for a sequence of seq_len tokens (see rcgqa.h)."""
    out = ctypes.c_float()
    _check(lib().rope_dynamic_ntk_theta(float(theta), int(head_dim), float(factor), int(seq_len), int(max_position),
                                        ctypes.byref(out)), "rope_dynamic_ntk_theta")
    return out.value


def rope_apply(q, k, position_ids=None, theta=10000.0, linear_factor=1.0):
    """Rotate q [B,S,Hq,D] and k [B,S,Hkv,D] in place, pairs (x[i], x[i+D/2]) (see rcgqa.h)."""
    return _rope("rope_apply", q, k, position_ids, theta, linear_factor)


def rope_apply_interleaved(q, k, position_ids=None, theta=10000.0, linear_factor=1.0):
    """Rotate q and k in place with adjacent pairs (x[2i], x[2i+1]) (see rcgqa.h)."""
    return _rope("rope_apply_interleaved", q, k, position_ids, theta, linear_factor)


def attn_prefill(q, k, v, out=None, causal=True, *, scale):
    """out [B,S,Hq,D] = attention(q [B,S,Hq,D], k/v [B,S,Hkv,D]) (see rcgqa.h)."""
    import torch
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B, S, Hq, D]")
    st = lib().attn_prefill(_dev(q, "q", dt, 4), _dev(k, "k", dt, 4), _dev(v, "v", dt, 4),
                            _dev(out, "out", dt, 4), B, S, Hq, Hkv, D, int(bool(causal)),
                            float(scale), dt, _stream(q))
    _check(st, "attn_prefill")
    return out


def attn_prefill_workspace_bytes(B, S, Hq, head_dim, causal=True):
    return int(lib().attn_prefill_workspace_bytes(B, S, Hq, head_dim, int(bool(causal))))


def attn_prefill_ws(q, k, v, out=None, causal=True, *, scale, workspace=None):
    """attn_prefill with a caller-owned workspace that lets small causal
    problems split each query tile's keys over several workgroups (see rcgqa.h).
    ``workspace`` (uint8, at least attn_prefill_workspace_bytes) must be zeroed
    before its first use; every call leaves it ready for the next.  Without one
    a zeroed buffer is allocated for this call."""
    import torch
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B, S, Hq, D]")
    if workspace is None:
        need = attn_prefill_workspace_bytes(B, S, Hq, D, causal) if dt == BF16 else 0
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().attn_prefill_ws(_dev(q, "q", dt, 4), _dev(k, "k", dt, 4), _dev(v, "v", dt, 4),
                               _dev(out, "out", dt, 4), B, S, Hq, Hkv, D, int(bool(causal)), float(scale), dt,
                               _dev(workspace, "workspace"), wbytes, _stream(q))
    _check(st, "attn_prefill_ws")
    return out


def attn_prefill_masked(q, k, v, mask, out=None, causal=False, *, scale):
    """attn_prefill plus an additive mask [B, 1 or Hq, S, L >= S] of the run dtype (see rcgqa.h)."""
    import torch
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if mask.dim() != 4 or mask.shape[0] != B or mask.shape[1] not in (1, Hq) or mask.shape[2] != S \
            or mask.shape[3] < S:
        raise ValueError("mask must be [B, 1 or Hq, S, L] with L >= S")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B, S, Hq, D]")
    st = lib().attn_prefill_masked(_dev(q, "q", dt, 4), _dev(k, "k", dt, 4), _dev(v, "v", dt, 4),
                                   _dev(mask, "mask", dt, 4), _dev(out, "out", dt, 4), B, S, Hq, Hkv, D,
                                   int(mask.shape[1]), int(mask.shape[3]), int(bool(causal)), float(scale), dt,
                                   _stream(q))
    _check(st, "attn_prefill_masked")
    return out


def attn_prefill_cache(q, k_cache, v_cache, kv_lens, out=None, causal=True, *, scale, window=0):
    """out [B,Sq,Hq,D] = attention of the Sq newest tokens q [B,Sq,Hq,D] of each
    sequence over its kv_lens[b] cached rows (caches [B,Hkv,max_kv,D]); with
    ``window`` > 0 a token sees only its ``window`` most recent positions."""
    import torch
    dt = _dtype_code(q)
    B, Sq, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_kv, D) or tuple(v_cache.shape) != (B, Hkv, max_kv, D):
        raise ValueError("caches must be [B, Hkv, max_kv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, Sq, Hq, D):
        raise ValueError("out must be [B, Sq, Hq, D]")
    st = lib().attn_prefill_cache(_dev(q, "q", dt, 4), _dev(k_cache, "k_cache", dt, 4),
                                  _dev(v_cache, "v_cache", dt, 4), _i32(kv_lens, "kv_lens", B),
                                  _dev(out, "out", dt, 4), B, Sq, Hq, Hkv, D, max_kv, int(bool(causal)),
                                  int(window), float(scale), dt, _stream(q))
    _check(st, "attn_prefill_cache")
    return out


def attn_prefill_cache_workspace_bytes(B, Sq, Hq, head_dim, max_kv, causal=True, window=0):
    return int(lib().attn_prefill_cache_workspace_bytes(B, Sq, Hq, head_dim, max_kv, int(bool(causal)), int(window)))


def attn_prefill_cache_ws(q, k_cache, v_cache, kv_lens, out=None, causal=True, *, scale, window=0, workspace=None):
    """attn_prefill_cache with a caller-owned workspace (stream-K for causal
    chunks without a window; see rcgqa.h).  ``workspace`` (uint8, at least
    attn_prefill_cache_workspace_bytes) must be zeroed before its first use;
    every call leaves it ready for the next.  Without one a zeroed buffer is
    allocated for this call."""
    import torch
    dt = _dtype_code(q)
    B, Sq, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_kv, D) or tuple(v_cache.shape) != (B, Hkv, max_kv, D):
        raise ValueError("caches must be [B, Hkv, max_kv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, Sq, Hq, D):
        raise ValueError("out must be [B, Sq, Hq, D]")
    if workspace is None:
        need = attn_prefill_cache_workspace_bytes(B, Sq, Hq, D, max_kv, causal, window) if dt == BF16 else 0
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().attn_prefill_cache_ws(_dev(q, "q", dt, 4), _dev(k_cache, "k_cache", dt, 4),
                                     _dev(v_cache, "v_cache", dt, 4), _i32(kv_lens, "kv_lens", B),
                                     _dev(out, "out", dt, 4), B, Sq, Hq, Hkv, D, max_kv, int(bool(causal)),
                                     int(window), float(scale), dt, _dev(workspace, "workspace"), wbytes, _stream(q))
    _check(st, "attn_prefill_cache_ws")
    return out


def attn_decode_workspace_bytes(B, Hq, head_dim, max_kv):
    return int(lib().attn_decode_workspace_bytes(B, Hq, head_dim, max_kv))


def attn_decode(q, k_cache, v_cache, kv_lens, out=None, *, scale, workspace=None):
    """out [B,Hq,D] = decode attention of q [B,Hq,D] over caches [B,Hkv,max_kv,D]."""
    import torch
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_kv, D) or tuple(v_cache.shape) != (B, Hkv, max_kv, D):
        raise ValueError("caches must be [B, Hkv, max_kv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    need = attn_decode_workspace_bytes(B, Hq, D, max_kv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode(_dev(q, "q", dt, 3), _dev(k_cache, "k_cache", dt, 4),
                           _dev(v_cache, "v_cache", dt, 4), _i32(kv_lens, "kv_lens", B),
                           _dev(out, "out", dt, 3), B, Hq, Hkv, D, max_kv, float(scale), dt,
                           _dev(workspace, "workspace"), wbytes, _stream(q))
    _check(st, "attn_decode")
    return out


def attn_decode_noalloc(q, k_cache, v_cache, kv_lens, out, scale):
    """attn_decode with the split-K partial states in the library's fixed per-GPU
    scratch (no workspace, no allocation inside the call; see rcgqa.h)."""
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_kv, D) or tuple(v_cache.shape) != (B, Hkv, max_kv, D):
        raise ValueError("caches must be [B, Hkv, max_kv, D] matching q")
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    st = lib().attn_decode_noalloc(_dev(q, "q", dt, 3), _dev(k_cache, "k_cache", dt, 4),
                                   _dev(v_cache, "v_cache", dt, 4), _i32(kv_lens, "kv_lens", B),
                                   _dev(out, "out", dt, 3), B, Hq, Hkv, D, max_kv, float(scale), dt, _stream(q))
    _check(st, "attn_decode_noalloc")
    return out


def kv_append(k_cache, v_cache, k_new, v_new, slots):
    """Write k_new/v_new [B,Hkv,D] into row slots[b] of the caches [B,Hkv,max_kv,D]."""
    dt = _dtype_code(k_cache)
    B, Hkv, max_kv, D = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must match k_cache")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    st = lib().kv_append(_dev(k_cache, "k_cache", dt, 4), _dev(v_cache, "v_cache", dt, 4),
                         _dev(k_new, "k_new", dt, 3), _dev(v_new, "v_new", dt, 3),
                         _i32(slots, "slots", B), B, Hkv, D, max_kv, dt, _stream(k_cache))
    _check(st, "kv_append")
    return k_cache, v_cache


def _workspace(need, like, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    return workspace, workspace.numel() * workspace.element_size()


def rope_attn_prefill_workspace_bytes(B, S, head_dim):
    return int(lib().rope_attn_prefill_workspace_bytes(B, S, head_dim))


def rope_attn_prefill(q, k, v, position_ids=None, out=None, causal=True, *, scale, theta=10000.0,
                      linear_factor=1.0, workspace=None):
    """out [B,S,Hq,D] = attention(rope(q), rope(k), v); k is rotated in place,
    q is left as it is (see rcgqa.h)."""
    import torch
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B, S, Hq, D]")
    pos = ctypes.c_void_p(0) if position_ids is None else _i32(position_ids, "position_ids", B * S)
    workspace, wbytes = _workspace(rope_attn_prefill_workspace_bytes(B, S, D), q, workspace)
    st = lib().rope_attn_prefill(_dev(q, "q", dt, 4), _dev(k, "k", dt, 4), _dev(v, "v", dt, 4),
                                 _dev(out, "out", dt, 4), pos, B, S, Hq, Hkv, D, int(bool(causal)), float(scale),
                                 float(theta), float(linear_factor), dt, _dev(workspace, "workspace"), wbytes,
                                 _stream(q))
    _check(st, "rope_attn_prefill")
    return out


def rope_attn_decode_workspace_bytes(B, Hq, head_dim, max_kv):
    return int(lib().rope_attn_decode_workspace_bytes(B, Hq, head_dim, max_kv))


def rope_attn_decode(q, k_new, v_new, k_cache, v_cache, kv_lens, position_ids=None, out=None, *, scale,
                     theta=10000.0, linear_factor=1.0, workspace=None):
    """One decode step: rotate q [B,Hq,D] and k_new [B,Hkv,D], append k_new/v_new at row
    kv_lens[b]-1 of the caches [B,Hkv,max_kv,D], attend (see rcgqa.h)."""
    import torch
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_kv, D) or tuple(v_cache.shape) != (B, Hkv, max_kv, D):
        raise ValueError("caches must be [B, Hkv, max_kv, D] matching q")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    pos = ctypes.c_void_p(0) if position_ids is None else _i32(position_ids, "position_ids", B)
    workspace, wbytes = _workspace(rope_attn_decode_workspace_bytes(B, Hq, D, max_kv), q, workspace)
    st = lib().rope_attn_decode(_dev(q, "q", dt, 3), _dev(k_new, "k_new", dt, 3), _dev(v_new, "v_new", dt, 3),
                                _dev(k_cache, "k_cache", dt, 4), _dev(v_cache, "v_cache", dt, 4),
                                _i32(kv_lens, "kv_lens", B), pos, _dev(out, "out", dt, 3), B, Hq, Hkv, D, max_kv,
                                float(scale), float(theta), float(linear_factor), dt,
                                _dev(workspace, "workspace"), wbytes, _stream(q))
    _check(st, "rope_attn_decode")
    return out
