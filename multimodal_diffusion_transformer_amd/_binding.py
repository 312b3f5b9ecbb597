"""ctypes binding of libmotattn (include/motattn.h).

Argument marshalling only: every function passes torch tensors' device
pointers, element strides and the current HIP stream to the C entry point of
the same name and raises ``MotError`` on a non-OK status.  No computation
happens here, and there is no fallback: if the library is missing, importing
this module fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmotattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libmotattn.so is not built; run `python multimodal_diffusion_transformer_amd/build.py` "
        "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

MOT_OK, MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED, MOT_ERR_HIP = 0, 1, 2, 3
MOT_BF16, MOT_FP32 = 0, 1
MOT_AR_CAUSAL_DM_FULL, MOT_CHUNK_CAUSAL_KV = 0, 1
MOT_EPI_NONE, MOT_EPI_GELU, MOT_EPI_ADD = 0, 1, 2

EXPORTED = [
    "mot_abi_version", "mot_status_string", "mot_build_layout", "mot_qkv_project",
    "mrope_apply", "mot_attention_fwd", "flow_euler_step", "mot_mask_materialize",
    "mot_tile_classes_host", "mot_sigma_schedule", "flow_cfg_euler_step", "mot_region_linear",
    "mot_layernorm_region", "mot_attention_merge",
]


class MotError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (status %d)" % (fn, mot_status_string(status), status))
        self.status = status


class mot_segment(ctypes.Structure):
    _fields_ = [("region", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("n_tokens", ctypes.c_int64), ("n_frames", ctypes.c_int64),
                ("n_views", ctypes.c_int64), ("grid_h", ctypes.c_int64),
                ("grid_w", ctypes.c_int64), ("rate", ctypes.c_double),
                ("frame0", ctypes.c_int64), ("step0", ctypes.c_int64)]


class mot_attn_args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("dt", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("mask", ctypes.c_int32),
                ("nq", ctypes.c_int64), ("nk", ctypes.c_int64), ("q0", ctypes.c_int64),
                ("q_ts", ctypes.c_int64), ("q_hs", ctypes.c_int64),
                ("k_ts", ctypes.c_int64), ("k_hs", ctypes.c_int64),
                ("v_ts", ctypes.c_int64), ("v_hs", ctypes.c_int64),
                ("o_ts", ctypes.c_int64), ("o_hs", ctypes.c_int64),
                ("n_ar", ctypes.c_int64), ("n_prefix", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64),
                ("q_pos", ctypes.c_void_p), ("k_pos", ctypes.c_void_p),
                ("sec_t", ctypes.c_int32), ("sec_h", ctypes.c_int32), ("sec_w", ctypes.c_int32),
                ("theta", ctypes.c_float), ("scale", ctypes.c_float),
                ("n_kv_heads", ctypes.c_int32), ("n_batch", ctypes.c_int32),
                ("q_bs", ctypes.c_int64), ("k_bs", ctypes.c_int64), ("v_bs", ctypes.c_int64),
                ("o_bs", ctypes.c_int64)]


_i64, _i32, _vp, _f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
_lib.mot_abi_version.restype = ctypes.c_int
_lib.mot_status_string.restype = ctypes.c_char_p
_lib.mot_status_string.argtypes = [ctypes.c_int32]
_lib.mot_build_layout.restype = ctypes.c_int
_lib.mot_build_layout.argtypes = [ctypes.POINTER(mot_segment), _i32, _i64, ctypes.POINTER(_i64),
                                  ctypes.POINTER(_i64), _vp, _vp]
_lib.mot_qkv_project.restype = ctypes.c_int
_lib.mot_qkv_project.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                 ctypes.c_int, _vp]
_lib.mot_region_linear.restype = ctypes.c_int
_lib.mot_region_linear.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, _vp, _vp]
_lib.mot_layernorm_region.restype = ctypes.c_int
_lib.mot_layernorm_region.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _f32,
                                      ctypes.c_int, ctypes.c_int, _vp]
_lib.mot_attention_merge.restype = ctypes.c_int
_lib.mot_attention_merge.argtypes = [_vp, _vp, _i32, _i64, _i64, _i32, _i32, _i64, _i64, _vp, _i64, _i64,
                                     _vp, ctypes.c_int, _vp]
_lib.mrope_apply.restype = ctypes.c_int
_lib.mrope_apply.argtypes = [_vp, ctypes.c_int, _i64, _i32, _i32, _i64, _i64, _vp, _i32, _i32,
                             _i32, _f32, _vp]
_lib.mot_attention_fwd.restype = ctypes.c_int
_lib.mot_attention_fwd.argtypes = [ctypes.POINTER(mot_attn_args), _vp]
_lib.flow_euler_step.restype = ctypes.c_int
_lib.flow_euler_step.argtypes = [_vp, _vp, ctypes.c_int, _i64, _f32, _f32, _vp, _vp]
_lib.flow_cfg_euler_step.restype = ctypes.c_int
_lib.flow_cfg_euler_step.argtypes = [_vp, _vp, _vp, ctypes.c_int, _i64, _f32, _f32, _f32, _vp, _vp]
_lib.mot_mask_materialize.restype = ctypes.c_int
_lib.mot_mask_materialize.argtypes = [ctypes.POINTER(mot_attn_args), _vp, _i32, _i32, _vp, _vp]
_lib.mot_tile_classes_host.restype = ctypes.c_int
_lib.mot_tile_classes_host.argtypes = [ctypes.POINTER(mot_attn_args), _i32, _i32, _vp]
_lib.mot_sigma_schedule.restype = ctypes.c_int
_lib.mot_sigma_schedule.argtypes = [_i32, ctypes.c_double, _vp]


def _check(fn, st):
    if st != MOT_OK:
        raise MotError(fn, st)


def mot_abi_version() -> int:
    return int(_lib.mot_abi_version())


def mot_status_string(status: int) -> str:
    return _lib.mot_status_string(int(status)).decode()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MOT_BF16
    if t.dtype == torch.float32:
        return MOT_FP32
    raise TypeError("motattn takes bf16 or fp32 tensors, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("motattn device calls take GPU tensors")


# ---------------------------------------------------------------------------
def mot_build_layout(segments):
    """segments: objects with the mot_segment fields -> (pos [N,3] float32,
    region [N] uint8, n_ar)."""
    arr = (mot_segment * len(segments))()
    for a, s in enumerate(segments):
        arr[a] = mot_segment(int(s.region), int(s.kind), int(s.n_tokens), int(s.n_frames),
                             int(s.n_views), int(s.grid_h), int(s.grid_w), float(s.rate),
                             int(s.frame0), int(s.step0))
    n, n_ar = _i64(0), _i64(0)
    st = _lib.mot_build_layout(arr, len(segments), 0, ctypes.byref(n), ctypes.byref(n_ar),
                               None, None)
    if n.value == 0:  # the segments themselves were rejected
        _check("mot_build_layout", st if st != MOT_OK else MOT_ERR_INVALID_ARG)
    cap = int(n.value)
    pos = np.zeros((cap, 3), dtype=np.float32)
    reg = np.zeros((cap,), dtype=np.uint8)
    st = _lib.mot_build_layout(arr, len(segments), cap, ctypes.byref(n), ctypes.byref(n_ar),
                               pos.ctypes.data_as(_vp), reg.ctypes.data_as(_vp))
    _check("mot_build_layout", st)
    return pos[: n.value], reg[: n.value], int(n_ar.value)


def mot_qkv_project(x, w_ar, w_dm, y, n_ar, stream=None):
    """y[r] = x[r] @ (r < n_ar ? w_ar : w_dm); contiguous row-major tensors.
    A room with no rows may pass None for its weights."""
    _need_cuda(x, w_ar, w_dm, y)
    for t in (x, w_ar, w_dm, y):
        if t is not None and not t.is_contiguous():
            raise ValueError("mot_qkv_project takes contiguous tensors")
    n_rows, d_in = x.shape
    d_out = y.shape[1]
    st = _lib.mot_qkv_project(_ptr(x), _ptr(w_ar), _ptr(w_dm), _ptr(y), n_rows, int(n_ar),
                              d_in, d_out, _dtype_code(x), _dtype_code(y), _stream(stream))
    _check("mot_qkv_project", st)


def mot_region_linear(x, w_ar, w_dm, y, n_ar, epilogue=MOT_EPI_NONE, residual=None, stream=None):
    """mot_qkv_project with an epilogue: GELU, or adding `residual` (which
    may be y itself); contiguous row-major tensors."""
    _need_cuda(x, w_ar, w_dm, y, residual)
    for t in (x, w_ar, w_dm, y, residual):
        if t is not None and not t.is_contiguous():
            raise ValueError("mot_region_linear takes contiguous tensors")
    if residual is not None and (residual.shape != y.shape or residual.dtype != y.dtype):
        raise ValueError("mot_region_linear: the residual has the output's shape and type")
    n_rows, d_in = x.shape
    st = _lib.mot_region_linear(_ptr(x), _ptr(w_ar), _ptr(w_dm), _ptr(y), n_rows, int(n_ar), d_in,
                                y.shape[1], _dtype_code(x), _dtype_code(y), int(epilogue),
                                _ptr(residual), _stream(stream))
    _check("mot_region_linear", st)


def mot_layernorm_region(x, y, n_ar, ln_ar, ln_dm, eps=1e-6, stream=None):
    """Region-split LayerNorm of contiguous [N, hidden] rows; ln_ar / ln_dm
    are (gamma, beta) fp32 device tensors (None for a room with no rows)."""
    ln_ar = ln_ar if ln_ar is not None else (None, None)
    ln_dm = ln_dm if ln_dm is not None else (None, None)
    _need_cuda(x, y, *ln_ar, *ln_dm)
    if not (x.is_contiguous() and y.is_contiguous()) or x.shape != y.shape:
        raise ValueError("mot_layernorm_region takes contiguous [N, hidden] x and y of one shape")
    st = _lib.mot_layernorm_region(_ptr(x), _ptr(y), x.shape[0], int(n_ar), x.shape[1], _ptr(ln_ar[0]),
                                   _ptr(ln_ar[1]), _ptr(ln_dm[0]), _ptr(ln_dm[1]), float(eps),
                                   _dtype_code(x), _dtype_code(y), _stream(stream))
    _check("mot_layernorm_region", st)


def mrope_apply(x, pos, sections, theta=10000.0, stream=None):
    """In-place mRoPE on a [N, H, D] view (last dim contiguous)."""
    _need_cuda(x, pos)
    n, h, d = x.shape
    if x.stride(2) != 1:
        raise ValueError("last dim must be contiguous")
    st = _lib.mrope_apply(_ptr(x), _dtype_code(x), n, h, d, x.stride(0), x.stride(1), _ptr(pos),
                          int(sections[0]), int(sections[1]), int(sections[2]), float(theta),
                          _stream(stream))
    _check("mrope_apply", st)


def attn_args(q, k, v, o, *, mask, q0=0, n_ar=0, n_prefix=0, chunk_len=0, lse=None,
              q_pos=None, k_pos=None, sections=(0, 0, 0), theta=10000.0, scale=0.0):
    """q/o [N, H, D] and k/v [N, H_kv, D] views, or with a leading batch
    dimension [B, N, H(_kv), D] whose stride is the batch stride (0 shares
    a tensor across the batch; overlapping views are fine for inputs)."""
    batched = q.dim() == 4
    if {t.dim() for t in (q, k, v, o)} != {4 if batched else 3}:
        raise ValueError("q, k, v and o must all be 3-D, or all 4-D with a batch dimension")
    if batched:
        nb = q.shape[0]
        if not (k.shape[0] == v.shape[0] == o.shape[0] == nb):
            raise ValueError("batch sizes differ")
        bs = [t.stride(0) for t in (q, k, v, o)]
        q, k, v, o = (t[0] for t in (q, k, v, o))
    nq, h, d = q.shape
    nk, hk = k.shape[0], k.shape[1]
    for t in (q, k, v, o):
        if t.stride(2) != 1:
            raise ValueError("last dim must be contiguous")
    a = mot_attn_args()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    a.dt = _dtype_code(q)
    a.n_heads, a.head_dim, a.mask = h, d, int(mask)
    a.nq, a.nk, a.q0 = nq, nk, int(q0)
    a.q_ts, a.q_hs = q.stride(0), q.stride(1)
    a.k_ts, a.k_hs = k.stride(0), k.stride(1)
    a.v_ts, a.v_hs = v.stride(0), v.stride(1)
    a.o_ts, a.o_hs = o.stride(0), o.stride(1)
    a.n_ar, a.n_prefix, a.chunk_len = int(n_ar), int(n_prefix), int(chunk_len)
    a.q_pos = None if q_pos is None else q_pos.data_ptr()
    a.k_pos = None if k_pos is None else k_pos.data_ptr()
    a.sec_t, a.sec_h, a.sec_w = (int(s) for s in sections)
    a.theta, a.scale = float(theta), float(scale)
    a.n_kv_heads = hk
    if batched:
        a.n_batch = nb
        a.q_bs, a.k_bs, a.v_bs, a.o_bs = bs
    return a


def mot_attention_fwd(q, k, v, o, *, mask, stream=None, **kw):
    """Masked attention; q/k/v/o are [N, H, D] views, see motattn.h."""
    _need_cuda(q, k, v, o, kw.get("lse"), kw.get("q_pos"), kw.get("k_pos"))
    a = attn_args(q, k, v, o, mask=mask, **kw)
    st = _lib.mot_attention_fwd(ctypes.byref(a), _stream(stream))
    _check("mot_attention_fwd", st)


def mot_attention_merge(o_parts, lse_parts, o, lse=None, stream=None):
    """Merge per-key-range attention outputs o_parts [B, nq, H, D] (batch
    stride = part stride) with their LSE [B, H, nq] into o [nq, H, D]."""
    _need_cuda(o_parts, lse_parts, o, lse)
    nb, nq, h, d = o_parts.shape
    if o_parts.stride(3) != 1 or o.stride(2) != 1 or not lse_parts.is_contiguous():
        raise ValueError("mot_attention_merge: last dims contiguous, LSE parts contiguous")
    if tuple(lse_parts.shape) != (nb, h, nq) or tuple(o.shape) != (nq, h, d):
        raise ValueError("mot_attention_merge: shapes differ")
    st = _lib.mot_attention_merge(_ptr(o_parts), _ptr(lse_parts), nb, o_parts.stride(0), nq, h, d,
                                  o_parts.stride(1), o_parts.stride(2), _ptr(o), o.stride(0), o.stride(1),
                                  _ptr(lse), _dtype_code(o), _stream(stream))
    _check("mot_attention_merge", st)


def mot_attention_fwd_args(a, stream=None):
    """Launch with a prepared mot_attn_args (no per-call marshalling)."""
    _check("mot_attention_fwd", _lib.mot_attention_fwd(ctypes.byref(a), _stream(stream)))


def flow_euler_step(x, v, sigma, sigma_next, x_bf16=None, stream=None):
    """x += (sigma_next - sigma) * v over contiguous tensors (x fp32)."""
    _need_cuda(x, v, x_bf16)
    import torch
    if x.dtype != torch.float32 or not x.is_contiguous() or not v.is_contiguous():
        raise ValueError("flow_euler_step: x contiguous fp32, v contiguous")
    if x.numel() != v.numel():
        raise ValueError("flow_euler_step: x and v sizes differ")
    if x_bf16 is not None and (x_bf16.numel() != x.numel() or not x_bf16.is_contiguous()
                               or x_bf16.dtype != torch.bfloat16):
        raise ValueError("flow_euler_step: x_bf16 must be a contiguous bf16 mirror of x")
    st = _lib.flow_euler_step(_ptr(x), _ptr(v), _dtype_code(v), x.numel(), float(sigma),
                              float(sigma_next), _ptr(x_bf16), _stream(stream))
    _check("flow_euler_step", st)


def flow_cfg_euler_step(x, v_cond, v_base, guidance, sigma, sigma_next, x_bf16=None, stream=None):
    """x += (sigma_next - sigma) * (v_base + guidance * (v_cond - v_base))
    over contiguous tensors (x fp32; v_cond and v_base of one dtype)."""
    _need_cuda(x, v_cond, v_base, x_bf16)
    import torch
    if x.dtype != torch.float32 or not all(t.is_contiguous() for t in (x, v_cond, v_base)):
        raise ValueError("flow_cfg_euler_step: x contiguous fp32, velocities contiguous")
    if not (x.numel() == v_cond.numel() == v_base.numel()) or v_cond.dtype != v_base.dtype:
        raise ValueError("flow_cfg_euler_step: sizes or velocity dtypes differ")
    if x_bf16 is not None and (x_bf16.numel() != x.numel() or not x_bf16.is_contiguous()
                               or x_bf16.dtype != torch.bfloat16):
        raise ValueError("flow_cfg_euler_step: x_bf16 must be a contiguous bf16 mirror of x")
    st = _lib.flow_cfg_euler_step(_ptr(x), _ptr(v_cond), _ptr(v_base), _dtype_code(v_cond),
                                  x.numel(), float(guidance), float(sigma), float(sigma_next),
                                  _ptr(x_bf16), _stream(stream))
    _check("flow_cfg_euler_step", st)


def mask_args(nq, nk, q0, mask, n_ar=0, n_prefix=0, chunk_len=0):
    a = mot_attn_args()
    a.mask, a.nq, a.nk, a.q0 = int(mask), int(nq), int(nk), int(q0)
    a.n_ar, a.n_prefix, a.chunk_len = int(n_ar), int(n_prefix), int(chunk_len)
    return a


def mot_mask_materialize(a, mask_dev=None, bm=128, bn=64, tiles_dev=None, stream=None):
    st = _lib.mot_mask_materialize(ctypes.byref(a), _ptr(mask_dev), int(bm), int(bn),
                                   _ptr(tiles_dev), _stream(stream))
    _check("mot_mask_materialize", st)


def mot_tile_classes_host(a, bm, bn):
    ntq = -(-a.nq // bm)
    ntk = -(-a.nk // bn)
    out = np.zeros((ntq, ntk), dtype=np.uint8)
    st = _lib.mot_tile_classes_host(ctypes.byref(a), int(bm), int(bn), out.ctypes.data_as(_vp))
    _check("mot_tile_classes_host", st)
    return out


def mot_sigma_schedule(n_steps, shift):
    """Noise levels sigma_0 = 1 .. sigma_n = 0 with the flow shift, as a
    float32 array of n_steps + 1 (host only)."""
    n = int(n_steps)
    out = np.zeros((max(n, 0) + 1,), dtype=np.float32)
    st = _lib.mot_sigma_schedule(n, float(shift), out.ctypes.data_as(_vp))
    _check("mot_sigma_schedule", st)
    return out


def raw_call(name, *args):
    """Call a C entry point directly and return its status (tests of the
    argument checks)."""
    return getattr(_lib, name)(*args)
