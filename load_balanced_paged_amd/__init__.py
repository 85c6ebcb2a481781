"""Python binding of liblbp (load-balanced paged decode attention, gfx950).

A thin ctypes layer over the C ABI in ``include/lbp.h``: the functions keep
the C names and only marshal arguments (torch tensors -> device pointers,
streams -> hipStream_t).  Every step of the computation runs in the HIP
kernels of ``liblbp.so``; there is no fallback.  If the library has not been
built, :func:`load` raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblbp.so")

LBP_OK = 0
LBP_ERR_INVALID_ARG = 1
LBP_ERR_UNSUPPORTED = 2
LBP_ERR_WORKSPACE_TOO_SMALL = 3
LBP_ERR_MISMATCH = 4
LBP_ERR_HIP = 5
LBP_ERR_SCRATCH_LIMIT = 6
NOALLOC_SCRATCH_BYTES = 32 << 20   # LBP_NOALLOC_SCRATCH_BYTES

LBP_KV_BF16 = 0
LBP_KV_FP8_E4M3 = 1

LBP_POLICY_DYNAMIC = 0
LBP_POLICY_STATIC_SPLITS = 1
LBP_POLICY_STATIC_CHUNK = 2

LBP_PLAN_MAGIC = 0x4C425031
HEAD_DIM = 128
PAGE_SIZE = 64

EXPORTED_SYMBOLS = (
    "lbp_status_string", "lbp_version", "lbp_query_workspace", "lbp_plan", "lbp_plan_static",
    "lbp_plan_layout", "lbp_attend", "lbp_attend_fused", "lbp_attend_partials",
    "lbp_attend_traced", "lbp_attend_fp8q", "lbp_prologue",
    "lbp_combine", "lbp_read_stream", "lbp_attend_noalloc", "lbp_taskmap_to_host",
)


class lbp_config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("min_tiles_per_bin", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("q_len", ctypes.c_int32),
    ]


class lbp_plan_info(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("policy", ctypes.c_int32),
        ("param", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_bins", ctypes.c_int32),
        ("max_desc", ctypes.c_int32),
        ("plan_bytes", ctypes.c_uint64),
        ("page_table_dev", ctypes.c_void_p),
        ("page_table_stride", ctypes.c_int64),
    ]


class lbp_prologue_args(ctypes.Structure):
    _fields_ = [
        ("qkv", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_table_stride", ctypes.c_int64),
        ("q_norm_weight", ctypes.c_void_p),
        ("k_norm_weight", ctypes.c_void_p),
        ("rope_cos_sin", ctypes.c_void_p),
        ("max_position", ctypes.c_int32),
        ("norm_eps", ctypes.c_float),
        ("q_fp8", ctypes.c_int32),
        ("q_out", ctypes.c_void_p),
        ("q_scale_out", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class lbp_plan_offsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("header", "bin_offset", "bin_first", "desc", "pair_first", "pair_count", "scratch",
                 "split_list", "arrive", "total")]


class LbpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_name(status)}")


_lib = None
_STATUS_NAMES = {0: "LBP_OK", 1: "LBP_ERR_INVALID_ARG", 2: "LBP_ERR_UNSUPPORTED",
                 3: "LBP_ERR_WORKSPACE_TOO_SMALL", 4: "LBP_ERR_MISMATCH", 5: "LBP_ERR_HIP",
                 6: "LBP_ERR_SCRATCH_LIMIT"}


def status_name(s: int) -> str:
    return _STATUS_NAMES.get(int(s), f"status {s}")


def load(path: str = LIB_PATH):
    """Load liblbp.so (once).  Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m load_balanced_paged_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(lbp_config)
    infop = ctypes.POINTER(lbp_plan_info)
    sig = {
        "lbp_status_string": (ctypes.c_char_p, [I32]),
        "lbp_version": (I32, []),
        "lbp_query_workspace": (I32, [cfgp, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "lbp_plan": (I32, [cfgp, P, I32, P, I64, P, SZ, infop, P]),
        "lbp_plan_static": (I32, [cfgp, I32, I32, P, I32, P, I64, P, SZ, infop, P]),
        "lbp_plan_layout": (I32, [infop, ctypes.POINTER(lbp_plan_offsets)]),
        "lbp_attend": (I32, [cfgp, infop, P, P, P, P, P, P, P, SZ, P, P]),
        "lbp_attend_fused": (I32, [cfgp, infop, P, P, P, P, P, P, P, SZ, P, P]),
        "lbp_attend_partials": (I32, [cfgp, infop, P, P, P, P, P, P, P, SZ, P, P]),
        "lbp_attend_traced": (I32, [cfgp, infop, P, P, P, P, P, P, P, SZ, P, P, P]),
        "lbp_attend_fp8q": (I32, [cfgp, infop, P, P, P, P, P, P, P, P, SZ, P, P]),
        "lbp_prologue": (I32, [cfgp, I32, ctypes.POINTER(lbp_prologue_args), P]),
        "lbp_combine": (I32, [cfgp, infop, P, P, SZ, P, P]),
        "lbp_read_stream": (I32, [P, SZ, P, I32, P]),
        "lbp_attend_noalloc": (I32, [cfgp, infop, P, P, P, P, P, P, P, P]),
        "lbp_taskmap_to_host": (I32, [infop, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t, what, dtype=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{what} is required")
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != LBP_OK:
        raise LbpError(status, what)


def make_config(num_q_heads, num_kv_heads, max_batch, max_pages_per_seq, kv_dtype="bf16",
                num_workgroups=0, min_tiles_per_bin=0, sm_scale=None, head_dim=HEAD_DIM,
                page_size=PAGE_SIZE, q_len=1) -> lbp_config:
    dt = {"bf16": LBP_KV_BF16, "fp8_e4m3": LBP_KV_FP8_E4M3}.get(kv_dtype, kv_dtype)
    return lbp_config(num_q_heads, num_kv_heads, head_dim, page_size, max_batch,
                      max_pages_per_seq, num_workgroups, min_tiles_per_bin, int(dt),
                      float(sm_scale if sm_scale is not None else head_dim ** -0.5), int(q_len))


# ---------------------------------------------------------------------------
# C entry points (same names)
# ---------------------------------------------------------------------------

def lbp_status_string(status: int) -> str:
    return load().lbp_status_string(int(status)).decode()


def lbp_version() -> int:
    return int(load().lbp_version())


def lbp_query_workspace(cfg: lbp_config, policy: int = LBP_POLICY_DYNAMIC, param: int = 0):
    """(plan_bytes, split_bytes) for cfg.max_batch."""
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().lbp_query_workspace(ctypes.byref(cfg), policy, param, ctypes.byref(pb),
                                      ctypes.byref(sb)), "lbp_query_workspace")
    return pb.value, sb.value


def lbp_plan(cfg, seq_lens, page_table, plan_ws, stream=None) -> lbp_plan_info:
    import torch
    info = lbp_plan_info()
    _check(load().lbp_plan(ctypes.byref(cfg), _ptr(seq_lens, "seq_lens", torch.int32),
                           int(seq_lens.numel()), _ptr(page_table, "page_table", torch.int32),
                           int(page_table.shape[1]), _ptr(plan_ws, "plan_ws"),
                           plan_ws.numel() * plan_ws.element_size(), ctypes.byref(info),
                           _stream(stream)), "lbp_plan")
    return info


def lbp_plan_static(cfg, policy, param, seq_lens, page_table, plan_ws, stream=None) -> lbp_plan_info:
    import torch
    info = lbp_plan_info()
    _check(load().lbp_plan_static(ctypes.byref(cfg), int(policy), int(param),
                                  _ptr(seq_lens, "seq_lens", torch.int32), int(seq_lens.numel()),
                                  _ptr(page_table, "page_table", torch.int32),
                                  int(page_table.shape[1]), _ptr(plan_ws, "plan_ws"),
                                  plan_ws.numel() * plan_ws.element_size(), ctypes.byref(info),
                                  _stream(stream)), "lbp_plan_static")
    return info


def lbp_plan_layout(info: lbp_plan_info) -> lbp_plan_offsets:
    off = lbp_plan_offsets()
    _check(load().lbp_plan_layout(ctypes.byref(info), ctypes.byref(off)), "lbp_plan_layout")
    return off


def _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale):
    import torch
    kv_t = torch.bfloat16 if cfg.kv_dtype == LBP_KV_BF16 else torch.uint8
    fp8 = cfg.kv_dtype == LBP_KV_FP8_E4M3
    return (_ptr(k_cache, "k_cache", kv_t), _ptr(v_cache, "v_cache", kv_t),
            _ptr(k_scale, "k_scale", torch.float32, optional=not fp8),
            _ptr(v_scale, "v_scale", torch.float32, optional=not fp8))


def _attend(fn, name, cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, split_ws, out,
            stream):
    import torch
    kp, vp, ksp, vsp = _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale)
    _check(fn(ctypes.byref(cfg), ctypes.byref(info), _ptr(plan_ws, "plan_ws"),
              _ptr(q, "q", torch.bfloat16), kp, vp, ksp, vsp, _ptr(split_ws, "split_ws"),
              split_ws.numel() * split_ws.element_size(), _ptr(out, "out", torch.bfloat16),
              _stream(stream)), name)


def lbp_attend(cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, split_ws, out,
               stream=None):
    _attend(load().lbp_attend, "lbp_attend", cfg, info, plan_ws, q, k_cache, v_cache, k_scale,
            v_scale, split_ws, out, stream)


def lbp_attend_fused(cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, split_ws, out,
                     stream=None):
    _attend(load().lbp_attend_fused, "lbp_attend_fused", cfg, info, plan_ws, q, k_cache, v_cache,
            k_scale, v_scale, split_ws, out, stream)


def lbp_attend_noalloc(cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, out,
                       stream=None):
    """lbp_attend with the split buffer in the library's fixed device array
    (no workspace argument; nothing is allocated)."""
    import torch
    kp, vp, ksp, vsp = _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale)
    _check(load().lbp_attend_noalloc(ctypes.byref(cfg), ctypes.byref(info),
                                     _ptr(plan_ws, "plan_ws"), _ptr(q, "q", torch.bfloat16),
                                     kp, vp, ksp, vsp, _ptr(out, "out", torch.bfloat16),
                                     _stream(stream)), "lbp_attend_noalloc")


def lbp_attend_fp8q(cfg, info, plan_ws, q_codes, q_scale, k_cache, v_cache, k_scale, v_scale,
                    split_ws, out, stream=None):
    """FP8 query (uint8 e4m3 codes [B, Hq, 128] + fp32 scales [B, Hq]) over FP8 KV."""
    import torch
    kp, vp, ksp, vsp = _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale)
    _check(load().lbp_attend_fp8q(ctypes.byref(cfg), ctypes.byref(info), _ptr(plan_ws, "plan_ws"),
                                  _ptr(q_codes, "q_codes", torch.uint8),
                                  _ptr(q_scale, "q_scale", torch.float32), kp, vp, ksp, vsp,
                                  _ptr(split_ws, "split_ws"),
                                  split_ws.numel() * split_ws.element_size(),
                                  _ptr(out, "out", torch.bfloat16), _stream(stream)),
           "lbp_attend_fp8q")


def lbp_prologue(cfg, qkv, seq_lens, page_table, q_norm_weight, k_norm_weight, rope_cos_sin,
                 q_out, k_cache, v_cache, k_scale=None, v_scale=None, q_scale_out=None,
                 norm_eps=1e-6, stream=None):
    """Fused QK-Norm + RoPE + KV-cache write (+ FP8 query when q_scale_out is given)."""
    import torch
    fp8_kv = cfg.kv_dtype == LBP_KV_FP8_E4M3
    kv_t = torch.uint8 if fp8_kv else torch.bfloat16
    q_fp8 = q_scale_out is not None
    a = lbp_prologue_args()
    a.qkv = _ptr(qkv, "qkv", torch.bfloat16)
    a.seq_lens = _ptr(seq_lens, "seq_lens", torch.int32)
    a.page_table = _ptr(page_table, "page_table", torch.int32)
    a.page_table_stride = int(page_table.shape[1])
    a.q_norm_weight = _ptr(q_norm_weight, "q_norm_weight", torch.float32)
    a.k_norm_weight = _ptr(k_norm_weight, "k_norm_weight", torch.float32)
    a.rope_cos_sin = _ptr(rope_cos_sin, "rope_cos_sin", torch.float32)
    a.max_position = int(rope_cos_sin.shape[0])
    a.norm_eps = float(norm_eps)
    a.q_fp8 = int(q_fp8)
    a.q_out = _ptr(q_out, "q_out", torch.uint8 if q_fp8 else torch.bfloat16)
    a.q_scale_out = _ptr(q_scale_out, "q_scale_out", torch.float32, optional=True)
    a.k_cache = _ptr(k_cache, "k_cache", kv_t)
    a.v_cache = _ptr(v_cache, "v_cache", kv_t)
    a.k_scale = _ptr(k_scale, "k_scale", torch.float32, optional=not fp8_kv)
    a.v_scale = _ptr(v_scale, "v_scale", torch.float32, optional=not fp8_kv)
    _check(load().lbp_prologue(ctypes.byref(cfg), int(seq_lens.numel()), ctypes.byref(a),
                               _stream(stream)), "lbp_prologue")


def lbp_attend_partials(cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, split_ws,
                        out, stream=None):
    import torch
    kp, vp, ksp, vsp = _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale)
    _check(load().lbp_attend_partials(ctypes.byref(cfg), ctypes.byref(info),
                                      _ptr(plan_ws, "plan_ws"), _ptr(q, "q", torch.bfloat16),
                                      kp, vp, ksp, vsp, _ptr(split_ws, "split_ws"),
                                      split_ws.numel() * split_ws.element_size(),
                                      _ptr(out, "out", torch.bfloat16), _stream(stream)),
           "lbp_attend_partials")


def lbp_attend_traced(cfg, info, plan_ws, q, k_cache, v_cache, k_scale, v_scale, split_ws, out,
                      trace, stream=None):
    """``trace`` is an int64 device tensor of at least 4 * info.num_bins entries."""
    import torch
    if trace.numel() < 4 * info.num_bins:
        raise ValueError("trace needs 4 * num_bins entries")
    kp, vp, ksp, vsp = _kv_ptrs(cfg, k_cache, v_cache, k_scale, v_scale)
    _check(load().lbp_attend_traced(ctypes.byref(cfg), ctypes.byref(info),
                                    _ptr(plan_ws, "plan_ws"), _ptr(q, "q", torch.bfloat16), kp,
                                    vp, ksp, vsp, _ptr(split_ws, "split_ws"),
                                    split_ws.numel() * split_ws.element_size(),
                                    _ptr(out, "out", torch.bfloat16),
                                    _ptr(trace, "trace", torch.int64), _stream(stream)),
           "lbp_attend_traced")


def lbp_combine(cfg, info, plan_ws, split_ws, out, stream=None):
    import torch
    _check(load().lbp_combine(ctypes.byref(cfg), ctypes.byref(info), _ptr(plan_ws, "plan_ws"),
                              _ptr(split_ws, "split_ws"),
                              split_ws.numel() * split_ws.element_size(),
                              _ptr(out, "out", torch.bfloat16), _stream(stream)), "lbp_combine")


def lbp_read_stream(buf, sink, blocks, stream=None):
    """Measurement reference (not the method): read every byte of `buf` once
    with `blocks` workgroups; sink is an int32 tensor of at least `blocks`."""
    import torch
    if sink.numel() < blocks:
        raise ValueError("sink needs one int32 per workgroup")
    _check(load().lbp_read_stream(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                  _ptr(sink, "sink", torch.int32), int(blocks), _stream(stream)),
           "lbp_read_stream")


# ---------------------------------------------------------------------------
# readers for host-side inspection (tests, benchmark)
# ---------------------------------------------------------------------------

def lbp_taskmap_to_host(plan_ws, info: lbp_plan_info, stream=None) -> np.ndarray:
    """The plan's task map as host bytes (lbp_taskmap_to_host: ordered on
    `stream`, waits for the copy)."""
    off = lbp_plan_layout(info)
    raw = np.empty(off.total, dtype=np.uint8)
    _check(load().lbp_taskmap_to_host(ctypes.byref(info), _ptr(plan_ws, "plan_ws"),
                                      raw.ctypes.data_as(ctypes.c_void_p), raw.nbytes,
                                      _stream(stream)), "lbp_taskmap_to_host")
    return raw


def read_taskmap(plan_ws, info: lbp_plan_info) -> dict:
    """Copy a plan's task map to the host (lbp_taskmap_to_host) and slice it
    by lbp_plan_layout."""
    off = lbp_plan_layout(info)
    raw = lbp_taskmap_to_host(plan_ws, info)
    words = raw.view(np.int32)
    h = words[off.header // 4: off.header // 4 + 16]
    D = int(h[7])
    npairs = info.num_kv_heads * info.batch

    def sl(o, n):
        return words[o // 4: o // 4 + n].copy()

    return {
        "magic": int(np.uint32(h[0])), "policy": int(h[1]), "num_bins": int(h[2]),
        "batch": int(h[3]), "num_kv_heads": int(h[4]),
        "header": (int(h[5]), int(h[6]), int(h[7]), int(h[8])), "status": int(h[9]),
        "bin_offset": sl(off.bin_offset, info.num_bins + 1),
        "bin_first": sl(off.bin_first, 8 * info.num_bins).reshape(-1, 8)[:, :4],
        "bin_pages": sl(off.bin_first, 8 * info.num_bins).reshape(-1, 8)[:, 4:6],
        "desc": sl(off.desc, 4 * D).reshape(D, 4),
        "pair_first": sl(off.pair_first, npairs),
        "pair_count": sl(off.pair_count, npairs),
        "split_list": sl(off.split_list, 4 * int(h[11])).reshape(-1, 4),
        "arrive": sl(off.arrive, 2 * info.max_desc if info.policy == LBP_POLICY_DYNAMIC else 0),
    }


def split_views(split_ws, info: lbp_plan_info, group: int):
    """(o_part [max_desc, G, 128], lse_part [max_desc, G]) fp32 views of a split buffer."""
    import torch
    flat = split_ws.view(-1).view(torch.uint8)
    md = info.max_desc
    o_bytes = md * group * HEAD_DIM * 4
    lse_off = (o_bytes + 255) // 256 * 256
    o = flat[:o_bytes].view(torch.float32).view(md, group, HEAD_DIM)
    lse = flat[lse_off:lse_off + md * group * 4].view(torch.float32).view(md, group)
    return o, lse
