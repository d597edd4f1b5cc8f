"""Striped ring attention on AMD MI355X: Python binding of libsra.

Thin ctypes layer over the C ABI in ``include/sra.h``; every function here
only marshals arguments (pointers, sizes, the current HIP stream) and calls
the library. All work runs in the library's HIP kernels. There is no CPU
fallback: if ``libsra.so`` is missing, every call raises.

Layouts (Striped Attention summary page, research.elamur.ai, "Summary"
¶1-2): ``CONTIGUOUS`` -- device d holds one contiguous chunk; ``STRIPED`` --
device d holds every N-th token, positions d, d+N, d+2N, ... Ring functions
take and return tensors in device layout ([B, S, H, Dh], slot d*L + j holds
device d's j-th token); ``stripe_permute`` / ``unstripe`` convert between
original order and striped device layout.
"""

import ctypes
import os

import torch  # torch's HIP runtime must be loaded before libsra (they share libamdhip64.so.7)

CONTIGUOUS = 0
STRIPED = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
SCHEDULE_PER_ROUND = 0
SCHEDULE_FUSED = 1
ORDER_DEVICE = 0     # tensors in device layout (slot d*L + j)
ORDER_ORIGINAL = 1   # tensors in original token order; the kernels address device rows in place

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsra.so")

_lib = None

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class SraDesc(ctypes.Structure):
    _fields_ = [
        ("batch", _i64), ("seq", _i64), ("heads", _i64), ("head_dim", _i64),
        ("n_dev", _i32), ("layout", _i32), ("dtype", _i32), ("schedule", _i32),
        ("scale", _f32), ("order", _i32),
    ]


class SraError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_PROTOS = {
    "sra_abi_version": (_i32, []),
    "sra_status_str": (ctypes.c_char_p, [_i32]),
    "sra_last_error": (ctypes.c_char_p, []),
    "sra_stripe_index": (_i32, [_i64, _i32, _i32, _vp]),
    "sra_count_live_tiles": (_i32, [ctypes.POINTER(SraDesc), _i64, _i64, _vp, _vp, _vp]),
    "sra_count_live_pairs": (_i32, [ctypes.POINTER(SraDesc), _vp]),
    "sra_kernel_tiles": (_i32, [ctypes.POINTER(SraDesc), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "sra_stripe_permute": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "sra_unstripe": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "sra_rope_permute": (_i32, [ctypes.POINTER(SraDesc), _vp, _vp, _vp, ctypes.c_double, _vp]),
    "sra_ring_round_attn": (_i32, [ctypes.POINTER(SraDesc), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sra_lse_merge": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "sra_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SraDesc)]),
    "sra_ring_attn_fwd": (_i32, [ctypes.POINTER(SraDesc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp, _vp]),
    "sra_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SraDesc)]),
    "sra_ring_attn_bwd": (_i32, [ctypes.POINTER(SraDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.c_size_t, _vp]),
    "sra_ring_attn_bwd_noalloc": (_i32, [ctypes.POINTER(SraDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp]),
}


def load(path=None):
    """Load libsra.so (once) and declare its prototypes. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libsra.so not found at {path}; build it with "
                           "`python -m striped_ring_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    return load()


def _check(status):
    if status != 0:
        L = lib()
        raise SraError(status, f"{L.sra_status_str(status).decode()}: {L.sra_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {dt}")


def make_desc(batch, seq, heads, head_dim, n_dev, layout, dtype=DTYPE_BF16, scale=0.0, schedule=SCHEDULE_PER_ROUND,
              order=ORDER_DEVICE):
    if isinstance(dtype, torch.dtype):
        dtype = _dtype_code(dtype)
    return SraDesc(batch, seq, heads, head_dim, n_dev, layout, dtype, schedule, scale, order)


def _desc_for(q, n_dev, layout, scale, schedule=SCHEDULE_PER_ROUND, order=ORDER_DEVICE):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, S, H, Dh]")
    B, S, H, D = q.shape
    return make_desc(B, S, H, D, n_dev, layout, _dtype_code(q.dtype), scale, schedule, order)


def _check_tensors(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")


# --------------------------------------------------------------- host-only --

def abi_version():
    return lib().sra_abi_version()


def stripe_index(seq, n_dev, layout):
    """perm[slot] = original position of device-layout slot (CPU int64 tensor)."""
    out = torch.empty(seq, dtype=torch.int64)
    _check(lib().sra_stripe_index(seq, n_dev, layout, _ptr(out)))
    return out


def count_live_tiles(seq, n_dev, layout, tile_q, tile_k):
    """(live, full, partial) tile counts per (round, device) for one (b, h): CPU int64 [N, N]."""
    live, full, part = (torch.empty(n_dev * n_dev, dtype=torch.int64) for _ in range(3))
    d = make_desc(1, seq, 1, 128, n_dev, layout)
    _check(lib().sra_count_live_tiles(ctypes.byref(d), tile_q, tile_k, _ptr(live), _ptr(full), _ptr(part)))
    return tuple(t.view(n_dev, n_dev) for t in (live, full, part))


def count_live_pairs(seq, n_dev, layout):
    """Live (query, key) pairs per (round, device) for one (b, h): CPU int64 [N, N]."""
    out = torch.empty(n_dev * n_dev, dtype=torch.int64)
    d = make_desc(1, seq, 1, 128, n_dev, layout)
    _check(lib().sra_count_live_pairs(ctypes.byref(d), _ptr(out)))
    return out.view(n_dev, n_dev)


def kernel_tiles(dtype=torch.bfloat16, head_dim=128):
    """(tile_q, tile_k) of the ring-round kernel for this dtype and head dim."""
    d = make_desc(1, 1, 1, head_dim, 1, STRIPED, _dtype_code(dtype))
    tq, tk = _i32(), _i32()
    _check(lib().sra_kernel_tiles(ctypes.byref(d), ctypes.byref(tq), ctypes.byref(tk)))
    return tq.value, tk.value


def fwd_workspace_bytes(q, n_dev, layout, schedule=SCHEDULE_PER_ROUND):
    d = _desc_for(q, n_dev, layout, 0.0, schedule)
    return lib().sra_fwd_workspace_bytes(ctypes.byref(d))


def bwd_workspace_bytes(q, n_dev, layout):
    """Workspace bytes sra_ring_attn_bwd needs for device-layout q (the per-row
    Delta = rowsum(dO * O) vector)."""
    d = _desc_for(q, n_dev, layout, 0.0)
    return int(lib().sra_bwd_workspace_bytes(ctypes.byref(d)))


# ------------------------------------------------------------------ device --

def _row_bytes(x):
    return x[0, 0].numel() * x.element_size() if x.dim() > 2 else x.element_size()


def stripe_permute(x, n_dev, out=None):
    """Original order -> striped device layout along dim 1 of x ([B, S, ...])."""
    _check_tensors(x, out)
    out = torch.empty_like(x) if out is None else out
    _check(lib().sra_stripe_permute(_ptr(x), _ptr(out), x.shape[0], x.shape[1], _row_bytes(x), n_dev, _stream()))
    return out


def unstripe(y, n_dev, out=None):
    """Striped device layout -> original order along dim 1 of y ([B, S, ...])."""
    _check_tensors(y, out)
    out = torch.empty_like(y) if out is None else out
    _check(lib().sra_unstripe(_ptr(y), _ptr(out), y.shape[0], y.shape[1], _row_bytes(y), n_dev, _stream()))
    return out


def rope_permute(x, n_dev, layout, pos=None, base=10000.0, order=ORDER_DEVICE, out=None):
    """Rotary embedding of x ([B, S, H, D], original order) at each token's
    original position (or pos, int64 [B, S]), written in striped device layout
    (order=ORDER_DEVICE, striped) or in original order (out may be x then)."""
    _check_tensors(x, out, pos)
    if pos is not None and (pos.dtype != torch.int64 or tuple(pos.shape) != tuple(x.shape[:2])):
        raise ValueError("pos must be int64 [B, S]")
    d = _desc_for(x, n_dev, layout, 0.0, order=order)
    out = torch.empty_like(x) if out is None else out
    _check(lib().sra_rope_permute(ctypes.byref(d), _ptr(x), _ptr(out), _ptr(pos), float(base), _stream()))
    return out


def ring_round_attn(q, k, v, n_dev, layout, round, device=-1, scale=0.0, o_part=None, lse_part=None,
                    live_counts=None, order=ORDER_DEVICE):
    """One ring round: partial (O fp32, LSE fp32) for the selected device(s)."""
    _check_tensors(q, k, v, o_part, lse_part, live_counts)
    d = _desc_for(q, n_dev, layout, scale, order=order)
    B, S, H, D = q.shape
    if o_part is None:
        o_part = torch.zeros((B, S, H, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.full((B, S, H), float("-inf"), dtype=torch.float32, device=q.device)
    _check(lib().sra_ring_round_attn(ctypes.byref(d), round, device, _ptr(q), _ptr(k), _ptr(v), _ptr(o_part),
                                     _ptr(lse_part), _ptr(live_counts), _stream()))
    return o_part, lse_part


def lse_merge(o_acc, lse_acc, o_part, lse_part):
    """In-place log-sum-exp merge of (o_part, lse_part) into (o_acc, lse_acc)."""
    _check_tensors(o_acc, lse_acc, o_part, lse_part)
    D = o_acc.shape[-1]
    rows = o_acc.numel() // D
    _check(lib().sra_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), rows, D, _stream()))
    return o_acc, lse_acc


def ring_attn_fwd(q, k, v, n_dev, layout, scale=0.0, schedule=SCHEDULE_PER_ROUND, out=None, lse=None,
                  workspace=None, live_counts=None, round_events=None, order=ORDER_DEVICE):
    """All N rounds of the ring; returns (O, LSE) in the order of q, k, v
    (device layout, or original token order with order=ORDER_ORIGINAL)."""
    _check_tensors(q, k, v, out, lse, workspace, live_counts)
    d = _desc_for(q, n_dev, layout, scale, schedule, order)
    B, S, H, D = q.shape
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, S, H), dtype=torch.float32, device=q.device) if lse is None else lse
    need = lib().sra_fwd_workspace_bytes(ctypes.byref(d))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ev = None
    if round_events is not None:
        ev = (ctypes.c_void_p * len(round_events))(*[e.cuda_event if hasattr(e, "cuda_event") else e
                                                     for e in round_events])
    _check(lib().sra_ring_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   _ptr(workspace), ws_bytes, _ptr(live_counts), ev, _stream()))
    return out, lse


def ring_attn_bwd(q, k, v, o, lse, dout, n_dev, layout, scale=0.0, dq=None, dk=None, dv=None, workspace=None,
                  order=ORDER_DEVICE):
    """Gradient of the ring forward on device-layout tensors; returns (dq, dk, dv)."""
    _check_tensors(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    d = _desc_for(q, n_dev, layout, scale, order=order)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = lib().sra_bwd_workspace_bytes(ctypes.byref(d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().sra_ring_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream()))
    return dq, dk, dv


def ring_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, n_dev, layout, scale=0.0, order=ORDER_DEVICE):
    """ring_attn_bwd into caller-given dq, dk, dv with no workspace: the
    library's own per-GPU statistics array is used, and nothing is allocated
    (calls overlapping in time on one GPU race)."""
    _check_tensors(q, k, v, o, lse, dout, dq, dk, dv)
    d = _desc_for(q, n_dev, layout, scale, order=order)
    _check(lib().sra_ring_attn_bwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                           _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream()))
    return dq, dk, dv


def striped_attention(q, k, v, n_dev, scale=0.0, schedule=None):
    """Original-order q, k, v -> striped ring over all rounds, the stripe
    permutation folded into the kernels' row addressing. The schedule
    defaults to the fused one for bf16 and per-round for fp32.

    Returns (O, LSE) in original order: exact causal attention."""
    if schedule is None:
        schedule = SCHEDULE_FUSED if q.dtype == torch.bfloat16 else SCHEDULE_PER_ROUND
    return ring_attn_fwd(q, k, v, n_dev, STRIPED, scale, schedule, order=ORDER_ORIGINAL)
