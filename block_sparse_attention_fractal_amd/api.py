"""Torch-facing binding of libbsa: tensors in, tensors out, no arithmetic here.

Every function validates tensor metadata, allocates outputs/workspace with
torch on the tensors' device, and calls the C ABI on the current HIP stream.
All computation runs in the HIP kernels.
"""
import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import BSA_BF16, BSA_F32, BSA_LAYOUT_FRACTAL, BSA_LAYOUT_ORIGINAL, check, lib

_LAYOUTS = {"original": BSA_LAYOUT_ORIGINAL, "fractal": BSA_LAYOUT_FRACTAL}


@dataclass(frozen=True)
class VideoGrid:
    """Token grid of one attention call: T x H x W tokens, fractal patch P, block N."""
    T: int
    H: int
    W: int
    patch: int = 8
    block: int = 64

    @property
    def L(self) -> int:
        return self.T * self.H * self.W

    @property
    def S(self) -> int:
        return self.L // self.block


@dataclass
class BlockMask:
    """CSR block mask on the device: row r = (b*heads + h)*S + i lists the kept key
    blocks of query block i, ascending.  col_idx has capacity batch*heads*S*S.
    shift (optional, aligned with col_idx) holds each entry's logit shift, as a
    sampled (SIP) mask produces it."""
    row_ptr: torch.Tensor     # int32 [rows + 1]
    col_idx: torch.Tensor     # int32 [capacity]
    nnz_dev: torch.Tensor     # int32 [1]
    rows: int
    S: int
    shift: Optional[torch.Tensor] = None   # float32 [capacity] or None

    def nnz(self) -> int:
        return int(self.nnz_dev.item())

    def density(self) -> float:
        return self.nnz() / float(self.rows * self.S)

    def as_struct(self) -> _lib.CSR:
        return _lib.CSR(self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.col_idx.numel(),
                        self.nnz_dev.data_ptr(), None if self.shift is None else self.shift.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _check_qkv(*ts: torch.Tensor):
    ref = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [batch, heads, L, head_dim]")
        if t.dim() != 4 or t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q/k/v must share shape [batch, heads, L, head_dim], dtype and device")


def make_problem(x: torch.Tensor, grid: VideoGrid, layout: str = "original") -> _lib.Problem:
    B, nh, L, D = x.shape
    if L != grid.L:
        raise ValueError(f"tensor has L={L} tokens but the grid has {grid.L}")
    return _lib.Problem(B, nh, grid.T, grid.H, grid.W, D, grid.patch, grid.block, _dtype_code(x),
                        _LAYOUTS[layout])


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def query_sizes(prob: _lib.Problem) -> dict:
    rows, max_nnz, mws, fws = (ctypes.c_int64() for _ in range(4))
    check(lib().bsa_query_sizes(ctypes.byref(prob), ctypes.byref(rows), ctypes.byref(max_nnz),
                                ctypes.byref(mws), ctypes.byref(fws)))
    return {"rows": rows.value, "max_nnz": max_nnz.value, "mask_ws": mws.value, "fwd_ws": fws.value}


def backward_workspace_bytes(prob: _lib.Problem) -> int:
    """Bytes of device workspace bsa_backward needs for this problem."""
    nbytes = ctypes.c_int64()
    check(lib().bsa_query_backward_ws(ctypes.byref(prob), ctypes.byref(nbytes)))
    return nbytes.value


def attend_workspace_bytes(prob: _lib.Problem) -> int:
    """Bytes of device workspace bsa_attend needs for this problem (work counters and order)."""
    nbytes = ctypes.c_int64()
    check(lib().bsa_query_attend_ws(ctypes.byref(prob), ctypes.byref(nbytes)))
    return nbytes.value


def attend_groups_workspace_bytes(prob: _lib.Problem) -> int:
    """Bytes of device workspace bsa_attend_groups needs for this problem (work counters and order)."""
    nbytes = ctypes.c_int64()
    check(lib().bsa_query_attend_groups_ws(ctypes.byref(prob), KEY_GROUP, ctypes.byref(nbytes)))
    return nbytes.value


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes or ws.data_ptr() % 256:
            raise ValueError(f"workspace must hold {nbytes} bytes and be 256-byte aligned")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def permute(x: torch.Tensor, grid: VideoGrid, inverse: bool = False) -> torch.Tensor:
    """Original (t,h,w) order -> fractal order (inverse=False) or back; bit-exact copy."""
    _check_qkv(x)
    y = torch.empty_like(x)
    prob = make_problem(x, grid)
    check(lib().bsa_permute(ctypes.byref(prob), x.data_ptr(), y.data_ptr(), int(inverse), _stream(x.device)))
    return y


ORDERS = {"fractal": _lib.BSA_ORDER_FRACTAL, "tile_major": _lib.BSA_ORDER_TILE_MAJOR,
          "hilbert": _lib.BSA_ORDER_HILBERT}


def order_table(grid: VideoGrid, order: str, head_dim: int = 128, dtype=torch.bfloat16) -> torch.Tensor:
    """int32 [L] CPU tensor: the original (t,h,w) index of the token at each position
    of the given order ("fractal", "tile_major" or "hilbert"), computed by the library."""
    if order not in ORDERS:
        raise ValueError(f"order must be one of {sorted(ORDERS)}")
    x = torch.empty((1, 1, 0, head_dim), dtype=dtype)          # shape carrier only
    prob = _lib.Problem(1, 1, grid.T, grid.H, grid.W, head_dim, grid.patch, grid.block, _dtype_code(x),
                        BSA_LAYOUT_FRACTAL)   # the layout does not enter the table; this one accepts any P
    table = torch.empty(grid.T * grid.H * grid.W, dtype=torch.int32)
    check(lib().bsa_order_table(ctypes.byref(prob), ORDERS[order], table.data_ptr()))
    return table


def permute_table(x: torch.Tensor, grid: VideoGrid, table: torch.Tensor, inverse: bool = False) -> torch.Tensor:
    """Rows of x into the order given by `table` (inverse=False) or back; bit-exact copy.
    table: int32 permutation of [0, L) (moved to x's device if needed)."""
    _check_qkv(x)
    if table.dtype != torch.int32 or table.numel() != x.shape[2]:
        raise ValueError("table must be int32 with one entry per token")
    t = table.to(x.device).contiguous()
    y = torch.empty_like(x)
    prob = make_problem(x, grid, "fractal")     # the layout does not enter a table copy
    check(lib().bsa_permute_table(ctypes.byref(prob), t.data_ptr(), x.data_ptr(), y.data_ptr(), int(inverse),
                                  _stream(x.device)))
    return y


def pool(q: torch.Tensor, k: torch.Tensor, grid: VideoGrid, layout: str = "original") -> Tuple[torch.Tensor, torch.Tensor]:
    """Block means of q and k, float64 [batch, heads, S, head_dim]."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    B, nh, _, D = q.shape
    qp = torch.empty((B, nh, grid.S, D), dtype=torch.float64, device=q.device)
    kp = torch.empty_like(qp)
    check(lib().bsa_pool(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), qp.data_ptr(), kp.data_ptr(),
                         _stream(q.device)))
    return qp, kp


def block_map(qp: torch.Tensor, kp: torch.Tensor, grid: VideoGrid, dtype=torch.bfloat16) -> torch.Tensor:
    """Reduced softmax map over pooled blocks, float64 [batch, heads, S, S]."""
    if qp.dtype != torch.float64 or kp.dtype != torch.float64 or not qp.is_contiguous() or not kp.is_contiguous():
        raise ValueError("qp, kp must be contiguous float64 tensors from pool()")
    B, nh, S, D = qp.shape
    probe = torch.empty((B, nh, grid.L, D), dtype=dtype, device="meta")
    prob = make_problem(probe, grid)
    out = torch.empty((B, nh, S, S), dtype=torch.float64, device=qp.device)
    check(lib().bsa_block_map(ctypes.byref(prob), qp.data_ptr(), kp.data_ptr(), out.data_ptr(),
                              _stream(qp.device)))
    return out


def build_mask(q: torch.Tensor, k: torch.Tensor, grid: VideoGrid, thr: float,
               window: Optional[Tuple[int, int, int]] = None, layout: str = "original",
               workspace: Optional[torch.Tensor] = None, sip_seed: Optional[int] = None) -> BlockMask:
    """Pool -> reduced map -> CDF cut at 1-thr (-> union with +-window tiles) -> CSR.
    With sip_seed set, the cut is replaced by SIP sampling (same budget per row,
    Philox key = sip_seed) and the mask carries per-entry logit shifts."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    sz = query_sizes(prob)
    dev = q.device
    row_ptr = torch.empty(sz["rows"] + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(sz["max_nnz"], dtype=torch.int32, device=dev)
    nnz = torch.empty(1, dtype=torch.int32, device=dev)
    shift = torch.empty(sz["max_nnz"], dtype=torch.float32, device=dev) if sip_seed is not None else None
    mask = BlockMask(row_ptr, col_idx, nnz, sz["rows"], grid.S, shift)
    ws = _workspace(sz["mask_ws"], dev, workspace)
    wt, wh, ww = window if window is not None else (-1, -1, -1)
    mode = _lib.BSA_MASK_SIP if sip_seed is not None else _lib.BSA_MASK_CDF
    mp = _lib.MaskParams(float(thr), wt, wh, ww, mode, 0 if sip_seed is None else int(sip_seed) % 2**64)
    csr = mask.as_struct()
    check(lib().bsa_build_mask(ctypes.byref(prob), ctypes.byref(mp), q.data_ptr(), k.data_ptr(),
                               ctypes.byref(csr), ws.data_ptr(), ws.numel(), _stream(dev)))
    return mask


def mask_from_csr(row_ptr: torch.Tensor, col_idx: torch.Tensor, S: int,
                  shift: Optional[torch.Tensor] = None) -> BlockMask:
    """Wrap a caller-made CSR (int32 device tensors, optional float32 per-entry
    logit shifts aligned with col_idx) for forward()."""
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    if shift is not None and (shift.dtype != torch.float32 or shift.numel() < col_idx.numel()):
        raise TypeError("shift must be float32 with one entry per col_idx entry")
    rows = row_ptr.numel() - 1
    nnz = row_ptr[-1:].clone()
    return BlockMask(row_ptr.contiguous(), col_idx.contiguous(), nnz, rows, S,
                     None if shift is None else shift.contiguous())


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: BlockMask, grid: VideoGrid,
            layout: str = "original", return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Attention of every query block over the tokens of its kept key blocks."""
    _check_qkv(q, k, v)
    prob = make_problem(q, grid, layout)
    sz = query_sizes(prob)
    if mask.rows != sz["rows"]:
        raise ValueError(f"mask has {mask.rows} rows, the problem needs {sz['rows']}")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(sz["fwd_ws"], q.device, workspace)
    csr = mask.as_struct()
    check(lib().bsa_forward(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(csr),
                            o.data_ptr(), lse.data_ptr() if lse is not None else None,
                            ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (o, lse) if return_lse else o


def prepare_v(v: torch.Tensor, grid: VideoGrid, layout: str = "original",
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 only: V in the attention kernel's layout (fractal block order, per-block
    transposed).  Returned as a flat bf16 tensor of V's size (written into `out` when given)."""
    _check_qkv(v)
    prob = make_problem(v, grid, layout)
    if out is not None and (out.numel() != v.numel() or out.dtype != v.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor with v's dtype and size")
    vt = torch.empty(v.numel(), dtype=v.dtype, device=v.device) if out is None else out
    check(lib().bsa_prepare_v(ctypes.byref(prob), v.data_ptr(), vt.data_ptr(), _stream(v.device)))
    return vt


def attend(q: torch.Tensor, k: torch.Tensor, vp: torch.Tensor, mask: BlockMask, grid: VideoGrid,
           layout: str = "original", return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None):
    """The attention kernel alone: `vp` = prepare_v(v) for bf16, or v itself for float32."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    sz = query_sizes(prob)
    if mask.rows != sz["rows"]:
        raise ValueError(f"mask has {mask.rows} rows, the problem needs {sz['rows']}")
    if vp.numel() != q.numel() or vp.dtype != q.dtype or not vp.is_contiguous():
        raise ValueError("vp must be a contiguous tensor with q's dtype and size")
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(attend_workspace_bytes(prob), q.device, workspace)
    csr = mask.as_struct()
    check(lib().bsa_attend(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), vp.data_ptr(), ctypes.byref(csr),
                           o.data_ptr(), lse.data_ptr() if lse is not None else None,
                           ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (o, lse) if return_lse else o


def attend_train(q: torch.Tensor, k: torch.Tensor, vp: torch.Tensor, mask: BlockMask, grid: VideoGrid,
                 layout: str = "original", workspace: Optional[torch.Tensor] = None, out=None):
    """bf16 training forward (bsa_attend_train): returns (o, o_lo, lse), with o + o_lo
    holding O to ~2^-16 for backward_train.  `vp` = prepare_v(v); `out` = (o, o_lo)."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    sz = query_sizes(prob)
    if mask.rows != sz["rows"]:
        raise ValueError(f"mask has {mask.rows} rows, the problem needs {sz['rows']}")
    if vp.numel() != q.numel() or vp.dtype != q.dtype or not vp.is_contiguous():
        raise ValueError("vp must be a contiguous tensor with q's dtype and size")
    o, o_lo = (torch.empty_like(q), torch.empty_like(q)) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws = _workspace(attend_workspace_bytes(prob), q.device, workspace)
    csr = mask.as_struct()
    check(lib().bsa_attend_train(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), vp.data_ptr(), ctypes.byref(csr),
                                 o.data_ptr(), o_lo.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(),
                                 _stream(q.device)))
    return o, o_lo, lse


def attend_static(q: torch.Tensor, k: torch.Tensor, vp: torch.Tensor, mask: BlockMask, grid: VideoGrid,
                  layout: str = "original", return_lse: bool = False, out: Optional[torch.Tensor] = None):
    """attend() through bsa_attend_static: no workspace argument (the library's static
    scratch holds the work order), for callers that cannot allocate device memory."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    if vp.numel() != q.numel() or vp.dtype != q.dtype or not vp.is_contiguous():
        raise ValueError("vp must be a contiguous tensor with q's dtype and size")
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    csr = mask.as_struct()
    check(lib().bsa_attend_static(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), vp.data_ptr(), ctypes.byref(csr),
                                  o.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(q.device)))
    return (o, lse) if return_lse else o


def attention(q, k, v, grid: VideoGrid, thr: float, window=None, layout: str = "original",
              return_lse: bool = False):
    """The whole hot path: mask from (q, k), then block-sparse attention."""
    mask = build_mask(q, k, grid, thr, window, layout)
    out = forward(q, k, v, mask, grid, layout, return_lse)
    return (out, mask)


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: BlockMask, grid: VideoGrid,
             lse: torch.Tensor, dout: torch.Tensor, layout: str = "original",
             workspace: Optional[torch.Tensor] = None, out=None):
    """Gradients (dq, dk, dv) of sum(o * dout) for o = forward(q, k, v, mask), given the
    forward's lse (the row term is recomputed from P and dP, so o is not needed).
    `out` = (dq, dk, dv) tensors shaped like q to write into (else new ones)."""
    _check_qkv(q, k, v, dout)
    if lse.dtype != torch.float32 or lse.shape != q.shape[:3] or not lse.is_contiguous():
        raise ValueError("lse must be float32 [batch, heads, L] as forward(return_lse=True) gives it")
    prob = make_problem(q, grid, layout)
    ws = _workspace(backward_workspace_bytes(prob), q.device, workspace)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _check_qkv(q, dq, dk, dv)
    csr = mask.as_struct()
    check(lib().bsa_backward(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(csr),
                             lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             ws.data_ptr(), ws.numel(), _stream(q.device)))
    return dq, dk, dv


def backward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: BlockMask, grid: VideoGrid,
                   o: torch.Tensor, o_lo: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                   layout: str = "original", workspace: Optional[torch.Tensor] = None, out=None):
    """Gradients (dq, dk, dv) from attend_train's (o, o_lo, lse): the row term is
    dO . (o + o_lo) (bsa_backward_train), so the walk over the kept tiles that
    backward() runs for it is skipped.  bf16, head_dim 128."""
    _check_qkv(q, k, v, dout, o, o_lo)
    if lse.dtype != torch.float32 or lse.shape != q.shape[:3] or not lse.is_contiguous():
        raise ValueError("lse must be float32 [batch, heads, L] as attend_train gives it")
    prob = make_problem(q, grid, layout)
    ws = _workspace(backward_workspace_bytes(prob), q.device, workspace)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _check_qkv(q, dq, dk, dv)
    csr = mask.as_struct()
    check(lib().bsa_backward_train(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(csr),
                                   o.data_ptr(), o_lo.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device)))
    return dq, dk, dv


# ---- 4-token key groups (gathered into 64-key tiles by the kernel) ----------
KEY_GROUP = _lib.KEY_GROUP


def query_group_sizes(prob: _lib.Problem) -> dict:
    max_nnz, mws, fws = (ctypes.c_int64() for _ in range(3))
    check(lib().bsa_query_group_sizes(ctypes.byref(prob), KEY_GROUP, ctypes.byref(max_nnz), ctypes.byref(mws),
                                      ctypes.byref(fws)))
    return {"max_nnz": max_nnz.value, "mask_ws": mws.value, "fwd_ws": fws.value}


def build_group_mask(q: torch.Tensor, k: torch.Tensor, grid: VideoGrid, thr: float,
                     window: Optional[Tuple[int, int, int]] = None, layout: str = "original",
                     workspace: Optional[torch.Tensor] = None) -> BlockMask:
    """Key-group mask: the reduced map of 64-token query blocks against 4-token key
    groups, CDF cut at 1-thr (-> union with the groups of +-window tiles) -> CSR of
    group ids (mask.S = L/4 columns per row)."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    rows = query_sizes(prob)["rows"]
    sz = query_group_sizes(prob)
    dev = q.device
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(sz["max_nnz"], dtype=torch.int32, device=dev)
    nnz = torch.empty(1, dtype=torch.int32, device=dev)
    mask = BlockMask(row_ptr, col_idx, nnz, rows, grid.L // KEY_GROUP)
    ws = _workspace(sz["mask_ws"], dev, workspace)
    wt, wh, ww = window if window is not None else (-1, -1, -1)
    mp = _lib.MaskParams(float(thr), wt, wh, ww, _lib.BSA_MASK_CDF, 0)
    csr = mask.as_struct()
    check(lib().bsa_build_group_mask(ctypes.byref(prob), KEY_GROUP, ctypes.byref(mp), q.data_ptr(), k.data_ptr(),
                                     ctypes.byref(csr), ws.data_ptr(), ws.numel(), _stream(dev)))
    return mask


def prepare_v_groups(v: torch.Tensor, grid: VideoGrid, layout: str = "original",
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 only: V as [batch, heads, L/4, D, 4] (each 4-token group channel-major), flat
    (written into `out` when given: a contiguous tensor of V's dtype and size)."""
    _check_qkv(v)
    prob = make_problem(v, grid, layout)
    if out is not None and (out.numel() != v.numel() or out.dtype != v.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor with v's dtype and size")
    vg = torch.empty(v.numel(), dtype=v.dtype, device=v.device) if out is None else out
    check(lib().bsa_prepare_v_groups(ctypes.byref(prob), KEY_GROUP, v.data_ptr(), vg.data_ptr(), _stream(v.device)))
    return vg


def _check_group_mask(mask: BlockMask, prob: _lib.Problem, grid: VideoGrid):
    rows = query_sizes(prob)["rows"]
    if mask.rows != rows or mask.S != grid.L // KEY_GROUP:
        raise ValueError(f"group mask has {mask.rows} rows of {mask.S} columns, the problem needs "
                         f"{rows} rows of {grid.L // KEY_GROUP}")
    if mask.shift is not None:
        raise ValueError("group masks carry no logit shifts")


def attend_groups(q: torch.Tensor, k: torch.Tensor, vp: torch.Tensor, mask: BlockMask, grid: VideoGrid,
                  layout: str = "original", return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None):
    """The gathered-group attention kernel alone: `vp` = prepare_v_groups(v) for bf16, v for float32."""
    _check_qkv(q, k)
    prob = make_problem(q, grid, layout)
    _check_group_mask(mask, prob, grid)
    if vp.numel() != q.numel() or vp.dtype != q.dtype or not vp.is_contiguous():
        raise ValueError("vp must be a contiguous tensor with q's dtype and size")
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(attend_groups_workspace_bytes(prob), q.device, workspace)
    csr = mask.as_struct()
    check(lib().bsa_attend_groups(ctypes.byref(prob), KEY_GROUP, q.data_ptr(), k.data_ptr(), vp.data_ptr(),
                                  ctypes.byref(csr), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                  ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (o, lse) if return_lse else o


def forward_groups(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: BlockMask, grid: VideoGrid,
                   layout: str = "original", return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Attention of every query block over the tokens of its kept 4-token key groups."""
    _check_qkv(q, k, v)
    prob = make_problem(q, grid, layout)
    _check_group_mask(mask, prob, grid)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(query_group_sizes(prob)["fwd_ws"], q.device, workspace)
    csr = mask.as_struct()
    check(lib().bsa_forward_groups(ctypes.byref(prob), KEY_GROUP, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   ctypes.byref(csr), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                   ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (o, lse) if return_lse else o
