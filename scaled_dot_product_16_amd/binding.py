"""ctypes binding of libattn (argument marshalling only).

Every step of the attention runs in the HIP library; this module turns torch
tensors into the C descriptors of ``include/attn.h`` and passes torch's
current stream.  PyTorch is used for device memory and streams only.  If the
library is not built, the first call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

# Enumerations of include/attn.h.
ATTN_OK = 0
STATUS = {0: "OK", 1: "E_NULL", 2: "E_SHAPE", 3: "E_LAYOUT", 4: "E_UNSUPPORTED", 5: "E_ALIAS",
          6: "E_LAUNCH", 7: "E_INVALID"}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
LAYOUT_BATCHED, LAYOUT_IMAGE = 0, 1
QKV_DTYPE, QKV_E4M3 = 0, 1
# Torch dtypes accepted for 8-bit E4M3 q, k, v (the codes as bytes).
E4M3_DTYPES = (torch.uint8, torch.float8_e4m3fn)
BIAS_NONE, BIAS_TABLE, BIAS_RELPOS, BIAS_ADDITIVE = 0, 1, 2, 3
MASK_NONE, MASK_ADDITIVE, MASK_SHIFT_REGIONS = 0, 1, 2


class AttnTensorC(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dims", ctypes.c_int64 * 4),
                ("strides", ctypes.c_int64 * 3), ("layout", ctypes.c_int32)]


class BiasDescC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("table", ctypes.c_void_p), ("rh", ctypes.c_void_p), ("rw", ctypes.c_void_p),
                ("add", ctypes.c_void_p), ("add_batch", ctypes.c_int64),
                ("add_strides", ctypes.c_int64 * 2), ("kgrid_h", ctypes.c_int32),
                ("kgrid_w", ctypes.c_int32), ("rh_rows", ctypes.c_int32), ("rw_rows", ctypes.c_int32)]


class WindowC(ctypes.Structure):
    _fields_ = [("img_h", ctypes.c_int32), ("img_w", ctypes.c_int32), ("win_h", ctypes.c_int32),
                ("win_w", ctypes.c_int32), ("shift_h", ctypes.c_int32), ("shift_w", ctypes.c_int32)]


class MaskDescC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("add", ctypes.c_void_p), ("n_win", ctypes.c_int64),
                ("add_strides", ctypes.c_int64 * 2), ("win", WindowC), ("value", ctypes.c_float)]


class OptionsC(ctypes.Structure):
    _fields_ = [("window_heads", ctypes.c_int32), ("qkv_format", ctypes.c_int32),
                ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float),
                ("v_descale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("lse", ctypes.c_void_p)]


class BwdOptionsC(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("reserved", ctypes.c_int32 * 4)]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"attn: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libattn.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_dot_product_16_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        h.attn_fwd.argtypes = [P(AttnTensorC), P(AttnTensorC), P(AttnTensorC), P(BiasDescC),
                               P(MaskDescC), P(AttnTensorC), ctypes.c_int32, ctypes.c_void_p]
        h.attn_fwd.restype = ctypes.c_int
        h.attn_check.argtypes = [P(AttnTensorC), P(AttnTensorC), P(AttnTensorC), P(BiasDescC),
                                 P(MaskDescC), P(AttnTensorC), ctypes.c_int32]
        h.attn_check.restype = ctypes.c_int
        h.attn_fwd_opt.argtypes = [P(AttnTensorC), P(AttnTensorC), P(AttnTensorC), P(BiasDescC),
                                   P(MaskDescC), P(AttnTensorC), ctypes.c_int32, P(OptionsC),
                                   ctypes.c_void_p]
        h.attn_fwd_opt.restype = ctypes.c_int
        h.attn_check_opt.argtypes = [P(AttnTensorC), P(AttnTensorC), P(AttnTensorC), P(BiasDescC),
                                     P(MaskDescC), P(AttnTensorC), ctypes.c_int32, P(OptionsC)]
        h.attn_check_opt.restype = ctypes.c_int
        T = P(AttnTensorC)
        h.attn_bwd.argtypes = [T, T, T, T, P(BiasDescC), P(MaskDescC), T, T, T, ctypes.c_void_p,
                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        h.attn_bwd.restype = ctypes.c_int
        h.attn_bwd_opt.argtypes = [T, T, T, T, P(BiasDescC), P(MaskDescC), T, T, T, ctypes.c_void_p,
                                   ctypes.c_int32, P(BwdOptionsC), ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
        h.attn_bwd_opt.restype = ctypes.c_int
        h.attn_bwd_check.argtypes = [T, T, T, T, P(BiasDescC), P(MaskDescC), T, T, T, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
        h.attn_bwd_check.restype = ctypes.c_int
        h.attn_bwd_workspace_size.argtypes = [T, T, T, T, P(BiasDescC), P(MaskDescC), ctypes.c_int32,
                                              P(ctypes.c_size_t)]
        h.attn_bwd_workspace_size.restype = ctypes.c_int
        h.attn_bwd_noalloc.argtypes = [T, T, T, T, P(BiasDescC), P(MaskDescC), T, T, T, ctypes.c_void_p,
                                       ctypes.c_int32, ctypes.c_void_p]
        h.attn_bwd_noalloc.restype = ctypes.c_int
        h.attn_strerror.argtypes = [ctypes.c_int]
        h.attn_strerror.restype = ctypes.c_char_p
        h.attn_version.argtypes = []
        h.attn_version.restype = ctypes.c_int
        _lib_handle = h
    return _lib_handle


# ---------------------------------------------------------------------------
# Python-side descriptions of bias and mask
# ---------------------------------------------------------------------------

@dataclass
class Window:
    img_h: int
    img_w: int
    win_h: int
    win_w: int
    shift_h: int = 0
    shift_w: int = 0

    def c(self) -> WindowC:
        return WindowC(self.img_h, self.img_w, self.win_h, self.win_w, self.shift_h, self.shift_w)


@dataclass
class TableBias:
    """Swin relative-position bias table [(2gh-1)(2gw-1), H]."""
    table: torch.Tensor
    grid: tuple


@dataclass
class RelposBias:
    """SAM decomposed relative position: Rh [2gh-1, d], Rw [2gw-1, d].

    ``kgrid`` (batched layout only): the key grid when it differs from the
    query grid ``grid``; Rh and Rw then need 2*max(gh, kgh)-1 and
    2*max(gw, kgw)-1 rows and the shorter axis is stretched onto the longer.
    Tables of another length (1 to 1023 rows) are resized by the kernel to
    the needed length (linear interpolation, end rows kept).
    """
    rh: torch.Tensor
    rw: torch.Tensor
    grid: tuple
    kgrid: Optional[tuple] = None


@dataclass
class AdditiveBias:
    """Dense additive bias [nB, Nq, Nk]; batch item b uses add[b % nB]."""
    add: torch.Tensor


@dataclass
class ShiftMask:
    """Swin shifted-window region mask (value where regions differ)."""
    window: Window
    value: float = -100.0


@dataclass
class AdditiveMask:
    """Dense additive mask [nW, Nq, Nk]; batch item b uses add[b % nW]."""
    add: torch.Tensor


def _tensor_c(t: torch.Tensor, layout: int) -> AttnTensorC:
    if t.dim() != 4:
        raise ValueError("q, k, v and out must be 4-D [B, H, N, d]")
    if t.stride(3) != 1:
        raise ValueError("the head_dim stride must be 1")
    return AttnTensorC(t.data_ptr(), (ctypes.c_int64 * 4)(*t.shape),
                       (ctypes.c_int64 * 3)(*t.stride()[:3]), layout)


def _descs(bias, mask, layout: int, window: Optional[Window], keep: list):
    bd = BiasDescC()
    if bias is None:
        bd.kind = BIAS_NONE
    elif isinstance(bias, TableBias):
        keep.append(bias.table.contiguous())
        bd.kind, (bd.grid_h, bd.grid_w), bd.table = BIAS_TABLE, bias.grid, keep[-1].data_ptr()
    elif isinstance(bias, RelposBias):
        keep += [bias.rh.contiguous(), bias.rw.contiguous()]
        bd.kind, (bd.grid_h, bd.grid_w) = BIAS_RELPOS, bias.grid
        if bias.kgrid is not None:
            bd.kgrid_h, bd.kgrid_w = bias.kgrid
        bd.rh, bd.rw = keep[-2].data_ptr(), keep[-1].data_ptr()
        bd.rh_rows, bd.rw_rows = bias.rh.shape[0], bias.rw.shape[0]
    elif isinstance(bias, AdditiveBias):
        a = bias.add if bias.add.dim() == 3 else bias.add.reshape(-1, *bias.add.shape[-2:])
        if a.stride(2) != 1:
            a = a.contiguous()
        keep.append(a)
        bd.kind, bd.add, bd.add_batch = BIAS_ADDITIVE, a.data_ptr(), a.shape[0]
        bd.add_strides[0], bd.add_strides[1] = a.stride(0), a.stride(1)
    else:
        raise TypeError(f"unknown bias {type(bias).__name__}")

    md = MaskDescC()
    md.value = -100.0
    if mask is None:
        md.kind = MASK_NONE
    elif isinstance(mask, ShiftMask):
        md.kind, md.value = MASK_SHIFT_REGIONS, mask.value
        window = window or mask.window
    elif isinstance(mask, AdditiveMask):
        a = mask.add if mask.add.dim() == 3 else mask.add.reshape(-1, *mask.add.shape[-2:])
        if a.stride(2) != 1:
            a = a.contiguous()
        keep.append(a)
        md.kind, md.add, md.n_win = MASK_ADDITIVE, a.data_ptr(), a.shape[0]
        md.add_strides[0], md.add_strides[1] = a.stride(0), a.stride(1)
    else:
        raise TypeError(f"unknown mask {type(mask).__name__}")
    if window is not None:
        md.win = window.c()
    return bd, md


def _check_extents(q, k, bias, mask, lay, window):
    """Shapes of the tables and dense tensors the kernel will index."""
    H, D = q.shape[1], q.shape[3]
    win = window or (mask.window if isinstance(mask, ShiftMask) else None)
    if lay == LAYOUT_IMAGE:
        if win is None:
            raise ValueError("image layout needs a window geometry")
        nq = nk = win.win_h * win.win_w
    else:
        nq, nk = q.shape[2], k.shape[2]
    if isinstance(bias, TableBias):
        gh, gw = bias.grid
        if tuple(bias.table.shape) != ((2 * gh - 1) * (2 * gw - 1), H):
            raise ValueError(f"table must be [{(2 * gh - 1) * (2 * gw - 1)}, {H}]")
    elif isinstance(bias, RelposBias):
        gh, gw = bias.grid
        if bias.rh.dim() != 2 or bias.rw.dim() != 2 or bias.rh.shape[1] != D or bias.rw.shape[1] != D:
            raise ValueError(f"rh, rw must be [rows, {D}]")
        if not (1 <= bias.rh.shape[0] <= 1023 and 1 <= bias.rw.shape[0] <= 1023):
            raise ValueError("rh, rw must hold 1 to 1023 rows")
    elif isinstance(bias, AdditiveBias):
        if tuple(bias.add.shape[-2:]) != (nq, nk):
            raise ValueError(f"additive bias must end in [{nq}, {nk}]")
    if isinstance(mask, AdditiveMask) and tuple(mask.add.shape[-2:]) != (nq, nk):
        raise ValueError(f"additive mask must end in [{nq}, {nk}]")


def _marshal(q, k, v, out, bias, mask, layout, window, e4m3: bool = False):
    """Descriptors of a call.  The compute dtype is out's; q, k, v have it
    too, or are E4M3 codes (uint8 or float8_e4m3fn) when ``e4m3``."""
    lay = {"batched": LAYOUT_BATCHED, "image": LAYOUT_IMAGE}[layout]
    if out.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {out.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if e4m3 and t.dtype not in E4M3_DTYPES:
            raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), not {t.dtype}")
        if not e4m3 and t.dtype != out.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, out has {out.dtype}")
    keep: list = []
    bd, md = _descs(bias, mask, lay, window, keep)
    for t in keep:
        if t.dtype != out.dtype:
            raise TypeError("bias/mask tensors must have the compute dtype")
        if t.device != q.device:
            raise ValueError("bias/mask tensors must be on the device of q")
    _check_extents(q, k, bias, mask, lay, window)
    return (_tensor_c(q, lay), _tensor_c(k, lay), _tensor_c(v, lay), bd, md,
            _tensor_c(out, lay), DTYPES[out.dtype], keep)


def _options(window_heads: Optional[int], qkv_descale=None, lse=None):
    if window_heads is None and qkv_descale is None and lse is None:
        return None
    o = OptionsC()
    o.window_heads = int(window_heads or 0)
    if qkv_descale is not None:
        o.qkv_format = QKV_E4M3
        o.q_descale, o.k_descale, o.v_descale = (float(x) for x in qkv_descale)
    if lse is not None:
        o.lse = lse.data_ptr()
    return ctypes.byref(o)


def _check_lse(lse, q):
    if lse is None:
        return
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise TypeError(f"lse must be a contiguous float32 tensor of shape {tuple(q.shape[:3])}")
    if lse.device != q.device:
        raise ValueError("lse must be on the device of q")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias=None, mask=None,
        out: Optional[torch.Tensor] = None, layout: str = "batched",
        window: Optional[Window] = None, stream=None,
        window_heads: Optional[int] = None, qkv_descale=None,
        out_dtype: torch.dtype = torch.float16, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = softmax(QK^T/sqrt(d) + bias + mask) V on the GPU via libattn.

    q: [B, H, Nq, d], k, v: [B, H, Nk, d] CUDA (HIP) tensors, last stride 1.
    layout "image": tensors are [B_img, H, img_h*img_w, d] and ``window`` (or
    the ShiftMask's window) gives the window geometry.  ``out`` may be given;
    otherwise it is allocated with torch.  Queued on ``stream`` (default:
    torch's current stream; a ``torch.cuda.Stream`` or a raw hipStream_t
    handle), with no host synchronisation.  ``window_heads`` (windows of at
    most 64 tokens): heads of one window per workgroup (None or 0: the
    library's choice), passed to attn_fwd_opt.  On another stream than the current
    one, the kernel is ordered after the work already queued on the current
    stream (where this function makes its temporaries), and those
    temporaries stay allocated until the kernel's stream has run it.

    ``qkv_descale`` = (q scale, k scale, v scale): q, k and v are E4M3 codes
    (uint8 or float8_e4m3fn tensors) standing for code * scale; the compute
    and output dtype is then ``out``'s, or ``out_dtype`` (f16 or bf16) when
    ``out`` is allocated here, and the tables must have it.  ``lse``: an
    optional float32 tensor [B, H, N] (q's first three dims) that receives
    each query row's log-sum-exp of its logits (natural log), for ``bwd``.
    """
    h = lib()
    e4m3 = qkv_descale is not None
    allocated = out is None
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype if e4m3 else q.dtype, device=q.device)
    if q.numel() == 0 and k.dim() == 4 and k.shape[2] > 0:
        # No query rows (or no batch items or heads): nothing to compute, and
        # the library, which takes only non-empty tensors, is not called.
        # Zero keys with queries present stay an error (a softmax over no
        # keys is undefined): the library rejects them.
        return out
    qc, kc, vc, bd, md, oc, dt, keep = _marshal(q, k, v, out, bias, mask, layout, window, e4m3)
    _check_lse(lse, q)
    cur = torch.cuda.current_stream(q.device)
    if stream is None:
        s_obj = cur
    elif isinstance(stream, torch.cuda.Stream):
        s_obj = stream
    else:  # a raw hipStream_t handle
        s_obj = torch.cuda.ExternalStream(int(stream), device=q.device)
    if s_obj != cur:
        # The temporaries above (contiguous copies of tables and dense terms,
        # and ``out`` when allocated here) were made on the current stream:
        # the kernel's stream waits for them, and the caching allocator keeps
        # their memory until the kernel's stream has passed this point.
        ev = torch.cuda.Event()
        ev.record(cur)
        s_obj.wait_event(ev)
        for t in keep + ([out] if allocated else []):
            t.record_stream(s_obj)
    st = h.attn_fwd_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                        ctypes.byref(md), ctypes.byref(oc), dt, _options(window_heads, qkv_descale, lse),
                        ctypes.c_void_p(s_obj.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, h.attn_strerror(st).decode())
    del keep
    return out


def check(q, k, v, bias=None, mask=None, out=None, layout: str = "batched",
          window: Optional[Window] = None, window_heads: Optional[int] = None,
          qkv_descale=None, out_dtype: torch.dtype = torch.float16, lse=None) -> int:
    """Status attn_fwd would return for these arguments (no GPU needed)."""
    h = lib()
    e4m3 = qkv_descale is not None
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype if e4m3 else q.dtype, device=q.device)
    qc, kc, vc, bd, md, oc, dt, keep = _marshal(q, k, v, out, bias, mask, layout, window, e4m3)
    opts = _options(window_heads, qkv_descale, lse)
    if opts is None:
        return h.attn_check(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                            ctypes.byref(md), ctypes.byref(oc), dt)
    return h.attn_check_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(bd),
                            ctypes.byref(md), ctypes.byref(oc), dt, opts)


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, bias=None, mask=None,
        layout: str = "batched", window: Optional[Window] = None, dq=None, dk=None, dv=None,
        dtable=None, workspace=None, stream=None, no_alloc: bool = False,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Gradients of sum(dout * O) for O = fwd(q, k, v, bias, mask) via attn_bwd.

    Returns (dq, dk, dv, dtable): dtable is fp32 [table rows, H] with a
    TableBias, the pair (dRh, dRw) (fp32 views [rows, d] of one
    [Rh rows + Rw rows, d] buffer) with a RelposBias, else None.  A given
    ``dtable`` must be that buffer.  Output and workspace tensors are allocated with
    torch when not given; the library itself allocates nothing.  Queued on
    ``stream`` (default: torch's current stream).  ``no_alloc``: call
    attn_bwd_noalloc (the library's fixed device array instead of a
    workspace; ``workspace`` is then ignored and none is allocated).  On a
    stream other than torch's current one, the kernels are ordered after the
    work queued on the current stream and the tensors made or passed here
    stay allocated until the kernels' stream has run them.  ``out`` and
    ``lse``: the forward's output and log-sum-exp (``fwd(..., lse=...)``),
    passed to attn_bwd_opt so the tiled path skips its statistics pass.
    """
    h = lib()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    qc, kc, vc, bd, md, oc, dt, keep = _marshal(q, k, v, dout, bias, mask, layout, window)
    lay = {"batched": LAYOUT_BATCHED, "image": LAYOUT_IMAGE}[layout]
    dqc, dkc, dvc = _tensor_c(dq, lay), _tensor_c(dk, lay), _tensor_c(dv, lay)
    if isinstance(bias, TableBias) and dtable is None:
        dtable = torch.empty(bias.table.shape, dtype=torch.float32, device=q.device)
    if isinstance(bias, RelposBias) and dtable is None:
        dtable = torch.empty(bias.rh.shape[0] + bias.rw.shape[0], q.shape[3], dtype=torch.float32,
                             device=q.device)
    if dtable is not None and (dtable.dtype != torch.float32 or not dtable.is_contiguous()):
        raise TypeError("dtable must be a contiguous float32 tensor")
    # Temporaries made here (contiguous table copies, outputs and workspace
    # allocated here) live on torch's current stream: a kernel queued on
    # another stream waits for them, and they stay allocated until that
    # stream has run it (as in fwd).
    cur = torch.cuda.current_stream(q.device)
    if stream is None:
        s_obj = cur
    elif isinstance(stream, torch.cuda.Stream):
        s_obj = stream
    else:  # a raw hipStream_t handle
        s_obj = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)), device=q.device)
    stream = s_obj.cuda_stream
    side = s_obj != cur

    def order_temporaries(extra):
        if side:
            ev = torch.cuda.Event()
            ev.record(cur)
            s_obj.wait_event(ev)
            for t in keep + [x for x in extra if x is not None]:
                t.record_stream(s_obj)

    if no_alloc:
        order_temporaries([dq, dk, dv, dtable])
        st = h.attn_bwd_noalloc(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc),
                                ctypes.byref(bd), ctypes.byref(md), ctypes.byref(dqc), ctypes.byref(dkc),
                                ctypes.byref(dvc), ctypes.c_void_p(dtable.data_ptr() if dtable is not None else 0),
                                dt, ctypes.c_void_p(stream))
        if st != ATTN_OK:
            raise AttnError(st, h.attn_strerror(st).decode())
        del keep
        return dq, dk, dv, _table_grads(bias, dtable)
    need = ctypes.c_size_t(0)
    st = h.attn_bwd_workspace_size(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc),
                                   ctypes.byref(bd), ctypes.byref(md), dt, ctypes.byref(need))
    if st != ATTN_OK:
        raise AttnError(st, h.attn_strerror(st).decode())
    if workspace is None and need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    order_temporaries([dq, dk, dv, dtable, workspace])
    bopt = None
    if out is not None or lse is not None:
        if out is None or lse is None:
            raise ValueError("out and lse are given together")
        _check_lse(lse, q)
        foc = _tensor_c(out, lay)
        bo = BwdOptionsC()
        bo.out, bo.lse = ctypes.addressof(foc), lse.data_ptr()
        bopt = ctypes.byref(bo)
        if side:
            out.record_stream(s_obj)
            lse.record_stream(s_obj)
    st = h.attn_bwd_opt(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), ctypes.byref(oc), ctypes.byref(bd),
                        ctypes.byref(md), ctypes.byref(dqc), ctypes.byref(dkc), ctypes.byref(dvc),
                        ctypes.c_void_p(dtable.data_ptr() if dtable is not None else 0), dt, bopt,
                        ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0),
                        ctypes.c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
                        ctypes.c_void_p(stream))
    if st != ATTN_OK:
        raise AttnError(st, h.attn_strerror(st).decode())
    del keep
    return dq, dk, dv, _table_grads(bias, dtable)


def _table_grads(bias, dtable):
    if isinstance(bias, TableBias):
        return dtable
    if isinstance(bias, RelposBias):
        nh = bias.rh.shape[0]
        return dtable[:nh], dtable[nh:]
    return None
