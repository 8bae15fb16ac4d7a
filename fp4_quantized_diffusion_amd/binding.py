"""ctypes binding of libfp4rollout.so (the C ABI in include/fp4rollout.h).

Two layers, argument marshalling only -- every step of the path runs in the
library's HIP kernels:
  * the raw entry points under their C names (fp4_quantize, fp4_quantize_lora, fp4_quantize_nv_grouped,
    fp4_panel_bytes, fp4_gemm_nv_grouped,
    fp4_gemm, fp4_gemm_panel, fp4_gemm_panel_gelu, fp4_gemm_panel_gelu_f32, fp4_gemm_panel_euler,
    fp4_gemm_panel_euler_reward,
    fp4_gemm_panel_euler_reward_noalloc, euler_step, fp4_proxy_reward,
    select_topk_bottomk), taking integers and device addresses and returning
    the status code;
  * torch-tensor helpers (quantize, quantize_lora, quantize_nv_grouped, gemm, gemm_gelu, gemm_euler, gemm_euler_reward,
    gemm_euler_reward_noalloc, euler,
    proxy_reward, select) that
    allocate outputs with torch, pass data_ptr()s and the current HIP stream,
    and raise Fp4Error on a non-zero status.
Loading fails loudly when the library has not been built; there is no
fallback path.
"""
import ctypes
import os
from typing import NamedTuple, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4rollout.so")

FMT_MX, FMT_NV = 0, 1
DT_F32, DT_BF16 = 0, 1
PRO_RMSNORM, PRO_GELU, TENSOR_SCALE_GIVEN, LAYOUT_PANEL = 0x1, 0x2, 0x100, 0x200
OK, INVALID_ARGUMENT, UNSUPPORTED, DEVICE_ERROR, INTERNAL = 0, 1, 2, 3, 4

_LIB = None

_i32, _i64, _f32, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_SIGS = {
    "fp4_quantize": [_i32, _p, _i32, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i32, _p],
    "fp4_quantize_lora": [_i32, _p, _i32, _i64, _i64, _i64, _p, _i64, _p, _i64, _i32, _i64, _f32, _p, _i64, _p, _i64,
                          _p, _i32, _p],
    "fp4_quantize_nv_grouped": [_p, _i32, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i32, _p],
    "fp4_panel_bytes": [_i64, _i64, _p, _p],
    "fp4_gemm": [_i32, _p, _i64, _p, _i64, _p, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _p, _i32, _i64, _p, _p],
    "fp4_gemm_nv_grouped": [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _p, _i32, _i64,
                            _p, _p],
    "fp4_gemm_panel": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _i64, _p, _p],
    "fp4_gemm_panel_gelu": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p],
    "fp4_gemm_panel_gelu_f32": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p],
    "fp4_gemm_panel_euler": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _f32, _f32, _p],
    "fp4_gemm_panel_euler_reward": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _f32, _f32, _p, _i64,
                                    _p, _p, _p],
    "fp4_gemm_panel_euler_reward_noalloc": [_i32, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _f32, _f32, _p,
                                            _i64, _p, _p],
    "euler_step": [_p, _p, _p, _i32, _i64, _f32, _f32, _p],
    "fp4_proxy_reward": [_p, _i64, _i64, _i64, _i64, _p, _p, _p],
    "select_topk_bottomk": [_p, _i64, _i64, _i64, _p, _p, _p, _p],
    "fp4_nft_noise": [_p, _p, _p, _i64, _i64, _p, _p],
    "fp4_nft_loss": [_p, _p, _p, _p, _p, _f32, _i64, _i64, _p, _p, _p, _p],
}
EXPORTS = tuple(_SIGS) + ("fp4_status_str", "fp4_abi_version")


class Fp4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_str(status)})")


def load_library(path=LIB_PATH):
    global _LIB
    if _LIB is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m fp4_quantized_diffusion_amd.build` "
                               "(the FP4 path has no fallback)")
        lib = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        lib.fp4_status_str.argtypes = [ctypes.c_int32]
        lib.fp4_status_str.restype = ctypes.c_char_p
        lib.fp4_abi_version.argtypes = []
        lib.fp4_abi_version.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def status_str(s):
    return load_library().fp4_status_str(int(s)).decode()


# ---------------------------------------------------------------- raw C names
def fp4_quantize(fmt, x, x_dtype, rows, k, ldx, codes, ld_codes, scales, ld_scales, tensor_scale, flags, stream):
    return load_library().fp4_quantize(fmt, x, x_dtype, rows, k, ldx, codes, ld_codes, scales, ld_scales,
                                       tensor_scale, flags, stream)


def fp4_quantize_lora(fmt, w, w_dtype, rows, k, ldw, lora_b, ld_b, lora_a, ld_a, ab_dtype, rank, scale, codes,
                      ld_codes, scales, ld_scales, tensor_scale, flags, stream):
    return load_library().fp4_quantize_lora(fmt, w, w_dtype, rows, k, ldw, lora_b, ld_b, lora_a, ld_a, ab_dtype,
                                            rank, scale, codes, ld_codes, scales, ld_scales, tensor_scale, flags,
                                            stream)


def fp4_gemm(fmt, a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs, b_ts, m, n, k, c, c_dtype,
             ldc, residual, stream):
    return load_library().fp4_gemm(fmt, a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs, b_ts,
                                   m, n, k, c, c_dtype, ldc, residual, stream)


def fp4_quantize_nv_grouped(x, x_dtype, rows, k, ldx, rows_per_group, codes, ld_codes, scales, ld_scales,
                            tensor_scales, flags, stream):
    return load_library().fp4_quantize_nv_grouped(x, x_dtype, rows, k, ldx, rows_per_group, codes, ld_codes, scales,
                                                  ld_scales, tensor_scales, flags, stream)


def fp4_gemm_nv_grouped(a_codes, lda, a_scales, ld_as, a_ts, a_rows_per_group, b_codes, ldb, b_scales, ld_bs, b_ts,
                        m, n, k, c, c_dtype, ldc, residual, stream):
    return load_library().fp4_gemm_nv_grouped(a_codes, lda, a_scales, ld_as, a_ts, a_rows_per_group, b_codes, ldb,
                                              b_scales, ld_bs, b_ts, m, n, k, c, c_dtype, ldc, residual, stream)


def fp4_panel_bytes(rows, k, code_bytes, scale_bytes):
    """code_bytes / scale_bytes: addresses of host int64s (ctypes.byref)."""
    return load_library().fp4_panel_bytes(rows, k, code_bytes, scale_bytes)


def fp4_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, c, c_dtype, ldc, residual, stream):
    return load_library().fp4_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, c, c_dtype, ldc,
                                         residual, stream)


def fp4_gemm_panel_gelu(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes, out_scales, stream):
    return load_library().fp4_gemm_panel_gelu(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes,
                                              out_scales, stream)


def fp4_gemm_panel_gelu_f32(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes, out_scales, stream):
    return load_library().fp4_gemm_panel_gelu_f32(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes,
                                                  out_scales, stream)


def fp4_gemm_panel_euler(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, residual, x, x_out, ldx, t_cur, t_next,
                         stream):
    return load_library().fp4_gemm_panel_euler(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, residual, x,
                                               x_out, ldx, t_cur, t_next, stream)


def fp4_gemm_panel_euler_reward(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, residual, x, x_out, ldx, t_cur,
                                t_next, u, rows_per_cand, partials, rewards, stream):
    return load_library().fp4_gemm_panel_euler_reward(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, residual,
                                                      x, x_out, ldx, t_cur, t_next, u, rows_per_cand, partials,
                                                      rewards, stream)


def fp4_gemm_panel_euler_reward_noalloc(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, residual, x, x_out, ldx,
                                        t_cur, t_next, u, rows_per_cand, rewards, stream):
    return load_library().fp4_gemm_panel_euler_reward_noalloc(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k,
                                                              residual, x, x_out, ldx, t_cur, t_next, u,
                                                              rows_per_cand, rewards, stream)


def euler_step(x_out, x, v, v_dtype, numel, t_cur, t_next, stream):
    return load_library().euler_step(x_out, x, v, v_dtype, numel, t_cur, t_next, stream)


def fp4_proxy_reward(x, n_cand, rows_per_cand, dim, ldx, u, rewards, stream):
    return load_library().fp4_proxy_reward(x, n_cand, rows_per_cand, dim, ldx, u, rewards, stream)


def select_topk_bottomk(rewards, n, k_top, k_bottom, top_idx, bottom_idx, r_norm, stream):
    return load_library().select_topk_bottomk(rewards, n, k_top, k_bottom, top_idx, bottom_idx, r_norm, stream)


def fp4_nft_noise(x0, eps, t, n, d, x_t, stream):
    return load_library().fp4_nft_noise(x0, eps, t, n, d, x_t, stream)


def fp4_nft_loss(v_old, v_theta, x0, eps, r, beta, n, d, partials, terms, loss, stream):
    return load_library().fp4_nft_loss(v_old, v_theta, x0, eps, r, beta, n, d, partials, terms, loss, stream)


def fp4_abi_version():
    return load_library().fp4_abi_version()


# ------------------------------------------------------------- torch helpers
def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(status, what):
    if status != OK:
        raise Fp4Error(status, what)


class QTensor(NamedTuple):
    """A quantized [rows, k] matrix. Row layout: packed codes [rows, >= k/2]
    (row stride a multiple of 16 bytes), scale bytes [rows, k/block], and for
    the NV format the fp32 tensor scale (a 1-element device tensor). Panel
    layout (MX): codes and scales are flat byte tensors in the panel order of
    include/fp4rollout.h, and `rows` gives the row count."""
    codes: object
    scales: object
    tensor_scale: Optional[object]
    fmt: int
    k: int
    layout: str = "row"
    rows: int = 0
    rows_per_group: int = 0  # NV: rows per tensor scale (0: one for all rows)

    @property
    def n_rows(self):
        return self.rows if self.layout == "panel" else self.codes.shape[0]


def _row_view_ok(x):
    return x.dim() == 2 and x.stride(1) == 1


def panel_bytes(rows, k):
    """(code bytes, scale bytes) of the panel layout of a [rows, k] operand."""
    cb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(fp4_panel_bytes(rows, k, ctypes.addressof(cb), ctypes.addressof(sb)), "fp4_panel_bytes")
    return cb.value, sb.value


def _alloc_panel(rows, k, device):
    torch = _torch()
    cb, sb = panel_bytes(rows, k)
    return QTensor(torch.empty(cb, dtype=torch.uint8, device=device), torch.empty(sb, dtype=torch.uint8, device=device),
                   None, FMT_MX, k, "panel", rows)


def _alloc_rows(rows, k, device, f):
    torch = _torch()
    blk = 32 if f == FMT_MX else 16
    ldc = ((k // 2 + 15) // 16) * 16
    codes = torch.empty((rows, ldc), dtype=torch.uint8, device=device)
    # scale rows padded to a multiple of 4 bytes: the GEMM then loads each
    # stage's scale bytes as whole words
    lds = ((max(k // blk, 1) + 3) // 4) * 4
    scales = torch.empty((rows, lds), dtype=torch.uint8, device=device)[:, : max(k // blk, 1)]
    ts = torch.empty(1, dtype=torch.float32, device=device) if f == FMT_NV else None
    return QTensor(codes, scales, ts, f, k)


def quantize(x, fmt="mx", prologue=None, tensor_scale=None, out=None, layout="row"):
    """x: 2-D CUDA tensor (fp32 or bf16, unit inner stride). prologue: None,
    "rmsnorm" or "gelu" (MX only). tensor_scale: a 1-element fp32 tensor whose
    value is used as s_g (NV only). layout: "row" or "panel" (MX only).
    out: a QTensor to write into (its layout wins)."""
    if not _row_view_ok(x):
        raise ValueError("x must be 2-D with unit inner stride")
    f = {"mx": FMT_MX, "nv": FMT_NV}[fmt]
    rows, k = x.shape
    flags = {None: 0, "rmsnorm": PRO_RMSNORM, "gelu": PRO_GELU}[prologue]
    if out is None and layout == "panel":
        out = _alloc_panel(rows, k, x.device)
    if out is not None and out.layout == "panel":
        if out.rows != rows or out.k != k:
            raise ValueError("out was allocated for another shape")
        st = fp4_quantize(f, x.data_ptr(), _dtype_code(x), rows, k, x.stride(0), out.codes.data_ptr(), 0,
                          out.scales.data_ptr(), 0, None, flags | LAYOUT_PANEL, _stream())
        _check(st, "fp4_quantize")
        return out
    if out is None:
        out = _alloc_rows(rows, k, x.device, f)
    ts = out.tensor_scale
    if f == FMT_NV and tensor_scale is not None:
        ts.copy_(tensor_scale.reshape(1))
        flags |= TENSOR_SCALE_GIVEN
    st = fp4_quantize(f, x.data_ptr(), _dtype_code(x), rows, k, x.stride(0), out.codes.data_ptr(),
                      out.codes.stride(0), out.scales.data_ptr(), out.scales.stride(0), _ptr(ts), flags, _stream())
    _check(st, "fp4_quantize")
    return out


def quantize_lora(w, lora_b, lora_a, scale, out=None, layout="row", fmt="mx", tensor_scale=None):
    """QTensor of W + scale * (B A) -- a LoRA adapter merged into the weight in
    fp32 and re-quantized (fp4_quantize_lora), the merged weight never written.
    w: [rows, k] fp32 or bf16; lora_b: [rows, rank] and lora_a: [rank, k] of
    one dtype (fp32 or bf16); all 2-D with unit inner stride. fmt: "mx" or
    "nv"; layout: "row" or "panel" (MX only); tensor_scale: a 1-element fp32
    tensor used as s_g (NV only); out: a QTensor to write into (its layout
    wins)."""
    for t in (w, lora_b, lora_a):
        if not _row_view_ok(t):
            raise ValueError("w, lora_b and lora_a must be 2-D with unit inner stride")
    if lora_b.dtype != lora_a.dtype:
        raise ValueError("lora_b and lora_a must have one dtype")
    f = {"mx": FMT_MX, "nv": FMT_NV}[fmt]
    rows, k = w.shape
    rank = lora_b.shape[1]
    if lora_b.shape[0] != rows or tuple(lora_a.shape) != (rank, k):
        raise ValueError("shapes do not chain: w [rows, k], lora_b [rows, rank], lora_a [rank, k]")
    if out is None:
        out = _alloc_panel(rows, k, w.device) if layout == "panel" else _alloc_rows(rows, k, w.device, f)
    if out.rows not in (0, rows) or out.k != k or out.fmt != f:
        raise ValueError("out was allocated for another shape or format")
    panel = out.layout == "panel"
    flags = LAYOUT_PANEL if panel else 0
    ts = out.tensor_scale
    if f == FMT_NV and tensor_scale is not None:
        ts.copy_(tensor_scale.reshape(1))
        flags |= TENSOR_SCALE_GIVEN
    st = fp4_quantize_lora(f, w.data_ptr(), _dtype_code(w), rows, k, w.stride(0), lora_b.data_ptr(),
                           lora_b.stride(0), lora_a.data_ptr(), lora_a.stride(0), _dtype_code(lora_a), rank,
                           float(scale), out.codes.data_ptr(), 0 if panel else out.codes.stride(0),
                           out.scales.data_ptr(), 0 if panel else out.scales.stride(0), _ptr(ts), flags, _stream())
    _check(st, "fp4_quantize_lora")
    return out


def quantize_nv_grouped(x, rows_per_group, tensor_scales=None, out=None):
    """NVFP4-style QTensor of x [rows, k] (fp32 or bf16) with one tensor scale
    per group of rows_per_group rows (fp4_quantize_nv_grouped); tensor_scales:
    optional fp32 [rows / rows_per_group] to use instead of computing them."""
    torch = _torch()
    if not _row_view_ok(x):
        raise ValueError("x must be 2-D with unit inner stride")
    rows, k = x.shape
    if rows_per_group < 1 or rows % rows_per_group:
        raise ValueError("rows_per_group must divide the row count")
    if out is None:
        out = _alloc_rows(rows, k, x.device, FMT_NV)
        out = out._replace(tensor_scale=torch.empty(rows // rows_per_group, dtype=torch.float32, device=x.device))
    out = out._replace(rows_per_group=rows_per_group)
    flags = 0
    if tensor_scales is not None:
        out.tensor_scale.copy_(tensor_scales.reshape(-1))
        flags = TENSOR_SCALE_GIVEN
    st = fp4_quantize_nv_grouped(x.data_ptr(), _dtype_code(x), rows, k, x.stride(0), rows_per_group,
                                 out.codes.data_ptr(), out.codes.stride(0), out.scales.data_ptr(),
                                 out.scales.stride(0), out.tensor_scale.data_ptr(), flags, _stream())
    _check(st, "fp4_quantize_nv_grouped")
    return out


def gemm(a, b, out_dtype="bf16", residual=None, out=None):
    """C = A_hat B_hat^T (+ residual) for QTensors a [m, k] and b [n, k] of
    one format and one layout."""
    torch = _torch()
    if a.fmt != b.fmt or a.k != b.k or a.layout != b.layout:
        raise ValueError("operands differ in format, layout or k")
    m, n, k = a.n_rows, b.n_rows, a.k
    if out_dtype not in ("bf16", "f32"):
        raise ValueError(f"out_dtype must be 'bf16' or 'f32', not {out_dtype!r}")
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if out is None:
        ldc = ((n + 3) // 4) * 4
        out = torch.empty((m, ldc), dtype=dt, device=a.codes.device)[:, :n]
    if out.dim() != 2 or tuple(out.shape) != (m, n) or out.stride(1) != 1 or out.dtype != dt:
        raise ValueError(f"out must be a [{m}, {n}] {dt} matrix with unit inner stride")
    if residual is not None:
        if out_dtype != "f32":
            raise ValueError("a residual needs fp32 output")
        if (residual.dim() != 2 or tuple(residual.shape) != (m, n) or residual.dtype != torch.float32
                or residual.stride(1) != 1 or residual.stride(0) != out.stride(0)):
            raise ValueError(f"residual must be a [{m}, {n}] fp32 matrix with out's row stride ({out.stride(0)})")
    if a.layout == "panel":
        st = fp4_gemm_panel(a.fmt, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
                            m, n, k, out.data_ptr(), _dtype_code(out), out.stride(0), _ptr(residual), _stream())
        _check(st, "fp4_gemm_panel")
        return out
    if a.rows_per_group:  # NV with one tensor scale per row group of A
        st = fp4_gemm_nv_grouped(a.codes.data_ptr(), a.codes.stride(0), a.scales.data_ptr(), a.scales.stride(0),
                                 a.tensor_scale.data_ptr(), a.rows_per_group, b.codes.data_ptr(), b.codes.stride(0),
                                 b.scales.data_ptr(), b.scales.stride(0), _ptr(b.tensor_scale), m, n, k,
                                 out.data_ptr(), _dtype_code(out), out.stride(0), _ptr(residual), _stream())
        _check(st, "fp4_gemm_nv_grouped")
        return out
    st = fp4_gemm(a.fmt, a.codes.data_ptr(), a.codes.stride(0), a.scales.data_ptr(), a.scales.stride(0),
                  _ptr(a.tensor_scale), b.codes.data_ptr(), b.codes.stride(0), b.scales.data_ptr(),
                  b.scales.stride(0), _ptr(b.tensor_scale), m, n, k, out.data_ptr(), _dtype_code(out),
                  out.stride(0), _ptr(residual), _stream())
    _check(st, "fp4_gemm")
    return out


def gemm_gelu(a, b, out=None, exact=False):
    """MXFP4 panel QTensor of GELU(bf16(A_hat B_hat^T)) for panel-layout
    QTensors a [m, k], b [n, k] (m, n multiples of 256); exact=True takes
    GELU of the fp32 sums instead (fp4_gemm_panel_gelu_f32)."""
    torch = _torch()
    if a.layout != "panel" or b.layout != "panel" or a.k != b.k:
        raise ValueError("gemm_gelu takes panel-layout operands of one k")
    m, n, k = a.n_rows, b.n_rows, a.k
    if out is None:
        cb, sb = panel_bytes(m, n)
        out = QTensor(torch.empty(cb, dtype=torch.uint8, device=a.codes.device),
                      torch.empty(sb, dtype=torch.uint8, device=a.codes.device), None, FMT_MX, n, "panel", m)
    if out.layout != "panel" or out.rows != m or out.k != n:
        raise ValueError("out was allocated for another shape")
    fn = fp4_gemm_panel_gelu_f32 if exact else fp4_gemm_panel_gelu
    st = fn(a.fmt, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
            m, n, k, out.codes.data_ptr(), out.scales.data_ptr(), _stream())
    _check(st, fn.__name__)
    return out


def gemm_euler(a, b, residual, x, t_cur, t_next, out=None):
    """out = x + (t_next - t_cur) (residual + A_hat B_hat^T) for panel-layout
    MXFP4 QTensors a [m, k], b [n, k] and fp32 residual, x [m, n] with unit
    inner stride and a common row stride; out may be x or residual."""
    torch = _torch()
    if a.layout != "panel" or b.layout != "panel" or a.k != b.k:
        raise ValueError("gemm_euler takes panel-layout operands of one k")
    m, n, k = a.n_rows, b.n_rows, a.k
    if out is None:
        out = torch.empty_like(x)
    for t in (residual, x, out):
        if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) != x.stride(0) or tuple(t.shape) != (m, n):
            raise ValueError("residual, x and out must be [m, n] with one row stride")
    st = fp4_gemm_panel_euler(a.fmt, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                              b.scales.data_ptr(), m, n, k, residual.data_ptr(), x.data_ptr(), out.data_ptr(),
                              x.stride(0), float(t_cur), float(t_next), _stream())
    _check(st, "fp4_gemm_panel_euler")
    return out


def gemm_euler_reward(a, b, residual, x, t_cur, t_next, u, rows_per_cand, out=None, rewards=None, partials=None):
    """gemm_euler plus the proxy reward of each candidate (rows_per_cand rows
    each) from the new state: returns (out, rewards). u: fp32 [n]; partials:
    optional fp32 workspace of (m / 256) (n / 256) 4 elements."""
    torch = _torch()
    if a.layout != "panel" or b.layout != "panel" or a.k != b.k:
        raise ValueError("gemm_euler_reward takes panel-layout operands of one k")
    m, n, k = a.n_rows, b.n_rows, a.k
    if out is None:
        out = torch.empty_like(x)
    for t in (residual, x, out):
        if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) != x.stride(0) or tuple(t.shape) != (m, n):
            raise ValueError("residual, x and out must be [m, n] with one row stride")
    if rows_per_cand < 1 or m % rows_per_cand:
        raise ValueError("rows_per_cand must divide m")
    if rewards is None:
        rewards = torch.empty(m // rows_per_cand, dtype=torch.float32, device=x.device)
    need = max(m // 256, 1) * max(n // 256, 1) * 4
    if partials is None or partials.numel() < need:
        partials = torch.empty(need, dtype=torch.float32, device=x.device)
    st = fp4_gemm_panel_euler_reward(a.fmt, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                                     b.scales.data_ptr(), m, n, k, residual.data_ptr(), x.data_ptr(), out.data_ptr(),
                                     x.stride(0), float(t_cur), float(t_next), u.data_ptr(), rows_per_cand,
                                     partials.data_ptr(), rewards.data_ptr(), _stream())
    _check(st, "fp4_gemm_panel_euler_reward")
    return out, rewards


def gemm_euler_reward_noalloc(a, b, residual, x, t_cur, t_next, u, rows_per_cand, out, rewards):
    """gemm_euler_reward into caller-supplied out and rewards, with the
    partial sums in the library's own device array (no workspace, and
    nothing allocated by this call: for use under graph capture)."""
    if a.layout != "panel" or b.layout != "panel" or a.k != b.k:
        raise ValueError("gemm_euler_reward_noalloc takes panel-layout operands of one k")
    m, n, k = a.n_rows, b.n_rows, a.k
    for t in (residual, x, out):
        if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) != x.stride(0) or tuple(t.shape) != (m, n):
            raise ValueError("residual, x and out must be [m, n] with one row stride")
    if rows_per_cand < 1 or m % rows_per_cand or rewards.numel() != m // rows_per_cand:
        raise ValueError("rows_per_cand must divide m, and rewards hold one value per candidate")
    st = fp4_gemm_panel_euler_reward_noalloc(a.fmt, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                                             b.scales.data_ptr(), m, n, k, residual.data_ptr(), x.data_ptr(),
                                             out.data_ptr(), x.stride(0), float(t_cur), float(t_next), u.data_ptr(),
                                             rows_per_cand, rewards.data_ptr(), _stream())
    _check(st, "fp4_gemm_panel_euler_reward_noalloc")
    return out, rewards


def euler(x, v, t_cur, t_next, out=None):
    """x_out = x + (t_next - t_cur) v over contiguous tensors (x fp32)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    if x.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("x and out must be fp32")
    for t in (x, v, out):
        if not t.is_contiguous() or t.numel() != x.numel():
            raise ValueError("x, v and out must be contiguous with one element count")
    st = euler_step(out.data_ptr(), x.data_ptr(), v.data_ptr(), _dtype_code(v), x.numel(), float(t_cur),
                    float(t_next), _stream())
    _check(st, "euler_step")
    return out


def proxy_reward(x, n_cand, rows_per_cand, u=None, out=None):
    """x: [n_cand * rows_per_cand, dim] fp32 (unit inner stride)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.float32:
        raise ValueError("x must be a 2-D fp32 matrix with unit inner stride")
    if x.shape[0] != n_cand * rows_per_cand:
        raise ValueError(f"x has {x.shape[0]} rows, not n_cand * rows_per_cand = {n_cand * rows_per_cand}")
    if u is not None and (u.dtype != torch.float32 or not u.is_contiguous() or u.numel() != x.shape[1]):
        raise ValueError("u must be a contiguous fp32 vector of one entry per column of x")
    if out is None:
        out = torch.empty(n_cand, dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != n_cand:
        raise ValueError("out must be a contiguous fp32 vector of n_cand entries")
    st = fp4_proxy_reward(x.data_ptr(), n_cand, rows_per_cand, x.shape[1], x.stride(0), _ptr(u), out.data_ptr(),
                          _stream())
    _check(st, "fp4_proxy_reward")
    return out


def select(rewards, k_top, k_bottom, normalize=True):
    """Returns (top [k_top] int32, bottom [k_bottom] int32, r_norm or None)."""
    torch = _torch()
    n = rewards.numel()
    top = torch.empty(max(k_top, 1), dtype=torch.int32, device=rewards.device)[:k_top]
    bottom = torch.empty(max(k_bottom, 1), dtype=torch.int32, device=rewards.device)[:k_bottom]
    rn = torch.empty(n, dtype=torch.float32, device=rewards.device) if normalize else None
    st = select_topk_bottomk(rewards.data_ptr(), n, k_top, k_bottom, top.data_ptr(), bottom.data_ptr(), _ptr(rn),
                             _stream())
    _check(st, "select_topk_bottomk")
    return top, bottom, rn


def _samples(*ts):
    n = ts[0].shape[0]
    for t in ts:
        if not t.is_contiguous() or t.shape[0] != n or t.numel() != ts[0].numel():
            raise ValueError("arrays must be contiguous with one shape [n, ...]")
    return n, ts[0].numel() // n


def nft_noise(x0, eps, t, out=None):
    """x_t = (1 - t) x0 + t eps per sample (fp4_nft_noise); x0, eps fp32
    [n, ...] contiguous, t fp32 [n]."""
    torch = _torch()
    n, d = _samples(x0, eps)
    if out is None:
        out = torch.empty_like(x0)
    _check(fp4_nft_noise(x0.data_ptr(), eps.data_ptr(), t.data_ptr(), n, d, out.data_ptr(), _stream()),
           "fp4_nft_noise")
    return out


def nft_loss(v_old, v_theta, x0, eps, r, beta):
    """DiffusionNFT loss (fp4_nft_loss): returns (loss [1], terms [n]) as fp32
    tensors; all inputs fp32 contiguous [n, ...], r fp32 [n]."""
    torch = _torch()
    n, d = _samples(v_old, v_theta, x0, eps)
    partials = torch.empty(n * 128, dtype=torch.float32, device=x0.device)
    terms = torch.empty(n, dtype=torch.float32, device=x0.device)
    loss = torch.empty(1, dtype=torch.float32, device=x0.device)
    _check(fp4_nft_loss(v_old.data_ptr(), v_theta.data_ptr(), x0.data_ptr(), eps.data_ptr(), r.data_ptr(),
                        float(beta), n, d, partials.data_ptr(), terms.data_ptr(), loss.data_ptr(), _stream()),
           "fp4_nft_loss")
    return loss, terms
