"""Python binding of libdg (fine-grained-scaled FP8 GEMM for MI355X / gfx950).

Argument marshalling only: every function here checks tensor devices, dtypes
and shapes, then calls the C entry point of the same name with raw device
pointers and the current HIP stream.  All computation happens in the HIP
kernels of libdg.so; there is no fallback.  Importing this package fails if
the library has not been built (see build.py).

Tensor conventions (torch dtypes standing in for the C types):
  e4m3 codes     torch.uint8       bf16 values  torch.bfloat16 (or int16 bits)
  fp32 scales    torch.float32     ids/counts   torch.int32
  UE8M0 scales   torch.uint8 (exponent bytes, 2^(E-127))
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libdg.so is not built ({LIB_PATH}); run moe_grouped_gemm_02_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_S = ctypes.c_size_t

_SIGNATURES = {
    "dg_fp8_gemm_nt": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_nt_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P]),
    "dg_grouped_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _P, _S, _P]),
    "dg_grouped_masked": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _P, _S, _P]),
    "dg_fp8_gemm_nt_ue8m0": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_grouped_contiguous_ue8m0": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _P, _S, _P]),
    "dg_grouped_masked_ue8m0": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _P, _S, _P]),
    "dg_fp8_gemm_nt_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _L, _P, _S, _P]),
    "dg_grouped_contiguous_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _P, _S, _P]),
    "dg_grouped_masked_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_nt_ue8m0_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _L, _P, _S, _P]),
    "dg_grouped_contiguous_ue8m0_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _P, _S, _P]),
    "dg_grouped_masked_ue8m0_qout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _P, _S, _P]),
    "dg_k_grouped_nt": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_nn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_tn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_tt": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_quant_1x128": (_I, [_P, _P, _P, _I, _I, _L, _I, _P]),
    "dg_quant_1x128_mn": (_I, [_P, _P, _P, _I, _I, _L, _P]),
    "dg_quant_1x128_mn_ue8m0": (_I, [_P, _P, _P, _I, _I, _L, _P]),
    "dg_fp8_gemm_nn_ue8m0": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_tn_ue8m0": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_fp8_gemm_tt_ue8m0": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _L, _P, _S, _P]),
    "dg_quant_128x128": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "dg_quant_1x128_ue8m0": (_I, [_P, _P, _P, _I, _I, _L, _I, _P]),
    "dg_quant_128x128_ue8m0": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "dg_get_ue8m0_sfb_leading_dim": (_L, [_I]),
    "dg_get_workspace_size": (_S, [_I, _I, _I, _I]),
    "dg_get_num_cus": (_I, []),
    "dg_set_num_cus": (_I, [_I]),
    "dg_get_m_alignment_for_contiguous_layout": (_I, []),
    "dg_get_sf_leading_dim": (_L, [_I]),
    "dg_get_last_error_string": (ctypes.c_char_p, []),
    "dg_describe_config": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.c_char_p, _S]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGNATURES)

LAYOUT_DENSE, LAYOUT_CONTIGUOUS, LAYOUT_MASKED, LAYOUT_K_GROUPED = 0, 1, 2, 3


class DGError(RuntimeError):
    """A libdg call returned a negative status."""

    def __init__(self, fn, status):
        msg = _lib.dg_get_last_error_string().decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise DGError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _expect(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")


_U8 = (torch.uint8, torch.float8_e4m3fn)
_BF = (torch.bfloat16, torch.int16)


def _row_major(t, name):
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------ GEMMs --
#
# Each GEMM and quantiser has an fp32-scale form and a UE8M0 form (power-of-two
# scales stored as exponent bytes).  Scale shapes:
#   fp32:  sfa [(G)][K/128][ld] float32,  sfb [(G)][ceil(N/128)][K/128] float32
#   UE8M0: sfa [(G)][K/128][ld] uint8,    sfb [(G)][K/128][ld_sfb] uint8,
#          ld_sfb = dg_get_ue8m0_sfb_leading_dim(N)


def _ue8m0_sfb_ld(n):
    return ((n + 127) // 128 + 3) // 4 * 4


def _sf_dtype(ue8m0):
    return (torch.uint8,) if ue8m0 else (torch.float32,)


def _sfb_shape(n, k, ue8m0):
    return (k // 128, _ue8m0_sfb_ld(n)) if ue8m0 else ((n + 127) // 128, k // 128)


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _gemm_nt(fn, a, sfa, b, sfb, d, workspace, ue8m0):
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 2), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 2), _expect(sfb, "sfb", _sf_dtype(ue8m0), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != _sfb_shape(n, k, ue8m0):
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {_sfb_shape(n, k, ue8m0)}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa")):
        _row_major(t, nm)
    _contig(sfb, "sfb")
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, a.stride(0), b.stride(0),
        d.stride(0), sfa.stride(0), _ptr(workspace), _ws(workspace), _stream(d)))
    return d


def _contiguous(fn, a, sfa, b, sfb, d, m_indices, workspace, ue8m0):
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 3), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 2), _expect(sfb, "sfb", _sf_dtype(ue8m0), 3)
    _expect(m_indices, "m_indices", (torch.int32,), 1)
    m_total, k = a.shape
    groups, n = b.shape[0], b.shape[1]
    if b.shape[2] != k or tuple(d.shape) != (m_total, n) or m_indices.shape[0] != m_total:
        raise ValueError("shape mismatch between a, b, d and m_indices")
    want_b = (groups,) + _sfb_shape(n, k, ue8m0)
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != want_b:
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {want_b}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfb, "sfb"), (m_indices, "m_indices")):
        _contig(t, nm)
    _row_major(sfa, "sfa")
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(m_indices), m_total, n, k,
        groups, sfa.stride(0), _ptr(workspace), _ws(workspace), _stream(d)))
    return d


def _masked(fn, a, sfa, b, sfb, d, masked_m, expected_m, workspace, ue8m0):
    _expect(a, "a", _U8, 3), _expect(b, "b", _U8, 3), _expect(d, "d", _BF, 3)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 3), _expect(sfb, "sfb", _sf_dtype(ue8m0), 3)
    _expect(masked_m, "masked_m", (torch.int32,), 1)
    groups, m_max, k = a.shape
    n = b.shape[1]
    if b.shape[0] != groups or b.shape[2] != k or tuple(d.shape) != (groups, m_max, n):
        raise ValueError("shape mismatch between a, b and d")
    if masked_m.shape[0] != groups:
        raise ValueError("masked_m must have one entry per group")
    want_b = (groups,) + _sfb_shape(n, k, ue8m0)
    if sfa.shape[:2] != (groups, k // 128) or tuple(sfb.shape) != want_b:
        raise ValueError(f"scale shapes must be sfa [G][K/128][ld] and sfb {want_b}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa"), (sfb, "sfb"), (masked_m, "masked_m")):
        _contig(t, nm)
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(masked_m), groups, m_max, n, k,
        int(expected_m), sfa.shape[2], _ptr(workspace), _ws(workspace), _stream(d)))
    return d


def dg_fp8_gemm_nt(a, sfa, b, sfb, d, workspace=None):
    """d[m][n] = bf16(A . B^T) with 1x128 (sfa [K/128][ld]) and 128x128 scales."""
    return _gemm_nt("dg_fp8_gemm_nt", a, sfa, b, sfb, d, workspace, False)


def dg_fp8_gemm_nt_noalloc(a, sfa, b, sfb, d):
    """dg_fp8_gemm_nt with the library's own per-GPU scratch instead of a
    workspace (allocates nothing; calls on one GPU must not overlap)."""
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 2), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(False), 2), _expect(sfb, "sfb", _sf_dtype(False), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != _sfb_shape(n, k, False):
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {_sfb_shape(n, k, False)}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa")):
        _row_major(t, nm)
    _contig(sfb, "sfb")
    _check("dg_fp8_gemm_nt_noalloc", _lib.dg_fp8_gemm_nt_noalloc(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, a.stride(0), b.stride(0),
        d.stride(0), sfa.stride(0), _stream(d)))
    return d


def dg_fp8_gemm_nt_ue8m0(a, sfa, b, sfb, d, workspace=None):
    """dg_fp8_gemm_nt with exponent-byte scales (sfb [K/128][ld_sfb] uint8)."""
    return _gemm_nt("dg_fp8_gemm_nt_ue8m0", a, sfa, b, sfb, d, workspace, True)


def _gemm_majors(fn, a_mn, b_mn, a, sfa, b, sfb, d, workspace, ue8m0=False):
    """Dense GEMM whose A is stored [K][M] (a_mn) and/or B [K][N] (b_mn)."""
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 2), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 2), _expect(sfb, "sfb", _sf_dtype(ue8m0), 2)
    k, m = a.shape if a_mn else a.shape[::-1]
    kb_, n = b.shape if b_mn else b.shape[::-1]
    if kb_ != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != _sfb_shape(n, k, ue8m0):
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {_sfb_shape(n, k, ue8m0)}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa")):
        _row_major(t, nm)
    _contig(sfb, "sfb")
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), m, n, k, a.stride(0), b.stride(0),
        d.stride(0), sfa.stride(0), _ptr(workspace), _ws(workspace), _stream(d)))
    return d


def dg_fp8_gemm_nn(a, sfa, b, sfb, d, workspace=None):
    """d[m][n] = bf16(A . B) with a [M][K] and b stored [K][N] (N-major); NT scale layouts."""
    return _gemm_majors("dg_fp8_gemm_nn", False, True, a, sfa, b, sfb, d, workspace)


def dg_fp8_gemm_tn(a, sfa, b, sfb, d, workspace=None):
    """d[m][n] = bf16(A^T . B) with a stored [K][M] and b stored [K][N]; NT scale layouts."""
    return _gemm_majors("dg_fp8_gemm_tn", True, True, a, sfa, b, sfb, d, workspace)


def dg_fp8_gemm_tt(a, sfa, b, sfb, d, workspace=None):
    """d[m][n] = bf16(A^T . B^T) with a stored [K][M] and b [N][K]; NT scale layouts."""
    return _gemm_majors("dg_fp8_gemm_tt", True, False, a, sfa, b, sfb, d, workspace)


def dg_fp8_gemm_nn_ue8m0(a, sfa, b, sfb, d, workspace=None):
    """dg_fp8_gemm_nn with exponent-byte scales (sfb [K/128][ld_sfb] uint8)."""
    return _gemm_majors("dg_fp8_gemm_nn_ue8m0", False, True, a, sfa, b, sfb, d, workspace, True)


def dg_fp8_gemm_tn_ue8m0(a, sfa, b, sfb, d, workspace=None):
    """dg_fp8_gemm_tn with exponent-byte scales."""
    return _gemm_majors("dg_fp8_gemm_tn_ue8m0", True, True, a, sfa, b, sfb, d, workspace, True)


def dg_fp8_gemm_tt_ue8m0(a, sfa, b, sfb, d, workspace=None):
    """dg_fp8_gemm_tt with exponent-byte scales."""
    return _gemm_majors("dg_fp8_gemm_tt_ue8m0", True, False, a, sfa, b, sfb, d, workspace, True)


def dg_grouped_contiguous(a, sfa, b, sfb, d, m_indices, workspace=None):
    """Contiguous grouped GEMM; b [G][N][K], m_indices [M_total] int32."""
    return _contiguous("dg_grouped_contiguous", a, sfa, b, sfb, d, m_indices, workspace, False)


def dg_grouped_contiguous_ue8m0(a, sfa, b, sfb, d, m_indices, workspace=None):
    """dg_grouped_contiguous with exponent-byte scales (sfb [G][K/128][ld_sfb])."""
    return _contiguous("dg_grouped_contiguous_ue8m0", a, sfa, b, sfb, d, m_indices, workspace, True)


def dg_grouped_masked(a, sfa, b, sfb, d, masked_m, expected_m=0, workspace=None):
    """Masked grouped GEMM; a [G][M_max][K], sfa [G][K/128][ld], masked_m [G] int32."""
    return _masked("dg_grouped_masked", a, sfa, b, sfb, d, masked_m, expected_m, workspace, False)


def dg_grouped_masked_ue8m0(a, sfa, b, sfb, d, masked_m, expected_m=0, workspace=None):
    """dg_grouped_masked with exponent-byte scales (sfb [G][K/128][ld_sfb])."""
    return _masked("dg_grouped_masked_ue8m0", a, sfa, b, sfb, d, masked_m, expected_m, workspace, True)


def _check_qout(dq, dsf, rows_shape, n, grouped, ue8m0=False):
    """dq e4m3 [(G)][rows][n] contiguous, dsf [(G)][n/128][ld] (fp32, or uint8
    exponents with ue8m0); returns ld."""
    _expect(dq, "dq", _U8, len(rows_shape) + 1), _expect(dsf, "dsf", _sf_dtype(ue8m0), len(rows_shape) + 1)
    if tuple(dq.shape) != tuple(rows_shape) + (n,):
        raise ValueError(f"dq must have shape {tuple(rows_shape) + (n,)}")
    want = ((rows_shape[0],) if grouped else ()) + (n // 128,)
    if tuple(dsf.shape[:-1]) != want:
        raise ValueError(f"dsf must be {want} + (ld,)")
    _contig(dq, "dq"), _contig(dsf, "dsf")
    return dsf.shape[-1]


def _gemm_nt_qout(fn, a, sfa, b, sfb, d, dq, dsf, workspace, ue8m0):
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 2), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 2), _expect(sfb, "sfb", _sf_dtype(ue8m0), 2)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != _sfb_shape(n, k, ue8m0):
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {_sfb_shape(n, k, ue8m0)}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa")):
        _row_major(t, nm)
    _contig(sfb, "sfb")
    ld_dsf = _check_qout(dq, dsf, (m,), n, False, ue8m0)
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(dq), _ptr(dsf), m, n, k, a.stride(0),
        b.stride(0), d.stride(0), sfa.stride(0), ld_dsf, _ptr(workspace), _ws(workspace), _stream(d)))
    return d, dq, dsf


def _contiguous_qout(fn, a, sfa, b, sfb, d, dq, dsf, m_indices, workspace, ue8m0):
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 3), _expect(d, "d", _BF, 2)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 2), _expect(sfb, "sfb", _sf_dtype(ue8m0), 3)
    _expect(m_indices, "m_indices", (torch.int32,), 1)
    m_total, k = a.shape
    groups, n = b.shape[0], b.shape[1]
    if b.shape[2] != k or tuple(d.shape) != (m_total, n) or m_indices.shape[0] != m_total:
        raise ValueError("shape mismatch between a, b, d and m_indices")
    want_b = (groups,) + _sfb_shape(n, k, ue8m0)
    if sfa.shape[0] != k // 128 or tuple(sfb.shape) != want_b:
        raise ValueError(f"scale shapes must be sfa [K/128][ld] and sfb {want_b}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfb, "sfb"), (m_indices, "m_indices")):
        _contig(t, nm)
    _row_major(sfa, "sfa")
    ld_dsf = _check_qout(dq, dsf, (m_total,), n, False, ue8m0)
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(dq), _ptr(dsf), _ptr(m_indices), m_total, n, k,
        groups, sfa.stride(0), ld_dsf, _ptr(workspace), _ws(workspace), _stream(d)))
    return d, dq, dsf


def _masked_qout(fn, a, sfa, b, sfb, d, dq, dsf, masked_m, expected_m, workspace, ue8m0):
    _expect(a, "a", _U8, 3), _expect(b, "b", _U8, 3), _expect(d, "d", _BF, 3)
    _expect(sfa, "sfa", _sf_dtype(ue8m0), 3), _expect(sfb, "sfb", _sf_dtype(ue8m0), 3)
    _expect(masked_m, "masked_m", (torch.int32,), 1)
    groups, m_max, k = a.shape
    n = b.shape[1]
    if b.shape[0] != groups or b.shape[2] != k or tuple(d.shape) != (groups, m_max, n):
        raise ValueError("shape mismatch between a, b and d")
    if masked_m.shape[0] != groups:
        raise ValueError("masked_m must have one entry per group")
    want_b = (groups,) + _sfb_shape(n, k, ue8m0)
    if sfa.shape[:2] != (groups, k // 128) or tuple(sfb.shape) != want_b:
        raise ValueError(f"scale shapes must be sfa [G][K/128][ld] and sfb {want_b}")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (sfa, "sfa"), (sfb, "sfb"), (masked_m, "masked_m")):
        _contig(t, nm)
    ld_dsf = _check_qout(dq, dsf, (groups, m_max), n, True, ue8m0)
    _check(fn, getattr(_lib, fn)(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(dq), _ptr(dsf), _ptr(masked_m), groups, m_max, n, k,
        int(expected_m), sfa.shape[2], ld_dsf, _ptr(workspace), _ws(workspace), _stream(d)))
    return d, dq, dsf


def dg_fp8_gemm_nt_qout(a, sfa, b, sfb, d, dq, dsf, workspace=None):
    """dg_fp8_gemm_nt that also writes the 1x128 quantisation of d: dq [M][N], dsf [N/128][ld]."""
    return _gemm_nt_qout("dg_fp8_gemm_nt_qout", a, sfa, b, sfb, d, dq, dsf, workspace, False)


def dg_grouped_contiguous_qout(a, sfa, b, sfb, d, dq, dsf, m_indices, workspace=None):
    """dg_grouped_contiguous that also writes the 1x128 quantisation of d."""
    return _contiguous_qout("dg_grouped_contiguous_qout", a, sfa, b, sfb, d, dq, dsf, m_indices, workspace, False)


def dg_grouped_masked_qout(a, sfa, b, sfb, d, dq, dsf, masked_m, expected_m=0, workspace=None):
    """dg_grouped_masked that also writes the 1x128 quantisation of d: dq [G][M_max][N], dsf [G][N/128][ld]."""
    return _masked_qout("dg_grouped_masked_qout", a, sfa, b, sfb, d, dq, dsf, masked_m, expected_m, workspace, False)


def dg_fp8_gemm_nt_ue8m0_qout(a, sfa, b, sfb, d, dq, dsf, workspace=None):
    """dg_fp8_gemm_nt_ue8m0 that also writes d's 1x128 UE8M0 quantisation (dsf uint8 exponents)."""
    return _gemm_nt_qout("dg_fp8_gemm_nt_ue8m0_qout", a, sfa, b, sfb, d, dq, dsf, workspace, True)


def dg_grouped_contiguous_ue8m0_qout(a, sfa, b, sfb, d, dq, dsf, m_indices, workspace=None):
    """dg_grouped_contiguous_ue8m0 that also writes d's 1x128 UE8M0 quantisation."""
    return _contiguous_qout("dg_grouped_contiguous_ue8m0_qout", a, sfa, b, sfb, d, dq, dsf, m_indices, workspace,
                            True)


def dg_grouped_masked_ue8m0_qout(a, sfa, b, sfb, d, dq, dsf, masked_m, expected_m=0, workspace=None):
    """dg_grouped_masked_ue8m0 that also writes d's 1x128 UE8M0 quantisation."""
    return _masked_qout("dg_grouped_masked_ue8m0_qout", a, sfa, b, sfb, d, dq, dsf, masked_m, expected_m,
                        workspace, True)


def dg_k_grouped_nt(a, sfa, b, sfb, d, k_offsets, workspace=None):
    """K-grouped GEMM: a [M][K], b [N][K] e4m3 with 1x128 scales sfa [K/128][ld_a],
    sfb [K/128][ld_b]; d [G][M][N]; k_offsets [G+1] int32 (device)."""
    _expect(a, "a", _U8, 2), _expect(b, "b", _U8, 2), _expect(d, "d", _BF, 3)
    _expect(sfa, "sfa", (torch.float32,), 2), _expect(sfb, "sfb", (torch.float32,), 2)
    _expect(k_offsets, "k_offsets", (torch.int32,), 1)
    m, k = a.shape
    n = b.shape[0]
    groups = d.shape[0]
    if b.shape[1] != k or tuple(d.shape) != (groups, m, n) or k_offsets.shape[0] != groups + 1:
        raise ValueError("shape mismatch between a, b, d and k_offsets")
    if sfa.shape[0] != k // 128 or sfb.shape[0] != k // 128:
        raise ValueError("scale shapes must be sfa [K/128][ld_a] and sfb [K/128][ld_b]")
    for t, nm in ((a, "a"), (b, "b"), (d, "d"), (k_offsets, "k_offsets")):
        _contig(t, nm)
    _row_major(sfa, "sfa"), _row_major(sfb, "sfb")
    _check("dg_k_grouped_nt", _lib.dg_k_grouped_nt(
        _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), _ptr(k_offsets), groups, m, n, k,
        sfa.stride(0), sfb.stride(0), _ptr(workspace), _ws(workspace), _stream(d)))
    return d


# ------------------------------------------------------------- quantisers --

def _quant_1x128(fn, x, q, sf, ue8m0):
    _expect(x, "x", _BF), _expect(q, "q", _U8), _expect(sf, "sf", _sf_dtype(ue8m0))
    if x.dim() not in (2, 3) or q.shape != x.shape or sf.dim() != x.dim():
        raise ValueError("x, q must match and sf must have the same rank")
    groups = 1 if x.dim() == 2 else x.shape[0]
    rows, cols = x.shape[-2], x.shape[-1]
    if sf.shape[-2] != cols // 128 or (x.dim() == 3 and sf.shape[0] != groups):
        raise ValueError("sf must be [(G)][C/128][ld]")
    for t, nm in ((x, "x"), (q, "q"), (sf, "sf")):
        _contig(t, nm)
    _check(fn, getattr(_lib, fn)(
        _ptr(x), _ptr(q), _ptr(sf), rows, cols, sf.shape[-1], groups, _stream(x)))
    return q, sf


def _quant_128x128(fn, w, q, sf, ue8m0):
    _expect(w, "w", _BF), _expect(q, "q", _U8), _expect(sf, "sf", _sf_dtype(ue8m0))
    if w.dim() not in (2, 3) or q.shape != w.shape:
        raise ValueError("w and q must match")
    groups = 1 if w.dim() == 2 else w.shape[0]
    rows, cols = w.shape[-2], w.shape[-1]
    want = _sfb_shape(rows, cols, ue8m0)
    if w.dim() == 3:
        want = (groups,) + want
    if tuple(sf.shape) != want:
        raise ValueError(f"sf must have shape {want}")
    for t, nm in ((w, "w"), (q, "q"), (sf, "sf")):
        _contig(t, nm)
    _check(fn, getattr(_lib, fn)(
        _ptr(w), _ptr(q), _ptr(sf), rows, cols, groups, _stream(w)))
    return q, sf


def dg_quant_1x128(x, q, sf):
    """x [R][C] or [G][R][C] bf16 -> q e4m3 codes, sf [(G)][C/128][ld] fp32."""
    return _quant_1x128("dg_quant_1x128", x, q, sf, False)


def _quant_1x128_mn(fn, x, q, sf, ue8m0):
    _expect(x, "x", _BF, 2), _expect(q, "q", _U8, 2), _expect(sf, "sf", _sf_dtype(ue8m0), 2)
    rows, cols = x.shape
    if tuple(q.shape) != (rows, cols) or sf.shape[0] != rows // 128:
        raise ValueError("q must match x and sf must be [rows/128][ld]")
    for t, nm in ((x, "x"), (q, "q"), (sf, "sf")):
        _contig(t, nm)
    _check(fn, getattr(_lib, fn)(_ptr(x), _ptr(q), _ptr(sf), rows, cols, sf.shape[1], _stream(x)))
    return q, sf


def dg_quant_1x128_mn(x, q, sf):
    """x stored [K][M] bf16 -> q [K][M] e4m3, sf [K/128][ld] fp32: 1x128 tiles along K (columns)."""
    return _quant_1x128_mn("dg_quant_1x128_mn", x, q, sf, False)


def dg_quant_1x128_mn_ue8m0(x, q, sf):
    """dg_quant_1x128_mn with UE8M0 exponent bytes (sf [K/128][ld] uint8)."""
    return _quant_1x128_mn("dg_quant_1x128_mn_ue8m0", x, q, sf, True)


def dg_quant_1x128_ue8m0(x, q, sf):
    """x [R][C] or [G][R][C] bf16 -> q e4m3 codes, sf [(G)][C/128][ld] uint8 exponents."""
    return _quant_1x128("dg_quant_1x128_ue8m0", x, q, sf, True)


def dg_quant_128x128(w, q, sf):
    """w [N][K] or [G][N][K] bf16 -> q e4m3 codes, sf [(G)][ceil(N/128)][K/128] fp32."""
    return _quant_128x128("dg_quant_128x128", w, q, sf, False)


def dg_quant_128x128_ue8m0(w, q, sf):
    """w [N][K] or [G][N][K] bf16 -> q e4m3 codes, sf [(G)][K/128][ld_sfb] uint8 exponents."""
    return _quant_128x128("dg_quant_128x128_ue8m0", w, q, sf, True)


# -------------------------------------------------------------- utilities --

def dg_get_workspace_size(m, n, k, num_groups=1):
    return int(_lib.dg_get_workspace_size(m, n, k, num_groups))


def dg_get_num_cus():
    v = _lib.dg_get_num_cus()
    if v < 0:
        raise DGError("dg_get_num_cus", v)
    return v


def dg_set_num_cus(num_cus):
    _check("dg_set_num_cus", _lib.dg_set_num_cus(int(num_cus)))


def dg_get_m_alignment_for_contiguous_layout():
    return int(_lib.dg_get_m_alignment_for_contiguous_layout())


def dg_get_sf_leading_dim(m):
    return int(_lib.dg_get_sf_leading_dim(int(m)))


def dg_get_ue8m0_sfb_leading_dim(n):
    return int(_lib.dg_get_ue8m0_sfb_leading_dim(int(n)))


def dg_get_last_error_string():
    return _lib.dg_get_last_error_string().decode()


def dg_describe_config(layout, m, n, k, num_groups=1, num_cus=256, expected_m=0):
    buf = ctypes.create_string_buffer(256)
    _check("dg_describe_config", _lib.dg_describe_config(layout, m, n, k, num_groups, expected_m, num_cus, buf, 256))
    return buf.value.decode()


def raw():
    """The loaded ctypes library (for calling entry points with raw pointers)."""
    return _lib
