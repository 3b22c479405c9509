"""Helpers for the GPU parity tests: host <-> device copies of numpy arrays and
thin wrappers that run the HIP path through the C ABI binding."""

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import moe_grouped_gemm_02_amd as dg  # raises if libdg.so is missing
    return dg


def dev(arr):
    """numpy -> device tensor (uint16 arrays become int16 bf16 bit carriers)."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(arr).cuda()


def host(t):
    """device tensor -> numpy (int16 bf16 carriers come back as uint16)."""
    a = t.detach().cpu()
    if a.dtype in (torch.bfloat16, torch.int16):
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


SENTINEL = 0x7FC1  # a bf16 NaN pattern the kernels never produce


def gpu_quant_1x128(dg, x_bits, ld=None):
    x = dev(x_bits)
    shape = x_bits.shape
    rows, cols = shape[-2], shape[-1]
    ld = dg.dg_get_sf_leading_dim(rows) if ld is None else ld
    q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    sf_shape = (cols // 128, ld) if len(shape) == 2 else (shape[0], cols // 128, ld)
    sf = torch.full(sf_shape, float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128(x, q, sf)
    return q, sf


def gpu_quant_128x128(dg, w_bits):
    w = dev(w_bits)
    shape = w_bits.shape
    rows, cols = shape[-2], shape[-1]
    sf_shape = ((rows + 127) // 128, cols // 128)
    if len(shape) == 3:
        sf_shape = (shape[0],) + sf_shape
    q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    sf = torch.full(sf_shape, float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(w, q, sf)
    return q, sf


def gpu_quant_1x128_ue8m0(dg, x_bits, ld=None):
    x = dev(x_bits)
    shape = x_bits.shape
    rows, cols = shape[-2], shape[-1]
    ld = dg.dg_get_sf_leading_dim(rows) if ld is None else ld
    q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    sf_shape = (cols // 128, ld) if len(shape) == 2 else (shape[0], cols // 128, ld)
    sf = torch.full(sf_shape, 0xEE, dtype=torch.uint8, device="cuda")
    dg.dg_quant_1x128_ue8m0(x, q, sf)
    return q, sf


def gpu_quant_128x128_ue8m0(dg, w_bits):
    w = dev(w_bits)
    shape = w_bits.shape
    rows, cols = shape[-2], shape[-1]
    sf_shape = (cols // 128, dg.dg_get_ue8m0_sfb_leading_dim(rows))
    if len(shape) == 3:
        sf_shape = (shape[0],) + sf_shape
    q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    sf = torch.full(sf_shape, 0xEE, dtype=torch.uint8, device="cuda")
    dg.dg_quant_128x128_ue8m0(w, q, sf)
    return q, sf
