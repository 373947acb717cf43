"""Shared helpers of the GPU parity tests: numpy <-> device tensors and the
oracle-side reference of one quantised layer."""

import numpy as np
import torch

from bit_nf4_quantized_22_amd import synth
from oracle import linear, nf4

DEV = "cuda:0"


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_np(t):
    return t.detach().float().cpu().numpy()


def weight_dev(W, dtype):
    """W as the device tensor the quantiser reads (fp32, or bf16 bits)."""
    return f32_dev(W) if dtype == "f32" else bf16_dev(W)


def weight_f32(W, dtype):
    return np.asarray(W, np.float32) if dtype == "f32" else synth.bf16_to_f32(W)


def oracle_quant(W, dtype, double_quant=True):
    """Oracle codes/constants and the fp32 dequantised weight of W[N, K]."""
    w32 = weight_f32(W, dtype)
    packed, absmax = nf4.quantize_nf4(w32)
    if double_quant:
        q8, c2 = nf4.double_quantize(absmax)
        scales = nf4.dequant_scales(q8, c2)
    else:
        q8 = c2 = None
        scales = absmax
    What = nf4.dequantize(packed, scales, w32.size).reshape(w32.shape)
    return dict(packed=packed, absmax=absmax, q8=q8, c2=c2, What=What)


def rel_frob(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


__all__ = ["DEV", "bf16_dev", "f32_dev", "to_bits16", "to_np", "weight_dev", "weight_f32",
           "oracle_quant", "rel_frob", "f64", "linear", "nf4", "synth"]
