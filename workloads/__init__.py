"""Seeded synthetic inputs for the layer-boundary workloads.

Both sides of every parity check draw their inputs from here, so this module
holds none of the boundary's arithmetic: it draws numbers (``gen.c``) and
stores them in the input formats (bf16 for rows, fp32 for weights and gates,
int32 for indices). The fp32 -> bf16 storage cast is torch's CPU cast.

Tensor streams are identified by ``tensor_id(kind, index, boundary)`` so no two
tensors of one workload share random numbers.

Workload recipes (sizes, distributions) follow the shapes of the pages'
workloads: a Qwen3-MoE-style decoder with hidden size 4096 (7168 for the
quantised case), TP partial sums of the producer output, the 2048-token fused
batch cap of the FlashInfer fusion study note (section on initialisation),
and top-8-of-128 MoE routing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libgen.so")
_lib = None

KIND_RESIDUAL = 1
KIND_WEIGHT = 2
KIND_PARTIAL = 3
KIND_OUTLIER_MASK = 4
KIND_ROUTER_LOGITS = 5
KIND_EXPERT_ROWS = 6
KIND_STACK_INPUT = 7


def tensor_id(kind: int, index: int = 0, boundary: int = 0) -> int:
    return (kind << 32) | (boundary << 16) | index


def build() -> str:
    """Compile gen.c into libgen.so (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
           "-o", _LIB_PATH, _SRC, "-lm"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def load(build_if_missing: bool = True):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{_LIB_PATH} is not built")
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
    ptr = ctypes.c_void_p
    lib.gen_normal_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, ptr]
    lib.gen_uniform_f64.argtypes = [u64, u64, u64, i64, ptr]
    lib.gen_outlier_normal_f32.argtypes = [u64, u64, u64, u64, i64, dbl, dbl, dbl, dbl, ptr]
    lib.gen_moe_routing.argtypes = [u64, u64, i64, ctypes.c_int, ctypes.c_int, ptr, ptr, ptr]
    lib.gen_moe_routing.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def normal_f32(seed: int, tid: int, shape, mean: float = 0.0, std: float = 1.0,
               first: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    load().gen_normal_f32(seed, tid, first, n, mean, std, _ptr(out))
    return out.reshape(shape)


def uniform_f64(seed: int, tid: int, shape, first: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    load().gen_uniform_f64(seed, tid, first, n, _ptr(out))
    return out.reshape(shape)


def outlier_normal_f32(seed: int, tid: int, mask_tid: int, shape, mean: float, std: float,
                       prob: float, factor: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    load().gen_outlier_normal_f32(seed, tid, mask_tid, 0, n, mean, std, prob, factor, _ptr(out))
    return out.reshape(shape)


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """Storage cast fp32 -> bf16 (torch CPU, round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 CPU tensor (a view, no copy when contiguous)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# workload recipes
# --------------------------------------------------------------------------

def fold_inputs(seed: int, T: int, H: int, P: int, *, c_std: float = 0.5, r_std: float = 1.0,
                w_mean: float = 1.0, w_std: float = 0.1, outlier_prob: float = 0.0,
                outlier_factor: float = 50.0, boundary: int = 0, with_residual: bool = True):
    """P bf16 partial contributions [T,H], a bf16 residual [T,H], an fp32 weight [H]."""
    partials = []
    for p in range(P):
        tid = tensor_id(KIND_PARTIAL, p, boundary)
        if outlier_prob > 0.0:
            a = outlier_normal_f32(seed, tid, tensor_id(KIND_OUTLIER_MASK, p, boundary), (T, H),
                                   0.0, c_std, outlier_prob, outlier_factor)
        else:
            a = normal_f32(seed, tid, (T, H), 0.0, c_std)
        partials.append(to_bf16(a))
    out = {
        "T": T, "H": H, "P": P,
        "partials": partials,
        "weight": torch.from_numpy(normal_f32(seed, tensor_id(KIND_WEIGHT, 0, boundary), (H,),
                                              w_mean, w_std)),
        "eps": 1e-6,
    }
    if with_residual:
        out["residual"] = to_bf16(normal_f32(seed, tensor_id(KIND_RESIDUAL), (T, H), 0.0, r_std))
    return out


def stack_input(seed: int, T: int, H: int, std: float = 1.0) -> torch.Tensor:
    """The bf16 input that enters the layer stack (the embedding output)."""
    return to_bf16(normal_f32(seed, tensor_id(KIND_STACK_INPUT), (T, H), 0.0, std))


def moe_inputs(seed: int, T: int, H: int, n_experts: int = 128, k: int = 8, *,
               e_std: float = 0.5, r_std: float = 1.0, w_mean: float = 1.0, w_std: float = 0.1):
    """Deferred MoE-finalize handoff: expert-major expert-output rows, gather index, gates."""
    idx = np.empty(T * k, dtype=np.int32)
    gate = np.empty(T * k, dtype=np.float32)
    expert = np.empty(T * k, dtype=np.int32)
    rc = load().gen_moe_routing(seed, tensor_id(KIND_ROUTER_LOGITS), T, n_experts, k,
                                _ptr(idx), _ptr(gate), _ptr(expert))
    if rc != 0:
        raise ValueError("gen_moe_routing rejected its arguments")
    rows = T * k
    return {
        "T": T, "H": H, "k": k, "n_experts": n_experts,
        "expert_rows": to_bf16(normal_f32(seed, tensor_id(KIND_EXPERT_ROWS), (rows, H), 0.0, e_std)),
        "idx": torch.from_numpy(idx),
        "gate": torch.from_numpy(gate),
        "expert": torch.from_numpy(expert),
        "residual": to_bf16(normal_f32(seed, tensor_id(KIND_RESIDUAL), (T, H), 0.0, r_std)),
        "weight": torch.from_numpy(normal_f32(seed, tensor_id(KIND_WEIGHT), (H,), w_mean, w_std)),
        "eps": 1e-6,
    }


# The five workloads of the hot path, with fixed seeds 1..5.
def tiny():
    """T=16, H=256, P=2; partials and residual N(0,1); weight N(1,0.1); eps 1e-6."""
    d = fold_inputs(1, 16, 256, 2, c_std=1.0, r_std=1.0)
    d["x_in"] = stack_input(1, 16, 256)
    return d


def decode_boundary(T: int, b: int, P: int = 4, H: int = 4096):
    """Boundary b (0-based) of the decode chain: fresh partials N(0,0.5) and weight N(1,0.1)."""
    return fold_inputs(2, T, H, P, c_std=0.5, boundary=b + 1, with_residual=False)


def decode_start(T: int, H: int = 4096):
    """Stack input of the decode chain, N(0,1), and the weight of the entering norm."""
    return {"x_in": to_bf16(normal_f32(2, tensor_id(KIND_RESIDUAL), (T, H), 0.0, 1.0)),
            "weight": torch.from_numpy(normal_f32(2, tensor_id(KIND_WEIGHT), (H,), 1.0, 0.1)),
            "eps": 1e-6}


def prefill():
    """T=2048 (the fused-batch cap), H=4096, P=8; partials N(0,0.5), residual N(0,1)."""
    return fold_inputs(3, 2048, 4096, 8, c_std=0.5, r_std=1.0)


def quantised():
    """T=2048, H=7168, P=8; partials N(0,0.5) with independent x50 outliers at p=1e-3."""
    return fold_inputs(4, 2048, 7168, 8, c_std=0.5, r_std=1.0, outlier_prob=1e-3,
                       outlier_factor=50.0)


def moe():
    """T=2048, H=4096, 128 experts, top-8; expert rows N(0,0.5); softmax gates over the picks."""
    return moe_inputs(5, 2048, 4096, 128, 8)


MOE_SLICE = (768, 256)  # reduce-scatter share r=3 of R=8 at T=2048: rows 768..1023
