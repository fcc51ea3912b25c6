"""Shared helpers for the tests: upload seeded storage arrays, run the oracle.

Only marshalling: numpy storage (bf16 bits, fp32, e4m3fn codes) <-> torch
tensors on the device.  The oracle is called on the exact bytes uploaded.
"""

import numpy as np
import torch

import oracle
import workloads

TOL_BF16 = 2e-2   # max |out - ref| / rms(ref), bf16 activations and weights (and fp32)
TOL_FP8 = 6e-2    # same metric, fp8 e4m3fn weights (reference: dequantised weights)
TOL_INT8 = 2e-2   # int8 weights: the reference is the dequantised weights, and the
                  # kernels widen the codes to bf16 exactly, so only the bf16 bound applies


def to_device(arr, dtype, device="cuda"):
    """numpy storage -> torch tensor with the library dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype == "e4m3fn":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).view(torch.float8_e4m3fn).to(device)
    if dtype == "int8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).view(torch.int8).to(device)
    raise ValueError(dtype)


def make_case(config_id, M, h, I_s, act, w, std_gu, std_down, k=0, weight_set=0):
    x = workloads.make_x(config_id, M, h, act, weight_set=weight_set)
    ws = workloads.make_shard_weights(config_id, h, I_s, k, w, std_gu, std_down, weight_set=weight_set)
    return x, ws


def upload_case(x, ws, act, w, device="cuda"):
    d = dict(x=to_device(x, act, device),
             w_gate=to_device(ws["w_gate"], w, device),
             w_up=to_device(ws["w_up"], w, device),
             w_down=to_device(ws["w_down"], w, device))
    for s in ("s_gate", "s_up", "s_down"):
        d[s] = None if ws[s] is None else torch.from_numpy(ws[s]).to(device)
    return d


def oracle_partial(x, ws, act, w, rows=None):
    """fp64 oracle P_k, optionally on a subset of token rows (rows are independent)."""
    xs = x if rows is None else x[rows]
    return oracle.rank_partial_from_storage(xs, act, ws["w_gate"], ws["w_up"], ws["w_down"], w,
                                            ws["s_gate"], ws["s_up"], ws["s_down"])
