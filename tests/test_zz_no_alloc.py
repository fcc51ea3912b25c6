"""The allocation-free forward (tp_mlp_shard_forward_noalloc) against the
workspace forward (tp_mlp_shard_forward) through the C ABI: the same kernels
on the same inputs, so the partials must agree bit for bit; both are also
checked against the fp64 oracle at the bf16 bound.  Two calls in a row share
the library's static scratch, the second with a smaller input (it must not
see the first call's leftovers), and a forward that needs more scratch than
the array holds is refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tp_amd as tp
from tensor_transformer_mlp_tp_amd import _lib
from helpers import TOL_BF16, TOL_FP8, make_case, upload_case, oracle_partial

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20   # TP_NOALLOC_SCRATCH_BYTES in include/tp_mlp.h


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(lib, d, t, k, partial, wc):
    M, h = d["x"].shape
    I_s = d["w_gate"].shape[0]
    return lib.tp_mlp_shard_forward_noalloc(
        M, h, I_s * t, t, k, _lib.TP_BF16, wc, _p(d["x"]), d["x"].stride(0), _p(d["w_gate"]), _p(d["w_up"]),
        d["w_gate"].stride(0), _p(d["w_down"]), d["w_down"].stride(0), _p(d["s_gate"]), _p(d["s_up"]),
        _p(d["s_down"]), _p(partial), partial.stride(0), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _workspace_forward(d, t, k):
    return tp.shard_forward(d["x"], d["w_gate"], d["w_up"], d["w_down"], t=t, k=k, s_gate=d["s_gate"],
                            s_up=d["s_up"], s_down=d["s_down"])


@pytest.mark.parametrize("w", ["bf16", "e4m3fn"])
def test_noalloc_matches_workspace_forward_twice(w):
    lib = _lib.load()
    wc = _lib.TP_BF16 if w == "bf16" else _lib.TP_FP8_E4M3FN
    t, k = 2, 1
    # first a prefill whose GEMMs have stream-K tails (counters and slots in the
    # scratch), then a smaller decode forward on the same scratch
    for M, h, I_s in ((300, 2112, 2112), (8, 1024, 512)):
        print("noalloc w=%s M=%d h=%d I_s=%d" % (w, M, h, I_s), flush=True)
        need = tp.workspace_bytes(M, h, I_s * t, t, torch.bfloat16,
                                  torch.bfloat16 if w == "bf16" else torch.float8_e4m3fn)
        assert 0 < need <= SCRATCH_BYTES
        x, ws = make_case(47, M, h, I_s, "bf16", w, 0.05, 0.05, weight_set=M)
        d = upload_case(x, ws, "bf16", w)
        ref = _workspace_forward(d, t, k)
        got = torch.full((M, h), float("nan"), dtype=torch.float32, device="cuda")
        st = _noalloc(lib, d, t, k, got, wc)
        assert st == _lib.TP_OK, lib.tp_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
        err = oracle.rms_normalised_max_error(got.cpu().numpy(), oracle_partial(x, ws, "bf16", w))
        assert err <= (TOL_FP8 if w == "e4m3fn" else TOL_BF16), err


def test_noalloc_refuses_forward_beyond_its_scratch():
    lib = _lib.load()
    M, h, I_s, t = 4096, 8192, 7168, 4          # A alone is 56 MiB
    assert tp.workspace_bytes(M, h, I_s * t, t) > SCRATCH_BYTES
    x = torch.empty((M, h), dtype=torch.bfloat16, device="cuda")
    wg = torch.empty((I_s, h), dtype=torch.bfloat16, device="cuda")
    wd = torch.empty((h, I_s), dtype=torch.bfloat16, device="cuda")
    p = torch.empty((M, h), dtype=torch.float32, device="cuda")
    d = dict(x=x, w_gate=wg, w_up=wg, w_down=wd, s_gate=None, s_up=None, s_down=None)
    assert _noalloc(lib, d, t, 0, p, _lib.TP_BF16) == _lib.TP_ERR_UNSUPPORTED
    assert b"allocation-free" in lib.tp_last_error()
