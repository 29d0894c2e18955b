"""The allocation-free forward (moe_forward_static) against moe_forward,
through the C ABI: two calls in a row, the second on a smaller batch, each
compared with moe_forward on the same inputs (same kernels, so every output
must be bit-identical), and the oracle's routing for good measure; plus the
rejection of a layer whose scratch need exceeds the static array."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from helpers import from_dev, inputs, normwise, to_dev, tol_for, weights_to_dev
from moe_inputs import get_config
from mixture_experts_layer_41_amd import _lib
from mixture_experts_layer_41_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run_pair(cfg):
    say(f"[case] static scratch forward {cfg.name} T={cfg.T}")
    t = inputs(cfg)
    o = oracle.forward(cfg, t)
    c = B.config_of(cfg)
    W = weights_to_dev(cfg, t)
    x = to_dev(t["x"], cfg.dtype)
    # the workspace moe_forward needs fits the static array
    F = B.Forward(c, W)
    assert F.ws_bytes <= _lib.MOE_STATIC_SCRATCH_BYTES
    y_ref = F(x).clone()
    y, idx, w, counts, aux = B.moe_forward_static(c, W, x)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    assert torch.equal(idx, F.topk_idx)
    assert torch.equal(w, F.topk_w)
    assert torch.equal(counts, F.expert_counts)
    assert torch.equal(aux, F.aux)
    assert np.array_equal(idx.cpu().numpy(), o["topk_idx"])
    err = normwise(from_dev(y), o["y"])
    assert err <= tol_for(cfg), f"normwise err {err:.3e}"
    say(f"[ok] {cfg.name} T={cfg.T} y_err={err:.2e}")


def test_static_forward_two_calls_second_smaller():
    # the Flash-shaped layer (capacity 1.25), then a smaller batch of a
    # different layer with shared experts: the second call reuses the array
    # the first one left behind
    _run_pair(get_config("c2"))
    _run_pair(get_config("c3", T=900))


def test_static_forward_rejects_a_layer_beyond_the_array():
    cfg = get_config("c4")   # 65536 tokens: several GB of scratch
    c = B.config_of(cfg)
    n = ctypes.c_size_t(0)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = dummy.data_ptr()
    w = _lib.MoeWeights(w_router=p, w1=p, w2=p, shared_w1=p, shared_w2=p)
    assert _lib.lib().moe_forward(ctypes.byref(c), ctypes.byref(w), None, None, None, None, None, None,
                                  None, None, ctypes.byref(n), None) == _lib.MOE_OK
    assert n.value > _lib.MOE_STATIC_SCRATCH_BYTES
    st = _lib.lib().moe_forward_static(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(p), None,
                                       ctypes.c_void_p(p), None, None, None, None,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.MOE_ERR_WORKSPACE
