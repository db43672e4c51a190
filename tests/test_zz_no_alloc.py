"""The allocation-free forward (llsa_forward_noalloc, static scratch) against
llsa_forward (caller workspace), through the C ABI: outputs identical bit for
bit, on two calls in a row on one GPU, the second with a smaller input (the
scratch then holds the first call's larger state)."""
import numpy as np
import pytest

import synth
from llsa_check import to_device

pytestmark = pytest.mark.gpu


def _noalloc_vs_forward(w, flags=0):
    import torch
    import sparse_attention_diffusion_order_amd as lib
    inp = synth.make_inputs(w, want_grad=False)
    q, k, v = (to_device(inp[n], w.dtype).reshape(w.B, w.H, w.N, w.d) for n in ("q", "k", "v"))
    out_ref, lse_ref, _ = lib.forward(q, k, v, w.topk, w.levels, flags)
    out = torch.full_like(q, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    dt = lib.BF16 if w.dtype == "bf16" else lib.F32
    lib.llsa_forward_noalloc(q, k, v, out, lse, w.B, w.H, w.N, w.d, 16, w.topk, w.levels, dt,
                             flags)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else (lambda t: t)
    assert torch.equal(bits(out), bits(out_ref))
    assert torch.equal(lse, lse_ref)


def test_noalloc_forward_matches_forward_twice():
    W = synth.Workload
    # 256x256, six heads (the largest standard workload that fits the
    # scratch), then a smaller one with three levels and another top-k
    _noalloc_vs_forward(synth.WORKLOADS["grid256_bf16_l2_k16"])
    _noalloc_vs_forward(W("small_l3", 1, 2, 128, 64, "bf16", 3, 2, 2.0))
    # fp32 and an enrichment variant on the same scratch
    _noalloc_vs_forward(W("small_f32", 1, 2, 32, 64, "f32", 2, 2, 2.0), flags=4)
    # causal rows (unused slots -1 in the scratch's index lists)
    _noalloc_vs_forward(W("small_causal", 1, 2, 64, 64, "bf16", 2, 4, 2.0), flags=16)


def test_noalloc_forward_refuses_a_shape_beyond_the_scratch():
    import torch
    import sparse_attention_diffusion_order_amd as lib
    x = torch.zeros(1, 6, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.LlsaError) as e:
        # 512x512 tokens, six heads, three levels: ~120 MB of forward state
        lib.llsa_forward_noalloc(x, x, x, x, x, 1, 6, 262144, 64, 16, 16, 3, lib.BF16, 0)
    assert e.value.code == -6
