"""sla_forward_noalloc against sla_forward, through the C ABI: the same
outputs and labels on two calls in a row, the second smaller than the first
(so that it runs over the first call's leftovers in the static scratch).
The two entry points run the same kernels, and the forward pass is bitwise
deterministic, so the outputs must be equal bit for bit."""
import ctypes

import numpy as np
import pytest

from sparse_attention_video_sla_amd import _lib

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype, crit share, negligible share): the second call of each
# pair is smaller than the first
CASES = [
    ((1, 12, 32760, 128, "bf16", 0.05, 0.10), (1, 2, 3000, 128, "bf16", 0.05, 0.10)),
    ((1, 2, 1050, 128, "f32", 0.05, 0.10), (1, 1, 700, 64, "f32", 0.10, 0.20)),
]


def run_pair(torch, shape):
    B, H, N, d, dt, rc, rn = shape
    g = torch.Generator(device="cpu").manual_seed(N * 7 + d)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(tdt).to(dev) for _ in range(3))
    w = (torch.randn(d, d, generator=g) / d ** 0.5).to(dev)
    Nb = -(-N // 64)
    code = _lib.SLA_BF16 if dt == "bf16" else _lib.SLA_F32
    L = _lib.load()
    st = torch.cuda.current_stream().cuda_stream
    n = ctypes.c_size_t()
    _lib.check(L.sla_workspace_size(B, H, N, d, 64, code, rc, rn, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    ref = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    ref_mask = torch.empty(B, H, Nb, Nb, dtype=torch.int8, device=dev)
    got = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device=dev)
    got_mask = torch.full((B, H, Nb, Nb), 5, dtype=torch.int8, device=dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), code, _lib.SLA_F32, B, H, N, d, 64, rc, rn,
            _lib.SLA_PHI_SOFTMAX)
    _lib.check(L.sla_forward(*args, ref.data_ptr(), ref_mask.data_ptr(), ws.data_ptr(), ws.numel(), st))
    _lib.check(L.sla_forward_noalloc(*args, got.data_ptr(), got_mask.data_ptr(), st))
    torch.cuda.synchronize()
    return ref.cpu().numpy(), ref_mask.cpu().numpy(), got.cpu().numpy(), got_mask.cpu().numpy()


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_equals_forward_on_two_calls(first, second):
    import torch
    for shape in (first, second):
        print("sla_forward_noalloc vs sla_forward", shape, flush=True)
        ref, ref_mask, got, got_mask = run_pair(torch, shape)
        assert np.isfinite(ref).all()
        assert np.array_equal(got_mask, ref_mask), shape
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
            (shape, float(np.abs(got - ref).max()))
