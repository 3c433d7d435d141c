"""qk_attention_rope_noalloc: the attention call that allocates nothing (its
chunk states live in the library's static per-GPU scratch) against the
workspace call qk_attention_rope on the same inputs, through the C ABI.

Two calls in a row, the second with smaller sizes (fewer heads, a shorter
cache, an earlier position), so the second reads a scratch that still holds
the first call's states: each must give outputs and cache rows bit-identical
to the workspace call's, and within the attention tolerance of the oracle."""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def one_case(qk, orc, nh, nkv, hd, P, pos, seed):
    import torch

    g = synth.rng(70, seed)
    stride = nkv * hd
    kc = (g.standard_normal((P, stride)) * 2).astype(np.float16)
    vc = g.standard_normal((P, stride)).astype(np.float16)
    q = g.standard_normal(nh * hd).astype(np.float32)
    k = g.standard_normal(nkv * hd).astype(np.float32)
    v = g.standard_normal(nkv * hd).astype(np.float32)
    c = torch.empty(P * hd // 2, device="cuda")
    s = torch.empty_like(c)
    qk.qk_rope_tables(P, hd, 10000.0, c, s)
    posd = torch.tensor([pos], dtype=torch.int32, device="cuda")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    # the workspace call
    K1, V1 = to_dev(kc.view(np.int16)), to_dev(vc.view(np.int16))
    ws = torch.full((qk.qk_attention_workspace_bytes(nh, hd, P) // 4,), float("nan"), device="cuda")
    out1 = torch.full((nh * hd,), float("nan"), device="cuda")
    qk.qk_attention_rope(qd, kd, vd, posd, P, c, s, nh, nkv, hd, K1, V1, stride, ws, out1)
    # the call without a workspace, on its own copy of the caches
    K2, V2 = to_dev(kc.view(np.int16)), to_dev(vc.view(np.int16))
    out2 = torch.full((nh * hd,), float("nan"), device="cuda")
    st = qk.lib.qk_attention_rope_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), posd.data_ptr(), P,
                                          c.data_ptr(), s.data_ptr(), nh, nkv, hd, K2.data_ptr(), V2.data_ptr(),
                                          stride, out2.data_ptr(), qk._stream(None))
    assert st == qk.QK_OK, qk.lib.qk_last_hip_error()
    torch.cuda.synchronize()
    o1, o2 = out1.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), "outputs differ from the workspace call's"
    assert torch.equal(K1, K2) and torch.equal(V1, V2), "cache rows differ from the workspace call's"
    # and the oracle, on the cache the call wrote
    ct = c.cpu().numpy().reshape(P, -1)[pos]
    sn = s.cpu().numpy().reshape(P, -1)[pos]
    kw = K2.cpu().numpy().view(np.uint16).reshape(P, stride)
    vw = V2.cpu().numpy().view(np.uint16).reshape(P, stride)
    ref, a = orc.attention(orc.rope(q, nh, hd, ct, sn), kw, vw, nh, nkv, hd, pos + 1, stride)
    err = np.abs(o2.astype(np.float64) - ref)
    assert np.all(err <= 1e-4 * a + 1e-6), float(np.nanmax(err / (1e-4 * a + 1e-6)))


def test_noalloc_matches_workspace_call_twice(qk, orc):
    # a 1.1B-shaped layer near the end of a 2048-row cache, then a smaller one
    one_case(qk, orc, nh=32, nkv=4, hd=64, P=2048, pos=1900, seed=1)
    one_case(qk, orc, nh=8, nkv=2, hd=128, P=300, pos=77, seed=2)


def test_noalloc_rejects_sizes_past_its_scratch(qk):
    lim = qk.lib.qk_attention_scratch_limit()
    assert lim == 8 << 20
    assert qk.qk_attention_workspace_bytes(32, 128, 65536) <= lim < qk.qk_attention_workspace_bytes(65, 128, 65536)
    A = 0x10000
    st = qk.lib.qk_attention_rope_noalloc(A, A, A, A, 65536, A, A, 65, 5, 128, A, A, 640, A, None)
    assert st == qk.QK_EINVAL_SHAPE and b"8 MiB" in qk.lib.qk_last_hip_error()
