"""vc_attention_noalloc (the library's static scratch in place of a caller
workspace) against vc_attention through the C ABI: the same kernels, so the
outputs must be identical, on two calls in a row with the second smaller,
with no device memory allocated by the calls."""
import numpy as np
import pytest
import torch

from bit_attention_video_amd import binding as vb
from bit_attention_video_amd import inputs
from layouts import to_device_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vb.lib()


def _case(name, H, N, p_mode=vb.EXPCAST, vsmooth=True):
    w = inputs.WORKLOADS[name]
    N = N or w.N
    q, k, v, init = inputs.gen_all(w, N=N, H=H)
    cfg = vb.make_config(w.B, H, N, w.d, w.kv_block, min(w.k, N), w.iters, vsmooth, vb.E4M3, False,
                         p_mode=p_mode, seed=w.seed)
    return cfg, to_device_bf16(q), to_device_bf16(k), to_device_bf16(v)


def test_noalloc_equals_vc_attention_on_two_calls():
    # the first call is larger than the second, which then runs on a scratch
    # holding the first call's leftovers
    cases = [_case("mid", 2, None), _case("tiny", 2, 700, p_mode=vb.EXPCAST_SHIFTED)]
    outs = [vb.alloc_out(c) for c, *_ in cases]
    refs = []
    for (cfg, Q, K, V) in cases:
        assert vb.workspace_bytes(cfg, attention=True) <= vb.noalloc_scratch_bytes()
        refs.append(vb.vc_attention(cfg, Q, K, V))
    torch.cuda.synchronize()
    for i, ((cfg, Q, K, V), out) in enumerate(zip(cases, outs)):
        vb.vc_attention_noalloc(cfg, Q, K, V, None, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), refs[i].view(torch.int16)), f"call {i} differs"
    # the scratch now holds the second call's data; the first configuration
    # again, with no device memory allocated by the call
    cfg, Q, K, V = cases[0]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    used0 = torch.cuda.memory_allocated()
    vb.vc_attention_noalloc(cfg, Q, K, V, None, outs[0])
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0 and torch.cuda.memory_allocated() == used0
    assert torch.equal(outs[0].view(torch.int16), refs[0].view(torch.int16))


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    w = inputs.WORKLOADS["mid"]
    cfg = vb.make_config(1, 24, w.N, w.d, w.kv_block, w.k, w.iters)
    assert vb.workspace_bytes(cfg, attention=True) > vb.noalloc_scratch_bytes()
    x = torch.zeros((1, 24, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vb.VcError, match="scratch") as e:
        vb.vc_attention_noalloc(cfg, x, x, x, None, torch.empty_like(x))
    assert e.value.status == -3          # VC_ERR_WORKSPACE, before anything runs
