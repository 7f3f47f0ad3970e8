"""The prefill entry point that allocates nothing (gdn_prefill_chunked_noalloc:
the chunk records live in the library's static device scratch) against
gdn_prefill_chunked with a caller workspace, through the C ABI: bit-identical
states and outputs on two calls in a row, the second with a smaller input
(so the scratch still holds the first call's records), and the size limit
refused on the host before any launch."""
import numpy as np
import pytest

from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, dev, dims_pair, host, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def run(sh, inp, T, noalloc):
    torch = torch_mod()
    A = act_dtype(sh.act)
    d, _ = dims_pair(sh, T=T)
    st = dev(inp["state"], torch.float32)
    cur = dev(inp["cur"], torch.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = dev(np.ascontiguousarray(inp["y"][:, :, :T]), A)
    g = dev(np.ascontiguousarray(inp["g"][:, :, :T]), A)
    be = dev(np.ascontiguousarray(inp["beta"][:, :, :T]), A)
    o = torch.full((sh.L, sh.B, T, sh.HV, sh.DV), float("nan"), device="cuda")
    if noalloc:
        B().gdn_prefill_chunked_noalloc(d, y, g, be, st, cur, o, 64, err)
    else:
        ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
        B().gdn_prefill_chunked(d, y, g, be, st, cur, o, 64, ws, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    return host(st), host(o)


@pytest.mark.parametrize("first,second", [(1024, 200), (640, 65)])
def test_noalloc_prefill_equals_workspace_prefill(first, second):
    sh = W.PREFILL.with_(B=1, HV=32, HK=16)
    inp = W.prefill_inputs(sh, seed=3900 + first, tokens=first)
    inp["state"] = W.random_state(sh, seed=3901)
    outs = []
    for T in (first, second):
        st_n, o_n = run(sh, inp, T, True)
        st_w, o_w = run(sh, inp, T, False)
        assert np.array_equal(st_n, st_w), T
        assert np.array_equal(o_n, o_w), T
        assert np.all(np.isfinite(o_n))
        outs.append(o_n)
    # the second call's outputs are those of its own tokens, not the first's
    assert np.array_equal(outs[1][:, :, :second], run(sh, inp, second, False)[1])


def test_noalloc_prefill_refuses_dims_over_the_scratch_size():
    torch = torch_mod()
    sh = W.PREFILL.with_(B=2, T=1024)
    d, _ = dims_pair(sh)
    assert B().gdn_workspace_size(d) > B().GDN_NOALLOC_SCRATCH_BYTES
    A = act_dtype(sh.act)
    y = torch.zeros((1, sh.B, sh.T, sh.C), dtype=A, device="cuda")
    g = torch.zeros((1, sh.B, sh.T, sh.HV), dtype=A, device="cuda")
    st = torch.zeros((1, sh.B, 1, sh.HV, sh.DK, sh.DV), device="cuda")
    o = torch.full((1, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    with pytest.raises(B().GdnError) as e:
        B().gdn_prefill_chunked_noalloc(d, y, g, g, st, None, o, 64)
    assert e.value.status == 6   # GDN_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
