"""The allocation-free attention layer (dash_attn_layer_noalloc), called through
the C ABI, against dash_attn_layer with a caller workspace: identical bits for
O, U and the score, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from workload import WORKLOADS, layer_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_delta_token_amd as d
    d.load()
    return d


def _inputs(S, seed):
    w = WORKLOADS[1].scaled(S=S)  # Qwen2.5-7B heads: hidden 3584, bf16
    x = layer_inputs(w, seed, 0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16)
    return dev(x["Q"]), dev(x["K"]), dev(x["V"]), dev(x["Wo"].T), w


def _run(dash, fn, Q, K, V, Wo, w, with_ws):
    S = Q.shape[0]
    O = torch.full((S, w.Hq * w.D), 7.0, device="cuda", dtype=torch.bfloat16)
    U = torch.full((S, w.hidden), 7.0, device="cuda", dtype=torch.bfloat16)
    score = torch.full((S,), -1.0, device="cuda", dtype=torch.float32)
    if with_ws:
        ws = dash.workspace(dash.DASH_OP_ATTN_LAYER, dash.make_shape(1, S, w.Hq, w.Hkv, w.D, w.hidden, dash.DASH_BF16),
                            S)
        fn(Q, K, V, Wo, O, U, score, ws)
    else:
        fn(Q, K, V, Wo, O, U, score)
    return O, U, score


def test_noalloc_matches_workspace_call(dash):
    for S, seed in ((5000, 1), (1300, 2)):  # the second call smaller: the scratch keeps the first call's partials
        print("no-alloc attention layer S", S, flush=True)
        Q, K, V, Wo, w = _inputs(S, seed)
        ref = _run(dash, dash.dash_attn_layer, Q, K, V, Wo, w, with_ws=True)
        got = _run(dash, dash.dash_attn_layer_noalloc, Q, K, V, Wo, w, with_ws=False)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        assert torch.all(got[2] > 0)


def test_noalloc_rejects_sizes_beyond_the_scratch(dash):
    # hidden 3584 needs 16 partials of 4 bytes per row: 16 MiB hold 262144 rows
    w = WORKLOADS[1]
    shape = dash.make_shape(1, 262145, w.Hq, w.Hkv, w.D, w.hidden, dash.DASH_BF16)
    import ctypes
    from attention_delta_token_amd import _lib as L
    fake = 0x10000  # never dereferenced: the size check fails first
    rc = L.load().dash_attn_layer_noalloc(None, ctypes.byref(shape), fake, fake, fake, fake, fake, fake, fake, None)
    assert rc == L.DASH_E_WORKSPACE
    assert "scratch" in L.load().dash_last_error().decode()
