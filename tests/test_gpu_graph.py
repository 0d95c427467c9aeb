"""The layer captured in a HIP graph and replayed.

Every entry point of the C ABI only enqueues kernels on the caller's stream: it
allocates nothing (the caller passes the workspace), records no memset and never
synchronises. So a caller can capture a whole layer step, forward or forward +
backward, into one graph and replay it, which removes the per-launch host cost
that dominates small layers. Each replay here is compared bit for bit with an
eager call on the same inputs; between replays the graph's input buffers are
overwritten in place, and eager work and synchronisations run in between. For
the same reason calls on two streams with separate buffers may overlap; the last
test checks that they give the bits of the same calls made one after another.
"""
import pytest
import torch

import mixture_experts_ffn_group_amd as moe
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(h):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in h.items()}


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("name", ["tiny", "mid_skewed"])
def test_forward_graph_replays_equal_eager(name):
    d = _dev(workloads.make_inputs(name))
    wl = d["workload"]
    x = d["x"].clone()  # the graph's input buffer
    ws = torch.empty(moe.workspace_bytes(wl.T, wl.emb, wl.mlp, wl.E, wl.k), dtype=torch.uint8, device=DEV)
    y = torch.empty((wl.T, wl.emb), dtype=torch.bfloat16, device=DEV)

    def fwd(xin, out, work):
        return moe.ffn_fwd(xin, d["wi"], d["wo"], wl.k, wr=d["wr"], bias=d["bias"], logits=d["logits_in"],
                           workspace=work, out=out)[0]

    fwd(x, y, ws)  # first use outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x, y, ws)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(11)
    ws_e = torch.empty_like(ws)
    for rep in range(4):
        xr = (torch.randn((wl.T, wl.emb), generator=gen) * (0.5 + rep)).to(torch.bfloat16).to(DEV)
        x.copy_(xr)
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref = fwd(xr, None, ws_e)  # eager, own workspace and output
        torch.cuda.synchronize()
        assert _same_bits(got, ref), f"{name}: replay {rep} differs from the eager forward"


def test_training_step_graph_replays_equal_eager():
    """Forward with the saved set, then the layer backward, in one graph."""
    d = _dev(workloads.make_inputs("mid_skewed"))
    wl = d["workload"]
    x = d["x"].clone()
    dy = torch.empty((wl.T, wl.emb), dtype=torch.bfloat16, device=DEV)

    def step(xin, dyin):
        y, saved = moe.ffn_fwd(xin, d["wi"], d["wo"], wl.k, wr=d["wr"], bias=d["bias"], logits=d["logits_in"],
                               save=True)
        g = moe.ffn_bwd(dyin, saved, d["wi"], d["wo"], wl.k)
        return y, g

    gen = torch.Generator().manual_seed(5)
    dy.copy_((torch.randn((wl.T, wl.emb), generator=gen) * 0.1).to(torch.bfloat16))
    step(x, dy)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_g, g_g = step(x, dy)
    torch.cuda.synchronize()

    for rep in range(3):
        xr = (torch.randn((wl.T, wl.emb), generator=gen) * (0.5 + rep)).to(torch.bfloat16).to(DEV)
        dyr = (torch.randn((wl.T, wl.emb), generator=gen) * 0.1).to(torch.bfloat16).to(DEV)
        x.copy_(xr)
        dy.copy_(dyr)
        graph.replay()
        torch.cuda.synchronize()
        got_y = y_g.clone()
        got = {k: v.clone() for k, v in g_g.items() if v is not None}
        y_e, g_e = step(xr, dyr)
        torch.cuda.synchronize()
        assert _same_bits(got_y, y_e), f"replay {rep}: y"
        for k, v in got.items():
            assert _same_bits(v, g_e[k]), f"replay {rep}: {k}"


def test_two_streams_with_separate_buffers_equal_sequential_calls():
    """Calls on different streams with separate buffers may run at the same time: the library keeps no
    state between calls. A forward of one workload and a training step (forward with the saved set, then
    the backward) of another, issued several times over on two streams at once, give the bits the same
    calls give one after the other."""
    a = _dev(workloads.make_inputs("mid_skewed"))
    b = _dev(workloads.make_inputs(workloads.custom(1000, 256, 192, 12, 3, seed=31, sigma_w=0.05, backward=True)))

    def fwd(d):
        wl = d["workload"]
        return moe.ffn_fwd(d["x"], d["wi"], d["wo"], wl.k, wr=d["wr"], bias=d["bias"], logits=d["logits_in"])[0]

    def train(d):
        wl = d["workload"]
        y, saved = moe.ffn_fwd(d["x"], d["wi"], d["wo"], wl.k, wr=d["wr"], bias=d["bias"], save=True)
        return y, moe.ffn_bwd(d["dy"], saved, d["wi"], d["wo"], wl.k)

    ref_a = fwd(a)
    ref_b, ref_g = train(b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = fwd(a)
        with torch.cuda.stream(s2):
            yb, g = train(b)
        outs.append((ya, yb, g))
    torch.cuda.synchronize()
    for ya, yb, g in outs:
        assert _same_bits(ya, ref_a)
        assert _same_bits(yb, ref_b)
        for n, v in ref_g.items():
            if v is not None:
                assert _same_bits(g[n], v), n
