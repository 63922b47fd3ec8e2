"""The layer's calls under HIP graph capture: a captured quantize + fwd + bwd
step, replayed several times with eager work and synchronisations between
the replays, gives the eager outputs bit for bit every time (the library
records no memset nodes and allocates nothing inside the calls).  Also the
decode forward, whose k-split counters persist in the workspace."""
import pytest
import torch

from tests.helpers import say, to_dev_bf16, to_dev_f32
from workloads import WORKLOADS, make_layer, workload_layer

pytestmark = pytest.mark.gpu


def capture_and_check(step, outs, replays=3):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(replays):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"replay {rep}: output {i} differs from the eager call"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_of_a_training_step():
    import bit_nf4_quantized_13_amd as q
    say("graph capture: quantize + fwd + bwd, M=1024 d=1024 k=2048 r=16")
    inp = make_layer(51, 0, 1024, 2048, 1024, 16)
    m, d, k, r, alpha = 1024, 1024, 2048, 16, 16.0
    w0 = to_dev_f32(inp.w0)
    x, a, b, dy = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    wq = q.NF4Weight.empty(d, k)
    qws = torch.empty(q.quantize_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    lws = torch.empty(q.linear_workspace_bytes(m, d, k, r), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((m, r), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((d, r), dtype=torch.float32, device="cuda")

    def step():
        q.qlora_nf4_quantize(w0, out=wq, workspace=qws)
        q.qlora_linear_fwd(wq, x, a, b, alpha, out=y, u_out=u, workspace=lws)
        q.qlora_linear_bwd(wq, x, dy, a, b, alpha, u=u, workspace=lws, outs=(dx, da, db))

    capture_and_check(step, [wq.codes, wq.absmax_q, wq.absmax_scale, wq.absmax_mean, y, u, dx, da, db])


@pytest.mark.parametrize("d", [512, 4096])
def test_graph_replay_of_decode(d):
    import bit_nf4_quantized_13_amd as q
    say(f"graph capture: decode d={d} k=4096 M=16 r=16")
    inp = make_layer(52, 0, d, 4096, 16, 16)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    x, a, b = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b))
    y = torch.empty((16, d), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    lws = torch.empty(q.linear_workspace_bytes(16, d, 4096, 16), dtype=torch.uint8, device="cuda")

    def step():
        q.qlora_linear_fwd(w, x, a, b, 32.0, out=y, u_out=u, workspace=lws)

    capture_and_check(step, [y, u])


@pytest.mark.parametrize("fmt", ["no_dq", "fp8"])
def test_graph_replay_of_a_dropout_step_in_other_formats(fmt):
    """The further weight formats and adapter dropout under capture: quantize,
    dropout forward and dropout backward (the mask regenerated from the seed in
    each replay) give the eager outputs bit for bit."""
    import bit_nf4_quantized_13_amd as q
    say(f"graph capture: {fmt} quantize + dropout fwd + bwd, M=600 d=512 k=1024 r=8")
    inp = make_layer(53, 0, 512, 1024, 600, 8)
    m, d, k, r, alpha, p, seed = 600, 512, 1024, 8, 16.0, 0.1, 77
    w0 = to_dev_f32(inp.w0)
    x, a, b, dy = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    wq = q.NF4Weight.empty(d, k, double_quant=fmt != "no_dq", c2_fp8=fmt == "fp8")
    qws = torch.empty(q.quantize_workspace_bytes(d, k, wq.dq_block), dtype=torch.uint8, device="cuda")
    lws = torch.empty(q.linear_workspace_bytes(m, d, k, r, dropout=True), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((m, r), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((d, r), dtype=torch.float32, device="cuda")

    def step():
        q.qlora_nf4_quantize(w0, out=wq, workspace=qws)
        q.qlora_linear_fwd(wq, x, a, b, alpha, out=y, u_out=u, workspace=lws, dropout=p, seed=seed)
        q.qlora_linear_bwd(wq, x, dy, a, b, alpha, u=u, workspace=lws, outs=(dx, da, db), dropout=p, seed=seed)

    outs = [wq.codes, wq.absmax_scale, y, u, dx, da, db] + ([wq.absmax_q, wq.absmax_mean] if fmt == "fp8" else [])
    capture_and_check(step, outs)
