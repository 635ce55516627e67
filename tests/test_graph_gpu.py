"""The entry points under HIP graph capture (through torch.cuda.CUDAGraph).

The library allocates nothing, clears nothing and copies nothing on the host
side, so its launches can be captured: a serving loop of decode steps and a
whole GDN block (prologue, chunked forward, epilogue) are captured once and
replayed several times, with eager work and synchronisations between the
replays; every replay must equal the eager run bit for bit (the kernels are
deterministic and read the same inputs).
"""
import pytest

import gdn_inputs as gi
from gpu_util import dev_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    import gated_delta_rule_03_amd as g
    assert torch.cuda.is_available()
    g.load()
    return g


def test_decode_loop_graph_replays(gdn):
    import torch
    steps, B, H, d = 16, 4, 8, 128
    w = gi.generate(gi.Spec("graph-dec", B=B, T=steps, H_qk=H, H_v=H, d_k=d, d_v=d, dtype="bf16", chunk=64,
                            seed=500))
    q, k, v = (dev_tensor(x) for x in (w.q, w.k, w.v))
    al, be = dev_tensor(w.alpha), dev_tensor(w.beta)
    # per-step operands as separate contiguous buffers (the graph reads fixed addresses)
    ops = [tuple(t[:, s:s + 1].contiguous() for t in (q, k, v, al, be)) for s in range(steps)]
    state0 = dev_tensor(gi.random_state((B, H, d, d), seed=501, scale=0.3))
    outs = [torch.empty((B, 1, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    def loop(state):
        for s in range(steps):
            gdn.decode_step(*ops[s], state, o=outs[s])

    eager_state = state0.clone()
    loop(eager_state)
    torch.cuda.synchronize()
    eager_o = [o.clone() for o in outs]

    state = state0.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop(state)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        loop(state)
    for r in range(3):
        state.copy_(state0)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(state, eager_state) and all(torch.equal(a, b) for a, b in zip(outs, eager_o))
        log(f"[graph decode] replay {r}: identical to eager = {same}")
        assert same


def test_whole_block_graph_replays(gdn):
    import torch
    B, T, H, d = 2, 200, 4, 128
    x = gi.block_inputs(B, T, H, H, d, d, "bf16", seed=510)
    dv = {n: dev_tensor(x[n]) for n in ("q_raw", "k_raw", "v_raw", "conv_q", "conv_k", "conv_v", "conv_q_bias",
                                        "conv_k_bias", "conv_v_bias", "a_raw", "b_raw", "log_A", "v_norm", "g_raw",
                                        "o_norm")}
    outs = (torch.empty_like(dv["q_raw"]), torch.empty_like(dv["k_raw"]), torch.empty_like(dv["v_raw"]),
            torch.empty((B, T, H), device="cuda"), torch.empty((B, T, H), device="cuda"))
    o = torch.empty_like(dv["v_raw"])
    hT = torch.empty((B, H, d, d), device="cuda")
    y = torch.empty_like(dv["v_raw"])
    ws = torch.empty(gdn.chunk_fwd_workspace_bytes(B, T, H, H, d, d, gdn.GDN_BF16, 64, 0), dtype=torch.uint8,
                     device="cuda")

    def block():
        gdn.block_prologue(dv["q_raw"], dv["k_raw"], dv["v_raw"], dv["conv_q"], dv["conv_k"], dv["conv_v"],
                           dv["a_raw"], dv["b_raw"], dv["log_A"], conv_q_bias=dv["conv_q_bias"],
                           conv_k_bias=dv["conv_k_bias"], conv_v_bias=dv["conv_v_bias"], v_norm_weight=dv["v_norm"],
                           q_scale=d ** -0.5, out=outs)
        gdn.chunk_fwd(*outs, chunk=64, o=o, hT=hT, workspace=ws)
        gdn.block_epilogue(o, dv["g_raw"], o_norm_weight=dv["o_norm"], y=y)

    block()
    torch.cuda.synchronize()
    ref_y, ref_h = y.clone(), hT.clone()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        block()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        block()
    for r in range(3):
        y.fill_(0)
        hT.fill_(0)
        ws.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(y, ref_y) and torch.equal(hT, ref_h)
        log(f"[graph block] replay {r}: identical to eager = {same}")
        assert same and bool(torch.isfinite(y.float()).all())
