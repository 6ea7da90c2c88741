"""The library's calls captured in a HIP graph (through torch.cuda.graph) and
replayed.  No call allocates, synchronizes or records a memset (the s_g slot
and other counters are cleared by kernels), so a captured sequence replays
like the eager one: every replay is compared bit for bit with the eager
results, with other eager library work and synchronizations between replays,
and again after new data has been copied into the captured input buffers."""
import pytest
import torch

from tests.gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


def _nv():
    from long_video_dit_amd import nvfp4
    return nvfp4


def test_graph_replays_match_eager():
    nv = _nv()
    gen = torch.Generator().manual_seed(4242)
    bf = torch.bfloat16

    def inputs(scale):
        return (torch.randn(2048, 3072, generator=gen).mul(scale).to(bf),
                torch.randn(8, 2048, 128, generator=gen).mul(scale).to(bf),
                torch.randn(8, 256, 128, generator=gen).to(bf))

    a_h, kv_h, q_h = inputs(1.0)
    a, kv, q = a_h.to(dev()), kv_h.to(dev()), q_h.to(dev())
    wq = nv.quantize((torch.randn(3072, 3072, generator=gen) * 0.02).to(bf).to(dev()))
    # static outputs, allocated once
    aq = nv.quantize(a)
    c = nv.gemm(aq, wq)
    kq = nv.kv_quantize(kv)
    deq = nv.kv_dequantize(*kq)
    sg = nv.global_scale(a)
    ws = torch.empty(nv.kv_attention_workspace_size(8, 256, 2048), dtype=torch.uint8, device=dev())
    o = nv.kv_attention(q, kq, kq, workspace=ws)
    outs = list(aq) + [c] + list(kq) + [deq, sg, o]

    def run():
        nv.quantize(a, out=aq[:2], s_g_out=aq[2])
        nv.gemm(aq, wq, out=c)
        nv.kv_quantize(kv, out=kq)
        nv.kv_dequantize(*kq, out=deq)
        nv.global_scale(a, out=sg)
        nv.kv_attention(q, kq, kq, out=o, workspace=ws)

    def eager_reference():
        run()
        torch.cuda.synchronize()
        return [t.clone() for t in outs]

    want = eager_reference()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    other = torch.randn(512, 1024, generator=gen).to(bf).to(dev())
    for data in range(2):
        if data:  # new inputs in the captured buffers, new eager reference
            a_h, kv_h, q_h = inputs(3.5)
            a.copy_(a_h.to(dev()))
            kv.copy_(kv_h.to(dev()))
            q.copy_(q_h.to(dev()))
            torch.cuda.synchronize()
            want = eager_reference()
            for t in outs:
                t.zero_()
            torch.cuda.synchronize()
        for rep in range(3):
            log("graph replay, data", data, "replay", rep)
            graph.replay()
            torch.cuda.synchronize()
            for i, (g, x) in enumerate(zip(outs, want)):
                assert torch.equal(g, x), "output %d differs on replay %d (data %d)" % (i, rep, data)
            nv.quantize(other)  # eager library work between replays
            torch.cuda.synchronize()
