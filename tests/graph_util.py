"""HIP-graph replay check shared by the GPU tests: a step captured into a graph must
reproduce its eager results on every replay, with eager work (a NaN fill of every
output) between the replays."""
import torch


def assert_replays_match_eager(step, outs, replays=3):
    """step() enqueues the calls on the current stream and writes the tensors in outs."""
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(replays):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else -1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(t, w), (rep, i)
