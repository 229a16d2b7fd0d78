"""Decode calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with the program's own eager work and synchronisations between
the replays, gives the eager result bit for bit.  The library's launches take
the caller's stream and workspace, record no memset and allocate nothing when
o and the workspace are given, so a captured call is the eager call."""
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import synth
from gpu_cases import hip_run, hip_run_k_eq_v, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


# (variant, dtype, B, capacity, paged, window, values_only, expected mode)
SHAPES = {
    "sliding-unit": ("sliding", "bf16", 64, 1104, False, None, False, "unit"),
    "sliding-stream-paged": ("sliding", "bf16", 4, 4096, True, None, False, "stream"),
    "sliding-f32-stream": ("sliding", "f32", 4, 2048, False, None, False, "stream"),
    "window-stream": ("sliding", "bf16", 4, 9008, True, 4096, False, "stream"),
    "global-unit": ("global", "bf16", 256, 512, False, None, False, "unit"),
    "global-group-paged": ("global", "bf16", 3, 16384, True, None, False, "group"),
    "values-only-group": ("global", "bf16", 3, 16384, True, None, True, "group"),
}


def _case(key, seed):
    variant, dtype, B, cap, paged, window, kfv, mode = SHAPES[key]
    assert gqa.gqa_decode_plan(variant, B, cap, window=window)["mode"] == mode
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, seed).tolist()
    lens[0] = cap
    c = to_gpu(synth.make_case(variant, dtype, B, cap, lens, paged=paged, seed=seed,
                               window=window))
    ws = torch.empty(max(gqa.gqa_decode_workspace_bytes(variant, B, cap, window), 256),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(c.q)
    if kfv:
        return c, lambda: hip_run_k_eq_v(c, workspace=ws, o=o), o, ws
    return c, lambda: hip_run(c, workspace=ws, o=o, window=window), o, ws


def _replay_matches(graph, outs_and_refs, ws_list):
    for rep in range(4):
        # eager work between replays: scribble over the outputs and workspaces
        # (NaN bytes) and run an unrelated product on the current stream
        for o, _ in outs_and_refs:
            o.view(torch.uint8).fill_(0xFF)
        for ws in ws_list:
            ws.fill_(0xFF)
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(outs_and_refs):
            assert torch.equal(o, ref), (rep, i)


@pytest.mark.parametrize("key", sorted(SHAPES))
def test_graph_replay_equals_eager(key):
    c, call, o, ws = _case(key, 900 + len(key))
    call()
    torch.cuda.synchronize()
    ref = o.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_matches(g, [(o, ref)], [ws])


def test_graph_of_several_calls():
    # a sliding and a global call, each twice, in one graph (the second of
    # each pair reuses the first's workspace)
    parts = [_case("sliding-stream-paged", 950), _case("global-group-paged", 951)]
    refs = []
    for _, call, o, _ in parts:
        call()
        torch.cuda.synchronize()
        refs.append(o.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, call, _, _ in parts:
            call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, call, _, _ in parts + parts:
            call()
    _replay_matches(g, [(p[2], r) for p, r in zip(parts, refs)], [p[3] for p in parts])
