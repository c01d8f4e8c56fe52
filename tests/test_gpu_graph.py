"""One encode + adaptation step captured in a HIP graph and replayed several times, each replay
on the same restored dictionary with eager work and synchronizations between the replays,
against the same step run eagerly: codes, replacements, atoms and usage counters bit-identical.
(The library's encode and adapt calls enqueue kernels only: no allocation, memset or
synchronization, so a caller may capture them.)"""
import pytest
import torch

from sparse_dictionary_coding_amd import fadkv, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("name,select", [("llama3b_decode", "gm"), ("llama3b_decode", "pl"),
                                         ("qwen4b_long_decode", "gm")])
def test_graph_replay_matches_eager_step(name, select):
    print(f"[gpu-graph] {name} {select}", flush=True)
    w = synth.WORKLOADS[name]
    g = synth.SyntheticKV(w, device=DEV)
    A0 = g.atoms()
    X = g.batch(A0, step=3)
    U0 = torch.zeros(w.num_dicts, w.N, dtype=torch.int32, device=DEV)
    U0[:, : w.N // 2] = 2          # half the atoms in use: the drifted rows find inactive slots
    p = fadkv.Params(n=w.n, s=w.s, select=select)
    T, M = w.num_dicts, w.M
    A, U = A0.clone(), U0.clone()
    pool = fadkv.Pool.empty(T, M, w.n, DEV)
    codes = fadkv.Codes.empty(T, M, w.s, DEV)
    replaced = torch.empty(T, M, dtype=torch.int32, device=DEV)
    ws = fadkv.make_workspace(A, p, M)

    def step(stream):
        fadkv.fadkv_screen(A, X, p, out=pool, stream=stream)
        fadkv.fadkv_select_support(A, X, p, pool, out=codes, stream=stream)
        fadkv.fadkv_adapt(A, U, X, codes, p, replaced=replaced, workspace=ws, stream=stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in (codes.idx, codes.coef, codes.relerr, codes.flags, replaced, A, U)]
    assert int((replaced >= 0).sum()) > 0          # the step really replaces atoms

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: restore the step-start state and scribble the outputs
        A.copy_(A0)
        U.copy_(U0)
        for t in (codes.idx, replaced):
            t.fill_(-7)
        codes.coef.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (codes.idx, codes.coef, codes.relerr, codes.flags, replaced, A, U)
        for i, (r, gt) in enumerate(zip(ref, got)):
            assert torch.equal(r, gt), f"replay {rep}: output {i} differs from the eager step"
