"""The library's calls under HIP graph capture, as a serving loop replays a
decode step: a few layers of the one-launch decode step (forced splits, so
the cross-split counters and partial states in the workspace are used), a
multi-token call and a copy-on-write block copy are captured once, then the
graph is replayed several times with eager work and synchronisations in
between.  Every replay must give the eager result bit for bit; the eager
result itself is checked against the oracle.  No call allocates or clears
memory inside the capture."""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu


def _layer_cases(wl, layers):
    return [Case(wl) for _ in range(layers)]


@pytest.mark.parametrize("types", [("bf16", "bf16", "bf16"), ("bf16", "fp8", "bf16")], ids=lambda t: "-".join(t))
def test_graph_replays_match_eager(types):
    contexts = (1, 17, 300, 825, 0, 2000)
    wl = workloads.Workload("graph-" + types[1], len(contexts), 16, 2, 128, 16, *types, 81, contexts=contexts,
                            extra_blocks=40)
    check_graph(wl, splits=3, m=4)


def test_graph_replays_with_the_lds_ring():
    """100 sequences x 8 KV heads: 800 workgroups, so the decode step and the
    several-token call (2 query heads x 4 tokens: one row tile) load K/V
    through the LDS ring inside the captured graph."""
    contexts = tuple((1, 17, 300, 825, 0, 2000)[i % 6] for i in range(100))
    wl = workloads.Workload("graph-ring", len(contexts), 16, 8, 128, 16, "bf16", "bf16", "bf16", 83,
                            contexts=contexts, extra_blocks=40)
    check_graph(wl, splits=1, m=4, layers=2)


def check_graph(wl, splits, m, layers=3):
    cases = _layer_cases(wl, layers)
    plan = cases[0].plan
    stream = torch.cuda.Stream()
    outs = [torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda") for _ in cases]
    ws = pkv.make_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, plan.max_context_len, splits)
    qm, qs = workloads.multi_queries(wl, [m] * wl.num_seqs, device="cuda")
    qs_t = torch.from_numpy(qs).cuda()
    out_m = torch.empty((qm.shape[0], wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
    ws_m = pkv.make_multi_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, m,
                                    plan.max_context_len, splits)
    free = [b for b in range(plan.num_blocks) if b not in set(cases[0].rp.block_tables.ravel().tolist())]
    pairs = torch.tensor([[free[0], free[1]], [free[2], free[3]]], dtype=torch.int32).cuda()
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        calls = [pkv.prepare_decode_step(o, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, c.block_tables,
                                         c.context_lens, max_context_len=plan.max_context_len, workspace=ws,
                                         k_scale=c.t.k_scale, v_scale=c.t.v_scale, num_splits=splits, stream=stream)
                 for o, c in zip(outs, cases)]
        c0 = cases[-1]
        calls.append(pkv.prepare_paged_attention_multi(out_m, qm, c0.t.k_cache, c0.t.v_cache, c0.block_tables,
                                                       c0.context_lens, qs_t, max_query_len=m,
                                                       max_context_len=plan.max_context_len, workspace=ws_m,
                                                       k_scale=c0.t.k_scale, v_scale=c0.t.v_scale,
                                                       num_splits=splits, stream=stream))
        cow = lambda: pkv.pkv_copy_blocks(cases[0].t.k_cache, cases[0].t.v_cache, pairs, stream=stream)
        print(f"[case] {wl.name} eager", flush=True)
        for call in calls:
            call()
        cow()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs] + [out_m.clone()]
    pools = [to_bits(cases[0].t.k_cache).copy(), to_bits(cases[0].t.v_cache).copy()]

    # the eager step is right: the oracle on the first and last layer
    for c, o in ((cases[0], eager[0]), (cases[-1], eager[layers - 1])):
        assert_close(o, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name}-eager")
    assert_close(out_m, cases[-1].oracle_multi(qm, qs), wl.kv_dtype, label=f"{wl.name}-multi-eager")

    graph = torch.cuda.CUDAGraph()
    print(f"[case] {wl.name} capture", flush=True)
    with torch.cuda.graph(graph, stream=stream):
        for call in calls:
            call()
        cow()
    torch.cuda.synchronize()
    for r in range(4):
        for o in outs + [out_m]:
            o.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        print(f"[case] {wl.name} replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs + [out_m]):
            assert torch.equal(o, eager[i]), f"replay {r}: output {i} differs from the eager call"
        assert np.array_equal(to_bits(cases[0].t.k_cache), pools[0]), f"replay {r}: K pool"
        assert np.array_equal(to_bits(cases[0].t.v_cache), pools[1]), f"replay {r}: V pool"
