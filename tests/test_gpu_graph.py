"""HIP-graph capture of the entry points: a captured block (attention boundary, FFN
boundary, FFN expand) replays to exactly the eager results, replay after replay,
with eager work and synchronisations in between (the library records no memsets,
allocations or host syncs). Decode size (64 tokens x 4 x 5120 bf16: 64-token
sweeps) and a ragged prefill-like size (1031 tokens x 4 x 1288 bf16: 128-token
sweeps). The eager block itself is checked against the oracle by the block parity
tests.
"""
import pytest
import torch

import hc_inputs
import hyper_connection_residual_mixes_amd as hc

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("w", [hc_inputs.DECODE, hc_inputs.Workload("graph_1031x1288", 1, 1031, 1288,
                                                                    torch.bfloat16)], ids=["decode", "wide"])
def test_block_graph_replays_match_eager(w):
    n, d = w.n, w.d
    inp = hc_inputs.block_inputs(w, seed=4, device=DEV)
    pi, _, _ = hc.hc_split_sinkhorn(*inp["prev"])
    ws = torch.empty(hc.workspace_size(n, 4, d), dtype=torch.uint8, device=DEV)
    o = dict(yA=torch.empty(n, d, dtype=w.dtype, device=DEV), yF=torch.empty(n, d, dtype=w.dtype, device=DEV),
             x1=torch.empty(n, 4, d, dtype=w.dtype, device=DEV), x2=torch.empty(n, 4, d, dtype=w.dtype, device=DEV),
             cA=tuple(torch.empty(sh, device=DEV) for sh in ((n, 4), (n, 4), (n, 4, 4))),
             cF=tuple(torch.empty(sh, device=DEV) for sh in ((n, 4), (n, 4), (n, 4, 4))))

    def step():
        a = hc.hc_fused_step(inp["x"], *inp["attn"], pre_mix=pi, y=o["yA"], out=o["cA"], workspace=ws)
        f = hc.hc_fused_step(inp["x"], *inp["ffn"], pre_mix=a["pre"], f_prev=inp["f_attn"], post_prev=a["post"],
                             comb_prev=a["comb"], streams_out=o["x1"], y=o["yF"], out=o["cF"], workspace=ws)
        hc.hc_post(inp["f_ffn"], f["streams"], f["post"], f["comb"], out=o["x2"])

    def outputs():
        return [o["yA"], o["yF"], o["x1"], o["x2"], *o["cA"], *o["cF"]]

    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in outputs():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(ref, outputs())):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager result"
        step()                        # eager work between replays
        torch.cuda.synchronize()
