"""The streaming step under HIP graph capture: dgq_append_decode (or dgq_append followed by
paged_decode_attn_int8) is captured once and the graph is replayed step after step, with the
step's token, query and positions copied into the captured input buffers in between.  Every
replay's output must equal, bit for bit, the same call made eagerly on a second copy of the cache,
the two caches must be identical at the end, and the last step's output is checked against the
oracle.  The library issues no memset, allocation or synchronization inside these calls, so a
captured step holds only their kernel launches."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q
from test_gpu_fused import _same_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("marker", [False, True], ids=["bitmap", "marker"])
def test_streaming_step_graph_replays(mode, marker):
    cfg = dgq_data.get_config(5, batch=4, seq_len=200, append_steps=40)
    seed, steps = 31, 40
    H.say("graph replay", mode, "marker" if marker else "bitmap")
    k, v, cu, lens = dgq_data.batch_kv(cfg, seed)
    lens = np.asarray(lens, np.int64)
    params = H.params_for(cfg, marker=marker)
    p = params.c
    bsz, hkv = cfg.batch, cfg.hkv
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pcu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    max_total = int((lens + steps).max())
    eager, graphed = Q.DGQCache(params, nblk, bsz), Q.DGQCache(params, nblk, bsz)
    for c in (eager, graphed):
        Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), pcu, dtable, c,
                       int(lens.max()), int(pk.shape[0]))
    ws_e = Q.workspace(Q.decode_workspace_size(params, bsz, max_total))
    ws_g = Q.workspace(Q.decode_workspace_size(params, bsz, max_total))

    # captured input and output buffers
    ktok = torch.zeros((bsz, hkv, cfg.head_dim), dtype=torch.float16, device="cuda")
    vtok = torch.zeros_like(ktok)
    q = torch.zeros((bsz, cfg.hq, cfg.head_dim), dtype=torch.float16, device="cuda")
    pos = torch.zeros(bsz, dtype=torch.int32, device="cuda")
    pos1 = torch.zeros_like(pos)
    out_g = torch.zeros((bsz, cfg.hq, cfg.head_dim), dtype=torch.float32, device="cuda")
    out_e = torch.zeros_like(out_g)

    def step(cache, out, ws):
        if mode == "fused":
            Q.dgq_append_decode(params, ktok, vtok, pos, q, dtable, cache, max_total, out=out, ws=ws)
        else:
            Q.dgq_append(params, ktok, vtok, pos, dtable, cache)
            Q.paged_decode_attn_int8(params, q, cache, dtable, pos1, max_total, out=out, ws=ws)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(graphed, out_g, ws_g)
    torch.cuda.synchronize()
    # capture records launches without running them: the graphed cache is still the compressed prefix
    _same_cache(eager, graphed, table, lens, p)

    for s in range(steps):
        cur = lens + s
        ktok.copy_(torch.from_numpy(np.stack([k[cu[b] + cur[b]] for b in range(bsz)])))
        vtok.copy_(torch.from_numpy(np.stack([v[cu[b] + cur[b]] for b in range(bsz)])))
        q.copy_(torch.from_numpy(dgq_data.queries(cfg, seed, 0, s)))
        pos.copy_(torch.from_numpy(cur.astype(np.int32)))
        pos1.copy_(pos + 1)
        step(eager, out_e, ws_e)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_e, out_g), f"step {s}: replay differs from the eager call"
    _same_cache(eager, graphed, table, lens + steps, p)

    # the last output against the oracle's append states
    heads = {}
    for b in range(bsz):
        for h in range(hkv):
            kk, vv = k[cu[b]:cu[b] + lens[b], h], v[cu[b]:cu[b] + lens[b], h]
            st = O.AppendState(O.compress_head(kk, vv, p.max_segments, p.tau, p.min_var, params.length_aware,
                                               H.fmt_of(params)), kk, p.block_size, p.seg_capacity, p.tau, p.min_var)
            for s in range(steps):
                st.append(k[cu[b] + lens[b] + s, h], v[cu[b] + lens[b] + s, h])
            heads[(b, h)] = st.snapshot()
    ref = H.oracle_decode(dgq_data.queries(cfg, seed, 0, steps - 1), heads, lens + steps, hkv, cfg.group)
    err = H.rel_err_rows(out_g.cpu().numpy(), ref)
    assert err <= 2e-3, err
