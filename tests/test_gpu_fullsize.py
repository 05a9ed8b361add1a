"""Parity at the workloads' full sizes, with the launches the benchmark makes.

Every workload runs whole on the GPU: the full batch is compressed in one call, the streaming
workload then appends and decodes step by step, and every decode covers the whole batch with
the same launch configuration the benchmark uses.  The oracle then checks (sequence, kv head)
units one at a time, every unit of the Llama-shaped layer, the 128K layer and the MHA batch and a
seeded sample of the streaming runs: segment table bit-exact, codes (acceptance bound),
boundary bits and tail state, and the decode outputs of that unit's query heads (max rel err
2e-3).  Inputs come from the device generator in dgq_data, and each sampled unit is copied back
to the host as the oracle's input, so both sides see the same fp16 values.
"""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu

SEED = 0

# (case id, workload id, overrides, sampled units, decode check steps of a streaming run,
#  marker format, fused append + decode)
CASES = [
    ("llama_layer_16x8192_append1", 2, dict(append_steps=1), 128, (0,), False, False),   # every unit
    ("long_context_131072_layer0", 3, {}, 8, (), False, False),   # every kv head of the layer
    ("mha_100_mixed_lengths", 4, {}, 3200, (), False, False),   # every unit
    ("streaming_64x2048_256steps", 5, {}, 128, (0, 63, 64, 255), False, False),
    ("streaming_64x2048_256steps_fused", 5, {}, 128, (0, 63, 64, 255), False, True),
    ("llama_layer_16x8192_append1_marker", 2, dict(append_steps=1), 128, (0,), True, False),
    ("streaming_64x2048_256steps_fused_marker", 5, {}, 32, (0, 127, 255), True, True),
]


def _units(cfg, n):
    rng = np.random.default_rng([SEED, cfg.cid, 99])
    pick = {(0, 0), (cfg.batch - 1, cfg.hkv - 1)}
    while len(pick) < min(n, cfg.batch * cfg.hkv):
        pick.add((int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))))
    return sorted(pick)


def _host_unit(x, cu, b, h, n):
    return x[int(cu[b]):int(cu[b]) + n, h].cpu().numpy()


def _prefix_pack(k, v, cu, lens):
    idx = torch.cat([torch.arange(int(cu[b]), int(cu[b]) + int(lens[b])) for b in range(len(lens))]).to(k.device)
    pcu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    return k.index_select(0, idx), v.index_select(0, idx), pcu


def _check_rows(out, q16, heads, group, what):
    worst = 0.0
    for (b, h), hc in heads.items():
        ref = O.decode_attention(q16[b, h * group:(h + 1) * group], hc.khat(), hc.vhat())
        worst = max(worst, H.rel_err_rows(out[b, h * group:(h + 1) * group], ref))
    print(f"{what}: sampled decode rows max rel err {worst:.3e}", flush=True)
    assert worst <= 2e-3, (what, worst)


@pytest.mark.parametrize("name,cid,over,nunits,checks,marker,fused", CASES, ids=[c[0] for c in CASES])
def test_full_size(name, cid, over, nunits, checks, marker, fused):
    cfg = dgq_data.get_config(cid, **over)
    steps = cfg.append_steps
    H.say("full-size", name, f"batch {cfg.batch} hkv {cfg.hkv} hq {cfg.hq} bs {cfg.block_size} steps {steps}")
    dev = torch.device("cuda")
    k, v, cu, lens = dgq_data.batch_kv_device(cfg, SEED, 0, dev)
    cu = cu.numpy().astype(np.int64)
    lens = np.asarray(lens, np.int64)
    pk, pv, pcu = _prefix_pack(k, v, cu, lens) if steps else (k, v, torch.from_numpy(cu.astype(np.int32)))
    total = int(pcu[-1])
    lmax = int(lens.max())
    table, nblk = dgq_data.block_tables(cfg, SEED, lens_total=lens + steps)
    dtable = torch.from_numpy(table).to(dev)
    params = H.params_for(cfg, marker=marker)
    p = params.c
    cache = Q.DGQCache(params, nblk, cfg.batch, dev)
    ws_c = Q.workspace(Q.compress_workspace_size(params, cfg.batch, total, lmax), dev)
    ws_d = Q.workspace(max(Q.decode_workspace_size(params, cfg.batch, lmax + s) for s in range(steps + 1)), dev)
    Q.dgq_compress(params, pk, pv, pcu.to(dev), dtable, cache, lmax, total, ws=ws_c)
    del pk, pv

    units = _units(cfg, nunits)
    host = {u: (_host_unit(k, cu, u[0], u[1], int(lens[u[0]]) + steps),
                _host_unit(v, cu, u[0], u[1], int(lens[u[0]]) + steps)) for u in units}
    states = {}
    for (b, h), (kk, vv) in host.items():
        n0 = int(lens[b])
        hc = O.compress_head(kk[:n0], vv[:n0], p.max_segments, p.tau, fmt=H.fmt_of(params))
        states[(b, h)] = O.AppendState(hc, kk[:n0], p.block_size, p.seg_capacity, p.tau)

    out = torch.empty((cfg.batch, cfg.hq, cfg.head_dim), dtype=torch.float32, device=dev)
    cu_dev = torch.from_numpy(cu).to(dev)
    lens_dev = torch.from_numpy(lens).to(dev)
    for s in range(steps):
        pos = lens_dev + s
        idx = cu_dev[:-1] + pos
        ktok, vtok = k.index_select(0, idx).contiguous(), v.index_select(0, idx).contiguous()
        q16 = dgq_data.queries(cfg, SEED, 0, s)
        if fused:
            Q.dgq_append_decode(params, ktok, vtok, pos.to(torch.int32), torch.from_numpy(q16).to(dev), dtable,
                                cache, lmax + s + 1, out=out, ws=ws_d)
        else:
            Q.dgq_append(params, ktok, vtok, pos.to(torch.int32), dtable, cache)
            Q.paged_decode_attn_int8(params, torch.from_numpy(q16).to(dev), cache, dtable, (pos + 1).to(torch.int32),
                                     lmax + s + 1, out=out, ws=ws_d)
        for (b, h), (kk, vv) in host.items():
            states[(b, h)].append(kk[int(lens[b]) + s], vv[int(lens[b]) + s])
        if s in checks:
            torch.cuda.synchronize()
            heads = {u: st.snapshot() for u, st in states.items()}
            _check_rows(out.cpu().numpy(), q16, heads, cfg.group, f"{name} step {s}")
    if not steps:
        q16 = dgq_data.queries(cfg, SEED)
        Q.paged_decode_attn_int8(params, torch.from_numpy(q16).to(dev), cache, dtable,
                                 torch.from_numpy(lens.astype(np.int32)).to(dev), lmax, out=out, ws=ws_d)
        torch.cuda.synchronize()
        _check_rows(out.cpu().numpy(), q16, {u: st.snapshot() for u, st in states.items()}, cfg.group, name)
    torch.cuda.synchronize()

    status = cache.status.cpu().numpy()
    assert status[1] == 0 and status[2] == 0, status
    assert status[0] == 0, "no workload here needs more segment rows than the table holds"
    starts, prm, nseg = cache.segment_table()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    bits = H.identifier_bits(cache, table, lens + steps)
    tails = cache.tail.cpu().numpy()
    koff, voff = PL.k_offsets(p.block_size, p.head_dim), PL.v_offsets(p.block_size, p.head_dim)
    for (b, h), st in states.items():
        hc = st.snapshot()
        assert nseg[b, h] == len(hc.segs), (b, h, nseg[b, h], hc.starts)
        for i, sg in enumerate(hc.segs):
            want = np.array([sg.kmin, sg.kmax, sg.vmin, sg.vmax, sg.kscale, sg.vscale], np.float32)
            assert starts[b, h, i] == sg.start and np.array_equal(prm[b, h, i].view(np.int32), want.view(np.int32)), \
                (b, h, i)
        H.compare_codes(PL.gather_head(kp, table[b], h, hc.length, koff), hc.kcodes, f"{name} K b{b} h{h}")
        H.compare_codes(PL.gather_head(vp, table[b], h, hc.length, voff), hc.vcodes, f"{name} V b{b} h{h}")
        if marker:
            H.compare_markers(PL.gather_head(kp, table[b], h, hc.length, koff), hc.kcodes, f"{name} K markers b{b} h{h}")
        assert np.array_equal(PL.gather_bits(bits, table[b], h, hc.length, p.block_size), hc.bits), (b, h)
        tl = tails[b, h]
        assert tl[0] == st.r0 and tl[1] == len(st.ring_a) and tl[2] == int(st.span_own), (b, h, tl[:3])
    print(f"{name}: {len(units)} units bit-exact; segments per head histogram "
          f"{np.bincount(nseg.reshape(-1), minlength=6).tolist()}", flush=True)


def test_full_size_group64_streaming():
    """The group-64 baseline on the streaming workload: 64 x 2048-token prefix quantized in one
    call, 256 one-token appends, decode over 2304 tokens; sampled units checked."""
    cfg = dgq_data.get_config(5)
    steps = cfg.append_steps
    H.say("full-size g64 streaming", cfg.batch, steps)
    dev = torch.device("cuda")
    k, v, cu, lens = dgq_data.batch_kv_device(cfg, SEED, 0, dev)
    cu = cu.numpy().astype(np.int64)
    lens = np.asarray(lens, np.int64)
    pk, pv, pcu = _prefix_pack(k, v, cu, lens)
    table, nblk = dgq_data.block_tables(cfg, SEED, lens_total=lens + steps)
    dtable = torch.from_numpy(table).to(dev)
    params = H.params_for(cfg)
    p = params.c
    cache = Q.DGQG64Cache(params, nblk, dev)
    max_total = int((lens + steps).max())
    Q.dgq_g64_quantize(params, pk, pv, pcu.to(dev), dtable, cache, int(lens.max()), int(pcu[-1]), max_total)
    cu_dev = torch.from_numpy(cu).to(dev)
    lens_dev = torch.from_numpy(lens).to(dev)
    one = torch.arange(cfg.batch + 1, dtype=torch.int32, device=dev)
    for s in range(steps):
        pos = lens_dev + s
        idx = cu_dev[:-1] + pos
        Q.dgq_g64_quantize(params, k.index_select(0, idx).contiguous(), v.index_select(0, idx).contiguous(), one,
                           dtable, cache, 1, cfg.batch, max_total, first_pos=pos.to(torch.int32))
    cur = lens + steps
    q16 = dgq_data.queries(cfg, SEED, 0, steps)
    out = Q.paged_decode_attn_g64(params, torch.from_numpy(q16).to(dev), cache, dtable,
                                  torch.from_numpy(cur.astype(np.int32)).to(dev), max_total).cpu().numpy()
    assert int(cache.status[2].item()) == 0
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    kr, vr = cache.k_range.cpu().numpy().view(np.uint32), cache.v_range.cpu().numpy().view(np.uint32)
    koff, voff = PL.k_offsets(p.block_size, p.head_dim), PL.v_offsets(p.block_size, p.head_dim)
    worst = 0.0
    for b, h in _units(cfg, 4):
        n = int(cur[b])
        kk, vv = _host_unit(k, cu, b, h, n), _host_unit(v, cu, b, h, n)
        kc, kmn, kmx = O.group64_compress(kk)
        vc, vmn, vmx = O.group64_compress(vv)
        H.compare_codes(PL.gather_head(kp, table[b], h, n, koff), kc, f"g64 K b{b} h{h}")
        H.compare_codes(PL.gather_head(vp, table[b], h, n, voff), vc, f"g64 V b{b} h{h}")
        t = np.arange(n)
        rk = kr[table[b][t // p.block_size], h, t % p.block_size]
        rv = vr[table[b][t // p.block_size], h, t % p.block_size]
        f16 = lambda x: np.asarray(x, np.float16).view(np.uint16).astype(np.uint32)  # noqa: E731
        assert np.array_equal(rk & 0xFFFF, f16(kmn)) and np.array_equal(rk >> 16, f16(kmx)), (b, h)
        assert np.array_equal(rv & 0xFFFF, f16(vmn)) and np.array_equal(rv >> 16, f16(vmx)), (b, h)
        g = cfg.group
        ref = O.decode_attention(q16[b, h * g:(h + 1) * g], O.group64_dequant(kc, kmn, kmx),
                                 O.group64_dequant(vc, vmn, vmx))
        worst = max(worst, H.rel_err_rows(out[b, h * g:(h + 1) * g], ref))
    print(f"g64 streaming: sampled decode rows max rel err {worst:.3e}", flush=True)
    assert worst <= 2e-3
