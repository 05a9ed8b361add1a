"""The fixed 64-channel group INT8 baseline on the GPU against the oracle: codes and per-(token,
group) ranges bit-exact (prefix and one-token appends), decode within 2e-3; and its error next to
DGQ's on the same data (reported)."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu


def _f16_bits(x):
    return np.asarray(x, np.float16).view(np.uint16).astype(np.uint32)


def run_g64(cfg, seed, steps):
    k, v, cu, lens = dgq_data.batch_kv(cfg, seed)            # prefix + appended tokens
    bsz, hkv, d = cfg.batch, cfg.hkv, cfg.head_dim
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    params = H.params_for(cfg)
    cache = Q.DGQG64Cache(params, nblk)
    max_total = int((lens + steps).max())
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Q.dgq_g64_quantize(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), torch.from_numpy(pcu).cuda(),
                       dtable, cache, int(lens.max()), int(pcu[-1]), max_total)
    one = torch.arange(bsz + 1, dtype=torch.int32, device="cuda")
    for s in range(steps):
        pos = lens + s
        ktok = np.stack([k[cu[b] + pos[b]] for b in range(bsz)])
        vtok = np.stack([v[cu[b] + pos[b]] for b in range(bsz)])
        Q.dgq_g64_quantize(params, torch.from_numpy(ktok).cuda(), torch.from_numpy(vtok).cuda(), one, dtable, cache,
                           1, bsz, max_total, first_pos=torch.from_numpy(pos.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert int(cache.status[2].item()) == 0
    cur = lens + steps
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    kr, vr = cache.k_range.cpu().numpy().view(np.uint32), cache.v_range.cpu().numpy().view(np.uint32)
    koff, voff = PL.k_offsets(cfg.block_size, d), PL.v_offsets(cfg.block_size, d)
    heads = {}
    for b in range(bsz):
        for h in range(hkv):
            L = int(cur[b])
            kk, vv = k[cu[b]:cu[b] + L, h], v[cu[b]:cu[b] + L, h]
            kc, kmn, kmx = O.group64_compress(kk)
            vc, vmn, vmx = O.group64_compress(vv)
            H.compare_codes(PL.gather_head(kp, table[b], h, L, koff), kc, f"g64 K b{b} h{h}")
            H.compare_codes(PL.gather_head(vp, table[b], h, L, voff), vc, f"g64 V b{b} h{h}")
            t = np.arange(L)
            rows_k = kr[table[b][t // cfg.block_size], h, t % cfg.block_size]
            rows_v = vr[table[b][t // cfg.block_size], h, t % cfg.block_size]
            assert np.array_equal(rows_k & 0xFFFF, _f16_bits(kmn)) and np.array_equal(rows_k >> 16, _f16_bits(kmx))
            assert np.array_equal(rows_v & 0xFFFF, _f16_bits(vmn)) and np.array_equal(rows_v >> 16, _f16_bits(vmx))
            heads[(b, h)] = (O.group64_dequant(kc, kmn, kmx), O.group64_dequant(vc, vmn, vmx), kk, vv)
    q16 = dgq_data.queries(cfg, seed)
    out = Q.paged_decode_attn_g64(params, torch.from_numpy(q16).cuda(), cache, dtable,
                                  torch.from_numpy(cur.astype(np.int32)).cuda(), max_total).cpu().numpy()
    ref = np.zeros_like(out, dtype=np.float64)
    exact = np.zeros_like(ref)
    g = cfg.group
    for (b, h), (kh, vh, kk, vv) in heads.items():
        ref[b, h * g:(h + 1) * g] = O.decode_attention(q16[b, h * g:(h + 1) * g], kh, vh)
        exact[b, h * g:(h + 1) * g] = O.decode_attention(q16[b, h * g:(h + 1) * g], kk.astype(np.float64),
                                                         vv.astype(np.float64))
    err = H.rel_err_rows(out, ref)
    print(f"g64 decode vs oracle {err:.3e}; g64 vs fp16 attention {H.rel_err_rows(out, exact):.3e}")
    assert err <= 2e-3
    return out, exact


@pytest.mark.parametrize("cid,over,steps", [
    (5, dict(batch=3, seq_len=200, append_steps=70), 70),
    (2, dict(batch=2, seq_len=700, append_steps=20), 20),
    (1, dict(hq=4, block_size=64, seq_len=300, append_steps=9), 9),
    (1, dict(seq_len=300, append_steps=9), 9),
    (4, dict(batch=3, seq_len=600, hkv=4, hq=4, append_steps=10), 10),
], ids=["bs64_stream", "bs16_stream", "d64_g2", "d64_g1", "mha_g1_ragged"])
def test_g64_matches_oracle(cid, over, steps):
    cfg = dgq_data.get_config(cid, **over)
    H.say("g64", cid, over)
    run_g64(cfg, 31, steps)
