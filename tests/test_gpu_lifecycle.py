"""Block lifecycle on the GPU: forking a sequence over shared blocks with copy-on-write of the tail
block, swapping a sequence out to host memory and back into other blocks, and whole-block copies.

Expected values: the oracle's AppendState (a fork is a copy of the parent's state fed with the
child's tokens), and bit-identity with a twin cache that never left the device."""

import copy

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu


def _oracle_states(params, k, v, c0, length):
    p = params.c
    out = {}
    for h in range(p.num_kv_heads):
        kk, vv = k[c0:c0 + length, h], v[c0:c0 + length, h]
        out[h] = O.AppendState(O.compress_head(kk, vv, p.max_segments, p.tau, p.min_var, params.length_aware,
                                               H.fmt_of(params)),
                               kk, p.block_size, p.seg_capacity, p.tau, p.min_var)
    return out


def _block_bytes(cache, ids):
    i = torch.tensor(ids, dtype=torch.long, device=cache.k_pool.device)
    bits = None if cache.bits is None else cache.bits[i].cpu().numpy()
    return (cache.k_pool[i].cpu().numpy(), cache.v_pool[i].cpu().numpy(), bits)


def _check_rows(cache, params, table, states, rows, lens, qseed, cfg):
    """Segment rows, codes and bits of the listed cache rows against oracle states; decode too."""
    p = params.c
    heads = {(r, h): states[r][h].snapshot() for r in rows for h in range(p.num_kv_heads)}
    starts, prm, nseg = cache.segment_table()
    bits = H.identifier_bits(cache, table, lens)
    for (r, h), hc in heads.items():
        assert nseg[r, h] == len(hc.segs), (r, h)
        assert list(starts[r, h, :len(hc.segs)]) == [s.start for s in hc.segs], (r, h)
        kc, vc = H.read_codes(cache, table, r, h, hc.length)
        H.compare_codes(kc, hc.kcodes, f"K r{r} h{h}")
        H.compare_codes(vc, hc.vcodes, f"V r{r} h{h}")
        if params.marker:
            H.compare_markers(kc, hc.kcodes, f"K markers r{r} h{h}")
        assert np.array_equal(PL.gather_bits(bits, table[r], h, hc.length, p.block_size), hc.bits), (r, h)
    q16 = dgq_data.queries(cfg, qseed)
    dl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache, torch.from_numpy(table).cuda(),
                                   dl, int(max(lens))).cpu().numpy()
    ref = H.oracle_decode(q16, heads, lens, p.num_kv_heads, cfg.group)
    err = H.rel_err_rows(out[list(rows)], ref[list(rows)])
    print(f"decode vs oracle {err:.3e}", flush=True)
    assert err <= 2e-3


@pytest.mark.parametrize("l0,steps,marker", [(1000, 90, False), (960, 70, False), (1000, 90, True)],
                         ids=["mid_block", "block_aligned", "mid_block_marker"])
def test_fork_with_copy_on_write(l0, steps, marker):
    """Row 0 is compressed, row 1 forks from it (shared blocks, copied state row); both then append
    their own tokens.  The first append into the shared tail block copies it for one of them; the
    frozen shared blocks are never written."""
    cfg = dgq_data.get_config(5, batch=2, seq_len=l0 + steps, append_steps=0)
    H.say("fork with copy-on-write", l0, steps, marker)
    params = H.params_for(cfg, marker=marker)
    p = params.c
    bs = p.block_size
    k, v, cu, lens = dgq_data.batch_kv(cfg, 7)
    max_blocks = (l0 + steps + bs - 1) // bs
    nblk = 4 * max_blocks
    pool = Q.BlockPool(nblk)
    pool.alloc(5)                                     # so that row ids are not 0..n
    table = np.zeros((2, max_blocks), np.int32)
    n0 = (l0 + bs - 1) // bs
    table[0, :n0] = pool.alloc(n0)
    cache = Q.DGQCache(params, nblk, 2)
    dk = torch.from_numpy(np.ascontiguousarray(k[cu[0]:cu[0] + l0])).cuda()
    dv = torch.from_numpy(np.ascontiguousarray(v[cu[0]:cu[0] + l0])).cuda()
    Q.dgq_compress(params, dk, dv, torch.tensor([0, l0], dtype=torch.int32, device="cuda"),
                   torch.from_numpy(table).cuda(), cache, l0, l0)
    # fork: row 1 takes row 0's blocks and a copy of its state row
    table[1, :n0] = table[0, :n0]
    pool.share(list(table[0, :n0]))
    Q.dgq_copy_seq_state(params, cache, torch.tensor([0], dtype=torch.int32, device="cuda"),
                         torch.tensor([1], dtype=torch.int32, device="cuda"))
    frozen = list(table[0, :l0 // bs])
    before = _block_bytes(cache, frozen)
    parent = _oracle_states(params, k, v, cu[0], l0)
    states = {0: parent, 1: copy.deepcopy(parent)}
    tokens = {0: (k[cu[0] + l0:], v[cu[0] + l0:]), 1: (k[cu[1]:], v[cu[1]:])}
    ws = Q.workspace(Q.decode_workspace_size(params, 2, l0 + steps))
    copies = 0
    for s in range(steps):
        pos = l0 + s
        for r in (0, 1):
            j = pos // bs
            if pos % bs == 0:
                table[r, j] = pool.alloc(1)[0]
            else:
                new = pool.cow([int(table[r, j])])[0]
                if new != table[r, j]:
                    Q.dgq_copy_blocks(params, cache, torch.tensor([table[r, j]], dtype=torch.int32, device="cuda"),
                                      torch.tensor([new], dtype=torch.int32, device="cuda"))
                    table[r, j] = new
                    copies += 1
        dtable = torch.from_numpy(table).cuda()
        ktok = np.stack([tokens[r][0][s] for r in (0, 1)])
        vtok = np.stack([tokens[r][1][s] for r in (0, 1)])
        dpos = torch.full((2,), pos, dtype=torch.int32, device="cuda")
        if s % 2:
            q16 = dgq_data.queries(cfg, 11, 0, s)
            Q.dgq_append_decode(params, torch.from_numpy(ktok).cuda(), torch.from_numpy(vtok).cuda(), dpos,
                                torch.from_numpy(q16).cuda(), dtable, cache, l0 + steps, ws=ws)
        else:
            Q.dgq_append(params, torch.from_numpy(ktok).cuda(), torch.from_numpy(vtok).cuda(), dpos, dtable, cache)
        for r in (0, 1):
            for h in range(p.num_kv_heads):
                states[r][h].append(ktok[r, h], vtok[r, h])
        if s in (0, steps // 2, steps - 1):
            torch.cuda.synchronize()
            _check_rows(cache, params, table, states, (0, 1), [pos + 1, pos + 1], 100 + s, cfg)
    torch.cuda.synchronize()
    assert copies == (1 if l0 % bs else 0)
    after = _block_bytes(cache, frozen)
    for a, b in zip(before, after):
        assert (a is None and b is None) or np.array_equal(a, b), "a frozen shared block was written"
    for i in frozen:
        assert pool.refcount(int(i)) == 2
    assert int(cache.status[2].item()) == 0


@pytest.mark.parametrize("marker,bs", [(False, 64), (True, 64), (False, 32)], ids=["bitmap", "marker", "bitmap_bs32"])
def test_swap_out_and_in(marker, bs):
    """Row 1 is swapped out to pinned host memory mid-stream, its blocks and state are overwritten,
    and it is swapped back into other block ids; from then on every decode output and the final
    cache equal those of a twin cache that was never swapped."""
    cfg = dgq_data.get_config(5, batch=3, seq_len=300, append_steps=80, block_size=bs)
    H.say("swap out and in", cfg.batch, cfg.seq_len, marker, bs)
    params = H.params_for(cfg, marker=marker)
    p = params.c
    bs = p.block_size
    k, v, cu, lens = dgq_data.batch_kv(cfg, 9)
    lens = np.asarray(lens, np.int64)
    steps = cfg.append_steps
    max_blocks = int((lens.max() + steps + bs - 1) // bs)
    nblk = 3 * cfg.batch * max_blocks
    pool = Q.BlockPool(nblk)
    table = np.zeros((cfg.batch, max_blocks), np.int32)
    for b in range(cfg.batch):
        table[b] = pool.alloc(max_blocks)
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(cfg.batch)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(cfg.batch)])
    pcu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    caches = [Q.DGQCache(params, nblk, cfg.batch) for _ in range(2)]
    tables = [table.copy(), table.copy()]
    for c in caches:
        Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), pcu,
                       torch.from_numpy(table).cuda(), c, int(lens.max()), int(pk.shape[0]))
    states = {b: _oracle_states(params, k, v, cu[b], int(lens[b])) for b in range(cfg.batch)}
    max_total = int((lens + steps).max())
    swap_at = 40
    for s in range(steps):
        pos = lens + s
        if s == swap_at:
            torch.cuda.synchronize()
            row = 1
            ids_old = tables[1][row].copy()
            nbytes = Q.swap_image_bytes(params, max_blocks)
            staging = Q.workspace(nbytes)
            host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
            Q.dgq_swap_out(params, caches[1], row, torch.from_numpy(ids_old).cuda(), staging, host)
            torch.cuda.synchronize()
            pool.free(list(ids_old))
            # another owner takes and overwrites the blocks and the row
            idx = torch.from_numpy(ids_old.astype(np.int64)).cuda()
            caches[1].k_pool[idx] = 0x5A
            caches[1].v_pool[idx] = -0x21
            if caches[1].bits is not None:
                caches[1].bits[idx] = 0xFF
            for t in (caches[1].segs, caches[1].nseg, caches[1].tail, caches[1].k_stage, caches[1].v_stage):
                t[row].zero_()
            staging.zero_()
            pool.alloc(len(ids_old))   # the other owner takes the freed blocks (last freed first)
            ids_new = np.asarray(pool.alloc(max_blocks), np.int32)
            assert not set(ids_new) & set(ids_old)
            Q.dgq_swap_in(params, caches[1], row, torch.from_numpy(ids_new).cuda(), staging, host)
            tables[1][row] = ids_new
        ktok = torch.from_numpy(np.stack([k[cu[b] + pos[b]] for b in range(cfg.batch)])).cuda()
        vtok = torch.from_numpy(np.stack([v[cu[b] + pos[b]] for b in range(cfg.batch)])).cuda()
        dpos = torch.from_numpy(pos.astype(np.int32)).cuda()
        q = torch.from_numpy(dgq_data.queries(cfg, 13, 0, s)).cuda()
        outs = [Q.dgq_append_decode(params, ktok, vtok, dpos, q, torch.from_numpy(tables[i]).cuda(), caches[i],
                                    max_total) for i in range(2)]
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {s}: output differs after the swap"
        for b in range(cfg.batch):
            for h in range(p.num_kv_heads):
                states[b][h].append(ktok[b, h].cpu().numpy(), vtok[b, h].cpu().numpy())
    final = lens + steps
    _check_rows(caches[1], params, tables[1], states, (0, 1, 2), list(final), 77, cfg)
    for name in ("segs", "nseg", "tail", "k_stage", "v_stage"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    for b in range(cfg.batch):
        for h in range(p.num_kv_heads):
            a = H.read_codes(caches[0], tables[0], b, h, int(final[b]))
            c = H.read_codes(caches[1], tables[1], b, h, int(final[b]))
            assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1]), (b, h)
    assert int(caches[1].status[2].item()) == 0


def test_copy_blocks_bytes_and_bad_ids():
    """Whole-block copies are byte-exact for every kv head; a pair naming a block outside the pool
    is skipped and counted, and the other pairs are still copied."""
    cfg = dgq_data.get_config(2, batch=1, seq_len=64)
    params = H.params_for(cfg)
    p = params.c
    H.say("copy blocks")
    nblk = 40
    cache = Q.DGQCache(params, nblk, 1)
    rng = np.random.default_rng(5)
    cache.k_pool.copy_(torch.from_numpy(rng.integers(-128, 128, cache.k_pool.shape).astype(np.int8)))
    cache.v_pool.copy_(torch.from_numpy(rng.integers(-128, 128, cache.v_pool.shape).astype(np.int8)))
    cache.bits.copy_(torch.from_numpy(rng.integers(0, 256, cache.bits.shape).astype(np.uint8)))
    src = np.array([3, 7, 11, 2, 5], np.int32)
    dst = np.array([20, 21, nblk + 3, 22, 23], np.int32)
    ref = [cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy(), cache.bits.cpu().numpy()]
    Q.dgq_copy_blocks(params, cache, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    got = [cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy(), cache.bits.cpu().numpy()]
    for r, g in zip(ref, got):
        want = r.copy()
        for s_, d_ in zip(src, dst):
            if d_ < nblk:
                want[d_] = r[s_]
        assert np.array_equal(g, want)
    assert int(cache.status[2].item()) == 1
    # a state row copy with a row outside the cache is skipped and counted too
    Q.dgq_copy_seq_state(params, cache, torch.tensor([0], dtype=torch.int32, device="cuda"),
                         torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(cache.status[2].item()) == 2
    assert p.num_kv_heads == 8
