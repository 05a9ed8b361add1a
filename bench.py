"""Benchmark of the DGQ hot path on one MI355X.

One step = one pass of the whole path over one batch of the Llama-3-8B-shaped layer workload
(16 sequences x 8192 tokens, 8 KV / 32 query heads, head_dim 128, 16-token blocks shuffled in
the pool):

  1. dgq_compress        the batch's fp16 K/V (16 x 8192 tokens) into INT8 DGQ blocks;
  2. dgq_append          one fp16 token per sequence into that cache;
  3. paged_decode_attn_int8  one decode query per sequence over a cache of 8193 tokens.

Four caches rotate: step i compresses and appends into cache i % 4 and decodes cache (i+2) % 4,
which was written two steps earlier, so the decode's 256 MiB of codes are read from HBM and not
from the 256 MB Infinity Cache.  Inputs are resident in HBM before the timed region.

After the timed DGQ steps, the fixed 64-channel group INT8 baseline runs the same step shape on
the same data (quantize the batch + the appended token, decode over 8193 tokens; two caches
rotate), and both decoders' outputs are compared with float32 attention over the unquantized
fp16 keys/values ("group64_baseline", "quality_vs_fp16").

The segment-count policies (segment cap, tau, the length-aware cap, the variance floor) are then
run on the same batch: segment histogram, compress time and error against fp16 attention
("segment_policies"), and both storage formats of the segment identifier, the bit tensor and the
marker bytes inside the codes, are compared on it ("identifier_formats").  The streaming workload (64 x 2048-token prefixes, 256 append + decode steps) is timed three
ways: two launches per step, the fused append + decode, and the group-64 baseline ("streaming").
Finally the 128K long-context workload (32 layers of one 131,072-token sequence, each layer
compressed into its own cache, decode looped over the layers) is timed per layer
("long_context_128k").

Prints one JSON line.  ``value`` is the decode attention's throughput in GB/s of algorithmic
bytes (INT8 K/V codes + block table + segment tables + q + out), from HIP events recorded around
every decode call on the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


class Timer:
    """HIP events for timing only, recorded on torch's current stream (the stream every library
    call runs on).  They are created with hipEventDisableSystemFence: a timing event needs no
    system-scope cache write-back and invalidate, and without it the fence's cost lands inside the
    interval being timed (about 2 us per event pair on a 60 us kernel)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch

        if Timer._hip is None:
            # the HIP runtime already in the process (torch's and the library's): load nothing new
            Timer._hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
            Timer._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                       ctypes.c_void_p]
            Timer._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            Timer._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            Timer._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._ctypes = ctypes
        self._torch = torch
        self.ev = ctypes.c_void_p()
        err = Timer._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), Timer.DISABLE_SYSTEM_FENCE)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")

    def record(self):
        err = Timer._hip.hipEventRecord(self.ev, self._torch.cuda.current_stream().cuda_stream)
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def elapsed_time(self, end: "Timer") -> float:
        """Milliseconds from this event to ``end`` (both recorded and complete)."""
        ms = self._ctypes.c_float()
        err = Timer._hip.hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(ms.value)

    def __del__(self):
        try:
            if self.ev:
                Timer._hip.hipEventDestroy(self.ev)
        except Exception:
            pass


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="time budget of the CPU oracle baseline (0 to skip)")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the streaming, high-concurrency, tiny and 32-layer 128K long-context figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (torch) a few times: the reference "
                         "kernel of known size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


DECODE_SOURCES = ("decode.hip", "decode_common.h", "dgq_internal.h")


def kernel_source_digest() -> str:
    """Digest of the sources the INT8 decode kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_paged_kv_dgq_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


COMPRESS_SOURCES = ("compress.hip", "dgq_internal.h")


def compress_source_digest() -> str:
    """Digest of the sources the compress kernels are compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in COMPRESS_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_paged_kv_dgq_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(what: str = "decode"):
    """HBM bytes per decode launch ("decode") or per dgq_compress call ("compress") from the
    committed counter profile, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_llama3_8b_layer_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split("#", 1)[0].strip()
    digest = kernel_source_digest() if what == "decode" else compress_source_digest()
    key = "decode_hbm_bytes_per_launch" if what == "decode" else "compress_hbm_bytes_per_call"
    if kv.get(f"{what}_source_sha256_16") != digest:
        return None
    try:
        return int(float(kv[key]))
    except (KeyError, ValueError):
        return None


def kernel_trace_decode_us():
    """Kernel-trace average duration of the step's decode launches (the Llama-3-8B-shaped layer
    decodes that follow the step's append) from the committed rocprofv3 summary, if it was taken
    on the current decode sources (else None).  HIP events recorded around one kernel also count
    the queue time the start event adds before the kernel (about 2-4 us here)."""
    path = os.path.join(ROOT, "profiles", "llama3_8b_layer_step_kernel_trace.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split("#", 1)[0].strip()
    if kv.get("decode_source_sha256_16") != kernel_source_digest():
        return None
    try:
        return float(kv["decode_c2_step_avg_us"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch

    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 512 << 20, "bytes_written": 512 << 20, "launches": 5}}))


def achievable_copy(dev):
    """A plain device copy of 512 MiB (torch's copy kernel), timed like the library's kernels:
    the bandwidth a simple streaming kernel reaches on this GPU, as a second yardstick beside the
    8 TB/s data-sheet peak.  Bytes counted: read + written."""
    import torch

    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = []
    for _ in range(10):
        e0, e1 = Timer(), Timer()
        e0.record()
        dst.copy_(src)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    del src, dst
    return {"bytes": 2 * (512 << 20), "us": round(us, 2), "gbs": round(2 * (512 << 20) / us / 1e3, 1)}


def cpu_baseline(cfg, seed, budget_s):
    """The oracle as it is, on one host core, on a bounded sample of the same workload: whole
    (sequence, kv head) units of config 2 until the budget is spent."""
    from threadpoolctl import threadpool_limits

    import dgq_data
    from oracle import dgq_oracle as O

    q16 = dgq_data.queries(cfg, seed)
    units = [(b, h) for b in range(cfg.batch) for h in range(cfg.hkv)]
    t_comp = t_dec = 0.0
    done = 0
    tokens = 0
    with threadpool_limits(limits=1):
        start = time.perf_counter()
        for b, h in units:
            k, v = dgq_data.head_kv(cfg, seed, 0, b, h, cfg.seq_len)
            t0 = time.perf_counter()
            hc = O.compress_head(k, v)
            t1 = time.perf_counter()
            O.decode_attention(q16[b, h * cfg.group:(h + 1) * cfg.group], hc.khat(), hc.vhat())
            t2 = time.perf_counter()
            t_comp += t1 - t0
            t_dec += t2 - t1
            done += 1
            tokens += cfg.seq_len
            if time.perf_counter() - start > budget_s and done >= 2:
                break
    dec_bytes = done * 2 * cfg.seq_len * cfg.head_dim
    return {
        "value": dec_bytes / t_dec / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {len(units)} (sequence, kv head) units of the {cfg.seq_len}-token layer; "
                  f"decode = dequantize + float64 attention for the {cfg.group} query heads",
        "compress_tokens_per_s": tokens / t_comp,
        "seconds": t_comp + t_dec,
        "all_cores": cpu_baseline_parallel(cfg, seed, units[:max(done, 1) * 4]),
    }


def _oracle_unit(args):
    """One (sequence, kv head) unit through the oracle on one core: (compress s, decode s)."""
    cid, seed, b, h = args
    from threadpoolctl import threadpool_limits

    import dgq_data
    from oracle import dgq_oracle as O

    cfg = dgq_data.get_config(cid)
    q16 = dgq_data.queries(cfg, seed)
    with threadpool_limits(limits=1):
        k, v = dgq_data.head_kv(cfg, seed, 0, b, h, cfg.seq_len)
        t0 = time.perf_counter()
        hc = O.compress_head(k, v)
        t1 = time.perf_counter()
        O.decode_attention(q16[b, h * cfg.group:(h + 1) * cfg.group], hc.khat(), hc.vhat())
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def cpu_baseline_parallel(cfg, seed, units):
    """The same oracle fanned out over (sequence, kv head) units, one process per allowed core
    (at most 16): the units are independent.  Each process times its own compress and decode
    while all of them run; throughput = bytes (tokens) / summed seconds x processes, i.e. the
    rate of that many cores each busy with the oracle."""
    import multiprocessing as mp

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    args = [(cfg.cid, seed, b, h) for b, h in units]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        times = pool.map(_oracle_unit, args, chunksize=1)
    wall = time.perf_counter() - t0
    t_comp = float(sum(a for a, _ in times))
    t_dec = float(sum(b for _, b in times))
    dec_bytes = len(units) * 2 * cfg.seq_len * cfg.head_dim
    return {"value": dec_bytes / t_dec * cores / 1e9, "unit": "GB/s", "cores": cores, "units": len(units),
            "compress_tokens_per_s": len(units) * cfg.seq_len / t_comp * cores, "wall_seconds": wall}


def fp16_reference(cfg, k, v, cu, q, k_tok=None, v_tok=None):
    """float32 attention of q over the unquantized fp16 keys/values (plus one appended token)."""
    import torch

    B, hkv, hq, d = cfg.batch, cfg.hkv, cfg.hq, cfg.head_dim
    G = hq // hkv
    ref = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    for b in range(B):
        a, e = int(cu[b]), int(cu[b + 1])
        kb, vb = k[a:e], v[a:e]
        if k_tok is not None:
            kb, vb = torch.cat([kb, k_tok[b:b + 1]]), torch.cat([vb, v_tok[b:b + 1]])
        kb = kb.float().permute(1, 0, 2).contiguous()   # [hkv][L][d]
        vb = vb.float().permute(1, 0, 2).contiguous()
        qb = q[b].float().view(hkv, G, d).contiguous()
        sc = torch.bmm(qb, kb.transpose(1, 2).contiguous()) / math.sqrt(d)
        ref[b] = torch.bmm(torch.softmax(sc, dim=-1), vb).reshape(hq, d)
    return ref


def rel_err_rows(o, ref):
    """(max, mean) over (sequence, query head) of ||o - ref||_inf / ||ref||_inf."""
    r = (o - ref).abs().amax(-1) / ref.abs().amax(-1)
    return float(r.max()), float(r.mean())


def quality_vs_fp16(cfg, k, v, cu, k_tok, v_tok, q, out_dgq, out_g64):
    """Max and mean over (sequence, query head) of ||o - o_fp16||_inf / ||o_fp16||_inf, where
    o_fp16 is float32 attention over the unquantized fp16 keys/values (all 8193 tokens)."""
    ref = fp16_reference(cfg, k, v, cu, q, k_tok, v_tok)
    e1, e2 = rel_err_rows(out_dgq, ref), rel_err_rows(out_g64, ref)
    return {"dgq_max_rel_err": round(e1[0], 6), "dgq_mean_rel_err": round(e1[1], 6),
            "group64_max_rel_err": round(e2[0], 6), "group64_mean_rel_err": round(e2[1], 6),
            "rows": cfg.batch * cfg.hq, "reference": "float32 attention over the unquantized fp16 K/V"}


POLICIES = [
    ("default: max 5 segments, tau 2", {}),
    ("max 3 segments", dict(max_segments=3)),
    ("max 8 segments", dict(max_segments=8)),
    ("tau 4", dict(tau=4.0)),
    ("length-aware cap (3 at 8192 tokens)", dict(length_aware=True)),
    ("variance floor 1e-3", dict(min_var=1e-3)),
    ("variance floor 1e-2", dict(min_var=1e-2)),
    ("variance floor 4e-2", dict(min_var=4e-2)),
    ("variance floor 1e-2, length-aware cap", dict(min_var=1e-2, length_aware=True)),
]


def segment_policies(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q):
    """Segment-count policies on the same batch (8192 tokens per sequence, no append): segment
    histogram, compress time (HIP events, median of 5) and decode error against float32
    attention over the unquantized keys/values."""
    import torch

    B, L, hkv, hq, d, bs = cfg.batch, cfg.seq_len, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    total = int(cu[-1])
    ref = fp16_reference(cfg, k, v, cu, q)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    rows = []
    for name, kw in POLICIES:
        params = Q.DGQParams(hkv, hq, d, bs, seg_capacity=16, **kw)
        cache = Q.DGQCache(params, nblk, B, dev)
        ws = Q.workspace(Q.compress_workspace_size(params, B, total, L), dev)
        ts = []
        for _ in range(5):
            e0, e1 = Timer(), Timer()
            e0.record()
            Q.dgq_compress(params, k, v, dcu, dtable, cache, L, total, ws=ws)
            e1.record()
            ts.append((e0, e1))
        out = Q.paged_decode_attn_int8(params, q, cache, dtable, lens, L)
        torch.cuda.synchronize()
        nseg = cache.nseg.cpu().numpy().reshape(-1)
        err = rel_err_rows(out, ref)
        rows.append({"policy": name, "segments_hist": np.bincount(nseg, minlength=9).tolist(),
                     "mean_segments": round(float(nseg.mean()), 3),
                     "compress_us": round(float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3, 2),
                     "max_rel_err_vs_fp16": round(err[0], 6), "mean_rel_err_vs_fp16": round(err[1], 6)})
        del cache, ws
    return rows


def marker_format(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q):
    """The two storage formats of the segment identifier on the same batch (DGQ article 3.2): the
    bit tensor, and the marker bytes inside the key codes (254 data levels, no bit tensor).
    Compress and decode time (HIP events, mean of 6; three caches rotate so every decode reads a
    cache written two compressions earlier), the marker read-back, stored bytes and the error
    against float32 attention over the unquantized keys/values."""
    import torch

    B, L, hkv, hq, d, bs = cfg.batch, cfg.seq_len, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    total = int(cu[-1])
    ref = fp16_reference(cfg, k, v, cu, q)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    rows = {}
    for fmt in ("bitmap", "marker"):
        params = Q.DGQParams(hkv, hq, d, bs, marker=(fmt == "marker"))
        caches = [Q.DGQCache(params, nblk, B, dev) for _ in range(3)]
        ws = Q.workspace(Q.compress_workspace_size(params, B, total, L), dev)
        wsd = Q.workspace(Q.decode_workspace_size(params, B, L), dev)
        out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
        for c in caches:
            Q.dgq_compress(params, k, v, dcu, dtable, c, L, total, ws=ws)
        ev = []
        for i in range(8):
            e = [Timer() for _ in range(3)]
            e[0].record()
            Q.dgq_compress(params, k, v, dcu, dtable, caches[i % 3], L, total, ws=ws)
            e[1].record()
            Q.paged_decode_attn_int8(params, q, caches[(i + 1) % 3], dtable, lens, L, out=out, ws=wsd)
            e[2].record()
            ev.append(e)
        torch.cuda.synchronize()
        ev = ev[2:]
        comp_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
        dec_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
        err = rel_err_rows(out, ref)
        nseg = caches[0].nseg.cpu().numpy().reshape(-1)
        row = {"compress_us": round(comp_us, 2), "decode_us": round(dec_us, 2),
               "max_rel_err_vs_fp16": round(err[0], 6), "mean_rel_err_vs_fp16": round(err[1], 6),
               "code_bytes": int(B * L * hkv * d * 2),
               "identifier_bytes": int(B * L * hkv // 8) if fmt == "bitmap" else 0,
               "segment_table_bytes": int(nseg.sum()) * 32}
        if fmt == "marker":
            got = torch.zeros_like(rows["bitmap"]["_bits"])
            Q.dgq_marker_bits(params, caches[0], dtable, lens, L, out=got)     # warm-up
            e0, e1 = Timer(), Timer()
            e0.record()
            for _ in range(5):
                Q.dgq_marker_bits(params, caches[0], dtable, lens, L, out=got)
            e1.record()
            torch.cuda.synchronize()
            row["marker_readback_us"] = round(e0.elapsed_time(e1) * 1e3 / 5, 2)
            row["readback_equals_bit_tensor"] = bool(torch.equal(got, rows["bitmap"]["_bits"]))
        else:
            row["_bits"] = caches[0].bits.clone()
        rows[fmt] = row
        del caches, ws, wsd
    rows["bitmap"].pop("_bits")
    return rows


def streaming(seed, dev, Q):
    """The streaming workload: 64 sequences with a 2048-token prefix compressed, then 256 steps of
    (append one token per sequence, decode one query per sequence), 8 KV / 32 query heads,
    head_dim 128, 64-token blocks.  Three copies of the same cache run the step three ways: DGQ
    dgq_append + paged_decode_attn_int8 (two launches), DGQ dgq_append_decode (one launch), and the
    group-64 baseline (quantize the token, decode).  Each way streams on its own cache; per-step
    times are the mean over the last 248 steps between one pair of HIP events.  Also the last
    step's error against float32 attention over the unquantized keys/values."""
    import torch

    import dgq_data

    cfg = dgq_data.get_config(5)
    B, L, S, hkv, hq, d, bs = cfg.batch, cfg.seq_len, cfg.append_steps, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    k, v, cu, lens = dgq_data.batch_kv_device(cfg, seed, 0, dev)
    cu = cu.numpy().astype(np.int64)
    idx = torch.cat([torch.arange(int(cu[b]), int(cu[b]) + L) for b in range(B)]).to(dev)
    pk, pv = k.index_select(0, idx), v.index_select(0, idx)
    pcu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device=dev)
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=np.full(B, L + S))
    dtable = torch.from_numpy(table).to(dev)
    params = Q.DGQParams(hkv, hq, d, bs)
    sep, fused = Q.DGQCache(params, nblk, B, dev), Q.DGQCache(params, nblk, B, dev)
    g64 = Q.DGQG64Cache(params, nblk, dev)
    for c in (sep, fused):
        Q.dgq_compress(params, pk, pv, pcu, dtable, c, L, B * L)
    Q.dgq_g64_quantize(params, pk, pv, pcu, dtable, g64, L, B * L, L + S)
    del pk, pv
    ws = [Q.workspace(Q.decode_workspace_size(params, B, L + S), dev) for _ in range(3)]
    outs = [torch.empty((B, hq, d), dtype=torch.float32, device=dev) for _ in range(3)]
    one = torch.arange(B + 1, dtype=torch.int32, device=dev)
    cu_dev = torch.from_numpy(cu).to(dev)
    # every step's inputs are on the device before the timed loops, so the GPU never waits for the host
    steps = torch.arange(S, device=dev)
    tok_idx = (cu_dev[:-1][None, :] + L + steps[:, None]).reshape(-1)
    k_steps = k.index_select(0, tok_idx).view(S, B, hkv, d)
    v_steps = v.index_select(0, tok_idx).view(S, B, hkv, d)
    q_steps = torch.from_numpy(np.stack([dgq_data.queries(cfg, seed, 0, s) for s in range(S)])).to(dev)
    pos_steps = (L + steps[:, None].expand(S, B)).to(torch.int32).contiguous()
    pos1_steps = (pos_steps + 1).contiguous()
    torch.cuda.synchronize()

    def step(mode, s):
        pos, pos1 = pos_steps[s], pos1_steps[s]
        kt, vt, q = k_steps[s], v_steps[s], q_steps[s]
        if mode == 0:
            Q.dgq_append(params, kt, vt, pos, dtable, sep)
            Q.paged_decode_attn_int8(params, q, sep, dtable, pos1, L + S, out=outs[0], ws=ws[0])
        elif mode == 1:
            Q.dgq_append_decode(params, kt, vt, pos, q, dtable, fused, L + S, out=outs[1], ws=ws[1])
        else:
            Q.dgq_g64_quantize(params, kt, vt, one, dtable, g64, 1, B, L + S, first_pos=pos)
            Q.paged_decode_attn_g64(params, q, g64, dtable, pos1, L + S, out=outs[2], ws=ws[2])

    # each way runs the whole stream on its own cache: 8 untimed steps, then the other 248 between
    # one pair of events (no event between steps, whose queue cost would land in every step)
    warm = 8
    med = []
    for mode in range(3):
        for s in range(warm):
            step(mode, s)
        t0, t1 = Timer(), Timer()
        t0.record()
        for s in range(warm, S):
            step(mode, s)
        t1.record()
        torch.cuda.synchronize()
        med.append(t0.elapsed_time(t1) * 1e3 / (S - warm))
    q = q_steps[S - 1]
    # reference over the L + S tokens of every sequence
    k_all = [k[int(cu[b]):int(cu[b]) + L + S] for b in range(B)]
    v_all = [v[int(cu[b]):int(cu[b]) + L + S] for b in range(B)]
    G = hq // hkv
    ref = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    for b in range(B):
        kb = k_all[b].float().permute(1, 0, 2).contiguous()
        vb = v_all[b].float().permute(1, 0, 2).contiguous()
        qb = q[b].float().view(hkv, G, d).contiguous()
        sc = torch.bmm(qb, kb.transpose(1, 2).contiguous()) / math.sqrt(d)
        ref[b] = torch.bmm(torch.softmax(sc, dim=-1), vb).reshape(hq, d)
    e_dgq, e_g64 = rel_err_rows(outs[1], ref), rel_err_rows(outs[2], ref)
    nseg = fused.nseg.cpu().numpy().reshape(-1)
    return {
        "workload": "streaming: 64 seqs x 2048-token prefix + 256 steps of append 1 token + decode 1 query, "
                    "8 KV / 32 q heads, head_dim 128, 64-token blocks",
        "dgq_append_then_decode_us_per_step": round(float(med[0]), 2),
        "dgq_fused_append_decode_us_per_step": round(float(med[1]), 2),
        "group64_quantize_then_decode_us_per_step": round(float(med[2]), 2),
        "fused_tokens_per_s": round(B / (float(med[1]) / 1e6), 1),
        "fused_outputs_equal_separate": bool(torch.equal(outs[0], outs[1])),
        "dgq_max_rel_err_vs_fp16": round(e_dgq[0], 6), "dgq_mean_rel_err_vs_fp16": round(e_dgq[1], 6),
        "group64_max_rel_err_vs_fp16": round(e_g64[0], 6), "group64_mean_rel_err_vs_fp16": round(e_g64[1], 6),
        "segments_per_head_hist": np.bincount(nseg, minlength=10).tolist(),
    }


def fixed_batch(cid, seed, dev, Q, ncache, reps):
    """Compress and decode of one whole configured batch (no append): ``ncache`` caches of the
    same batch rotate, so consecutive decodes read different caches and their codes come from
    HBM.  Mean of back-to-back calls between one pair of HIP events; algorithmic bytes as for the
    main workload (codes + block table + segment rows + q + out for the decode, 3 B per element +
    identifier bits + segment rows for the compress); error against float32 attention over the
    unquantized keys/values."""
    import torch

    import dgq_data

    cfg = dgq_data.get_config(cid)
    B, hkv, hq, d, bs = cfg.batch, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    k, v, cu, lens = dgq_data.batch_kv_device(cfg, seed, 0, dev)
    total, L = int(cu[-1]), int(lens.max())
    dcu = cu.to(dev)
    table, nblk = dgq_data.block_tables(cfg, seed)
    dtable = torch.from_numpy(table).to(dev)
    params = Q.DGQParams(hkv, hq, d, bs)
    caches = [Q.DGQCache(params, nblk, B, dev) for _ in range(ncache)]
    ws_c = Q.workspace(Q.compress_workspace_size(params, B, total, L), dev)
    ws_d = Q.workspace(Q.decode_workspace_size(params, B, L), dev)
    q = torch.from_numpy(dgq_data.queries(cfg, seed)).to(dev)
    dl = torch.from_numpy(np.asarray(lens, np.int32)).to(dev)
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    for c in caches:
        Q.dgq_compress(params, k, v, dcu, dtable, c, L, total, ws=ws_c)
    # compress and decode each timed as `reps` back-to-back calls (rotating caches) between one
    # pair of events, after two untimed calls
    def timed(fn):
        for i in range(2):
            fn(i)
        e0, e1 = Timer(), Timer()
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    c_s = timed(lambda i: Q.dgq_compress(params, k, v, dcu, dtable, caches[i % ncache], L, total, ws=ws_c))
    d_s = timed(lambda i: Q.paged_decode_attn_int8(params, q, caches[i % ncache], dtable, dl, L, out=out, ws=ws_d))
    G = hq // hkv
    ref = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    cu64 = cu.numpy().astype(np.int64)
    for b in range(B):
        kb = k[int(cu64[b]):int(cu64[b + 1])].float().permute(1, 0, 2).contiguous()
        vb = v[int(cu64[b]):int(cu64[b + 1])].float().permute(1, 0, 2).contiguous()
        qb = q[b].float().view(hkv, G, d).contiguous()
        sc = torch.bmm(qb, kb.transpose(1, 2).contiguous()) / math.sqrt(d)
        ref[b] = torch.bmm(torch.softmax(sc, dim=-1), vb).reshape(hq, d)
    err = rel_err_rows(out, ref)
    nseg = caches[0].nseg.cpu().numpy()
    lens64 = np.asarray(lens, np.int64)
    seg_bytes = float(nseg.sum()) * 32
    dec_bytes = float(2 * lens64.sum() * hkv * d + np.ceil(lens64 / bs).sum() * 4 + seg_bytes + B * hq * d * 6)
    comp_bytes = float(total * hkv * d * 2 * 3 + total * hkv / 8 + seg_bytes)
    return {
        "decode_us": round(d_s * 1e6, 2),
        "decode_gbs_alg": round(dec_bytes / d_s / 1e9, 1),
        "decode_frac_hbm_peak": round(dec_bytes / d_s / 1e9 / HBM_PEAK_GBS, 4),
        "decode_kv_tokens_per_s": round(float(lens64.sum()) / d_s, 1),
        "compress_us": round(c_s * 1e6, 2),
        "compress_tokens_per_s": round(total / c_s, 1),
        "compress_gbs_alg": round(comp_bytes / c_s / 1e9, 1),
        "tokens": total,
        "decode_bytes": int(dec_bytes),
        "segments_per_head_hist": np.bincount(nseg.reshape(-1), minlength=6).tolist(),
        "dgq_max_rel_err_vs_fp16": round(err[0], 6), "dgq_mean_rel_err_vs_fp16": round(err[1], 6),
    }


def high_concurrency(seed, dev, Q):
    """The high-concurrency MHA workload: 100 sequences with lengths uniform in [512, 4096],
    32 heads (multi-head, one query head per kv head), head_dim 128, 16-token blocks shuffled in a
    shared pool; one decode query per sequence."""
    rec = {"workload": "high-concurrency MHA: 100 seqs, lengths U[512, 4096], 32 KV = 32 q heads, "
                       "head_dim 128, 16-token blocks shuffled"}
    rec.update(fixed_batch(4, seed, dev, Q, ncache=3, reps=12))
    return rec


def tiny(seed, dev, Q):
    """The tiny workload (1 sequence x 256 tokens, 2 heads, head_dim 64): launch-latency bound,
    reported in microseconds only."""
    r = fixed_batch(1, seed, dev, Q, ncache=2, reps=20)
    return {"workload": "tiny: 1 seq x 256 tokens, 2 KV = 2 q heads, head_dim 64, 16-token blocks",
            "compress_us": r["compress_us"], "decode_us": r["decode_us"],
            "segments_per_head_hist": r["segments_per_head_hist"],
            "dgq_max_rel_err_vs_fp16": r["dgq_max_rel_err_vs_fp16"]}


def long_context(seed, dev, Q):
    """The 128K long-context workload: 32 layers of one 131,072-token sequence (8 KV / 32 query
    heads, head_dim 128, 64-token blocks, 1% outliers at 8 sigma), each layer compressed into its
    own cache, then one decode query per layer, looped over the layers.  8 GiB of codes in all, so
    every layer's decode reads HBM.  Compress: median of per-layer HIP-event times; decode: median
    over three passes of the 32 layers (one event pair per pass) divided by 32."""
    import torch

    import dgq_data

    cfg = dgq_data.get_config(3)
    L, hkv, hq, d, bs = cfg.seq_len, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    params = Q.DGQParams(hkv, hq, d, bs)
    table, nblk = dgq_data.block_tables(cfg, seed)
    dtable = torch.from_numpy(table).to(dev)
    caches = [Q.DGQCache(params, nblk, 1, dev) for _ in range(cfg.layers)]
    ws_c = Q.workspace(Q.compress_workspace_size(params, 1, L, L), dev)
    ws_d = Q.workspace(Q.decode_workspace_size(params, 1, L), dev)
    comp_ms = []
    for layer in range(cfg.layers):
        k, v, cu, _ = dgq_data.batch_kv_device(cfg, seed, layer, dev)
        dcu = cu.to(dev)
        e0, e1 = Timer(), Timer()
        e0.record()
        Q.dgq_compress(params, k, v, dcu, dtable, caches[layer], L, L, ws=ws_c)
        e1.record()
        comp_ms.append((e0, e1))
        del k, v
    qs = [torch.from_numpy(dgq_data.queries(cfg, seed, layer)).to(dev) for layer in range(cfg.layers)]
    lens = torch.full((1,), L, dtype=torch.int32, device=dev)
    out = torch.empty((1, hq, d), dtype=torch.float32, device=dev)
    # one pass = the 32 layers' decodes back to back between one pair of events (an event between
    # two kernels adds several microseconds of queue time to the interval it opens); the first
    # pass is untimed
    dec = []
    for rep in range(4):
        e0, e1 = Timer(), Timer()
        e0.record()
        for layer in range(cfg.layers):
            Q.paged_decode_attn_int8(params, qs[layer], caches[layer], dtable, lens, L, out=out, ws=ws_d)
        e1.record()
        if rep > 0:
            dec.append((e0, e1))
    torch.cuda.synchronize()
    c_us = float(np.median([a.elapsed_time(b) for a, b in comp_ms])) * 1e3
    d_us = float(np.median([a.elapsed_time(b) for a, b in dec])) * 1e3 / cfg.layers
    nseg = torch.stack([c.nseg for c in caches]).cpu().numpy()
    dec_bytes = (2 * L * hkv * d + math.ceil(L / bs) * 4 + float(nseg.mean()) * hkv * 32 + hq * d * 2 + hq * d * 4)
    return {
        "workload": "128K long context: 1 seq x 131072 tokens, 32 layers looped, 8 KV / 32 q heads, "
                    "head_dim 128, 64-token blocks, 1% outliers at 8 sigma",
        "decode_us_per_layer": round(d_us, 2),
        "decode_gbs_alg": round(dec_bytes / d_us / 1e3, 1),
        "decode_frac_hbm_peak": round(dec_bytes / d_us / 1e3 / HBM_PEAK_GBS, 4),
        "compress_us_per_layer": round(c_us, 2),
        "compress_tokens_per_s": round(L / (c_us / 1e6), 1),
        "segments_per_head_hist": np.bincount(nseg.reshape(-1), minlength=6).tolist(),
        **kv_memory(cfg, caches[0]),
    }


def kv_memory(cfg, cache):
    """KV-cache bytes of all layers of the sequence: fp16 K and V against the DGQ layout (codes,
    identifier bits and segment-table rows at their allocated capacity)."""
    fp16 = 2 * cfg.seq_len * cfg.hkv * cfg.head_dim * 2 * cfg.layers
    per_layer = 2 * cfg.seq_len * cfg.hkv * cfg.head_dim + cfg.seq_len * cfg.hkv // 8
    per_layer += cache.segs.numel() * cache.segs.element_size() + cache.nseg.numel() * 4
    return {"kv_bytes_fp16_all_layers": fp16, "kv_bytes_dgq_all_layers": per_layer * cfg.layers,
            "compression_vs_fp16": round(fp16 / (per_layer * cfg.layers), 4)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import dgq_data

    cfg = dgq_data.get_config(2)
    cpu = cpu_baseline(cfg, args.seed, args.cpu_seconds) if args.cpu_seconds > 0 else None

    import torch

    import quantized_paged_kv_dgq_amd as Q

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    B, L, hkv, hq, d, bs = cfg.batch, cfg.seq_len, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size
    k, v, cu, lens = dgq_data.batch_kv_device(cfg, args.seed, 0, dev)
    total = int(cu[-1])
    dcu = cu.to(dev)
    table, nblk = dgq_data.block_tables(cfg, args.seed, lens_total=lens + 1)
    dtable = torch.from_numpy(table).to(dev)
    params = Q.DGQParams(hkv, hq, d, bs)
    ncache = 4
    caches = [Q.DGQCache(params, nblk, B, dev) for _ in range(ncache)]
    ws_c = Q.workspace(Q.compress_workspace_size(params, B, total, L), dev)
    ws_d = Q.workspace(Q.decode_workspace_size(params, B, L + 1), dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 17)
    k_tok = (torch.randn((B, hkv, d), generator=gen, device=dev) * 0.2).half()
    v_tok = (torch.randn((B, hkv, d), generator=gen, device=dev) * 0.2).half()
    q = torch.from_numpy(dgq_data.queries(cfg, args.seed)).to(dev)
    pos = torch.full((B,), L, dtype=torch.int32, device=dev)
    dec_lens = torch.full((B,), L + 1, dtype=torch.int32, device=dev)
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)

    def compress(i):
        Q.dgq_compress(params, k, v, dcu, dtable, caches[i % ncache], L, total, ws=ws_c)

    def append(i):
        Q.dgq_append(params, k_tok, v_tok, pos, dtable, caches[i % ncache])

    def decode(i):
        Q.paged_decode_attn_int8(params, q, caches[(i + 2) % ncache], dtable, dec_lens, L + 1, out=out, ws=ws_d)

    # fill every cache once (untimed), then warm up
    for i in range(ncache):
        compress(i)
        append(i)
    for i in range(args.warmup):
        compress(i)
        append(i)
        decode(i)
    torch.cuda.synchronize()

    K = args.steps

    # The timed region: K whole steps between one pair of events, nothing recorded inside (an
    # event between two kernels adds queue time on some boxes); then the per-call times from events
    # recorded around each call, over another K steps.
    t_start, t_end = Timer(), Timer()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        compress(i)
        append(i)
        decode(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # per-call times from events recorded around each call
    ev = [[Timer() for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        e = ev[i]
        e[0].record()
        compress(i)
        e[1].record()
        append(i)
        e[2].record()
        decode(i)
        e[3].record()
    torch.cuda.synchronize()
    comp_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    app_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])

    # the group-64 baseline on the same data, same step shape: quantize the batch, quantize the
    # appended token, decode over 8193 tokens; two caches rotate so the decoded one is cold
    g_caches = [Q.DGQG64Cache(params, nblk, dev) for _ in range(2)]
    one = torch.arange(B + 1, dtype=torch.int32, device=dev)
    out_g = torch.empty_like(out)

    def g_quant(i):
        c = g_caches[i % 2]
        Q.dgq_g64_quantize(params, k, v, dcu, dtable, c, L, total, L + 1)
        Q.dgq_g64_quantize(params, k_tok, v_tok, one, dtable, c, 1, B, L + 1, first_pos=pos)

    def g_decode(i):
        Q.paged_decode_attn_g64(params, q, g_caches[(i + 1) % 2], dtable, dec_lens, L + 1, out=out_g, ws=ws_d)

    for i in range(2 + args.warmup):
        g_quant(i)
        g_decode(i)
    torch.cuda.synchronize()
    gev = [[Timer() for _ in range(3)] for _ in range(K)]
    for i in range(K):
        e = gev[i]
        e[0].record()
        g_quant(i)
        e[1].record()
        g_decode(i)
        e[2].record()
    torch.cuda.synchronize()
    gq_ms = np.array([e[0].elapsed_time(e[1]) for e in gev])
    gd_ms = np.array([e[1].elapsed_time(e[2]) for e in gev])
    quality = quality_vs_fp16(cfg, k, v, cu, k_tok, v_tok, q, out, out_g)
    copy = achievable_copy(dev)
    policies = segment_policies(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q)
    formats = marker_format(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q)

    # algorithmic bytes
    Ld = L + 1
    nseg = torch.stack([c.nseg for c in caches]).cpu().numpy()
    seg_rows = float(nseg.mean()) * B * hkv
    dec_bytes = (B * 2 * Ld * hkv * d + B * math.ceil(Ld / bs) * 4 + seg_rows * 32
                 + B * hq * d * 2 + B * hq * d * 4)
    comp_elems = total * hkv * d * 2
    comp_bytes = comp_elems * 3 + total * hkv / 8 + seg_rows * 32
    dec_s = float(np.mean(dec_ms)) / 1e3
    comp_s = float(np.mean(comp_ms)) / 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    comp_gbs = comp_bytes / comp_s / 1e9
    hist = np.bincount(nseg.reshape(-1), minlength=6).tolist()
    g_dec_s = float(np.mean(gd_ms)) / 1e3
    g_dec_bytes = (B * 2 * Ld * hkv * d + B * Ld * hkv * (d // 64) * 4 * 2 + B * math.ceil(Ld / bs) * 4
                   + B * hq * d * 2 + B * hq * d * 4)

    kt_us = kernel_trace_decode_us()
    rec = {
        "metric": "INT8 paged decode-attn GB/s (% HBM peak) + dgq_compress tokens/s",
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B-shaped layer: 16 seqs x 8192 tokens, 8 KV / 32 q heads, head_dim 128, "
                        "16-token blocks shuffled; step = compress + append 1 token + decode 1 query",
            "global_batch": B, "seq_len": L, "block_size": bs, "kv_heads": hkv, "q_heads": hq, "head_dim": d,
        },
        "decode_frac_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_s * 1e6, 2),
        "decode_kv_tokens_per_s": round(B * Ld / dec_s, 1),
        "compress_tokens_per_s": round(total / comp_s, 1),
        "compress_gbs_alg": round(comp_gbs, 1),
        "compress_us": round(comp_s * 1e6, 2),
        "append_us": round(float(np.mean(app_ms)) * 1e3, 2),
        "segments_per_head_hist": hist,
        "roofline": {
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "frac_of_measured_copy": round(dec_gbs / copy["gbs"], 4),
            "measured_copy": copy,
            "traffic": measured_traffic(),
            "kernel": "decode_partition_kernel<128,4,16> (one launch per paged_decode_attn_int8 call; "
                      "HIP events around the call on its stream)",
            "kernel_trace_avg_us": kt_us,
            "kernel_trace_frac": round(dec_bytes / (kt_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if kt_us else None,
        },
        "roofline_compress": {
            "bound": "hbm", "achieved": round(comp_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("compress"),
            "kernel": "dgq_compress (stats + scores + select + encode, HIP events around the call)",
        },
        "wall_s_timed": round(wall, 4),
        "group64_baseline": {
            "decode_us": round(g_dec_s * 1e6, 2),
            "decode_gbs_alg": round(g_dec_bytes / g_dec_s / 1e9, 1),
            "decode_frac_hbm_peak": round(g_dec_bytes / g_dec_s / 1e9 / HBM_PEAK_GBS, 4),
            "quantize_us": round(float(np.mean(gq_ms)) * 1e3, 2),
            "quantize_tokens_per_s": round((total + B) / (float(np.mean(gq_ms)) / 1e3), 1),
            "decode_bytes": int(g_dec_bytes),
            "dgq_decode_bytes": int(dec_bytes),
            "dgq_decode_speedup": round(g_dec_s / dec_s, 4),
        },
        "quality_vs_fp16": quality,
        "segment_policies": policies,
        "identifier_formats": formats,
    }
    if not args.no_long_context:
        del caches, g_caches, k, v, ws_c
        torch.cuda.empty_cache()
        rec["streaming"] = streaming(args.seed, dev, Q)
        torch.cuda.empty_cache()
        rec["high_concurrency_mha"] = high_concurrency(args.seed, dev, Q)
        torch.cuda.empty_cache()
        rec["tiny"] = tiny(args.seed, dev, Q)
        torch.cuda.empty_cache()
        rec["long_context_128k"] = long_context(args.seed, dev, Q)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
