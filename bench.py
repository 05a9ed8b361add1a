"""Benchmark of the DGQ hot path on one MI355X.

Headline workload: the 128K long context (one 131,072-token sequence, 32 layers looped on one
GPU, 8 KV / 32 query heads, head_dim 128, 64-token blocks permuted in the pool, 1 % outliers at
8 sigma).  The fp16 K/V of all 32 layers (16 GiB) are resident in HBM before the timed region.
One step = one pass of the whole hot path over that input:

  1. dgq_compress            every layer's 131,072-token prefix into its own INT8 DGQ cache;
  2. dgq_append              one fp16 token into every layer's cache;
  3. paged_decode_attn_int8  one decode query per layer over its 131,073 cached tokens.

Each phase runs its 32 launches back to back.  A decode reads a cache written at least 31
compressions (8 GiB of codes and 24 GiB of fp16 reads) earlier, so its codes come from HBM and
not from the 256 MB Infinity Cache.  ``ms_per_step`` times K whole steps between one pair of HIP
events with nothing recorded inside; the per-launch figures come from another K steps with one
event pair around each phase (32 launches), so no event sits between two decodes.

``value`` is the decode's throughput in GB/s of algorithmic bytes per launch (INT8 K/V codes +
block table + segment rows + q + out) over its mean launch time; ``roofline`` compares it with
the 8 TB/s HBM peak and carries the HBM bytes the committed counter profile measured.

Sections, each on its own data: the Llama-3-8B-shaped layer (16 x 8192 tokens, 16-token blocks;
compress + append + decode with rotating caches, the group-64 baseline on the same data, error
against fp16 attention, the segment-count policies and both identifier formats), the streaming
workload (64 x 2048-token prefixes, 256 append + decode steps, three ways), the high-concurrency
MHA batch and the tiny case.  ``cpu_baseline`` times the CPU oracle on the host cores: one core
on a bounded sample of the headline workload, and every workload fanned out over the allowed
cores (with the host's CPU model, affinity and thread settings).

Prints one JSON line.
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the one-core CPU oracle sample (0 skips the whole CPU baseline)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the 128K long-context step (no Llama-layer, streaming, MHA or tiny sections)")
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


def _profile_kv(name: str) -> dict:
    """key: value lines of a committed profile summary (comments and indented lines skipped)."""
    path = os.path.join(ROOT, "profiles", name)
    kv = {}
    if not os.path.exists(path):
        return kv
    for line in open(path):
        if ":" in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split("#", 1)[0].strip()
    return kv


HEADLINE_PROFILE = "decode_128k_layer_trace_and_traffic.txt"
LLAMA_PROFILE = "decode_llama3_8b_layer_hbm_traffic.txt"
WORKLOADS_PROFILE = "workloads_hbm_traffic.txt"


def measured_traffic(what: str = "decode", profile: str = HEADLINE_PROFILE, prefix: str = ""):
    """HBM bytes per decode launch ("decode") or per dgq_compress call ("compress") from a
    committed counter profile (keys with an optional section prefix, e.g. "mha_"), if it was taken
    on the current kernel sources (else None)."""
    kv = _profile_kv(profile)
    digest = kernel_source_digest() if what == "decode" else compress_source_digest()
    key = prefix + ("decode_hbm_bytes_per_launch" if what == "decode" else "compress_hbm_bytes_per_call")
    if kv.get(f"{what}_source_sha256_16") != digest:
        return None
    try:
        return int(float(kv[key]))
    except (KeyError, ValueError):
        return None


def kernel_trace_decode_us(profile: str = HEADLINE_PROFILE):
    """Kernel-trace average duration of the headline decode launches from the committed rocprofv3
    summary of the same bench command, if it was taken on the current decode sources (else None)."""
    kv = _profile_kv(profile)
    if kv.get("decode_source_sha256_16") != kernel_source_digest():
        return None
    try:
        return float(kv["decode_avg_us"])
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


def host_info():
    """The host the CPU baseline ran on: CPU model, core counts and thread settings."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info = {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                    "MKL_NUM_THREADS", "MAX_JOBS")}}
    try:
        from threadpoolctl import threadpool_info
        info["blas_pools"] = [{"api": p.get("internal_api"), "threads": p.get("num_threads")}
                              for p in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    info["oracle_threads_per_process"] = 1
    return info


def _oracle_unit(job):
    """One (layer, sequence, kv head) of a workload through the oracle on one core (BLAS limited
    to one thread): compress the prefix, then either one decode over it or ``steps`` rounds of
    (append one token, decode over the cache).  Each timed part is the median of ``reps`` runs
    (the data is drawn once, untimed)."""
    cid, seed, layer, b, h, steps, reps, q = job
    from threadpoolctl import threadpool_limits

    import dgq_data
    from oracle import dgq_oracle as O

    cfg = dgq_data.get_config(cid)
    L = int(dgq_data.seq_lens(cfg, seed)[b])
    d = cfg.head_dim
    k, v = dgq_data.head_kv(cfg, seed, layer, b, h, L)
    comp, dec, app = [], [], []
    dbytes = 0
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t0 = time.perf_counter()
            hc = O.compress_head(k[:L], v[:L])
            t1 = time.perf_counter()
            comp.append(t1 - t0)
            if steps == 0:
                O.decode_attention(q, hc.khat(), hc.vhat())
                dec.append(time.perf_counter() - t1)
                app.append(0.0)
                dbytes = 2 * L * d
                continue
            st = O.AppendState(hc, k[:L], cfg.block_size)
            ta = td = 0.0
            dbytes = 0
            for s_ in range(steps):
                a0 = time.perf_counter()
                st.append(k[L + s_], v[L + s_])
                a1 = time.perf_counter()
                snap = st.snapshot()
                O.decode_attention(q[s_], snap.khat(), snap.vhat())
                a2 = time.perf_counter()
                ta += a1 - a0
                td += a2 - a1
                dbytes += 2 * (L + s_ + 1) * d
            app.append(ta)
            dec.append(td)
    return {"compress_s": float(np.median(comp)), "decode_s": float(np.median(dec)),
            "append_s": float(np.median(app)), "tokens": L, "decode_bytes": dbytes, "appended": steps}


def _unit_jobs(cid, seed, units, steps=0, reps=1):
    """Oracle jobs of (layer, sequence, kv head) units, with their query rows drawn up front."""
    import dgq_data

    cfg = dgq_data.get_config(cid)
    g = cfg.group
    qcache = {}
    jobs = []
    for layer, b, h in units:
        if steps == 0:
            if layer not in qcache:
                qcache[layer] = dgq_data.queries(cfg, seed, layer)
            q = qcache[layer][b, h * g:(h + 1) * g]
        else:
            for s_ in range(steps):
                if (layer, s_) not in qcache:
                    qcache[(layer, s_)] = dgq_data.queries(cfg, seed, layer, s_)
            q = np.stack([qcache[(layer, s_)][b, h * g:(h + 1) * g] for s_ in range(steps)])
        jobs.append((cid, seed, layer, b, h, steps, reps, q))
    return jobs


def _summarize(results, cores, wall, desc):
    t_c = float(sum(r["compress_s"] for r in results))
    t_d = float(sum(r["decode_s"] for r in results))
    t_a = float(sum(r["append_s"] for r in results))
    tok = float(sum(r["tokens"] for r in results))
    db = float(sum(r["decode_bytes"] for r in results))
    out = {"sample": desc, "units": len(results), "cores": cores,
           "compress_tokens_per_s_per_core": round(tok / t_c, 1),
           "decode_gbs_per_core": round(db / t_d / 1e9, 4),
           "compress_tokens_per_s": round(tok / t_c * cores, 1),
           "decode_gbs": round(db / t_d / 1e9 * cores, 4),
           "oracle_core_seconds": round(t_c + t_d + t_a, 3), "wall_seconds": round(wall, 3)}
    appended = float(sum(r["appended"] for r in results))
    if appended:
        out["append_tokens_per_s_per_core"] = round(appended / t_a, 1)
    return out


def _fan_out(pool, cores, jobs, desc):
    t0 = time.perf_counter()
    res = pool.map(_oracle_unit, jobs, chunksize=1)
    return _summarize(res, cores, time.perf_counter() - t0, desc)


def cpu_baseline(seed, budget_s):
    """The oracle as it is, on the host cores (run before the GPU is touched: the fan-out forks).

    * ``value``: one core (BLAS limited to one thread) on a bounded sample of the headline
      workload, whole (layer, kv head) units of the 131,072-token sequence until ``budget_s`` is
      spent; decode GB/s of codes (the metric's unit) and compress tokens/s.
    * ``per_workload``: every workload fanned out over (layer, sequence, kv head) units, one
      process per allowed core (at most 16), each process timing its own units: the tiny case,
      the Llama-3-8B-shaped layer and the 100-sequence MHA batch whole (each part the median of 3
      runs per unit), 8 of the 128K long context's 32 layers (8 heads each, one run; the 32-layer
      time is the per-layer mean x 32), and the streaming workload on one kv head per sequence
      (64 of 512 units, all 256 append + decode steps).  Rates are per core times the process
      count."""
    import multiprocessing as mp

    import dgq_data

    cfg3 = dgq_data.get_config(3)
    units3 = [(layer, 0, h) for layer in range(cfg3.layers) for h in range(cfg3.hkv)]
    jobs3 = _unit_jobs(3, seed, units3)
    res1 = []
    start = time.perf_counter()
    for job in jobs3:
        res1.append(_oracle_unit(job))
        if time.perf_counter() - start > budget_s:
            break
    one = _summarize(res1, 1, time.perf_counter() - start,
                     f"{len(res1)} of {len(units3)} (layer, kv head) units of the 131,072-token sequence "
                     "(compress + dequantize and float64 attention for the 4 query heads)")
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    per = {}
    with mp.get_context("fork").Pool(cores) as pool:
        c1 = dgq_data.get_config(1)
        per["tiny"] = _fan_out(pool, cores, _unit_jobs(1, seed, [(0, 0, h) for h in range(c1.hkv)], reps=3),
                               "all 2 heads, median of 3 runs")
        c2 = dgq_data.get_config(2)
        per["llama3_8b_layer"] = _fan_out(
            pool, cores, _unit_jobs(2, seed, [(0, b, h) for b in range(c2.batch) for h in range(c2.hkv)], reps=3),
            "all 128 (sequence, kv head) units, median of 3 runs each")
        c4 = dgq_data.get_config(4)
        per["high_concurrency_mha"] = _fan_out(
            pool, cores, _unit_jobs(4, seed, [(0, b, h) for b in range(c4.batch) for h in range(c4.hkv)], reps=3),
            "all 3200 (sequence, head) units, median of 3 runs each")
        lc = _fan_out(pool, cores, jobs3[:8 * cfg3.hkv],
                      "8 of the 32 layers x 8 kv heads, one run each; the 32-layer figure scales the "
                      "per-layer mean by 32 (the layers are drawn alike)")
        lc["oracle_core_seconds_32_layers"] = round(lc["oracle_core_seconds"] * cfg3.layers / 8, 3)
        per["long_context_128k"] = lc
        c5 = dgq_data.get_config(5)
        per["streaming"] = _fan_out(
            pool, cores, _unit_jobs(5, seed, [(0, b, b % c5.hkv) for b in range(c5.batch)], steps=c5.append_steps),
            "64 of 512 units (kv head b % 8 of sequence b): 2048-token prefix compress, then 256 x (append, decode)")
    lc = per["long_context_128k"]
    return {
        "value": one["decode_gbs_per_core"],
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": one["sample"],
        "compress_tokens_per_s": one["compress_tokens_per_s_per_core"],
        "seconds": one["oracle_core_seconds"],
        "long_context_32_layers_core_seconds": lc["oracle_core_seconds_32_layers"],
        "per_workload": per,
        "host": host_info(),
    }


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
    rec["decode_traffic"] = measured_traffic(profile=WORKLOADS_PROFILE, prefix="mha_")
    rec["roofline_compress"] = {
        "bound": "hbm", "achieved": rec["compress_gbs_alg"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(rec["compress_gbs_alg"] / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic("compress", profile=WORKLOADS_PROFILE, prefix="mha_"),
        "kernel": "dgq_compress of the batch (tile map + stats + select + encode; HIP events around "
                  "back-to-back calls)",
    }
    return rec


def tiny(seed, dev, Q):
    """The tiny workload (1 sequence x 256 tokens, 2 heads, head_dim 64): launch-latency bound,
    reported in microseconds only."""
    r = fixed_batch(1, seed, dev, Q, ncache=2, reps=200)
    return {"workload": "tiny: 1 seq x 256 tokens, 2 KV = 2 q heads, head_dim 64, 16-token blocks",
            "compress_us": r["compress_us"], "decode_us": r["decode_us"],
            "segments_per_head_hist": r["segments_per_head_hist"],
            "dgq_max_rel_err_vs_fp16": r["dgq_max_rel_err_vs_fp16"]}


def kv_memory(cfg, cache):
    """KV-cache bytes of all layers of the sequence: fp16 K and V against the DGQ layout (codes,
    identifier bits and segment-table rows at their allocated capacity)."""
    fp16 = 2 * cfg.seq_len * cfg.hkv * cfg.head_dim * 2 * cfg.layers
    per_layer = 2 * cfg.seq_len * cfg.hkv * cfg.head_dim + cfg.seq_len * cfg.hkv // 8
    per_layer += cache.segs.numel() * cache.segs.element_size() + cache.nseg.numel() * 4
    return {"kv_bytes_fp16_all_layers": fp16, "kv_bytes_dgq_all_layers": per_layer * cfg.layers,
            "compression_vs_fp16": round(fp16 / (per_layer * cfg.layers), 4)}


def long_context_step(args, dev, Q):
    """The headline: the 128K long-context workload, one step = compress all 32 layers, append one
    token to every layer, decode every layer (see the module text)."""
    import torch

    import dgq_data

    cfg = dgq_data.get_config(3)
    L, hkv, hq, d, bs, nl = cfg.seq_len, cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size, cfg.layers
    params = Q.DGQParams(hkv, hq, d, bs)
    table, nblk = dgq_data.block_tables(cfg, args.seed, lens_total=np.array([L + 1]))
    dtable = torch.from_numpy(table).to(dev)
    kv = []
    for layer in range(nl):
        k, v, cu, _ = dgq_data.batch_kv_device(cfg, args.seed, layer, dev)
        kv.append((k, v))
    dcu = cu.to(dev)
    caches = [Q.DGQCache(params, nblk, 1, dev) for _ in range(nl)]
    ws_c = Q.workspace(Q.compress_workspace_size(params, 1, L, L), dev)
    ws_d = Q.workspace(Q.decode_workspace_size(params, 1, L + 1), dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 23)
    toks = [((torch.randn((1, hkv, d), generator=gen, device=dev) * 0.2).half(),
             (torch.randn((1, hkv, d), generator=gen, device=dev) * 0.2).half()) for _ in range(nl)]
    qs = [torch.from_numpy(dgq_data.queries(cfg, args.seed, layer)).to(dev) for layer in range(nl)]
    pos = torch.full((1,), L, dtype=torch.int32, device=dev)
    dec_lens = torch.full((1,), L + 1, dtype=torch.int32, device=dev)
    outs = [torch.empty((1, hq, d), dtype=torch.float32, device=dev) for _ in range(nl)]

    def compress_all():
        for layer in range(nl):
            Q.dgq_compress(params, kv[layer][0], kv[layer][1], dcu, dtable, caches[layer], L, L, ws=ws_c)

    def append_all():
        for layer in range(nl):
            Q.dgq_append(params, toks[layer][0], toks[layer][1], pos, dtable, caches[layer])

    def decode_all():
        for layer in range(nl):
            Q.paged_decode_attn_int8(params, qs[layer], caches[layer], dtable, dec_lens, L + 1,
                                     out=outs[layer], ws=ws_d)

    for _ in range(args.warmup):
        compress_all()
        append_all()
        decode_all()
    torch.cuda.synchronize()

    K = args.steps
    # the timed region: K whole steps between one pair of events
    t_start, t_end = Timer(), Timer()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(K):
        compress_all()
        append_all()
        decode_all()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # per-phase times: another K steps, one event pair around each phase of 32 launches
    ev = [[Timer() for _ in range(4)] for _ in range(K)]
    for i in range(K):
        e = ev[i]
        e[0].record()
        compress_all()
        e[1].record()
        append_all()
        e[2].record()
        decode_all()
        e[3].record()
    torch.cuda.synchronize()
    comp_s = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3 / nl
    app_s = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) / 1e3 / nl
    dec_s = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) / 1e3 / nl

    nseg = torch.stack([c.nseg for c in caches]).cpu().numpy()
    Ld = L + 1
    dec_bytes = (2 * Ld * hkv * d + math.ceil(Ld / bs) * 4 + float(nseg.mean()) * hkv * 32
                 + hq * d * 2 + hq * d * 4)
    comp_bytes = L * hkv * d * 2 * 3 + L * hkv / 8 + float(nseg.mean()) * hkv * 32
    dec_gbs = dec_bytes / dec_s / 1e9
    comp_gbs = comp_bytes / comp_s / 1e9
    # error of the last decode of every layer against float32 attention over the unquantized fp16 K/V
    errs = []
    for layer in range(nl):
        k, v = kv[layer]
        kk = torch.cat([k, toks[layer][0]])
        vv = torch.cat([v, toks[layer][1]])
        ref = fp16_reference(cfg, kk, vv, np.array([0, Ld]), qs[layer])
        errs.append(rel_err_rows(outs[layer], ref))
    kt_us = kernel_trace_decode_us()
    copy = achievable_copy(dev)
    rec = {
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(total_ms / K, 4),
        "config": {
            "workload": "128K long context: 1 seq x 131072 tokens, 32 layers looped on one GPU, 8 KV / 32 q heads, "
                        "head_dim 128, 64-token blocks permuted, 1% outliers at 8 sigma; step = compress all 32 "
                        "layers + append 1 token per layer + decode 1 query per layer over 131073 tokens",
            "global_batch": 1, "seq_len": L, "layers": nl, "block_size": bs, "kv_heads": hkv, "q_heads": hq,
            "head_dim": d,
        },
        "decode_frac_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us_per_layer": round(dec_s * 1e6, 2),
        "decode_kv_tokens_per_s": round(Ld / dec_s, 1),
        "compress_us_per_layer": round(comp_s * 1e6, 2),
        "compress_tokens_per_s": round(L / comp_s, 1),
        "compress_gbs_alg": round(comp_gbs, 1),
        "append_us_per_layer": round(app_s * 1e6, 2),
        "step_tokens_per_s": round(nl * L / (total_ms / K / 1e3), 1),
        "segments_per_head_hist": np.bincount(nseg.reshape(-1), minlength=6).tolist(),
        "dgq_max_rel_err_vs_fp16": round(max(e[0] for e in errs), 6),
        "dgq_mean_rel_err_vs_fp16": round(float(np.mean([e[1] for e in errs])), 6),
        "roofline": {
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": int(dec_bytes),
            "launch_us": round(dec_s * 1e6, 2),
            "frac_of_measured_copy": round(dec_gbs / copy["gbs"], 4),
            "measured_copy": copy,
            "kernel": "decode_partition_kernel<128,4,64> (one launch per paged_decode_attn_int8 call, 32 x 8 x 1 "
                      "workgroups; HIP events around the 32 back-to-back decodes of a step on their stream)",
            "kernel_trace_avg_us": kt_us,
            "kernel_trace_frac": round(dec_bytes / (kt_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if kt_us else None,
        },
        "roofline_compress": {
            "bound": "hbm", "achieved": round(comp_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("compress"),
            "kernel": "dgq_compress per layer (stats + scores + select + encode; HIP events around the 32 "
                      "compresses of a step)",
        },
        "wall_s_timed": round(wall, 4),
        **kv_memory(cfg, caches[0]),
    }
    del kv, caches, ws_c, ws_d
    return rec


def llama_layer(args, dev, Q):
    """The Llama-3-8B-shaped layer: 16 sequences x 8192 tokens, 8 KV / 32 query heads, head_dim 128,
    16-token blocks shuffled.  Step = compress the batch + append one token per sequence + decode
    one query per sequence over 8193 tokens; four caches rotate (step i compresses and appends
    into cache i % 4 and decodes cache (i + 2) % 4, written two steps earlier).  Also the group-64
    baseline on the same data, the error of both against fp16 attention, the segment-count
    policies and the two identifier formats."""
    import torch

    import dgq_data

    cfg = dgq_data.get_config(2)
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

    for i in range(ncache):
        compress(i)
        append(i)
    for i in range(args.warmup):
        compress(i)
        append(i)
        decode(i)
    torch.cuda.synchronize()
    K = args.steps
    t_start, t_end = Timer(), Timer()
    t_start.record()
    for i in range(K):
        compress(i)
        append(i)
        decode(i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ev = [[Timer() for _ in range(4)] for _ in range(K)]
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
    policies = segment_policies(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q)
    formats = marker_format(cfg, k, v, cu, dcu, dtable, nblk, q, dev, Q)

    Ld = L + 1
    nseg = torch.stack([c.nseg for c in caches]).cpu().numpy()
    seg_rows = float(nseg.mean()) * B * hkv
    dec_bytes = (B * 2 * Ld * hkv * d + B * math.ceil(Ld / bs) * 4 + seg_rows * 32
                 + B * hq * d * 2 + B * hq * d * 4)
    comp_bytes = total * hkv * d * 2 * 3 + total * hkv / 8 + seg_rows * 32
    dec_s = float(np.mean(dec_ms)) / 1e3
    comp_s = float(np.mean(comp_ms)) / 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    comp_gbs = comp_bytes / comp_s / 1e9
    g_dec_s = float(np.mean(gd_ms)) / 1e3
    g_dec_bytes = (B * 2 * Ld * hkv * d + B * Ld * hkv * (d // 64) * 4 * 2 + B * math.ceil(Ld / bs) * 4
                   + B * hq * d * 2 + B * hq * d * 4)
    rec = {
        "workload": "Llama-3-8B-shaped layer: 16 seqs x 8192 tokens, 8 KV / 32 q heads, head_dim 128, 16-token "
                    "blocks shuffled; step = compress + append 1 token + decode 1 query, four caches rotating",
        "ms_per_step": round(total_ms / K, 4),
        "decode_us": round(dec_s * 1e6, 2),
        "decode_gbs_alg": round(dec_gbs, 1),
        "decode_frac_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_kv_tokens_per_s": round(B * Ld / dec_s, 1),
        "decode_bytes": int(dec_bytes),
        "decode_traffic": measured_traffic(profile=LLAMA_PROFILE),
        "compress_us": round(comp_s * 1e6, 2),
        "compress_tokens_per_s": round(total / comp_s, 1),
        "compress_gbs_alg": round(comp_gbs, 1),
        "compress_frac_hbm_peak": round(comp_gbs / HBM_PEAK_GBS, 4),
        "compress_traffic": measured_traffic("compress", profile=LLAMA_PROFILE),
        "append_us": round(float(np.mean(app_ms)) * 1e3, 2),
        "segments_per_head_hist": np.bincount(nseg.reshape(-1), minlength=6).tolist(),
        "group64_baseline": {
            "decode_us": round(g_dec_s * 1e6, 2),
            "decode_gbs_alg": round(g_dec_bytes / g_dec_s / 1e9, 1),
            "decode_frac_hbm_peak": round(g_dec_bytes / g_dec_s / 1e9 / HBM_PEAK_GBS, 4),
            "quantize_us": round(float(np.mean(gq_ms)) * 1e3, 2),
            "quantize_tokens_per_s": round((total + B) / (float(np.mean(gq_ms)) / 1e3), 1),
            "decode_bytes": int(g_dec_bytes),
            "dgq_decode_speedup": round(g_dec_s / dec_s, 4),
        },
        "quality_vs_fp16": quality,
        "segment_policies": policies,
        "identifier_formats": formats,
    }
    del caches, g_caches, k, v, ws_c, ws_d
    return rec


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first: its fan-out forks, which must happen before the GPU is touched
    cpu = cpu_baseline(args.seed, args.cpu_seconds) if args.cpu_seconds > 0 else None

    import torch

    import quantized_paged_kv_dgq_amd as Q

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    head = long_context_step(args, dev, Q)
    torch.cuda.empty_cache()
    rec = {
        "metric": "INT8 paged decode-attn GB/s (% HBM peak) + dgq_compress tokens/s",
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": head.pop("config"),
    }
    rec.update(head)
    if not args.headline_only:
        rec["llama3_8b_layer"] = llama_layer(args, dev, Q)
        torch.cuda.empty_cache()
        rec["streaming"] = streaming(args.seed, dev, Q)
        torch.cuda.empty_cache()
        rec["high_concurrency_mha"] = high_concurrency(args.seed, dev, Q)
        torch.cuda.empty_cache()
        rec["tiny"] = tiny(args.seed, dev, Q)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
