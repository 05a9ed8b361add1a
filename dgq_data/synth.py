"""Seeded synthetic inputs shaped like the workloads the source pages describe.

Nothing here computes any part of dynamic-group quantization or attention: the module only
draws keys, values, queries, sequence lengths and block tables, so that the CPU oracle's tests
and the GPU path can be fed the same data.

Statistics the draws imitate (the pages, where the numbers come from):

* per-token key standard deviation from about 0.03 up to 0.47, changing from one stretch of the
  sequence to the next (DeepSeek DGQ article, section 2.2);
* Llama-3-8B-like shapes: 8 KV heads, 32 query heads, head_dim 128, 128K context (same article,
  section 3.3 memory formula);
* 100 concurrent requests with d_model 4096 and 32 heads (DeepSeek-V4 KV-cache article, "KV cache
  mechanism" and the measured-results table);
* 64-token pages for long contexts (DeepSeek-V4 KV-cache article, long-context section; grab-bag
  article, section 3.2 page tables).

Recipe (stated once, used everywhere):

* every (config, layer, sequence, kv head) has its own generator
  ``np.random.default_rng([seed, cid, layer, seq, head, 0])``; it first draws the sigma profile
  (``sigma_profile``), then the keys, then the values, then (if the config has outliers) the
  outlier masks and signs for keys and values;
* sigma profile: ``n_s`` segments with cut positions uniform over the sequence, redrawn until every
  segment is at least 32 tokens long; sigma per segment drawn from the config's set (without
  replacement) or uniformly from [lo, hi];
* K[t, d], V[t, d] ~ N(0, sigma_t^2) drawn in float32 and rounded to float16 (round to nearest
  even); outliers replace an element with +-mag * sigma_t;
* queries ~ N(0, 1) float16 from ``default_rng([seed, cid, layer, 0, 0, 1])``;
* sequence lengths (configs with varying lengths) from ``default_rng([seed, cid, 0, 0, 0, 2])``;
* block tables: every sequence receives ceil(len / block_size) physical ids, handed out in logical
  order from a free list that is either 0..n-1 (sequential) or a permutation drawn from
  ``default_rng([seed, cid, 0, 0, 0, 3])`` (shuffled pool).

``batch_kv_device`` draws the normals with a seeded torch generator on the GPU instead (same sigma
profiles, a different sample of the same distribution) so that the 128K-token workloads can be
made in well under a second; whoever checks such data against the oracle copies the sampled heads
back to the host.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    batch: int
    layers: int
    hkv: int
    hq: int
    head_dim: int
    block_size: int
    seq_len: int                 # fixed length, or the upper bound when lengths vary
    min_len: int = 0             # lower bound when lengths vary (0: fixed lengths)
    append_steps: int = 0        # streaming: tokens appended after the compressed prefix
    nseg_choices: Tuple[int, ...] = (2, 3, 4, 5)
    sigma_set: Tuple[float, ...] = ()
    sigma_lo: float = 0.03
    sigma_hi: float = 0.47
    outlier_frac: float = 0.0
    outlier_mag: float = 8.0
    table: str = "shuffled"      # "sequential" or "shuffled"
    min_segment: int = 32

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def total_len(self, prefix_len: int) -> int:
        return prefix_len + self.append_steps


CONFIGS = {
    1: WorkloadConfig(cid=1, name="tiny", batch=1, layers=1, hkv=2, hq=2, head_dim=64,
                      block_size=16, seq_len=256, nseg_choices=(3,),
                      sigma_set=(0.03, 0.15, 0.47), table="sequential"),
    2: WorkloadConfig(cid=2, name="llama3_8b_layer", batch=16, layers=1, hkv=8, hq=32,
                      head_dim=128, block_size=16, seq_len=8192),
    3: WorkloadConfig(cid=3, name="long_context_128k", batch=1, layers=32, hkv=8, hq=32,
                      head_dim=128, block_size=64, seq_len=131072, nseg_choices=(5,),
                      outlier_frac=0.01, outlier_mag=8.0),
    4: WorkloadConfig(cid=4, name="high_concurrency_mha", batch=100, layers=1, hkv=32, hq=32,
                      head_dim=128, block_size=16, seq_len=4096, min_len=512),
    5: WorkloadConfig(cid=5, name="streaming_decode", batch=64, layers=1, hkv=8, hq=32,
                      head_dim=128, block_size=64, seq_len=2048, append_steps=256),
}


def get_config(cid: int, **overrides) -> WorkloadConfig:
    """Config ``cid`` (1..5), optionally with fields replaced (smaller sizes for quick tests)."""
    return dataclasses.replace(CONFIGS[cid], **overrides)


def _head_rng(cfg: WorkloadConfig, seed: int, layer: int, seq: int, head: int):
    return np.random.default_rng([seed, cfg.cid, layer, seq, head, 0])


def sigma_profile(rng: np.random.Generator, length: int, cfg: WorkloadConfig):
    """Per-token sigma (float32 [length]), plus the true cut positions and segment sigmas."""
    n_s = int(rng.choice(np.asarray(cfg.nseg_choices)))
    ms = cfg.min_segment
    n_s = max(1, min(n_s, length // ms if length >= ms else 1))
    cuts = np.zeros(0, dtype=np.int64)
    if n_s > 1:
        lo, hi = ms, length - ms
        while True:
            cuts = np.sort(rng.choice(np.arange(lo, hi + 1), size=n_s - 1, replace=False))
            edges = np.concatenate([[0], cuts, [length]])
            if np.all(np.diff(edges) >= ms):
                break
    if cfg.sigma_set:
        sig = rng.permutation(np.asarray(cfg.sigma_set, dtype=np.float64))[:n_s]
    else:
        sig = rng.uniform(cfg.sigma_lo, cfg.sigma_hi, size=n_s)
    per_tok = np.empty(length, dtype=np.float32)
    edges = np.concatenate([[0], cuts, [length]])
    for j in range(n_s):
        per_tok[edges[j]:edges[j + 1]] = sig[j]
    return per_tok, cuts, sig


def seq_lens(cfg: WorkloadConfig, seed: int) -> np.ndarray:
    """Compressed (prefix) length of every sequence, int64 [batch]."""
    if cfg.min_len:
        rng = np.random.default_rng([seed, cfg.cid, 0, 0, 0, 2])
        return rng.integers(cfg.min_len, cfg.seq_len + 1, size=cfg.batch).astype(np.int64)
    return np.full(cfg.batch, cfg.seq_len, dtype=np.int64)


def head_kv(cfg: WorkloadConfig, seed: int, layer: int, seq: int, head: int, prefix_len: int):
    """Keys and values of one (layer, sequence, kv head): float16 [total_len][head_dim] each.

    ``total_len`` = prefix_len + cfg.append_steps; the sigma profile spans the whole length, so
    appended tokens may cross a true boundary.
    """
    length = cfg.total_len(prefix_len)
    rng = _head_rng(cfg, seed, layer, seq, head)
    sig, _, _ = sigma_profile(rng, length, cfg)
    d = cfg.head_dim
    k = rng.standard_normal((length, d), dtype=np.float32) * sig[:, None]
    v = rng.standard_normal((length, d), dtype=np.float32) * sig[:, None]
    if cfg.outlier_frac > 0.0:
        for x in (k, v):
            mask = rng.random((length, d), dtype=np.float32) < cfg.outlier_frac
            sign = rng.integers(0, 2, size=(length, d)).astype(np.float32) * 2.0 - 1.0
            x[mask] = (sign * np.float32(cfg.outlier_mag) * sig[:, None])[mask]
    return k.astype(np.float16), v.astype(np.float16)


def head_profile(cfg: WorkloadConfig, seed: int, layer: int, seq: int, head: int, prefix_len: int):
    """The sigma profile that ``head_kv`` uses for this head (for tests about true boundaries)."""
    rng = _head_rng(cfg, seed, layer, seq, head)
    return sigma_profile(rng, cfg.total_len(prefix_len), cfg)


def batch_kv(cfg: WorkloadConfig, seed: int, layer: int = 0):
    """Token-major keys/values of a whole batch for one layer.

    Returns (k, v, cu_seqlens, lens): k, v float16 [sum(total_len)][hkv][head_dim], cu_seqlens
    int32 [batch+1] over the *total* lengths (prefix + appends), lens int64 [batch] = prefix lengths.
    """
    lens = seq_lens(cfg, seed)
    tot = lens + cfg.append_steps
    cu = np.zeros(cfg.batch + 1, dtype=np.int64)
    cu[1:] = np.cumsum(tot)
    k = np.empty((int(cu[-1]), cfg.hkv, cfg.head_dim), dtype=np.float16)
    v = np.empty_like(k)
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            kk, vv = head_kv(cfg, seed, layer, b, h, int(lens[b]))
            k[cu[b]:cu[b + 1], h] = kk
            v[cu[b]:cu[b + 1], h] = vv
    return k, v, cu.astype(np.int32), lens


def batch_kv_device(cfg: WorkloadConfig, seed: int, layer: int = 0, device="cuda"):
    """Like ``batch_kv`` but the normals are drawn on ``device`` with a seeded torch generator.

    The sigma profiles are the numpy ones of ``head_kv`` (same generator stream); the Gaussian
    draws and the outlier masks come from ``torch.Generator(device)`` seeded from
    (seed, cid, layer).  Returns torch tensors (k, v on ``device``; cu_seqlens, lens on the host).
    """
    import torch

    lens = seq_lens(cfg, seed)
    tot = lens + cfg.append_steps
    cu = np.zeros(cfg.batch + 1, dtype=np.int64)
    cu[1:] = np.cumsum(tot)
    total = int(cu[-1])
    sig = np.empty((total, cfg.hkv), dtype=np.float32)
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            s, _, _ = sigma_profile(_head_rng(cfg, seed, layer, b, h), int(tot[b]), cfg)
            sig[cu[b]:cu[b + 1], h] = s
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, cfg.cid, layer, 7]).generate_state(1)[0]))
    sig_t = torch.from_numpy(sig).to(device).unsqueeze(-1)
    shape = (total, cfg.hkv, cfg.head_dim)
    out = []
    for _ in range(2):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * sig_t
        if cfg.outlier_frac > 0.0:
            mask = torch.rand(shape, generator=gen, device=device) < cfg.outlier_frac
            sign = torch.randint(0, 2, shape, generator=gen, device=device).float() * 2.0 - 1.0
            x = torch.where(mask, sign * cfg.outlier_mag * sig_t, x)
        out.append(x.half())
        del x
    return out[0], out[1], torch.from_numpy(cu.astype(np.int32)), lens


def queries(cfg: WorkloadConfig, seed: int, layer: int = 0, step: int = 0) -> np.ndarray:
    """Decode queries, float16 [batch][hq][head_dim] ~ N(0, 1); ``step`` indexes streaming steps."""
    rng = np.random.default_rng([seed, cfg.cid, layer, step, 0, 1])
    return rng.standard_normal((cfg.batch, cfg.hq, cfg.head_dim), dtype=np.float32).astype(np.float16)


def block_tables(cfg: WorkloadConfig, seed: int, lens_total: Optional[np.ndarray] = None,
                 spare_blocks: int = 0):
    """Physical block ids for every sequence: (table int32 [batch][max_blocks], num_blocks).

    ``lens_total`` defaults to prefix + appended lengths.  Unused table slots hold -1.  The pool
    has exactly the blocks the sequences need plus ``spare_blocks`` that no sequence uses.
    """
    if lens_total is None:
        lens_total = seq_lens(cfg, seed) + cfg.append_steps
    bs = cfg.block_size
    nb = [int(math.ceil(int(n) / bs)) for n in lens_total]
    num_blocks = int(sum(nb)) + int(spare_blocks)
    if cfg.table == "sequential":
        order = np.arange(num_blocks)
    else:
        order = np.random.default_rng([seed, cfg.cid, 0, 0, 0, 3]).permutation(num_blocks)
    max_blocks = max(nb) if nb else 0
    table = np.full((cfg.batch, max(max_blocks, 1)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nb):
        table[b, :n] = order[pos:pos + n]
        pos += n
    return table, num_blocks
