"""A seeded sweep over shapes and settings that the named workloads do not combine: kv heads
1..8, GQA groups 1, 2 and 4, head_dim 64 and 128, 16- and 64-token blocks, fixed and ragged
lengths (down to one token), sequential and shuffled block tables, outliers, segment limits 2..8,
tau 1.25..3, the length-aware cap, the variance floor, and both identifier formats.  Every case
runs the full oracle comparison of the compress tests (segments, codes, identifiers, append state,
decode); stream cases then append token by token, and fused cases run the fused step against the
separate calls, all against the oracle.  Long cases (8,200 to 24,000 tokens) take the tiled
selection with the same random settings; long fused cases split each sequence over several
workgroups, so the appending one hands the row count to the one that merges."""

import numpy as np
import pytest

import dgq_data
import gpu_helpers as H
from test_gpu_append import run_stream
from test_gpu_compress import compress_and_check
from test_gpu_fused import run_fused

pytestmark = pytest.mark.gpu


def draw_case(idx: int, streaming: bool):
    """Shape, data and parameters of sweep case idx (seeded by its index)."""
    rng = np.random.default_rng([2026, idx, int(streaming)])
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4]))
    head_dim = int(rng.choice([64, 128]))
    block_size = int(rng.choice([16, 32, 64]))
    batch = int(rng.integers(1, 5))
    if streaming:
        seq_len = int(rng.integers(1, 500))
        over = dict(append_steps=int(rng.integers(12, 60)), min_len=0)
    else:
        seq_len = int(rng.integers(1, 1600))
        over = dict(append_steps=0, min_len=int(rng.choice([0, 1, max(1, seq_len // 2)])))
    over.update(batch=batch, hkv=hkv, hq=hkv * group, head_dim=head_dim, block_size=block_size,
                seq_len=seq_len, table=str(rng.choice(["sequential", "shuffled"])),
                outlier_frac=float(rng.choice([0.0, 0.01])),
                nseg_choices=tuple(int(x) for x in rng.choice([2, 3, 4, 5], size=2)))
    cfg = dgq_data.get_config(2, **over)
    max_segments = int(rng.choice([2, 3, 4, 5, 8]))
    kw = dict(max_segments=max_segments, tau=float(rng.choice([1.25, 2.0, 3.0])),
              length_aware=bool(rng.integers(0, 2)), min_var=float(rng.choice([0.0, 1e-3, 1e-2])),
              marker=bool(rng.integers(0, 2)))
    if streaming and rng.integers(0, 2):
        kw["seg_capacity"] = max_segments + int(rng.integers(1, 4))   # small tables fill up
    return cfg, kw


def draw_long_case(idx: int, append_steps: int = 0):
    """A batch whose longest sequence takes the tiled selection (more than 8,192 tokens), with the
    random settings of draw_case (its own seeds, so the other cases are unchanged)."""
    rng = np.random.default_rng([2026, idx, 2])
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4]))
    seq_len = int(rng.integers(8200, 24001))
    over = dict(append_steps=append_steps, min_len=int(rng.choice([0, 1, seq_len // 2])), batch=int(rng.integers(1, 3)),
                hkv=hkv, hq=hkv * group, head_dim=int(rng.choice([64, 128])),
                block_size=int(rng.choice([16, 32, 64])), seq_len=seq_len,
                table=str(rng.choice(["sequential", "shuffled"])), outlier_frac=float(rng.choice([0.0, 0.01])),
                nseg_choices=tuple(int(x) for x in rng.choice([2, 3, 4, 5], size=2)))
    cfg = dgq_data.get_config(2, **over)
    kw = dict(max_segments=int(rng.choice([2, 3, 5, 8])), tau=float(rng.choice([1.0, 1.25, 2.0, 3.0])),
              length_aware=bool(rng.integers(0, 2)), min_var=float(rng.choice([0.0, 1e-3, 1e-2])),
              marker=bool(rng.integers(0, 2)))
    return cfg, kw


@pytest.mark.parametrize("idx", range(16))
def test_sweep_compress_decode(idx):
    cfg, kw = draw_case(idx, False)
    H.say("sweep compress", idx, cfg, kw)
    compress_and_check(cfg, 100 + idx, params=H.params_for(cfg, **kw))


@pytest.mark.parametrize("idx", range(8))
def test_sweep_append_stream(idx):
    cfg, kw = draw_case(idx, True)
    H.say("sweep stream", idx, cfg, kw)
    steps = cfg.append_steps
    run_stream(cfg, 200 + idx, steps, params=H.params_for(cfg, **kw), check_every=max(1, steps // 3))


@pytest.mark.parametrize("idx", range(8, 14))
def test_sweep_fused_step(idx):
    cfg, kw = draw_case(idx, True)
    H.say("sweep fused", idx, cfg, kw)
    steps = cfg.append_steps
    run_fused(cfg, 300 + idx, steps, {steps // 2, steps - 1}, params=H.params_for(cfg, **kw))


@pytest.mark.parametrize("idx", range(6))
def test_sweep_long_compress_decode(idx):
    cfg, kw = draw_long_case(idx)
    H.say("sweep long compress", idx, cfg, kw)
    compress_and_check(cfg, 400 + idx, params=H.params_for(cfg, **kw))


@pytest.mark.parametrize("idx", range(6, 9))
def test_sweep_long_fused_step(idx):
    cfg, kw = draw_long_case(idx, append_steps=40)
    H.say("sweep long fused", idx, cfg, kw)
    run_fused(cfg, 500 + idx, 40, {20, 39}, params=H.params_for(cfg, **kw))
