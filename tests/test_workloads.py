"""Seeded input generators: determinism, shapes, and agreement with the pages' layouts (CPU)."""
import json
import os

import numpy as np

from workloads import make_workload
from workloads.configs import BF16, F32, GQA, IN_PLACE, MLA, PATCH

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_layouts.json")


def test_layouts_match_pages():
    g = json.load(open(GOLDEN))
    c2 = make_workload("C2", num_layers=1, num_chunks=1, tokens=16).layout
    assert (c2.num_kv_heads, c2.head_dim, c2.row_width) == (g["qwen2.5-vl_gqa"]["kv_heads"],
                                                             g["qwen2.5-vl_gqa"]["head_dim"], g["qwen2.5-vl_gqa"]["row"])
    c5 = make_workload("C5", num_layers=1, num_chunks=4, tokens=32).layout
    assert (c5.num_kv_heads, c5.head_dim, c5.row_width) == (8, 128, g["qwen3-vl_gqa"]["row"])
    c3 = make_workload("C3", num_layers=1, num_chunks=1, tokens=16).layout
    assert (c3.latent_dim, c3.rope_dim) == (g["kimi-vl_mla"]["latent_dim"], g["kimi-vl_mla"]["rope_dim"])
    assert c3.rope_dim // 2 == g["kimi-vl_mla"]["rope_pairs"]
    assert make_workload("C2", num_layers=1).chunks[0].num_tokens == g["video_segment_tokens"]["value"]


def test_generators_are_deterministic_and_addressable():
    a = make_workload("C2", num_layers=2, num_chunks=2, tokens=64)
    b = make_workload("C2", num_layers=2, num_chunks=2, tokens=64)
    assert [c.delta for c in a.chunks] == [c.delta for c in b.chunks]
    assert np.array_equal(a.canonical(1, 1, 0), b.canonical(1, 1, 0))
    assert not np.array_equal(a.canonical(1, 1, 0), a.canonical(1, 0, 0))
    u1, v1 = a.factor(a.chunks[0], 0, 1)
    u2, v2 = b.factor(b.chunks[0], 0, 1)
    assert np.array_equal(u1, u2) and np.array_equal(v1, v2)
    assert u1.dtype == np.uint16 and u1.shape == (64, 32) and v1.shape == (512, 32)


def test_outlier_channels_and_orthonormal_factors():
    w = make_workload("C2", num_layers=1, num_chunks=1, tokens=1024)
    cols = w.outlier_columns(0)
    assert len(cols) == 16 and len(set(cols // 128)) == 4
    k = w.canonical(0, 0, 0).astype(np.uint32) << 16
    kf = k.view(np.float32)
    assert np.std(kf[:, cols]) > 5 and abs(np.std(np.delete(kf, cols, axis=1)) - 1) < 0.05
    u, v = w._factor_fp64(w.chunks[0].factors[0], 1024, 0)
    vt = v.T
    s = np.linalg.svd(u, compute_uv=False)
    assert np.allclose(s, 0.3 * 0.9 ** np.arange(32), rtol=1e-10)
    assert np.allclose(vt @ vt.T, np.eye(32), atol=1e-12)


def test_config_shapes():
    c1 = make_workload("C1")
    assert c1.layout.dtype == F32 and c1.layout.row_width == 128 and c1.chunks[0].num_tokens == 256
    assert c1.chunks[0].factors[0].rank == 8 and 0 <= c1.chunks[0].delta <= 4096
    c4 = make_workload("C4", num_layers=1, tokens=64)
    assert len(c4.chunks) == 24
    perms = {tuple(c.canon_id for c in c4.chunks[o * 4:(o + 1) * 4]) for o in range(6)}
    assert len(perms) == 6 and all(p[3] == 3 for p in perms)
    assert all(c.delta == (c.dst_row0) for c in c4.chunks)
    c5 = make_workload("C5", num_layers=1)
    surv = [c for c in c5.chunks if c.flags == IN_PLACE]
    rec = [c for c in c5.chunks if c.flags & PATCH]
    assert len(surv) == 48 and len(rec) == 16
    assert len({c.delta for c in surv}) == 1 and surv[0].delta < 0
    assert all(256 <= c.num_tokens <= 2048 for c in c5.chunks)
    pages = np.concatenate([c.block_table for c in c5.chunks])
    assert len(set(pages.tolist())) == len(pages) and pages.max() < c5.num_pages
    c3 = make_workload("C3", num_layers=1, num_chunks=2)
    assert c3.layout.family == MLA and [f.col0 for f in c3.chunks[0].factors] == [0, 512]
    assert c3.layout.dtype == BF16 and c3.layout.family != GQA
