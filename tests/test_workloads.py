"""Seeded workload generator and work accounting (CPU only)."""
import json
import os

import numpy as np

import workloads as W
from workloads import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_sizing_figures():
    with open(os.path.join(GOLDEN, "page_sizing.json")) as f:
        g = json.load(f)
    for c in g["score_matrix_fp16"]:
        assert A.score_matrix_bytes(c["n"]) == c["bytes"]
    for c in g["kv_cache_dense"]:
        b = A.kv_cache_bytes_dense(c["batch"], c["seq_len"], c["layers"], c["hidden"],
                                   c["elem_bytes"])
        assert round(b / 1e9, 1) == c["page_says_gb"]
    for c in g["block_kv_bytes"]:
        assert c["tokens"] * c["head_dim"] * c["elem_bytes"] == c["bytes"]


def test_token_bytes():
    assert A.token_bytes(128, 8) == 140     # 128 codes + 4 fp16 scales + 4 zeros
    assert A.token_bytes(128, 4) == 76


def test_decode_4k_bytes():
    s = W.WORKLOADS["decode_4k"]
    kv = A.decode_kv_bytes(128, [4096], [8, 8])
    assert kv == 4096 * 2 * 280 == 2_293_760
    assert A.decode_bytes(1, 8, 128, [4096], [8, 8]) == kv + 4096
    assert s.cap == 4096


def test_decode_128k_mixed_bytes():
    kv = A.decode_kv_bytes(128, [131072] * 8, [8, 8, 4, 4, 4, 4, 4, 4])
    assert kv == 1_543_503_872


def test_prefill_flops_closed_forms():
    L = 8192
    assert A.prefill_flops(32, 128, [L]) == 4 * 128 * 32 * L * (L + 1) // 2
    # dense mask equals no mask
    m = np.tril(np.ones((3, 3), np.uint8))
    assert A.causal_pairs(384, 384, m) == 384 * 385 // 2
    assert A.causal_pairs(300, 300, m) == 300 * 301 // 2
    # brute force on a tiny masked case
    m[2, 1] = 0
    n = 300
    want = sum(1 for i in range(n) for j in range(i + 1) if m[i // 128, j // 128])
    assert A.causal_pairs(n, n, m) == want
    m4 = np.tril(np.ones((4, 4), np.uint8))
    m4[3, 1] = m4[2, 1] = 0
    want = sum(1 for i in range(512) for j in range(i + 1) if m4[i // 128, j // 128])
    assert A.causal_pairs_fast(512, m4) == want == A.causal_pairs(512, 512, m4)


def test_sparse_mask_structure_and_count():
    s = W.WORKLOADS["prefill_128k_sparse"]
    rng = np.random.default_rng(s.seed)
    m = W.skip_mask(s.context, s.skip_frac, rng)
    n = 1024
    assert m.shape == (n, n)
    assert np.all(np.triu(m, 1) == 0)
    assert np.all(np.diag(m) == 1)
    assert np.all(m[:, 0] == 1)
    eligible = (n - 1) * (n - 2) // 2
    assert eligible == 522_753
    dropped = int(np.tril(1 - m, -1).sum())
    assert dropped == round(0.25 * eligible) == 130_688
    pairs = A.causal_pairs_fast(s.context, m)
    kept_off = n * (n - 1) // 2 - dropped
    assert pairs == kept_off * 16384 + n * 8256 == 6_448_807_936
    assert A.prefill_flops(32, 128, [s.context], m) == 4 * 128 * 32 * pairs


def test_generator_is_seeded_and_structured():
    spec = W.small("decode", B=3, Hq=4, Hkv=2, ragged=(5, 300), bits=4, seed=9,
                   n_int8_heads=1, outlier_frac=0.05, outlier_scale=8.0)
    a = W.make_inputs(spec)
    b = W.make_inputs(spec)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert a.k.dtype == np.float16 and a.k.shape == (3, 2, spec.cap, 128)
    for bi, n in enumerate(a.structure.seq_lens):
        assert 5 <= n <= 300
        assert not a.k[bi, :, n:].any() and not a.v[bi, :, n:].any()
    assert sorted(a.structure.head_bits.tolist()) == [4, 8]
    assert len(a.structure.outliers) == round(0.05 * 2 * 128)
    c = W.make_inputs(spec, seed=10)
    assert not np.array_equal(a.q, c.q)


def test_ragged_lengths_of_the_batched_decode_workload():
    s = W.WORKLOADS["decode_ragged"]
    st = W._draw_structure(s, np.random.default_rng(s.seed))
    assert st.seq_lens.shape == (64,)
    assert st.seq_lens.min() >= 1024 and st.seq_lens.max() <= 32768
    assert s.cap == 32768
