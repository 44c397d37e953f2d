"""Work accounting: closed forms against brute-force counts of the oracle's mask,
and the per-workload figures used by the benchmark."""

import numpy as np
import pytest

import oracle
from exact_io_aware_attn_amd import accounting as acc
from exact_io_aware_attn_amd.inputs import WORKLOADS, frame_block_mask


@pytest.mark.parametrize("nq,nk", [(1, 1), (7, 7), (5, 13), (13, 5), (64, 64), (1, 40)])
def test_causal_pairs_match_mask_count(nq, nk):
    brute = int(oracle.element_mask(nq, nk, causal=True).sum())
    assert acc.attended_pairs(nq, nk, causal=True) == brute


def test_causal_square_closed_form():
    for n in (1, 2, 17, 1024, 8192):
        assert acc.attended_pairs(n, n, causal=True) == n * (n + 1) // 2


@pytest.mark.parametrize("causal", [False, True])
def test_block_pairs_match_mask_count(causal):
    rng = np.random.default_rng(3)
    bm = (rng.random((4, 6)) < 0.5).astype(np.uint8)
    brute = int(oracle.element_mask(64, 96, causal=causal, block_mask=bm, block_q=16, block_k=16).sum())
    assert acc.attended_pairs(64, 96, causal=causal, block_mask=bm, block_q=16, block_k=16) == brute


def test_flop_rule_matches_dense_gemm_counts():
    # S = Q K^T is N x N outputs of length-d dot products (2 N^2 d), and P V the same
    N, d = 300, 64
    assert acc.prefill_flops(1, 1, d, acc.attended_pairs(N, N)) == 2 * (2 * N * N * d)


def test_decode_bytes_and_intensity():
    # one head, N cached keys: K alone is N d elements; K and V together 2 N d
    N, d = 1000, 128
    assert acc.decode_kv_bytes([N], 1, d, elem_bytes=2) == 2 * N * d * 2
    # arithmetic intensity 2/sizeof per query head sharing the KV head
    assert acc.decode_flops([N], 1, d) / acc.decode_kv_bytes([N], 1, d, 2) == pytest.approx(1.0)


def test_workload_figures():
    w = WORKLOADS["gpt2-causal"]
    assert acc.attended_pairs(w.Nq, w.Nk, causal=True) == 524_800
    assert acc.workload_work(w)[0] == 524_800 * 96 * 256
    w = WORKLOADS["llama3-8b-gqa-causal-8k"]
    assert acc.attended_pairs(w.Nq, w.Nk, causal=True) == 33_558_528
    w = WORKLOADS["video-frames-16x880"]
    bm = frame_block_mask(w.frames, w.frame_len, w.block)
    assert bm.shape == (176, 176) and int(bm.sum()) == 7260
    pairs = acc.attended_pairs(w.Nq, w.Nk, block_mask=bm, block_q=80, block_k=80)
    assert pairs == 46_464_000
    assert acc.workload_work(w, block_mask=bm)[0] == 46_464_000 * 24 * 512


def test_backward_work_counts():
    # 10 d FLOPs per attended pair: S recomputed, then dV, dP, dQ and dK, each a
    # length-d product per pair, i.e. 2.5 times the forward's 4 d
    w = WORKLOADS["llama3-8b-gqa-causal-8k-bwd"]
    f, b = acc.workload_work(w)
    pairs = 8192 * 8193 // 2
    assert f == 10 * 128 * pairs * 32
    assert f * 2 == 5 * acc.workload_work(WORKLOADS["llama3-8b-gqa-causal-8k"])[0]
    # read Q, O, dO (queries) and K, V; write dQ, dK, dV; read the LSE
    assert b == 2 * 128 * (8192 * 32 * 4 + 8192 * 8 * 4) + 4 * 32 * 8192
