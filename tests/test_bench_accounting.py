"""Host checks of bench.py's algorithmic work accounting (no GPU): visible
(query, key) pairs counted by enumeration, bytes by tensor sizes, and the
one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _pairs(T, T_kv, causal):
    # query i is the token at position T_kv - T + i; it sees keys at positions <= its own
    return sum(1 for i in range(T) for j in range(T_kv) if not causal or j <= T_kv - T + i)


def test_prefill_flops_count_visible_pairs():
    for T, T_kv, causal in ((7, 7, True), (3, 11, True), (5, 5, False), (4, 9, False), (1, 6, True)):
        for D, DV in ((8, 8), (12, 5)):
            want = 2 * 3 * _pairs(T, T_kv, causal) * 2 * (D + DV)
            assert bench.prefill_flops(2, 3, T, D, causal=causal, T_kv=T_kv, DV=DV) == want


def test_prefill_bytes_are_tensor_sizes():
    B, Hq, Hkv, T, T_kv, D, DV = 2, 16, 1, 1024, 8192, 512, 512
    q = B * Hq * T * D
    out = B * Hq * T * DV
    kv = B * Hkv * T_kv * (D + DV)
    assert bench.prefill_bytes(B, Hq, Hkv, T, D, T_kv=T_kv, DV=DV) == 2 * (q + out + kv)
    assert bench.prefill_bytes(1, 128, 128, 8192, 192, DV=128) == 2 * 128 * 8192 * (192 + 128) * 2


def test_decode_and_mla_bytes():
    sl = np.array([5, 7], dtype=np.int32)
    assert bench.decode_bytes(2, 4, 2, 8, sl) == 12 * 2 * 2 * 8 * 2 + 2 * 4 * 8 * 2 * 2
    # each latent row (576 values) is read once; value aliases the key
    assert bench.mla_bytes(2, 4, 576, sl) == 12 * 576 * 2 + 2 * 4 * 576 * 2 + 2 * 4 * 512 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_dispatch_assignment_walks_the_step_order():
    # two steps of two workloads, with set-up and library kernels between
    names = ["mqa_prefill_bf16_b2_t4096", "mqa_decode_bf16_b64_l8192"]
    step = ["void mqa::kv_pack_kernel<512, 512, 32>(...)", "at::native::fill(...)",
            "void mqa::prefill_bf16_kernel<512, 512, 1, 4, 32, true, false, false>(...)",
            "void mqa::decode_split_kernel<512, 1, 4, false>(...)",
            "void mqa::lse_merge_kernel<512, false, false>(...)"]
    seq = ["at::native::copy(...)"] + step + step
    got = bench.assign_dispatches(seq, names)
    want_step = [(names[0], 0), None, (names[0], 1), (names[1], 0), (names[1], 1)]
    assert got == [None] + want_step + want_step


def test_dispatch_assignment_keeps_shared_kernel_names_apart():
    # the chunked prefill dispatches the same kernels as the full prefill;
    # only the position in the step tells them apart
    names = ["mqa_prefill_bf16_b2_t4096", "mqa_chunk_prefill_bf16_b2_q1024_kv8192"]
    k = ["mqa::kv_pack_kernel<512, 512, 32>", "mqa::prefill_bf16_kernel<512, 512, 1, 4, 32, true, false, false>"]
    got = bench.assign_dispatches(k * 4, names)
    assert got == [(names[0], 0), (names[0], 1), (names[1], 0), (names[1], 1)] * 2


def test_dispatch_assignment_covers_a_whole_step():
    # one dispatch per kernel slot of every workload, in step order, twice:
    # every dispatch is assigned (a stale pattern would leave the walk
    # waiting and drop whole steps)
    seq = []
    for n, _ in bench.ORDER:
        seq += [f"void mqa::{pat}_x>(...)" for pat in bench.CALL_KERNELS[n]]
    got = bench.assign_dispatches(seq + seq)
    assert all(a is not None for a in got)
    assert sum(1 for a in got if a == (bench.ORDER[0][0], 0)) == 2


def test_mla_workloads_name_the_mla_merge():
    # the MLA decodes merge their partials with their own kernel
    for n in ("mla_decode_bf16_b32_l32768", "mla_sparse_decode_bf16_b32_l32768_k2048"):
        assert bench.CALL_KERNELS[n][1] == "mla_merge_kernel"
    src = open(os.path.join(ROOT, "attention_mqa_gqa_amd", "csrc", "mla_decode.hip")).read()
    assert "mla_merge_kernel<" in src and "merge_launch(" not in src
