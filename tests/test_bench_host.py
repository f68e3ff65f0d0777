"""Host-side checks of bench.py (no GPU): the kernel-source hash that ties
the stored traffic counters to the kernels covers every kernel source (the
ABI's host-only argument checks are not kernel code), and
the algorithmic work counts follow their definitions."""
import glob
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_hash_covers_every_kernel_source():
    csrc = sorted(os.path.relpath(f, ROOT) for f in
                  glob.glob(os.path.join(ROOT, "tiled_attention_transformer_amd", "csrc", "*"))
                  if f.endswith((".hip", ".h"))
                  and not os.path.basename(f).startswith(("attn_api", "host_checks")))
    assert sorted(bench.KERNEL_SOURCES) == csrc


def test_prefill_flops_counts_allowed_pairs():
    # causal Sq = Skv = S: S(S+1)/2 pairs per head, 4d flops each
    assert bench.prefill_flops(1, 1, 4, 4, 8, True) == 4 * 8 * 10
    assert bench.prefill_flops(2, 3, 5, 7, 16, False) == 4 * 16 * 5 * 7 * 6
    # bottom-right causal with Sq < Skv: row i sees i + Skv - Sq + 1 keys
    assert bench.prefill_flops(1, 1, 2, 5, 1, True) == 4 * (4 + 5)
    # the causal C2 workload of the benchmark
    assert bench.prefill_flops(4, 16, 2048, 2048, 128, True) == 68753031168


def test_decode_bytes_of_the_decode_workload():
    # K + V 1 GiB, Q and O 0.5 MiB each, LSE 8 KiB
    assert bench.decode_bytes(64, 32, 8, 4096, 128) == 1074798592
    # fp8 codes halve the cache bytes only
    assert bench.decode_bytes(64, 32, 8, 4096, 128, kv_elem_bytes=1) == 537927680
