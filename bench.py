#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * the causal prefill workload B=4, H=16 (MHA), Sq=Skv=2048, d=128, through
    attn_fwd (Q tile load, K/V tile streaming, Q*K^T, mask, online softmax,
    P*V, epilogue), and
  * the GQA decode workload B=64, Hq=32, Hkv=8, Skv=4096, d=128, 8 key
    chunks, through attn_decode (chunked attention + log-sum-exp merge of
    the chunks).
Inputs are seeded bf16 N(0,1) draws already resident in HBM when timing
starts.  ``value`` is the prefill throughput in algorithmic TFLOP/s (4*d per
allowed query/key pair); the decode rate in algorithmic GB/s (K and V read
once, plus Q, O and LSE) is reported beside it.

Timing: after the cold first calls, steps run back to back for ``--settle``
seconds (the GPU clocks ramp up under load), then ``--warmup`` steps, then
the K timed steps: their K prefill calls back to back, then their K decode
calls, with HIP events on the launch stream before, between and after the
two blocks (an event between every two kernels would add several
microseconds of idle time per kernel).  Each kernel's average duration is its
block's time / K.

Prints ONE JSON line.  ``--gpus N`` with N > 1 is refused: the benchmark runs
on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "attn fwd TFLOP/s (bf16 causal prefill) + decode KV GB/s, % of roofline"
KERNEL_SOURCES = ["tiled_attention_transformer_amd/csrc/attn_fwd.hip",
                  "tiled_attention_transformer_amd/csrc/attn_decode.hip",
                  "tiled_attention_transformer_amd/csrc/kmeans_assign.hip",
                  "tiled_attention_transformer_amd/csrc/tile_common.h",
                  "tiled_attention_transformer_amd/csrc/tile_config.h",
                  "tiled_attention_transformer_amd/csrc/kernels.h",
                  "tiled_attention_transformer_amd/csrc/fastdiv.h",
                  "tiled_attention_transformer_amd/csrc/exp2_poly.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_flops(B, H, Sq, Skv, d, causal):
    if causal:
        off = Skv - Sq
        pairs = sum(max(0, min(Skv, i + off + 1)) for i in range(Sq))
    else:
        pairs = Sq * Skv
    return 4.0 * d * pairs * B * H


def decode_bytes(B, Hq, Hkv, Skv, d, kv_elem_bytes=2):
    """K and V read once (bf16, or 1-byte fp8 codes), Q read, O and LSE written."""
    kv = 2 * B * Skv * Hkv * d * kv_elem_bytes
    return kv + B * Hq * d * 2 + B * Hq * d * 2 + B * Hq * 4


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")
# which kernels make up each reported path (substrings of the rocprofv3 names)
TRAFFIC_KERNELS = {"prefill": ["attn_fwd_pp_kernel<128, true, false, 4, false, 0>"],
                   "decode": ["attn_decode_split_kernel<128, false, true, false>",
                              "attn_decode_combine_kernel<128, false>"],
                   "decode_fp8": ["attn_decode_split_kernel<128, true, false, false>"],
                   "kmeans": ["kmeans_assign_kernel<128, 128>"]}
# paths whose kernels only run with a context line (absent from a run without it)
TRAFFIC_OPTIONAL = {"decode_fp8", "kmeans"}


def load_traffic(kind: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on this kernel."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    try:
        t = json.load(open(TRAFFIC_PATH))
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or kind not in t:
        return None
    return t[kind]["bytes"]


def write_traffic(fetch_dir: str, write_dir: str):
    """Turn two ``rocprofv3 --pmc`` runs of ``bench.py --copy-calibration``
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) into bytes per launch.

    Each counter is scaled by what it reads for the plain 1 GiB device copy
    in the same run, so that the copy counts as 1 GiB read and 1 GiB written.
    """
    import csv
    import glob

    def per_kernel(d, counter):
        """kernel name -> counter values of its dispatches"""
        (path,) = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch_all, write_all = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    fetch = {k: sum(v) / len(v) for k, v in fetch_all.items()}
    write = {k: sum(v) / len(v) for k, v in write_all.items()}
    copy_kib = float(1 << 20)

    def copy_value(d):
        # the 1 GiB calibration copy: the largest dispatch of the runtime's
        # device-to-device copy kernel (the run makes a few small copies
        # too; torch's dtype conversions are elementwise kernels)
        vals = [max(v) for k, v in d.items() if "copyBuffer" in k]
        if len(vals) != 1:
            sys.exit("expected exactly one device copy kernel in the counter run")
        return vals[0]

    f_scale, w_scale = copy_kib / copy_value(fetch_all), copy_kib / copy_value(write_all)
    out = {"kernel_hash": kernel_hash(),
           "calibration": {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                           "copy_bytes": 1 << 30}}
    for kind, names in TRAFFIC_KERNELS.items():
        rd = wr = 0.0
        seen = []
        for n in names:          # a kernel the path did not launch is skipped
            kf = [k for k in fetch if n in k]
            kw = [k for k in write if n in k]
            if len(kf) > 1 or len(kw) > 1:
                sys.exit("ambiguous kernel name %r in the counter run" % n)
            if kf and kw:
                rd += fetch[kf[0]] * f_scale * 1024
                wr += write[kw[0]] * w_scale * 1024
                seen.append(kf[0])
        if not seen:
            if kind in TRAFFIC_OPTIONAL:
                continue
            sys.exit("no %s kernel in the counter run" % kind)
        out[kind] = {"bytes": int(round(rd + wr)), "read_bytes": int(round(rd)),
                     "write_bytes": int(round(wr)), "kernels": seen}
    with open(TRAFFIC_PATH, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


COUNTERS_PATH = os.path.join(ROOT, "profiles", "sq_counters.json")
# One rocprofv3 --pmc pass each (at most 8 SQ counters and 2 GRBM per pass).
COUNTER_PASSES = [
    ["MfmaUtil", "VALUBusy", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES",
     "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_WAVE_CYCLES",
     "SQ_WAIT_ANY", "SQ_INSTS_MFMA"],
    ["GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS",
     "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_INSTS_VMEM", "SQ_ACTIVE_INST_ANY"],
]
COUNTER_KERNELS = {"prefill": "attn_fwd_pp_kernel<128, true, false, 4, false, 0>",
                   "decode": "attn_decode_split_kernel<128, false, true, false>",
                   "decode_fp8": "attn_decode_split_kernel<128, true, false, false>",
                   "kmeans": "kmeans_assign_kernel<128, 128>"}


def write_counters(dirs):
    """Turn ``rocprofv3 --pmc`` runs (one folder per pass of COUNTER_PASSES)
    into per-kernel means per dispatch, plus:

      mfma_util  = rocprofv3's MfmaUtil (MFMA-busy cycles over all SIMDs'
                   active cycles), as a fraction
      valu_busy  = rocprofv3's VALUBusy, as a fraction
      coexec     = share of SIMD cycles in which the MFMA unit was busy and
                   a plain VALU instruction issued (MfmaUtil scaled by
                   SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES)
      wait_any   = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of wave time waiting)
      mfma_flop  = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (matrix FLOP executed)
    """
    import csv
    import glob
    vals = {}
    for d in dirs:
        (path,) = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        per = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Counter_Name"], r.get("Dispatch_Id", ""))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (kn, cn, _), v in per.items():
            vals.setdefault(kn, {}).setdefault(cn, []).append(v)
    out = {"kernel_hash": kernel_hash(), "passes": COUNTER_PASSES, "kernels": {}}
    for kind, name in COUNTER_KERNELS.items():
        ks = [k for k in vals if name in k]
        if len(ks) != 1:
            continue
        c = {cn: sum(v) / len(v) for cn, v in vals[ks[0]].items()}
        der = {}
        if "MfmaUtil" in c:
            der["mfma_util"] = c["MfmaUtil"] / 100.0
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                der["coexec"] = der["mfma_util"] * c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / \
                    c["SQ_VALU_MFMA_BUSY_CYCLES"]
        if "VALUBusy" in c:
            der["valu_busy"] = c["VALUBusy"] / 100.0
        if c.get("SQ_WAVE_CYCLES"):
            der["wait_any"] = c.get("SQ_WAIT_ANY", 0.0) / c["SQ_WAVE_CYCLES"]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            der["mfma_flop"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        out["kernels"][kind] = {"name": ks[0], "dispatches": len(vals[ks[0]].get("GRBM_GUI_ACTIVE", [])),
                                "counters": c,
                                "derived": {k: round(v, 4) for k, v in der.items()}}
    with open(COUNTERS_PATH, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def load_counters(kind: str):
    """Derived unit utilisations of a kernel, if taken on these kernel sources."""
    try:
        t = json.load(open(COUNTERS_PATH))
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or kind not in t.get("kernels", {}):
        return None
    return t["kernels"][kind]["derived"]


EXTRAS = ("decode_auto", "fp8", "skewed", "kmeans", "long", "ragged", "exp2_poly")


def extra_workloads(api, dev, stream, which=EXTRAS, calls=20, dec_ms=None, dec_inputs=None):
    """Context lines beside the headline: the long causal workload (B1 H32
    S16384 d128), the ragged causal batch (16 sequences, lengths drawn
    U{128..8192} with seed 5, H32 d128), the decode workload's sizes with
    an fp8 (e4m3fn) KV cache, and the fused k-means assignment (N=65536,
    K=1024, d=128; algorithmic FLOP 2*N*K*d).  Timing only: the inputs are seeded N(0,1)
    draws made on the GPU (the lengths follow the same recipe as the test
    inputs); K of the long workload is scaled per head by U(0.5, 2) as in its
    test recipe; the fp8 cache holds the codes of x / (max|x| / 448) per
    tensor, as the test recipe does; the k-means points and centroids follow
    the test recipe's mixture; the skewed decode has the decode workload's
    heads with one sequence of 32768 keys among 63 of 256 (cache capacity
    32768).  ``which`` names the lines to run (a subset of EXTRAS)."""
    import torch
    out = {}
    gen = torch.Generator(device=dev)
    d = 128

    def timed(fn, warm=0, n=calls, settle=0.2):
        # fresh buffers: the first calls also pay first-touch address
        # translation, and the clocks ramp up under load, so calls run back
        # to back for `settle` seconds first; then n calls back to back
        # between one pair of events
        t = time.perf_counter()
        while time.perf_counter() - t < settle:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
        for _ in range(warm):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # the decode workload with the library's split choice (whole sequences
    # per workgroup, waves merged in the kernel, no workspace)
    if "decode_auto" in which and dec_inputs is not None:
        dq, dk, dv, do, dlse, spec = dec_inputs
        ms = timed(lambda: api.attn_decode(dq, dk, dv, o=do, lse=dlse, scale=spec["scale"],
                                           num_splits=0, stream=stream), n=50)
        nb = decode_bytes(spec["B"], spec["Hq"], spec["Hkv"], spec["Skv"], spec["d"])
        gbs = nb / (ms * 1e-3) / 1e9
        out["decode_library_choice_B64_Hq32_Hkv8_Skv4096_d128"] = {
            "ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_of_8000": round(gbs / PEAK_HBM_GBS, 4),
            "num_splits": api.attn_decode_pick_splits(spec["B"], spec["Hq"], spec["Hkv"], spec["Skv"]),
            "algorithmic_bytes": nb, "traffic": load_traffic("decode_auto"),
            "kernel": "attn_decode_split_kernel<128, false, false, false> (whole sequences per "
                      "workgroup, the four waves merged in the kernel)"}
    # decode with an fp8 KV cache (the decode workload's sizes)
    if "fp8" in which:
        fp8_decode(api, dev, stream, gen, d, timed, out, dec_ms)
    if "skewed" in which:
        skewed_decode(api, dev, stream, gen, d, timed, out)
    if "kmeans" in which:
        kmeans_assign(api, dev, stream, gen, d, timed, out)
    if "long" in which:
        long_causal(api, dev, stream, gen, d, timed, out)
    if "ragged" in which:
        ragged_causal(api, dev, stream, gen, d, timed, out)
    if "exp2_poly" in which:
        exp2_poly_prefill(api, dev, stream, gen, d, timed, out)
    return out


def exp2_poly_prefill(api, dev, stream, gen, d, timed, out):
    """The causal prefill workload (B4 H16 S2048) and the long one (B1 H32
    S16384) with 0 (attn_fwd), 4, 8 and 16 of each lane's 32 exponentials per
    key tile on the library's exp2 polynomial (attn_fwd_exp2_poly), timed
    one after the other on the same inputs."""
    import torch
    res = {}
    for name, (B, H, S, seed, n) in (("B4_H16_S2048", (4, 16, 2048, 2, 50)),
                                     ("B1_H32_S16384", (1, 32, 16384, 3, 10))):
        gen.manual_seed(seed)
        q, k, v = (torch.randn((B, S, H, d), generator=gen, device=dev, dtype=torch.float32)
                   .to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        fl = prefill_flops(B, H, S, S, d, True)
        line = {}
        for share in (0, 4, 8, 16):
            if share == 0:
                fn = lambda: api.attn_fwd(q, k, v, o=o, lse=lse, causal=True, stream=stream)
            else:
                fn = (lambda sh: lambda: api.attn_fwd_exp2_poly(q, k, v, sh, o=o, lse=lse,
                                                                causal=True, stream=stream))(share)
            ms = timed(fn, n=n)
            line["poly_%d_of_32" % share] = {
                "ms": round(ms, 5), "frac_of_2500": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        res["causal_" + name + "_d128"] = line
        del q, k, v, o, lse
    out["prefill_exp2_poly_share"] = res


def fp8_decode(api, dev, stream, gen, d, timed, out, dec_ms):
    import torch
    gen.manual_seed(4)
    B, Hq, Hkv, Skv = 64, 32, 8, 4096
    q = torch.randn((B, Hq, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    codes, scales = [], []
    for _ in range(2):
        x = torch.randn((B, Skv, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
        sc = float(x.abs().max()) / 448.0
        codes.append((x / sc).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
        scales.append(sc)
        del x
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    # the library's split choice (whole sequences per workgroup at these sizes)
    ws = torch.empty(max(1, api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, 0)),
                     dtype=torch.uint8, device=dev)
    ms = timed(lambda: api.attn_decode_fp8(q, codes[0], codes[1], scales[0], scales[1], o=o,
                                           lse=lse, num_splits=0, workspace=ws, stream=stream),
               n=50)
    nb = decode_bytes(B, Hq, Hkv, Skv, d, kv_elem_bytes=1)
    gbs = nb / (ms * 1e-3) / 1e9
    out["decode_fp8_kv_B64_Hq32_Hkv8_Skv4096_d128"] = {
        "ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_of_8000": round(gbs / PEAK_HBM_GBS, 4),
        "algorithmic_bytes": nb, "traffic": load_traffic("decode_fp8"),
        "kernel": "attn_decode_split_kernel<128, true, false, false> (library's split choice: "
                  "whole sequences per workgroup)",
        "speedup_vs_bf16_cache": None if dec_ms is None else round(dec_ms / ms, 3)}
    del q, codes, o, lse, ws


def skewed_decode(api, dev, stream, gen, d, timed, out):
    """ragged decode (per-sequence key counts on the device) with one long
    sequence: the split by the lengths (the library's choice with a
    workspace of attn_decode_varlen_workspace_bytes: the kernel reads the
    lengths and gives every wave an equal run of key tiles), the split by the
    capacity (the library's choice with the smaller workspace: the host never
    sees the lengths) and an explicit 16-way split"""
    import torch
    gen.manual_seed(6)
    B, Hq, Hkv, cap = 64, 32, 8, 32768
    lens = [256] * 17 + [cap] + [256] * 46
    k, v = (torch.randn((B, cap, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
            .to(torch.bfloat16) for _ in range(2))
    q = torch.randn((B, Hq, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    nb = sum(lens) * Hkv * d * 2 * 2 + 2 * B * Hq * d * 2 + B * Hq * 4
    line = {"algorithmic_bytes": nb, "lengths": "17 x 256, 1 x 32768, 46 x 256"}
    runs = (("split_by_lengths", 0, api.attn_decode_varlen_workspace_bytes(B, Hq, Hkv, cap, d)),
            ("split_by_capacity", 0, api.attn_decode_workspace_bytes(B, Hq, Hkv, cap, d, 0)),
            ("splits_16", 16, api.attn_decode_workspace_bytes(B, Hq, Hkv, cap, d, 16)))
    for name, ns, nbytes in runs:
        ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
        ms = timed(lambda: api.attn_decode_varlen(q, k, v, sl, o=o, lse=lse, scale=d ** -0.5,
                                                  num_splits=ns, workspace=ws, stream=stream),
                   n=50)
        gbs = nb / (ms * 1e-3) / 1e9
        r = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_of_8000": round(gbs / PEAK_HBM_GBS, 4),
             "workspace_bytes": nbytes}
        if name != "split_by_lengths":
            r["num_splits"] = api.attn_decode_pick_splits(B, Hq, Hkv, cap) if ns == 0 else ns
        else:
            r["kernel"] = ("attn_decode_split_kernel<128, false, true, true> (an equal run of key "
                           "tiles per wave) + attn_decode_combine_kernel<128, true>")
        line[name] = r
        del ws
    out["decode_varlen_skewed_B64_Hq32_Hkv8_cap32768_d128"] = line
    del k, v, q, o, lse, sl


def kmeans_assign(api, dev, stream, gen, d, timed, out):
    """fused k-means assignment (N=65536 points, K=1024 centroids, d=128: the
    Flash-KMeans article's assignment workload), mixture recipe as in the tests"""
    import torch
    gen.manual_seed(7)
    N, K = 65536, 1024
    mu = torch.randn((K, d), generator=gen, device=dev, dtype=torch.float32)
    lab = torch.randint(0, K, (N,), generator=gen, device=dev)
    x = (mu[lab] + 0.5 * torch.randn((N, d), generator=gen, device=dev)).to(torch.bfloat16)
    c = (mu + 0.25 * torch.randn((K, d), generator=gen, device=dev)).to(torch.bfloat16)
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    dist = torch.empty(N, dtype=torch.float32, device=dev)
    ms = timed(lambda: api.attn_kmeans_assign(x, c, idx=idx, dist=dist, stream=stream), n=50)
    fl = 2.0 * N * K * d
    out["kmeans_assign_N65536_K1024_d128"] = {
        "ms": round(ms, 5), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
        "frac_of_2500": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flop": fl, "traffic": load_traffic("kmeans"),
        "kernel": "kmeans_assign_kernel<128, 128>"}
    del mu, lab, x, c, idx, dist


def long_causal(api, dev, stream, gen, d, timed, out):
    import torch
    gen.manual_seed(3)
    B, H, S = 1, 32, 16384
    q, k, v = (torch.randn((B, S, H, d), generator=gen, device=dev, dtype=torch.float32)
               for _ in range(3))
    k = k * (0.5 + 1.5 * torch.rand((1, 1, H, 1), generator=gen, device=dev))
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ms = timed(lambda: api.attn_fwd(q, k, v, o=o, lse=lse, causal=True, stream=stream))
    fl = prefill_flops(B, H, S, S, d, True)
    out["long_causal_B1_H32_S16384_d128"] = {
        "ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
        "frac_of_2500": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, o, lse


def ragged_causal(api, dev, stream, gen, d, timed, out):
    import torch
    lengths = np.random.default_rng(5).integers(128, 8192 + 1, 16)
    cu = np.zeros(17, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    total, H = int(cu[-1]), 32
    gen.manual_seed(5)
    q, k, v = (torch.randn((total, H, d), generator=gen, device=dev, dtype=torch.float32)
               .to(torch.bfloat16) for _ in range(3))
    cu_d = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    mx = int(lengths.max())
    ms = timed(lambda: api.attn_fwd_varlen(q, k, v, cu_d, cu_d, mx, mx, o=o, lse=lse,
                                           causal=True, stream=stream))
    fl = float(sum(4.0 * d * H * L * (L + 1) / 2 for L in lengths))
    out["ragged_causal_16seq_H32_d128"] = {
        "ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
        "frac_of_2500": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "total_tokens": total, "algorithmic_flop": fl}


def cpu_baseline(spec, data, max_pairs):
    """The C oracle on a bounded sample of the prefill workload (rank 0 only)."""
    from oracle import cpu
    B, H, S, d = spec["B"], spec["Hq"], spec["Sq"], spec["d"]
    # whole heads, taken in a fixed order, until the sample holds max_pairs pairs
    pairs_per_head = S * (S + 1) // 2
    nheads = max(1, min(B * H, int(max_pairs // pairs_per_head)))
    heads = [(b, h) for b in range(B) for h in range(H)][:nheads]
    rows = np.array([(b, h, i) for (b, h) in heads for i in range(S)], dtype=np.int64)
    threads = cpu.num_threads(0)
    t0 = time.perf_counter()
    cpu.attn_rows(data["q"], data["k"], data["v"], spec["scale"], True, rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * d * pairs_per_head * nheads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d of %d (batch, head) pairs of the causal prefill workload, all %d rows "
                      "each (fp64 C loops, OpenMP)" % (nheads, B * H, S)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the timed ones")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of back-to-back steps before the warm-up steps, so the "
                         "GPU clocks have ramped up (reported as settle_s / settle_steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", default="all",
                    help="context workloads beside the headline: all, none, or a comma list "
                         "of %s" % ",".join(EXTRAS))
    ap.add_argument("--no-extra", action="store_true",
                    help="skip every context line (same as --extra none)")
    ap.add_argument("--cpu-pairs", type=float, default=2.0e8,
                    help="allowed query/key pairs in the CPU-baseline sample")
    ap.add_argument("--write-counters", nargs="+", metavar="DIR",
                    help="write profiles/sq_counters.json from rocprofv3 --pmc output folders "
                         "(one per counter pass) and exit (no GPU use)")
    ap.add_argument("--counter-pass", type=int, metavar="N",
                    help="print the counters of pass N (for rocprofv3 --pmc) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--extra-only", action="store_true",
                    help="time only the context workloads named by --extra (no headline step, "
                         "no CPU baseline) and print them as one JSON line: for profiling one "
                         "workload at a time")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output folders "
                         "and exit (no GPU use)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_counters:
        write_counters(args.write_counters)
        return
    if args.counter_pass is not None:
        print(" ".join(COUNTER_PASSES[args.counter_pass]))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.extra not in ("all", "none") and not set(args.extra.split(",")) <= set(EXTRAS):
        sys.exit("--extra takes all, none, or a comma list of " + ",".join(EXTRAS))
    if args.steps < 1 or args.warmup < 0:
        sys.exit("steps must be >= 1 and warmup >= 0")

    import torch
    import synth_inputs as si
    from tiled_attention_transformer_amd import api

    dev = torch.device("cuda:0")
    api._lib.load()
    if args.extra_only:
        which = EXTRAS if args.extra == "all" else tuple(x for x in args.extra.split(",") if x)
        which = tuple(x for x in which if x != "decode_auto")   # needs the headline's inputs
        print(json.dumps({"extra": extra_workloads(api, dev, torch.cuda.current_stream(),
                                                   which=which), "kernel_hash": kernel_hash()}),
              flush=True)
        return

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    pspec, pdata = si.make_workload("causal_prefill")
    dspec, ddata = si.make_workload("gqa_decode")
    q, k, v = (to_dev(pdata[n]) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((pspec["B"], pspec["Hq"], pspec["Sq"]), dtype=torch.float32, device=dev)
    dq, dk, dv = (to_dev(ddata[n]) for n in "qkv")
    do = torch.empty_like(dq)
    dlse = torch.empty((dspec["B"], dspec["Hq"]), dtype=torch.float32, device=dev)
    nsplit = dspec["num_splits"]
    ws = torch.empty(max(1, api.attn_decode_workspace_bytes(dspec["B"], dspec["Hq"], dspec["Hkv"],
                                                            dspec["Skv"], dspec["d"], nsplit)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def prefill():
        api.attn_fwd(q, k, v, o=o, lse=lse, scale=pspec["scale"], causal=True, stream=stream)

    def decode():
        api.attn_decode(dq, dk, dv, o=do, lse=dlse, scale=dspec["scale"], num_splits=nsplit,
                        workspace=ws, stream=stream)

    # cold (first) calls, reported apart from the steady state
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    prefill()
    e1.record(stream)
    decode()
    e2.record(stream)
    torch.cuda.synchronize()
    cold_prefill_ms, cold_decode_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)

    # Clock settle: the GPU clocks take some tens of milliseconds of steady
    # load to ramp up, so steps run back to back for args.settle seconds
    # before the warm-up steps, whatever their count (reported apart).
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(10):
            prefill()
            decode()
        settle_steps += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle

    for _ in range(args.warmup):
        prefill()
        decode()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Timed region: the K steps' prefill calls launched back to back, then
    # their K decode calls, with one event before, between and after the two
    # blocks on the launch stream.  An event recorded between two kernels
    # adds several microseconds of idle GPU time (measured ~5 us per event
    # against a kernel trace), so events go only at the block boundaries;
    # the kernels' averages are then block time / K, launch gaps included.
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(K):
        prefill()
    ev[1].record(stream)
    for _ in range(K):
        decode()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_avg = ev[0].elapsed_time(ev[1]) / K
    dec_avg = ev[1].elapsed_time(ev[2]) / K
    step_ms = ev[0].elapsed_time(ev[2]) / K

    flops = prefill_flops(pspec["B"], pspec["Hq"], pspec["Sq"], pspec["Skv"], pspec["d"], True)
    nbytes = decode_bytes(dspec["B"], dspec["Hq"], dspec["Hkv"], dspec["Skv"], dspec["d"])
    tflops = flops / (pre_avg * 1e-3) / 1e12
    gbs = nbytes / (dec_avg * 1e-3) / 1e9

    traffic = load_traffic("prefill")
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "settle_s": round(settle_s, 3),
        "settle_steps": settle_steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1))",
        "config": {
            "workload": "causal prefill B4 H16 Sq=Skv=2048 d128 + GQA decode B64 Hq32 Hkv8 "
                        "Skv4096 d128 split into %d KV chunks, then the LSE merge kernel" % nsplit,
            "prefill": {"B": 4, "Hq": 16, "Hkv": 16, "S": 2048, "d": 128, "causal": True,
                        "seed": pspec["seed"], "algorithmic_flop": flops},
            "decode": {"B": 64, "Hq": 32, "Hkv": 8, "Skv": 4096, "d": 128, "num_splits": nsplit,
                       "seed": dspec["seed"], "algorithmic_bytes": nbytes},
        },
        "prefill_ms": {"mean": round(pre_avg, 5), "cold": round(cold_prefill_ms, 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_pp_kernel<128, true, false, 4, false, 0>",
                     "counters": load_counters("prefill")},
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s",
            "ms": {"mean": round(dec_avg, 5), "cold": round(cold_decode_ms, 5)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("decode"), "counters": load_counters("decode"),
                         "kernel": "attn_decode_split_kernel<128, false, true, false> (%d key chunks "
                                   "per sequence, one chunk per wave at a time) + "
                                   "attn_decode_combine_kernel<128, false> (LSE merge of the chunks)"
                                   % nsplit},
        },
        "kernel_hash": kernel_hash(),
    }
    which = () if args.no_extra or args.extra == "none" else \
        EXTRAS if args.extra == "all" else tuple(args.extra.split(","))
    if which:
        result["extra"] = extra_workloads(api, dev, stream, which=which, dec_ms=dec_avg,
                                          dec_inputs=(dq, dk, dv, do, dlse, dspec))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pspec, pdata, args.cpu_pairs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
