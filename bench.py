#!/usr/bin/env python3
"""Throughput of the tree-verify MLA-absorb attention step on one MI355X.

One step = one pass of the whole hot path over one batch of trees:
  tv_tree_rope    rotate the queries and the tree's own key rows at
                  prefix + depth (float64 angles), in place, then
  tv_verify_attn  prefix + ancestor masked softmax attention in the absorbed
                  latent space, writing out [B, q_len, H, d_c].
The prefix key rows are rotated once before timing (the cache holds keys
rotated when they were written).  Inputs are seeded synthetic tensors already
resident in HBM when the timed region starts.

Prints ONE JSON line.  `value` is steps (verify calls) per second.  The
`roofline` object is for the attention kernel, timed with HIP events on the
stream it runs on; `cpu_baseline` times the float64 CPU oracle on a bounded
sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-attn calls/sec + achieved HBM GB/s (% roofline) at B,H,prefix,budget"
HBM_PEAK_GBS = 8000.0
PEAKS_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32_mfma": 157.3, "f32_valu": 157.3}

# Which kernel the library runs for each cache dtype, the arithmetic it does,
# and the roofline that bounds it.
KERNELS = {
    # (query_terms: the score product runs once per bf16 term of the queries)
    "bf16": dict(name="attn_mfma_q2_kernel",
                 source=["tree_verify_mla_tv_amd/csrc/attn_mfma_q2.hip", "tree_verify_mla_tv_amd/csrc/attn_mfma_q2_asm.h",
                         "tree_verify_mla_tv_amd/csrc/attn_mfma_common.h", "tree_verify_mla_tv_amd/csrc/attn_mfma_asm.h",
                         "tree_verify_mla_tv_amd/csrc/tv_kernels.h"],
                 bound="mfma", peak="bf16", dtype="bf16", query_terms=2),
    # tv_verify_attn_ex with TV_ATTN_BF16_QUERIES: the queries rounded to one bf16 term
    "bf16_queries": dict(name="attn_mfma_bf16_kernel",
                         source=["tree_verify_mla_tv_amd/csrc/attn_mfma.hip",
                                 "tree_verify_mla_tv_amd/csrc/attn_mfma_common.h",
                                 "tree_verify_mla_tv_amd/csrc/attn_mfma_asm.h",
                                 "tree_verify_mla_tv_amd/csrc/tv_kernels.h"],
                         bound="mfma", peak="bf16", dtype="bf16"),
    "f32": dict(name="attn_mfma_f32_kernel", source=["tree_verify_mla_tv_amd/csrc/attn_mfma_f32.hip",
                                                    "tree_verify_mla_tv_amd/csrc/tv_kernels.h"], bound="mfma",
                peak="f32_mfma", dtype="f32"),
}


def strip_comments(text: str) -> str:
    """C/C++ source without its // and /* */ comments (string and character
    literals kept whole), whitespace runs collapsed: edits to comments or
    layout leave it unchanged, any change to the code does not."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(rels) -> str:
    """First 16 hex digits of sha256 over the kernel's source files, in order,
    each without its comments (strip_comments)."""
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def algorithmic_counts(w, parent) -> dict:
    """Bytes and flops of the step's tensors, each touched once (per call)."""
    import numpy as np
    kvb = 2 if w.kv_dtype == "bf16" else 4
    B, q, H, P, kv, dc, dr = w.B, w.q_len, w.H, w.prefix_len, w.kv_len, w.d_c, w.d_r
    depth = np.zeros_like(parent)
    for b in range(B):
        for i in range(1, q):
            depth[b, i] = depth[b, parent[b, i]] + 1
    visible_pairs = int(H * (P + depth + 1).sum())
    flops = visible_pairs * (2 * (dc + dr) + 2 * dc)
    attn_bytes = (B * q * H * dc * 4 + B * q * H * dr * 4 + B * kv * dc * kvb + B * kv * dr * kvb
                  + B * q * 4 + B * q * H * dc * 4)
    rope_bytes = 2 * (B * q * H * dr * 4 + B * q * dr * kvb) + B * q * 4
    return dict(visible_pairs=visible_pairs, flops=flops, attn_bytes=attn_bytes, rope_bytes=rope_bytes,
                step_bytes=attn_bytes + rope_bytes)


def cpu_baseline(inp, w, n_sample: int) -> dict:
    """The oracle as it stands, on the first n_sample trees of the same batch
    (the whole batch, i.e. one whole call, by default)."""
    import threadpoolctl
    from oracle import tv_oracle as O
    s = slice(0, n_sample)
    t0 = time.perf_counter()
    O.verify_step(inp["q_lat"][s], inp["q_rope"][s], inp["c_kv"][s], inp["k_rope"][s], inp["parent"][s],
                  w.prefix_len, w.theta, w.sm_scale, w.kv_dtype)
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    return {"value": round(1.0 / (dt * w.B / n_sample), 6), "seconds_per_call": round(dt * w.B / n_sample, 3),
            "unit": "calls/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "sample": (f"float64 numpy oracle (RoPE + attention), one whole call (all {w.B} trees), {dt:.2f} s"
                       if n_sample == w.B else
                       f"float64 numpy oracle (RoPE + attention) on {n_sample} of {w.B} trees of the same batch, "
                       f"{dt:.2f} s, scaled x{w.B / n_sample:g} to one call")
                      + f"; host CPUs available: {len(os.sched_getaffinity(0))}"}


def load_traffic(kernel: dict, workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kernel["source"]):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(torch) -> int:
    """A plain copy of known size: each launch reads and writes exactly 1 GiB."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "launches": 3, "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n}), flush=True)
    return 0


def _time_ms(torch, fn, reps: int, warmup: int = 1) -> float:
    """Mean ms per call over reps calls after warmup untimed ones, HIP events
    on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


SMALL_ROWS = [(1, 1, 1, 5000), (1, 1, 1, 32768), (4, 1, 1, 8192), (1, 16, 1, 8192), (1, 16, 2, 8192),
              (1, 64, 1, 8192), (8, 8, 1, 4096), (32, 1, 1, 8192), (32, 16, 1, 8192)]


def small_rows(torch, tv, W) -> dict:
    """bf16-cache attention (d_c 512, d_r 64) at small R = H x q_len, the
    library's own kernel choice: us per call (HIP events around 50 calls) and
    the cache stream rate."""
    import numpy as np
    out = {}
    for B, H, q, P in SMALL_ROWS:
        rng = np.random.default_rng(0)
        kv = P + q
        gen = torch.Generator(device="cuda").manual_seed(0)
        ql = torch.randn(B, q, H, 512, device="cuda", generator=gen) * 0.5
        qr = torch.randn(B, q, H, 64, device="cuda", generator=gen) * 0.5
        ck = (torch.randn(B, kv, 512, device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
        kr = (torch.randn(B, kv, 64, device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
        par = torch.from_numpy(np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)).cuda()
        o = torch.empty_like(ql)
        ws = torch.empty(max(tv.workspace_size(B, H, q, P, 512, 64, tv.TV_BF16), 1), dtype=torch.uint8,
                         device="cuda")
        f = lambda: tv.verify_attn(ql, qr, ck, kr, par, P, 0.04, out=o, workspace=ws)
        for _ in range(20):
            f()
        us = _time_ms(torch, f, 50) * 1e3
        cache_bytes = B * kv * 576 * 2
        out[f"b{B}_h{H}_q{q}_p{P}"] = {"R": H * q, "us": round(us, 2),
                                      "cache_tbs": round(cache_bytes / (us * 1e-6) / 1e12, 3)}
    return out


def rope_back_to_back(torch, fn, n: int) -> float:
    """Mean ms per launch of n launches of fn captured in one graph."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def next_rows(torch, tv, W, inp, w, c_kv, k_rope, parent, with_oracle: bool) -> dict:
    """The steps around verify on the same batch: the target's greedy token per
    node over a K2-class vocabulary (fp32 logits), greedy tree accept,
    compaction of the accepted rows of the bf16 cache, and (before verify) the
    best-first tree builder on synthetic drafter proposals."""
    import numpy as np
    dev = c_kv.device
    x = W.make_accept_inputs(inp["parent"], W.SERVE_VOCAB, seed=1234)
    logits = torch.from_numpy(x["logits"]).to(dev)
    draft = torch.from_numpy(x["draft"]).to(dev)
    target = torch.empty(w.B, w.q_len, dtype=torch.int32, device=dev)
    ms_argmax = _time_ms(torch, lambda: tv.argmax_rows(logits, out=target), 20)
    path, n, bonus = tv.tree_accept(parent, draft, target)
    ms_accept = _time_ms(torch, lambda: tv.tree_accept(parent, draft, target), 50)
    c2, r2 = c_kv.clone(), k_rope.clone()
    ms_compact = _time_ms(torch, lambda: tv.kv_compact(c2, r2, path, n, w.prefix_len), 50)
    n_host = n.cpu().numpy()
    # The step before verify: best-first trees from synthetic drafter proposals.
    bx = W.make_build_inputs(w.B, W.BUILD_DEPTH, W.BUILD_TOPK, seed=99)
    b_lp = torch.from_numpy(bx["logp"]).to(dev)
    b_tok = torch.from_numpy(bx["cand_tok"]).to(dev)
    b_root = torch.from_numpy(bx["root_tok"]).to(dev)
    budget = w.q_len - 1
    ms_build = _time_ms(torch, lambda: tv.tree_build(b_lp, b_tok, b_root, budget), 50)
    logit_bytes = logits.numel() * 4
    moved_bytes = int(n_host.sum()) * 2 * (w.d_c + w.d_r) * 2
    out = {
        "workload": f"B={w.B} q_len={w.q_len} vocab={W.SERVE_VOCAB} fp32 logits; bf16 cache d_c={w.d_c} d_r={w.d_r}",
        "argmax_rows": {"ms": round(ms_argmax, 4), "bytes": logit_bytes,
                        "achieved_gbs": round(logit_bytes / (ms_argmax * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(logit_bytes / (ms_argmax * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "tree_accept": {"ms": round(ms_accept, 4), "accepted_mean": round(float(n_host.mean()), 3),
                        "bound": "launch latency (integer walk, one wave per tree)"},
        "kv_compact": {"ms": round(ms_compact, 4), "bytes_moved": moved_bytes,
                       "bound": "launch latency (a few hundred KB)"},
        "tree_build": {"ms": round(ms_build, 4), "budget": budget, "depth": W.BUILD_DEPTH, "topk": W.BUILD_TOPK,
                       "bound": "launch latency (one wave per request, budget dependent pops)"},
    }
    if with_oracle:
        from oracle import accept_oracle as A
        t0 = time.perf_counter()
        tg = A.greedy_tokens(x["logits"][:4])
        A.tree_accept(inp["parent"][:4], x["draft"][:4], tg)
        dt = (time.perf_counter() - t0) * w.B / 4
        out["cpu_oracle_ms"] = {"value": round(dt * 1e3, 1), "sample": "greedy tokens + accept on 4 of 32 trees, "
                                                                       "scaled x8"}
        from oracle import tree_build_oracle as T
        t0 = time.perf_counter()
        T.best_first_tree(bx["logp"], bx["cand_tok"], bx["root_tok"], budget)
        out["tree_build"]["cpu_oracle_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
    return out


def reference_gemm(torch, n: int = 8192, reps: int = 10) -> dict:
    """The vendor bf16 GEMM (torch.matmul, hipBLASLt) on N(0,1) operands, timed
    on the same box: what dense bf16 matrix work reaches here with random data
    (the part runs at its power limit, so this sits well below the datasheet
    peak).  Context for roofline.frac, not a competitor."""
    g = torch.Generator(device="cuda:0")
    g.manual_seed(3)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    ms = _time_ms(torch, lambda: torch.matmul(a, b, out=c), reps)
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"what": f"torch.matmul bf16 {n}x{n}x{n}, N(0,1) operands", "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAKS_TFLOPS["bf16"], 4)}


def cpu_baseline_fp32(w, inp) -> float:
    """The oracle as it stands on one fp32 configuration's whole call (inputs
    already rotated, as the GPU timing has them): median of 5, microseconds."""
    import numpy as np
    from oracle import tv_oracle as O
    args = (O.as_f64(inp["q_lat"], "f32"), O.as_f64(inp["q_rope"], "f32"), O.as_f64(inp["c_kv"], "f32"),
            O.as_f64(inp["k_rope"], "f32"), inp["parent"], w.prefix_len, w.sm_scale)
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        O.verify_attn(*args)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)) * 1e6


def fp32_configs(torch, tv, W, with_oracle: bool = False) -> dict:
    """The fp32-cache configurations: microseconds per verify_attn call
    (inputs already rotated; the fp32 matrix-core kernel at d_c 512 / d_r 64,
    the VALU kernel at 64 / 32), TFLOP/s against the fp32 peak (157.3 for
    both) and GB/s, from the algorithmic counts; with_oracle adds the float64
    oracle's time for the same call on the host (median of 5) and the ratio."""
    import numpy as np
    dev = "cuda:0"
    out = {}
    for name, w in W.WORKLOADS.items():
        if w.kv_dtype != "f32":
            continue
        inp = W.make_inputs(w)
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
             for k in ("q_lat", "q_rope", "c_kv", "k_rope", "parent")}
        o = torch.empty_like(t["q_lat"])
        ws_n = tv.workspace_size(w.B, w.H, w.q_len, w.prefix_len, w.d_c, w.d_r, tv.TV_F32)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        fn = lambda: tv.verify_attn(t["q_lat"], t["q_rope"], t["c_kv"], t["k_rope"], t["parent"], w.prefix_len,
                                    w.sm_scale, out=o, workspace=ws)
        for _ in range(20):
            fn()
        ms = _time_ms(torch, fn, 200)
        c = algorithmic_counts(w, inp["parent"])
        mfma = (w.d_c, w.d_r) == (512, 64)
        # The library's choice of form: 32-row workgroups when the batch has at
        # most 128 blocks of 64 rows.
        narrow = mfma and w.B * -(-(w.q_len * w.H) // 64) <= 128
        out[name] = {"us": round(ms * 1e3, 2), "tflops": round(c["flops"] / (ms * 1e-3) / 1e12, 2),
                     "frac_of_fp32_peak": round(c["flops"] / (ms * 1e-3) / 1e12 / PEAKS_TFLOPS["f32_mfma"], 4),
                     "kernel": ("attn_mfma_f32_narrow_kernel" if narrow else "attn_mfma_f32_kernel") if mfma
                     else "attn_valu_kernel",
                     "gbs": round(c["attn_bytes"] / (ms * 1e-3) / 1e9, 1)}
        if narrow:
            # the 64-row form on the same call, for comparison
            ws_w = tv.workspace_size(w.B, w.H, w.q_len, w.prefix_len, w.d_c, w.d_r, tv.TV_F32, tv.TV_ATTN_F32_WIDE)
            wsw = torch.empty(max(ws_w, 1), dtype=torch.uint8, device=dev)
            fw = lambda: tv.verify_attn_ex(t["q_lat"], t["q_rope"], t["c_kv"], t["k_rope"], t["parent"],
                                           w.prefix_len, w.sm_scale, tv.TV_ATTN_F32_WIDE, out=o, workspace=wsw)
            for _ in range(20):
                fw()
            ms_w = _time_ms(torch, fw, 200)
            out[name]["wide_form_us"] = round(ms_w * 1e3, 2)
        if with_oracle:
            cpu_us = cpu_baseline_fp32(w, inp)
            out[name]["cpu_oracle_us"] = round(cpu_us, 1)
            out[name]["gpu_over_oracle"] = round(cpu_us / (ms * 1e3), 1)
    return out


def verify_variants(torch, tv, W) -> dict:
    """The verify attention beyond the serving batch: a long prefix with one
    request, a ragged batch of mixed prefixes and tree sizes, a 256-node tree
    (synthetic bf16 caches, N(0,1) x 0.5), and 8 trees of the serving shape
    with an fp32 cache (N(0,1)); branching trees; flops counted on the
    visible (row, key) pairs."""
    import numpy as np
    dev = "cuda:0"
    H, d_c, d_r = 64, 512, 64
    sm = 1.0 / (d_c + d_r) ** 0.5
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rng = np.random.default_rng(7)

    def visible_pairs(parent_rows, P):
        depth = np.zeros(len(parent_rows), dtype=np.int64)
        for i in range(1, len(parent_rows)):
            depth[i] = depth[parent_rows[i]] + 1
        return int((P + depth + 1).sum())

    def cache(B, S):
        return ((torch.randn(B, S, d_c, device=dev, generator=g) * 0.5).to(torch.bfloat16),
                (torch.randn(B, S, d_r, device=dev, generator=g) * 0.5).to(torch.bfloat16))

    out = {}
    # One request, 200k-token prefix (kv split into pieces + merge).
    for name, B, q, P in (("long_prefix_b1_p200000_q33", 1, 33, 200000), ("big_tree_b4_p4096_q256", 4, 256, 4096)):
        q_lat = torch.randn(B, q, H, d_c, device=dev, generator=g) * 0.5
        q_rope = torch.randn(B, q, H, d_r, device=dev, generator=g) * 0.5
        c_kv, k_rope = cache(B, P + q)
        par = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
        parent = torch.from_numpy(par).to(dev)
        o = torch.empty_like(q_lat)
        ws = torch.empty(max(tv.workspace_size(B, H, q, P, d_c, d_r, tv.TV_BF16), 1), dtype=torch.uint8, device=dev)
        ms = _time_ms(torch, lambda: tv.verify_attn(q_lat, q_rope, c_kv, k_rope, parent, P, sm, out=o, workspace=ws),
                      20, warmup=5)
        flops = H * sum(visible_pairs(par[b], P) for b in range(B)) * (2 * (d_c + d_r) + 2 * d_c)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        del q_lat, q_rope, c_kv, k_rope, o, ws
    # Ragged: 32 requests, q_len in {9, 17, 33}, prefixes 2k-16k.
    q_lens = [int(x) for x in rng.choice([9, 17, 33], 32)]
    prefixes = [int(x) for x in rng.integers(2048, 16384, 32)]
    B, N, S = 32, sum(q_lens), max(p + q for p, q in zip(prefixes, q_lens))
    q_lat = torch.randn(N, H, d_c, device=dev, generator=g) * 0.5
    q_rope = torch.randn(N, H, d_r, device=dev, generator=g) * 0.5
    c_kv, k_rope = cache(B, S)
    pars = [W.tree_branch(q, rng).astype(np.int32) for q in q_lens]
    parent = torch.from_numpy(np.concatenate(pars)).to(dev)
    pl = torch.tensor(prefixes, dtype=torch.int32, device=dev)
    ql = torch.tensor(q_lens, dtype=torch.int32, device=dev)
    o = torch.empty_like(q_lat)
    ws = torch.empty(tv.load().tv_verify_attn_ragged_workspace_size(B, H, max(q_lens), S, d_c, d_r, tv.TV_BF16),
                     dtype=torch.uint8, device=dev)
    ms = _time_ms(torch, lambda: tv.verify_attn_ragged(q_lat, q_rope, c_kv, k_rope, parent, pl, ql, max(q_lens), sm,
                                                       out=o, workspace=ws), 20, warmup=5)
    flops = H * sum(visible_pairs(p_, P) for p_, P in zip(pars, prefixes)) * (2 * (d_c + d_r) + 2 * d_c)
    out["ragged_b32_q9to33_p2kto16k"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    del q_lat, q_rope, c_kv, k_rope, o, ws
    # The fp32 cache at the serving batch's per-tree shape (8 trees): the
    # fp32 matrix-core kernel's 64-row form with every CU busy, against the
    # fp32 peak.
    B, q, P = 8, 33, 8192
    q_lat = torch.randn(B, q, H, d_c, device=dev, generator=g)
    q_rope = torch.randn(B, q, H, d_r, device=dev, generator=g)
    c_kv = torch.randn(B, P + q, d_c, device=dev, generator=g)
    k_rope = torch.randn(B, P + q, d_r, device=dev, generator=g)
    par = np.stack([W.tree_branch(q, rng) for _ in range(B)]).astype(np.int32)
    parent = torch.from_numpy(par).to(dev)
    o = torch.empty_like(q_lat)
    ws = torch.empty(max(tv.workspace_size(B, H, q, P, d_c, d_r, tv.TV_F32), 1), dtype=torch.uint8, device=dev)
    ms = _time_ms(torch, lambda: tv.verify_attn(q_lat, q_rope, c_kv, k_rope, parent, P, sm, out=o, workspace=ws),
                  10, warmup=3)
    flops = H * sum(visible_pairs(par[b], P) for b in range(B)) * (2 * (d_c + d_r) + 2 * d_c)
    tf = flops / (ms * 1e-3) / 1e12
    out["fp32_b8_h64_p8192_q33"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                    "frac_of_fp32_peak": round(tf / PEAKS_TFLOPS["f32_mfma"], 4),
                                    "kernel": "attn_mfma_f32_kernel"}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-sample", type=int, default=1 << 30,
                    help="trees the CPU oracle times (default: the whole batch, one call; 0 = skip)")
    ap.add_argument("--no-next-rows", dest="next_rows", action="store_false",
                    help="skip timing the steps after verify (greedy tokens, tree accept, KV compaction)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (the reference launch that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    ap.add_argument("--small-rows", action="store_true",
                    help="only time the bf16-cache attention at small H x q_len (decode-like shapes, where the "
                         "products are far from dense), print one JSON line and exit")
    ap.add_argument("--fp32-configs", action="store_true",
                    help="only time the fp32-cache configurations (next_rows.fp32_configs), print them as one "
                         "JSON line and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the verify "
              f"step shards over batch entries with no exchange, so the one-GPU figure is one shard's "
              f"throughput.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        return copy_calibration(torch)

    from tree_verify_mla_tv_amd import tv
    from tree_verify_mla_tv_amd import workloads as W

    if args.fp32_configs:
        print(json.dumps({"fp32_configs": fp32_configs(torch, tv, W)}), flush=True)
        return 0
    if args.small_rows:
        print(json.dumps({"small_rows": small_rows(torch, tv, W)}), flush=True)
        return 0

    w = W.WORKLOADS[args.workload or W.SERVING]
    tv.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    inp = W.make_inputs(w)

    def cache(a):
        if w.kv_dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q_lat = torch.from_numpy(inp["q_lat"]).to(dev)
    q_rope = torch.from_numpy(inp["q_rope"]).to(dev)
    c_kv = cache(inp["c_kv"])
    k_rope = cache(inp["k_rope"])
    parent = torch.from_numpy(inp["parent"]).to(dev)
    P = w.prefix_len
    if P > 0:
        tv.rope_neox_strided(k_rope[:, :P, :], None, w.theta)  # cache fill, outside the timed region
    out = torch.empty_like(q_lat)
    dt_code = tv.TV_BF16 if w.kv_dtype == "bf16" else tv.TV_F32
    ws_bytes = tv.workspace_size(w.B, w.H, w.q_len, P, w.d_c, w.d_r, dt_code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(evr=None, ev0=None, ev1=None):
        if evr is not None:
            evr.record()
        tv.tree_rope(q_rope, k_rope, parent, P, w.theta)
        if ev0 is not None:
            ev0.record()
        tv.verify_attn(q_lat, q_rope, c_kv, k_rope, parent, P, w.sm_scale, out=out, workspace=ws)
        if ev1 is not None:
            ev1.record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for er, e0, e1 in evs:
        step(er, e0, e1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = float(np.mean([e0.elapsed_time(e1) for _, e0, e1 in evs]))
    rope_ms = float(np.mean([er.elapsed_time(e0) for er, e0, _ in evs]))

    counts = algorithmic_counts(w, inp["parent"])
    kern = KERNELS[w.kv_dtype]
    achieved_tflops = counts["flops"] / (attn_ms * 1e-3) / 1e12
    peak = PEAKS_TFLOPS[kern["peak"]]
    traffic = load_traffic(kern, w.name)
    value = 1e3 / ms_per_step
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kern["dtype"],
        "data": "synthetic (seeded N(0,1) inputs, random trees; no dataset or weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "prefix": P, "budget": w.q_len - 1,
                   "q_len": w.q_len, "kv_len": w.kv_len, "d_c": w.d_c, "d_r": w.d_r, "kv_cache": w.kv_dtype,
                   "tree": w.tree},
        "hbm_gbs": round(counts["step_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(counts["step_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": kern["name"],
            "bound": kern["bound"],
            "achieved": round(achieved_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved_tflops / peak, 4),
            "traffic": traffic,
            "avg_launch_ms": round(attn_ms, 5),
            "timed": "HIP events on the launch stream around each verify_attn call: the attention kernel and "
                     "its split-kv merge pass (about 9 us of the call), so the rate is slightly conservative",
            "algorithmic_flops": counts["flops"],
            "algorithmic_bytes": counts["attn_bytes"],
            "achieved_hbm_gbs": round(counts["attn_bytes"] / (attn_ms * 1e-3) / 1e9, 1),
        },
    }
    # The step's RoPE (the queries and the tree's own key rows), timed by HIP
    # events around each tree_rope call of the same timed steps.
    # Each call is also timed back to back: 50 launches captured in a HIP
    # graph (so host-side launch cost does not pace them), the graph replayed
    # between two events.  The in-step events above add the event packets and
    # a dispatch to a ~10 us kernel; this mean spreads them over 50 calls.  The
    # rotation is applied again each time (values stay finite; timing only).
    rope_b = rope_back_to_back(torch, lambda: tv.tree_rope(q_rope, k_rope, parent, P, w.theta), 50)
    rec["rope"] = {"kernel": "tree_rope_kernel", "ms": round(rope_b, 5), "bytes": counts["rope_bytes"],
                   "achieved_gbs": round(counts["rope_bytes"] / (rope_b * 1e-3) / 1e9, 1),
                   "frac_of_hbm_peak": round(counts["rope_bytes"] / (rope_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "timed": "HIP events around 50 back-to-back tv_tree_rope launches (per-launch mean)",
                   "in_step_ms": round(rope_ms, 5),
                   "in_step_timed": "HIP events around each tv_tree_rope call of the timed steps"}
    if kern.get("query_terms", 1) > 1:
        # The matrix work the scheme itself does per visible (row, key) pair:
        # the score product once per query term, the value product once.
        factor = (kern["query_terms"] * 2 * (w.d_c + w.d_r) + 2 * w.d_c) / (2 * (w.d_c + w.d_r) + 2 * w.d_c)
        rec["roofline"]["scheme_matrix_work"] = {
            "what": f"score product over {kern['query_terms']} bf16 query terms: matrix-core flops per algorithmic "
                    "flop (padding and masked keys not counted)",
            "factor": round(factor, 4),
            "tflops": round(achieved_tflops * factor, 1),
            "frac_of_peak": round(achieved_tflops * factor / peak, 4)}
    if w.kv_dtype == "bf16":
        rec["roofline"]["reference_gemm"] = reference_gemm(torch)
    if args.cpu_sample > 0:
        rec["cpu_baseline"] = cpu_baseline(inp, w, min(args.cpu_sample, w.B))
        rec["cpu_baseline"]["gpu_over_oracle"] = round(value / rec["cpu_baseline"]["value"], 1)
    if args.next_rows and w.kv_dtype == "bf16":
        rec["next_rows"] = next_rows(torch, tv, W, inp, w, c_kv, k_rope, parent, args.cpu_sample > 0)
        rec["next_rows"]["verify_variants"] = verify_variants(torch, tv, W)
        rec["next_rows"]["fp32_configs"] = fp32_configs(torch, tv, W, args.cpu_sample > 0)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
