#!/usr/bin/env python3
"""Decode attention over a low-rank-compressed KV cache on one MI355X.

One step = one decode call (``lrkv_decode_attn``: projected-query scoring of the
codes, full-rank anchors, one softmax, rank-space value sums, one up-projection)
for a whole layer.  The default workload is the Llama-3.1-8B-shaped 32K-context
layer (batch 4, 32 query / 8 KV heads, d = 128, r_k = 64, r_v = 32, first token
+ last 128 as anchors, 32 context splits).  ``--workload`` selects any of the
five workloads:

  tiny_f32            1 head, n 256, float32 storage
  qwen3_1p7b_4k       batch 8, 16/8 heads, n 4096, ranks 64/32, anchors 1 + 64
  llama31_8b_32k      (default) as above
  llama31_8b_hc_8k    batch 64, 32/8 heads, n 8192, ranks 32/16, anchors 1 + 32
  llama31_8b_32layer  32 layers of batch 4, 32/8 heads, n 32768, each layer with
                      its own mixed ranks (r_k in {32, 48, 64, 96}, r_v in
                      {16, 32} per KV head); prefill compression of every layer,
                      then decode steps, a step being, for each of the 32 layers,
                      the cache maintenance of the new token (``lrkv_append``)
                      and the layer's decode call

The cache is built on the GPU by the library's own prefill compression of seeded
keys and values.  Single-layer workloads are replicated so that successive calls
rotate over >= 1 GiB of cache (as the layers of a model would) and read from HBM
rather than the 256 MB last-level cache; the 32-layer cache is 5.6 GB already.

Timing.  Launches are enqueued by a Python loop whose per-call host cost can
exceed a short call's GPU time, so every timed loop starts behind a bounded spin
kernel that keeps the GPU busy while the host enqueues the whole loop: the events
then time the GPU's back-to-back execution of the calls, as a serving loop that
issues ahead (or a captured graph) would see it.  ``value`` comes from one event
pair around the loop; ``per_call_us`` from one event pair per call.

Prints one JSON line: tokens*heads/s of whole calls (whole steps for the
32-layer workload), the roofline of the dominant kernel (the stage-1 partials:
algorithmic bytes over its event-timed duration), the read-stream ceiling of the
same box for the same bytes, and the CPU oracle timed on a bounded sample.

``--codes int8`` / ``--codes int4`` run a single-layer workload with int8 or
4-bit codes and per-token float32 scales instead of bf16 codes; ``--head-group``,
``--lowram``, ``--rope-base`` and ``--versions`` select the other cache variants.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DOMINANT_KERNEL = "k_partials_mfma (stage 1: code splits + anchors)"
LAYER_WORKLOADS = ("tiny_f32", "qwen3_1p7b_4k", "llama31_8b_32k", "llama31_8b_hc_8k")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_mfma.hip", "decode_common.h", "mfma_util.h", "lrkv_internal.h"):
        with open(os.path.join(ROOT, "rank_kv_cache_lrkv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, n, bits=16, hg=1, resid=0, versions=1, ranks=None):
    """Bytes the method must move for one decode call of one layer, and the part
    the partials kernel moves (codes, anchors, U_K, q).  ``ranks`` = (r_k[h],
    r_v[h]) per code stream (default: the workload's uniform ranks).  Quantised
    codes: r bytes (int8) or r / 2 bytes (4-bit) per code row plus its 4-byte
    scale.  Group-head latents (hg KV heads per code stream): one code row per
    group and token, bases of hg * 128 rows per group, anchors per KV head.
    LowRAM values (resid = R > 0): key codes only, R residual rows (256 bytes and
    a 4-byte slot) per 32-slot block, and the row's predictor (r_k x 128) in place
    of U_V.  Basis versions (codes made under several bases): every version's U_K
    and U_V rows."""
    import oracle
    s = 4 if w.dtype == "f32" else 2
    c = len(oracle.code_positions(n, w.window))
    a = len(oracle.anchor_positions(n, w.window))
    n_lat = w.n_kv_heads // hg
    if ranks is None:
        rks, rvs = [w.rank_k] * n_lat, [w.rank_v] * n_lat
    else:
        rks, rvs = [int(x) for x in ranks[0]], [int(x) for x in ranks[1]]
    rk_sum, rv_sum = sum(rks), sum(rvs)
    if bits < 16:
        codes = w.batch * c * ((rk_sum + rv_sum) * bits // 8 + 8 * n_lat)
    else:
        codes = w.batch * c * (rk_sum + rv_sum) * s
    anchors = w.batch * w.n_kv_heads * a * 2 * 128 * s
    u_k = versions * hg * 128 * rk_sum * s
    u_v = versions * hg * 128 * rv_sum * s
    if resid:
        nblk = (c + 31) // 32
        codes = w.batch * (c * rk_sum * s + n_lat * nblk * resid * (128 * s + 4))
        u_v = w.batch * rk_sum * 128 * s
    q = w.batch * w.n_q_heads * 128 * s
    out = w.batch * w.n_q_heads * 128 * 4
    return {"call": codes + anchors + u_k + u_v + q + out, "partials": codes + anchors + u_k + q,
            "codes": codes, "anchors": anchors}


def compress_bytes(w, c, ranks, bits=16, hg=1, resid=0):
    """Bytes one prefill compression of keys and values moves: every compressed
    token's key and value rows read (2 x 128 elements per KV head) and its code
    rows written (plus the scales of quantised codes); LowRAM layers write key
    codes and the kept residual rows instead of value codes."""
    s = 2 if w.dtype == "bf16" else 4
    rks, rvs = [int(x) for x in ranks[0]], [int(x) for x in ranks[1]]
    rows_in = w.batch * w.n_kv_heads * c * 2 * 128 * s
    if resid:
        nblk = (c + 31) // 32
        return rows_in + w.batch * (c * sum(rks) * s + len(rks) * nblk * resid * (128 * s + 8))
    if bits < 16:
        return rows_in + w.batch * c * ((sum(rks) + sum(rvs)) * bits // 8 + 8 * len(rks))
    return rows_in + w.batch * c * (sum(rks) + sum(rvs)) * s


# ---------------------------------------------------------------------------
# host, GPU and library context recorded with every line
# ---------------------------------------------------------------------------

def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        import numpy as np
        from threadpoolctl import threadpool_info
        np.ones((64, 64)) @ np.ones((64, 64))
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            b = libs[0]
            blas = f"{b.get('internal_api')} {b.get('version')} ({b.get('num_threads')} threads, " \
                   f"{b.get('architecture')})"
    except Exception as e:  # pragma: no cover - informational only
        blas = f"unknown ({e.__class__.__name__})"
    return {"model": model, "blas": blas, "affinity_cpus": len(os.sched_getaffinity(0))}


def gpu_state():
    """Clocks and power of GPU 0 as rocm-smi reports them right after the timed
    work (informational; None if the tool is unavailable).  Skipped under the
    profiler: its preloaded library would follow the tool's launcher into the
    child process."""
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return {"skipped": "run under the profiler"}
    try:
        r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=30)
        d = json.loads(r.stdout)
        card = next(iter(d.values()))
        keep = {k: v for k, v in card.items() if "clk" in k.lower() or "power" in k.lower()}
        return keep or None
    except Exception as e:
        return {"error": f"rocm-smi: {e.__class__.__name__}"}


class Timer:
    """Event timing of loops of launches on one stream, each loop started behind
    a bounded spin kernel so the GPU runs the enqueued launches back to back."""

    def __init__(self, stream):
        import torch

        from rank_kv_cache_lrkv_amd import measure
        self.torch, self.measure = torch, measure
        self.stream = stream
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.host_us = {}

    def _spin(self, key, n):
        us = min(400_000.0, 200.0 + 1.5 * n * self.host_us[key])
        self.measure.spin_us(us, self.sink, self.stream.cuda_stream)

    def calibrate(self, key, fn, n=8):
        """Host time to enqueue one fn(i) (the GPU drained before and after)."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        dt = time.perf_counter() - t0
        torch.cuda.synchronize()
        self.host_us[key] = max(1.0, dt / n * 1e6)
        return self.host_us[key]

    def total_ms(self, key, fn, n):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        self._spin(key, n)
        e0.record(self.stream)
        for i in range(n):
            fn(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def per_call_ms(self, key, fn, n):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        self._spin(key, n)
        for i in range(n):
            ev[i][0].record(self.stream)
            fn(i)
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]


def percentiles_us(ms):
    import numpy as np
    a = np.asarray(ms) * 1e3
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "mean": round(float(a.mean()), 3), "n": len(a)}


def stream_ceiling(timer, nbytes, launches=12):
    """The fastest plain read of ``nbytes`` bytes from HBM on this machine: the
    read-stream probe over a sweep of launch shapes, each reading one of several
    buffers in turn (>= 1 GiB in all, so the reads miss the last-level cache);
    the per-launch mean of the best shape."""
    torch = timer.torch
    from rank_kv_cache_lrkv_amd import measure
    if nbytes < (16 << 20):  # a read this small is launch-bound: no ceiling to state
        return None
    nbytes = (nbytes + 4095) // 4096 * 4096
    nbuf = min(64, max(2, math.ceil((1 << 30) / nbytes) + 1))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    s = timer.stream.cuda_stream
    best, sweep = None, []
    for grid in (512, 768, 1024, 2048, 4096, 8192):
        for unroll in (2, 4, 8):
            for nt in (False, True):
                fn = lambda i: measure.read(bufs[i % nbuf], nbytes, sink, grid, unroll, nt, s)
                key = ("read", grid, unroll, nt)
                timer.calibrate(key, fn, 2)
                fn(0)
                ms = timer.total_ms(key, fn, launches) / launches
                gbps = nbytes / (ms * 1e-3) / 1e9
                sweep.append([grid, unroll, int(nt), round(gbps, 1)])
                if best is None or gbps > best["gbps"]:
                    best = {"gbps": round(gbps, 1), "us_per_launch": round(ms * 1e3, 3), "bytes": nbytes,
                            "grid": grid, "block": 256, "unroll": unroll, "nontemporal": nt}
    del bufs
    best["sweep"] = sweep
    return best


# ---------------------------------------------------------------------------
# single-layer workloads
# ---------------------------------------------------------------------------

def rotate_rows(x, positions, base):
    """Rotate-half RoPE of rows x (..., t, 128) at positions (t,) on the GPU in
    float64 (input preparation for caches whose key codes are pre-RoPE: the
    anchors the caller stores are post-RoPE keys)."""
    import torch
    half = 64
    theta = torch.tensor([float(base) ** (-2.0 * i / 128) for i in range(half)], dtype=torch.float64,
                         device=x.device)
    ang = positions.to(torch.float64)[:, None] * theta[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    xf = x.to(torch.float64)
    a, b = xf[..., :half], xf[..., half:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1).to(x.dtype)


def build_cache(w, B, dev, bits=16, hg=1, resid=0, rope_base=0.0):
    """Prefill on the GPU: compress tokens 1..n-W-1, store token 0 and the window."""
    import torch

    import synth
    from rank_kv_cache_lrkv_amd import layout

    rk, rv = synth.ranks(w, 0)
    if hg > 1:  # one basis pair per group of hg KV heads (uniform ranks)
        n_lat = w.n_kv_heads // hg
        rk, rv = rk[:n_lat], rv[:n_lat]
        bases = layout.pack_bases([synth.group_basis(w, 0, g, hg, "k", int(rk[g])) for g in range(n_lat)],
                                  [synth.group_basis(w, 0, g, hg, "v", int(rv[g])) for g in range(n_lat)])
    else:
        bases = layout.pack_bases([synth.basis(w, 0, h, "k", int(rk[h])) for h in range(w.n_kv_heads)],
                                  [synth.basis(w, 0, h, "v", int(rv[h])) for h in range(w.n_kv_heads)])
    n = w.n_ctx
    c = max(0, n - 1 - w.window)
    dtype = {8: B.LRKV_BF16_Q8, 4: B.LRKV_BF16_Q4}.get(bits, B.LRKV_BF16 if w.dtype == "bf16" else B.LRKV_F32)
    L = B.Layer.allocate(dtype=dtype, batch=w.batch,
                         n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, window=w.window,
                         cap=layout.round_cap(c), rank_k=rk, rank_v=rv, bases=dev(bases), head_group=hg,
                         lowram_resid=resid, rope_base=rope_base)
    td = L.torch_dtype
    K = torch.empty((w.batch, w.n_kv_heads, n, 128), dtype=td, device="cuda")
    V = torch.empty_like(K)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            K[b, h] = dev(synth.unit_kv(w, 0, h, b, "k")[:n])
            V[b, h] = dev(synth.unit_kv(w, 0, h, b, "v")[:n])
    # prefill compression (LowRAM: keys, then the predictor fit and residuals), timed once warm
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    fit_ws = torch.empty(max(1, B.lrkv_lowram_workspace_size(L)), dtype=torch.uint8, device="cuda") if resid else None
    for rep in range(2):
        ev[0].record()
        B.lrkv_compress(L, 0, K[:, :, 1:], c, 0)
        if resid:
            B.lrkv_lowram_fit(L, V[:, :, 1:], c, ws=fit_ws)
        else:
            B.lrkv_compress(L, 1, V[:, :, 1:], c, 0)
        ev[1].record()
    KA = K
    if rope_base:  # the codes took the pre-RoPE keys; anchors hold the keys rotated to their positions
        KA = rotate_rows(K, torch.arange(n, device="cuda"), rope_base)
    B.lrkv_store_anchors(L, KA[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, KA[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    del KA
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    moved = compress_bytes(w, c, (rk, rv), bits, hg, resid)
    compress = {"ms": round(ms, 4), "tokens": c, "alg_bytes": moved,
                "gbps": round(moved / (ms * 1e-3) / 1e9, 1)}
    oja = None
    if bits == 16 and w.dtype == "bf16" and hg == 1 and not resid and not rope_base:
        # one Oja step of the key bases over the whole prompt (OjaKV's prefill
        # adaptation), version 0 -> 1 of a two-version copy of the bases
        Lo = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads,
                              n_kv_heads=w.n_kv_heads, window=w.window, cap=32, rank_k=rk, rank_v=rv,
                              n_versions=2)
        Lo.bases[:L.bases.numel()] = L.bases
        ws = torch.empty(B.lrkv_oja_workspace_size(Lo), dtype=torch.uint8, device="cuda")
        for rep in range(2):
            ev[0].record()
            B.lrkv_oja_update(Lo, 0, K[:, :, 1:], n - 1, 0.5, 0, 1, ws=ws)
            ev[1].record()
        torch.cuda.synchronize()
        oms = ev[0].elapsed_time(ev[1])
        obytes = w.batch * w.n_kv_heads * (n - 1) * 128 * 2
        oja = {"ms": round(oms, 4), "rows": w.batch * (n - 1), "alg_bytes": obytes,
               "gbps": round(obytes / (oms * 1e-3) / 1e9, 1)}
        del Lo, ws
    del K, V
    return L, compress, oja


def with_versions(L, B, nver, n):
    """The same cache read as codes made under nver basis versions: bases holds nver
    copies of the layer's bases, and row b's code slots are cut into nver runs of
    whole 32-slot blocks (version v from slot 32 * floor(v * blocks / nver))."""
    import torch
    c = max(0, n - 1 - L.window)
    nblk = (c + 31) // 32
    starts = [32 * (v * nblk // nver) for v in range(nver)]
    vs = torch.tensor([starts] * L.batch, dtype=torch.int32, device="cuda")
    return B.Layer(L.dtype, L.batch, L.n_q_heads, L.n_kv_heads, L.window, L.cap, L.rank_k, L.rank_v,
                   torch.cat([L.bases] * nver), L.codes_k, L.codes_v, L.anchor_k, L.anchor_v,
                   L.scales_k, L.scales_v, n_versions=nver, version_start=vs)


def replicate(L, B):
    sc = lambda t: None if t is None else t.clone()
    return B.Layer(L.dtype, L.batch, L.n_q_heads, L.n_kv_heads, L.window, L.cap, L.rank_k, L.rank_v,
                   L.bases.clone(), L.codes_k.clone(), sc(L.codes_v), L.anchor_k.clone(),
                   L.anchor_v.clone(), sc(L.scales_k), sc(L.scales_v), n_versions=L.n_versions,
                   version_start=sc(L.version_start), head_group=L.head_group,
                   value_mode=L.value_mode, resid_per_block=L.resid_per_block, predictor=sc(L.predictor),
                   resid=sc(L.resid), resid_slot=sc(L.resid_slot), resid_norm=sc(L.resid_norm),
                   rope_base=L.rope_base)


def cpu_baseline(w, seconds, layer=0, n=None):
    """The oracle as it stands, timed on this host's cores over a bounded sample
    of (batch row, KV head) units of the same workload at full context."""
    import numpy as np

    import oracle
    import synth

    info = cpu_info()
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    n = w.n_ctx if n is None else n
    rk, rv = synth.ranks(w, layer)
    cpos, apos = oracle.code_positions(n, w.window), oracle.anchor_positions(n, w.window)
    g = w.group
    scale = oracle.default_scale()
    spent, done, units = 0.0, 0, []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            units.append((b, h))
    prepared = []
    for b, h in units[:: max(1, len(units) // 8)]:
        k = synth.unit_kv(w, layer, h, b, "k")[:n].astype(np.float64)
        v = synth.unit_kv(w, layer, h, b, "v")[:n].astype(np.float64)
        uk = synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64)
        uv = synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64)
        rnd = oracle.bf16_round if w.dtype == "bf16" else (lambda x: x.astype(np.float32).astype(np.float64))
        ck = rnd(oracle.oracle_compress(k[cpos], uk))
        cv = rnd(oracle.oracle_compress(v[cpos], uv))
        q = synth.queries(w, layer, 0, b)[h * g:(h + 1) * g].astype(np.float64)
        prepared.append((q, uk, uv, ck, cv, k[apos], v[apos]))
        if len(prepared) == 8:
            break
    # cycle over the prepared units until the time budget is spent
    while spent < seconds:
        for args in prepared:
            t0 = time.perf_counter()
            oracle.oracle_decode_unit(*args, scale)
            spent += time.perf_counter() - t0
            done += 1
    value = done * g * n / spent
    return {"value": value, "unit": "tokens*heads/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": info["model"], "blas": info["blas"],
            "sample": f"{done} unit decodes cycling over {len(prepared)} of the {len(units)} "
                      f"(batch row, KV head) units of layer {layer} at context n={n}, {g} query heads each; "
                      f"float64 NumPy oracle_decode_unit, {spent:.1f} s of decode time "
                      f"(code preparation untimed)"}


def traffic_from_profile(source_hash, workload, codes="bf16", hg=1):
    """HBM traffic per launch of the dominant kernel, from the committed counter
    summary, if it was taken on the current kernel source."""
    name = f"decode_partials_{workload}" + ("" if codes == "bf16" else f"_{codes}") + \
        ("" if hg == 1 else f"_hg{hg}") + "_traffic.json"
    p = os.path.join(ROOT, "profiles", name)
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("source_hash") != source_hash:
        return None
    return d.get("bytes_per_launch")


def run_layer(args, w):
    import numpy as np
    import torch

    import synth
    from rank_kv_cache_lrkv_amd import binding as B

    td = torch.float32 if w.dtype == "f32" else torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(td).cuda()
    log(f"workload {w.name}: batch {w.batch}, heads {w.n_q_heads}/{w.n_kv_heads}, n {w.n_ctx}, "
        f"ranks {w.rank_k}/{w.rank_v}, window {w.window}")
    t0 = time.time()
    bits = {"bf16": 16, "int8": 8, "int4": 4}[args.codes]
    assert not (bits < 16 and w.dtype != "bf16"), "quantised codes are for the bf16 workloads"
    hg = args.head_group
    assert hg == 1 or (w.dtype == "bf16" and w.n_kv_heads % hg == 0), "head groups need bf16 storage"
    resid = args.lowram
    assert not resid or (bits == 16 and hg == 1 and w.dtype == "bf16"), "LowRAM values: bf16 codes, no head groups"
    if resid:
        w = w.scaled(v_from_k=0.8)
    rope_base = args.rope_base
    assert not rope_base or (bits == 16 and hg == 1 and not resid and w.dtype == "bf16"), \
        "pre-RoPE key codes: bf16 codes, no head groups, value codes"
    nver = args.versions
    assert nver == 1 or (bits == 16 and hg == 1 and not resid and not rope_base and w.dtype == "bf16"), \
        "basis versions: bf16 codes, no head groups, value codes, keys after RoPE"
    L0, compress, oja = build_cache(w, B, dev, bits, hg, resid, rope_base)
    if nver > 1:
        L0 = with_versions(L0, B, nver, w.n_ctx)
    log(f"cache built and compressed on the GPU in {time.time() - t0:.1f} s "
        f"(compress {compress['ms']:.3f} ms, {compress['gbps']} GB/s)")
    if oja:
        log(f"Oja step over the prompt's keys: {oja['ms']:.3f} ms ({oja['gbps']} GB/s of rows)")
    n_lat = w.n_kv_heads // hg
    nb = algorithmic_bytes(w, w.n_ctx, bits, hg, resid, nver,
                           ranks=(L0.rank_k[:n_lat], L0.rank_v[:n_lat]))
    R = args.replicas or max(1, math.ceil((1 << 30) / nb["call"]))
    layers = [L0] + [replicate(L0, B) for _ in range(R - 1)]
    n = w.n_ctx
    # splits per code stream: the workload's count per KV head, times the group size
    # with head groups (so the grid keeps its size); otherwise the library's choice
    S = w.n_splits * hg if (w.n_splits and not resid and not rope_base) else B.lrkv_decode_auto_splits(L0, n)
    S = args.splits or S
    q = dev(np.stack([synth.queries(w, 0, 0, b) for b in range(w.batch)]))
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
    ws = B.workspace(L0, S)
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()
    timer = Timer(stream)

    def call(i):
        B.lrkv_decode_attn(layers[i % R], n, q, out, scale, S, ws, stream=stream)

    def partials(i):
        B.lrkv_decode_partials(layers[i % R], n, q, scale, S, ws, stream=stream)

    log(f"{R} cache replicas ({R * nb['call'] / 2**30:.2f} GiB), {S} splits; warmup {args.warmup}")
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite decode output"
    host_us = timer.calibrate("call", call)
    timer.calibrate("partials", partials)

    # timed region: whole calls back to back, one event pair around the loop
    ms_per_step = timer.total_ms("call", call, args.steps) / args.steps
    per_call = percentiles_us(timer.per_call_ms("call", call, args.steps))
    log(f"timed {args.steps} calls: {ms_per_step * 1e3:.2f} us per call "
        f"(per call: median {per_call['median']} us, p10 {per_call['p10']}, p90 {per_call['p90']}; "
        f"host enqueue {host_us:.1f} us per call)")
    # the dominant kernel alone: the same number of stage-1 launches back to back
    k_ms = timer.total_ms("partials", partials, args.steps) / args.steps
    per_launch = percentiles_us(timer.per_call_ms("partials", partials, args.steps))
    log(f"stage 1 (dominant kernel): {k_ms * 1e3:.2f} us per launch (median {per_launch['median']} us)")
    gstate = gpu_state()

    ceiling = None if args.no_stream_ceiling else stream_ceiling(timer, nb["partials"])
    if ceiling:
        log(f"read-stream ceiling for {ceiling['bytes']} bytes: {ceiling['gbps']} GB/s "
            f"({ceiling['us_per_launch']} us per launch)")

    t_call = ms_per_step * 1e-3
    value = w.batch * w.n_q_heads * n / t_call
    kernel = DOMINANT_KERNEL if w.dtype == "bf16" else "k_partials_generic (stage 1)"
    if bits < 16:
        kernel = f"k_partials_mfma, {args.codes} codes (stage 1: code splits + anchors)"
    if hg > 1:
        kernel += f", {hg} KV heads per code stream"
    if resid:
        kernel = f"k_partials_mfma, LowRAM values (key codes + {resid} residual rows per block)"
    if rope_base:
        kernel = "k_partials_rope, pre-RoPE key codes (keys reconstructed and rotated per block)"
    if nver > 1:
        kernel += f", codes under {nver} basis versions"
    k_bytes = nb["partials"]
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = None if (resid or rope_base or nver > 1) else traffic_from_profile(src_hash, w.name, args.codes, hg)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.3e} tokens*heads/s on {cpu['cores']} threads")

    line = {
        "metric": "compressed-KV decode attention tokens*heads/s (+ achieved HBM GB/s vs peak)",
        "value": value,
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded decaying-spectrum keys/values, calibration-SVD bases)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": 128, "n_ctx": n, "rank_k": w.rank_k,
                   "rank_v": w.rank_v, "window": w.window, "n_splits": S, "cache_replicas": R,
                   "codes": args.codes, "head_group": hg, "lowram_resid": resid, "rope_base": rope_base,
                   "basis_versions": nver},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": k_bytes,
                     "us_per_launch": round(k_ms * 1e3, 3), "per_launch_us": per_launch,
                     "source_hash": src_hash,
                     "stream_ceiling_gbps": ceiling["gbps"] if ceiling else None,
                     "frac_of_stream_ceiling": round(achieved / ceiling["gbps"], 4) if ceiling else None},
        "per_call_us": per_call,
        "host_enqueue_us_per_call": round(host_us, 2),
        "call_hbm_gbps": round(nb["call"] / t_call / 1e9, 1),
        "call_alg_bytes": nb["call"],
        "call_frac_of_peak": round(nb["call"] / t_call / 1e9 / HBM_PEAK_GBS, 4),
        "stream_ceiling": ceiling,
        "gpu_state": gstate,
        "compress": compress,
        "oja_update": oja,
        "cpu_baseline": cpu,
    }
    return line


# ---------------------------------------------------------------------------
# the 32-layer workload: prefill of every layer, then decode steps
# ---------------------------------------------------------------------------

def run_32layer(args, w):
    import numpy as np
    import torch

    import synth
    from rank_kv_cache_lrkv_amd import binding as B, layout

    n0, W = w.n_ctx, w.window
    c0 = n0 - 1 - W
    cap = layout.round_cap(c0 + w.n_steps)
    nl = w.n_layers
    warm = min(args.warmup, w.n_steps - 1)
    steps = min(args.steps, w.n_steps - warm)
    log(f"workload {w.name}: {nl} layers, batch {w.batch}, heads {w.n_q_heads}/{w.n_kv_heads}, "
        f"prefill n {n0}, window {W}, mixed ranks; {warm} warmup + {steps} timed decode steps")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    t0 = time.time()
    layers, new_k, new_v, ranks = [], [], [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    comp_ms, comp_bytes = [], []
    for l in range(nl):
        rk, rv = synth.ranks(w, l)
        ranks.append((rk, rv))
        bases = layout.pack_bases([synth.basis(w, l, h, "k", int(rk[h])) for h in range(w.n_kv_heads)],
                                  [synth.basis(w, l, h, "v", int(rv[h])) for h in range(w.n_kv_heads)])
        L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                             window=W, cap=cap, rank_k=rk, rank_v=rv, bases=bf(bases))
        K = synth.layer_kv_device(w, l, "k")
        V = synth.layer_kv_device(w, l, "v")
        ev[0].record()
        B.lrkv_compress(L, 0, K[:, :, 1:], c0, 0)
        B.lrkv_compress(L, 1, V[:, :, 1:], c0, 0)
        ev[1].record()
        B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
        B.lrkv_store_anchors(L, K[:, :, n0 - W:n0], V[:, :, n0 - W:n0], n0 - W, W)
        # the decode steps' new tokens, [step][batch][kv head][128]
        new_k.append(K[:, :, n0:n0 + w.n_steps].permute(2, 0, 1, 3).contiguous())
        new_v.append(V[:, :, n0:n0 + w.n_steps].permute(2, 0, 1, 3).contiguous())
        torch.cuda.synchronize()
        comp_ms.append(ev[0].elapsed_time(ev[1]))
        comp_bytes.append(compress_bytes(w, c0, (rk, rv)))
        del K, V
        layers.append(L)
    log(f"{nl} layers generated and compressed in {time.time() - t0:.1f} s "
        f"(compress per layer: mean {np.mean(comp_ms):.3f} ms)")
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()
    timer = Timer(stream)
    # splits per layer: the library's choice at the last step's context
    S = [B.lrkv_decode_auto_splits(L, n0 + w.n_steps) for L in layers]
    ws = torch.empty(max(B.lrkv_decode_workspace_size(L, s) for L, s in zip(layers, S)), dtype=torch.uint8,
                     device="cuda")
    qs = [[bf(np.stack([synth.queries(w, l, t + 1, b) for b in range(w.batch)])) for t in range(w.n_steps)]
          for l in range(nl)]
    outs = torch.empty((nl, w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")

    def step(t):
        pos = n0 + t
        for l, L in enumerate(layers):
            B.lrkv_append(L, new_k[l][t], new_v[l][t], pos, stream=stream)
            B.lrkv_decode_attn(L, pos + 1, qs[l][t], outs[l], scale, S[l], ws, stream=stream)

    for t in range(warm):
        step(t)
    torch.cuda.synchronize()
    assert torch.isfinite(outs).all(), "non-finite decode output"
    # host cost of a step, measured without side effects: decode calls only
    dec = lambda i: B.lrkv_decode_attn(layers[i % nl], n0 + warm, qs[i % nl][warm - 1], outs[i % nl],
                                       scale, S[i % nl], ws, stream=stream)
    host_us = timer.calibrate("call", dec, 2 * nl)
    timer.host_us["step"] = 2.2 * nl * host_us
    ms_total = timer.total_ms("step", lambda i: step(warm + i), steps)
    ms_per_step = ms_total / steps
    n_mean = n0 + warm + (steps + 1) / 2.0
    log(f"timed {steps} steps: {ms_per_step:.3f} ms per step ({nl} appends + {nl} decode calls)")
    torch.cuda.synchronize()
    assert torch.isfinite(outs).all(), "non-finite decode output"

    # at the final context (cache no longer changing): per-layer decode calls and
    # stage-1 launches, rotating over the layers
    n_end = n0 + w.n_steps
    q_end = [qs[l][w.n_steps - 1] for l in range(nl)]
    call = lambda i: B.lrkv_decode_attn(layers[i % nl], n_end, q_end[i % nl], outs[i % nl], scale, S[i % nl], ws,
                                        stream=stream)
    part = lambda i: B.lrkv_decode_partials(layers[i % nl], n_end, q_end[i % nl], scale, S[i % nl], ws,
                                            stream=stream)
    reps = 4 * nl
    timer.calibrate("call", call, nl)
    timer.calibrate("partials", part, nl)
    call_ms = timer.total_ms("call", call, reps) / reps
    per_call = percentiles_us(timer.per_call_ms("call", call, reps))
    part_each = timer.per_call_ms("partials", part, reps)
    part_ms = timer.total_ms("partials", part, reps) / reps
    gstate = gpu_state()
    lb = [algorithmic_bytes(w, n_end, ranks=ranks[l]) for l in range(nl)]
    part_bytes = sum(b["partials"] for b in lb) / nl
    call_bytes = sum(b["call"] for b in lb) / nl
    achieved = part_bytes / (part_ms * 1e-3) / 1e9
    # per layer: bytes over the mean of its own stage-1 launches
    per_layer = []
    for l in range(nl):
        mine = [part_each[i] for i in range(reps) if i % nl == l]
        us = float(np.mean(mine)) * 1e3
        per_layer.append({"layer": l, "us": round(us, 2), "gbps": round(lb[l]["partials"] / (us * 1e-6) / 1e9, 1),
                          "splits": S[l], "rank_k": ranks[l][0].tolist(), "rank_v": ranks[l][1].tolist()})
    log(f"per-layer decode call {call_ms * 1e3:.2f} us (median {per_call['median']}), stage 1 "
        f"{part_ms * 1e3:.2f} us per launch: {achieved:.0f} GB/s on {part_bytes / 1e6:.1f} MB")
    ceiling = None if args.no_stream_ceiling else stream_ceiling(timer, int(part_bytes))
    value = sum(w.batch * w.n_q_heads * (n0 + warm + i + 1) * nl for i in range(steps)) / (ms_total * 1e-3)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, args.cpu_seconds, layer=0, n=n0 + 1)
        cpu["sample"] += " (one layer-step of the 32-layer workload; the metric counts every layer)"
        log(f"oracle: {cpu['value']:.3e} tokens*heads/s on {cpu['cores']} threads")
    src_hash = kernel_source_hash()
    return {
        "metric": "compressed-KV decode attention tokens*heads/s (+ achieved HBM GB/s vs peak)",
        "value": value,
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded decaying-spectrum keys/values drawn on the GPU, calibration-SVD bases)",
        "config": {"workload": w.name, "layers": nl, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": 128, "n_ctx_prefill": n0,
                   "n_ctx_mean_timed": n_mean, "window": W, "ranks": "mixed per (layer, KV head)",
                   "step": f"{nl} x (lrkv_append + lrkv_decode_attn)", "n_splits": "library choice per layer"},
        "roofline": {"bound": "hbm", "kernel": "k_partials_mfma (stage 1), mixed ranks, 32 layers",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": round(part_bytes), "us_per_launch": round(part_ms * 1e3, 3),
                     "source_hash": src_hash,
                     "stream_ceiling_gbps": ceiling["gbps"] if ceiling else None,
                     "frac_of_stream_ceiling": round(achieved / ceiling["gbps"], 4) if ceiling else None},
        "per_call_us": per_call,
        "per_layer_stage1": per_layer,
        "host_enqueue_us_per_call": round(host_us, 2),
        "call_us_mean": round(call_ms * 1e3, 3),
        "call_alg_bytes_mean": round(call_bytes),
        "call_hbm_gbps": round(call_bytes / (call_ms * 1e-3) / 1e9, 1),
        "call_frac_of_peak": round(call_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stream_ceiling": ceiling,
        "gpu_state": gstate,
        "compress": {"ms_per_layer_mean": round(float(np.mean(comp_ms)), 4), "tokens": c0,
                     "alg_bytes_per_layer_mean": round(float(np.mean(comp_bytes))),
                     "gbps": round(float(np.sum(comp_bytes)) / (float(np.sum(comp_ms)) * 1e-3) / 1e9, 1)},
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama31_8b_32k",
                    choices=LAYER_WORKLOADS + ("llama31_8b_32layer",))
    ap.add_argument("--codes", choices=("bf16", "int8", "int4"), default="bf16",
                    help="code storage (bf16 workloads): bf16, or int8 / int4 with per-token scales")
    ap.add_argument("--head-group", type=int, default=1,
                    help="KV heads sharing one code stream (group-head latents; bf16 workloads)")
    ap.add_argument("--lowram", type=int, default=0, metavar="R",
                    help="LowRAM values: predicted from the key codes, R residual rows per 32-slot block "
                         "(bf16 workloads; values partly predictable from keys)")
    ap.add_argument("--rope-base", type=float, default=0.0,
                    help="> 1: key codes of pre-RoPE keys, reconstructed and rotated in the decode "
                         "(rotate-half RoPE with this base; bf16 codes)")
    ap.add_argument("--versions", type=int, default=1, metavar="V",
                    help="codes made under V basis versions (OjaKV), the row's code slots cut into V "
                         "equal runs of whole blocks; every version holds the same basis, so the output "
                         "is that of one version (bf16 codes)")
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas rotated (0: >= 1 GiB)")
    ap.add_argument("--splits", type=int, default=0,
                    help="context splits per code stream (single-layer workloads; 0: the workload's "
                         "count, else the library's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before anything else, fill a buffer of this size and copy it once "
                         "(device to device): the reference dispatches that scale hardware "
                         "traffic counters in a profiled run")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step in this build; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibration_copy_mib > 0:
        nbytes = args.calibration_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)  # writes nbytes
        dst = torch.empty_like(src)
        dst.copy_(src)                                                       # reads and writes nbytes
        torch.cuda.synchronize()
        log(f"calibration: fill then copy of {nbytes} bytes")
        del src, dst
    w = synth.WORKLOADS[args.workload]
    if w.n_layers != 1:
        assert args.codes == "bf16" and args.head_group == 1 and not args.lowram and not args.rope_base \
            and args.versions == 1, "the 32-layer workload runs bf16 codes of the plain method"
        line = run_32layer(args, w)
    else:
        line = run_layer(args, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
