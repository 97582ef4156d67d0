#!/usr/bin/env python3
"""Decode attention over a low-rank-compressed KV cache on one MI355X.

One step = one decode call (``lrkv_decode_attn``: projected-query scoring of the
codes, full-rank anchors, one softmax, rank-space value sums, one up-projection)
for a whole layer of the Llama-3.1-8B-shaped 32K-context workload (batch 4,
32 query / 8 KV heads, d = 128, r_k = 64, r_v = 32, first token + last 128 as
anchors, 32 context splits).  The cache is built on the GPU by the library's own
prefill compression from seeded synthetic keys and values, and is replicated so
that successive calls rotate over >= 1 GiB of cache (as the layers of a model
would) and read from HBM rather than the 256 MB last-level cache.

Prints one JSON line: tokens*heads/s of whole calls, the roofline of the
dominant kernel (its algorithmic bytes over its event-timed duration) and the
CPU oracle timed on a bounded sample of the same workload.

``--codes int8`` / ``--codes int4`` run the same workload with int8 or 4-bit
codes and per-token float32 scales (bf16 bases, anchors and queries) instead of
bf16 codes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DOMINANT_KERNEL = "k_partials_mfma (stage 1: code splits + anchors)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_mfma.hip", "decode_common.h", "mfma_util.h", "lrkv_internal.h"):
        with open(os.path.join(ROOT, "rank_kv_cache_lrkv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, n, bits=16, hg=1, resid=0, versions=1):
    """Bytes the method must move for one decode call of one layer, and the part
    the partials kernel moves (codes, anchors, U_K, q).  Quantised codes: r bytes
    (int8) or r / 2 bytes (4-bit) per code row plus its 4-byte scale.  Group-head
    latents (hg KV heads per code stream): one code row per group and token, bases
    of hg * 128 rows per group, anchors per KV head.  LowRAM values (resid = R >
    0): key codes only, R residual rows (256 bytes and a 4-byte slot) per 32-slot
    block, and the row's predictor (r_k x 128) in place of U_V.  Basis versions
    (codes made under several bases): every version's U_K and U_V rows."""
    import oracle
    s = 4 if w.dtype == "f32" else 2
    c = len(oracle.code_positions(n, w.window))
    a = len(oracle.anchor_positions(n, w.window))
    units = w.batch * w.n_kv_heads // hg
    if bits < 16:
        codes = units * c * ((w.rank_k + w.rank_v) * bits // 8 + 8)
    else:
        codes = units * c * (w.rank_k + w.rank_v) * s
    anchors = w.batch * w.n_kv_heads * a * 2 * 128 * s
    u_k = versions * w.n_kv_heads * 128 * w.rank_k * s
    u_v = versions * w.n_kv_heads * 128 * w.rank_v * s
    if resid:
        nblk = (c + 31) // 32
        codes = units * (c * w.rank_k * s + nblk * resid * (128 * s + 4))
        u_v = units * w.rank_k * 128 * s
    q = w.batch * w.n_q_heads * 128 * s
    out = w.batch * w.n_q_heads * 128 * 4
    return {"call": codes + anchors + u_k + u_v + q + out, "partials": codes + anchors + u_k + q,
            "codes": codes, "anchors": anchors}


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
    import numpy as np
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
    s = 2 if w.dtype == "bf16" else 4
    row = (2 * 128 * s + (w.rank_k + w.rank_v) * bits // 8 + 8) if bits < 16 else (2 * 128 + w.rank_k + w.rank_v) * s
    moved = w.batch * w.n_kv_heads * c * 2 * 128 * s + w.batch * (w.n_kv_heads // hg) * c * (row - 2 * 128 * s)
    if resid:  # keys and values in, key codes and the kept residual rows out (the fit reads both twice)
        moved = w.batch * w.n_kv_heads * (c * (2 * 128 * s + w.rank_k * s) + ((c + 31) // 32) * resid * (128 * s + 8))
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


def cpu_baseline(w, seconds):
    """The oracle as it stands, timed on this host's cores over a bounded sample
    of (batch row, KV head) units of the same workload at full context."""
    import numpy as np

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    n = w.n_ctx
    rk, rv = synth.ranks(w, 0)
    cpos, apos = oracle.code_positions(n, w.window), oracle.anchor_positions(n, w.window)
    g = w.group
    scale = oracle.default_scale()
    spent, done, units = 0.0, 0, []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            units.append((b, h))
    prepared = []
    for b, h in units:
        k = synth.unit_kv(w, 0, h, b, "k")[:n].astype(np.float64)
        v = synth.unit_kv(w, 0, h, b, "v")[:n].astype(np.float64)
        uk = synth.basis(w, 0, h, "k", int(rk[h])).astype(np.float64)
        uv = synth.basis(w, 0, h, "v", int(rv[h])).astype(np.float64)
        rnd = oracle.bf16_round if w.dtype == "bf16" else (lambda x: x.astype(np.float32).astype(np.float64))
        ck = rnd(oracle.oracle_compress(k[cpos], uk))
        cv = rnd(oracle.oracle_compress(v[cpos], uv))
        q = synth.queries(w, 0, 0, b)[h * g:(h + 1) * g].astype(np.float64)
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
            "sample": f"{done} unit decodes cycling over {len(prepared)} of the {len(units)} "
                      f"(batch row, KV head) units at full context n={n}, {g} query heads each; "
                      f"float64 NumPy oracle_decode_unit, {spent:.1f} s of decode time "
                      f"(code preparation untimed)"}


def traffic_from_profile(source_hash, codes="bf16", hg=1):
    """HBM traffic per launch of the dominant kernel, from the committed counter
    summary, if it was taken on the current kernel source."""
    name = "decode_partials_llama31_8b_32k" + ("" if codes == "bf16" else f"_{codes}") + \
        ("" if hg == 1 else f"_hg{hg}") + "_traffic.json"
    p = os.path.join(ROOT, "profiles", name)
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("source_hash") != source_hash:
        return None
    return d.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama31_8b_32k")
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before anything else, fill a buffer of this size and copy it once "
                         "(device to device): the reference dispatches that scale hardware "
                         "traffic counters in a profiled run")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step in this build; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from rank_kv_cache_lrkv_amd import binding as B

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
        w = w.scaled(n_layers=1, n_steps=0, mixed_ranks=False)
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
    nb = algorithmic_bytes(w, w.n_ctx, bits, hg, resid, nver)
    R = args.replicas or max(1, math.ceil((1 << 30) / nb["call"]))
    layers = [L0] + [replicate(L0, B) for _ in range(R - 1)]
    n = w.n_ctx
    # splits per code stream: the workload's count per KV head, times the group size
    # with head groups (so the grid keeps its size); the library's choice for the
    # LowRAM and pre-RoPE kernels (three workgroups per CU resident, not four)
    S = w.n_splits * hg if (w.n_splits and not resid and not rope_base) else B.lrkv_decode_auto_splits(L0, n)
    q = dev(np.stack([synth.queries(w, 0, 0, b) for b in range(w.batch)]))
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
    ws = B.workspace(L0, S)
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()

    def call(i):
        B.lrkv_decode_attn(layers[i % R], n, q, out, scale, S, ws, stream=stream)

    log(f"{R} cache replicas ({R * nb['call'] / 2**30:.2f} GiB), {S} splits; warmup {args.warmup}")
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite decode output"

    # timed region: whole calls, events on the stream the kernels run on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} calls: {ms_per_step * 1e3:.2f} us per call")

    # the dominant kernel alone: the same number of stage-1 launches back to back
    # (rotating over the replicas), events on their stream around the whole run
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        B.lrkv_decode_partials(layers[i % R], n, q, scale, S, ws, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    k_ms = ev0.elapsed_time(ev1) / args.steps
    log(f"stage 1 (dominant kernel): {k_ms * 1e3:.2f} us per launch")

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
        kernel = "k_partials_mfma, pre-RoPE key codes (keys reconstructed and rotated per block)"
    if nver > 1:
        kernel += f", codes under {nver} basis versions"
    k_bytes = nb["partials"]
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = None if (resid or rope_base or nver > 1) else traffic_from_profile(src_hash, args.codes, hg)
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
                     "us_per_launch": round(k_ms * 1e3, 3), "source_hash": src_hash},
        "call_hbm_gbps": round(nb["call"] / t_call / 1e9, 1),
        "call_alg_bytes": nb["call"],
        "compress": compress,
        "oja_update": oja,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
