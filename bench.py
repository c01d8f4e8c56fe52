"""Benchmark of the FAD-KV encoder hot path on one MI355X.

One step = one batch of key/value head vectors through every stage: screening + Top-n pool
(fadkv_screen), support/ridge/residual (fadkv_select_support) and the fixed-size adaptation
commit (fadkv_adapt).  Inputs are synthetic and already resident in HBM when timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3b_decode]

Prints one JSON line (rank 0).  `value` is encoded vectors per second over the K timed steps
(wall clock, synchronised on both sides).  Each stage is also bracketed by HIP events on the
stream the library launches on; the dominant kernel's average duration gives `roofline`.
By default the step rotates over enough independent dictionary sets to exceed the 256 MB
Infinity Cache, so the dictionaries stream from HBM (`--warm` keeps one set).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "encoded KV vectors/sec (decode step & prefill) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6   # dense bf16/fp16 (256 CU x 2.4 GHz x 4096 flop/clk)
ALU_PEAK_TFLOPS = 157.3          # 256 CU x 64 lanes x 2.4 GHz x 4 flop (v_dot2_f32_{f16,bf16})
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3b_decode")
    ap.add_argument("--select", default="gm", choices=["gm", "pl"])
    ap.add_argument("--warm", action="store_true", help="one dictionary set (cache-resident)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--path", default="encode", choices=["encode", "attend"],
                    help="encode: the encoder hot path (default); attend: decode attention of "
                         "one layer over the sparse codes")
    ap.add_argument("--tokens", type=int, default=2048, help="cached tokens per row (--path attend)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB three times (a plain "
                         "device copy of known size, for scaling memory-traffic counters)")
    return ap.parse_args()


def measured_traffic(workload, select, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("record: "):
                rec = json.loads(line[len("record: "):])
    if rec is None or rec.get("select") != select or kernel not in rec:
        return None
    csrc = os.path.join(ROOT, "sparse_dictionary_coding_amd", "csrc")
    src = {"select_kernel": "select.hip", "score_topn_kernel": "score_topn.hip"}[kernel]
    h = hashlib.sha256()
    for name in (src, "common.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec[kernel]["sources_sha256_16"]:
        return None
    return rec[kernel]["bytes"]


def cpu_baseline(w, select, seconds):
    """Time the CPU oracle, as it stands, on whole dictionaries of the same workload until
    about `seconds` of work: encode every row of a dictionary, then commit its adaptation."""
    import numpy as np
    import torch

    import oracle
    from sparse_dictionary_coding_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    p = oracle.OracleParams(n=w.n, s=w.s, select=select,
                            ridge_abs=float(np.float32(1e-4)), ridge_rel=float(np.float32(0.2)))
    gen = synth.SyntheticKV(w, device="cpu", num_dicts=min(w.num_dicts, 64))
    A = synth.to_f64(gen.atoms())
    rows_per_dict = min(w.M, 256)
    X = synth.to_f64(gen.batch(torch.from_numpy(A).to(synth.TORCH_DTYPES[w.dtype]),
                               M=rows_per_dict))
    done = 0
    dicts = 0
    t0 = time.perf_counter()
    for t in range(gen.T):
        codes = oracle.encode(A[t:t + 1], X[t:t + 1], p, dict_ids=[t])
        oracle.adapt(A[t:t + 1], np.zeros((1, w.N), np.int64), X[t:t + 1], codes, p, w.dtype)
        done += rows_per_dict
        dicts += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "vectors/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{dicts} of {w.num_dicts} dictionaries x {rows_per_dict} vectors "
                      f"(encode + adapt, NumPy fp64), {dt:.1f} s"}


def bench_attend(args):
    """Decode attention of one layer over its sparse-coded cache: R = KV heads x sequences rows
    of `--tokens` tokens, each coded by this library's encoder from synthetic K/V vectors, and G
    query heads per KV head.  Prints one JSON line; `value` is query-token pairs per second."""
    import numpy as np
    import torch

    from sparse_dictionary_coding_amd import fadkv, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    heads, seqs, G = 8, w.M // 8, 3        # Llama-3.2-3B: 8 KV heads, 3 query heads per KV head
    R, T, d, N, s = heads * seqs, args.tokens, w.d, w.N, w.s
    gen = synth.SyntheticKV(w, device=dev, num_dicts=2)
    atoms = gen.atoms()                    # dictionary 0 = keys, 1 = values of the layer
    p = fadkv.Params(n=w.n, s=s)
    X = gen.batch(atoms, M=R * T)
    codes = fadkv.fadkv_encode(atoms, X, p)
    del X
    ki = codes.idx[0].reshape(R, T, s).contiguous()
    kc = codes.coef[0].reshape(R, T, s).contiguous()
    vi = codes.idx[1].reshape(R, T, s).contiguous()
    vc = codes.coef[1].reshape(R, T, s).contiguous()
    lens = torch.full((R,), T, dtype=torch.int32, device=dev)
    q = torch.randn(R, G, d, device=dev).to(atoms.dtype)
    out = torch.empty(R, G, d, dtype=torch.float32, device=dev)
    ws = torch.empty(fadkv.fadkv_attend_workspace_bytes(atoms, R, G), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(d))
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fadkv.fadkv_attend(atoms, 0, ki, kc, vi, vc, lens, q, scale, out=out, workspace=ws,
                           stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fadkv.fadkv_attend(atoms, 0, ki, kc, vi, vc, lens, q, scale, out=out, workspace=ws,
                           stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    esize = atoms.element_size()
    code_bytes = 2 * R * T * s * 8
    alg_bytes = code_bytes + 2 * N * d * esize + R * G * d * (esize + 4)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    # context: dense attention over the rebuilt cache (what the codes replace)
    K = fadkv.fadkv_reconstruct(atoms[0:1], ki.view(1, R * T, s), kc.view(1, R * T, s)).view(R, T, d)
    V = fadkv.fadkv_reconstruct(atoms[1:2], vi.view(1, R * T, s), vc.view(1, R * T, s)).view(R, T, d)
    for _ in range(3):
        torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)
    b.record(stream)
    torch.cuda.synchronize()
    dense_ms = a.elapsed_time(b) / args.steps
    res = {
        "metric": "decode attention over sparse-coded KV: query-token pairs/s",
        "value": R * G * T * args.steps / wall, "unit": "query-token pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name} attention, one layer", "rows": R, "kv_heads": heads,
                   "sequences": seqs, "query_heads_per_kv_head": G, "tokens": T, "N": N, "s": s,
                   "d": d},
        "roofline": {"kernel": "fadkv_attend (3 kernels)", "bound": "hbm", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None},
        "attend_ms": ms, "algorithmic_bytes": alg_bytes, "code_bytes": code_bytes,
        "dense_sdpa_ms": dense_ms, "dense_kv_bytes": 2 * R * T * d * esize,
    }
    if not args.no_cpu_baseline:
        from oracle import attend_oracle
        A = atoms.double().cpu().numpy()
        kin, kcn, vin, vcn = (t.cpu().numpy() for t in (ki, kc, vi, vc))
        qn = q.double().cpu().numpy()
        t1 = time.perf_counter()
        rows = 0
        while time.perf_counter() - t1 < args.cpu_seconds and rows < R:
            attend_oracle.attend_row(A[0], A[1], kin[rows], kcn[rows], vin[rows], vcn[rows],
                                     qn[rows], scale)
            rows += 1
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": rows * G * T / dt, "unit": "query-token pairs/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{rows} of {R} rows x {G} queries x {T} tokens "
                                         f"(NumPy fp64, Python loops), {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(dictionaries shard by layer with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.path == "attend":
        bench_attend(args)
        return

    import torch

    from sparse_dictionary_coding_amd import fadkv, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    p = fadkv.Params(n=w.n, s=w.s, select=args.select)
    T, M, N, d = w.num_dicts, w.M, w.N, w.d
    esize = 2 if w.dtype != "f32" else 4
    dict_bytes = T * N * d * esize
    R = 1 if args.warm else max(1, -(-(MALL_BYTES + (MALL_BYTES >> 2)) // dict_bytes))
    R = min(R, 8)

    gen = synth.SyntheticKV(w, device=dev)
    base_atoms = gen.atoms()
    sets = [base_atoms.clone() for _ in range(R)]
    usages = [torch.zeros(T, N, dtype=torch.int32, device=dev) for _ in range(R)]
    n_batches = min(args.steps + args.warmup, 16 if M * T <= 65536 else 1)
    batches = [gen.batch(base_atoms, step=i) for i in range(n_batches)]
    pool = fadkv.Pool.empty(T, M, w.n, dev)
    codes = fadkv.Codes.empty(T, M, w.s, dev)
    replaced = torch.empty(T, M, dtype=torch.int32, device=dev)
    ws = fadkv.make_workspace(base_atoms, p, M)
    stream = torch.cuda.current_stream()

    def step(k, ev=None):
        A, U, X = sets[k % R], usages[k % R], batches[k % n_batches]
        if ev is not None:
            ev[0].record(stream)
        fadkv.fadkv_screen(A, X, p, out=pool, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fadkv.fadkv_select_support(A, X, p, pool, out=codes, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        fadkv.fadkv_adapt(A, U, X, codes, p, replaced=replaced, workspace=ws, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = [0.0, 0.0, 0.0]
    for e in evs:
        for i in range(3):
            stage_ms[i] += e[i].elapsed_time(e[i + 1])
    stage_ms = [x / args.steps for x in stage_ms]
    G = T * M
    vec_per_step = G
    value = vec_per_step * args.steps / wall

    # algorithmic work per launch
    screen_flops = 2.0 * N * d * G
    screen_bytes = dict_bytes + G * d * esize + G * w.n * 6 + G
    sel_cols = (w.s - 1) if args.select == "gm" else 0
    sel_flops = 2.0 * G * (sel_cols * w.n * d + w.s * w.s * d / 2 + w.s * d)
    adapt_bytes = G * (w.s * 8 + 5) + 2 * T * N * 4
    kernels = {
        "screen_topn": {"ms": stage_ms[0], "flops": screen_flops, "bytes": screen_bytes},
        "select_support": {"ms": stage_ms[1], "flops": sel_flops},
        "adapt": {"ms": stage_ms[2], "bytes": adapt_bytes},
    }
    dominant = max(("screen_topn", "select_support"), key=lambda k: kernels[k]["ms"])
    if dominant == "screen_topn":
        ach = screen_flops / (stage_ms[0] * 1e-3) / 1e12
        roof = {"kernel": "score_topn_kernel", "bound": "mfma", "achieved": ach,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                "traffic": measured_traffic(w.name, args.select, "score_topn_kernel")}
    else:
        ach = sel_flops / (stage_ms[1] * 1e-3) / 1e12
        roof = {"kernel": "select_kernel", "bound": "alu", "achieved": ach,
                "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / ALU_PEAK_TFLOPS,
                "traffic": measured_traffic(w.name, args.select, "select_kernel")}
    # the screening kernel against HBM as well (the decode-step figure of merit)
    screen_gbs = screen_bytes / (stage_ms[0] * 1e-3) / 1e9
    trig = int((codes.flags & fadkv.FLAG_TRIGGER).ne(0).sum().item())
    rep = int((replaced >= 0).sum().item())

    out = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_dicts": T, "vectors_per_dict": M, "N": N, "n": w.n,
                   "s": w.s, "d": d, "select": args.select,
                   "dictionary_sets": R, "cache": "warm" if R == 1 else
                   f"cold: {R} rotating dictionary sets ({R * dict_bytes / 2**20:.0f} MiB)"},
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "screen_hbm": {"achieved": screen_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": screen_gbs / HBM_PEAK_GBS},
        "last_step": {"triggers": trig, "replaced": rep},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.select, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
