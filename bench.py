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
    ap.add_argument("--eager", action="store_true",
                    help="time decode-sized steps as eager launches instead of replaying one "
                         "HIP graph per step (per-kernel times always come from an eager pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 3B prefill measurement added to the default decode line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--path", default="encode", choices=["encode", "attend", "growth", "omp"],
                    help="encode: the encoder hot path (default); attend: decode attention of "
                         "one layer over the sparse codes; growth: a long run committed both "
                         "fixed-size and append-only, with the dictionary-size trace; omp: "
                         "coding cost of GM and PL relative to the full-dictionary greedy "
                         "yardstick, and the pool recall of the yardstick's atoms")
    ap.add_argument("--growth-steps", type=int, default=0,
                    help="decode steps of the long run (--path growth; default: the workload's)")
    ap.add_argument("--trace-out", default="", help="per-step trace as JSON (--path growth)")
    ap.add_argument("--tau-c", type=int, default=64,
                    help="usage threshold below which an atom is inactive (--path growth).  The "
                         "synthetic prefill uses every atom a few times, so with the library's "
                         "default of 1 no atom is inactive afterwards; 64 leaves about 12%% of "
                         "them inactive")
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
    src = {"select_kernel": ("select.hip",), "score_topn_kernel": ("score_topn.hip", "tiles.h")}[kernel]
    h = hashlib.sha256()
    for name in (*src, "common.h"):
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
    def run(budget):
        done = 0
        dicts = 0
        t0 = time.perf_counter()
        for t in range(gen.T):
            codes = oracle.encode(A[t:t + 1], X[t:t + 1], p, dict_ids=[t])
            oracle.adapt(A[t:t + 1], np.zeros((1, w.N), np.int64), X[t:t + 1], codes, p, w.dtype)
            done += rows_per_dict
            dicts += 1
            if time.perf_counter() - t0 >= budget:
                break
        return done, dicts, time.perf_counter() - t0

    done, dicts, dt = run(seconds)
    res = {"value": done / dt, "unit": "vectors/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{dicts} of {w.num_dicts} dictionaries x {rows_per_dict} vectors "
                     f"(encode + adapt, NumPy fp64), {dt:.1f} s"}
    try:   # the same oracle on one thread, on a quarter of the time budget
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, n1, t1 = run(seconds / 4)
        res["single_thread"] = {"value": d1 / t1, "unit": "vectors/s", "cores": 1,
                                "sample": f"{n1} dictionaries x {rows_per_dict} vectors, {t1:.1f} s"}
    except ImportError:
        pass
    return res


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


def bench_growth(args):
    """The long run (prefill, then sequential decode steps whose drifted vectors move linearly
    over the run) committed two ways from identical inputs: fixed-size adaptation (fadkv_adapt:
    N never changes, inactive atoms are overwritten) and append-only growth (fadkv_adapt_append:
    every triggering row adds an atom).  Each mode encodes against its own dictionary.  The
    append-only dictionary is kept in a buffer re-sized every RELAYOUT steps to its current
    size plus the most it can grow before the next re-size, so its encode cost follows its size
    (the zero slots past n_atoms score 0 and are never selected).

    Prints one JSON line: `value` is the fixed-size run's encoded vectors per second of GPU time
    (encode + commit, HIP events; input generation and re-sizing are outside), and `trace` the
    dictionary size, per-step time and code quality of both modes at evenly spaced steps."""
    import torch

    from sparse_dictionary_coding_amd import fadkv, synth

    RELAYOUT = 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload if synth.WORKLOADS[args.workload].steps > 1 else "qwen4b_long_decode"
    wd = synth.WORKLOADS[name]
    wp = synth.WORKLOADS.get(name.replace("_decode", "_prefill"))
    steps = args.growth_steps or wd.steps
    every = max(1, steps // 16)
    gd = synth.SyntheticKV(wd, device=dev)
    A0 = gd.atoms()
    T, N, d = A0.shape
    p = fadkv.Params(n=wd.n, s=wd.s, tau_c=args.tau_c)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def code_stats(codes, rep):
        f = codes.flags
        return torch.stack([(f & fadkv.FLAG_TRIGGER).ne(0).sum().float(),
                            rep.ge(0).sum().float(),
                            (f & fadkv.FLAG_EXHAUSTED).ne(0).sum().float(),
                            codes.relerr.mean()])

    def clone_codes(c):
        return fadkv.Codes(c.idx.clone(), c.coef.clone(), c.relerr.clone(), c.flags.clone())

    # ---- prefill: one encode, committed both ways ----------------------------------------
    A_fix = A0.clone()
    U_fix = torch.zeros(T, N, dtype=torch.int32, device=dev)
    prefill = {"vectors": 0, "ms": 0.0}
    cap = N + RELAYOUT * wd.M
    if wp is not None:
        gp = synth.SyntheticKV(wp, device=dev)
        assert torch.equal(gp.atoms(), A0), "prefill and decode draw the same dictionaries"
        Xp = gp.batch(A0)
        e = [ev() for _ in range(3)]
        e[0].record(stream)
        cp = fadkv.fadkv_encode(A0, Xp, p, stream=stream)
        ca = clone_codes(cp)
        e[1].record(stream)
        rp = fadkv.fadkv_adapt(A_fix, U_fix, Xp, cp, p, stream=stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        trig_max = int((ca.flags & fadkv.FLAG_TRIGGER).ne(0).sum(1).max().item())
        cap = N + trig_max + RELAYOUT * wd.M
        prefill = {"vectors": T * wp.M, "ms": e[0].elapsed_time(e[2]),
                   "encode_ms": e[0].elapsed_time(e[1]),
                   "triggers": int((cp.flags & fadkv.FLAG_TRIGGER).ne(0).sum().item()),
                   "replaced_fixed": int(rp.ge(0).sum().item())}
    A_app = torch.zeros(T, cap, d, dtype=A0.dtype, device=dev)
    A_app[:, :N] = A0
    U_app = torch.zeros(T, cap, dtype=torch.int32, device=dev)
    n_app = torch.full((T,), N, dtype=torch.int32, device=dev)
    if wp is not None:
        fadkv.fadkv_adapt_append(A_app, U_app, Xp, ca, p, n_app, stream=stream)
        torch.cuda.synchronize()
        prefill["inactive_after_prefill_fixed"] = float((U_fix < p.tau_c).sum(1).float().mean())
        prefill["n_atoms_after_prefill_append"] = float(n_app.float().mean())
        del Xp, cp, ca, rp
        torch.cuda.empty_cache()

    # ---- decode steps ---------------------------------------------------------------------
    M = wd.M
    cf, cA = fadkv.Codes.empty(T, M, wd.s, dev), fadkv.Codes.empty(T, M, wd.s, dev)
    rf = torch.empty(T, M, dtype=torch.int32, device=dev)
    ra = torch.empty(T, M, dtype=torch.int32, device=dev)
    ws_f = fadkv.make_workspace(A_fix, p, M)
    ws_a = fadkv.make_workspace(A_app, p, M)
    st_f = torch.zeros(steps, 4, device=dev)
    st_a = torch.zeros(steps, 4, device=dev)
    n_hist = torch.zeros(steps, T, dtype=torch.int32, device=dev)
    caps = []
    evs = [[ev() for _ in range(4)] for _ in range(steps)]
    inactive = {}
    t_wall = time.perf_counter()
    for k in range(steps):
        X = gd.batch(A0, step=k)
        if k % RELAYOUT == 0:
            need = int(n_app.max().item()) + RELAYOUT * M
            need = min(65535, -(-need // 32) * 32)
            if need != A_app.shape[1]:
                keep = min(need, A_app.shape[1])
                A2 = torch.zeros(T, need, d, dtype=A0.dtype, device=dev)
                A2[:, :keep] = A_app[:, :keep]
                U2 = torch.zeros(T, need, dtype=torch.int32, device=dev)
                U2[:, :keep] = U_app[:, :keep]
                A_app, U_app = A2, U2
                ws_a = fadkv.make_workspace(A_app, p, M)
        caps.append(A_app.shape[1])
        e = evs[k]
        e[0].record(stream)
        fadkv.fadkv_encode(A_fix, X, p, out=cf, workspace=ws_f, stream=stream)
        fadkv.fadkv_adapt(A_fix, U_fix, X, cf, p, replaced=rf, workspace=ws_f, stream=stream)
        e[1].record(stream)
        e[2].record(stream)
        fadkv.fadkv_encode(A_app, X, p, out=cA, workspace=ws_a, stream=stream)
        fadkv.fadkv_adapt_append(A_app, U_app, X, cA, p, n_app, replaced=ra, workspace=ws_a,
                                 stream=stream)
        e[3].record(stream)
        st_f[k] = code_stats(cf, rf)
        st_a[k] = code_stats(cA, ra)
        n_hist[k] = n_app
        if (k + 1) % every == 0 or k + 1 == steps:
            inactive[k] = (U_fix < p.tau_c).sum(1).float().mean()
        if (k + 1) % 64 == 0:
            print(f"[growth] step {k + 1}/{steps}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    assert A_fix.shape == (T, N, d)
    ms_f = [e[0].elapsed_time(e[1]) for e in evs]
    ms_a = [e[2].elapsed_time(e[3]) for e in evs]
    st_f, st_a, n_hist = st_f.cpu().tolist(), st_a.cpu().tolist(), n_hist.cpu()
    rows = T * M
    trace = []
    for k in sorted(set(list(range(every - 1, steps, every)) + [steps - 1])):
        lo = max(0, k + 1 - every)
        win = range(lo, k + 1)

        def avg(st, j):
            return sum(st[i][j] for i in win) / len(win)

        trace.append({
            "step": k + 1,
            "fixed": {"N": N, "inactive": round(float(inactive[k]), 1),
                      "ms": round(sum(ms_f[i] for i in win) / len(win), 4),
                      "trigger_frac": round(avg(st_f, 0) / rows, 4),
                      "replaced_per_step": round(avg(st_f, 1), 1),
                      "exhausted_frac": round(avg(st_f, 2) / rows, 4),
                      "relerr_mean": round(avg(st_f, 3), 4)},
            "append": {"n_atoms_mean": round(float(n_hist[k].float().mean()), 1),
                       "n_atoms_max": int(n_hist[k].max()), "buffer_N": caps[k],
                       "ms": round(sum(ms_a[i] for i in win) / len(win), 4),
                       "trigger_frac": round(avg(st_a, 0) / rows, 4),
                       "appended_per_step": round(avg(st_a, 1), 1),
                       "exhausted_frac": round(avg(st_a, 2) / rows, 4),
                       "relerr_mean": round(avg(st_a, 3), 4)},
        })
    esize = A0.element_size()
    gpu_ms_fixed = prefill["ms"] + sum(ms_f)
    vecs = prefill["vectors"] + steps * rows
    final_n = n_hist[steps - 1].float()
    res = {
        "metric": "long run: encoded KV vectors/s, fixed-size vs append-only dictionary",
        "value": vecs / (gpu_ms_fixed * 1e-3), "unit": "vectors/s", "n_gpus": 1,
        "steps": steps, "warmup": 0, "ms_per_step": sum(ms_f) / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wd.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wp.name if wp else ''} + {wd.name}", "num_dicts": T, "N": N,
                   "n": wd.n, "s": wd.s, "d": d, "decode_vectors_per_dict": M,
                   "prefill_vectors_per_dict": wp.M if wp else 0, "tau_c": p.tau_c,
                   "timing": "HIP events around encode + commit; generation outside"},
        "prefill": prefill,
        "fixed": {"N_final": N, "dictionary_MiB": T * N * d * esize / 2**20,
                  "decode_ms_total": sum(ms_f), "decode_vectors_per_s": steps * rows / (sum(ms_f) * 1e-3)},
        "append": {"n_atoms_final_mean": float(final_n.mean()),
                   "n_atoms_final_max": int(final_n.max()),
                   "dictionary_MiB": float(final_n.sum()) * d * esize / 2**20,
                   "decode_ms_total": sum(ms_a),
                   "decode_vectors_per_s": steps * rows / (sum(ms_a) * 1e-3)},
        "wall_s": t_wall,
        "trace": trace,
    }
    if args.trace_out:
        with open(args.trace_out, "w") as f:
            json.dump({"ms_fixed": ms_f, "ms_append": ms_a, "stats_fixed": st_f,
                       "stats_append": st_a, "n_atoms_mean": n_hist.float().mean(1).tolist(),
                       "buffer_N": caps}, f)
    print(json.dumps(res), flush=True)


def bench_omp(args):
    """Table 4's Cost column measured: the time of the screening encoder (GM, PL) relative to
    the full-dictionary greedy yardstick on the same step, plus Fig. 1b's pool recall (share of
    the yardstick's atoms inside the Top-n pool, over every vector of the step, for several n).
    Same cold-dictionary protocol as the main path.  Prints one JSON line whose `value` is the
    GM/yardstick time ratio (lower is better)."""
    import numpy as np
    import torch

    from sparse_dictionary_coding_amd import fadkv, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    T, M, N, d = w.num_dicts, w.M, w.N, w.d
    esize = 2 if w.dtype != "f32" else 4
    dict_bytes = T * N * d * esize
    R = 1 if args.warm else min(8, max(1, -(-(MALL_BYTES + (MALL_BYTES >> 2)) // dict_bytes)))
    gen = synth.SyntheticKV(w, device=dev)
    base = gen.atoms()
    sets = [base.clone() for _ in range(R)]
    X = gen.batch(base)
    pg, pp = fadkv.Params(n=w.n, s=w.s, select="gm"), fadkv.Params(n=w.n, s=w.s, select="pl")
    ws = fadkv.make_workspace(base, pg, M)
    ws_omp = torch.empty(fadkv.fadkv_omp_workspace_bytes(base, pg, M), dtype=torch.uint8,
                         device=dev)
    cg, cp, co = (fadkv.Codes.empty(T, M, w.s, dev) for _ in range(3))
    stream = torch.cuda.current_stream()
    runs = {
        "gm": lambda A: fadkv.fadkv_encode(A, X, pg, out=cg, workspace=ws, stream=stream),
        "pl": lambda A: fadkv.fadkv_encode(A, X, pp, out=cp, workspace=ws, stream=stream),
        "omp": lambda A: fadkv.fadkv_encode_omp(A, X, pg, out=co, workspace=ws_omp, stream=stream),
    }
    ms = {}
    for name, fn in runs.items():
        for k in range(args.warmup):
            fn(sets[k % R])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(ev):
            a.record(stream)
            fn(sets[(args.warmup + k) % R])
            b.record(stream)
        torch.cuda.synchronize()
        ms[name] = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    G = T * M
    # pool recall of the yardstick's atoms, over every vector of the step
    oi = co.idx.to(torch.int64)
    recall = {}
    for n in sorted({32, 64, 128, w.n, min(2 * w.n, 512)}):
        if n < w.s or n > min(N, 512):
            continue
        pool = fadkv.fadkv_screen(base, X, fadkv.Params(n=n, s=w.s))
        P = pool.atom_indices()
        hit = torch.zeros((), dtype=torch.int64, device=dev)
        for t0 in range(0, T, 8):
            sl = slice(t0, t0 + 8)
            hit += ((oi[sl, :, :, None] == P[sl, :, None, :]).any(-1) & (oi[sl] >= 0)).sum()
        recall[n] = float(hit) / float((oi >= 0).sum())
    same_support = float((torch.sort(cg.idx, -1).values == torch.sort(co.idx, -1).values)
                         .all(-1).float().mean())
    ratio_gm, ratio_pl = ms["gm"] / ms["omp"], ms["pl"] / ms["omp"]
    flops = 2.0 * N * d * w.s * G        # s correlation passes over the whole dictionary
    ach = flops / (ms["omp"] * 1e-3) / 1e12
    res = {
        "metric": "sparse-coding cost relative to the full-dictionary greedy (Table 4 Cost)",
        "value": ratio_gm, "unit": "GM time / full-dictionary time", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms["gm"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": ratio_gm / 0.19,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_dicts": T, "vectors_per_dict": M, "N": N, "n": w.n,
                   "s": w.s, "d": d, "dictionary_sets": R},
        "ms": {k: round(v, 5) for k, v in ms.items()},
        "cost_ratio": {"gm": ratio_gm, "pl": ratio_pl, "pages_gm": 0.19, "pages_pl": 0.13},
        "pool_recall": recall,
        "gm_equals_full_support_frac": same_support,
        "mean_relerr": {"gm": float(cg.relerr.nan_to_num().mean()),
                        "pl": float(cp.relerr.nan_to_num().mean()),
                        "omp": float(co.relerr.nan_to_num().mean())},
        "roofline": {"kernel": "fadkv_encode_omp (all launches)", "bound": "mfma",
                     "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        A = synth.to_f64(base[:1])
        Xs = synth.to_f64(X[:1])
        op = oracle.OracleParams(n=w.n, s=w.s, select="omp",
                                 ridge_abs=float(np.float32(1e-4)), ridge_rel=float(np.float32(0.2)))
        t1 = time.perf_counter()
        rows = 0
        while time.perf_counter() - t1 < args.cpu_seconds and rows < M:
            oracle.encode_vector(A[0], Xs[0, rows], op, op.delta(0))
            rows += 1
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": rows / dt, "unit": "vectors/s (full-dictionary greedy)",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{rows} vectors of dictionary 0 (NumPy fp64), {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def measure_encode(args, name, steps, warmup):
    """Time `steps` encode + commit steps of workload `name` (after `warmup` untimed ones) and
    return (workload, result dict) as printed by the default path."""
    import torch

    from sparse_dictionary_coding_amd import fadkv, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[name]
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
    n_batches = min(steps + warmup, 16 if M * T <= 65536 else 1)
    batches = [gen.batch(base_atoms, step=i) for i in range(n_batches)]
    pool = fadkv.Pool.empty(T, M, w.n, dev)
    codes = fadkv.Codes.empty(T, M, w.s, dev)
    replaced = torch.empty(T, M, dtype=torch.int32, device=dev)
    ws = fadkv.make_workspace(base_atoms, p, M)
    stream = torch.cuda.current_stream()

    def step(k, ev=None, strm=None):
        st = stream if strm is None else strm
        A, U, X = sets[k % R], usages[k % R], batches[k % n_batches]
        if ev is not None:
            ev[0].record(st)
        fadkv.fadkv_screen(A, X, p, out=pool, stream=st)
        if ev is not None:
            ev[1].record(st)
        fadkv.fadkv_select_support(A, X, p, pool, out=codes, stream=st)
        if ev is not None:
            ev[2].record(st)
        fadkv.fadkv_adapt(A, U, X, codes, p, replaced=replaced, workspace=ws, stream=st)
        if ev is not None:
            ev[3].record(st)

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    # per-kernel times: HIP events on the launch stream around every launch of the K steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(warmup + k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # whole-step throughput of decode-sized steps: the same K steps (same dictionary sets and
    # batches, in the same order) replayed as one captured HIP graph each, so that the three
    # launches of a step reach the GPU back to back
    use_graph = not args.eager and T * M <= 65536
    if use_graph:
        combos = sorted({((warmup + k) % R, (warmup + k) % n_batches) for k in range(steps)})
        graphs = {}
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for (ri, bi) in combos:
                kk = next(k for k in range(R * n_batches) if (k % R, k % n_batches) == (ri, bi))
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(kk, strm=torch.cuda.current_stream())
                graphs[(ri, bi)] = g
        stream.wait_stream(side)
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            graphs[((warmup + k) % R, (warmup + k) % n_batches)].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    stage_ms = [0.0, 0.0, 0.0]
    for e in evs:
        for i in range(3):
            stage_ms[i] += e[i].elapsed_time(e[i + 1])
    stage_ms = [x / steps for x in stage_ms]
    G = T * M
    vec_per_step = G
    value = vec_per_step * steps / wall

    # algorithmic work per launch (per-unit figures of the hot-path table, times the units)
    code_bytes = G * (w.s * 8 + 5)                 # idx + coef per slot, relerr, flags
    screen_flops = 2.0 * N * d * G
    screen_bytes = dict_bytes + G * d * esize      # the dictionary once + the vectors
    # GM: 2 s n d flops per vector (a pool-wide Gram column per greedy step); the kernel skips
    # the column of the last step, so it executes (s - 1) / s of that figure
    sel_flops = 2.0 * G * w.s * w.n * d if args.select == "gm" else 2.0 * G * w.s * w.s * d
    sel_flops_executed = (2.0 * G * (w.s - 1) * w.n * d if args.select == "gm"
                          else 2.0 * G * w.s * w.s * d)
    adapt_bytes = code_bytes + 2 * T * N * 4
    step_bytes = dict_bytes + G * d * esize + code_bytes + 2 * T * N * 4
    kernels = {
        "screen_topn": {"ms": stage_ms[0], "flops": screen_flops, "bytes": screen_bytes},
        "select_support": {"ms": stage_ms[1], "flops": sel_flops,
                           "flops_executed": sel_flops_executed},
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
    # the screening kernel against HBM, and the whole step (the decode-step figure of merit)
    screen_gbs = screen_bytes / (stage_ms[0] * 1e-3) / 1e9
    step_gbs = step_bytes / (wall / steps) / 1e9
    trig = int((codes.flags & fadkv.FLAG_TRIGGER).ne(0).sum().item())
    rep = int((replaced >= 0).sum().item())

    out = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_dicts": T, "vectors_per_dict": M, "N": N, "n": w.n,
                   "s": w.s, "d": d, "select": args.select,
                   "dictionary_sets": R, "cache": "warm" if R == 1 else
                   f"cold: {R} rotating dictionary sets ({R * dict_bytes / 2**20:.0f} MiB)",
                   "launch": "hip graph per step" if use_graph else "eager"},
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "screen_hbm": {"achieved": screen_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": screen_gbs / HBM_PEAK_GBS, "bytes": screen_bytes},
        "step_hbm": {"achieved": step_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": step_gbs / HBM_PEAK_GBS, "bytes": step_bytes,
                     "what": "dictionary + vectors + codes + usage read/write per step, over "
                             "the whole step's time"},
        "last_step": {"triggers": trig, "replaced": rep},
    }
    return w, out


def yardsticks(dev):
    """Measured references beside the published peaks: a plain device copy (bytes read +
    written per second) and the library's bf16 GEMM of the 3B prefill score shape (per
    dictionary 65536 x 128 times 128 x 4096, product written to HBM in bf16), timed over
    chunks of 8 dictionaries with random operands."""
    import torch

    from sparse_dictionary_coding_amd import synth
    out = {}
    n = 1 << 28                                    # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    out["copy"] = {"gbs": 2 * n * 4 / (ms * 1e-3) / 1e9, "bytes_per_copy": 2 * n * 4,
                   "what": "dst.copy_(src) of 1 GiB, read + write"}
    del src, dst
    w = synth.WORKLOADS["llama3b_prefill"]
    T = 8
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    X = torch.randn(T, w.M, w.d, device=dev, dtype=torch.bfloat16, generator=g)
    Dt = torch.randn(T, w.d, w.N, device=dev, dtype=torch.bfloat16, generator=g).contiguous()
    prod = torch.empty(T, w.M, w.N, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        torch.bmm(X, Dt, out=prod)
    torch.cuda.synchronize()
    reps = 5
    e0.record()
    for _ in range(reps):
        torch.bmm(X, Dt, out=prod)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * T * w.M * w.N * w.d
    out["gemm_bf16"] = {"tflops": flops / (ms * 1e-3) / 1e12,
                        "ms_all_dictionaries": ms * w.num_dicts / T,
                        "shape": f"{w.num_dicts} x ({w.M} x {w.d}) . ({w.d} x {w.N}), bf16 out",
                        "what": "torch.bmm (the library GEMM), 8 dictionaries per call"}
    del X, Dt, prod
    torch.cuda.empty_cache()
    return out


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
    if args.path == "growth":
        bench_growth(args)
        return
    if args.path == "omp":
        bench_omp(args)
        return

    w, out = measure_encode(args, args.workload, args.steps, args.warmup)
    if args.workload == "llama3b_decode" and not args.no_prefill:
        # the prefill configuration of the same model, reported beside the decode step
        import torch
        torch.cuda.empty_cache()
        wp, pre = measure_encode(args, "llama3b_prefill", 3, 1)
        out["prefill"] = {k: pre[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                               "roofline", "kernels")}
        out["prefill"]["screen_mfma"] = {
            "achieved": pre["kernels"]["screen_topn"]["flops"] / (pre["kernels"]["screen_topn"]["ms"] * 1e-3) / 1e12,
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        out["prefill"]["screen_mfma"]["frac"] = out["prefill"]["screen_mfma"]["achieved"] / MFMA_BF16_PEAK_TFLOPS
        out["prefill"]["steps"], out["prefill"]["warmup"] = 3, 1
        ys = yardsticks(torch.device("cuda:0"))
        out["yardsticks"] = ys
        out["screen_hbm"]["frac_of_copy"] = out["screen_hbm"]["achieved"] / ys["copy"]["gbs"]
        out["prefill"]["screen_mfma"]["frac_of_gemm"] = (
            out["prefill"]["screen_mfma"]["achieved"] / ys["gemm_bf16"]["tflops"])
        # the other decode configurations, each a nested object of the same line
        for other in ("llama8b_decode", "qwen4b_long_decode"):
            torch.cuda.empty_cache()
            _, o = measure_encode(args, other, args.steps, args.warmup)
            out[other] = {k: o[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                             "roofline", "kernels", "screen_hbm", "step_hbm")}
            out[other]["steps"], out[other]["warmup"] = args.steps, args.warmup
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.select, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
