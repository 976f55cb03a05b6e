"""Benchmark: 3-bit compressed-space decode attention at 32K context on one MI355X.

One step is one decode step of a 48-layer model whose every layer has the
long-context shape (batch 1, 32 query heads, 4 KV heads, head_dim 128, 32768
cached tokens, bf16 K/V/Q drawn as in the long32k workload): one
iq_decode_attention_append launch rotates, quantizes and packs the new token's
K and V of every layer into the caches and runs attention of all layers on
the packed caches (layers are passed as batch entries, each with its own
rotation).  Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is KV tokens/s: cached token positions
attended per second, summed over layers, each position covering all 4 KV
heads.  The roofline object is for that launch (the split-K kernel with the
append, plus its small combine kernel), timed with HIP events on the stream
it runs on; its algorithmic bytes are the packed K/V codes and scales read,
104 bytes per (token, KV head), plus the new tokens read and written.
`traffic` is the HBM bytes per launch from the committed rocprofv3 counter
runs (profiles/decode_traffic.json), reported only while the decode kernel
source is the one those counters were taken on.  Extra fields report the
decode alone, the append then decode as two launches, a single-layer decode,
the GQA 8K and ragged-batch decode shapes, and the bulk prefill quantization
(48 layers x 4 KV heads x 32768 tokens, K and V Student-t(3), bf16).

Timing: a read-only stream probe and --settle seconds of untimed steps run
first whatever --warmup says (the GPU's clocks need about a second of work to
settle), then --warmup untimed steps, then --steps steps, each between its own
pair of HIP events on the call's stream.  ms_per_step is the median; min and
max are reported beside it, and the roofline uses the mean.  The CPU baseline
times the oracle on bounded samples of every workload, single-threaded and on
all of BLAS's threads, and states the host's CPU model and counts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LAYERS, HQ, HKV, T, D = 48, 32, 4, 32768, 128
BYTES_PER_TOKEN_HEAD = 2 * (48 + 4)          # K and V: 48-byte record + fp32 scale
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def measured_traffic():
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, or None
    when the decode kernel source has changed since those counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps, each between its own HIP events")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps right before the timed ones")
    ap.add_argument("--settle", type=float, default=2.0,
                    help="seconds of untimed steps before the warm-up, whatever --warmup says (the GPU's "
                         "clocks need about a second of work to settle)")
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-other-shapes", action="store_true", help="skip the gqa8k and ragged decode timings")
    ap.add_argument("--no-isotropy", action="store_true", help="skip the isotropy diagnostics")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the 2/4-bit, Lloyd-Max and asymmetric record formats")
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="time of each oracle sample (5 workloads, single-threaded and all cores)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and exit: the "
                         "reference reading for the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the timed steps (for counter runs); prints a short JSON line")
    ap.add_argument("--multi-only", type=int, default=0, metavar="Q",
                    help="only --warmup then --steps multi-token decode calls of Q query tokens on the "
                         "48-layer cache (for counter runs); prints a short JSON line")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def time_calls(fn, iters, stream):
    """Average duration (s) of fn() over iters calls, HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / iters


def time_each(fn, iters, stream):
    """Durations (s) of iters calls of fn(), each between its own pair of HIP events on `stream`
    (the calls are still enqueued back to back).  Returns the sorted list."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for s_, e_ in ev:
        s_.record(stream)
        fn()
        e_.record(stream)
    torch.cuda.synchronize()
    return sorted(s_.elapsed_time(e_) / 1e3 for s_, e_ in ev)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def settle(fn, seconds):
    """Untimed calls of fn() for at least `seconds` of wall time (in batches, synchronised), so
    that the GPU's clocks have reached their steady state before anything is timed.  Returns the
    number of calls."""
    import torch
    calls, t0 = 0, time.time()
    while True:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        calls += 50
        if time.time() - t0 >= seconds:
            return calls


def host_info():
    """The host the CPU baseline runs on: CPU model, logical CPUs, CPUs this process may use and
    the BLAS thread count."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": int(blas)}


def cpu_baselines(seconds):
    """The CPU oracle timed on bounded samples of every workload, single-threaded and with all of
    BLAS's threads: decode (unpack of the packed K/V records + fp64 decode attention) in KV
    tokens/s for the tiny, gqa8k, long32k and ragged shapes, and quantize (rotation, 3-bit codes,
    packing) in vectors/s for the prefill shape.  The packed records are random bytes (every byte
    pattern is a valid record; the oracle's work does not depend on the values), the rotations,
    queries and prefill vectors come from the seeded workloads.  A sample that covers some of the
    KV heads or sequences is scaled to the whole step by its share of the (token, KV head) pairs.
    Each sample repeats until `seconds` have passed."""
    import oracle
    from threadpoolctl import threadpool_limits
    from compressed_space_decode_amd import workloads as W
    rng = np.random.default_rng(2024)
    res = {}

    def run(fn, work):
        out = {}
        for label, lim in (("single_thread", 1), ("all_cores", None)):
            with threadpool_limits(lim):
                n, t0 = 0, time.perf_counter()
                while True:
                    fn()
                    n += 1
                    el = time.perf_counter() - t0
                    if el >= seconds:
                        break
            out[label] = work * n / el
        return out

    def decode_sample(name, B, Hq, Hkv, lens, heads):
        G = Hq // Hkv
        T = int(max(lens))
        rec_k = rng.integers(0, 256, size=(B, heads, T, 48), dtype=np.uint8)
        rec_v = rng.integers(0, 256, size=(B, heads, T, 48), dtype=np.uint8)
        sk = rng.uniform(0.05, 1.0, size=(B, heads, T)).astype(np.float32)
        sv = rng.uniform(0.05, 1.0, size=(B, heads, T)).astype(np.float32)
        q = rng.standard_normal((B, heads * G, 128))
        params = W.rotation_params(rng, B * heads).reshape(B, heads, 32, 8)
        lens = np.asarray(lens)

        def fn():
            oracle.decode_attention(q, oracle.unpack(rec_k), sk, oracle.unpack(rec_v), sv, params, lens)

        r = run(fn, float(np.sum(lens)) * heads / Hkv)     # KV tokens (all heads) per sample
        return r

    info = W.SHAPES
    B, Hq, Hkv, T, _ = info["tiny"]
    res["tiny"] = dict(decode_sample("tiny", B, Hq, Hkv, [T] * B, Hkv), unit="KV tokens/s",
                       sample="the whole step: %d KV heads x %d tokens" % (Hkv, T))
    B, Hq, Hkv, T, _ = info["gqa8k"]
    res["gqa8k"] = dict(decode_sample("gqa8k", B, Hq, Hkv, [T] * B, Hkv), unit="KV tokens/s",
                        sample="the whole step: %d KV heads x %d tokens, %d query heads" % (Hkv, T, Hq))
    B, Hq, Hkv, T, _ = info["long32k"]
    res["long32k"] = dict(decode_sample("long32k", 1, Hq, Hkv, [T], 1), unit="KV tokens/s",
                          sample="1 of %d KV heads (with its %d query heads) x %d tokens, scaled by %d" %
                                 (Hkv, Hq // Hkv, T, Hkv))
    B, Hq, Hkv, T, _ = info["ragged"]
    lens_r = W.decode_workload("ragged")["seq_lens"]
    res["ragged"] = dict(decode_sample("ragged", 1, Hq, Hkv, [int(lens_r[0])], 1), unit="KV tokens/s",
                         sample="sequence 0 of %d (%d tokens), 1 of %d KV heads (with its %d query heads); "
                                "rate per (token, KV head) pair over %d KV heads" %
                                (B, int(lens_r[0]), Hkv, Hq // Hkv, Hkv))
    k, _, pparams = W.prefill_layer(0, tokens=8192)
    x = W.to_f64(k[0], "bf16")
    params = pparams[0]

    def quant():
        codes, _, _, _ = oracle.quantize(x, params)
        oracle.pack(codes)

    res["prefill"] = dict(run(quant, x.shape[0]), unit="vectors/s",
                          sample="8192 K vectors of prefill layer 0, head 0 (Student-t(3), bf16): rotation, "
                                 "codes, scale and packing")
    return res


def isotropy_summary(iq, W, x, rot, seed):
    """The isotropy statistics of x [S][H][T][128] under every transform, summarised over the
    heads: mean and largest per-coordinate kurtosis, mean 3-bit quantization error (relative) and
    mean peak-to-average power ratio."""
    import torch
    S, H = x.shape[:2]
    dense = torch.from_numpy(W.dense_rotations(seed, S * H)).to(x.device)
    out = {}
    for mode in iq.TRANSFORMS:
        st = iq.isotropy_stats(x, mode, rot=rot, dense=dense).cpu().numpy().reshape(S * H, -1)
        out[mode] = {"kurtosis_mean": float(st[:, 0:128].mean()), "kurtosis_max": float(st[:, 0:128].max()),
                     "vector_kurtosis": float(st[:, 256].mean()), "rel_quant_mse": float(st[:, 257].mean()),
                     "papr": float(st[:, 258].mean())}
    return out


def time_graph(fn, per_graph, replays, stream):
    """Duration (s) of one fn() call from per_graph calls captured in one HIP graph, replayed
    `replays` times on `stream` (the median replay over per_graph): the GPU's time for a call
    without the host's per-call overhead (which is larger than a small call's GPU time).  fn must
    allocate nothing."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):          # one call off the capture, as torch asks
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    with torch.cuda.stream(stream):
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t = time_each(graph.replay, replays, stream)
    return median(t) / per_graph


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch

    import compressed_space_decode_amd as iq
    from compressed_space_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    L = args.layers

    # ---------------- inputs (seeded, synthetic) ----------------
    t0 = time.time()
    w = W.decode_workload("long32k", batch=L)
    log("generated %d layers of long32k inputs in %.1fs" % (L, time.time() - t0))

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    k_all = bf16(w["k"])                      # [L][Hkv][T][128]
    v_all = bf16(w["v"])
    q = bf16(w["q"])                          # [L][Hq][128]
    rot = torch.from_numpy(w["params"]).to(dev)   # [L][Hkv][32][8]
    del w
    kc = torch.empty((L, HKV, T, 48), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((L, HKV, T), dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    iq.quantize_kv(k_all, v_all, rot, kc, ks, vc, vs)          # prefill the caches
    lens = torch.full((L,), T, dtype=torch.int32, device=dev)
    out = torch.empty((L, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(iq.decode_workspace_bytes(L, HQ, HKV, T), dtype=torch.uint8, device=dev)
    k_new = k_all[:, :, T - 1]                # the step's new token: position T-1 of every layer
    v_new = v_all[:, :, T - 1]                # [L][Hkv][128] views
    positions = torch.full((L,), T - 1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    if args.multi_only:                       # counter runs of the multi-token kernel
        Qm = args.multi_only
        qm = bf16(W.multi_token_queries(L, Qm, HQ))
        outm = torch.empty((L, Qm, HQ, D), dtype=torch.float32, device=dev)
        wsm = torch.empty(iq.decode_workspace_bytes(L * Qm, HQ, HKV, T), dtype=torch.uint8, device=dev)

        def dec_m():
            iq.decode_attention_multi(qm, kc, ks, vc, vs, rot, seq_lens=lens, out=outm, workspace=wsm)

        settle(dec_m, args.settle)
        for _ in range(args.warmup):
            dec_m()
        torch.cuda.synchronize()
        t_m = median(time_each(dec_m, args.steps, stream))
        print(json.dumps({"multi_query_tokens": Qm, "ms": t_m * 1e3}), flush=True)
        return

    def step():                               # one launch: append the new token, then attend
        iq.decode_attention_append(q, k_new, v_new, positions, kc, ks, vc, vs, rot, out=out, workspace=ws)

    def append():
        iq.quantize_kv(k_new[:, :, None], v_new[:, :, None], rot, kc, ks, vc, vs, tok_offset=T - 1)

    def decode():
        iq.decode_attention(q, kc, ks, vc, vs, rot, seq_lens=lens, out=out, workspace=ws)

    def two_calls():
        append()
        decode()

    decode_bytes = L * T * HKV * BYTES_PER_TOKEN_HEAD
    step_bytes = decode_bytes + L * HKV * 2 * (2 * D + 48 + 4)   # + the new K/V: bf16 read, record written
    tokens_per_step = L * T

    # ---------------- untimed work first: the clocks settle ----------------
    # the device's read-only streaming rate over as many bytes as the step reads (libiq_probe.so):
    # the measured ceiling beside the nominal 8 TB/s.  It runs before the timed steps, and the step
    # itself then runs untimed for --settle seconds, whatever --warmup says: a GPU that has just
    # started needs about a second of work before its clocks are steady.
    stream_gbs = t_stream = None
    t_streams = {}
    if not args.decode_only:
        sbuf = torch.empty(decode_bytes, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4, dtype=torch.uint8, device=dev)

        # both load policies; the faster one is the ceiling
        for nt in (False, True):
            def stream_pass(nt=nt):
                iq.stream_read(sbuf, sink, 2048, nontemporal=nt)

            settle(stream_pass, 0.5)
            t_streams[nt] = median(time_each(stream_pass, 50, stream))
        t_stream = min(t_streams.values())
        stream_gbs = decode_bytes / t_stream / 1e9
        del sbuf
        log("read-only stream of %d bytes: %.1f us with default loads, %.1f us with non-temporal loads "
            "(medians of 50), ceiling %.0f GB/s" % (decode_bytes, t_streams[False] * 1e6, t_streams[True] * 1e6,
                                                    stream_gbs))
    n_settle = settle(step, args.settle)
    log("settle: %d untimed steps in >= %.1f s" % (n_settle, args.settle))

    # ---------------- timed steps ----------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps_t = time_each(step, args.steps, stream)
    t_step = median(steps_t)
    t_decode = median(time_each(decode, args.steps, stream))
    t_append = median(time_each(append, args.steps, stream))
    t_two = median(time_each(two_calls, args.steps, stream))
    log("step median %.1f us (min %.1f, max %.1f over %d); decode alone %.1f us, append alone %.1f us, "
        "append then decode %.1f us" % (t_step * 1e6, steps_t[0] * 1e6, steps_t[-1] * 1e6, len(steps_t),
                                        t_decode * 1e6, t_append * 1e6, t_two * 1e6))
    step_gbs = step_bytes / t_step / 1e9
    t_step_mean = sum(steps_t) / len(steps_t)
    step_gbs_mean = step_bytes / t_step_mean / 1e9

    if args.decode_only:
        print(json.dumps({"step_us": t_step * 1e6, "decode_us": t_decode * 1e6, "step_GBs": step_gbs}), flush=True)
        return

    # single-layer decode call (the one-layer shape, unadjusted)
    ws1 = torch.empty(iq.decode_workspace_bytes(1, HQ, HKV, T), dtype=torch.uint8, device=dev)
    out1 = torch.empty((1, HQ, D), dtype=torch.float32, device=dev)

    def decode1():
        iq.decode_attention(q[:1], kc[:1], ks[:1], vc[:1], vs[:1], rot[:1], seq_lens=lens[:1], out=out1,
                            workspace=ws1)

    settle(decode1, 0.2)
    t_eager1 = median(time_each(decode1, max(20, args.steps), stream))
    t_decode1 = time_graph(decode1, 20, max(10, args.steps // 10), stream)
    single = {"ms": t_decode1 * 1e3, "GBs": T * HKV * BYTES_PER_TOKEN_HEAD / t_decode1 / 1e9,
              "kv_tokens_per_s": T / t_decode1, "timing": "graph of 20 calls, replayed",
              "eager_ms": t_eager1 * 1e3}
    log("single-layer decode %.1f us from graph replays (%.1f us eager)" % (t_decode1 * 1e6, t_eager1 * 1e6))

    # ---------------- record formats: quantize + decode time and attention error per format ----------------
    formats = {}
    if not args.no_formats:
        def exact_attention(qx, kx, vx):
            """fp32 attention of qx [Hq][128] on unquantized kx, vx [Hkv][T][128] (the accuracy reference)."""
            Gx = qx.shape[0] // kx.shape[0]
            r = torch.empty_like(qx)
            for g in range(kx.shape[0]):
                s_ = (qx[g * Gx:(g + 1) * Gx] @ kx[g].t().contiguous()) / np.sqrt(D)
                r[g * Gx:(g + 1) * Gx] = torch.softmax(s_, dim=-1) @ vx[g]
            return r

        def rel_err(a, b):
            return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))

        ref = exact_attention(q[0].float(), k_all[0].float(), v_all[0].float())
        # a Gaussian workload (Q, K, V ~ N(0,1), 4 heads, 512 tokens, fp32): attention spread over many tokens
        wt = W.decode_workload("tiny")
        kt, vt, qt = (torch.from_numpy(wt[n]).to(dev) for n in ("k", "v", "q"))
        rott = torch.from_numpy(wt["params"]).to(dev)
        Tt = kt.shape[2]
        ref_t = exact_attention(qt[0], kt[0], vt[0])
        for fmt in ("u2", "u3", "u4", "lm3", "a3"):
            rb = 16 * iq.FORMAT_BITS[fmt]
            sw = 2 if fmt == "a3" else 1                 # fp32 per vector: (s, m) for the asymmetric format
            kcf = torch.empty((L, HKV, T, rb), dtype=torch.uint8, device=dev)
            vcf = torch.empty_like(kcf)
            ksf = torch.empty(iq.scale_shape((L, HKV, T), fmt), dtype=torch.float32, device=dev)
            vsf = torch.empty_like(ksf)

            def quant_f(fmt=fmt):
                iq.quantize_kv(k_all, v_all, rot, kcf, ksf, vcf, vsf, fmt=fmt)

            def dec_f(fmt=fmt):
                iq.decode_attention(q, kcf, ksf, vcf, vsf, rot, seq_lens=lens, out=out, workspace=ws, fmt=fmt)

            quant_f()
            dec_f()
            torch.cuda.synchronize()
            err = rel_err(out[0], ref)
            kct = torch.empty((1, kt.shape[1], Tt, rb), dtype=torch.uint8, device=dev)
            vct = torch.empty_like(kct)
            kst = torch.empty(iq.scale_shape((1, kt.shape[1], Tt), fmt), dtype=torch.float32, device=dev)
            vst = torch.empty_like(kst)
            iq.quantize_kv(kt, vt, rott, kct, kst, vct, vst, fmt=fmt)
            err_t = rel_err(iq.decode_attention(qt, kct, kst, vct, vst, rott, fmt=fmt)[0], ref_t)
            del kct, vct, kst, vst
            # each timing starts on steady clocks, like the headline's (the calls before were short)
            settle(quant_f, 0.2)
            t_qf = median(time_each(quant_f, 7, stream))
            settle(dec_f, 0.3)
            t_df = median(time_each(dec_f, 21, stream))
            cache_b = L * HKV * T * 2 * (rb + 4 * sw)
            formats[fmt] = {"bits": iq.FORMAT_BITS[fmt], "record_bytes": rb,
                            "attention_rel_error_long32k_layer0": err, "attention_rel_error_gaussian": err_t,
                            "quantize_ms": t_qf * 1e3, "decode_ms": t_df * 1e3,
                            "decode_GBs": cache_b / t_df / 1e9, "cache_bytes": cache_b}
            log("format %s: attention error %.4f (long32k layer 0), %.4f (Gaussian), quantize %.2f ms, "
                "decode %.1f us (%.0f GB/s)" % (fmt, err, err_t, t_qf * 1e3, t_df * 1e6, cache_b / t_df / 1e9))
            del kcf, vcf, ksf, vsf
        del ref, ref_t, kt, vt, qt

    # ---------------- several query tokens per sequence on the same 48-layer cache ----------------
    multi = {}
    if not args.no_other_shapes:
        for Qm in (4, 16):
            qm = bf16(W.multi_token_queries(L, Qm, HQ))
            outm = torch.empty((L, Qm, HQ, D), dtype=torch.float32, device=dev)
            wsm = torch.empty(iq.decode_workspace_bytes(L * Qm, HQ, HKV, T), dtype=torch.uint8, device=dev)

            def dec_m():
                iq.decode_attention_multi(qm, kc, ks, vc, vs, rot, seq_lens=lens, out=outm, workspace=wsm)

            for _ in range(20):
                dec_m()
            settle(dec_m, 0.3)
            t_m = median(time_each(dec_m, max(20, args.steps // 8), stream))
            flops = 2 * 2 * L * Qm * HQ * T * D       # QK and PV multiply-adds, causal tail ignored
            multi["q%d" % Qm] = {"query_tokens": Qm, "ms": t_m * 1e3, "kv_tokens_per_s": L * T / t_m,
                                 "query_token_kv_per_s": L * T * Qm / t_m,
                                 "GBs_packed_cache": decode_bytes / t_m / 1e9, "TFLOPs": flops / t_m / 1e12}
            log("multi-token decode Q=%d: %.1f us, %.0f GB/s of packed cache, %.1f TFLOP/s" %
                (Qm, t_m * 1e6, decode_bytes / t_m / 1e9, flops / t_m / 1e12))
            del qm, outm, wsm

    # ---------------- the other decode shapes: GQA at 8K and the ragged batch ----------------
    others = {}
    iso_quality = {}
    if not args.no_isotropy:
        iso_quality["long32k"] = isotropy_summary(iq, W, k_all[:1], rot[:1], seed=100)
    if not args.no_other_shapes:
        for name in ("gqa8k", "ragged"):
            wo = W.decode_workload(name)
            Bo, Hkvo, To = wo["k"].shape[:3]
            Hqo = wo["q"].shape[1]
            ko, vo = bf16(wo["k"]), bf16(wo["v"])
            roto = torch.from_numpy(wo["params"]).to(dev)
            kco = torch.empty((Bo, Hkvo, To, 48), dtype=torch.uint8, device=dev)
            vco = torch.empty_like(kco)
            kso = torch.empty((Bo, Hkvo, To), dtype=torch.float32, device=dev)
            vso = torch.empty_like(kso)
            iq.quantize_kv(ko, vo, roto, kco, kso, vco, vso)
            if not args.no_isotropy:
                iso_quality[name] = isotropy_summary(iq, W, ko, roto, seed=len(iso_quality))
            del ko, vo
            qo = bf16(wo["q"])
            lo = torch.from_numpy(wo["seq_lens"]).to(dev)
            outo = torch.empty((Bo, Hqo, D), dtype=torch.float32, device=dev)
            wso = torch.empty(iq.decode_workspace_bytes(Bo, Hqo, Hkvo, To), dtype=torch.uint8, device=dev)

            def dec_o():
                iq.decode_attention(qo, kco, kso, vco, vso, roto, seq_lens=lo, out=outo, workspace=wso)

            settle(dec_o, 0.2)
            t_e = median(time_each(dec_o, max(20, args.steps // 4), stream))
            t_o = time_graph(dec_o, 20, max(10, args.steps // 10), stream)
            toks = int(wo["seq_lens"].sum())
            others[name] = {"batch": int(Bo), "n_q_heads": int(Hqo), "n_kv_heads": int(Hkvo), "cache_cap": int(To),
                            "kv_tokens": toks, "ms": t_o * 1e3, "kv_tokens_per_s": toks / t_o,
                            "GBs": toks * Hkvo * BYTES_PER_TOKEN_HEAD / t_o / 1e9,
                            "frac_of_hbm_peak": toks * Hkvo * BYTES_PER_TOKEN_HEAD / t_o / 1e9 / HBM_PEAK_GBS,
                            "timing": "graph of 20 calls, replayed", "eager_ms": t_e * 1e3}
            log("%s decode %.1f us from graph replays (%.1f us eager), %.0f GB/s" %
                (name, t_o * 1e6, t_e * 1e6, others[name]["GBs"]))
            del kco, vco, kso, vso, wso, wo
        torch.cuda.empty_cache()

    # ---------------- bulk prefill quantization ----------------
    prefill = None
    iso_timing = None
    if not args.no_prefill:
        del k_all, v_all
        torch.cuda.empty_cache()
        t0 = time.time()
        data = W.prefill_layers(range(LAYERS))
        pk = torch.empty((LAYERS, HKV, T, D), dtype=torch.bfloat16, device=dev)
        pv = torch.empty_like(pk)
        prot = torch.from_numpy(np.stack([d[2] for d in data])).to(dev)
        for l, (kk, vv, _) in enumerate(data):
            pk[l] = bf16(kk)
            pv[l] = bf16(vv)
        del data
        log("generated prefill inputs in %.1fs" % (time.time() - t0))
        pkc = torch.empty((LAYERS, HKV, T, 48), dtype=torch.uint8, device=dev)
        pvc = torch.empty_like(pkc)
        pks = torch.empty((LAYERS, HKV, T), dtype=torch.float32, device=dev)
        pvs = torch.empty_like(pks)

        def quant():
            iq.quantize_kv(pk, pv, prot, pkc, pks, pvc, pvs)

        quant()
        torch.cuda.synchronize()
        settle(quant, 0.3)
        t_q = median(time_each(quant, max(10, args.steps // 4), stream))
        qbytes = LAYERS * HKV * T * 2 * (D * 2 + 48 + 4)
        prefill = {"workload": "prefill 48x4x32768 K+V bf16 Student-t(3)", "ms": t_q * 1e3,
                   "GBs": qbytes / t_q / 1e9, "frac_of_hbm_peak": qbytes / t_q / 1e9 / HBM_PEAK_GBS,
                   "vectors_per_s": LAYERS * HKV * T * 2 / t_q}
        log("prefill quantize %.2f ms, %.0f GB/s" % (t_q * 1e3, prefill["GBs"]))
        if not args.no_isotropy:
            iso_quality["prefill"] = isotropy_summary(iq, W, pk[:1], prot[:1], seed=101)
            # throughput of the statistics kernels over the 48-layer K (bf16), per transform
            pdense = torch.from_numpy(W.dense_rotations(102, LAYERS * HKV)).to(dev)
            st_buf = torch.empty((LAYERS, HKV, iq.N_STATS), dtype=torch.float64, device=dev)
            ws_iso = torch.empty(iq.isotropy_workspace_bytes(LAYERS, HKV, T), dtype=torch.uint8, device=dev)
            iso_bytes = LAYERS * HKV * T * D * 2
            iso_timing = {}
            for mode in iq.TRANSFORMS:
                def iso_fn(mode=mode):
                    iq.isotropy_stats(pk, mode, rot=prot, dense=pdense, stats=st_buf, workspace=ws_iso)
                iso_fn()
                torch.cuda.synchronize()
                t_i = time_calls(iso_fn, 10 if mode == "dense" else 20, stream)
                iso_timing[mode] = {"ms": t_i * 1e3, "GBs": iso_bytes / t_i / 1e9,
                                    "frac_of_hbm_peak": iso_bytes / t_i / 1e9 / HBM_PEAK_GBS}
                log("isotropy stats (%s) %.2f ms, %.0f GB/s" % (mode, t_i * 1e3, iso_bytes / t_i / 1e9))
            del pdense, ws_iso

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        host = host_info()
        by_cfg = cpu_baselines(args.cpu_seconds)
        log("cpu oracle baselines in %.1fs: %s" % (time.time() - t0, ", ".join(
            "%s %.3g/%.3g %s (1 thread / all)" % (k, v["single_thread"], v["all_cores"], v["unit"])
            for k, v in by_cfg.items())))
        main_cfg = by_cfg["long32k"]
        cpu = {"value": main_cfg["all_cores"], "unit": "KV tokens/s", "cores": host["blas_threads"],
               "kind": "oracle",
               "sample": "long32k shape, one layer: %s; oracle unpack of the packed K/V records + fp64 decode "
                         "attention, repeated for %.1f s, with BLAS's %d threads (numpy itself single-threaded)" %
                         (main_cfg["sample"], args.cpu_seconds, host["blas_threads"]),
               "single_thread_value": main_cfg["single_thread"],
               "host": host,
               "by_workload": by_cfg}
    res = {
        "metric": "3-bit KV decode attention: KV tokens/s and achieved HBM GB/s (% peak) at 32K",
        "value": tokens_per_step / t_step,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "step_timing": {"how": "median of --steps calls, each between its own HIP event pair on the call's "
                               "stream, after a read-only stream probe, %d untimed steps over >= %.1f s and "
                               "--warmup more" % (n_settle, args.settle),
                        "median_us": t_step * 1e6, "min_us": steps_t[0] * 1e6, "max_us": steps_t[-1] * 1e6},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "long32k decode step x%d layers (per layer: batch 1, 32 query / 4 KV heads, "
                               "head_dim 128, 32768 cached tokens, bf16 inputs, 3-bit packed KV; the new token's "
                               "K/V appended and layer-stacked decode attention in one launch)" % L,
                   "layers": L, "batch": 1, "n_q_heads": HQ, "n_kv_heads": HKV, "context": T,
                   "head_dim": D, "kv_bits": 3},
        "roofline": {"bound": "hbm", "achieved": step_gbs_mean, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": step_gbs_mean / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "iq_decode_attention_append (decode_split_kernel with the append, combine_kernel)",
                     "algorithmic_bytes_per_launch": step_bytes, "avg_launch_us": t_step_mean * 1e6,
                     "median_launch_us": t_step * 1e6, "frac_at_median": step_gbs / HBM_PEAK_GBS,
                     "frac_of_measured_stream": step_gbs_mean / stream_gbs},
        "stream_read": {"GBs": stream_gbs, "bytes": decode_bytes, "us": t_stream * 1e6,
                        "us_default_loads": t_streams[False] * 1e6 if t_streams else None,
                        "us_nontemporal_loads": t_streams[True] * 1e6 if t_streams else None,
                        "kernel": "iq_probe_stream_read / iq_probe_stream_read_nt (libiq_probe.so): 16-byte "
                                  "loads, grid-stride, 2048 x 256 threads; the faster of the two"},
        "decode_only": {"ms": t_decode * 1e3, "GBs": decode_bytes / t_decode / 1e9},
        "append_then_decode_ms": t_two * 1e3,
        "append_alone_ms": t_append * 1e3,
        "single_layer_decode": single,
        "other_decode_shapes": others,
        "record_formats": {"workload": "long32k x48 layers: K+V quantize and decode time; relative error of the "
                                       "attention output against fp32 attention on the unquantized K/V, for long32k "
                                       "layer 0 (peaked scores) and for the Gaussian tiny workload",
                           "by_format": formats},
        "multi_token_decode": {"workload": "long32k x48 layers, the last Q positions as Q query tokens "
                                           "(causal), per layer 32 query / 4 KV heads", "by_tokens": multi},
        "prefill_quantize": prefill,
        "isotropy": None if args.no_isotropy else {
            "timing": {"workload": "K of prefill 48x4x32768 bf16 Student-t(3), stats per (layer, head)",
                       "by_transform": iso_timing},
            "quality": iso_quality},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
