"""Throughput of the Lightning Attention-2 forward + backward on one MI355X.

Workload: the fixed-token length sweep -- 131,072 tokens per batch at
(B, T) = (128, 1K), (32, 4K), (8, 16K), (2, 64K), (1, 128K), H = 16 heads,
d = d_v = 128, tile T_B = 128, no decay, bf16 in HBM with fp32 accumulation,
synthetic seeded inputs.  One step is the whole hot path (la2_forward then
la2_backward_saved on the same workspace, the training step) over each of the
five batches; every input is resident in HBM before the timed region starts.

Prints one JSON line: whole-job tokens/s over the timed steps, the per-length
tokens/s, the roofline of the dominant kernel measured with HIP events on the
stream the kernels run on, and the CPU oracle's tokens/s on a bounded sample.
The per-length forward / backward split comes from an instrumented pass of the
same steps (HIP events around every call) run before the timed region; inside
the timed region the only events bracket the two calls of the 1K point, each one
kernel launch (the backward's is the dominant kernel).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/sec on 1 MI355X vs T (1K–128K); % bf16 MFMA / HBM roofline"

# HBM bytes per launch of the dominant kernels at the 1K point, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs (one counter per run), each scaled by what the same counter reads for a plain 1 GiB
# device copy (FETCH_SIZE x 1.9999, WRITE_SIZE x 1.0000).  Each figure is valid only for the kernel
# source it was taken on (sha256 of the listed files, concatenated); for any other source the roofline
# reports traffic as null.
# At the 1K point: the backward reads q, k, v, dO and the final states (2176.4 MiB) and writes dq, dk, dv
# (1536.2 MiB); the forward reads q, k, v (1536.3 MiB) and writes o and the final states (640.0 MiB).
TRAFFIC = {
    "bwd1": {"sources": ("la2_bwd1_bf16.hip", "la2_tile64_bf16.h", "la2_bf16_common.h"),
             "sha256_16": "31e94894fcdcd234", "bytes": 3892799864},
    "fwd": {"sources": ("la2_fwd1_bf16.hip", "la2_tile64_bf16.h", "la2_bf16_common.h"),
            "sha256_16": "79a596ca0751e976", "bytes": 2281922299},
    # the same kernel's normalized elu + 1 instance (bench.py --normalized, forward-sized workspace):
    # q, k, v read (1536.4 MiB), o written (512.0 MiB)
    "nfwd": {"sources": ("la2_fwd1_bf16.hip", "la2_tile64_bf16.h", "la2_bf16_common.h"),
             "sha256_16": "79a596ca0751e976", "bytes": 2147886386},
}
PEAK_HBM_GBS = 8000.0


def traffic_of(name):
    """TRAFFIC[name]'s counted bytes per launch while its kernel sources still hash to what they were
    taken on, else None."""
    t = TRAFFIC[name]
    csrc = os.path.join(ROOT, "causal_linear_attention_amd", "csrc")
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in t["sources"]))
    return t["bytes"] if t["bytes"] is not None and sha.hexdigest()[:16] == t["sha256_16"] else None
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 5 for the length sweep, 50 for one --workload)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps before the timed ones (default 10 for the length sweep, 50 "
                         "for one --workload: the GPU needs some tens of ms of work before its clocks settle)")
    ap.add_argument("--points", default="all", help="comma list of sweep lengths in K (e.g. 1,128) or 'all'")
    ap.add_argument("--workload", default=None,
                    help="time one named workload of inputs.WORKLOADS (e.g. tnl15b_layer, long128k_outliers) "
                         "instead of the length sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=128,
                    help="sequences of the 1K point the oracle runs for the CPU baseline")
    ap.add_argument("--decode", action="store_true",
                    help="time la2_decode_step (one new token per sequence from a carried state) instead")
    ap.add_argument("--decode-batch", type=int, default=512,
                    help="sequences per decode step (512 x 16 heads: 512 MiB of fp32 state, beyond the "
                         "256 MiB memory-side cache)")
    ap.add_argument("--normalized", action="store_true",
                    help="time la2_forward_normalized (numerator over denominator, phi = elu + 1) on the 1K "
                         "point of the sweep instead, with the plain forward timed beside it")
    ap.add_argument("--compare", action="store_true",
                    help="comparison curves over T at a fixed token count: the tiled scan, the token-serial "
                         "recurrence kernel and torch's causal softmax attention (flash / memory-efficient "
                         "backends only), H = 12, d = 128, bf16")
    ap.add_argument("--compare-points", default="0.25,0.5,1,2,4,8,16,32,64,128",
                    help="sequence lengths in K for --compare")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device-to-device copies (reference for HBM byte counters)")
    ap.add_argument("--stream", action="store_true",
                    help="time the test build's plain HBM stream (16-byte lane accesses, 1 GiB per buffer) at the "
                         "read:write mixes of the tile kernels, over launch shapes and both cache policies")
    ap.add_argument("--cache-probe", action="store_true",
                    help="time the test build's memory-side cache probe: a state-only pass fused ahead of the "
                         "output pass against the two as separate launches, over item sizes")
    args = ap.parse_args()
    single = args.workload is not None
    if args.steps is None:
        args.steps = 50 if single else 5
    if args.warmup is None:
        args.warmup = 50 if single else 10
    return args


def copy_calibration():
    """Five plain copies of 1 GiB: a kernel of known traffic (1 GiB read + 1 GiB written per copy)."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": src.numel() * src.element_size(), "copies": 5}))


def stream_bench(args):
    """The bandwidth a plain stream reaches on this GPU for the kernels' read:write mixes: a copy (1:1),
    the forward output scan (3 tensors read, 1 written) and the one-pass backward (4 read, 3 written).
    Each dst = the sum of the srcs, 1 GiB per buffer, grid-stride over 16-byte chunks; the best of a
    sweep of launch shapes, with and without the nontemporal hint.  A ceiling for the tile kernels'
    GB/s that includes what HBM, the fabric and the memory pipeline of this chip deliver to 16-byte
    lane accesses, which the 8 TB/s peak does not."""
    import torch
    from causal_linear_attention_amd import binding

    nbytes = 1 << 30
    bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(7)]
    mixes = {"copy 1:1": (1, 1), "forward 3:1": (3, 1), "backward 4:3": (4, 3)}
    shapes = [(b, t) for b in (256, 512, 1024, 2048, 4096, 8192) for t in (256, 512)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    results, rows = {}, []
    for name, (ns, nd) in mixes.items():
        srcs, dsts = bufs[:ns], bufs[ns:ns + nd]
        best = None
        for nt in (1, 0):
            for b, t in shapes:
                for _ in range(2):
                    binding.stream_probe(srcs, dsts, b, t, nt)
                torch.cuda.synchronize()
                reps = 5
                ev[0].record()
                for _ in range(reps):
                    binding.stream_probe(srcs, dsts, b, t, nt)
                ev[1].record()
                torch.cuda.synchronize()
                ms = ev[0].elapsed_time(ev[1]) / reps
                gbs = (ns + nd) * nbytes / (ms * 1e-3) / 1e9
                rows.append({"mix": name, "nontemporal": bool(nt), "blocks": b, "threads": t,
                             "ms": round(ms, 4), "GBs": round(gbs, 1)})
                if best is None or gbs > best["GBs"]:
                    best = rows[-1]
        results[name] = best
        print(f"[stream] {name}: best {best['GBs']} GB/s ({best['blocks']} x {best['threads']}, "
              f"nontemporal {best['nontemporal']})", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "plain HBM stream, best launch shape per read:write mix", "unit": "GB/s",
                      "bytes_per_buffer": nbytes, "peak": PEAK_HBM_GBS, "best": results, "all": rows}), flush=True)


def cache_probe_bench(args):
    """Whether a state-only pass fused ahead of the output pass could take its second read of k and v
    from the memory-side cache instead of HBM: four 512 MiB tensors (q, k, v, o of 16 chains x 128K
    positions x 128 bf16, the 128K point) cut into items of L positions, one workgroup per item and
    one per CU (la2_test_reread).  Per L: phase B alone (the output pass), A then B in one workgroup,
    A alone, and A; B as two launches (the split-chain plan's order).  The best of 10 launches each."""
    import torch
    from causal_linear_attention_amd import binding

    nbytes = 512 << 20
    q, k, v, o = (torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(4))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(modes, nt, item, reps=10):
        best = None
        for _ in range(reps):
            ev[0].record()
            for m in modes:
                binding.reread_probe(q, k, v, o, item, m, nt)
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1])
            best = ms if best is None else min(best, ms)
        return best

    for _ in range(20):                       # some tens of ms of work first: clocks settle
        binding.reread_probe(q, k, v, o, 1 << 18, 1, 1)
    torch.cuda.synchronize()
    rows = []
    for L in (256, 512, 1024, 2048, 4096, 8192):
        item = L * 128 * 2
        for nt in (1, 0):
            r = {"L": L, "items": nbytes // item, "nontemporal": bool(nt),
                 "B_ms": round(best_ms((0,), nt, item), 4), "A_then_B_ms": round(best_ms((1,), nt, item), 4),
                 "A_ms": round(best_ms((2,), nt, item), 4), "A_B_two_launches_ms": round(best_ms((2, 0), nt, item), 4)}
            r["fused_over_B"] = round(r["A_then_B_ms"] / r["B_ms"], 3)
            r["two_launches_over_B"] = round(r["A_B_two_launches_ms"] / r["B_ms"], 3)
            rows.append(r)
            print(f"[cache] L={L} nt={nt}: B {r['B_ms']} ms, A then B {r['A_then_B_ms']} ms "
                  f"({r['fused_over_B']}x), A {r['A_ms']} ms, A; B {r['A_B_two_launches_ms']} ms "
                  f"({r['two_launches_over_B']}x)", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "memory-side cache re-read probe (state-only pass fused ahead of the output pass)",
                      "unit": "ms", "bytes_per_tensor": nbytes, "rows": rows}), flush=True)


def decode_bench(args):
    """One generated token per sequence: B sequences (default 512) x H = 16 heads, d = d_v = 128, bf16
    q/k/v/o, fp32 state (the carried summary of each sequence's prefix), per-head decay.  Each step
    reads and rewrites every state once, so it is HBM-bound: bytes per step = chains x (8 d d_v +
    2 (2d + 2d_v)).  Below ~256 MiB of state (B <= 256) the states stay in the memory-side cache."""
    import torch
    import causal_linear_attention_amd as la2
    from causal_linear_attention_amd import inputs
    B, H, d, dv = args.decode_batch, 16, 128, 128
    g = torch.Generator().manual_seed(5)
    dev = torch.device("cuda:0")
    steps_in = [[(torch.randn((B, H, n), generator=g) / math.sqrt(n)).to(torch.bfloat16).to(dev)
                 for n in (d, d, dv)] for _ in range(4)]
    decay = inputs.head_decays(H).to(dev)
    state = (torch.randn((B, H, d, dv), generator=g) * 0.1).to(dev)
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v = steps_in[i % 4]
        la2.la2_decode_step(q, k, v, decay, o, state, stream)

    for i in range(max(args.warmup, 1) * 10):
        step(i)
    torch.cuda.synchronize()
    n = max(args.steps, 1) * 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / n
    chains = B * H
    bytes_step = chains * (8 * d * dv + 2 * (2 * d + 2 * dv))
    achieved = bytes_step / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's state-carrying forward, one position at a time from the same kind of state: 128
        # sequences, 16 positions (the state handed from each call to the next)
        import oracle
        nb, nsteps = min(128, B), 16
        s_cur = state[:nb].double().cpu().numpy()
        lam = decay.double().cpu().numpy()
        ins = [[t[:nb].double().cpu().numpy()[:, :, None, :] for t in steps_in[i % 4]] for i in range(nsteps)]
        ta = time.perf_counter()
        for q, k, v in ins:
            _, s_cur = oracle.forward_state(q, k, v, lam, s_cur)
        tc = time.perf_counter() - ta
        cpu = {"value": round(nb * nsteps / tc, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"{nsteps} positions of {nb} sequences x {H} heads, each from the "
                                           f"fp32 state the previous one left, fp64, {tc:.2f} s",
               "host": host_info()}
    print(json.dumps({
        "metric": "decode tokens/sec (one new token per sequence from a carried state)", "value": round(B / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": max(args.warmup, 1) * 10,
        "ms_per_step": round(ms, 5), "wall_ms_per_step": round(wall / n * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 q/k/v/o, f32 state", "data": "synthetic",
        "config": {"workload": f"decode step: B={B} sequences, H={H}, d=d_v={d}, per-head decay, fp32 state",
                   "chains": chains, "state_MiB": chains * d * dv * 4 >> 20,
                   "cache_resident": chains * d * dv * 4 <= (256 << 20), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel<bf16,D=128,DV=128>", "avg_launch_ms": round(ms, 5),
                     "algorithmic_bytes_per_launch": bytes_step},
        "cpu_baseline": cpu,
    }), flush=True)


def normalized_bench(args):
    """The normalized forward o_t = phi(q_t)^T S_t / phi(q_t)^T z_t with phi = elu + 1 on the 1K point
    of the length sweep (B = 128, H = 16, T = 1024, d = d_v = 128, bf16, no decay).  Its algorithmic
    bytes are those of the plain forward (read q, k, v; write o): 4 d e per token-head, and at this
    shape the library moves just those, in one launch (phi applied to the tiles on chip, numerator and
    denominator together); the plain forward is timed beside it.  The backward of the training step
    reuses what the forward left in the workspace (la2_backward_normalized_saved; given that larger
    workspace the forward also writes phi(q), phi(k) and the denominators); the backward that
    recomputes them is timed beside it."""
    import torch
    import causal_linear_attention_amd as la2
    from causal_linear_attention_amd import inputs
    w = inputs.WORKLOADS["sweep131k_t1k"]
    x = inputs.make(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    decay = None if x["decay"] is None else x["decay"].to(dev)
    o = torch.empty_like(v)
    ws_n = la2.normalized_workspace_for(q, v, "elu1", w.block)
    ws_f = la2.workspace_for(q, v, w.block, False)
    stream = torch.cuda.current_stream()
    n = max(args.steps, 1) * 10

    def timed(fn):
        for _ in range(max(args.warmup, 1) * 3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_n = timed(lambda: la2.la2_forward_normalized(q, k, v, decay, o, "elu1", w.block, ws_n, stream))
    ms_f = timed(lambda: la2.la2_forward(q, k, v, decay, o, w.block, ws_f, stream))
    # the backward of the same normalized forward (o from it), reusing its workspace, and recomputing
    do = x["do"].to(dev)
    ws_b = la2.normalized_workspace_for(q, v, "elu1", w.block, True)
    la2.la2_forward_normalized(q, k, v, decay, o, "elu1", w.block, ws_b, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ms_b = timed(lambda: la2.la2_backward_normalized(q, k, v, decay, o, do, dq, dk, dv, "elu1", w.block, ws_b,
                                                     stream, saved=True))
    ws_r = la2.normalized_workspace_for(q, v, "elu1", w.block, True)
    ms_r = timed(lambda: la2.la2_backward_normalized(q, k, v, decay, o, do, dq, dk, dv, "elu1", w.block, ws_r,
                                                     stream))
    th = w.B * w.H * w.T
    byts = th * 4 * w.d * 2
    achieved = byts / (ms_n * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nb = 32
        ta = time.perf_counter()
        oracle.forward_normalized(*(x[n][:nb].double().numpy() for n in ("q", "k", "v")), None, "elu1")
        tc = time.perf_counter() - ta
        cpu = {"value": round(nb * w.T / tc, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"{nb} sequences x {w.H} heads x {w.T} tokens, fp64, {tc:.1f} s",
               "host": host_info()}
    print(json.dumps({
        "metric": "normalized forward tokens/sec (phi = elu + 1, numerator / denominator)",
        "value": round(w.B * w.T / (ms_n * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": max(args.warmup, 1) * 3, "ms_per_step": round(ms_n, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B}, H={w.H}, T={w.T}, d=d_v={w.d}, T_B={w.block}, no decay",
                   "parallelism": "none (1 GPU)"},
        "plain_forward_ms": round(ms_f, 5),
        "plain_forward_tokens_per_s": round(w.B * w.T / (ms_f * 1e-3), 1),
        "backward_ms": round(ms_b, 5),
        "backward_recomputing_ms": round(ms_r, 5),
        "fwd_bwd_tokens_per_s": round(w.B * w.T / ((ms_n + ms_b) * 1e-3), 1),
        "backward_hbm_frac": round(th * 7 * w.d * 2 / (ms_b * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_of("nfwd"),
                     "kernel": "fwd1_bf16_kernel, elu + 1 instance (one launch: phi on the tiles, numerator and "
                               "denominator together, each row divided before it is rounded)",
                     "avg_launch_ms": round(ms_n, 5), "algorithmic_bytes_per_launch": byts},
        "cpu_baseline": cpu,
    }), flush=True)


def compare_bench(args):
    """Wall clock of three ways to attend causally over the same tokens, at 131,072 tokens per batch
    (B = 128K / T), H = 12 heads, d = d_v = 128, bf16, seeded N(0, 1/d) inputs, no decay -- the shape
    of the pages' comparison of the tiled scan with a FlashAttention kernel and with the serial
    recurrence, on this GPU:
      lightning: la2_forward (+ la2_backward_saved), T_B = 128;
      serial:    la2_forward_serial, the recurrence one position after another (forward only);
      softmax:   torch.nn.functional.scaled_dot_product_attention(is_causal=True) on the flash or
                 memory-efficient backend (the math backend is never allowed), forward and
                 forward + backward through autograd.
    Each timing is the median of 3 measurements, each of back-to-back calls covering about 20 ms
    (at least one call), after at least 3 warm-up calls and 50 ms of work; HIP events on the current
    stream."""
    import torch
    import causal_linear_attention_amd as la2
    from torch.nn.attention import SDPBackend, sdpa_kernel
    dev = torch.device("cuda:0")
    H, d, tokens = 12, 128, 131072
    stream = torch.cuda.current_stream()

    def t_ms(fn, reps=3):
        # warm-up: at least 3 calls and about 50 ms of GPU work, so that the clocks have settled;
        # then `reps` measurements of back-to-back calls (about 20 ms of work each, at least one
        # call), median of the per-call times
        t0, n = time.perf_counter(), 0
        while n < 3 or time.perf_counter() - t0 < 0.05:
            fn()
            torch.cuda.synchronize()
            n += 1
        calls = max(1, int(0.02 / max((time.perf_counter() - t0) / n, 1e-6)))
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / calls)
        return sorted(out)[len(out) // 2]

    backend = None
    curves = []
    for tk in [float(x) for x in args.compare_points.split(",")]:
        T = int(tk * 1024)
        B = tokens // T
        g = torch.Generator().manual_seed(17 + T)
        q, k, v, do = [(torch.randn((B, H, T, d), generator=g) / (math.sqrt(d) if i < 3 else 1.0)).to(torch.bfloat16)
                       .to(dev) for i in range(4)]
        row = {"T": T, "B": B}
        o = torch.empty_like(v)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = la2.workspace_for(q, v, 128, True)
        row["lightning_fwd_ms"] = round(t_ms(lambda: la2.la2_forward(q, k, v, None, o, 128, ws)), 4)
        row["lightning_fwd_bwd_ms"] = round(t_ms(lambda: (la2.la2_forward(q, k, v, None, o, 128, ws),
                                                          la2.la2_backward_saved(q, k, v, None, do, dq, dk, dv, 128,
                                                                                 ws))), 4)
        row["serial_fwd_ms"] = round(t_ms(lambda: la2.la2_forward_serial(q, k, v, None, o)), 4)
        print(f"[compare] T={T} lightning and serial timed", file=sys.stderr, flush=True)
        qg, kg, vg = (t.detach().clone().requires_grad_(True) for t in (q, k, v))
        for cand in ([SDPBackend.FLASH_ATTENTION], [SDPBackend.EFFICIENT_ATTENTION]) if backend is None else [backend]:
            try:
                with sdpa_kernel(cand):
                    row["softmax_fwd_ms"] = round(t_ms(lambda: torch.nn.functional.scaled_dot_product_attention(
                        q, k, v, is_causal=True)), 4)

                    def fb():
                        out = torch.nn.functional.scaled_dot_product_attention(qg, kg, vg, is_causal=True)
                        out.backward(do)
                    row["softmax_fwd_bwd_ms"] = round(t_ms(fb), 4)
                backend = cand
                break
            except RuntimeError as e:
                row["softmax_error"] = str(e).splitlines()[0][:200]
        if backend is not None:
            row.pop("softmax_error", None)
        for key in ("lightning_fwd_bwd_ms", "softmax_fwd_bwd_ms", "serial_fwd_ms", "lightning_fwd_ms", "softmax_fwd_ms"):
            if key in row:
                row[key.replace("_ms", "_tokens_per_s")] = round(B * T / (row[key] * 1e-3), 1)
        curves.append(row)
        print(f"[compare] T={T} done", file=sys.stderr, flush=True)
        del q, k, v, do, o, dq, dk, dv, ws, qg, kg, vg
        torch.cuda.empty_cache()
    last = curves[-1]
    print(json.dumps({
        "metric": "fwd+bwd tokens/sec vs T: tiled lightning scan vs causal softmax attention vs token-serial recurrence",
        "value": last.get("lightning_fwd_bwd_tokens_per_s"), "unit": "tokens/s", "n_gpus": 1,
        "steps": 3, "warmup": 3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "comparison: 131072 tokens per batch, H=12, d=d_v=128, no decay, T_B=128",
                   "softmax_backend": None if backend is None else str(backend[0]), "parallelism": "none (1 GPU)"},
        "curves": curves,
    }), flush=True)


def algorithmic(w):
    """Algorithmic bytes and flops of one forward and one backward over workload w (per call), as the
    pages count them: whole tiles of the requested T_B."""
    th = w.B * w.H * w.T                      # token-heads
    e = 2 if w.dtype == "bf16" else 4
    d = w.d
    tb = w.block
    return {
        "fwd_bytes": th * 4 * d * e,          # read q, k, v; write o
        "bwd_bytes": th * 7 * d * e,          # read q, k, v, do; write dq, dk, dv
        "fwd_flops": th * (4 * tb * d + 4 * d * d),
        "bwd_flops": th * (10 * tb * d + 10 * d * d),
        # the same products over the causal triangle only (diagonal included)
        "fwd_flops_causal": th * (2 * d * (tb + 1) + 4 * d * d),
        "bwd_flops_causal": th * (5 * d * (tb + 1) + 10 * d * d),
    }


def _segments(chains, T, tile):
    """(segments per chain, tiles per segment) of the library's plan at this tile length: chains that
    do not fill the 256 compute units are cut into min(256 // chains, tiles) segments."""
    nt = -(-T // tile)
    nseg = min(256 // chains, nt) if chains < 256 and nt > 1 else 1
    seg_tiles = -(-nt // max(nseg, 1))
    return -(-nt // seg_tiles), seg_tiles


def one_pass_backward(w):
    """True where la2_backward_saved runs the one-pass backward, and la2_forward the producer/consumer
    scan over 64-position tiles: no decay, bf16, d = d_v = 128."""
    return not w.decay and w.dtype == "bf16" and w.d == 128 and w.dv == 128


def executed(w):
    """MFMA flops the bf16 kernels execute for one forward and one training-step backward
    (la2_backward_saved) over workload w (d = d_v): score and output products over the causal 32 x 32
    blocks of the tiles the kernels actually run (without decay at d = 128 the forward and backward
    kernels run 64 positions, otherwise output scans min(max(T_B, 64), 128) and the backward kernels
    64), the inter products and state updates (2 d^2 each per token), and the state-only passes of
    split chains (2 d^2 per token of every segment whose state is needed)."""
    d, T, chains = w.d, w.T, w.B * w.H
    th = chains * T
    tf = 64 if one_pass_backward(w) else min(max(w.block, 64), 128)
    nb = tf // 32
    intra_f = (nb + 1) * 32 * d * 2           # per token: Q K^T and P V over (nb + 1) / 2 blocks of 32
    tp = min(max(w.block, 64), 128)           # the plan's tile: segments are whole tiles of it
    nseg, seg_tiles = _segments(chains, T, tp)
    state_f = 2 * d * d * chains * min(T, (nseg - 1) * seg_tiles * tp) if nseg > 1 else 0
    fwd = th * (intra_f + 4 * d * d) + state_f
    causal64 = 3 * 2 * 32 * 32 * d // 64      # per token: one product over 3 causal 32 x 32 blocks of a 64-tile
    if one_pass_backward(w):
        # one reverse walk over 64-tiles: 2 score and 3 output products, 3 inter products, 2 state updates
        # (R and the undoing of S); the reverse state-only pass over every segment but the first
        state_b = 2 * d * d * chains * max(0, T - seg_tiles * tp) if nseg > 1 else 0
        bwd = th * (5 * causal64 + 10 * d * d) + state_b
    else:
        # dQ = forward scan of (do, v, k) reusing the forward's states; fused dK/dV over 64-tiles:
        # 2 score and 2 output products, 2 inter products, 1 state update
        nseg64, seg64 = _segments(chains, T, 64)
        state_b = 2 * d * d * chains * max(0, T - seg64 * 64) if nseg64 > 1 else 0
        bwd = th * (intra_f + 4 * d * d) + th * (4 * causal64 + 6 * d * d) + state_b
    return {"fwd_flops_executed": fwd, "bwd_flops_executed": bwd}


def host_info():
    model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                 "unknown CPU")
    return f"{model}, {os.cpu_count()} logical CPUs"


def oracle_rate(x, nb, nh, backward, threads=None):
    """Token-heads per second of the C oracle (fp64 token recurrence) on the first nb sequences and nh
    heads of workload inputs x, forward (+ backward)."""
    import oracle
    sub = lambda t: t[:nb, :nh].double().numpy()
    q, k, v = (sub(x[n]) for n in ("q", "k", "v"))
    lam = None if x["decay"] is None else x["decay"][:nh].double().numpy()
    before = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    used = oracle.num_threads()
    try:
        ta = time.perf_counter()
        oracle.forward(q, k, v, lam)
        if backward:
            oracle.backward(q, k, v, sub(x["do"]), lam)
        tc = time.perf_counter() - ta
    finally:
        oracle.set_num_threads(before)
    return nb * nh * x["workload"].T / tc, tc, used


def cpu_baseline(x, nb, nh, backward, one_thread=None):
    """The oracle as it stands on a bounded sample of workload x, all host threads, reported as tokens/s over
    all H heads; `one_thread` = (nb, nh) of a smaller sample timed on one thread."""
    w = x["workload"]
    rate, tc, used = oracle_rate(x, nb, nh, backward)
    what = "forward + backward" if backward else "forward"
    out = {"value": round(rate / w.H, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{nb} sequence(s) x {nh} of {w.H} heads x {w.T} tokens of {w.name}, {what}, fp64 token "
                     f"recurrence, {tc:.1f} s",
           "host": host_info()}
    if one_thread:
        r1, t1, _ = oracle_rate(x, one_thread[0], one_thread[1], backward, threads=1)
        out["one_thread"] = {"value": round(r1 / w.H, 1), "unit": "tokens/s",
                             "sample": f"{one_thread[0]} sequence(s) x {one_thread[1]} heads, {t1:.1f} s"}
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stream:
        stream_bench(args)
        return
    if args.cache_probe:
        cache_probe_bench(args)
        return
    if args.decode:
        decode_bench(args)
        return
    if args.normalized:
        normalized_bench(args)
        return
    if args.compare:
        compare_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); "
              "chains shard across GPUs with no communication, but no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import causal_linear_attention_amd as la2
    from causal_linear_attention_amd import inputs

    dev = torch.device("cuda:0")
    names = inputs.SWEEP_NAMES
    if args.workload:
        if args.workload not in inputs.WORKLOADS:
            print(f"bench.py: unknown workload {args.workload!r}", file=sys.stderr)
            sys.exit(2)
        names = [args.workload]
    elif args.points != "all":
        want = {int(p) for p in args.points.split(",")}
        names = [n for n in names if inputs.WORKLOADS[n].T // 1024 in want]

    # ---- inputs resident in HBM --------------------------------------------
    cases = []
    for n in names:
        x = inputs.make(n)
        w = x["workload"]
        q, k, v = (x[t].to(dev) for t in ("q", "k", "v"))
        do = x["do"].to(dev) if w.backward else None
        decay = None if x["decay"] is None else x["decay"].to(dev)
        ws_n = max(la2.la2_workspace_bytes(w.B, w.H, w.T, w.d, w.dv, w.block, q.dtype, b) for b in (0, 1))
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
        o = torch.empty_like(v)
        dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if w.backward else (None,) * 3
        cases.append(dict(w=w, q=q, k=k, v=v, do=do, decay=decay, ws=ws, o=o, dq=dq, dk=dk, dv=dv,
                          host=x if ((w.T == 1024 or args.workload) and not args.no_cpu_baseline) else None))
        print(f"[bench] {w.name}: B={w.B} T={w.T} workspace={ws_n} B", file=sys.stderr, flush=True)
        del x
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # Dominant kernel: at the 1K point (2048 chains fill the GPU, no chain is split) la2_forward is one
    # launch of the forward output scan and la2_backward_saved one launch of its backward kernel (the
    # one-pass backward without decay), so the event times around the two calls are those launches.
    dom = next((i for i, c in enumerate(cases) if c["w"].backward and c["w"].dtype == "bf16"
                and _segments(c["w"].B * c["w"].H, c["w"].T, 128)[0] == 1), None)

    def step(record=None, only=None):
        for i, c in enumerate(cases):
            ev = record[i] if record is not None and (only is None or i == only) else None
            if ev:
                ev[0].record(stream)
            la2.la2_forward(c["q"], c["k"], c["v"], c["decay"], c["o"], c["w"].block, c["ws"], stream)
            if ev:
                ev[1].record(stream)
            # the training step's backward: reuses the segment states la2_forward left in the workspace
            if c["w"].backward:
                la2.la2_backward_saved(c["q"], c["k"], c["v"], c["decay"], c["do"], c["dq"], c["dk"], c["dv"],
                                       c["w"].block, c["ws"], stream)
            if ev:
                ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-length forward / backward split: an instrumented pass of the same steps (events around every
    # call), outside the timed region
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in cases] for _ in range(args.steps)]
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    fwd_ms = [sum(events[s_][i][0].elapsed_time(events[s_][i][1]) for s_ in range(args.steps)) / args.steps
              for i in range(len(cases))]
    bwd_ms = [sum(events[s_][i][1].elapsed_time(events[s_][i][2]) for s_ in range(args.steps)) / args.steps
              for i in range(len(cases))]

    # the timed region: K steps; HIP events only around the dominant kernel's launch
    dom_events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in cases]
                  for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(dom_events[s_] if dom is not None else None, only=dom)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if dom is not None:
        dom_fwd_ms = sum(dom_events[s_][dom][0].elapsed_time(dom_events[s_][dom][1])
                         for s_ in range(args.steps)) / args.steps
        dom_bwd_ms = sum(dom_events[s_][dom][1].elapsed_time(dom_events[s_][dom][2])
                         for s_ in range(args.steps)) / args.steps

    tokens_per_step = sum(c["w"].tokens for c in cases)
    value = tokens_per_step * args.steps / wall
    sweep = {}
    for c, f, b in zip(cases, fwd_ms, bwd_ms):
        w = c["w"]
        alg = algorithmic(w)
        alg.update(executed(w))
        if not w.backward:
            b = 0.0
            for key in ("bwd_bytes", "bwd_flops", "bwd_flops_causal", "bwd_flops_executed"):
                alg[key] = 0
        t = (f + b) * 1e-3
        byts, flops = alg["fwd_bytes"] + alg["bwd_bytes"], alg["fwd_flops"] + alg["bwd_flops"]
        peak_flops = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS) * 1e12
        sweep[f"T={w.T}"] = {
            "B": w.B, "fwd_ms": round(f, 4), "bwd_ms": round(b, 4) if w.backward else None,
            "tokens_per_s": round(w.tokens / t, 1),
            "fwd_GBs": round(alg["fwd_bytes"] / (f * 1e-3) / 1e9, 1),
            "bwd_GBs": round(alg["bwd_bytes"] / (b * 1e-3) / 1e9, 1) if w.backward else None,
            "fwd_bwd_TFLOPs": round(flops / t / 1e12, 1),
            "fwd_bwd_TFLOPs_causal": round((alg["fwd_flops_causal"] + alg["bwd_flops_causal"]) / t / 1e12, 1),
            "hbm_frac": round(byts / t / (PEAK_HBM_GBS * 1e9), 4),
            # MFMA utilisation from the flops the kernels execute (causal blocks at the tile they run)
            "mfma_frac": round((alg["fwd_flops_executed"] + alg["bwd_flops_executed"]) / t / peak_flops, 4),
            # the same from the pages' count (whole tiles of the requested T_B)
            "mfma_frac_nominal": round(flops / t / peak_flops, 4),
            # t_roof / t_measured, t_roof = max(algorithmic bytes / peak HBM, algorithmic flops / peak MFMA)
            "roofline_frac": round(max(byts / (PEAK_HBM_GBS * 1e9), flops / peak_flops) / t, 4),
        }
        if byts <= (256 << 20):
            sweep[f"T={w.T}"]["cache_resident"] = True   # inputs and outputs fit the 256 MiB memory-side cache
    tps = [v["tokens_per_s"] for v in sweep.values()]

    roofline = None
    traffic = traffic_of

    if dom is not None:
        w = cases[dom]["w"]
        alg, ex = algorithmic(w), executed(w)
        fwd_gbs = alg["fwd_bytes"] / (dom_fwd_ms * 1e-3) / 1e9
        fwd_tf = ex["fwd_flops_executed"] / (dom_fwd_ms * 1e-3) / 1e12
        forward_kernel = {
            "kernel": "fwd1_bf16_kernel (forward output scan over 64-position tiles, writing each chain's final "
                      "state)",
            "avg_launch_ms": round(dom_fwd_ms, 4), "achieved_GBs": round(fwd_gbs, 1),
            "frac": round(fwd_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": alg["fwd_bytes"],
            "traffic": traffic("fwd"), "mfma_TFLOPs": round(fwd_tf, 1),
            "mfma_frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        }
        if one_pass_backward(w):
            achieved = alg["bwd_bytes"] / (dom_bwd_ms * 1e-3) / 1e9
            bwd_tf = ex["bwd_flops_executed"] / (dom_bwd_ms * 1e-3) / 1e12
            roofline = {
                "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic("bwd1"),
                "kernel": "bwd1_bf16_kernel (one-pass backward: dq, dk, dv from q, k, v, dout and the final state)",
                "launch": f"la2_backward_saved at T={w.T}, B={w.B}: one launch per call",
                "avg_launch_ms": round(dom_bwd_ms, 4),
                "algorithmic_bytes_per_launch": alg["bwd_bytes"],
                # MFMA rate from the flops the launch executes (causal 32 x 32 blocks of its 64-position tiles)
                "mfma_TFLOPs": round(bwd_tf, 1), "mfma_frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "mfma_frac_nominal": round(alg["bwd_flops"] / (dom_bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "forward_kernel": forward_kernel,
            }
        else:
            roofline = {
                "bound": "hbm", "achieved": forward_kernel["achieved_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": forward_kernel["frac"], "traffic": forward_kernel["traffic"],
                "kernel": forward_kernel["kernel"], "launch": f"la2_forward at T={w.T}, B={w.B}: one launch per call",
                "avg_launch_ms": forward_kernel["avg_launch_ms"],
                "algorithmic_bytes_per_launch": alg["fwd_bytes"],
                "mfma_TFLOPs": forward_kernel["mfma_TFLOPs"], "mfma_frac": forward_kernel["mfma_frac"],
            }

    cpu = None
    hostc = next((c for c in cases if c["host"] is not None), None)
    if hostc is not None:
        x = hostc["host"]
        w = x["workload"]
        if not args.workload:
            # the 1K point: up to --cpu-sample-seqs sequences, all heads
            cpu = cpu_baseline(x, min(args.cpu_sample_seqs, w.B), w.H, True, one_thread=(4, w.H))
        elif w.T * w.B * w.H <= (1 << 20):
            cpu = cpu_baseline(x, w.B, w.H, w.backward, one_thread=(1, min(w.H, 4)))
        else:
            # long sequences: a few heads of the first sequence
            cpu = cpu_baseline(x, 1, min(w.H, 8), w.backward)

    out = {
        "metric": METRIC if all(c["w"].backward for c in cases) else "forward tokens/sec on 1 MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if any(c["w"].dtype == "f32" for c in cases) else "bf16", "data": "synthetic",
        "config": ({
            "workload": "fixed-token length sweep: 131072 tokens per batch at (B,T) in "
                        + ",".join(f"({c['w'].B},{c['w'].T})" for c in cases)
                        + "; H=16, d=d_v=128, T_B=128, no decay; one step = fwd+bwd over every batch",
            "tokens_per_step": tokens_per_step, "heads": 16, "d": 128, "d_v": 128, "block": 128,
            "parallelism": "none (1 GPU)",
        } if not args.workload else {
            "workload": f"{cases[0]['w'].name}: B={cases[0]['w'].B}, H={cases[0]['w'].H}, T={cases[0]['w'].T}, "
                        f"d=d_v={cases[0]['w'].d}, T_B={cases[0]['w'].block}, "
                        f"{'per-head decay' if cases[0]['w'].decay else 'no decay'}"
                        f"{', 1% outlier rows x8' if cases[0]['w'].outlier_frac else ''}; one step = "
                        f"{'fwd+bwd' if cases[0]['w'].backward else 'fwd'}",
            "tokens_per_step": tokens_per_step, "heads": cases[0]["w"].H, "d": cases[0]["w"].d,
            "d_v": cases[0]["w"].dv, "block": cases[0]["w"].block, "parallelism": "none (1 GPU)",
        }),
        "sweep": sweep,
        "flatness": round(min(tps) / max(tps), 4) if tps else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
