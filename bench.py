"""Benchmark of the Mamba2 SSD hot path on one MI355X.

One step = one pass over every stage of the path on synthetic inputs:
  1. chunked-scan prefill of 256 sequences x 2048 tokens (H=32, G=1, P=64,
     N=128, chunk 256, bf16 x/dt/B/C/y, fp32 state), boundary states out;
  2. boundary commit of those sequences into an exact-replay cache;
  3. R exact-replay decode steps over a batch of 256 sequences whose caches
     hold a boundary state plus 0..255 buffered tokens (chunk 256);
  4. R recurrent state-update steps over the same batch (comparison path);
  5. R exact-replay decode steps with chunk 16 (refresh every 16 tokens).
Inputs are resident in HBM before timing starts. Every stage is timed with
HIP events on the stream the library launches on. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps R]

Counter runs: `--prefill-only` launches only the prefill (W + K times) and
then one plain 512 MiB device copy, whose FETCH_SIZE / WRITE_SIZE readings
scale the prefill's; `--traffic FETCH.csv WRITE.csv` turns the two rocprofv3
counter files into profiles/prefill_w1b_traffic.json (no GPU needed).
`--decode-only` does the same for the exact-replay decode at B=256, chunk 256
((W + K) x R steps), and `--decode-traffic FETCH.csv WRITE.csv` writes
profiles/decode_b256_q256_traffic.json: each decode dispatch's counted bytes
against its algorithmic bytes (the buffer fills of every step are known).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD prefill tokens/s + replay-decode steps/s at B=256; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
PAGE_TOKENS = 64             # rows per buffer page in the paged replay-decode leg
BF16_MFMA_PEAK_TFLOPS = 2500.0
# MI355X fp32 vector peak without packed fp32 (the library is built with
# packed fp32 instructions off, which halves the 157.3 TFLOP/s packed figure)
FP32_VALU_PEAK_TFLOPS = 78.6
KERNEL_SOURCES = ["ssd_device.hpp", "ssd_scalar.hip", "ssd_mfma.hip", "ssd_api.cpp",
                  "ssd_internal.hpp", "ssd_conv.hip", "ssd_scratch.hip"]   # (not the probe)
W1A_COPIES = 48              # input copies the 1 x 2048 latency leg rotates through
CONV_W = 4                   # conv kernel width of the conv legs
SPEC_BATCH, SPEC_T = 512, 4  # speculative verification: sequences, drafts each
RECOVER_T = 255              # packed-history recovery: generated tokens replayed


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_replay_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_bytes(T, S, H, G, P, N, io=2, dtb=2):
    """Algorithmic HBM bytes of one prefill launch: read x, dt, B, C once,
    write y and the per-sequence fp32 boundary state."""
    return T * H * P * io * 2 + T * H * dtb + 2 * T * G * N * io + S * H * P * N * 4


def prefill_flops(T, H, G, P, N, Q):
    """Algorithmic flops (2 per MAC, causal half): per token and head
    (Q+1)P for the intra-chunk product and 4NP for chunk state and the
    state read-out; per token and group (Q+1)N for C.B^T."""
    return T * (H * ((Q + 1) * P + 4 * N * P) + G * (Q + 1) * N)


def replay_step_bytes(ks, Q, H, G, P, N, io=2, dtb=2, with_C=False):
    """Algorithmic bytes of one replay-decode step for buffer fills ks: the
    bf16 copy of the boundary state (the read-out operand), the buffered
    tokens' x, B and raw dt, the new token, its append and y; when the token
    fills the chunk, the chunk-state update reads the fp32 state and the
    chunk's tokens and writes the new state and its bf16 copy."""
    ks = np.asarray(ks, dtype=np.int64)
    state_bf = H * P * N * 2
    per_buf_tok = H * P * io + G * N * io + H * dtb          # x, B, raw dt re-read
    new_tok = H * P * io + H * dtb + 2 * G * N * io          # inputs
    append = H * P * io + H * dtb + G * N * io * (2 if with_C else 1)
    y = H * P * io
    commits = int(np.sum(ks + 1 == Q))
    # a commit reads the fp32 state and the chunk's Q buffered tokens, and
    # writes the new fp32 state and its bf16 copy
    return int(len(ks) * (state_bf + new_tok + append + y) + ks.sum() * per_buf_tok
               + commits * (H * P * N * (4 + 4 + 2) + Q * per_buf_tok))


def conv_prefill_bytes(T, S, cd, W, io=2):
    """Algorithmic bytes of one conv prefill launch: read xBC once, write
    x | B | C once, read and write each sequence's conv state, read the taps
    and bias."""
    return 2 * T * cd * io + 2 * S * cd * (W - 1) * io + cd * (W + 1) * 4


def conv_update_bytes(batch, cd, W, io=2):
    """One conv decode step: the token's xBC in, x | B | C out, the conv
    state read and written, the taps and bias."""
    return batch * (2 * cd * io + 2 * cd * (W - 1) * io) + cd * (W + 1) * 4


def verify_step_bytes(ks, T, Q, H, G, P, N, io=2, dtb=2):
    """One speculative verification of T drafts per sequence with ks
    committed tokens: the state read-out operand (bf16 copy, or the fp32
    state when the drafts cross the chunk end), the committed rows' x, B and
    raw dt, the drafts' x, dt, B, C and their outputs."""
    ks = np.asarray(ks, dtype=np.int64)
    cross = ks + T > Q
    state = np.where(cross, H * P * N * 4, H * P * N * 2)
    per_buf_tok = H * P * io + G * N * io + H * dtb
    draft = H * P * io + H * dtb + 2 * G * N * io + H * P * io
    return int(state.sum() + ks.sum() * per_buf_tok + len(ks) * T * draft)


def accept_step_bytes(ks, acc, Q, H, G, P, N, io=2, dtb=2):
    """Committing acc drafts per sequence: read and append them; a chunk that
    fills reads the fp32 state and the chunk's rows and writes the state and
    its bf16 copy."""
    ks, acc = np.asarray(ks, dtype=np.int64), np.asarray(acc, dtype=np.int64)
    per_tok = H * P * io + G * N * io + H * dtb
    fills = (ks + acc) >= Q
    commit = H * P * N * (4 + 4 + 2) + Q * per_tok
    return int(2 * acc.sum() * per_tok + fills.sum() * commit)


def recovery_bytes(S, T, H, G, P, N, io=2, dtb=2, sb=4):
    """Packed-history recovery of T tokens for S sequences: each state read
    and written once (cache dtype, sb bytes), every token's x, dt, B, C read
    and y written."""
    return S * 2 * H * P * N * sb + S * T * (2 * H * P * io + H * dtb + 2 * G * N * io)


def ssu_step_bytes(batch, H, G, P, N, io=2, dtb=2):
    return batch * (2 * H * P * N * 4 + 2 * H * P * io + H * dtb + 2 * G * N * io)


def load_traffic(sha):
    """HBM traffic per prefill launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "prefill_w1b_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


CALIB_BYTES = 512 * 2 ** 20
PREFILL_KERNEL = "k_scan_mfma<64, 128, ssd::IoBF16, false, false>"
COPY_KERNEL = "copyBuffer"
DECODE_KERNEL = "k_decode_mfma<64, 128, ssd::IoBF16, false, true>"


def counter_means(path, counter):
    """Per-dispatch value of one counter for the prefill kernel (mean over its
    dispatches) and for the calibration copy (the largest copy dispatch: the
    run's other copies are small host-to-device transfers), from a rocprofv3
    *_counter_collection.csv file."""
    vals = {"prefill": [], "copy": []}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            key = "prefill" if PREFILL_KERNEL in name else "copy" if COPY_KERNEL in name else None
            if key:
                vals[key].append(float(row["Counter_Value"]))
    if not vals["prefill"] or not vals["copy"]:
        raise SystemExit(f"{path}: no {counter} rows for the prefill kernel and the copy")
    return {"prefill": sum(vals["prefill"]) / len(vals["prefill"]), "copy": max(vals["copy"])}


def write_traffic(fetch_csv, write_csv, cmds, out=None):
    S, T, H, G, P, N = 256, 2048, 32, 1, 64, 128
    f = counter_means(fetch_csv, "FETCH_SIZE")
    w = counter_means(write_csv, "WRITE_SIZE")
    ff = CALIB_BYTES / 1024 / f["copy"]          # bytes a copy reads, over what the counter says
    wf = CALIB_BYTES / 1024 / w["copy"]
    traffic = 1024 * (f["prefill"] * ff + w["prefill"] * wf)
    rec = {
        "what": "HBM traffic of one prefill launch on 256 sequences x 2048 tokens (H=32, G=1, "
                "P=64, N=128, chunk 256, bf16 I/O, fp32 state), kernel " + PREFILL_KERNEL,
        "commands": cmds,
        "fetch_kib_per_dispatch": f["prefill"], "write_kib_per_dispatch": w["prefill"],
        "copy_calibration": {"bytes": CALIB_BYTES, "fetch_kib": f["copy"],
                             "write_kib": w["copy"], "fetch_factor": ff, "write_factor": wf},
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": prefill_bytes(S * T, S, H, G, P, N),
        "kernel_source_sha": kernel_source_sha(),
    }
    out = out or os.path.join(ROOT, "profiles", "prefill_w1b_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))
    return rec



def decode_counters(path, counter):
    """Per-dispatch values of one counter for the decode kernel (in dispatch
    order) and the calibration copy's reading, from a rocprofv3
    *_counter_collection.csv file of a --decode-only run."""
    dec, copy = [], []
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            if DECODE_KERNEL in name:
                dec.append((int(row["Dispatch_Id"]), float(row["Counter_Value"])))
            elif COPY_KERNEL in name:
                copy.append(float(row["Counter_Value"]))
    if not dec or not copy:
        raise SystemExit(f"{path}: no {counter} rows for the decode kernel and the copy")
    return [v for _, v in sorted(dec)], max(copy)


def write_decode_traffic(fetch_csv, write_csv, cmds, out=None):
    S, H, G, P, N, Q = 256, 32, 1, 64, 128, 256
    from exact_replay_decode_amd import synth   # seeded inputs only (no GPU)
    f, fc = decode_counters(fetch_csv, "FETCH_SIZE")
    w, wc = decode_counters(write_csv, "WRITE_SIZE")
    if len(f) != len(w):
        raise SystemExit("the two counter runs hold different numbers of decode dispatches")
    ff = CALIB_BYTES / 1024 / fc
    wf = CALIB_BYTES / 1024 / wc
    k0 = synth.replay_prefix_lengths(S, Q, 1) % Q
    alg = np.array([replay_step_bytes((k0 + i) % Q, Q, H, G, P, N) for i in range(len(f))],
                   dtype=np.float64)
    traffic = 1024 * (np.array(f) * ff + np.array(w) * wf)
    fills = np.array([int(np.sum((k0 + i) % Q == Q - 1)) for i in range(len(f))])
    rec = {
        "what": "HBM traffic of the exact-replay decode kernel, B=256 (H=32, G=1, P=64, N=128, "
                "chunk 256, bf16 I/O, fp32 state), buffers holding 0..255 tokens, kernel "
                + DECODE_KERNEL + " (the chunk-state update of the filling slots inside)",
        "commands": cmds,
        "dispatches": len(f),
        "fetch_kib_per_dispatch_mean": float(np.mean(f)),
        "write_kib_per_dispatch_mean": float(np.mean(w)),
        "copy_calibration": {"bytes": CALIB_BYTES, "fetch_kib": fc, "write_kib": wc,
                             "fetch_factor": ff, "write_factor": wf},
        "traffic_bytes_per_dispatch_mean": float(traffic.mean()),
        "algorithmic_bytes_per_dispatch_mean": float(alg.mean()),
        "traffic_over_algorithmic": float(traffic.sum() / alg.sum()),
        "traffic_over_algorithmic_without_fill": float(
            traffic[fills == 0].sum() / alg[fills == 0].sum()) if (fills == 0).any() else None,
        "kernel_source_sha": kernel_source_sha(),
    }
    out = out or os.path.join(ROOT, "profiles", "decode_b256_q256_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))
    return rec

STACK_LAYERS = 24            # layer-stack leg: layers, prompt, decode steps, chunk calls
STACK_PROMPT, STACK_STEPS, STACK_CHUNK, STACK_CHUNKS = 600, 32, 100, 9
GROUPED_PACK, GROUPED_COPIES = (600, 300, 900, 248), 64


def other_workloads(erd, synth, torch, dev, warmup, steps):
    """Further measurement workloads (a latency case, grouped heads and a
    layer stack), each timed with HIP events on the launch stream after its
    own warm-up:
      - prefill latency of one 2048-token sequence (H=32, G=1, P=64, N=128,
        chunk 256; launch-bound: 32 workgroups);
      - prefill throughput of the grouped-heads pack {600, 300, 900, 248} x 64
        (256 sequences, 131,072 tokens; H=64, G=8, P=64, N=128, chunk 256);
      - a 24-layer stack at batch 1 (H=24, G=1, P=64, N=128, chunk 256): per
        layer a 600-token exact-replay prefill, then decode steps of all 24
        layers (launched one by one, and from a captured HIP graph), then 900
        more tokens as 100-token chunked-prefill calls."""
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n   # seconds per call

    out = {}
    # W1a: one sequence. The launches rotate through W1A_COPIES copies of the
    # inputs and outputs (about 0.45 GB), more than the last-level cache
    # holds, so each launch reads its inputs from HBM.
    H, G, P, N, Q, T = 32, 1, 64, 128, 256, 2048
    sh = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 0)
    A, D, bias = (torch.from_numpy(v).to(dev) for v in (hp.A, hp.D, hp.dt_bias))
    copies = []
    for i in range(W1A_COPIES):
        xi, dti, Bi, Ci = synth.make_tokens_torch(T, H, G, P, N, 7 + i, dev)
        copies.append((xi, dti, Bi, Ci, torch.empty_like(xi),
                       torch.empty((1, H, P, N), dtype=torch.float32, device=dev)))
    cu_host = synth.cu_seqlens([T])
    cu = torch.from_numpy(cu_host).to(dev)
    rot = [0]

    def w1a():
        xi, dti, Bi, Ci, yi, bi = copies[rot[0] % W1A_COPIES]
        rot[0] += 1
        erd.ssd_prefill_varlen(sh, cu, xi, dti, A, Bi, Ci, D, bias, y=yi, boundary_state=bi,
                               cu_seqlens_host=cu_host, want_final=False)

    t = timed(w1a, max(steps, W1A_COPIES))
    out["prefill_1x2048"] = {"us_per_launch": 1e6 * t, "tokens_per_s": T / t,
                             "hbm_frac": prefill_bytes(T, 1, H, G, P, N) / t / 1e9 / HBM_PEAK_GBS,
                             "input_copies_rotated": W1A_COPIES}
    del copies

    # W2: grouped heads, pack x 64
    H, G = 64, 8
    sh = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 1)
    A, D, bias = (torch.from_numpy(v).to(dev) for v in (hp.A, hp.D, hp.dt_bias))
    lens = list(GROUPED_PACK) * GROUPED_COPIES
    T = sum(lens)
    x, dt, B, C = synth.make_tokens_torch(T, H, G, P, N, 8, dev)
    cu_host = synth.cu_seqlens(lens)
    cu = torch.from_numpy(cu_host).to(dev)
    y = torch.empty_like(x)
    bnd = torch.empty((len(lens), H, P, N), dtype=torch.float32, device=dev)
    t = timed(lambda: erd.ssd_prefill_varlen(sh, cu, x, dt, A, B, C, D, bias, y=y,
                                             boundary_state=bnd, cu_seqlens_host=cu_host,
                                             want_final=False), steps)
    gb = prefill_bytes(T, len(lens), H, G, P, N)
    out["prefill_grouped_pack_x64"] = {"ms_per_launch": 1e3 * t, "tokens_per_s": T / t,
                                       "hbm_gbs": gb / t / 1e9,
                                       "hbm_frac": gb / t / 1e9 / HBM_PEAK_GBS,
                                       "sequences": len(lens), "tokens": T}
    del x, dt, B, C, y, bnd

    # W4: 24-layer stack at batch 1
    H, G, L = 24, 1, STACK_LAYERS
    sh = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    ndec = (warmup + steps) * STACK_STEPS
    ntok = STACK_PROMPT + ndec + STACK_CHUNK * (warmup + STACK_CHUNKS)
    layers = []
    for li in range(L):
        hp = synth.make_head_params(H, 100 + li)
        prm = tuple(torch.from_numpy(v).to(dev) for v in (hp.A, hp.D, hp.dt_bias))
        toks = synth.make_tokens_torch(ntok, H, G, P, N, 100 + li, dev)
        cache = erd.ReplayCache(sh, 1, dev)
        erd.ssd_replay_prefill(sh, cache, [0, STACK_PROMPT], *(v[:STACK_PROMPT] for v in toks),
                               *prm)
        plan = erd.DecodePlan(sh, 1, *prm, cache=cache)
        layers.append((prm, toks, cache, plan))
    yd = torch.empty((1, H, P), dtype=torch.bfloat16, device=dev)
    pos = [STACK_PROMPT]

    def decode_step():
        p0 = pos[0]
        for prm, (x, dt, B, C), cache, plan in layers:
            plan(x[p0:p0 + 1], dt[p0:p0 + 1], B[p0:p0 + 1], C[p0:p0 + 1], yd)
        pos[0] = p0 + 1

    t_dec = timed(decode_step, steps * STACK_STEPS)
    chunk_cu = [0, STACK_CHUNK]

    def chunk_call():
        p0 = pos[0]
        for prm, toks, cache, plan in layers:
            erd.ssd_replay_prefill(sh, cache, chunk_cu, *(v[p0:p0 + STACK_CHUNK] for v in toks),
                                   *prm)
        pos[0] = p0 + STACK_CHUNK

    t_chunk = timed(chunk_call, STACK_CHUNKS)

    # the same 24-layer decode step captured once in a HIP graph and replayed
    # (the step needs no host-side metadata; the replays decode the captured
    # input buffers, which hold one token per layer)
    cs = torch.cuda.Stream()
    gplans = [erd.DecodePlan(sh, 1, *prm, cache=cache, stream=cs)
              for prm, toks, cache, plan in layers]
    gin = [tuple(v[pos[0]:pos[0] + 1].clone() for v in toks) for prm, toks, cache, plan in layers]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for gp, xs in zip(gplans, gin):
            gp(*xs, yd)
    t_graph = timed(graph.replay, steps * STACK_STEPS)
    out["layer_stack_24"] = {"decode_ms_per_step": 1e3 * t_dec,
                             "decode_us_per_layer": 1e6 * t_dec / L,
                             "decode_ms_per_step_hip_graph": 1e3 * t_graph,
                             "chunked_prefill_ms_per_100_tokens": 1e3 * t_chunk,
                             "layers": L, "heads": H, "batch": 1}
    return out


def fused_conv_decode(erd, synth, torch, dev, shape, S, R, warmup, steps, pre, cw, cbias, prm,
                      cd):
    """The conv's decode form and the replay decode step at B=256, chunk 256
    (the bench's decode workload): as one launch per step
    (ssd_replay_decode_conv) and as the two calls it replaces (conv update,
    then decode), each timed over steps x R steps after its own warm-up, on
    separate caches and conv states of the same contents."""
    A, D, bias = prm
    n = (warmup + steps) * R
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    px, pdt, pB, pC = synth.make_tokens_torch(int(pre.sum()), H, G, P, N, 1, dev)
    xbc = synth.make_xbc_torch(n * S, cd, 13, dev).view(n, S, cd)
    dts = synth.make_tokens_torch(n * S, H, G, P, N, 14, dev)[1].view(n, S, H)
    stream = torch.cuda.current_stream()
    out = {}
    for form in ("one_launch", "two_launches"):
        cache = erd.ReplayCache(shape, S, dev)
        erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), px, pdt, pB, pC, A, D, bias)
        cst = torch.zeros((S, cd, CONV_W - 1), dtype=torch.bfloat16, device=dev)
        x = torch.empty((S, H, P), dtype=torch.bfloat16, device=dev)
        Bt = torch.empty((S, G, N), dtype=torch.bfloat16, device=dev)
        Ct = torch.empty_like(Bt)
        y = torch.empty_like(x)
        if form == "one_launch":
            plan = erd.ConvDecodePlan(shape, S, A, cache, cw, cst, D, bias, bias=cbias)
            call = lambda k: plan(xbc[k], dts[k], x, Bt, Ct, y)  # noqa: E731
        else:
            cplan = erd.ConvUpdatePlan(shape, S, cw, cst, cbias)
            dplan = erd.DecodePlan(shape, S, A, D, bias, cache=cache)

            def call(k):
                cplan(xbc[k], x, Bt, Ct)
                dplan(x, dts[k], Bt, Ct, y)
        for k in range(warmup * R):
            call(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(warmup * R, n):
            call(k)
        e1.record(stream)
        torch.cuda.synchronize()
        out[form + "_us_per_step"] = 1e3 * e0.elapsed_time(e1) / (steps * R)
    out["batch"], out["chunk_size"], out["conv_width"] = S, shape.chunk_size, CONV_W
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(x, dt, B, C, hp, Q, T, target_s=10.0):
    """Time the fp64 oracle, as it is, on bounded samples of the workloads:
    the prefill (whole 2048-token sequences read back exactly from the
    device, all host threads; the headline figure), one 2048-token sequence
    on one thread, a sequence of each length of the grouped-heads pack, the
    B=256 decode step and the 24-layer stack's decode step at batch 1 (the
    last three from host-drawn inputs of the same distributions; a decode
    step is one token per sequence through the recurrence from a carried
    state)."""
    from exact_replay_decode_amd import synth, to_f64
    from oracle import scan, set_threads, threads

    def run(n):
        xs, dts = to_f64(x[:n * T]), to_f64(dt[:n * T])
        Bs, Cs = to_f64(B[:n * T]), to_f64(C[:n * T])
        cu = np.arange(n + 1, dtype=np.int64) * T
        t0 = time.perf_counter()
        scan(xs, dts, hp.A, Bs, Cs, cu, Q, D=hp.D, dt_bias=hp.dt_bias)
        return time.perf_counter() - t0

    cores = threads()
    t1 = run(1)
    n = int(max(1, min(x.shape[0] // T, round(target_s / max(t1, 1e-3)))))
    tn = run(n) if n > 1 else t1
    set_threads(1)
    try:
        t_single = run(1)
    finally:
        set_threads(cores)

    def host_scan(lengths, H, G, seed, init=False, reps=1):
        """Seconds per scan of host-drawn sequences of the given lengths
        (P=64, N=128, chunk 256), from carried states when init is set."""
        P, N = 64, 128
        hpp = synth.make_head_params(H, seed)
        tok = synth.concat([synth.make_tokens(L, H, G, P, N, seed, stream=i)
                            for i, L in enumerate(lengths)]).f64()
        h0 = (np.random.default_rng(seed).standard_normal((len(lengths), H, P, N)) * 0.1
              if init else None)
        cu = synth.cu_seqlens(lengths)
        t0 = time.perf_counter()
        for _ in range(reps):
            scan(*tok[:2], hpp.A, *tok[2:], cu, 256, D=hpp.D, dt_bias=hpp.dt_bias, init=h0)
        return (time.perf_counter() - t0) / reps

    # grouped pack: one sequence of each length (2048 tokens), H=64, G=8
    t_w2 = host_scan(list(GROUPED_PACK), 64, 8, 21)
    # decode at B=256 (H=32): 32 sequences x 1 token from carried states
    t_w3 = host_scan([1] * 32, 32, 1, 22, init=True, reps=4) * (256 / 32)
    # 24-layer stack at batch 1 (H=24): one layer's token, times 24
    t_w4 = host_scan([1], 24, 1, 23, init=True, reps=16) * STACK_LAYERS
    return {"value": n * T / tn, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of 256 sequences x {T} tokens of the prefill workload "
                      f"({tn:.1f} s, fp64 sequential recurrence, OpenMP over sequence x head)",
            "cpu": cpu_model(),
            "single_thread_1x2048": {"tokens_per_s": T / t_single, "cores": 1,
                                     "seconds": t_single},
            "grouped_pack": {"tokens_per_s": sum(GROUPED_PACK) / t_w2, "cores": cores,
                             "sample": "one sequence of each pack length (2048 tokens), "
                                       "H=64 G=8"},
            "decode_b256": {"steps_per_s": 1.0 / t_w3, "cores": cores,
                            "sample": "32 of 256 sequences x 1 token from carried states, "
                                      "4 repeats, scaled to 256"},
            "layer_stack_24": {"steps_per_s": 1.0 / t_w4, "cores": cores,
                               "sample": "one layer's decode token (H=24) from a carried "
                                         "state, 16 repeats, times 24 layers"}}


def copy_gbs(torch, dev, reps=5):
    """Device-to-device copy of CALIB_BYTES (read + write), GB/s: the
    measured ceiling for streaming kernels on this GPU."""
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * CALIB_BYTES * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return gbs


def read_gbs(torch, dev, reps=10):
    """A plain streaming read of 1 GiB (the probe kernel of libssd_probe.so),
    GB/s: the measured ceiling for read-dominated kernels on this GPU."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_replay_decode_amd", "libssd_probe.so"))
    lib.ssd_probe_stream_read.restype = ctypes.c_int
    lib.ssd_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p]
    nbytes, blocks = 1 << 30, 4096
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.ssd_probe_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                       stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ssd_probe_stream_read failed ({rc})")
    for _ in range(2):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf, sink
    return gbs


def load_decode_ratio(sha):
    """Counted over algorithmic bytes of the B=256 chunk-256 decode kernel,
    from the committed counter summary, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "decode_b256_q256_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("traffic_over_algorithmic")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill launches, then one 512 MiB calibration copy")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 counter files")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the B=256 chunk-256 decode steps, then the calibration copy")
    ap.add_argument("--decode-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the decode traffic summary from two rocprofv3 counter files")
    args = ap.parse_args()
    if args.decode_traffic:
        cmds = [f"cd /tmp && rocprofv3 --pmc {c} -f csv -d <out> -o run -- python3 "
                f"<repo>/bench.py --decode-only --steps 2 --warmup 1"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds.append("python3 bench.py --decode-traffic <fetch counter csv> <write counter csv>")
        write_decode_traffic(*args.decode_traffic, cmds)
        return
    if args.traffic:
        cmds = [f"cd /tmp && rocprofv3 --pmc {c} -f csv -d <out> -o run -- python3 "
                f"<repo>/bench.py --prefill-only --steps 1 --warmup 1"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds.append("python3 bench.py --traffic <fetch counter csv> <write counter csv>")
        write_traffic(*args.traffic, cmds)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan shards by sequence and head with no "
              "exchange, and no multi-GPU path is built (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_replay_decode_amd as erd
    from exact_replay_decode_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S, T, H, G, P, N, Q = 256, 2048, 32, 1, 64, 128, 256
    R = args.decode_steps
    total_decode = R * (args.steps + args.warmup)
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    shape16 = erd.Shape(H, G, P, N, 16, "bf16", "bf16")
    hp = synth.make_head_params(H, 0)
    A, D, bias = (torch.from_numpy(v).to(dev) for v in (hp.A, hp.D, hp.dt_bias))

    # ---- prefill workload (resident in HBM) ----
    x, dt, B, C = synth.make_tokens_torch(S * T, H, G, P, N, 0, dev)
    cu_host = synth.cu_seqlens([T] * S)
    cu = torch.from_numpy(cu_host).to(dev)
    y = torch.empty_like(x)
    bnd = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    commit_cache = erd.ReplayCache(shape, S, dev)

    if args.prefill_only:
        def launch():
            erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias, y=y, boundary_state=bnd,
                                   cu_seqlens_host=cu_host, want_final=False)
        for _ in range(args.warmup):
            launch()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        calib_dst = torch.empty_like(calib_src)
        torch.cuda.synchronize()
        calib_dst.copy_(calib_src)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"prefill_avg_launch_ms": ms, "steps": args.steps,
                          "achieved_gbs": prefill_bytes(S * T, S, H, G, P, N) / ms / 1e6,
                          "calibration_copy_bytes": CALIB_BYTES,
                          "kernel_source_sha": kernel_source_sha()}), flush=True)
        return

    # ---- decode workload: prefix 256 + k_i, then R*(K+W) decode tokens ----
    pre = synth.replay_prefix_lengths(S, Q, 1)
    px, pdt, pB, pC = synth.make_tokens_torch(int(pre.sum()), H, G, P, N, 1, dev)
    dx, ddt, dB, dC = synth.make_tokens_torch(total_decode * S, H, G, P, N, 2, dev)
    dx, ddt = dx.view(total_decode, S, H, P), ddt.view(total_decode, S, H)
    dB, dC = dB.view(total_decode, S, G, N), dC.view(total_decode, S, G, N)
    ydec = torch.empty((S, H, P), dtype=torch.bfloat16, device=dev)
    cu_pre = synth.cu_seqlens(pre)
    cache256 = erd.ReplayCache(shape, S, dev)
    cache16 = erd.ReplayCache(shape16, S, dev)
    # the same workload over paged buffers: pages of PAGE_TOKENS rows, every
    # slot's pages scattered over the pool
    npages = S * (Q // PAGE_TOKENS)
    cachepg = erd.ReplayCache(shape, S, dev, page_tokens=PAGE_TOKENS, num_pages=npages)
    perm = np.random.default_rng(0).permutation(npages).astype(np.int32)
    cachepg.buf_pages.copy_(torch.from_numpy(perm.reshape(S, Q // PAGE_TOKENS)))
    erd.ssd_replay_prefill(shape, cache256, cu_pre, px, pdt, pB, pC, A, D, bias)
    erd.ssd_replay_prefill(shape16, cache16, cu_pre, px, pdt, pB, pC, A, D, bias)
    erd.ssd_replay_prefill(shape, cachepg, cu_pre, px, pdt, pB, pC, A, D, bias)
    _, ssu_state, _ = erd.ssd_prefill_varlen(shape, cu_pre, px, pdt, A, pB, pC, D, bias,
                                             want_boundary=False)
    plan256 = erd.DecodePlan(shape, S, A, D, bias, cache=cache256)
    plan16 = erd.DecodePlan(shape16, S, A, D, bias, cache=cache16)
    planpg = erd.DecodePlan(shape, S, A, D, bias, cache=cachepg)
    plan_ssu = erd.DecodePlan(shape, S, A, D, bias, state=ssu_state)
    plan256.check(dx[0], ddt[0], dB[0], dC[0], ydec)
    if args.decode_only:
        # decode dispatch i sees buffer fills (pre % Q + i) % Q
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(total_decode):
            plan256(dx[k], ddt[k], dB[k], dC[k], ydec)
        e1.record(stream)
        torch.cuda.synchronize()
        calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        calib_dst = torch.empty_like(calib_src)
        torch.cuda.synchronize()
        calib_dst.copy_(calib_src)
        torch.cuda.synchronize()
        print(json.dumps({"decode_steps": total_decode,
                          "decode_avg_step_us": 1e3 * e0.elapsed_time(e1) / total_decode,
                          "calibration_copy_bytes": CALIB_BYTES,
                          "kernel_source_sha": kernel_source_sha()}), flush=True)
        return

    # conv before the scan (width CONV_W over x | B | C): prefill over the
    # same 256 x 2048 pack, decode steps at B=256
    cd = H * P + 2 * G * N
    cparams = synth.make_conv_params(cd, CONV_W, 11)
    cw = torch.from_numpy(cparams.weight).to(dev)
    cbias = torch.from_numpy(cparams.bias).to(dev)
    xbc = synth.make_xbc_torch(S * T, cd, 11, dev)
    cstate = torch.zeros((S, cd, CONV_W - 1), dtype=torch.bfloat16, device=dev)
    conv_out = (torch.empty_like(x), torch.empty_like(B), torch.empty_like(C))
    dxbc = synth.make_xbc_torch(total_decode * S, cd, 12, dev).view(total_decode, S, cd)
    ustate = torch.zeros((S, cd, CONV_W - 1), dtype=torch.bfloat16, device=dev)
    uout = (torch.empty((S, H, P), dtype=torch.bfloat16, device=dev),
            torch.empty((S, G, N), dtype=torch.bfloat16, device=dev),
            torch.empty((S, G, N), dtype=torch.bfloat16, device=dev))
    conv_plan = erd.ConvUpdatePlan(shape, S, cw, ustate, cbias)
    conv_plan.check(dxbc[0], *uout)

    # speculative decoding: SPEC_BATCH sequences, SPEC_T drafts verified per
    # step, a seeded number of them accepted (drafts drawn from a pool of 8
    # steps' worth of tokens)
    SB, ST = SPEC_BATCH, SPEC_T
    spre = synth.replay_prefix_lengths(SB, Q, 5)
    sx, sdt, sB, sC = synth.make_tokens_torch(int(spre.sum()), H, G, P, N, 5, dev)
    scache = erd.ReplayCache(shape, SB, dev)
    erd.ssd_replay_prefill(shape, scache, synth.cu_seqlens(spre), sx, sdt, sB, sC, A, D, bias)
    del sx, sdt, sB, sC
    pool = [synth.make_tokens_torch(SB * ST, H, G, P, N, 100 + i, dev) for i in range(8)]
    scu_host = synth.cu_seqlens([ST] * SB)
    scu = torch.from_numpy(scu_host).to(dev)
    sy = torch.empty((SB * ST, H, P), dtype=torch.bfloat16, device=dev)
    arng = np.random.default_rng(7)
    accs = arng.integers(0, ST + 1, size=(total_decode, SB)).astype(np.int32)
    accs_dev = torch.from_numpy(accs).to(dev)
    sks = (spre % Q).astype(np.int64)

    # packed-history recovery: RECOVER_T generated tokens of each of the S
    # sequences replayed with one multi-token recurrent update (fp32 cache)
    rx, rdt, rB, rC = synth.make_tokens_torch(S * RECOVER_T, H, G, P, N, 6, dev)
    rcu_host = synth.cu_seqlens([RECOVER_T] * S)
    rcu = torch.from_numpy(rcu_host).to(dev)
    rstate = torch.zeros((S, H, P, N), dtype=torch.float32, device=dev)
    ry = torch.empty_like(rx)
    ks256 = (pre % Q).astype(np.int64)
    ks16 = (pre % 16).astype(np.int64)
    kspg = ks256.copy()

    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    bytes_decode256 = bytes_decode16 = bytes_decodepg = 0
    bytes_verify = bytes_accept = 0
    decode_i = 0

    def step(record):
        nonlocal decode_i, bytes_decode256, bytes_decode16, bytes_decodepg, ks256, ks16, kspg
        nonlocal sks, bytes_verify, bytes_accept
        # events 0..8 bracket the legs; 9.. follow every verification and
        # every acceptance of the speculative leg; the last one follows the
        # recovery
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(10 + 2 * R)] if record else None
        if record:
            ev[0].record(stream)
        erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias, y=y, boundary_state=bnd,
                               cu_seqlens_host=cu_host, want_final=False)
        if record:
            ev[1].record(stream)
        erd.ssd_commit_boundary(shape, commit_cache, cu, x, dt, B, C, bnd,
                                cu_seqlens_host=cu_host)
        if record:
            ev[2].record(stream)
        for r in range(R):
            k = decode_i + r
            plan256(dx[k], ddt[k], dB[k], dC[k], ydec)
            if record:
                bytes_decode256 += replay_step_bytes(ks256, Q, H, G, P, N)
            ks256 = (ks256 + 1) % Q
        if record:
            ev[3].record(stream)
        for r in range(R):
            k = decode_i + r
            plan_ssu(dx[k], ddt[k], dB[k], dC[k], ydec)
        if record:
            ev[4].record(stream)
        for r in range(R):
            k = decode_i + r
            plan16(dx[k], ddt[k], dB[k], dC[k], ydec)
            if record:
                bytes_decode16 += replay_step_bytes(ks16, 16, H, G, P, N)
            ks16 = (ks16 + 1) % 16
        if record:
            ev[5].record(stream)
        for r in range(R):
            k = decode_i + r
            planpg(dx[k], ddt[k], dB[k], dC[k], ydec)
            if record:
                bytes_decodepg += replay_step_bytes(kspg, Q, H, G, P, N)
            kspg = (kspg + 1) % Q
        if record:
            ev[6].record(stream)
        erd.ssd_conv1d_varlen(shape, cu, xbc, cw, cbias, conv_state=cstate, out=conv_out,
                              cu_seqlens_host=cu_host)
        if record:
            ev[7].record(stream)
        for r in range(R):
            conv_plan(dxbc[decode_i + r], *uout)
        if record:
            ev[8].record(stream)
        # speculative rounds: verify SPEC_T drafts, accept a seeded count
        for r in range(R):
            k = decode_i + r
            dxs, ddts, dBs, dCs = pool[k % len(pool)]
            erd.ssd_replay_verify(shape, scache, scu, dxs, ddts, dBs, dCs, A, D, bias, y=sy,
                                  cu_seqlens_host=scu_host)
            if record:
                bytes_verify += verify_step_bytes(sks, ST, Q, H, G, P, N)
                ev[9 + 2 * r].record(stream)
            erd.ssd_replay_accept(shape, scache, scu, accs_dev[k], dxs, ddts, dBs, dCs, A, bias,
                                  cu_seqlens_host=scu_host)
            if record:
                bytes_accept += accept_step_bytes(sks, accs[k], Q, H, G, P, N)
                ev[10 + 2 * r].record(stream)
            sks = (sks + accs[k]) % Q
        erd.ssm_state_update_varlen(shape, rstate, rcu, rx, rdt, rB, rC, A, D, bias, y=ry,
                                    cu_seqlens_host=rcu_host)
        if record:
            ev[9 + 2 * R].record(stream)
        decode_i += R
        return ev

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = [step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def span(i, j):
        return sum(e[i].elapsed_time(e[j]) for e in evs) / 1e3   # seconds, summed

    def spread(pairs, per=1):
        """Per bench step: the leg's time (the sum over the event pairs), ms
        per unit (per = units per bench step): mean, p10, p90 over steps."""
        v = np.array([sum(e[i].elapsed_time(e[j]) for i, j in pairs) for e in evs]) / per
        return {"ms_mean": float(v.mean()), "ms_p10": float(np.percentile(v, 10)),
                "ms_p90": float(np.percentile(v, 90))}

    legs = {
        "prefill": spread([(0, 1)]),
        "commit": spread([(1, 2)]),
        "replay_decode_q256_per_step": spread([(2, 3)], R),
        "ssu_per_step": spread([(3, 4)], R),
        "replay_decode_q16_per_step": spread([(4, 5)], R),
        "replay_decode_q256_paged_per_step": spread([(5, 6)], R),
        "conv_prefill": spread([(6, 7)]),
        "conv_update_per_step": spread([(7, 8)], R),
        "verify_per_round": spread([(8 if r == 0 else 8 + 2 * r, 9 + 2 * r) for r in range(R)],
                                   R),
        "accept_per_round": spread([(9 + 2 * r, 10 + 2 * r) for r in range(R)], R),
        "recovery": spread([(8 + 2 * R, 9 + 2 * R)]),
    }
    ceiling = copy_gbs(torch, dev)
    read_ceiling = read_gbs(torch, dev)

    others = other_workloads(erd, synth, torch, dev, args.warmup, args.steps)
    fused = fused_conv_decode(erd, synth, torch, dev, shape, S, R, args.warmup, args.steps,
                              pre, cw, cbias, (A, D, bias), cd)

    K = args.steps
    t_prefill = span(0, 1)
    t_commit = span(1, 2)
    t_dec256 = span(2, 3)
    t_ssu = span(3, 4)
    t_dec16 = span(4, 5)
    t_decpg = span(5, 6)
    t_conv = span(6, 7)
    t_convu = span(7, 8)
    t_verify = sum(span(8 if r == 0 else 8 + 2 * r, 9 + 2 * r) for r in range(R))
    t_accept = sum(span(9 + 2 * r, 10 + 2 * r) for r in range(R))
    t_recover = span(8 + 2 * R, 9 + 2 * R)
    t_total = span(0, 9 + 2 * R)

    pb = prefill_bytes(S * T, S, H, G, P, N)
    pf = prefill_flops(S * T, H, G, P, N, Q)
    prefill_launch_s = t_prefill / K
    achieved = pb / prefill_launch_s / 1e9
    sha = kernel_source_sha()
    traffic = load_traffic(sha)
    dec_steps = K * R
    dec256_gbs = bytes_decode256 / t_dec256 / 1e9
    dec_ratio = load_decode_ratio(sha)
    dec16_gbs = bytes_decode16 / t_dec16 / 1e9
    decpg_gbs = bytes_decodepg / t_decpg / 1e9
    conv_gbs = conv_prefill_bytes(S * T, S, cd, CONV_W) * K / t_conv / 1e9
    verify_gbs = bytes_verify / t_verify / 1e9
    accept_gbs = bytes_accept / t_accept / 1e9
    recover_gbs = recovery_bytes(S, RECOVER_T, H, G, P, N) * K / t_recover / 1e9
    convu_gbs = conv_update_bytes(S, cd, CONV_W) * dec_steps / t_convu / 1e9
    ssu_gbs = ssu_step_bytes(S, H, G, P, N) * dec_steps / t_ssu / 1e9

    out = {
        "metric": METRIC,
        "value": S * T / prefill_launch_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * t_total / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill 256 seqs x 2048 tokens (H=32 G=1 P=64 N=128 chunk 256, "
                        "bf16 x/dt/B/C/y, fp32 state) + boundary commit + replay decode "
                        "B=256 (chunk 256 and 16, 0..255 buffered tokens; chunk 256 also "
                        "over paged buffers) + recurrent update B=256 + causal conv1d "
                        "(width 4 over x|B|C) prefill on the same pack and decode at B=256 + "
                        "speculative verification of 4 drafts and acceptance at B=512 + "
                        "packed-history recovery of 255 tokens x 256 sequences",
            "global_batch": S, "seq_len": T, "heads": H, "groups": G, "headdim": P,
            "dstate": N, "chunk_size": Q, "decode_steps_per_step": R,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "k_scan (prefill)", "algorithmic_bytes_per_launch": pb,
            "avg_launch_ms": 1e3 * prefill_launch_s,
            "mfma_util": pf / prefill_launch_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "algorithmic_flops_per_launch": pf,
            "measured_copy_gbs": ceiling,
            "frac_of_measured_copy": achieved / ceiling,
            "measured_read_gbs": read_ceiling,
        },
        "decode": {
            "replay_q256_steps_per_s": dec_steps / t_dec256,
            "replay_q256_hbm_gbs": dec256_gbs,
            "replay_q256_frac": dec256_gbs / HBM_PEAK_GBS,
            # the same steps scored on the bytes the counters see (the
            # committed decode traffic summary's counted / algorithmic ratio)
            "replay_q256_counter_frac": (dec256_gbs * dec_ratio / HBM_PEAK_GBS
                                         if dec_ratio else None),
            "replay_q256_us_per_step": 1e6 * t_dec256 / dec_steps,
            # against the streaming-read ceiling measured in the same run
            "replay_q256_frac_of_measured_read": dec256_gbs / read_ceiling,
            "replay_q16_frac_of_measured_read": dec16_gbs / read_ceiling,
            "replay_q16_us_per_step": 1e6 * t_dec16 / dec_steps,
            "replay_q16_steps_per_s": dec_steps / t_dec16,
            "replay_q16_hbm_gbs": dec16_gbs,
            "replay_q16_frac": dec16_gbs / HBM_PEAK_GBS,
            "replay_q256_paged_steps_per_s": dec_steps / t_decpg,
            "replay_q256_paged_hbm_gbs": decpg_gbs,
            "replay_q256_paged_frac": decpg_gbs / HBM_PEAK_GBS,
            "page_tokens": PAGE_TOKENS,
            "ssu_steps_per_s": dec_steps / t_ssu,
            "ssu_hbm_gbs": ssu_gbs,
            "ssu_frac": ssu_gbs / HBM_PEAK_GBS,
            "batch": S,
        },
        "conv": {
            "width": CONV_W, "conv_dim": cd,
            "prefill_ms": 1e3 * t_conv / K,
            "prefill_tokens_per_s": S * T * K / t_conv,
            "prefill_hbm_gbs": conv_gbs,
            "prefill_frac": conv_gbs / HBM_PEAK_GBS,
            "update_steps_per_s": dec_steps / t_convu,
            "update_hbm_gbs": convu_gbs,
            "update_frac": convu_gbs / HBM_PEAK_GBS,
        },
        "speculative": {
            "batch": SPEC_BATCH, "drafts": SPEC_T, "chunk_size": Q,
            "verify_steps_per_s": dec_steps / t_verify,
            "verify_tokens_per_s": dec_steps * SPEC_BATCH * SPEC_T / t_verify,
            "verify_hbm_gbs": verify_gbs,
            "verify_frac": verify_gbs / HBM_PEAK_GBS,
            "accept_steps_per_s": dec_steps / t_accept,
            "accept_hbm_gbs": accept_gbs,
            "accept_frac": accept_gbs / HBM_PEAK_GBS,
        },
        "recovery": {
            "sequences": S, "tokens": RECOVER_T, "state": "f32",
            "ms": 1e3 * t_recover / K,
            "tokens_per_s": S * RECOVER_T * K / t_recover,
            "hbm_gbs": recover_gbs,
            "frac": recover_gbs / HBM_PEAK_GBS,
            # sequential in tokens: bound by fp32 vector arithmetic and its
            # latency, 5 flops per state element and token, against the fp32
            # vector peak without packed instructions
            "alu_tflops": 5 * H * P * N * S * RECOVER_T * K / t_recover / 1e12,
            "alu_frac": 5 * H * P * N * S * RECOVER_T * K / t_recover / 1e12 / FP32_VALU_PEAK_TFLOPS,
            "alu_peak_tflops": FP32_VALU_PEAK_TFLOPS,
        },
        "other_workloads": others,
        "conv_decode_fused": fused,
        "legs": legs,
        "commit_ms": 1e3 * t_commit / K,
        "wall_s": wall,
        "kernel_source_sha": sha,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, dt, B, C, hp, Q, T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
