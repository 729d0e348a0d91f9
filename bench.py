"""Benchmark of the ThinKV decode hot path on one MI355X.

One step = one pass of the whole path over one batch: paged decode attention
over the mixed-precision, hole-bearing cache (with the staged self token) ->
thought classification and kv_append_quant of the new token at its label's
precision (one call, kv_classify_append) -> kv_plan_budget (token budget
ladder) -> kv_evict_segment (the two in one call, kv_plan_budget_evict).  With
--policy anneal the ladder is replaced by kv_plan_anneal (the TBE annealing
schedule of the retention, r0 = 64 by default), applied to the built state
until it plans nothing before anything is timed.  With --compact every step
also compacts the sequences it evicted from (tkv_compact, the gather-
compaction baseline that in-place slot reuse avoids), after every sequence
was compacted once before timing.  --workload churn256 runs the B256 decode
loop (lengths 4k..32k, 5% budget) instead of the default.  --formats page
stores the classes as FP8 E4M3 / FP4 E2M1 / ternary codes.  Workload: the
Llama-8B-like reasoning-decode layer (B32, Hq32/Hkv8, D128, g64, 16k generated
tokens per sequence, 10% budget -> 1638 retained, R/E/T 8/4/2-bit) with
planted-temperature queries, synthetic data.

The state is replicated into enough copies to exceed the 256 MB Infinity Cache
and consecutive steps rotate through them, so each step reads its cache from
HBM.  All inputs are resident in HBM before the timed region.

Prints ONE JSON line (see the fields below).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
CLASS_BITS = (8, 4, 2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence: recording one then costs no system-scope cache
    writeback / invalidation, which a default event performs and which would
    both slow the following work and inflate what the event pair measures."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, torch_events=False):
        import ctypes as C
        self.C = C
        self.torch_events = torch_events
        if torch_events:
            import torch
            self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            return
        self.hip = C.CDLL("libamdhip64.so.7")          # the runtime already in the process
        self.hip.hipEventCreateWithFlags.argtypes = [C.c_void_p, C.c_uint]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        self.ev = []
        for _ in range(n):
            e = C.c_void_p()
            if self.hip.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream):
        if self.torch_events:
            self.ev[i].record()
        elif self.hip.hipEventRecord(self.ev[i], self.C.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        if self.torch_events:
            return self.ev[i].elapsed_time(self.ev[j])
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def state_class_tokens(exported, L):
    """Retained tokens per (sequence, class) from an exported state."""
    out = np.zeros((L.max_seqs, 3), np.int64)
    seq = exported["seq"].reshape(L.max_seqs, 16)
    bt = exported["btab"].reshape(L.max_seqs, 3, L.max_blocks_per_seq)
    blocks_used = np.zeros((L.max_seqs, 3), np.int64)
    for c in range(3):
        masks = exported[f"blk{c}"].reshape(-1, 4)[:, 0].astype(np.uint32)
        pop = np.array([bin(int(m)).count("1") for m in range(1 << 16)], np.int64)
        for s in range(L.max_seqs):
            nb = int(seq[s, c])
            ids = bt[s, c, :nb]
            out[s, c] = int(pop[masks[ids]].sum())
            blocks_used[s, c] = nb
    return out, blocks_used


def algorithmic_bytes(tokens_c, blocks_c, L, batch, self_token=True):
    """Bytes one attention call must move: codes + fp16 (scale, zero) of every
    attended cached token and KV head, the block id and mask word of every
    visited block (per KV head), the queries, outputs, statistics and the
    staged self token."""
    D, g, Hkv, Hq = L.head_dim, L.group_size, L.num_kv_heads, L.num_q_heads
    NG = D // g
    per_tok = [Hkv * 2 * (D * b // 8 + NG * 4) for b in CLASS_BITS]
    kv = sum(int(tokens_c[:, c].sum()) * per_tok[c] for c in range(3))
    blk = int(blocks_c.sum()) * Hkv * (4 + 4)
    io = batch * Hq * D * 2 + batch * Hq * D * 4 + batch * Hq * 12
    if self_token:
        io += batch * Hkv * D * 4 * 2
    return kv + blk + io, kv


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary
    (profiles/), if the kernel's source files are still the ones the counters
    were taken with; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_attn_llama8b_B32_hbm_traffic.json")
    try:
        with open(path) as f:
            j = json.load(f)
        h = hashlib.sha256()
        for name in j["source_files"]:
            with open(os.path.join(ROOT, name), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return float(j["traffic_bytes_per_launch"]) if h.hexdigest() == j["source_sha256"] else None


def cpu_baseline(w, state, ch, n_seq, budget_s=12.0, max_reps=1000, policy="ladder", r0=64, compact=False):
    """The oracle as it stands, on a sample of n_seq sequences of the same
    workload: one full step (attention with the self token, classify, append,
    ladder or annealing plan, evict) per repetition, on all host cores the
    process may use."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import helpers
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    oc = oracle.OracleCache(helpers.oracle_layout(w.layout), w.block_order)
    oc.import_(state)
    sel = np.arange(n_seq, dtype=np.int32)
    q, k, v, pos = ch.step_inputs(0)
    tokens = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        p = (pos[:n_seq] + reps).astype(np.int32)
        out, st, na = oc.attention(sel, p, q[:n_seq], k_self=k[:n_seq], v_self=v[:n_seq])
        lab = oracle.classify(st.astype(np.float32), *ch.tau)
        oc.append(sel, p, lab, k[:n_seq], v[:n_seq])
        if policy == "anneal":
            ops = oc.plan_anneal(sel, r0, 256)
        else:
            ops = oc.plan_budget(sel, ch.budget[0], ch.budget[1], 256)
        if ops[0].size:
            oc.evict(*ops)
            if compact:
                oc.compact(ops[0])
        tokens += int(na.sum())
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= max_reps:
            break
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": tokens / dt, "unit": "KV tokens/s", "cores": min(threads, cores), "kind": "oracle",
            "sample": f"{reps} full steps (attention+classify+append+{policy}+evict"
                      f"{'+compact' if compact else ''}) on {n_seq} of "
                      f"{w.seq_ids.size} sequences of the same cache, fp64 attention, {dt:.1f} s"}


def workload_name(args):
    return (workload_name_1(args)
            + (f"; {args.layers} layers per step sharing the block tables (each layer holds the "
               f"one-layer state's records)" if args.layers > 1 else "")
            + ("; page code formats (R FP8 E4M3, E FP4 E2M1, T ternary)" if args.formats == "page" else ""))


def workload_name_1(args):
    if args.workload == "llama8b":
        head = "llama8b-like reasoning decode, one layer: B32, Hq32/Hkv8, D128, g64, "
        if args.policy == "ladder":
            body = ("16k generated tokens/seq, 10% budget (1638 retained), R/E/T 8/4/2-bit, "
                    "planted-temperature queries; step = attention+classify+append+ladder+evict")
        else:
            body = (f"16k generated tokens/seq, R/E/T 8/4/2-bit, TBE annealing schedule (r0 {args.r0}) applied "
                    f"to the built state, planted-temperature queries; step = attention+classify+append+anneal+evict")
    else:
        head = "B256 reasoning decode loop, one layer: Hq32/Hkv8, D128, g64, "
        body = ("lengths U{4k..32k}, 5% budget, R/E/T 8/4/2-bit, planted-temperature queries; step = "
                "attention+classify+append+" + ("ladder" if args.policy == "ladder" else f"anneal (r0 {args.r0})")
                + "+evict")
    return head + body + ("+compact (gather-compaction baseline, dense start)" if args.compact else "")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--copies", type=int, default=0, help="state copies (0 = enough for > 1 GiB)")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--policy", choices=("ladder", "anneal"), default="ladder",
                    help="eviction planner of the step: the token-budget ladder, or the TBE annealing schedule")
    ap.add_argument("--r0", type=int, default=64, help="first retention of the annealing schedule")
    ap.add_argument("--compact", action="store_true",
                    help="compact the sequences each step evicted from (gather-compaction baseline)")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers per decode step sharing the block tables (the one-layer state replicated)")
    ap.add_argument("--workload", choices=("llama8b", "churn256"), default="llama8b",
                    help="the llama8b-like layer (B32, 16k, 10%% budget) or the B256 decode loop (4k..32k, 5%% budget)")
    ap.add_argument("--formats", choices=("int", "page"), default="int",
                    help="code formats of the 8/4/2-bit classes: asymmetric integer, or FP8 E4M3 / FP4 E2M1 / ternary")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-only", action="store_true", help="time only the attention call (diagnostic)")
    ap.add_argument("--torch-events", action="store_true", help="time with torch's default events (diagnostic)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed region, copy MIB MiB device-to-device 3 times (a plain copy kernel of "
                         "known size, to scale hardware byte counters by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path shards by "
              f"sequence with no exchange, so N GPUs would run N independent copies of this step.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from thought_adaptive_mixed_amd import binding, synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import helpers
    dv0 = lambda a: helpers.dev(a, np.int32)

    total_steps = args.warmup + args.steps
    log("[bench] building workload")
    t0 = time.time()
    ch = synth.bench_cycle(steps=total_steps) if args.workload == "llama8b" else synth.churn(steps=total_steps)
    if args.formats == "page":
        ch.base = synth.page_formats(ch.base)
    w = ch.base
    L = w.layout
    B = w.seq_ids.size
    sizes = binding.buffer_sizes(helpers.gpu_layout(L))
    state_bytes = sum(sizes[:-1])
    R = args.copies or max(2, math.ceil((1 << 30) / state_bytes))
    log(f"[bench] state {state_bytes / 1e6:.1f} MB, {R} copies")
    c0 = helpers.build_gpu(w)
    torch.cuda.synchronize()
    if args.policy == "anneal":
        # the built state has never been annealed: apply the schedule until it plans nothing
        m_all = L.max_tokens_per_call
        t_ops = [torch.zeros(m_all, dtype=torch.int32, device="cuda") for _ in range(3)]
        t_bits = torch.zeros(m_all, dtype=torch.uint8, device="cuda")
        t_n = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(1000):
            c0.plan_anneal(dv0(w.seq_ids), args.r0, m_all, t_n, *t_ops, t_bits)
            c0.evict(*t_ops, t_bits, n_ops_dev=t_n, n_ops=m_all)
            if int(t_n.item()) == 0:
                break
        torch.cuda.synchronize()
    if args.compact:
        # start dense: every sequence compacted once (one per call, so each needs only its own room)
        for s in w.seq_ids:
            c0.compact(dv0([s]))
        torch.cuda.synchronize()
    state = c0.export()
    NL = max(1, args.layers)
    if NL > 1:
        # every layer of the layered cache holds the one-layer state's records (same bytes and work per layer)
        state1 = state
        state = dict(state1)
        for cc in range(3):
            P = L.pool_blocks[cc]
            state[f"pool{cc}"] = np.repeat(state1[f"pool{cc}"].reshape(P, 1, -1), NL, axis=1).ravel()
        del c0
        L = dataclasses.replace(L, num_layers=NL)
        sizes = binding.buffer_sizes(helpers.gpu_layout(L))
        R = args.copies or max(2, math.ceil((1 << 30) / sum(sizes[:-1])))
        caches = [binding.Cache(helpers.gpu_layout(L), w.block_order) for _ in range(R)]
        for c in caches:
            c.import_(state)
        log(f"[bench] {NL} layers: state {sum(sizes[:-1]) / 1e6:.1f} MB, {R} copies")
        state = state1
    else:
        caches = [c0] + [binding.Cache(helpers.gpu_layout(L), w.block_order) for _ in range(R - 1)]
        for c in caches[1:]:
            c.import_(state)
    tok_c, blk_c = state_class_tokens(state, dataclasses.replace(L, num_layers=1))
    abytes, kvbytes = algorithmic_bytes(tok_c, blk_c, L, B)
    log(f"[bench] built in {time.time() - t0:.1f} s; algorithmic bytes per attention call {abytes / 1e6:.2f} MB")

    # inputs for every step, resident on the device
    dv = helpers.dev
    seq_d = dv(w.seq_ids, np.int32)
    # Step s runs on copy s % R, and it is that copy's (s // R)-th decode step:
    # each copy replays the same decode sequence (positions, planted thought
    # types, new tokens), so every copy sees the planted segment process as
    # one cache would, not every R-th step of it.
    per_copy = []
    for i in range((total_steps + R - 1) // R):
        q, k, v, pos = ch.step_inputs(i)
        # with layers: each layer attends with the same query and self-token rows; the append takes every layer's
        kl, vl = np.tile(k, (1, NL, 1)), np.tile(v, (1, NL, 1))
        per_copy.append((dv(q, np.uint16), dv(k, np.float32), dv(v, np.float32), dv(pos, np.int32),
                         dv(kl, np.float32) if NL > 1 else None, dv(vl, np.float32) if NL > 1 else None))
    steps_in = [per_copy[s // R] for s in range(total_steps)]
    Hq, D = L.num_q_heads, L.head_dim
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    stats = torch.empty(B, NL, Hq, 3, dtype=torch.float32, device="cuda")   # every layer's rows of a step
    n_att = torch.zeros(total_steps, B, dtype=torch.int32, device="cuda")   # one row per step
    ws = torch.empty(max(caches[0].workspace_bytes(B), 16), dtype=torch.uint8, device="cuda")
    labels = torch.empty(B, dtype=torch.uint8, device="cuda")
    max_ops = 256
    n_ops = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_seq = torch.zeros(max_ops, dtype=torch.int32, device="cuda")
    o_seg, o_keep = torch.zeros_like(o_seq), torch.zeros_like(o_seq)
    o_bits = torch.zeros(max_ops, dtype=torch.uint8, device="cuda")
    ev = HipEvents(2 * total_steps + 2, torch_events=args.torch_events)   # (before, after) each attention

    # every call's C arguments are converted once, before anything is timed
    sh = torch.cuda.current_stream().cuda_stream
    calls_a, calls_b = [], []
    for s in range(total_steps):
        c = caches[s % R]
        q, k, v, pos, kl, vl = steps_in[s]
        calls_a.append([c.attention(seq_d, pos, q, out, ws, stats=stats[:, l], n_attended=n_att[s], k_self=k,
                                    v_self=v, layer=l, stats_stride=NL * Hq * 3, stream=sh, prepare=True)
                        for l in range(NL)])
        calls_b.append([
            # classification of every layer's statistics rows, inside the append's allocation kernel
            c.classify_append(seq_d, pos, stats.view(B, NL * Hq, 3), ch.tau[0], ch.tau[1], kl if NL > 1 else k,
                              vl if NL > 1 else v, labels_out=labels, stream=sh, prepare=True),
        ] + ([c.plan_anneal_evict(seq_d, args.r0, max_ops, n_ops, o_seq, o_seg, o_keep, o_bits, stream=sh,
                                  prepare=True)]
             if args.policy == "anneal" else
             # the planner and the eviction's planning in one kernel (kv_plan_budget_evict / kv_plan_anneal_evict)
             [c.plan_budget_evict(seq_d, ch.budget[0], ch.budget[1], max_ops, n_ops, o_seq, o_seg, o_keep, o_bits,
                                  stream=sh, prepare=True)])
          + ([c.compact(o_seq, n_dev=n_ops, n=max_ops, stream=sh, prepare=True)] if args.compact else []))

    # Steps are launched eagerly on torch's current stream: on this stack a
    # replayed HIP graph per step measured slower than direct launches.  The
    # attention launch is bracketed by events on the same stream.
    def step(s):
        ev.record(2 * s, sh)
        for f in calls_a[s]:
            f()
        ev.record(2 * s + 1, sh)
        if not args.attn_only:
            for f in calls_b[s]:
                f()

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {nbytes} bytes read + written")
        del src, dst

    log("[bench] warmup")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    log("[bench] timed")
    T0, T1 = 2 * total_steps, 2 * total_steps + 1
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    ev.record(T0, sh)
    for s in range(args.warmup, total_steps):
        step(s)
    ev.record(T1, sh)
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    ms_total = ev.elapsed_ms(T0, T1)
    log(f"[bench] host enqueue {(h1 - h0) * 1e6 / args.steps:.1f} us/step, device {ms_total * 1e3 / args.steps:.1f} us/step")
    attn_ms = [ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(args.warmup, total_steps)]
    errs = [c.get_error() for c in caches]
    if any(e[0] for e in errs):
        log(f"[bench] WARNING device errors: {errs}")
    tokens1 = int(n_att[args.warmup:].sum().item())        # one layer's attended tokens
    tokens = tokens1 * NL                                   # KV tokens attended over all layers
    ms_step = ms_total / args.steps
    attn_avg = float(np.mean(attn_ms))                      # every layer's attention of a step
    # the cache changes a little from step to step (appends, evictions): scale
    # the KV part of the byte count by the attended tokens actually seen
    init_tokens = int(tok_c[:B].sum())
    abytes_step = abytes - kvbytes + kvbytes * (tokens1 / args.steps) / max(init_tokens, 1)
    achieved = abytes_step / (attn_avg / NL * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": tokens / (ms_total * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f16 MFMA (int8/4/2 codes as exact fp16 subnormals), f32 accumulate" if args.formats == "int" else
                  "f16 MFMA (FP8 E4M3 / FP4 E2M1 codes converted exactly to fp16, ternary codes as fp16 "
                  "subnormals), f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": workload_name(args),
                   "batch": B, "copies": R, "attended_per_step": tokens / args.steps,
                   "launch": "eager, one stream", **({"layers": NL} if NL > 1 else {})},
        "attn_ms": attn_avg,
        "attn_kv_tokens_per_s": (tokens / args.steps) / (attn_avg * 1e-3),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if (args.workload == "llama8b" and args.policy == "ladder"
                                                       and not args.compact and NL == 1
                                                       and args.formats == "int") else None,
                     "kernel": "k_attn (paged_decode_attn; one launch per layer and step)",
                     "bytes_per_launch": abytes_step},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, state, ch, args.cpu_seqs, policy=args.policy, r0=args.r0,
                                              compact=args.compact)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
