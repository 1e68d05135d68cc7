#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of one attention layer for the whole batch:
pa_copy_blocks (copy-on-write pairs of the step; none in these workloads),
then pa_decode over every sequence's paged KV cache, which also stores each
sequence's new token into its slot (fused append; --separate-write runs
pa_write_kv first instead).  Inputs are seeded, synthetic and resident in HBM
before timing starts.  R replicas (disjoint block sets of one pool, their
own queries and new tokens) are cycled so that consecutive steps read
different KV bytes, as successive layers would, and the 256 MB last-level
cache cannot serve them.

Protocol: untimed priming (every replica twice and at least --prime-seconds
of back-to-back steps, so that no replica is first touched inside the timed
region and the clocks have settled), --warmup untimed steps, then exactly
--steps timed steps between two synchronizations.

Prints one JSON line.  value = KV bytes read per step / seconds per step
(GB/s); seq_steps_per_s = sequences / seconds per step.  roofline covers
pa_decode, timed with HIP events on the stream it runs on.  read_ceiling
times a loads-only probe of the same tiles.  cpu_baseline is the fp64 CPU
oracle timed on this host's cores over a bounded sample.  The default
(LLaMA-13B-shaped) run adds the mixed-length and long-context workloads
under extra_configs, measured the same way.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="llama13b_f16",
                    choices=["llama13b_f16", "mixed_gqa_bf16", "long_bf16", "prefill_llama13b_f16",
                             "shared_prefix_bf16", "cow_bf16"])
    ap.add_argument("--no-prefix-groups", action="store_true",
                    help="shared_prefix_bf16 and cow_bf16: decode with pa_decode (every sequence "
                         "reads the shared prefix itself) instead of pa_decode_prefix")
    ap.add_argument("--replicas", type=int, default=0, help="0 = as many as the pool allows (max 16)")
    ap.add_argument("--partition-size", type=int, default=-1, help="-1 = the workload's own")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget; 0 = skip")
    ap.add_argument("--profile-steps", action="store_true", help="no cpu baseline (for profilers)")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the new tokens with pa_write_kv, then pa_decode (default: "
                         "pa_decode appends them itself)")
    ap.add_argument("--kv", default="same", choices=["same", "i8", "fp8"],
                    help="KV-cache type: the workload's own element type, or INT8 codes with "
                         "per-token scales (queries keep the workload's type)")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32, 64],
                    help="tokens per cache block (the workloads are defined at 16; the pool keeps "
                         "its bytes)")
    ap.add_argument("--no-host-lens", action="store_true",
                    help="do not pass the host copy of the context lengths (the library then "
                         "launches every (sequence, partition) pair max_context_len allows)")
    ap.add_argument("--prime-seconds", type=float, default=0.3,
                    help="untimed steps before the warm-up: every replica twice and at least this "
                         "long (-1 = none)")
    ap.add_argument("--no-extra-configs", dest="extra_configs", action="store_false",
                    help="headline workload only (by default the LLaMA-13B-shaped run also measures "
                         "the mixed-length and long-context workloads as extra keys)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the read-ceiling probe (pa_probe_read) of the step's tiles")
    ap.add_argument("--products", default="auto", choices=["auto", "matrix", "valu"],
                    help="one query head per KV head: compute both products on the matrix cores "
                         "or on the vector ALU (default: the library's choice)")
    ap.add_argument("--calib-bytes", type=int, default=0,
                    help="first run one plain device-to-device copy of this many bytes (a "
                         "known-size reference for hardware byte counters)")
    return ap.parse_args()


def random_q8_pools(case, kv, g, dev):
    """Two 8-bit pools [NB, Hkv, tile] on the device: random codes (INT8 in
    [-127, 127]; FP8: random sign, exponent field 4..13, mantissa, as bits),
    then per-token scales uniform in [0.01, 0.04].  FP8 pools are
    float8_e4m3fn tensors, INT8 ones uint8."""
    import torch
    from paged_kv_cache_328_amd import workloads as wl
    tile, cb = wl.i8_tile_bytes(case.D, case.BS), case.D * case.BS
    shape = (case.NB, case.Hkv, tile)
    pools = []
    for _ in range(2):
        if kv == "fp8":
            e = torch.randint(4, 14, shape, dtype=torch.int32, device=dev, generator=g)
            m = torch.randint(0, 8, shape, dtype=torch.int32, device=dev, generator=g)
            sgn = torch.randint(0, 2, shape, dtype=torch.int32, device=dev, generator=g)
            p = ((sgn << 7) | (e << 3) | m).to(torch.uint8)
        else:
            p = torch.randint(-127, 128, shape, dtype=torch.int8, device=dev, generator=g).view(torch.uint8)
        sc = torch.rand((case.NB, case.Hkv, case.BS), device=dev, generator=g) * 0.03 + 0.01
        p[:, :, cb:] = sc.view(torch.uint8)
        pools.append(p.view(torch.float8_e4m3fn) if kv == "fp8" else p)
    return pools


def build_case(name, replicas, kv_dtype=None, block_size=16):
    from paged_kv_cache_328_amd import workloads as wl
    kw = dict(fill=False, kv_dtype=kv_dtype, block_size=block_size)
    if name == "llama13b_f16":
        probe = wl.llama13b_f16(**kw)
        need = int(sum(-(-int(c) // probe.BS) for c in probe.context_lens))
        R = replicas or min(16, probe.NB // need)
        return wl.llama13b_f16(replicas=R, **kw)
    if name == "mixed_gqa_bf16":
        return wl.mixed_gqa_bf16(replicas=replicas or 4, **kw)
    return wl.long_bf16(replicas=replicas or 2, **kw)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(one process drives one GPU; sharding sequences or KV heads over several GPUs "
              "is not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa

    pa.lib()  # fail loudly if the library is not built
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.config.startswith("prefill"):
        return bench_prefill(args, dev)
    if args.config == "shared_prefix_bf16":
        return bench_shared_prefix(args, dev)
    if args.config == "cow_bf16":
        return bench_cow(args, dev)
    result, keep = run_decode(args, dev, args.config)
    if args.cpu_seconds > 0 and not args.profile_steps:
        result["cpu_baseline"] = cpu_baseline(*keep, args.cpu_seconds)
    del keep
    torch.cuda.empty_cache()
    # The headline run also measures the other two bandwidth-bound workloads
    # (mixed lengths with GQA, long context) in the same process and the same
    # protocol, reported as extra keys of the one JSON line.
    if (args.config == "llama13b_f16" and args.extra_configs and not args.profile_steps
            and args.kv == "same" and args.block_size == 16 and args.partition_size < 0):
        extra = {}
        for name in ("mixed_gqa_bf16", "long_bf16"):
            r, keep = run_decode(args, dev, name)
            del keep
            torch.cuda.empty_cache()
            extra[name] = {k: r[k] for k in ("ms_per_step", "gpu_ms_per_step", "value", "pct_hbm_peak",
                                             "seq_steps_per_s", "prime")}
            extra[name]["config"] = {k: r["config"][k] for k in ("workload", "num_seqs", "q_heads", "kv_heads",
                                                                 "head_dim", "block_size", "context_tokens",
                                                                 "partition_size", "replicas")}
            extra[name]["roofline"] = {k: r["roofline"][k] for k in ("kernel", "achieved", "frac", "traffic",
                                                                     "avg_launch_ms",
                                                                     "algorithmic_bytes_per_launch")}
            extra[name]["read_ceiling"] = r.get("read_ceiling")
        result["extra_configs"] = extra
    print(json.dumps(result), flush=True)


def prime(step, R, min_seconds):
    """Untimed steps before the warm-up: every replica at least twice, and
    for at least min_seconds of back-to-back work, so that the timed steps
    meet no first touch of a replica and the GPU's clocks have settled
    whatever --warmup is.  Returns (steps, seconds)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < 2 * R or time.perf_counter() - t0 < min_seconds:
        step(n)
        n += 1
        if n % R == 0:
            torch.cuda.synchronize()  # keep the launch queue short
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_steps(step, steps, stream):
    """K steps enqueued back to back between two synchronizations: (wall
    seconds per step, GPU milliseconds per step from one pair of HIP events on
    the launch stream).  No event sits between launches (an event record
    between two kernels adds several microseconds of its own)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, e0.elapsed_time(e1) / steps


def run_decode(args, dev, name):
    """One decode workload on the protocol of the module docstring.  Returns
    (result dict, (case, k pool, v pool) for the CPU baseline)."""
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa
    from paged_kv_cache_328_amd import workloads as wl

    i8 = args.kv in ("i8", "fp8")  # 8-bit pools (INT8 or FP8 codes)
    case = build_case(name, args.replicas, args.kv if i8 else None, args.block_size)
    R, S, dtype = case.replicas, case.S, case.dtype
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    P = case.partition_size if args.partition_size < 0 else args.partition_size

    # ---- inputs, resident in HBM
    g = torch.Generator(device=dev)
    g.manual_seed(wl.base_seed(case.name))
    if i8:
        kd, vd = random_q8_pools(case, args.kv, g, dev)
        tile_bytes = wl.i8_tile_bytes(case.D, case.BS)
    else:
        ks, vs = wl.pool_shapes(case.NB, case.Hkv, case.D, case.BS, dtype)
        kd = torch.randn(ks, dtype=tdt, device=dev, generator=g)
        vd = torch.randn(vs, dtype=tdt, device=dev, generator=g)
        tile_bytes = case.D * case.BS * wl.ELEM_BYTES[dtype]

    def dev_storage(a):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    tables = [torch.from_numpy(np.ascontiguousarray(case.block_tables[r])).to(dev) for r in range(R)]
    lens = torch.from_numpy(case.context_lens).to(dev)
    qs = [dev_storage(case.q[r]) for r in range(R)]
    knew = [dev_storage(case.new_k[r]) for r in range(R)]
    vnew = [dev_storage(case.new_v[r]) for r in range(R)]
    slots = [torch.from_numpy(np.ascontiguousarray(case.slot_mapping[r])).to(dev) for r in range(R)]
    no_pairs = torch.zeros((0, 2), dtype=torch.int32, device=dev)
    max_ctx = case.max_context
    stream = torch.cuda.current_stream()
    # arguments are marshalled once per replica; the timed loop only enqueues
    outs = [torch.empty_like(qs[0]) for _ in range(R)]
    fused = not args.separate_write
    # the scheduler's host copy of the lengths lets the library launch only
    # the (sequence, partition) units that exist
    host_lens = None if args.no_host_lens else case.context_lens
    decode = [pa.prepare_decode(outs[r], qs[r], kd, vd, tables[r], lens, case.scale, max_ctx,
                                partition_size=P, stream=stream,
                                k_new=knew[r] if fused else None, v_new=vnew[r] if fused else None,
                                context_lens_host=host_lens, products=args.products)
              for r in range(R)]
    write = [pa.prepare_write_kv(knew[r], vnew[r], kd, vd, slots[r], stream=stream) for r in range(R)]
    if fused:
        write = [lambda: None] * R
    copy = pa.prepare_copy_blocks(kd, vd, no_pairs, stream=stream, head_dim=case.D)
    a0 = pa.make_decode_args(outs[0], qs[0], kd, vd, tables[0], lens, case.scale, max_ctx, P,
                             products=args.products)
    P_eff = pa.pa_decode_partition_size(a0)
    valu = pa.pa_decode_products(a0) == pa.PA_PRODUCTS_VALU
    split = P_eff < max_ctx

    if args.calib_bytes > 0:
        src = torch.empty(args.calib_bytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i):
        r = i % R
        copy()
        write[r]()
        decode[r]()

    primed = prime(step, R, args.prime_seconds) if args.prime_seconds >= 0 else (0, 0.0)
    for i in range(args.warmup):
        step(i)
    sec_per_step, gpu_ms_per_step = time_steps(step, args.steps, stream)
    # The decode launch alone: in the fused step it is the step's only launch;
    # with --separate-write it is timed in a second loop of decode launches.
    if fused:
        decode_ms = gpu_ms_per_step
    else:
        decode_ms = time_steps(lambda i: decode[i % R](), args.steps, stream)[1]

    # ---- algorithmic bytes of one pa_decode launch
    esz = wl.ELEM_BYTES[dtype]
    kv_bytes = case.kv_bytes()
    n_blocks = int(sum(-(-int(c) // case.BS) for c in case.context_lens))
    decode_bytes = kv_bytes + n_blocks * 4 + S * 4 + 2 * S * case.Hq * case.D * esz
    if fused:  # the appended token is also written to its slot (INT8: codes and a scale)
        decode_bytes += 2 * S * case.Hkv * ((case.D + 4) if i8 else case.D * esz)
    achieved = decode_bytes / (decode_ms * 1e-3) / 1e9

    ceiling = None
    if not args.no_probe and not args.profile_steps:
        ceiling = read_ceiling(args, case, kd, vd, tile_bytes, stream, decode_ms)

    # ---- host bookkeeping (allocator) for one step, reported separately
    A = pa.Allocator(case.NB, case.BS)
    for s in range(S):
        A.pa_seq_add(s)
        for _ in range(int(case.context_lens[s]) - 1):
            A.pa_seq_append_slot(s)
    th = time.perf_counter()
    n_rep = 200
    for _ in range(n_rep):
        A.pa_seq_append_slots(list(range(S)))
    host_us = (time.perf_counter() - th) / n_rep * 1e6
    A.close()

    result = {
        "metric": "paged decode attention: achieved KV GB/s (% HBM peak) and seq-steps/s",
        "value": round(kv_bytes / sec_per_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 5),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "pct_hbm_peak": round(100 * kv_bytes / sec_per_step / 1e9 / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(S / sec_per_step, 1),
        "prime": {"primed_replicas": R if primed[0] >= R else primed[0], "steps": primed[0],
                  "seconds": round(primed[1], 3)},
        "config": {"workload": case.name + (" (INT8 KV)" if i8 else "")
                   + (f" (block size {case.BS})" if case.BS != 16 else ""), "kv_dtype": case.kv_dtype,
                   "num_seqs": S, "q_heads": case.Hq, "kv_heads": case.Hkv,
                   "head_dim": case.D, "block_size": case.BS, "num_blocks": case.NB,
                   "context_tokens": int(case.context_lens.sum()),
                   "max_context": max_ctx, "partition_size": P_eff, "replicas": R,
                   "host_context_lens": host_lens is not None,
                   "kv_bytes_per_step": kv_bytes,
                   "step": ("pa_copy_blocks(0 pairs) + pa_decode(fused append of the new token)"
                            if fused else "pa_copy_blocks(0 pairs) + %s + pa_decode"
                            % ({"i8": "pa_write_kv_i8", "fp8": "pa_write_kv_fp8"}.get(args.kv, "pa_write_kv")))},
        "roofline": {"kernel": "decode_mfma_kernel" + (" (vector-ALU products)" if valu else "")
                     + (" (fused append)" if fused else "")
                     + (" + merge_kernel (split-K)" if split else ""),
                     "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(case.name + (":" + args.kv if i8 else "")
                                                 + (f":bs{case.BS}" if case.BS != 16 else ""), P_eff, fused,
                                                 host_lens is not None),
                     "avg_launch_ms": round(decode_ms, 5),
                     "algorithmic_bytes_per_launch": decode_bytes},
        "host_bookkeeping_us": round(host_us, 2),
    }
    if ceiling is not None:
        result["read_ceiling"] = ceiling
    return result, (case, kd, vd)


def read_ceiling(args, case, kd, vd, tile_bytes, stream, decode_ms):
    """Read ceilings of the step's access pattern, from pa_probe_read (loads
    only, no arithmetic), timed like the decode over the same replicas:
      tiles:      every (block, KV head) K and V tile the decode step reads,
                  in (sequence, KV head, block) order;
      contiguous: the same number of bytes as consecutive tiles of the pools.
    decode_vs_tiles = the tile probe's time / the decode launch's time."""
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa
    dev = kd.device
    R, Hkv, BS = case.replicas, case.Hkv, case.BS
    nblk = [-(-int(c) // BS) for c in case.context_lens]
    offs = []
    for r in range(R):
        t = case.block_tables[r]
        o = [(int(t[s, j]) * Hkv + h) * tile_bytes for s in range(case.S) for h in range(Hkv)
             for j in range(nblk[s])]
        offs.append(torch.tensor(o, dtype=torch.int64, device=dev))
    n = offs[0].numel()
    pool_bytes = kd.numel() * kd.element_size()
    contig = []
    span = n * tile_bytes
    for r in range(R):
        base = (r * span) % max(pool_bytes - span + 1, 1)
        base -= base % tile_bytes
        contig.append(torch.arange(n, dtype=torch.int64, device=dev) * tile_bytes + base)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    kb, vb = kd.view(-1).view(torch.uint8), vd.view(-1).view(torch.uint8)
    out = {"range_bytes": tile_bytes, "ranges_per_step": n, "bytes_per_step": 2 * n * tile_bytes}
    for label, lists in (("tiles", offs), ("contiguous", contig)):
        calls = [pa.prepare_probe_read(kb, vb, lists[r], tile_bytes, sink, stream=stream) for r in range(R)]
        step = lambda i: calls[i % R]()
        prime(step, R, 0.05)
        ms = time_steps(step, max(args.steps, 20), stream)[1]
        out[label + "_gbs"] = round(2 * n * tile_bytes / (ms * 1e-3) / 1e9, 1)
        out[label + "_ms"] = round(ms, 5)
    out["decode_vs_tiles"] = round(out["tiles_ms"] / decode_ms, 4)
    return out


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix cores


def bench_prefill(args, dev):
    """One step = one pa_prefill call: every sequence's chunk attends causally
    over its paged context.  value = algorithmic TFLOP/s (QK and PV, 4 * D
    flops per (row, head, key)); the roofline is the dense f16 MFMA peak."""
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa
    from paged_kv_cache_328_amd import workloads as wl
    i8 = args.kv in ("i8", "fp8")
    case = wl.prefill_llama13b_f16(fill=False, kv_dtype=args.kv if i8 else None,
                                   block_size=args.block_size)
    dtype = case.dtype
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(wl.base_seed(case.name))
    if i8:
        kd, vd = random_q8_pools(case, args.kv, g, dev)
    else:
        ks, vs = wl.pool_shapes(case.NB, case.Hkv, case.D, case.BS, dtype)
        kd = torch.randn(ks, dtype=tdt, device=dev, generator=g)
        vd = torch.randn(vs, dtype=tdt, device=dev, generator=g)
    qd = torch.from_numpy(np.ascontiguousarray(case.q)).to(dev)
    out = torch.empty_like(qd)
    tables = torch.from_numpy(np.ascontiguousarray(case.block_tables)).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    qs = torch.from_numpy(case.query_start).to(dev)
    stream = torch.cuda.current_stream()
    call = pa.prepare_prefill(out, qd, kd, vd, tables, lens, qs, case.scale, case.max_query_len,
                              case.max_context, stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    flops = case.flops()
    rows = int(case.query_start[-1])
    result = {
        "metric": "paged prefill attention: achieved TFLOP/s (% of dense MFMA peak) and prompt tokens/s",
        "value": round(flops / sec / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5), "gpu_ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "tokens_per_s": round(rows / sec, 1),
        "config": {"workload": case.name + (" (INT8 KV)" if i8 else "")
                   + (f" (block size {case.BS})" if case.BS != 16 else ""), "kv_dtype": case.kv_dtype,
                   "num_seqs": case.S, "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
                   "block_size": case.BS, "chunk_rows": rows,
                   "context_tokens": int(case.context_lens.sum()),
                   "flops_per_step": flops, "step": "pa_prefill"},
        "roofline": {"kernel": "prefill_lds_kernel", "bound": "mfma",
                     "achieved": round(flops / (ms * 1e-3) / 1e12, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(ms, 5), "algorithmic_flops_per_launch": flops},
    }
    if args.cpu_seconds > 0 and not args.profile_steps:
        result["cpu_baseline"] = cpu_baseline_prefill(case, kd, vd, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_shared_prefix(args, dev):
    """One step = one decode step of 32 sequences that share a 2048-token
    prefix (block size 32, private suffixes of 1..512 tokens, 32 query / 8 KV
    heads, bf16), with the fused append: pa_decode_prefix reads the shared
    blocks once for the group (--no-prefix-groups: pa_decode, every sequence
    reads them).  R replicas (own prefix and suffix blocks) are cycled.
    value = logical KV bytes (every sequence's whole context) per second."""
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa
    from paged_kv_cache_328_amd import workloads as wl
    name = "shared_prefix_bf16"
    seed = wl.base_seed("cow_bf16")
    rng = np.random.default_rng(seed)
    n, BS, R = 32, 32, args.replicas or 8
    suffix = rng.integers(1, 512, size=n, endpoint=True).tolist()
    case, gs, shared = wl.shared_prefix_case(seed + 1, [(2048 // BS, suffix)] * R, 32, 8, 128, BS,
                                             "bf16", fill=False)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    ks, vs = wl.pool_shapes(case.NB, case.Hkv, case.D, case.BS, "bf16")
    kd = torch.randn(ks, dtype=torch.bfloat16, device=dev, generator=g)
    vd = torch.randn(vs, dtype=torch.bfloat16, device=dev, generator=g)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    stream = torch.cuda.current_stream()
    calls = []
    lens_all = case.context_lens
    use_groups = not args.no_prefix_groups
    for r in range(R):
        rows = slice(r * n, (r + 1) * n)
        tables = torch.from_numpy(np.ascontiguousarray(case.block_tables[0][rows])).to(dev)
        lens = torch.from_numpy(np.ascontiguousarray(lens_all[rows])).to(dev)
        q = dev_bf16(case.q[0][rows])
        out = torch.empty_like(q)
        kn, vn = dev_bf16(case.new_k[0][rows]), dev_bf16(case.new_v[0][rows])
        max_ctx = int(lens_all[rows].max())
        if use_groups:
            gst = torch.tensor([0, n], dtype=torch.int32, device=dev)
            pl = torch.tensor([int(shared[r])], dtype=torch.int32, device=dev)
            calls.append(pa.prepare_decode_prefix(out, q, kd, vd, tables, lens, case.scale, max_ctx,
                                                  gst, pl, n, int(shared[r]), stream=stream,
                                                  k_new=kn, v_new=vn, min_prefix_len=int(shared[r])))
        else:
            calls.append(pa.prepare_decode(out, q, kd, vd, tables, lens, case.scale, max_ctx,
                                           stream=stream, k_new=kn, v_new=vn,
                                           context_lens_host=None if args.no_host_lens
                                           else lens_all[rows]))
    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        calls[i % R]()
    e1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    per_tok = 2 * case.Hkv * case.D * 2
    logical = int(lens_all[:n].sum()) * per_tok
    unique = (int(shared[0]) + sum(suffix)) * per_tok
    alg = (unique if use_groups else logical) + 2 * n * case.Hq * case.D * 2 + 2 * n * case.Hkv * case.D * 2
    result = {
        "metric": "paged decode attention with a shared prefix: logical KV GB/s and seq-steps/s",
        "value": round(logical / sec / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5), "gpu_ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "seq_steps_per_s": round(n / sec, 1),
        "config": {"workload": name + ("" if use_groups else " (pa_decode, no prefix groups)"),
                   "num_seqs": n, "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
                   "block_size": BS, "shared_prefix_tokens": int(shared[0]),
                   "context_tokens": int(lens_all[:n].sum()), "replicas": R,
                   "logical_kv_bytes_per_step": logical, "unique_kv_bytes_per_step": unique,
                   "step": "pa_decode_prefix(fused append)" if use_groups else "pa_decode(fused append)"},
        "roofline": {"kernel": ("decode_mfma_kernel prefix pass + suffix decode + merge_kernel"
                                if use_groups else "decode_mfma_kernel (fused append) + merge_kernel"),
                     "bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 5), "algorithmic_bytes_per_launch": alg},
    }
    print(json.dumps(result), flush=True)


def bench_cow(args, dev):
    """One step of the copy-on-write workload: 32 sequences forked from one
    2048-token prefix (block size 32, bf16, 32 query / 8 KV heads), each with a
    private suffix of 1..512 tokens and forked once more (parallel sampling),
    so every partly filled tail block is shared by two sequences.  The native
    block manager builds this state and takes the step's append: it returns
    one slot per sequence and a (source, copy) pair per shared partial tail.
    One step = pa_copy_blocks over those pairs, then the decode, which stores
    each new token into its slot (now in the copy) and attends:
    pa_decode_prefix with the 2048 shared tokens as the group's prefix
    (--no-prefix-groups: pa_decode).  R replicas of the whole arrangement sit
    in disjoint block ranges of one pool and are cycled; a replica's copies
    and token stores repeat with the same result each cycle, so every step
    does the same work.  value = logical KV bytes (every sequence's whole
    context) per second."""
    import torch
    from paged_kv_cache_328_amd import pagedattn as pa
    from paged_kv_cache_328_amd import workloads as wl
    plan = wl.cow_plan()
    BS, NB, n, Hq, Hkv, D = plan["BS"], plan["NB"], plan["n"], plan["Hq"], plan["Hkv"], plan["D"]
    R = args.replicas or 8
    A = pa.Allocator(NB, BS, plan["init_free_order"])
    A.pa_seq_add(0)
    for _ in range(plan["prefix"]):
        A.pa_seq_append_slot(0)
    for i in range(1, n):
        A.pa_seq_fork(0, i)
    for i in range(n):
        for _ in range(plan["suffix"][i]):
            A.pa_seq_append_slot(i)
    for i in range(n):
        A.pa_seq_fork(i, 1000 + i)
    th = time.perf_counter()
    slots, pairs = A.pa_seq_append_slots(list(range(n)))
    host_us = (time.perf_counter() - th) * 1e6
    lens = np.array([A.pa_seq_len(i) for i in range(n)], np.int32)
    tables = [A.pa_seq_block_table(i) for i in range(n)]
    A.close()
    table = np.zeros((n, max(len(t) for t in tables)), np.int32)
    for i, t in enumerate(tables):
        table[i, :len(t)] = t
    pairs = np.asarray(pairs, np.int32).reshape(-1, 2)
    shared = plan["prefix"]  # whole blocks shared by every sequence after the copies
    max_ctx = int(lens.max())

    g = torch.Generator(device=dev)
    g.manual_seed(wl.base_seed("cow_bf16"))
    ks, vs = wl.pool_shapes(NB * R, Hkv, D, BS, "bf16")
    kd = torch.randn(ks, dtype=torch.bfloat16, device=dev, generator=g)
    vd = torch.randn(vs, dtype=torch.bfloat16, device=dev, generator=g)
    stream = torch.cuda.current_stream()
    lens_d = torch.from_numpy(lens).to(dev)
    use_groups = not args.no_prefix_groups
    steps = []
    for r in range(R):
        tab_d = torch.from_numpy(table + r * NB).to(dev)
        pairs_d = torch.from_numpy(pairs + r * NB).to(dev)
        q = torch.randn((n, Hq, D), dtype=torch.bfloat16, device=dev, generator=g)
        kn = torch.randn((n, Hkv, D), dtype=torch.bfloat16, device=dev, generator=g)
        vn = torch.randn((n, Hkv, D), dtype=torch.bfloat16, device=dev, generator=g)
        out = torch.empty_like(q)
        copy = pa.prepare_copy_blocks(kd, vd, pairs_d, stream=stream, head_dim=D)
        if use_groups:
            gst = torch.tensor([0, n], dtype=torch.int32, device=dev)
            pl = torch.tensor([shared], dtype=torch.int32, device=dev)
            dec = pa.prepare_decode_prefix(out, q, kd, vd, tab_d, lens_d, plan["scale"], max_ctx, gst,
                                           pl, n, shared, stream=stream, k_new=kn, v_new=vn,
                                           min_prefix_len=shared)
        else:
            dec = pa.prepare_decode(out, q, kd, vd, tab_d, lens_d, plan["scale"], max_ctx,
                                    stream=stream, k_new=kn, v_new=vn, context_lens_host=lens)
        steps.append((copy, dec))

    def step(i):
        copy, dec = steps[i % R]
        copy()
        dec()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    per_tok = 2 * Hkv * D * 2
    logical = int(lens.sum()) * per_tok
    unique = (shared + int((lens - shared).sum())) * per_tok
    copy_bytes = 2 * len(pairs) * 2 * Hkv * D * BS * 2  # K and V tiles, read and written
    alg = (unique if use_groups else logical) + copy_bytes + 2 * n * Hq * D * 2 + n * per_tok
    result = {
        "metric": "paged decode attention: achieved KV GB/s (% HBM peak) and seq-steps/s",
        "value": round(logical / sec / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5), "gpu_ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "seq_steps_per_s": round(n / sec, 1),
        "unique_kv_gbs": round(unique / sec / 1e9, 2),
        "config": {"workload": "cow_bf16" + ("" if use_groups else " (pa_decode, no prefix groups)"),
                   "num_seqs": n, "forked_siblings": n, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": BS, "shared_prefix_tokens": shared, "cow_pairs": int(len(pairs)),
                   "context_tokens": int(lens.sum()), "replicas": R,
                   "logical_kv_bytes_per_step": logical, "unique_kv_bytes_per_step": unique,
                   "step": "pa_copy_blocks(%d pairs) + %s(fused append)"
                           % (len(pairs), "pa_decode_prefix" if use_groups else "pa_decode")},
        "roofline": {"kernel": "copy_blocks_kernel + " + ("prefix_suffix_kernel" if use_groups
                                                          else "decode_mfma_kernel") + " + merge_kernel",
                     "bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(ms, 5), "algorithmic_bytes_per_launch": alg},
        "host_bookkeeping_us": round(host_us, 2),
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_prefill(case, kd, vd, budget_s):
    """The fp64 CPU oracle on a bounded sample: the first 64 rows of sequence 0
    (all heads), repeated until ~budget_s of CPU work."""
    import torch
    from oracle import oracle
    from paged_kv_cache_328_amd import workloads as wl
    cores = len(os.sched_getaffinity(0))
    n = int(min(64, case.query_start[1]))
    c = int(case.context_lens[0]) - int(case.query_start[1]) + n  # rows keep their positions
    nblk = -(-c // case.BS)
    used = case.block_tables[0, :nblk].astype(np.int64)
    idx = torch.from_numpy(used).to(kd.device)
    tables = np.arange(nblk, dtype=np.int32).reshape(1, nblk)
    lens = np.array([c], np.int32)
    qs = np.array([0, n], np.int32)
    q = np.ascontiguousarray(case.q[:n])
    i8 = wl.is_q8(case.kv_dtype)
    as_bytes = (lambda x: x.view(torch.uint8)) if i8 else (lambda x: x)  # 8-bit pools as bytes
    kc = as_bytes(kd).index_select(0, idx).cpu().contiguous().numpy()
    vc = as_bytes(vd).index_select(0, idx).cpu().contiguous().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        if i8:
            oracle.prefill_i8(q, case.dtype, kc, vc, tables, lens, qs, case.scale, case.D, case.BS,
                              num_threads=cores, fmt=case.kv_dtype)
        else:
            oracle.prefill(q, kc, vc, tables, lens, qs, case.scale, case.dtype, num_threads=cores)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / reps
    flops = 4 * case.D * case.Hq * sum(range(c - n + 1, c + 1))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"pa_prefill of the first {n} chunk rows of sequence 0 (positions {c - n}..{c - 1}, "
                      f"all {case.Hq} query heads), {reps} repetitions in {reps * dt:.1f} s, "
                      f"{cores} OpenMP threads"}


def measured_traffic(workload, partition_size, fused, host_lens):
    """HBM bytes per pa_decode call (pass 1 and, when split, the merge) from
    the committed rocprofv3 byte counters (profiles/traffic.json: FETCH_SIZE
    and WRITE_SIZE, each scaled by what the counter reads for a plain copy of
    known size), or None when no record matches this launch or the kernel
    sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if (not rec or rec.get("partition_size") != partition_size or rec.get("fused_append") != fused
            or rec.get("host_context_lens") != host_lens):
        return None
    return rec["bytes_per_launch"] if kernel_source_digest() == rec["kernel_sources_sha256"] else None


def kernel_source_digest():
    """SHA-256 of the decode kernels' source with comments and blank space
    removed: byte counters stay valid across comment-only edits and go stale
    on any change of code."""
    import hashlib
    h = hashlib.sha256()
    for f in ["paged_kv_cache_328_amd/csrc/pa_decode.hip", "paged_kv_cache_328_amd/csrc/pa_device.h"]:
        h.update(_strip_comments(open(os.path.join(ROOT, f), encoding="utf-8").read()).encode())
    return h.hexdigest()


def _strip_comments(src):
    """C++ source without // and /* */ comments (string and character
    literals kept), every run of white space folded to one blank."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, kd, vd, budget_s):
    """The fp64 CPU oracle on a bounded sample: the first sequences of replica
    0 (all heads), repeated until ~2/3 of budget_s on every core of the
    process's affinity mask, then until ~1/3 of it on one core."""
    import torch
    from oracle import oracle
    from paged_kv_cache_328_amd import workloads as wl
    dtype = case.dtype
    cores = len(os.sched_getaffinity(0))
    n = min(case.S, 4)
    t = case.block_tables[0][:n]
    lens = np.ascontiguousarray(case.context_lens[:n])
    used = np.unique(np.concatenate([t[s, :-(-int(lens[s]) // case.BS)] for s in range(n)]))
    remap = {int(b): i for i, b in enumerate(used)}
    tables = np.zeros((n, t.shape[1]), np.int32)
    for s in range(n):
        for j in range(-(-int(lens[s]) // case.BS)):
            tables[s, j] = remap[int(t[s, j])]
    idx = torch.from_numpy(used.astype(np.int64)).to(kd.device)

    def host(x):
        if x.dtype == torch.float8_e4m3fn:  # FP8 pools as bytes
            x = x.view(torch.uint8)
        x = x.index_select(0, idx).cpu().contiguous()
        return (x.view(torch.int16).numpy().view(np.uint16)
                if x.dtype == torch.bfloat16 else x.numpy())

    kc, vc = host(kd), host(vd)
    q = np.ascontiguousarray(case.q[0][:n])
    i8 = wl.is_q8(case.kv_dtype)
    per_tok = (case.D + 4) if i8 else case.D * wl.ELEM_BYTES[dtype]

    def timed(rows, threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            if i8:
                oracle.decode_i8(q[rows], dtype, kc, vc, tables[rows], lens[rows], case.scale, case.D,
                                 case.BS, num_threads=threads, fmt=case.kv_dtype)
            else:
                oracle.decode(q[rows], kc, vc, tables[rows], lens[rows], case.scale, dtype,
                              num_threads=threads)
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = (time.perf_counter() - t0) / reps
        nseq = rows.stop - rows.start
        kv = 2 * int(lens[rows].sum()) * case.Hkv * per_tok
        return kv / dt / 1e9, nseq / dt, reps, reps * dt

    gbs, sps, reps, sec = timed(slice(0, n), cores, budget_s * 2 / 3)
    gbs1, sps1, reps1, sec1 = timed(slice(0, 1), 1, budget_s / 3)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seq_steps_per_s": round(sps, 3), "cpu_model": cpu_model(),
            "value_1core": round(gbs1, 4), "seq_steps_per_s_1core": round(sps1, 3),
            "sample": f"pa_decode of sequences 0..{n - 1} of replica 0 ({int(lens.sum())} context "
                      f"tokens, all {case.Hq} query heads), {reps} repetitions in {sec:.1f} s, "
                      f"{cores} OpenMP threads; 1 core: sequence 0 ({int(lens[0])} tokens), "
                      f"{reps1} repetitions in {sec1:.1f} s"}


if __name__ == "__main__":
    main()
