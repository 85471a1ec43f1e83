#!/usr/bin/env python3
"""Throughput of the whole merge -> keep -> lengths -> scan -> emit path on one
MI355X, on the 8M+8M base64-key workload (or another named workload).

One step is one pass of the whole hot path over inputs already resident in
HBM.  Paths:
  fused (default)  em_partition, em_merge_lengths (co-rank, merge, keep-newer,
                   LCPs, lengths, bit offsets), em_emit_merged (emission); no
                   host read inside a step
  merge            em_partition, em_merge_keep, host read of S, em_fc_lengths,
                   em_scan, host read of T, em_emit
  collision        em_collision_rank_mode (--collision-mode 512, 2048,
                   512-tiled, 512-compact) in place of partition + merge_keep
W untimed warm-up steps, then exactly K timed steps between two device
synchronisations.  Prints one JSON line.

  value      merged records/s = (|A| + |B|) * K / elapsed
  GB/s       B_io / step time, B_io = both sides' key and value arenas, u32
             offsets and tombstone bytes, plus the payload bytes
  roofline   the dominant kernel's algorithmic bytes per launch over its
             average launch time (HIP events on the launch stream); the
             algorithmic bytes are the input and output bytes the call must
             move (arenas, offsets, tombstone flags, payload), not the
             references, lengths and offsets one kernel hands to another
  parity     before any timing, the payload, S and T of the timed
             configuration are compared with the oracle's digests of the same
             workload (tests/golden/full_size_digests.json) or, for a scaled
             workload, with the oracle run on the same host buffers; a
             mismatch exits with status 3 and no timing
  cpu_baseline  the CPU oracle (one thread) on the same host buffers as the
             timed step, its payload compared with the GPU's
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "merged records/s and pipeline GB/s (% of HBM peak) at 8M+8M string keys, 1 GPU"


# the kernel each timed call launches (em_merge_lengths also runs a one-workgroup
# scan of partition totals, about 1% of its time)
KERNEL_OF = {"em_partition": "k_partition", "em_merge_keep": "k_merge_keep", "em_fc_lengths": "k_fc_lengths",
             "em_scan": "k_scan", "em_emit": "k_emit",
             "em_collision_rank_mode": "k_mark, rank build, scatter or compact + merge",
             "em_merge_lengths": "k_merge_len + k_tile_scan", "em_emit_merged": "k_emit",
             "em_merge_fc_onepass": "k_onepass + k_op_edges",
             "em_merge_fc": "k_merge_len + k_tile_scan + k_emit"}


def measured_traffic(call, workload_name):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of the call's kernel,
    from profiles/traffic_<workload>.md, while its sources still hash to the
    fingerprint recorded there by the rocprofv3 run (else None)."""
    from merge_front_coded_amd import profiling
    return profiling.measured_traffic(call, workload_name)


def make_pipeline(A, B, path="fused", items=None, coarse_parts=0, collision_mode="512-tiled"):
    """The pipeline in the configuration the benchmark times: the fused paths
    keep no per-record arrays (final refs, ordinals, lengths, LCPs and offsets
    are not written; the emitter's inputs live in the workspace)."""
    import merge_front_coded_amd as em
    fused = path in ("fused", "onepass", "onecall")
    extra = {"coarse_parts": coarse_parts} if (fused and coarse_parts) else {}
    if path == "collision":
        extra["collision_mode"] = collision_mode
    if path == "onepass":
        extra["one_pass"] = True
    if path == "onecall":
        extra["one_call"] = True
    return em.Pipeline(A, B, items_per_part=items or None, path="fused" if fused else path,
                       keep_all=not fused, **extra)


def payload_digest(pl) -> str:
    import hashlib
    return hashlib.sha256(pl.payload_bytes()).hexdigest()


def reference_digest(workload_id, scale=1.0):
    """The oracle's (S, T, payload SHA-256) for a full-size workload, from the
    digests tests/golden/make_full_size_digests.py wrote (None if absent)."""
    path = os.path.join(ROOT, "tests", "golden", "full_size_digests.json")
    if scale != 1.0 or not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f).get(str(workload_id))
    return None if d is None else (d["S"], d["T"], d["payload"])


def oracle_run(Ah, Bh):
    """The CPU oracle on the given host buffers: merge, keep-newer, bitwise
    encoding.  Returns (S, T, payload SHA-256, seconds)."""
    import hashlib
    import oracle
    t0 = time.perf_counter()
    refs = oracle.merge(Ah, Bh)
    final, _, _, S = oracle.keep(Ah, Bh, refs)
    _, _, _, T, payload = oracle.encode(Ah, Bh, final)
    dt = time.perf_counter() - t0
    return S, T, hashlib.sha256(payload.tobytes()).hexdigest(), dt


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)  # (about 50 ms timed: enough steps to average out run-to-run spread)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="workload number 1..5 (3 = 8M+8M)")
    ap.add_argument("--path", choices=("fused", "onecall", "onepass", "merge", "collision"), default="fused")
    ap.add_argument("--items", type=int, default=0,
                    help="outputs per merge partition (0: chosen from the mean key length)")
    ap.add_argument("--collision-mode", choices=("512", "2048", "512-tiled", "512-compact"),
                    default="512-tiled", help="collision path: rank layout and A placement")
    ap.add_argument("--coarse-parts", type=int, default=0,
                    help="fused path: partitions per coarse partition (0: library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scale", type=float, default=1.0,
                    help="fraction of the workload's record counts (parity then comes from the oracle run here)")
    ap.add_argument("--navigation", action="store_true",
                    help="also time em_ef_navigation (the output navigation) on the step's outputs")
    ap.add_argument("--byte-profile", action="store_true",
                    help="also time the byte-profile encoding (em_bp_lengths, em_scan, em_bp_emit) of the step's "
                         "survivors")
    ap.add_argument("--fcin", action="store_true",
                    help="also time decoding the step's payload back into arenas (em_fcin_parse + _materialize)")
    ap.add_argument("--owner-search", action="store_true",
                    help="also time comparing the equal keys of the two inputs, each front-coded alone, through "
                         "their literal owners (em_fcin_compare) against materializing both inputs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the plain 1 GiB device copy (the default; kept for the counter-scaling commands)")
    ap.add_argument("--no-copy", action="store_true",
                    help="skip the plain 1 GiB device copy that measures the achievable copy rate")
    return ap.parse_args()


def side_bytes(h) -> int:
    return int(h.keys.size + h.vals.size + h.key_off.nbytes + h.val_off.nbytes + h.tomb.size)


def algorithmic_bytes(Ah, Bh, pl, path):
    """Per-launch algorithmic bytes of each call (what it must read and write once)."""
    import numpy as np
    S, T, N = pl.S, pl.T, Ah.n + Bh.n
    keys = int(Ah.keys.size + Bh.keys.size)
    offs = 4 * (Ah.n + 1 + Bh.n + 1)
    final = pl.final_host if pl.path == "fused" else pl.host("final", S)
    lcp = pl.lcp_host if pl.path == "fused" else pl.host("lcp", S)
    nA = Ah.n
    isA = final < nA
    ia = final[isA].astype(np.int64)
    ib = final[~isA].astype(np.int64) - nA
    klen = np.empty(S, np.int64)
    klen[isA] = (Ah.key_off[ia + 1].astype(np.int64) - Ah.key_off[ia])
    klen[~isA] = (Bh.key_off[ib + 1].astype(np.int64) - Bh.key_off[ib])
    vlen = np.empty(S, np.int64)
    vlen[isA] = (Ah.val_off[ia + 1].astype(np.int64) - Ah.val_off[ia])
    vlen[~isA] = (Bh.val_off[ib + 1].astype(np.int64) - Bh.val_off[ib])
    suffix_bytes = int(np.sum(klen - (lcp.astype(np.int64) >> 3)))
    survivor_key_bytes = int(np.sum(klen))
    value_bytes = int(np.sum(vlen))
    payload = 4 * ((T + 31) // 32)
    vmeta = 4 * (Ah.n + 1 + Bh.n + 1) + int(Ah.tomb.size + Bh.tomb.size)  # value offsets, tombstones
    out = {
        # merge: every key byte, both offset arrays; writes refs and both ordinal arrays
        "em_merge_keep": keys + offs,
        # lengths: the survivors' keys, offsets and tombstones
        "em_fc_lengths": survivor_key_bytes + S * (8 + 8 + 1),
        "em_scan": 0,
        "em_emit": S * (8 + 8 + 1) + suffix_bytes + value_bytes + payload,
        "em_partition": 0,
        "em_collision_rank_mode": keys + offs,
        # the whole path: every input byte once, the payload once
        "em_merge_fc": side_bytes(Ah) + side_bytes(Bh) + payload,
        # merge, keep, LCPs, lengths: every key byte, key and value offsets,
        # tombstones (the references, LCPs and offsets it hands to the
        # emitter are not counted)
        "em_merge_lengths": keys + offs + vmeta,
        # emission: the survivors' key_off and val_off pairs and tombstone
        # flags, key suffixes and values; writes the payload (the references,
        # LCPs and offsets it reads from the first kernel are not counted)
        "em_emit_merged": S * (8 + 8 + 1) + suffix_bytes + value_bytes + payload,
        # the single pass: every input byte once, the payload once
        "em_merge_fc_onepass": side_bytes(Ah) + side_bytes(Bh) + payload,
    }
    return out


def _key_hash(X, weights):
    """A 64-bit hash of every key of a device side (a weighted sum of its
    bytes, one random weight per byte position, wrapping, mixed with the
    length): equal keys hash alike."""
    import torch
    off = X.key_off[:X.n + 1].long()
    lens = off[1:] - off[:-1]
    nbytes = int(off[-1].item())
    pos = torch.arange(nbytes, device=off.device) - torch.repeat_interleave(off[:-1], lens)
    c = torch.zeros(nbytes + 1, dtype=torch.int64, device=off.device)
    c[1:] = torch.cumsum(X.keys[:nbytes].long() * weights[pos], 0)
    return (c[off[1:]] - c[off[:-1]]) * 1000003 + lens


def owner_search_leg(A, B, items, steps, stream, replaced):
    """A merge of the two inputs given front-coded instead of as arenas:
    each input front-coded alone by this path and parsed; the pairs of equal
    keys, whose comparisons every merge of the two must finish past its eight
    cached bytes, compared from byte 8 by owner search (em_fcin_compare),
    beside materializing both inputs into arenas.  Timings only; the
    comparisons' parity is covered by the tests."""
    import torch
    import gen
    import merge_front_coded_amd as em
    empty = em.DeviceSide.from_host(gen.side_from_records([]))
    ins = []
    for X in (A, B):
        px = em.Pipeline(X, empty, items_per_part=items, path="fused", keep_all=True)
        px.run()
        torch.cuda.synchronize()
        wsx = torch.empty(max(em.em_fcin_workspace_bytes(px.S), 256), dtype=torch.uint8, device="cuda")
        tot = torch.zeros(3, dtype=torch.int64, device="cuda")
        em.em_fcin_parse(px.payload, px.T, px.S, tot, wsx, off=px.off)
        kb, vb, err = (int(x) for x in tot.cpu())
        assert err == 0 and px.S == X.n
        ins.append((px, wsx, tot, kb, vb))
    # the pairs of equal keys: every merge finishes these comparisons past its cache
    maxlen = int(max((A.key_off[1:A.n + 1] - A.key_off[:A.n]).max().item() if A.n else 0,
                     (B.key_off[1:B.n + 1] - B.key_off[:B.n]).max().item() if B.n else 0))
    g = torch.Generator(device="cuda").manual_seed(12345)
    weights = torch.randint(-(1 << 62), 1 << 62, (maxlen + 1,), generator=g, dtype=torch.int64, device="cuda")
    ha, order = torch.sort(_key_hash(A, weights))
    hb = _key_hash(B, weights)
    pos = torch.searchsorted(ha, hb).clamp(max=max(A.n - 1, 0))
    hit = ha[pos] == hb
    ia = order[pos[hit]].to(torch.int32).contiguous()
    jb = torch.nonzero(hit).flatten().to(torch.int32).contiguous()
    del ha, hb, order, pos, hit
    n = int(ia.numel())
    lcp = torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    cmp = torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    (xa, wa, ta, kba, vba), (xb, wb, tb, kbb, vbb) = ins
    ev_c, ev_m, ev_p = [], [], []
    keys_a = torch.zeros(kba + 64, dtype=torch.uint8, device="cuda")
    keys_b = torch.zeros(kbb + 64, dtype=torch.uint8, device="cuda")
    vals_a = torch.zeros(vba + 64, dtype=torch.uint8, device="cuda")
    vals_b = torch.zeros(vbb + 64, dtype=torch.uint8, device="cuda")
    offs = [torch.empty(x.S + 1, dtype=torch.int32, device="cuda") for x in (xa, xa, xb, xb)]
    tombs = [torch.empty(max(x.S, 1), dtype=torch.uint8, device="cuda") for x in (xa, xb)]
    pfx = [torch.empty(max(x.S, 1), dtype=torch.int64, device="cuda") for x in (xa, xb)]
    for it in range(steps + 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        em.em_fcin_compare(xa.payload, xa.S, wa, xb.payload, xb.S, wb, n, ia, jb, 8, lcp_bits=lcp, cmp=cmp,
                           stream=stream)
        e[1].record(stream)
        em.em_fcin_materialize(xa.payload, xa.S, keys_a, offs[0], vals_a, offs[1], tombs[0], ta, wa, stream=stream)
        em.em_fcin_materialize(xb.payload, xb.S, keys_b, offs[2], vals_b, offs[3], tombs[1], tb, wb, stream=stream)
        e[2].record(stream)
        em.em_fcin_prefix8(xa.payload, xa.S, pfx[0], wa, stream=stream)
        em.em_fcin_prefix8(xb.payload, xb.S, pfx[1], wb, stream=stream)
        e[3].record(stream)
        if it:
            ev_c.append((e[0], e[1]))
            ev_m.append((e[1], e[2]))
            ev_p.append((e[2], e[3]))
    torch.cuda.synchronize()
    assert int(ta[2].item()) == 0 and int(tb[2].item()) == 0
    equal = int((cmp[:n] == 0).sum().item()) if n else 0

    def avg(ev):
        return sum(x.elapsed_time(y) for x, y in ev) / len(ev)

    return {"calls": ["em_fcin_compare", "em_fcin_materialize", "em_fcin_prefix8"],
            "pairs": n, "pairs_equal": equal, "replaced_records": replaced,
            "compare_from_byte_8_ms": avg(ev_c), "materialize_both_inputs_ms": avg(ev_m),
            "prefix_cache_from_owners_both_inputs_ms": avg(ev_p)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the path is single-device "
                                   "(see the sharding note in the design document)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import gen
    import merge_front_coded_amd as em

    w = gen.WORKLOADS[args.workload]
    if args.scale != 1.0:
        w = w.scaled(args.scale)
    t_gen = time.perf_counter()
    Ah, Bh = gen.make(w)
    t_gen = time.perf_counter() - t_gen
    print(f"# generated {w.name}: {Ah.n}+{Bh.n} records in {t_gen:.1f}s", file=sys.stderr, flush=True)
    A = em.DeviceSide.from_host(Ah)
    B = em.DeviceSide.from_host(Bh)
    fused = args.path in ("fused", "onecall", "onepass")
    extra = {"coarse_parts": args.coarse_parts} if (fused and args.coarse_parts) else {}
    pl = make_pipeline(A, B, args.path, args.items, args.coarse_parts, args.collision_mode)
    torch.cuda.synchronize()

    # ---- parity of the timed configuration, before any timing ----
    pl.run()
    torch.cuda.synchronize()
    gpu_sha = payload_digest(pl)
    ref = reference_digest(args.workload, args.scale)
    oracle_result = None
    if ref is not None:
        parity_src = f"tests/golden/full_size_digests.json[{args.workload}] (S, T, payload SHA-256)"
    else:
        print("# running the CPU oracle on the same host buffers for parity", file=sys.stderr, flush=True)
        oracle_result = oracle_run(Ah, Bh)
        ref = oracle_result[:3]
        parity_src = "CPU oracle run on the same host buffers (S, T, payload SHA-256)"
    if (pl.S, pl.T, gpu_sha) != tuple(ref):
        print(json.dumps({"error": "parity check failed before timing", "workload": w.name, "path": args.path,
                          "got": {"S": pl.S, "T": pl.T, "payload_sha256": gpu_sha},
                          "want": {"S": ref[0], "T": ref[1], "payload_sha256": ref[2]}, "reference": parity_src}),
              flush=True)
        sys.exit(3)
    print(f"# parity ok against {parity_src}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        pl.run()
    torch.cuda.synchronize()
    print(f"# warm-up done: S={pl.S} T={pl.T}", file=sys.stderr, flush=True)

    # per-call HIP events on the launch stream (torch's current stream, which
    # the binding passes to the library)
    stream = torch.cuda.current_stream()
    calls = {"merge": ["em_partition", "em_merge_keep", "em_fc_lengths", "em_scan", "em_emit"],
             "collision": ["em_collision_rank_mode", "em_fc_lengths", "em_scan", "em_emit"],
             "fused": ["em_partition", "em_merge_lengths", "em_emit_merged"],
             "onecall": ["em_partition", "em_merge_fc"],
             "onepass": ["em_partition", "em_merge_fc_onepass"]}[args.path]
    ev = {c: [] for c in calls}
    orig = {c: getattr(em.pipeline.em, c) for c in calls}

    def timed(name):
        f = orig[name]

        def g(*a, **k):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            f(*a, **k)
            e.record(stream)
            ev[name].append((s, e))
        return g

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    for c in calls:
        setattr(em.pipeline.em, c, timed(c))
    step_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    try:
        start.record(stream)
        for k in range(args.steps):
            pl.run(read_counts=not fused)  # the fused path needs no host read inside a step
            step_end[k].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
    finally:
        for c in calls:
            setattr(em.pipeline.em, c, orig[c])
    wall = time.perf_counter() - t0
    steps_ms = [(start if k == 0 else step_end[k - 1]).elapsed_time(step_end[k]) for k in range(args.steps)]
    complete_ms = None
    if fused:
        pl.read_counts()
        # the same steps with the host reading S and T after each (the
        # "complete" time; the six-call path's steps already include them)
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(args.steps):
            pl.run(read_counts=True)
        e0.record(stream)
        torch.cuda.synchronize()
        complete_ms = s0.elapsed_time(e0) / args.steps
        # the per-record arrays, for the algorithmic-byte count only (not timed)
        pl2 = em.Pipeline(A, B, items_per_part=pl.items, path="fused", keep_all=True,
                          one_pass=args.path == "onepass", **extra)
        pl2.run()
        torch.cuda.synchronize()
        assert (pl2.S, pl2.T) == (pl.S, pl.T)
        pl.final_host, pl.lcp_host = pl2.host("final", pl.S), pl2.host("lcp", pl.S)
        ord_A = pl2.host("ord_A", Ah.n)
        del pl2
    else:
        ord_A = pl.host("ord_A", Ah.n)
    # value bytes of the replaced A records: B_io less these is the minimum
    # any path must move
    a_vlen = np.diff(Ah.val_off.astype(np.int64))
    if Ah.tomb is not None:
        a_vlen = np.where(Ah.tomb != 0, 0, a_vlen)
    replaced_val_bytes = int(a_vlen[ord_A == 0xFFFFFFFF].sum())
    dev_ms = start.elapsed_time(end)
    ms_per_step = dev_ms / args.steps
    per_call_ms = {c: sum(s.elapsed_time(e) for s, e in ev[c]) / len(ev[c]) for c in calls}

    N = Ah.n + Bh.n
    payload_bytes = 4 * ((pl.T + 31) // 32)
    b_io = side_bytes(Ah) + side_bytes(Bh) + payload_bytes
    gbps = b_io / (ms_per_step * 1e-3) / 1e9
    alg = algorithmic_bytes(Ah, Bh, pl, args.path)
    dominant = max((c for c in calls if c != "em_partition"), key=lambda c: per_call_ms[c])
    ach = alg[dominant] / (per_call_ms[dominant] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "records/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": w.name, "nA": Ah.n, "nB": Bh.n, "items_per_part": pl.items,
                   "path": args.path, "parallelism": "single-gpu",
                   **({"coarse_items": pl.coarse} if fused else {}),
                   **({"collision_mode": args.collision_mode} if args.path == "collision" else {})},
        "survivors": pl.S,
        "payload_bits": pl.T,
        "B_io_bytes": b_io,
        "pipeline_GBps": gbps,
        "pipeline_hbm_frac": gbps / HBM_PEAK_GBPS,
        "survivors_per_s": pl.S / (ms_per_step * 1e-3),
        "wall_s_timed": wall,
        "per_call_ms": per_call_ms,
        "roofline": {"bound": "hbm", "kernel": KERNEL_OF[dominant], "call": dominant, "achieved": ach,
                     "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(dominant, w.name),
                     "algorithmic_bytes_per_launch": alg[dominant],
                     "avg_launch_ms": per_call_ms[dominant],
                     # the whole step: B_io over the step time
                     "pipeline": {"achieved": gbps, "frac": gbps / HBM_PEAK_GBPS, "bytes": b_io,
                                  "ms": ms_per_step}},
        "parity": {"reference": parity_src, "S": pl.S, "T": pl.T, "payload_sha256": gpu_sha, "match": True},
    }
    if args.navigation:
        # the output navigation built from this step's outputs (the step after
        # emit; not part of the timed step above)
        if fused:
            pn = em.Pipeline(A, B, items_per_part=pl.items, path="fused", keep_all=True, **extra)
            pn.run()
        else:
            pn = pl
        for _ in range(2):
            pn.ef_navigation()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(args.steps):
            pn.ef_navigation(stream)
        e.record(stream)
        torch.cuda.synchronize()
        nav = pn.nav.host()
        nav_ms = s.elapsed_time(e) / args.steps
        # reads: final refs, value offset pairs and tombstones for the common
        # width, the sampled offsets; writes: the sections
        nav_bytes = pn.S * (4 + 8 + 1) + 8 * nav["n"] + 8 * (nav["low_words"] + nav["high_words"] +
                                                             2 * nav["groups"] + nav["n_exceptions"])
        result["navigation"] = {"call": "em_ef_navigation", "ms": nav_ms, "entries": nav["n"], "L": nav["L"],
                                "width": nav["width"], "sparse_entries": nav["n_exceptions"],
                                "algorithmic_bytes": nav_bytes, "GBps": nav_bytes / (nav_ms * 1e-3) / 1e9}
        if pn is not pl:
            del pn
    if args.byte_profile:
        # the byte-profile encoding of this step's survivors (lengths and
        # width, scan, emit; T is known from the warm-up pass, so the timed
        # passes need no host read)
        if fused:
            pn = em.Pipeline(A, B, items_per_part=pl.items, path="fused", keep_all=True, **extra)
            pn.run()
        else:
            pn = pl
        W, T = pn.byte_profile()
        torch.cuda.synchronize()
        S = pn.S
        ev = []
        for it in range(args.steps + 1):
            a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            a.record(stream)
            em.em_bp_lengths(A, B, pn.final, pn.lcp, S, pn.bp_len, pn.bp_width, pn.bp_ws, stream)
            b.record(stream)
            em.em_scan(pn.bp_len, S, pn.bp_off, pn.ws, stream)
            c.record(stream)
            em.em_bp_emit(A, B, pn.final, pn.lcp, S, pn.bp_off, T, pn.bp_width, pn.bp_payload, pn.bp_over, stream)
            d.record(stream)
            if it:  # the first pass warms up
                ev.append((a, b, c, d))
        torch.cuda.synchronize()
        assert int(pn.bp_over.item()) == 0 and int(pn.bp_off[S].item()) == T
        part = [sum(x[k].elapsed_time(x[k + 1]) for x in ev) / len(ev) for k in range(3)]
        # one pass's minimum: refs, LCPs, key and value offset pairs and tags
        # read; the suffix and value bytes read (at most T); offsets and the
        # payload written
        bp_bytes = S * (4 + 4 + 8 + 8 + 1) + T + 8 * (S + 1) + T
        result["byte_profile"] = {"calls": ["em_bp_lengths", "em_scan", "em_bp_emit"], "width": W, "T_bytes": T,
                                  "lengths_ms": part[0], "scan_ms": part[1], "emit_ms": part[2],
                                  "ms": sum(part), "algorithmic_bytes": bp_bytes,
                                  "GBps": bp_bytes / (sum(part) * 1e-3) / 1e9}
        if pn is not pl:
            del pn
    if args.fcin:
        # the payload decoded back into arenas (the front-coded input path),
        # block starts from the record offsets; parse and materialize are
        # timed separately (the host reads the arena sizes between them)
        if fused:
            pn = em.Pipeline(A, B, items_per_part=pl.items, path="fused", keep_all=True, **extra)
            pn.run()
        else:
            pn = pl
        torch.cuda.synchronize()
        S, T = pn.S, pn.T
        ws = torch.empty(max(em.em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device="cuda")
        tot = torch.zeros(3, dtype=torch.int64, device="cuda")
        em.em_fcin_parse(pn.payload, T, S, tot, ws, off=pn.off)
        kb, vb, err = (int(x) for x in tot.cpu())
        assert err == 0, f"front-coded input: error bits {err}"
        keys = torch.zeros(kb + 64, dtype=torch.uint8, device="cuda")
        vals = torch.zeros(vb + 64, dtype=torch.uint8, device="cuda")
        key_off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
        val_off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
        tomb = torch.empty(max(S, 1), dtype=torch.uint8, device="cuda")
        pfx = torch.empty(max(S, 1), dtype=torch.int64, device="cuda")
        ev_p, ev_m, ev_c = [], [], []
        for it in range(args.steps + 1):
            a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            a.record(stream)
            em.em_fcin_parse(pn.payload, T, S, tot, ws, off=pn.off, stream=stream)
            b.record(stream)
            em.em_fcin_materialize(pn.payload, S, keys, key_off, vals, val_off, tomb, tot, ws, stream=stream)
            c.record(stream)
            em.em_fcin_prefix8(pn.payload, S, pfx, ws, stream=stream)
            d.record(stream)
            if it:  # the first pass warms up
                ev_p.append((a, b))
                ev_m.append((b, c))
                ev_c.append((c, d))
        torch.cuda.synchronize()
        assert int(tot[2].item()) == 0
        parse_ms = sum(x.elapsed_time(y) for x, y in ev_p) / len(ev_p)
        mat_ms = sum(x.elapsed_time(y) for x, y in ev_m) / len(ev_m)
        pfx_ms = sum(x.elapsed_time(y) for x, y in ev_c) / len(ev_c)
        fcin_bytes = (T + 7) // 8 + kb + vb + 8 * (S + 1) + S
        result["front_coded_input"] = {"calls": ["em_fcin_parse", "em_fcin_materialize"], "parse_ms": parse_ms,
                                       "materialize_ms": mat_ms, "key_bytes": kb, "value_bytes": vb,
                                       # the prefix cache filled from the literal owners, no key
                                       # arena (em_fcin_prefix8): its cost beside the materialization
                                       "prefix_cache_from_owners_ms": pfx_ms,
                                       "algorithmic_bytes": fcin_bytes,
                                       "GBps": fcin_bytes / ((parse_ms + mat_ms) * 1e-3) / 1e9}
        if pn is not pl:
            del pn
    if args.owner_search:
        result["owner_search"] = owner_search_leg(A, B, pl.items, args.steps, stream, A.n + B.n - pl.S)
    result["step_ms"] = {"median": float(np.median(steps_ms)), "min": min(steps_ms), "max": max(steps_ms)}
    result["ms_per_step_with_host_reads"] = complete_ms if fused else ms_per_step
    result["B_min_bytes"] = b_io - replaced_val_bytes
    result["pipeline_GBps_B_min"] = (b_io - replaced_val_bytes) / (ms_per_step * 1e-3) / 1e9
    if not args.no_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        result["copy_GBps"] = 2 * n * 10 / (s.elapsed_time(e) * 1e-3) / 1e9
    if not args.no_cpu_baseline:
        if oracle_result is None:
            print("# timing the CPU oracle on the same host buffers", file=sys.stderr, flush=True)
            oracle_result = oracle_run(Ah, Bh)
        oS, oT, osha, dt = oracle_result
        if (oS, oT, osha) != (pl.S, pl.T, gpu_sha):
            print(json.dumps({"error": "the CPU oracle's payload differs from the timed GPU payload",
                              "oracle": {"S": oS, "T": oT, "payload_sha256": osha}}), flush=True)
            sys.exit(3)
        result["parity"]["oracle_same_run"] = True
        result["cpu_baseline"] = {"value": N / dt, "unit": "records/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole timed workload ({w.name}: {Ah.n}+{Bh.n} records, the same "
                                            f"host buffers as the GPU step): merge + keep-newer + bitwise encode, "
                                            f"{dt:.1f} s on one thread; payload identical to the GPU's",
                                  "seconds": dt, "GBps": b_io / dt / 1e9, **host_cpu()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
