"""Dispatch sweep: time every kernel variant on a grid of shapes and report how
far the library's automatic choice is from the fastest one.

    python -m precision_gemm_amd.tune [--shapes default|quick|wide|mid] [--hbm] [--json out.json]
                                      [--write-overrides overrides.json [--min-regret 0.02]
                                       [--both-modes]]
                                      [--load-overrides overrides.json]
    python -m precision_gemm_amd.tune --splitk [--json out.json]

For each shape every applicable variant is timed on the same device buffers,
interleaved over several rounds (so clock drift hits all variants alike); a
variant's time is the median of its rounds. A round replays a HIP graph that
holds a run of back-to-back launches of the variant (so the host's per-call
cost does not pace short kernels), between two HIP events, after an untimed
replay of the same graph. With --hbm the launches of the run cycle through
copies of A, B and C, at least four and at least 1.25 GiB in all, so each
launch reads operands that the others have pushed out of L2 and the 256 MB
Infinity Cache: the operands come from HBM, as in a real workload whose
operands do not stay cached.
The report lists the fastest variant, the one `sgemm_select_variant` picks and
the regret (automatic time / fastest time - 1). The cost model in the host
dispatcher is fitted to these tables. --write-overrides turns the shapes it
misses into a per-shape table for `sgemm_set_dispatch_overrides`, which the
automatic choice then follows for exactly those shapes.

Inputs are U(-1, 1) fp32 from a fixed seed. Only whether beta is zero changes
the work (C is read iff beta != 0), so a nonzero beta is timed as 1.0, which
keeps C bounded over the repeated launches (C is not restored between them).
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
import time

# (transA, transB, M, N, K, batch, beta)
DEFAULT_SHAPES = [
    (0, 0, 128, 128, 128, 1, 0.0),
    (0, 0, 512, 512, 512, 1, 0.0),
    (0, 0, 768, 768, 768, 1, 0.0),
    (0, 0, 1024, 1024, 1024, 1, 3.0),
    (1, 1, 1000, 1000, 1000, 1, 1.0),
    (0, 0, 1536, 1536, 1536, 1, 0.0),
    (0, 0, 2048, 2048, 2048, 1, 0.0),
    (0, 0, 2048, 2048, 512, 1, 0.0),
    (0, 0, 2560, 2560, 2560, 1, 0.0),
    (0, 0, 3072, 3072, 3072, 1, 0.0),
    (0, 0, 4092, 4092, 4092, 1, 0.5),
    (0, 0, 4096, 4096, 1024, 1, 0.0),
    (0, 0, 6144, 6144, 6144, 1, 0.0),
    (0, 0, 8192, 8192, 8192, 1, 0.0),
    (0, 0, 1024, 1024, 4096, 1, 0.0),
    (0, 0, 512, 512, 8192, 1, 0.0),
    (1, 0, 512, 512, 520, 64, 0.0),
    (0, 0, 256, 256, 256, 128, 0.0),
    (0, 0, 512, 512, 2048, 8, 0.0),
    (0, 1, 16384, 64, 4096, 1, 1.0),
    (0, 1, 16384, 64, 2048, 1, 1.0),
    (0, 1, 64, 8192, 4096, 1, 0.0),
    (0, 0, 16384, 64, 4096, 1, 0.0),
    (1, 1, 16384, 64, 4096, 1, 0.0),
]
QUICK_SHAPES = [DEFAULT_SHAPES[i] for i in (3, 6, 10, 16, 19)]
# Shapes the cost model was not fitted on: non-square, every transpose pair,
# odd sizes, short K, batches, and narrow products (one dimension 1 to 32).
WIDE_SHAPES = [
    (1, 0, 4096, 4096, 4096, 1, 0.0), (0, 1, 4096, 4096, 4096, 1, 1.0),
    (1, 1, 4096, 4096, 4096, 1, 0.0), (0, 0, 3000, 3000, 3000, 1, 0.0),
    (0, 0, 5000, 5000, 5000, 1, 0.5), (1, 0, 2000, 3000, 1000, 1, 0.0),
    (0, 0, 8192, 1024, 4096, 1, 0.0), (0, 0, 1024, 8192, 4096, 1, 0.0),
    (0, 1, 16384, 512, 2048, 1, 0.0), (0, 0, 512, 16384, 2048, 1, 0.0),
    (0, 0, 4096, 4096, 256, 1, 0.0), (0, 0, 8192, 8192, 128, 1, 1.0),
    (0, 0, 2048, 2048, 64, 1, 0.0), (0, 0, 1536, 1536, 4096, 1, 0.0),
    (0, 0, 2304, 2304, 2304, 1, 0.0), (0, 0, 3584, 3584, 3584, 1, 0.0),
    (1, 0, 256, 256, 1024, 256, 0.0), (0, 1, 128, 128, 2048, 512, 0.0),
    (0, 0, 1024, 1024, 1024, 16, 0.0), (0, 0, 384, 768, 3072, 32, 0.0),
    (0, 1, 32768, 128, 4096, 1, 0.0), (0, 0, 128, 32768, 4096, 1, 0.0),
    (0, 0, 96, 96, 96, 1, 0.0), (0, 0, 640, 480, 2000, 1, 0.0),
    (0, 0, 16384, 1, 4096, 1, 0.0), (0, 0, 16384, 16, 4096, 1, 0.0),
    (0, 1, 65536, 32, 4096, 1, 0.0), (0, 0, 32, 16384, 4096, 1, 0.0),
    (1, 0, 8, 65536, 2048, 1, 0.0), (0, 0, 4096, 24, 1024, 4, 0.0),
    (0, 1, 16384, 4, 4096, 1, 0.0), (0, 0, 4096, 8, 4096, 1, 0.0),
    (0, 1, 4, 16384, 4096, 1, 0.0), (0, 1, 8, 16384, 4096, 1, 0.0),
]

# Mid-size grids over deep K (one to five rounds of tiles), where the 64 x 32
# streaming tile competes with the 64 x 64 tiles through the cost model.
MID_SHAPES = [
    (0, 0, 1536, 1536, 4096, 1, 0.0), (0, 0, 1536, 1536, 8192, 1, 0.0),
    (0, 0, 1280, 1280, 4096, 1, 0.0), (0, 0, 1792, 1792, 4096, 1, 0.0),
    (0, 0, 1536, 1536, 2048, 1, 0.0), (0, 0, 2048, 1024, 4096, 1, 0.0),
    (0, 0, 1152, 1152, 4096, 1, 0.0), (0, 0, 1536, 1536, 3072, 1, 0.0),
    (1, 0, 1536, 1536, 4096, 1, 0.0), (0, 1, 1536, 1536, 4096, 1, 0.0),
    (0, 0, 1024, 1024, 8192, 1, 0.0), (0, 0, 2560, 2560, 4096, 1, 0.0),
    (0, 0, 768, 768, 4096, 1, 0.0), (0, 0, 896, 896, 4096, 1, 0.0),
    (0, 0, 1536, 768, 4096, 2, 0.0), (0, 0, 640, 640, 640, 1, 0.0),
    (0, 0, 512, 256, 2048, 1, 0.0), (0, 0, 256, 256, 512, 2, 0.0),
]


# Bytes of operand copies the --hbm mode cycles through (five times the
# Infinity Cache).
ROTATE_BYTES = 5 << 28


def time_variant(torch, pg, stream, call, launches: int) -> float:
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        call()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / launches * 1e3  # microseconds


def graph_of(torch, dev, launch, n: int):
    """A HIP graph holding launch(0), ..., launch(n - 1) on its capture stream
    (launch takes the copy index and the stream handle)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                launch(i, side.cuda_stream)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    return g


def time_graph(torch, stream, g, launches: int) -> float:
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / launches * 1e3  # microseconds


def sweep(shapes, rounds: int = 3, target_ms: float = 20.0, hbm: bool = False, out=sys.stdout):
    import torch

    import precision_gemm_amd as pg

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    gen = torch.Generator(device=dev).manual_seed(1234)

    # Let the clock ramp up before the first measurement.
    X = torch.rand(4096, 4096, device=dev, generator=gen)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.4:
        pg.sgemm(0, 0, 4096, 4096, 4096, 1.0, X, 4096, X, 4096, 0.0, X, 4096)
        torch.cuda.synchronize(dev)
    del X

    results = []
    for tA, tB, M, N, K, batch, beta in shapes:
        beta_t = 1.0 if beta != 0.0 else 0.0
        per = 4 * batch * (M * K + K * N + M * N)
        # (at most 2048 copies: for the smallest problems that is still more
        # than the Infinity Cache holds, and it bounds the graph's length)
        copies = max(4, min(2048, -(-ROTATE_BYTES // per))) if hbm else 1

        def buf(rows, cols):
            return torch.rand((copies, batch, rows, cols), device=dev, generator=gen) * 2 - 1
        A = buf(K, M) if tA else buf(M, K)
        B = buf(N, K) if tB else buf(K, N)
        C = buf(M, N)
        lda, ldb = A.shape[3], B.shape[3]
        sa, sb, sc = A.stride(1), B.stride(1), C.stride(1)
        # The library first describes a stride-1 vector operand as contiguous
        # in k; its choice, and whether the GEMV kernels take the call (N == 1
        # or M == 1 with the vector contiguous in k; a few vectors, 2 to 8,
        # against a matrix contiguous in k, or the mirror), follow that
        # description.
        cA, cB = tA, tB
        if N == 1 and tB == 0 and ldb == 1 and 1 < K:
            cB = 1
        if M == 1 and tA == 1 and lda == 1 and 1 < K:
            cA = 0
        gemv_ok = ((N == 1 and cB == 1) or (M == 1 and cA == 0) or
                   (2 <= N <= 8 and cA == 0 and (cB == 1 or N % 4 == 0)) or
                   (2 <= M <= 8 and cB == 1 and (cA == 0 or M % 4 == 0)))
        auto = pg.sgemm_select_variant(cA, cB, M, N, K, batch, 1, cus)
        variants = [v for v in range(pg.VARIANT_COUNT)
                    if v not in (pg.VARIANT_S64x64_V1, pg.VARIANT_W64x64, pg.VARIANT_W64x64_V1,
                                 pg.VARIANT_P128x128, pg.VARIANT_P64x64)
                    and (v != pg.VARIANT_GEMV or gemv_ok)]

        def launcher(v):
            def launch(i, stream_handle):
                j = i % copies
                st = pg.sgemm_strided_batched_variant(
                    tA, tB, M, N, K, 1.0, A[j], lda, B[j], ldb, beta_t, C[j], N, batch, sa, sb,
                    sc, v, stream=stream_handle, check=False)
                if st != 0:
                    raise pg.SgemmError(st, pg.sgemm_status_string(st))
            return launch
        launches, graphs = {}, {}
        for v in variants:
            launch = launcher(v)
            one_call = (lambda lv=launch: lv(0, stream.cuda_stream))
            for _ in range(2):
                one_call()
            torch.cuda.synchronize(dev)
            one = time_variant(torch, pg, stream, one_call, 3)
            n = max(3, min(500, int(target_ms * 1e3 / max(one, 1.0))))
            if hbm:
                n = max(n, 2 * copies)
            launches[v] = n
            graphs[v] = graph_of(torch, dev, launch, n)
        # Each timed replay follows an untimed one of the same graph: the
        # clock settles differently after an under-filled grid (a large tile
        # on a small problem leaves most CUs idle) and needs a few ms to
        # return to the level the variant itself sustains.
        times = {v: [] for v in variants}
        for _ in range(rounds):
            for v in variants:
                time_graph(torch, stream, graphs[v], launches[v])
                times[v].append(time_graph(torch, stream, graphs[v], launches[v]))
        med = {v: statistics.median(ts) for v, ts in times.items()}
        best = min(med, key=med.get)
        flops = 2.0 * M * N * K * batch
        row = {
            "shape": {"transA": tA, "transB": tB, "M": M, "N": N, "K": K, "batch": batch,
                      "beta": beta},
            "mode": "hbm_resident" if hbm else "back_to_back",
            "copies": copies,
            "us": {pg.VARIANT_NAMES[v]: round(t, 2) for v, t in med.items()},
            "best": pg.VARIANT_NAMES[best],
            "auto": pg.VARIANT_NAMES[auto],
            "auto_tflops": round(flops / med[auto] / 1e6, 1),
            "regret": round(med[auto] / med[best] - 1.0, 4),
        }
        results.append(row)
        print(f"{'NT'[tA]}{'NT'[tB]} {M}x{N}x{K} b{batch} beta {beta}: best {row['best']} "
              f"{med[best]:.1f} us, auto {row['auto']} {med[auto]:.1f} us "
              f"({row['auto_tflops']} TFLOP/s), regret {100 * row['regret']:.1f} %  | " +
              " ".join(f"{pg.VARIANT_NAMES[v]}={t:.1f}" for v, t in med.items()),
              file=out, flush=True)
        del graphs, A, B, C
        torch.cuda.empty_cache()
    return results


NOT_OVERRIDABLE = ("GEMV", "P128x128", "P64x64")  # variants that run only some shapes


def overrides_from(rows, min_regret=0.02, other=None):
    """Dispatch override records (sgemm_set_dispatch_overrides) from a sweep:
    one per shape whose fastest variant beat the automatic choice by at least
    `min_regret`, naming that variant. The shape is given as the automatic
    choice receives it, a vector operand with adjacent k elements described
    contiguous in k (the sweep's leading dimensions are the stored row
    lengths, so an N == 1 op(B) untransposed and an M == 1 op(A) transposed
    are such vectors).

    With `other`, the rows of the same shapes timed in the other mode, a
    variant is judged by the sum of its two times: a table tuned with the
    operands in cache then does not pick a variant that loses with them
    streamed from HBM (1024^3: the plain 64 x 64 tile is 3 % faster than the
    K-split tile back to back and 25 % slower HBM-resident)."""
    if other is not None:
        paired = {tuple(sorted(o["shape"].items())): o for o in other}
        merged = []
        for r in rows:
            o = paired.get(tuple(sorted(r["shape"].items())))
            if o is None or o["auto"] != r["auto"]:
                continue
            us = {v: t + o["us"][v] for v, t in r["us"].items() if v in o["us"]}
            if r["auto"] not in us:
                continue
            best = min(us, key=us.get)
            merged.append({"shape": r["shape"], "best": best, "auto": r["auto"],
                           "regret": us[r["auto"]] / us[best] - 1.0})
        rows = merged
    records = []
    for r in rows:
        if r["best"] == r["auto"] or r["regret"] < min_regret or r["best"] in NOT_OVERRIDABLE:
            continue
        s = r["shape"]
        tA, tB = s["transA"], s["transB"]
        if s["N"] == 1 and tB == 0 and s["K"] > 1:
            tB = 1
        if s["M"] == 1 and tA == 1 and s["K"] > 1:
            tA = 0
        records.append([tA, tB, s["M"], s["N"], s["K"], s["batch"], r["best"]])
    return records


# Deep-K shapes with few output tiles, for the split-K comparison.
SPLITK_SHAPES = [
    (0, 0, 256, 256, 4096, 1), (0, 0, 256, 256, 16384, 1), (0, 0, 128, 128, 65536, 1),
    (0, 0, 512, 512, 8192, 1), (1, 0, 512, 512, 16384, 1), (0, 0, 640, 640, 8192, 1),
    (0, 0, 768, 768, 16384, 1), (0, 1, 64, 64, 262144, 1), (0, 0, 64, 64, 8192, 16),
    (0, 0, 1024, 1024, 4096, 1), (0, 0, 1024, 1024, 16384, 1),
]


def splitk_sweep(shapes, rounds: int = 3, target_ms: float = 20.0, out=sys.stdout):
    """Time the plain automatic call against the split-K automatic call (with
    the workspace sgemm_workspace_size asks for) on each shape."""
    import torch

    import precision_gemm_amd as pg

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    gen = torch.Generator(device=dev).manual_seed(1234)
    X = torch.rand(4096, 4096, device=dev, generator=gen)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.4:
        pg.sgemm(0, 0, 4096, 4096, 4096, 1.0, X, 4096, X, 4096, 0.0, X, 4096)
        torch.cuda.synchronize(dev)
    del X
    results = []
    for tA, tB, M, N, K, batch in shapes:
        def buf(rows, cols):
            return torch.rand((batch, rows, cols), device=dev, generator=gen) * 2 - 1
        A = buf(K, M) if tA else buf(M, K)
        B = buf(N, K) if tB else buf(K, N)
        C = buf(M, N)
        lda, ldb = A.shape[2], B.shape[2]
        sa, sb, sc = A.stride(0), B.stride(0), C.stride(0)
        need = pg.sgemm_workspace_size(tA, tB, M, N, K, batch)
        ws = torch.empty(max(1, need // 4), device=dev)
        v = pg.sgemm_select_variant(tA, tB, M, N, K, batch, 1, cus)
        # a streaming variant never splits; with a workspace the library swaps
        # in a 64 x 64 tile when splitting that pays
        if v in (pg.VARIANT_T64x64, pg.VARIANT_T32x64, pg.VARIANT_T64x32):
            vs = pg.VARIANT_S64x64_K2 if K >= 768 else pg.VARIANT_S64x64
        else:
            vs = v
        splits = pg.sgemm_select_splits(tA, tB, M, N, K, batch, vs, cus) if need else 1
        calls = {
            "plain": lambda: pg.sgemm_strided_batched(tA, tB, M, N, K, 1.0, A, lda, B, ldb, 0.0,
                                                      C, N, batch, sa, sb, sc,
                                                      stream=stream.cuda_stream),
            "split": lambda: pg.sgemm_strided_batched_ws(tA, tB, M, N, K, 1.0, A, lda, B, ldb,
                                                         0.0, C, N, batch, sa, sb, sc, ws,
                                                         stream=stream.cuda_stream),
        }
        launches = {}
        for k, call in calls.items():
            call()
            torch.cuda.synchronize(dev)
            one = time_variant(torch, pg, stream, call, 3)
            launches[k] = max(3, min(500, int(target_ms * 1e3 / max(one, 1.0))))
        times = {k: [] for k in calls}
        for _ in range(rounds):
            for k in calls:
                time_variant(torch, pg, stream, calls[k], max(2, launches[k] // 2))
                times[k].append(time_variant(torch, pg, stream, calls[k], launches[k]))
        med = {k: statistics.median(t) for k, t in times.items()}
        flops = 2.0 * M * N * K * batch
        row = {"shape": {"transA": tA, "transB": tB, "M": M, "N": N, "K": K, "batch": batch},
               "variant": pg.VARIANT_NAMES[vs if need else v], "splits": splits,
               "workspace_bytes": need, "plain_us": round(med["plain"], 2),
               "split_us": round(med["split"], 2),
               "split_tflops": round(flops / med["split"] / 1e6, 1),
               "speedup": round(med["plain"] / med["split"], 2)}
        results.append(row)
        print(f"{'NT'[tA]}{'NT'[tB]} {M}x{N}x{K} b{batch}: plain {med['plain']:.1f} us, split-K "
              f"S={splits} ({row['variant']}, workspace {need} B) {med['split']:.1f} us "
              f"({row['split_tflops']} TFLOP/s), x{row['speedup']}", file=out, flush=True)
        del A, B, C, ws
    return results


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", choices=["default", "quick", "wide", "mid"],
                    default="default")
    ap.add_argument("--splitk", action="store_true",
                    help="compare the plain and split-K automatic calls on deep-K shapes")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--hbm", action="store_true",
                    help="rotate operand copies so that every launch reads them from HBM")
    ap.add_argument("--json", default=None, help="write the table as JSON here")
    ap.add_argument("--write-overrides", default=None, metavar="PATH",
                    help="write dispatch overrides for the shapes the automatic choice "
                         "misses (load them with precision_gemm_amd.load_dispatch_overrides)")
    ap.add_argument("--min-regret", type=float, default=0.02,
                    help="smallest regret that earns an override (default 0.02)")
    ap.add_argument("--both-modes", action="store_true",
                    help="sweep back to back and HBM-resident, and judge each variant by "
                         "the sum of its two times (for --write-overrides)")
    ap.add_argument("--load-overrides", default=None, metavar="PATH",
                    help="install these dispatch overrides first, so that the automatic "
                         "choice measured is the overridden one")
    args = ap.parse_args(argv)
    if args.load_overrides:
        import precision_gemm_amd as pg
        pg.load_dispatch_overrides(args.load_overrides)
        print(f"{pg.sgemm_dispatch_override_count()} dispatch overrides installed", flush=True)
    if args.splitk:
        res = splitk_sweep(SPLITK_SHAPES, rounds=args.rounds)
        if args.json:
            with open(args.json, "w") as f:
                json.dump(res, f, indent=1)
        return 0
    shapes = {"default": DEFAULT_SHAPES, "quick": QUICK_SHAPES, "wide": WIDE_SHAPES,
              "mid": MID_SHAPES}[args.shapes]
    runs = [sweep(shapes, rounds=args.rounds, hbm=hbm)
            for hbm in ((False, True) if args.both_modes else (args.hbm,))]
    for res in runs:
        regrets = [r["regret"] for r in res]
        print(f"shapes {len(res)} ({res[0]['mode'] if res else '-'}): mean regret "
              f"{100 * statistics.mean(regrets):.2f} %, max {100 * max(regrets):.2f} %",
              flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump([r for res in runs for r in res], f, indent=1)
    if args.write_overrides:
        records = overrides_from(runs[0], args.min_regret,
                                 other=runs[1] if len(runs) > 1 else None)
        with open(args.write_overrides, "w") as f:
            json.dump(records, f, indent=1)
        print(f"{len(records)} dispatch overrides written to {args.write_overrides}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
