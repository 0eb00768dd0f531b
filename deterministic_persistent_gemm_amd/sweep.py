"""Offline sweeper for the (dtype, N, K) key table.

    python -m deterministic_persistent_gemm_amd.sweep --key f32:256:4096 --key bf16:4096:4096 \
        [--profile decode|prefill|balanced] [--out DIR] [--write-table]

GateLinear page, "Perf" and "Update: is the M=4096 cost avoidable?": the
config of a key is chosen by a sweep in the production weight.t() layout
(the nn.Linear weight [N, K] row-major) and is keyed on (dtype, N, K) only;
no single choice wins at both decode and prefill, so the choice depends on
the deployment (decode-heavy RL rollout vs prefill-heavy serving).

Here the only choice that is part of the numerics is the recipe's tile
partial width block_k; everything else (decode kernel form, the M where the
persistent kernel takes over, the persistent tile shape per M range) only
picks kernel shapes.  For each candidate block_k of a key the sweeper times,
with cold weights (rotating copies, beyond the Infinity Cache):

  * every decode form that serves the candidate (two launches with a
    workspace fold, one launch with an LDS fold, direct-to-LDS streaming for
    a chained bf16 recipe, one launch with the XCD hand-over fold) at M in
    DECODE_M and at the prefill sizes up to DECODE_PROBE_MAX (the decode
    limit may lie beyond the decode sizes);
  * every persistent tile shape at M in PREFILL_M and at the decode sizes
    where the persistent kernel might take over;
  * both at CROSS_M, which only places the decode limit between the
    prefill sizes (it counts in neither total);
  * every persistent tile shape at SEGMENT_M, which only places the tile
    ranges between the prefill sizes (it counts in no total);

Times are per-call averages over a replayed HIP graph of the calls.  The
sweeper then checks that every path and tile shape of the candidate gives the same bits
(they carry out one recipe) and that a row computed alone equals the same
row inside the batch, then picks the entry for the profile:

  decode    least total decode time (M <= 128)
  prefill   least total prefill time
  balanced  least mean of decode and prefill times, each relative to the
            best candidate

(candidates within --tie of the best keep the key's served recipe, so noise
does not change a key's bits; --keep-recipe considers the served block_k
only, so a re-sweep changes kernel shapes and never a key's bits),

and emits it as a JSON report and a line of bi_table.inc.  --write-table
merges the entries into csrc/bi_table.inc (replacing the keys swept); the
library must then be rebuilt.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(PKG, "csrc", "bi_table.inc")

DECODE_M = (1, 8, 16, 32, 64, 128)
PREFILL_M = (256, 1024, 4096)
CROSS_M = (512,)            # timed on both sides to place the decode limit, not in either total
SEGMENT_M = (2048,)         # timed for the tile shapes only, to place their ranges, in no total
DECODE_PROBE_MAX = 1024     # decode forms are also timed at the prefill sizes up to this M
DECODE_MARGIN = 0.05        # the persistent kernel takes over once it is this much faster
TABLE_HEADER = ("// Measured key table, written by deterministic_persistent_gemm_amd/sweep.py.\n"
                "// {dtype, N, K, block_k, m_decode_max, decode_path, m_a, tile_a, m_b, tile_b, tile_c, "
                "m_xcd_max}\n")
F32_CODES = tuple(range(1, 11)) + (23, 24, 28, 29)
BF16_CODES = tuple(range(11, 23))
PATH_DECODE, PATH_PERSISTENT, PATH_DECODE_WG, PATH_DECODE_DMA, PATH_DECODE_XCD = 1, 2, 3, 4, 5


def parse_key(s: str, profile: str = "decode"):
    """dtype:N:K[:profile]"""
    f = s.split(":")
    if len(f) not in (3, 4) or f[0] not in ("f32", "bf16"):
        raise ValueError(f"key must be dtype:N:K[:profile] with dtype f32 or bf16: {s}")
    prof = f[3] if len(f) == 4 else profile
    if prof not in ("decode", "prefill", "balanced"):
        raise ValueError(f"unknown profile in {s}")
    return f[0], int(f[1]), int(f[2]), prof


def stage_k(code: int) -> int:
    """k per LDS stage of a persistent tile shape (shapes whose stage does
    not divide K are served by the 32-k-stage shape of the dtype)."""
    return 32 if code in (7, 8, 17) else 128 if code in (9, 10, 13, 16) else 64   # 20-24, 28, 29: 64


def tile_codes(dt: str, K: int, block_k: int):
    """The distinct tile shapes a recipe can run: shapes whose stage does not
    divide K, the 256x256 shapes (single k tile only: 18, 19 and the
    ring-fed 21, 22) of a recipe with several k tiles, and the ring-fed fp32
    shapes (23, 24 and their k-split forms 28, 29: an even number of k tiles
    of 64-k multiples) of a recipe without, would fall back to another shape
    and are left out."""
    codes = F32_CODES if dt == "f32" else BF16_CODES
    rings_f32 = (K // block_k) % 2 == 0 and block_k % 64 == 0
    return tuple(c for c in codes if K % stage_k(c) == 0 and not (c in (18, 19, 21, 22) and block_k != K)
                 and not (c in (23, 24, 28, 29) and not rings_f32))


def block_k_candidates(dt: str, K: int):
    base = (128, 256, 512, K) if dt == "f32" else (512, 1024, K)
    return sorted({b for b in base if b % 32 == 0 and K % b == 0 and b <= K})


# ----------------------------------------------------------------- selection

def summarize(cand: dict) -> dict:
    """From one candidate's timings (us) derive its decode/persistent bests,
    the decode limit and the tile choices.

    cand = {"block_k": b, "decode": {M: {path: us}}, "persistent": {M: {code: us}}}"""
    best_dec = {M: min(v.values()) for M, v in cand["decode"].items() if v}
    best_dec_path = {M: min(v, key=v.get) for M, v in cand["decode"].items() if v}
    # decode_path names the form that serves M above the XCD hand-over's
    # range, so it is picked among the other forms
    other = {M: {p: t for p, t in v.items() if p != PATH_DECODE_XCD} for M, v in cand["decode"].items()}
    best_other_path = {M: min(v, key=v.get) for M, v in other.items() if v}
    best_per = {M: min(v.values()) for M, v in cand["persistent"].items() if v}
    best_code = {M: min(v, key=v.get) for M, v in cand["persistent"].items() if v}
    # decode serves M up to the last grid point before the persistent kernel
    # wins by more than DECODE_MARGIN (near the crossing the two are within
    # noise, and the grid is coarse: the decode form is kept there)
    m_dec = 0
    for M in sorted(best_dec):
        if M in best_per and best_per[M] < best_dec[M] * (1.0 - DECODE_MARGIN):
            break
        m_dec = M
    dec_ms = [M for M in sorted(best_dec) if M <= m_dec]
    # the XCD hand-over serves M from 1 up to the last grid point of an
    # unbroken run where it is the best decode form
    m_xcd = 0
    for M in dec_ms:
        if best_dec_path[M] != PATH_DECODE_XCD:
            break
        m_xcd = M
    paths = [best_other_path[M] for M in dec_ms if M > m_xcd and M in best_other_path] or \
        [best_other_path[M] for M in dec_ms if M in best_other_path]
    decode_path = max(set(paths), key=paths.count) if paths else 0
    tiles = tile_segments(cand["persistent"], [M for M in best_code if M > m_dec])
    decode_total = sum(min(best_dec.get(M, math.inf), best_per.get(M, math.inf)) for M in DECODE_M
                       if M in best_dec or M in best_per)
    prefill_total = sum(best_per[M] for M in PREFILL_M if M in best_per)
    return {"block_k": cand["block_k"], "m_decode_max": m_dec, "decode_path": decode_path, "m_xcd_max": m_xcd,
            **tiles,
            "decode_total_us": round(decode_total, 3), "prefill_total_us": round(prefill_total, 3)}


def tile_segments(per: dict, points: list) -> dict:
    """Persistent tile codes for the M ranges above the decode limit: the best
    code of each measured M, runs of equal codes merged, and while more than
    three ranges remain the neighbouring pair whose common code costs the
    least extra time merged.  Range i covers M up to its last measured point."""
    points = sorted(points)
    if not points:
        return {"m_a": 0, "tile_a": 0, "m_b": 0, "tile_b": 0, "tile_c": 0}
    segs = []                                   # [points, code]
    for M in points:
        code = min(per[M], key=per[M].get)
        if segs and segs[-1][1] == code:
            segs[-1][0].append(M)
        else:
            segs.append([[M], code])

    def merged(a, b):
        ms = a[0] + b[0]
        common = [c for c in per[ms[0]] if all(c in per[M] for M in ms)]
        best = min(common, key=lambda c: sum(per[M][c] for M in ms))
        extra = sum(per[M][best] - min(per[M].values()) for M in ms)
        return [ms, best], extra

    while len(segs) > 3:
        i = min(range(len(segs) - 1), key=lambda i: merged(segs[i], segs[i + 1])[1])
        segs[i:i + 2] = [merged(segs[i], segs[i + 1])[0]]
    while len(segs) < 3:
        segs.append([segs[-1][0], segs[-1][1]])
    return {"m_a": segs[0][0][-1], "tile_a": segs[0][1], "m_b": segs[1][0][-1], "tile_b": segs[1][1],
            "tile_c": segs[2][1]}


def objective(summaries: list, profile: str):
    d0 = min(s["decode_total_us"] for s in summaries)
    p0 = min(s["prefill_total_us"] for s in summaries)
    if profile == "decode":
        return lambda s: s["decode_total_us"] / d0
    if profile == "prefill":
        return lambda s: s["prefill_total_us"] / p0
    if profile == "balanced":
        return lambda s: 0.5 * (s["decode_total_us"] / d0 + s["prefill_total_us"] / p0)
    raise ValueError(profile)


def choose(summaries: list, profile: str, keep_block_k: int | None = None, tie: float = 0.0) -> dict:
    """The candidate with the least objective.  Candidates within `tie`
    (relative) of the best count as equal; among equals the recipe the key
    already has (keep_block_k) is kept, so measurement noise does not change
    a key's bits; otherwise the secondary total decides."""
    f = objective(summaries, profile)
    best = min(f(s) for s in summaries)
    equal = [s for s in summaries if f(s) <= best * (1.0 + tie)]
    for s in equal:
        if s["block_k"] == keep_block_k:
            return s
    second = "prefill_total_us" if profile == "decode" else "decode_total_us"
    return min(equal, key=lambda s: (f(s), s[second]))


def table_line(dt: str, N: int, K: int, e: dict) -> str:
    d = "BI_F32" if dt == "f32" else "BI_BF16"
    return (f"{{{d}, {N}, {K}, {e['block_k']}, {e['m_decode_max']}, {e['decode_path']}, "
            f"{e['m_a']}, {e['tile_a']}, {e['m_b']}, {e['tile_b']}, {e['tile_c']}, {e.get('m_xcd_max', 0)}}},")


def merge_table(text: str, lines: dict) -> str:
    """Replace or add table lines keyed by their (dtype, N, K) prefix."""
    out, seen = [], set()
    for ln in text.splitlines():
        s = ln.strip()
        if s.startswith("{"):
            key = ",".join(x.strip() for x in s.strip("{},").split(",")[:3])
            if key in lines:
                out.append(lines[key])
                seen.add(key)
                continue
        out.append(ln)
    body = [ln for ln in out if ln.strip()]
    if not body or not body[0].startswith("// Measured key table"):
        body = TABLE_HEADER.strip().splitlines() + body
    body += [v for k, v in lines.items() if k not in seen]
    return "\n".join(body) + "\n"


def parse_table(text: str):
    rows = []
    for ln in text.splitlines():
        s = ln.strip()
        if not s.startswith("{"):
            continue
        f = [x.strip() for x in s.strip("{},").split(",")]
        rows.append({"dtype": f[0], "N": int(f[1]), "K": int(f[2]), "block_k": int(f[3]),
                     "m_decode_max": int(f[4]), "decode_path": int(f[5]), "m_a": int(f[6]),
                     "tile_a": int(f[7]), "m_b": int(f[8]), "tile_b": int(f[9]), "tile_c": int(f[10]),
                     "m_xcd_max": int(f[11]) if len(f) > 11 else 0})
    return rows


# ------------------------------------------------------------------ measuring

def _timeit(torch, fns, reps=3):
    """Average device time (us) of one call, rotating over fns (cold weights).

    The calls are captured into one HIP graph on a side stream (after an
    eager pass there, which also sizes the workspace) and the graph is
    replayed back to back, so neither host launch cost nor per-call events
    enter the figure."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for f in fns:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1_000_000)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * len(fns))


def sweep_key(dt: str, N: int, K: int, profile: str, tie: float = 0.03, log=print, keep_recipe: bool = False):
    import numpy as np
    import torch

    import deterministic_persistent_gemm_amd as bi

    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(N * 1009 + K)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    wbytes = N * K * (4 if dt == "f32" else 2)
    ncopies = max(2, min(128, math.ceil((512 << 20) / wbytes)))
    w0 = (torch.randn(N, K, generator=g) * 0.02).to(tdt)
    ws = [w0.to(dev)] + [w0.to(dev).clone() for _ in range(ncopies - 1)]
    grid = sorted(set(DECODE_M + PREFILL_M + CROSS_M + SEGMENT_M))
    xs = {M: torch.randn(M, K, generator=g).to(tdt).to(dev) for M in grid}
    odt = torch.float32
    served = bi.bi_describe_recipe(bi.BI_F32 if dt == "f32" else bi.BI_BF16, N, K).block_k
    cands, summaries = [], []
    for bk in ([served] if keep_recipe else block_k_candidates(dt, K)):
        r = bi.bi_describe_recipe(bi.BI_F32 if dt == "f32" else bi.BI_BF16, N, K)
        r.block_k = bk
        cand = {"block_k": bk, "decode": {}, "persistent": {}, "bits_ok": True}
        for M in grid:
            x = xs[M]
            out = torch.empty(M, N, dtype=odt, device=dev)
            ref = None

            def run(path, wt=ws[0]):
                return bi.bi_lab_linear(x, wt.t(), None, recipe=r, path=path, out_dtype=odt, out=out)

            def check(tag):
                nonlocal ref
                got = out.clone()
                if ref is None:
                    ref = got
                elif not torch.equal(got.view(torch.int32), ref.view(torch.int32)):
                    cand["bits_ok"] = False
                    log(f"  BITS DIFFER: {dt}:{N}:{K} block_k={bk} M={M} {tag}")

            if M in DECODE_M or M <= DECODE_PROBE_MAX:
                cand["decode"][M] = {}
                for path in (PATH_DECODE, PATH_DECODE_WG, PATH_DECODE_DMA, PATH_DECODE_XCD):
                    try:
                        run(path)
                    except bi.BIError:
                        continue                       # a form that does not serve this recipe / M
                    check(f"decode path {path}")
                    cand["decode"][M][path] = _timeit(torch, [lambda w=w, p=path: run(p, w) for w in ws])
            cand["persistent"][M] = {}
            for code in tile_codes(dt, K, bk):
                path = PATH_PERSISTENT | (code << 8)
                run(path)
                check(f"tile {code}")
                cand["persistent"][M][code] = _timeit(torch, [lambda w=w, p=path: run(p, w) for w in ws])
            # a row alone equals the same row in the batch
            solo = bi.bi_lab_linear(x[M - 1:M].contiguous(), ws[0].t(), None, recipe=r, out_dtype=odt)
            full = bi.bi_lab_linear(x, ws[0].t(), None, recipe=r, out_dtype=odt)
            if not torch.equal(solo[0].view(torch.int32), full[M - 1].view(torch.int32)):
                cand["bits_ok"] = False
                log(f"  ROW NOT INVARIANT: {dt}:{N}:{K} block_k={bk} M={M}")
            log(f"  {dt}:{N}:{K} block_k={bk} M={M}: decode "
                f"{ {p: round(t, 2) for p, t in cand['decode'].get(M, {}).items()} } persistent best "
                f"{min(cand['persistent'][M].values()):.2f} us (tile {min(cand['persistent'][M], key=cand['persistent'][M].get)})")
        cands.append(cand)
        if cand["bits_ok"]:
            summaries.append(summarize(cand))
    if not summaries:
        raise RuntimeError(f"no candidate of {dt}:{N}:{K} passed the bit checks")
    entry = choose(summaries, profile, keep_block_k=served, tie=tie)
    return {"key": f"{dt}:{N}:{K}", "profile": profile, "tie": tie, "served_block_k": served,
            "weight_copies": ncopies, "entry": entry,
            "summaries": summaries,
            "candidates": [{"block_k": c["block_k"], "bits_ok": c["bits_ok"],
                            "decode": {str(M): v for M, v in c["decode"].items()},
                            "persistent": {str(M): v for M, v in c["persistent"].items()}} for c in cands],
            "table_line": table_line(dt, N, K, entry)}


def entry_from_report(rep: dict, profile: str | None = None, tie: float | None = None) -> dict:
    """Re-derive a key's entry from a saved report (no measuring): the
    candidates that passed the bit checks, the profile and tie band given (or
    the report's own)."""
    profile = profile or rep["profile"]
    tie = rep.get("tie", 0.0) if tie is None else tie
    sums = []
    for c in rep["candidates"]:
        if not c["bits_ok"]:
            continue
        dec = {int(M): {int(p): t for p, t in v.items()} for M, v in c["decode"].items()}
        per = {int(M): {int(k): t for k, t in v.items()} for M, v in c["persistent"].items()}
        sums.append(summarize({"block_k": c["block_k"], "decode": dec, "persistent": per}))
    return choose(sums, profile, keep_block_k=rep.get("served_block_k"), tie=tie)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--key", action="append", default=[],
                    help="dtype:N:K[:profile], dtype f32 or bf16, profile as --profile")
    ap.add_argument("--from-json", action="append", default=[],
                    help="re-derive the entry of a saved report instead of measuring")
    ap.add_argument("--profile", choices=("decode", "prefill", "balanced"), default="decode")
    ap.add_argument("--tie", type=float, default=None,
                    help="relative objective difference treated as a tie (the served recipe is kept); "
                         "default 0.03 when sweeping, the report's own with --from-json")
    ap.add_argument("--keep-recipe", action="store_true",
                    help="sweep only the block_k each key already serves (kernel shapes change, bits do not)")
    ap.add_argument("--out", default=None, help="directory for the JSON reports")
    ap.add_argument("--write-table", action="store_true", help="merge the entries into csrc/bi_table.inc")
    args = ap.parse_args(argv)
    keys = [parse_key(k, args.profile) for k in args.key]
    lines = {}
    for path in args.from_json:
        rep = json.load(open(path))
        dt, N, K = parse_key(rep["key"])[:3]
        e = entry_from_report(rep, tie=args.tie)
        lines[f"{'BI_F32' if dt == 'f32' else 'BI_BF16'},{N},{K}"] = table_line(dt, N, K, e)
        print(f"{rep['key']} ({rep['profile']}): {table_line(dt, N, K, e)}", flush=True)
    for dt, N, K, prof in keys:
        print(f"sweeping {dt}:{N}:{K} ({prof})", flush=True)
        rep = sweep_key(dt, N, K, prof, tie=0.03 if args.tie is None else args.tie,
                        log=lambda s: print(s, flush=True), keep_recipe=args.keep_recipe)
        print(f"  entry: {rep['table_line']}", flush=True)
        if args.out:
            os.makedirs(args.out, exist_ok=True)
            with open(os.path.join(args.out, f"sweep_{dt}_{N}_{K}_{prof}.json"), "w") as f:
                json.dump(rep, f, indent=1)
        d = "BI_F32" if dt == "f32" else "BI_BF16"
        lines[f"{d},{N},{K}"] = rep["table_line"]
    if args.write_table:
        text = open(TABLE).read() if os.path.exists(TABLE) else TABLE_HEADER
        with open(TABLE, "w") as f:
            f.write(merge_table(text, lines))
        print(f"wrote {TABLE}; rebuild the library", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
