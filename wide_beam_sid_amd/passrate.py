"""Synthetic pass-rate study of the post stage (GRACE Section 6.2, Table 3
style): decode the same requests with catalog-valid decoding only (CD), with
CD + GTM, and with static and dynamic k-way partitioned matchers (the four
modes of Section 6), expand the finished SIDs into ads and run the exact
ad-level matcher (gr_post_filter) on each.  Also reports the matchers' fill
rate per decoding position (Table 2 style).

The pages measure this on an internal dataset with a trained model; here the
decoder's logits are seeded N(0, 1) draws, so beams follow random
catalog-valid paths and the comparison isolates what the GTM matchers do to
the ads that reach the post stage.  CD-only decoding uses the same catalog
with no matchers (a trie built without Bloom rows and an all-zero user
bitmask, so eq 5 always holds).

    python -m wide_beam_sid_amd.passrate --workload main_b16_m1024
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import sys
import time

import numpy as np

# requests are bucketed by the ads generated before the exact matcher, with
# the bucket edges of the pages' Table 3
BUCKETS = [(0, 5000, "<5k"), (5000, 10000, "5k-9.9k"), (10000, 1 << 62, "10k+")]


def fill_rates(trie, L: int) -> dict:
    """Mean fill (set-bit fraction) of the stored bitmask and Bloom matchers
    of the child entries at each decoding position 1..L; an entry's k-way
    partitions count as separate matchers."""
    v = trie.host_view()
    depth = v["node_depth"][1:]                     # entry e is node e + 1
    bm, bl = v["bitmask_table"], v["bloom_table"]
    def row_fill(tab):
        return (np.unpackbits(tab.view(np.uint8), axis=1).sum(axis=1) / (64.0 * tab.shape[1])
                if tab.size else np.zeros(0))
    fb, fl = row_fill(bm), row_fill(bl)
    if "kway_offsets" in v:
        off = v["kway_offsets"]
        ent = np.repeat(np.arange(off.size - 1), np.diff(off))
        bmi, bli, dep = v["kway_bitmask_index"], v["kway_bloom_index"], depth[ent]
    else:
        bmi, bli, dep = v["bitmask_index"], v["bloom_index"], depth
    out = {}
    for d in range(1, L + 1):
        sel = dep == d
        out[f"pos{d}"] = {"bitmask": float(fb[bmi[sel]].mean()) if sel.any() else 0.0,
                          "bloom": float(fl[bli[sel]].mean()) if sel.any() and fl.size else 0.0,
                          "matchers": int(sel.sum())}
    return out


def run(workload: str, seed: int, n_sids: int = 0, sets: int = 1, kway: bool = True) -> dict:
    import torch

    import wide_beam_sid_amd as gr
    from synth import workload as W
    from wide_beam_sid_amd.runner import Decoder

    w = W.WORKLOADS[workload]
    if n_sids:
        w = dataclasses.replace(w, n_sids=n_sids)
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    req = W.make_requests(w, seed)
    index = gr.AdIndex(sids, w.V, w.w_bm, [ads])
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gtm_locs = req.locs if w.bloom_bits else None
    build = lambda **kw: gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads],
                                       keep_host=True, **kw)
    modes = {
        "cd_only": (gr.Trie.build(sids, w.V, w.w_bm, 0, 0, [ads]),
                    np.zeros_like(req.user_bm), None, 0),
        "cd_gtm": (build(), req.user_bm, gtm_locs, w.n_loc),
    }
    if kway:
        # the pages' settings: static k = (64, 64, 32, 8) by decoding
        # position; dynamic k_max = 32 with a 0.25 fill target
        ks = (64, 64, 32, 8) + (8,) * max(0, w.L - 4)
        modes["static_kway"] = (build(kway_mode=1, kway_k=ks[:w.L]), req.user_bm, gtm_locs,
                                w.n_loc)
        modes["dynamic_kway"] = (build(kway_mode=2, kway_kmax=32, kway_target_fill=0.25),
                                 req.user_bm, gtm_locs, w.n_loc)
    out = {"workload": w.name, "n_sids": w.n_sids, "B": w.B, "k_final": w.schedule[-1],
           "seed": seed, "input_sets": sets, "modes": {}}
    for mode, (trie, ubm, locs, n_loc) in modes.items():
        probes = (gr.bloom_probes(locs.reshape(-1), w.bloom_bits, w.bloom_k)
                  if locs is not None else np.zeros((1, 1), np.uint32))
        dubm = torch.from_numpy(ubm.view(np.int64)).to(dev)
        dupr = torch.from_numpy(probes.view(np.int32)).to(dev)
        counts, post_s = [], 0.0
        for s in range(sets):
            g = torch.Generator(device=dev)
            g.manual_seed(seed * 1000 + s)   # the same decoder outputs in both modes
            ctx = [torch.randn((w.B, w.H, w.T_ctx, w.d_h), generator=g, device=dev).to(tdt)
                   for _ in range(2)]
            steps = []
            for t in range(w.L):
                R = w.rows(t)
                inp = {k: torch.randn((R, w.H, w.d_h), generator=g, device=dev).to(tdt)
                       for k in ("qx", "q", "k", "v")}
                inp["logits"] = torch.randn((R, w.V), generator=g, device=dev).to(tdt)
                steps.append(inp)
            dec = Decoder(trie, w.B, w.V, w.schedule, w.H, w.d_h, w.T_ctx, w.dtype)
            dec.run(dubm, dupr if locs is not None else None, n_loc, ctx[0], ctx[1], steps)
            torch.cuda.synchronize()
            tokens = dec.tokens[w.L].cpu().numpy()
            t0 = time.perf_counter()
            c, _ = index.post_filter(tokens, w.schedule[-1], req.user_bm,
                                     req.locs if w.n_loc else None)
            post_s += time.perf_counter() - t0
            counts.append(c.reshape(w.B, w.schedule[-1], 4).sum(axis=1))
        per_req = np.concatenate(counts)          # [requests, 4]
        tot = per_req.sum(axis=0)
        rate = lambda c: [float(c[1] / c[0]) if c[0] else 0.0, float(c[2] / c[0]) if c[0] else 0.0,
                          float(c[3] / c[0]) if c[0] else 0.0]
        bm, geo, fin = rate(tot)
        res = {"ads_generated": int(tot[0]), "bitmask_pass": bm, "location_pass": geo,
               "final_pass": fin, "post_stage_ms_per_batch": post_s / sets * 1e3, "buckets": []}
        for lo, hi, name in BUCKETS:
            sel = (per_req[:, 0] >= lo) & (per_req[:, 0] < hi)
            c = per_req[sel].sum(axis=0)
            b, gg, f = rate(c)
            res["buckets"].append({"bucket": name, "requests": float(sel.mean()),
                                   "bitmask_pass": b, "location_pass": gg, "final_pass": f})
        if mode != "cd_only":
            res["fill"] = fill_rates(trie, w.L)
        out["modes"][mode] = res
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="main_b16_m1024")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--n-sids", type=int, default=0)
    ap.add_argument("--sets", type=int, default=4, help="independent batches of requests' inputs")
    ap.add_argument("--no-kway", action="store_true", help="skip the k-way modes")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        print("the pass-rate study decodes on a GPU", file=sys.stderr)
        sys.exit(1)
    res = run(args.workload, args.seed, args.n_sids, args.sets, kway=not args.no_kway)
    for mode, r in res["modes"].items():
        print(f"{mode:12s} ads {r['ads_generated']:9d}  bitmask {100 * r['bitmask_pass']:6.2f}%  "
              f"location {100 * r['location_pass']:6.2f}%  final {100 * r['final_pass']:6.3f}%",
              file=sys.stderr)
        for pos, f in r.get("fill", {}).items():
            print(f"    {pos}: bitmask fill {f['bitmask']:.3f}  bloom fill {f['bloom']:.3f}  "
                  f"({f['matchers']} matchers)", file=sys.stderr)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
