#!/usr/bin/env python3
"""Benchmark of the render + analytic score replay path on one MI355X.

One step = gs_project -> gs_bin_sort -> gs_render -> gs_score_replay (tokens
written) over one synthetic scene whose parameters and observation already sit
in HBM.  Prints ONE JSON line with the throughput (rendered+replayed Mpix/s),
Gaussian-pixel contributions/s, per-stage times (HIP events on the stream the
kernels run on), the roofline of the dominant kernel (the score replay: its
fp32 VALU fraction and its HBM fraction), the score overhead (replay + finalize
over the render path, and over the render path plus the renderer backward: a
render/update step), the workspace and peak device memory, and the CPU oracle
timed on a bounded sample on the host cores.  The other workload
configurations are measured the same way and reported under "configs".  The
renderer backward (gs_backward of 1/2 |C_hat - C_obs|^2 over the last step's
render) is timed separately and reported under "backward", and so are a
9-channel feature composite and a 2-channel attribution scatter
("attributes"); they are not part of the step.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5] [--configs 1,2,4,5]

The default workload is the ATSplat-like compact scene: one 512x960 view of
311,296 Gaussians (19,456 anchors x 16 offsets), SH degree 3.  Only one GPU is
supported.
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

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, 8 TB/s
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12     # fp32 VALU lane-ops/s (256 CU x 4 SIMD x 16 lanes x 2.4 GHz)

# Algorithmic fp32 operations per unit of work (one VALU lane-op each), the method's own counts:
OPS_EVAL = 12           # per evaluated (pixel, list entry): offsets, exponent, exponential, alpha, tests
OPS_CONTRIB_FWD = 10    # per contribution, the forward accumulation (T (1 - alpha), w, colour sums, count)
OPS_CONTRIB_SCORE = 40  # per contribution, the replay's suffix, rho, masks and 7 accumulators
OPS_CONTRIB_REPLAY = OPS_CONTRIB_FWD + OPS_CONTRIB_SCORE   # the replay re-accumulates the prefix as it goes
OPS_CONTRIB_BWD = 70    # forward 20, suffix 6, <g,c> and <g,S> 6, 1-alpha, reciprocal, u and its mask 4,
                        # the 9 partials 8, their wave reduction 26 (eight-value reduce-scatter + one sum)
# Algorithmic HBM bytes of the replay: per (tile, Gaussian) pair it walks -- in each tile, the list entries up
# to the deepest one any of the tile's pixels evaluates before it stops -- its sorted Gaussian id (4) and the
# 40 B of the record it evaluates (centre 8, exponent factors 12, opacity 4, colour 12, slot 4); per pixel the
# rendered colour and transmittance (16) and the observation (12); per (Gaussian, view) record its 7
# accumulated partial scores, written once (28)
REPLAY_BYTES_PAIR = 44
REPLAY_BYTES_PIXEL = 28
REPLAY_BYTES_RECORD = 28

def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    p.add_argument("--configs", default="1,2,4,5",
                   help="further workload configurations measured the same way (fewer steps) and reported "
                        "under 'configs'; empty to skip")
    p.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                   help="budget of rendering work for the CPU oracle sample (0 disables)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip the separately timed renderer backward (gs_backward of 1/2 |C_hat - C|^2)")
    p.add_argument("--antialiased", action="store_true",
                   help="run the whole path in the antialiased (opacity-compensated) mode")
    p.add_argument("--no-attributes", action="store_true",
                   help="skip the separately timed 9-channel feature composite and 2-channel attribution scatter")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the benchmark line: view-count / resolution scaling (4, 8, 16, 32 views at "
                        "256x448 and 512x960 over a fixed Gaussian set), one JSON line per point")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="before the steps, copy a buffer of this many MiB once (untimed), so that "
                        "hardware byte counters can be scaled against a copy of known size")
    return p.parse_args()


def stage_bytes(stage, c):
    """Algorithmic HBM bytes per launch of a stage: every array the stage must
    read or write once, at its element size (per-record and per-pair terms,
    annotated line by line below)."""
    G, V, d, P, VG = c["G"], c["V"], c["d"], c["P"], c["G"] * c["V"]
    pk = 4 if c["packable"] else 0   # the rectangle packed to 32 bits by preprocess for the depth sort
    if stage == "project":       # Gaussian parameters in; 48-byte record, rectangle, depth key, tile count out
        return G * (4 * 3 + 4 * 4 + 4 * 3 + 4 + 4 * 3 * d) + VG * (48 + 8 + 4 + 4 + pk)
    if stage == "depth_sort":    # slot scan 8, histogram 4, then with carried packed rectangles: pass 0 (key+rect
        if pk:                   # in, key+id+rect out) 20, passes 1-2 24 each, pass 3 (key+id+rect in, id and rect out) 20
            return VG * (8 + 4 + 20 + 2 * 24 + 20)
        # gathered: pass 0 (key in, key+id out) 12, passes 1-2 16 each, pass 3 (key+id in, id out, the 8-byte
        return VG * (8 + 4 + 12 + 2 * 16 + 32)   # rectangle gathered by record, rectangle + tile count out) 32
    if stage == "scan":
        return VG * 8
    if stage == "emit":          # per record: id, rect, tile count, offset in; per pair: tile key and Gaussian out
        return VG * (4 + 4 + 4 + (0 if pk else 8)) + P * (4 if c["packed"] else 8)  # (packed rect 4 B instead of rect
                                                                       # and count 12 B; one word per pair if it fits)
    if stage == "tile_sort":     # pass 1 key+value in and out, pass 2 key+value in, value out (the digit counts
        return P * (8 + 8) if c["packed"] else P * (16 + 12)  # come from emit); packed words: 4 B in, 4 B out
    if stage == "ranges":        # ranges set to {~0u, 0} (the last tile-sort pass records them) and the 1 MiB of
        return V * c["T"] * 8 + (1 << 20)   # histogram rows zeroed for the tile sort's digit counts
    return None


def _sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gaussian_splatting_rasterizer_amd", "csrc")
    for n in ["gsr_device.hpp", "gsr_internal.hpp"] + list(names):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "gsr.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


KERNEL_SOURCES = {"k_project": ["project.hip"], "k_render": ["render.hip"], "k_replay": ["replay.hip"],
                  "k_gather_slots": ["replay.hip"], "k_tokens": ["replay.hip"], "k_onesweep": ["binning.hip"],
                  "k_emit": ["binning.hip"], "k_ranges": ["binning.hip"], "k_digit_hist": ["binning.hip"],
                  "k_backward": ["backward.hip"], "k_grads": ["backward.hip"],
                  "k_render_features": ["attributes.hip"], "k_attribute": ["attributes.hip"],
                  "k_sum_views": ["attributes.hip"]}


def kernel_source_sha256(kernel):
    return _sources_sha256(KERNEL_SOURCES[kernel])


def measured_traffic(kernel, workload, antialiased=False):
    """HBM bytes per launch from the committed counter summary of this workload,
    or None when there is none, the kernel's sources changed since, or the run
    is in the antialiased mode (the counters are taken in the plain mode)."""
    if antialiased:
        return None
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get("kernels", {}).get(kernel)
    base = kernel.split("<", 1)[0]  # a template instance hashes its template's sources
    if not entry or entry.get("source_sha256") != kernel_source_sha256(base):
        return None
    return int(entry["bytes_per_launch"])


def measure(config, args, dev, stream, steps, warmup, extras):
    """Time `steps` steps of workload `config` after `warmup` untimed ones; with `extras`, also
    the renderer backward and the attribute kernels.  Returns (scene, result dict)."""
    import torch

    import scenes
    from gaussian_splatting_rasterizer_amd import binding

    sc = scenes.make_scene(config)
    torch.cuda.reset_peak_memory_stats(dev)
    with torch.cuda.stream(stream):
        # observation: render of the scene with perturbed means + pixel noise (setup, untimed)
        rp = binding.rasterizer_for_scene(sc.perturbed(), device=dev, antialiased=args.antialiased)
        rp.project_and_bin()
        obs_col, _, _ = rp.render()
        obs = (obs_col + torch.from_numpy(sc.pixel_noise).to(dev)).contiguous()
        rp.close()
        del rp, obs_col

        if extras and args.copy_calibration_mib > 0:
            n = args.copy_calibration_mib * (1 << 20) // 4
            src_buf = torch.ones(n, dtype=torch.float32, device=dev)
            dst_buf = torch.empty_like(src_buf)
            dst_buf.copy_(src_buf)
            stream.synchronize()
            del src_buf, dst_buf

        r = binding.rasterizer_for_scene(sc, device=dev, antialiased=args.antialiased)
        r.project_and_bin()
        r._alloc(int(r.n_pairs * 1.1) + 4096)      # right-size the workspace once
        workspace_bytes = int(r.workspace.numel())
        outputs = r.new_outputs()
        tokens = torch.empty((sc.n, 9 + 3 * sc.d), dtype=torch.float32, device=dev)
        for _ in range(warmup):
            r.step(obs, outputs, tokens)
        stream.synchronize()

        # timed region: only the dominant kernel's stage carries HIP events (every timed stage adds two event
        # records, i.e. idle GPU time at its boundaries)
        binding.gs_profile_stages(r.ctx, ["replay"])
        binding.gs_profile_read(r.ctx)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            r.step(obs, outputs, tokens)
        stream.synchronize()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        prof_timed = binding.gs_profile_read(r.ctx)
        # per-stage breakdown from separate steps with every stage timed
        n_prof = min(steps, 10)
        binding.gs_profile_enable(r.ctx, True)
        for _ in range(n_prof):
            r.step(obs, outputs, tokens)
        stream.synchronize()
        prof = binding.gs_profile_read(r.ctx)
        binding.gs_profile_enable(r.ctx, False)

        # renderer backward of 1/2 |C_hat - C_obs|^2 on the same render, timed on its own (every configuration:
        # the score overhead is also reported against the render plus this backward, a gradient update step)
        bwd = None
        if not args.no_backward:
            grad_color = (outputs[0] - obs).contiguous()
            grads = r.new_grads()
            for _ in range(warmup):
                r.backward(grad_color, grads)
            stream.synchronize()
            binding.gs_profile_stages(r.ctx, ["backward"])
            binding.gs_profile_read(r.ctx)
            tb = time.perf_counter()
            for _ in range(steps):
                r.backward(grad_color, grads)
            stream.synchronize()
            tb = time.perf_counter() - tb
            bprof = binding.gs_profile_read(r.ctx)
            binding.gs_profile_stages(r.ctx, ["backward_finalize"])
            for _ in range(n_prof):
                r.backward(grad_color, grads)
            stream.synchronize()
            bprof["backward_finalize"] = binding.gs_profile_read(r.ctx)["backward_finalize"]
            binding.gs_profile_enable(r.ctx, False)
            bwd = dict(ms=1e3 * tb / steps,
                       stages={k: bprof[k][0] / max(bprof[k][1], 1) for k in ("backward", "backward_finalize")},
                       finite=bool(all(torch.isfinite(t).all().item() for t in grads.values())))

        # feature composite of 9 channels (ReCoSplat-style conditioning features) and attribution scatter of a
        # 2-channel map (squared residual, coverage: the error + coverage token), each timed on its own
        attrs = None
        if extras and not args.no_attributes:
            gen = torch.Generator(device=dev).manual_seed(5)
            feats = torch.randn((sc.n, 9), generator=gen, device=dev, dtype=torch.float32)
            feat_out = torch.empty((sc.n_views, sc.height, sc.width, 9), dtype=torch.float32, device=dev)
            resid2 = ((outputs[0] - obs) ** 2).sum(-1)
            amap = torch.stack([resid2, torch.ones_like(resid2)], dim=-1).contiguous()
            aout = torch.empty((sc.n, 2), dtype=torch.float32, device=dev)
            for _ in range(warmup):
                r.render_features(feats, out=feat_out)
                r.attribute(amap, out=aout)
            stream.synchronize()
            binding.gs_profile_enable(r.ctx, True)
            binding.gs_profile_read(r.ctx)
            for _ in range(steps):
                r.render_features(feats, out=feat_out)
            for _ in range(steps):
                r.attribute(amap, out=aout)
            stream.synchronize()
            aprof = binding.gs_profile_read(r.ctx)
            binding.gs_profile_enable(r.ctx, False)
            attrs = {k: aprof[k][0] / max(aprof[k][1], 1) for k in ("features", "attribute")}
            attrs["finite"] = bool(torch.isfinite(feat_out).all().item() and torch.isfinite(aout).all().item())

        color, T, n = outputs
        stats = r.export(binding.GS_EXPORT_PIXEL_STATS).view(-1, 2).to(torch.int64)
        K = int(n.to(torch.int64).sum().item())
        E = int(stats[:, 0].sum().item())
        E_cut = int(stats[:, 1].sum().item())
        # pairs walked: per tile, the deepest list entry any of its pixels evaluates
        V_, H_, W_ = sc.n_views, sc.height, sc.width
        ev = stats[:, 0].view(V_, H_, W_)
        ev = torch.nn.functional.pad(ev, (0, (-W_) % 16, 0, (-H_) % 16))
        P_walk = int(ev.view(V_, ev.shape[1] // 16, 16, ev.shape[2] // 16, 16).amax(dim=(2, 4)).sum().item())
        P = int(r.n_pairs)
        finite = bool(torch.isfinite(tokens).all().item())
        rec = r.export(binding.GS_EXPORT_RECORDS)
        n_live = int((rec[3, :, 1] != 0).sum().item())
        stream.synchronize()
        peak_bytes = int(torch.cuda.max_memory_allocated(dev))
        r.close()
        del r, rec, stats, outputs, tokens, obs
    torch.cuda.empty_cache()

    V, H, W = sc.n_views, sc.height, sc.width
    T_tiles = ((W + 15) // 16) * ((H + 15) // 16)
    N_px = V * H * W
    ms_step = 1e3 * elapsed / steps
    workload = scenes.CONFIG_NAMES[config]
    bits_for = lambda x: max(int(x - 1).bit_length(), 1)
    c = dict(G=sc.n, V=V, d=sc.d, P=P, T=T_tiles, n_live=n_live,
             packed=bits_for(V * T_tiles) + bits_for(sc.n) <= 32,
             packable=(W + 15) // 16 <= 256 and (H + 15) // 16 <= 256 and sc.n * V > (1 << 19))
    stages = {k: (ms / max(cnt, 1), cnt) for k, (ms, cnt) in prof.items() if cnt > 0}
    # The dominant single kernel is the score replay (one launch per step, the "replay" stage); its duration
    # is the one measured live over the timed steps.  Bound: fp32 VALU (each gathered record is evaluated by up
    # to 256 pixels), counted with the method's per-unit operations; its HBM fraction is reported beside it.
    rep_ms = prof_timed["replay"][0] / max(prof_timed["replay"][1], 1)
    t_rep = rep_ms * 1e-3
    ops = OPS_EVAL * E + OPS_CONTRIB_REPLAY * K
    achieved = ops / t_rep / 1e12
    rep_bytes = REPLAY_BYTES_PAIR * P_walk + REPLAY_BYTES_PIXEL * N_px + REPLAY_BYTES_RECORD * V * sc.n
    traffic = measured_traffic("k_replay", workload, args.antialiased)
    roofline = {"kernel": "k_replay", "bound": "alu", "achieved": round(achieved, 3),
                "peak": round(ALU_PEAK_TOPS, 2), "unit": "T lane-ops/s (fp32 VALU)",
                "frac": round(achieved / ALU_PEAK_TOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(rep_ms, 4), "ops_per_launch": ops,
                "ops_per_unit": {"evaluation": OPS_EVAL, "contribution": OPS_CONTRIB_REPLAY},
                "units": {"evaluations": E, "contributions": K},
                "hbm": {"algorithmic_bytes": rep_bytes, "achieved_gbs": round(rep_bytes / t_rep / 1e9, 1),
                        "peak_gbs": HBM_PEAK_GBS, "frac": round(rep_bytes / t_rep / 1e9 / HBM_PEAK_GBS, 4),
                        "measured_gbs": None if traffic is None else round(traffic / t_rep / 1e9, 1),
                        "measured_frac": None if traffic is None else round(traffic / t_rep / 1e9 / HBM_PEAK_GBS, 4)}}
    t_ren = stages["render"][0] * 1e-3
    # the render skips, by its quadrant boxes, entries that fail the distance cut at every pixel of a quadrant,
    # so its evaluations are counted as those inside the cut (the ones no exact culling can skip)
    ops_r = OPS_EVAL * E_cut + OPS_CONTRIB_FWD * K
    secondary = {"k_render": {"bound": "alu", "achieved": round(ops_r / t_ren / 1e12, 3),
                              "frac": round(ops_r / t_ren / 1e12 / ALU_PEAK_TOPS, 4),
                              "units": {"evaluations_in_cut": E_cut, "contributions": K},
                              "traffic": measured_traffic("k_render<false>", workload, args.antialiased),
                              "avg_launch_ms": round(stages["render"][0], 4)}}
    for st in ("project", "depth_sort", "emit", "tile_sort", "ranges"):
        if st not in stages:
            continue
        by = stage_bytes(st, c)
        t = stages[st][0] * 1e-3
        secondary[st] = {"bound": "hbm", "achieved_gbs": round(by / t / 1e9, 1),
                         "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": by,
                         "avg_launch_ms": round(stages[st][0], 4)}
    render_ms = sum(stages[k][0] for k in RENDER_STAGES if k in stages)
    score_ms = sum(stages[k][0] for k in SCORE_STAGES if k in stages)

    out = {
        "value": round(N_px / (elapsed / steps) / 1e6, 2),
        "ms_per_step": round(ms_step, 4),
        "steps": steps,
        "config": {"workload": workload, "views": V, "height": H, "width": W, "gaussians": sc.n,
                   "sh_degree": sc.sh_degree, "pairs": P, "parallelism": "none",
                   "mode": "antialiased" if args.antialiased else "plain"},
        "contribs_per_s": round(K / (elapsed / steps), 1),
        "work_per_step": {"contributions": K, "evaluations": E, "evaluations_in_cut": E_cut, "pairs": P,
                          "pairs_walked": P_walk,
                          "live_records": n_live},
        "stages_ms": {k: round(v[0], 4) for k, v in stages.items()},
        "score_overhead": round(score_ms / render_ms, 4),
        # the same over a render/update step: the render path plus the renderer backward of the same frame
        "score_overhead_vs_update": None if bwd is None else round(score_ms / (render_ms + bwd["ms"]), 4),
        "roofline": roofline,
        "stage_rooflines": secondary,
        "memory": {"workspace_bytes": workspace_bytes, "peak_device_bytes": peak_bytes},
        "tokens_finite": finite,
    }
    if bwd is not None:
        t_b = bwd["stages"]["backward"] * 1e-3
        ops_b = OPS_EVAL * E + OPS_CONTRIB_BWD * K
        out["backward"] = {"ms": round(bwd["ms"], 4), "mpix_per_s": round(N_px / (bwd["ms"] * 1e-3) / 1e6, 2),
                           "stages_ms": {k: round(v, 4) for k, v in bwd["stages"].items()},
                           "k_backward": {"bound": "alu", "achieved": round(ops_b / t_b / 1e12, 3),
                                          "frac": round(ops_b / t_b / 1e12 / ALU_PEAK_TOPS, 4),
                                          "traffic": measured_traffic("k_backward", workload, args.antialiased),
                                          "avg_launch_ms": round(bwd["stages"]["backward"], 4),
                                          "ops_per_launch": ops_b},
                           "grads_finite": bwd["finite"], "loss": "1/2 |C_hat - C_obs|^2"}
    if attrs is not None:
        out["attributes"] = {"feature_composite_9ch_ms": round(attrs["features"], 4),
                             "attribution_2ch_ms": round(attrs["attribute"], 4), "finite": attrs["finite"]}
    return sc, out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the path is not sharded across GPUs)", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    if args.sweep:
        return sweep(args, dev, stream)

    sc, main_res = measure(args.config, args, dev, stream, args.steps, args.warmup, extras=True)
    others = {}
    for cfg in [int(x) for x in args.configs.split(",") if x.strip()]:
        if cfg == args.config:
            continue
        _, res = measure(cfg, args, dev, stream, max(1, min(args.steps, 10)), max(1, min(args.warmup, 2)),
                         extras=False)
        others[res["config"]["workload"]] = {k: res[k] for k in (
            "value", "ms_per_step", "steps", "config", "contribs_per_s", "work_per_step", "stages_ms",
            "score_overhead", "score_overhead_vs_update", "roofline", "stage_rooflines", "memory",
            "tokens_finite")}
        if "backward" in res:
            others[res["config"]["workload"]]["backward_ms"] = res["backward"]["ms"]

    out = {
        "metric": "render+score-replay Mpix/s",
        "value": main_res["value"],
        "unit": "Mpix/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
    }
    for k in ("config", "contribs_per_s", "work_per_step", "stages_ms", "score_overhead", "score_overhead_vs_update",
              "roofline", "stage_rooflines", "memory", "tokens_finite", "backward", "attributes"):
        if k in main_res:
            out[k] = main_res[k]
    if others:
        out["configs"] = others
    if not args.no_cpu_baseline and args.cpu_baseline_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(sc, args.cpu_baseline_seconds, antialiased=args.antialiased)
    print(json.dumps(out), flush=True)
    return 0


RENDER_STAGES = ("project", "depth_sort", "scan", "emit", "tile_sort", "ranges", "render")
SCORE_STAGES = ("replay", "finalize")


def sweep(args, dev, stream):
    """View-count and resolution scaling of the whole step over a fixed Gaussian
    set (the ReSplat-like pixel-aligned Gaussians of 8 source views), with the
    score-replay overhead = (replay + gather + tokens) / (project .. render)."""
    import numpy as np
    import torch

    import scenes
    from gaussian_splatting_rasterizer_amd import binding

    steps = max(1, min(args.steps, 10))
    for (W, H) in ((448, 256), (960, 512)):
        for V in (4, 8, 16, 32):
            sc = scenes.view_sweep(n_views=V, W=W, H=H)
            with torch.cuda.stream(stream):
                r = binding.rasterizer_for_scene(sc, device=dev)
                obs = torch.from_numpy(0.5 + sc.pixel_noise).to(dev)
                r.project_and_bin()
                r._alloc(int(r.n_pairs * 1.1) + 4096)
                outputs = r.new_outputs()
                tokens = torch.empty((sc.n, 9 + 3 * sc.d), dtype=torch.float32, device=dev)
                for _ in range(2):
                    r.step(obs, outputs, tokens)
                stream.synchronize()
                # the step time without stage events (each timed stage adds two event records to the stream),
                # then the same number of steps with every stage timed for the breakdown
                t0 = time.perf_counter()
                for _ in range(steps):
                    r.step(obs, outputs, tokens)
                stream.synchronize()
                elapsed = (time.perf_counter() - t0) / steps
                binding.gs_profile_enable(r.ctx, True)
                binding.gs_profile_read(r.ctx)
                for _ in range(steps):
                    r.step(obs, outputs, tokens)
                stream.synchronize()
                prof = binding.gs_profile_read(r.ctx)
                binding.gs_profile_enable(r.ctx, False)
                # the renderer backward of the same frame (a render/update step's other half), timed on its own
                grad_color = (outputs[0] - obs).contiguous()
                grads = r.new_grads()
                r.backward(grad_color, grads)
                stream.synchronize()
                tb = time.perf_counter()
                for _ in range(steps):
                    r.backward(grad_color, grads)
                stream.synchronize()
                bwd_ms = 1e3 * (time.perf_counter() - tb) / steps
                K = int(outputs[2].to(torch.int64).sum().item())
                P = int(r.n_pairs)
                r.close()
            del r, obs, outputs, tokens, grad_color, grads
            torch.cuda.empty_cache()
            st = {k: ms / max(cnt, 1) for k, (ms, cnt) in prof.items()}
            render_ms = sum(st[k] for k in RENDER_STAGES)
            score_ms = sum(st[k] for k in SCORE_STAGES)
            pix = V * H * W
            print(json.dumps({"sweep": "views_resolution", "views": V, "width": W, "height": H,
                              "gaussians": sc.n, "pairs": P, "contributions": K,
                              "ms_per_step": round(1e3 * elapsed, 4), "render_path_ms": round(render_ms, 4),
                              "score_ms": round(score_ms, 4), "score_overhead": round(score_ms / render_ms, 4),
                              "backward_ms": round(bwd_ms, 4),
                              "score_overhead_vs_update": round(score_ms / (render_ms + bwd_ms), 4),
                              "mpix_per_s": round(pix / elapsed / 1e6, 2),
                              "ns_per_pixel": round(1e9 * elapsed / pix, 3),
                              "stages_ms": {k: round(v, 4) for k, v in st.items()}}), flush=True)
            del sc
    return 0


def _host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(sc, budget_s, antialiased=False):
    """Oracle time of one frame of `sc`: full preprocess + tile lists, render + replay of an evenly
    spaced subset of tiles (score sums for every Gaussian) scaled to the frame, then tokens."""
    import numpy as np

    import oracle

    obs = (0.5 + sc.pixel_noise).astype(np.float32)   # the oracle is only timed here
    t0 = time.perf_counter()
    o = oracle.OracleScene(sc, antialiased=antialiased)
    o.build_lists()
    t_fixed = time.perf_counter() - t0
    o.select(None)
    n_tiles = o.V * o.T
    probe = np.arange(0, n_tiles, max(1, n_tiles // 64), dtype=np.int64)
    t1 = time.perf_counter()
    o.render(tiles=probe, obs=obs)
    t_probe = time.perf_counter() - t1
    per_tile = t_probe / len(probe)
    want = int(min(n_tiles, max(len(probe), budget_s / max(per_tile, 1e-9))))
    stride = max(1, n_tiles // want)
    sample = np.arange(stride // 2, n_tiles, stride, dtype=np.int64)
    o.select(None)
    t2 = time.perf_counter()
    o.render(tiles=sample, obs=obs)
    t_tiles = time.perf_counter() - t2
    t3 = time.perf_counter()
    o.tokens()
    t_tok = time.perf_counter() - t3
    full = t_fixed + t_tiles * (n_tiles / len(sample)) + t_tok
    pixels = o.V * o.H * o.W
    o.close()
    return {"value": round(pixels / full / 1e6, 4), "unit": "Mpix/s",
            "sample": f"preprocess + lists of all {sc.n} Gaussians x {sc.n_views} views, render+replay of "
                      f"{len(sample)}/{n_tiles} tiles (every {stride}th) scaled to the frame, tokens of all",
            "seconds": {"preprocess_lists": round(t_fixed, 3), "tiles": round(t_tiles, 3),
                        "tokens": round(t_tok, 3), "extrapolated_frame": round(full, 3)}}


def cpu_baseline(sc, budget_s, antialiased=False):
    """The oracle as it stands, timed on the host cores on a bounded sample of the same
    workload (all threads), plus single-thread rates of the same workload and of the
    occlusion toy on smaller samples."""
    import oracle
    import scenes

    threads = oracle.num_threads()
    res = _oracle_rate(sc, budget_s, antialiased)
    res.update({"cores": threads, "kind": "oracle", "host_cpu": _host_cpu_model()})
    one = {}
    oracle.set_num_threads(1)
    try:
        for name, s1 in ((scenes.CONFIG_NAMES[1], scenes.make_scene(1)), (sc.name, sc)):
            r1 = _oracle_rate(s1, budget_s / 5, antialiased)
            one[name] = {"value": r1["value"], "unit": "Mpix/s", "sample": r1["sample"],
                         "extrapolated_frame_s": r1["seconds"]["extrapolated_frame"]}
    finally:
        oracle.set_num_threads(threads)
    res["one_thread"] = one
    return res


if __name__ == "__main__":
    sys.exit(main())
