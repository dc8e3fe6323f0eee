"""Benchmark of the VC-Attention hot path on one MI355X.

One step = the whole path on one batch of synthetic video-DiT-shaped input already resident
in HBM: k-means grouping + label sort (vc_vsmooth_group), K/V smoothing and E4M3 operands
(vc_vsmooth_demean_quant) and the FP8 attention with ExpCast-FP8 (vc_attn_fwd).

Prints one JSON line.  `value` is attention work 4*B*H*N^2*d per step over the whole step's
time (grouping included on every step, the worst case); the attention kernel alone is also
timed with HIP events on the launch stream and reported against the FP8 MFMA peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config video|medium|reuse|long]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, vendor figure
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense FP4/FP6 MFMA, vendor figure
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "attn_fwd_video_traffic.json")
ATTN_SOURCES = ["bit_attention_video_amd/csrc/attn_fwd.hip", "bit_attention_video_amd/csrc/attn_common.h",
                "bit_attention_video_amd/csrc/vc_common.h"]


def attn_source_hash():
    """Hash of the attention kernel's sources, comments and blank lines left out: counters
    taken on other code are stale, while a comment edit does not change the kernel."""
    import hashlib
    import re
    tok = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            code = tok.sub(lambda m: "" if m.group(0).startswith("/") else m.group(0), fh.read())
        lines = [ln.rstrip() for ln in code.split("\n")]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_flops(B, H, N, d):
    return 4.0 * B * H * N * N * d


def cpu_baseline(cfg, Q, K, V, perm0, rows=16384):
    """The oracle's emulated VC attention for `rows` query rows of head 0 (full N keys)."""
    from oracle import attention as T
    from oracle import formats as F
    from oracle import vsmooth as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    Qh, Kh, Vh = (F.bf16_value_from_bits(x[0, 0]) for x in (Q, K, V))
    sel = np.unique(np.linspace(0, cfg.N - 1, rows).round().astype(np.int64))
    t0 = time.perf_counter()
    qc, sQ = S.quantize_q(Qh)
    kc, sK = S.quantize_k(Kh, perm0)
    vq = S.quantize_v(Vh, perm0)
    T.attention_tiled(F.e4m3_decode(qc), sQ, F.e4m3_decode(kc), sK, F.e4m3_decode(vq["codes"]),
                      vq["mu_t"], vq["sV"], rows=sel)
    dt = time.perf_counter() - t0
    flops = 4.0 * len(sel) * cfg.N * cfg.d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"emulated VC attention (operand quantisation + tiled ExpCast recurrence) for "
                      f"{len(sel)} query rows x {cfg.N} keys of one head, {dt:.1f} s; "
                      f"value = 4*rows*N*d / time"}


def measured_fp8_peak(vc, torch, workgroups=4096, iters=2000):
    """The device's attainable dense FP8 rate: the library's FP8 matrix-instruction loop
    (the instruction the attention kernel uses), timed with HIP events, best of three; and the
    shader clock (GHz, median over workgroups) the loop sustained in that best run."""
    vc.vc_test_mfma_fp8_rate(workgroups, 10)
    best, clock = float("inf"), None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, mhz = vc.vc_test_mfma_fp8_rate(workgroups, iters, clock=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if ms < best:
            best, clock = ms, float(mhz.median()) * 1e-3
    return workgroups * iters * 4194304.0 / (best * 1e-3) / 1e12, clock


def attn_clock_probe(vc, torch, Qd, ops, O, reps=5):
    """The attention kernel with its clock stamps on (vc_test_attn_fwd_clock), `reps` launches
    back to back timed with HIP events on the launch stream.  Returns (ms per launch, the shader
    clock in GHz the last launch ran at: its workgroups' summed shader cycles over their summed
    constant-rate ticks, times the counter's rate)."""
    args = (Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
    _, clk = vc.vc_test_attn_fwd_clock(*args, out=O)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        vc.vc_test_attn_fwd_clock(*args, out=O, clk=clk)
    e1.record()
    torch.cuda.synchronize()
    c = clk.cpu().numpy().astype(np.float64)
    ghz = (c[:, 2] - c[:, 0]).sum() / (c[:, 3] - c[:, 1]).sum() * vc.wall_clock_mhz() * 1e-3
    return e0.elapsed_time(e1) / reps, float(ghz)


def accuracy(cfg, Q, K, V, g, O, Ob, Oe, heads, nrows=256, O4=None, O6=None):
    """Accuracy of the timed path on sampled heads (computed after the timed region): the GPU output
    against the oracle's emulated recurrence on the GPU's permutation and against FP64 exact
    attention; the two unsmoothed sequence-order baselines (same P path, and exp-then-cast P)
    against exact; the grouping objective against the oracle's Lloyd from the same start; and,
    when given, the 4-bit and 6-bit paths' outputs on the same permutation against exact."""
    from oracle import attention as T
    from oracle import formats as F
    from oracle import vsmooth as S
    import torch
    perm = g["perm"].cpu().numpy()
    J = g["J"].cpu().numpy()
    val = lambda t: F.bf16_value_from_bits(t.cpu().view(torch.int16).numpy().view(np.uint16))
    O, Ob, Oe = val(O), val(Ob), val(Oe)
    O4 = val(O4) if O4 is not None else None
    O6 = val(O6) if O6 is not None else None
    rows = np.unique(np.linspace(0, cfg.N - 1, nrows).round().astype(np.int64))
    r = {"emu": [], "vc": [], "base": [], "etc": [], "J": [], "mx4": [], "mx6": []}
    for h in heads:
        Qh, Kh, Vh = (F.bf16_value_from_bits(x[0, h]) for x in (Q, K, V))
        qc, sQ = S.quantize_q(Qh)
        kc, sK = S.quantize_k(Kh, perm[0, h])
        vq = S.quantize_v(Vh, perm[0, h])
        emu = T.attention_tiled(F.e4m3_decode(qc), sQ, F.e4m3_decode(kc), sK, F.e4m3_decode(vq["codes"]),
                                vq["mu_t"], vq["sV"], rows=rows)
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        r["emu"].append(T.rel_l2(O[0, h][rows], emu))
        r["vc"].append(T.rel_l2(O[0, h][rows], exact))
        r["base"].append(T.rel_l2(Ob[0, h][rows], exact))
        r["etc"].append(T.rel_l2(Oe[0, h][rows], exact))
        if O4 is not None:
            r["mx4"].append(T.rel_l2(O4[0, h][rows], exact))
        if O6 is not None:
            r["mx6"].append(T.rel_l2(O6[0, h][rows], exact))
        J_ref = S.vsmooth_group(Vh, cfg.k, cfg.iters)["J"]
        r["J"].append(abs(float(J[0, h]) - J_ref) / J_ref)
    mean = lambda k: float(np.mean(r[k]))
    return {"heads": list(heads), "rows_per_head": int(len(rows)),
            "rel_l2_vs_emulated_max": round(max(r["emu"]), 6), "tolerance_vs_emulated": 5e-3,
            "rel_l2_vs_exact": round(mean("vc"), 6),
            "unsmoothed_same_p_vs_exact": round(mean("base"), 6),
            "unsmoothed_exp_then_cast_vs_exact": round(mean("etc"), 6),
            "vc_below_unsmoothed": mean("vc") < mean("base"),
            "kmeans_J_rel_err_max": float(f"{max(r['J']):.3e}"),
            **({"mx4_vs_exact": round(mean("mx4"), 6)} if r["mx4"] else {}),
            **({"mx6_vs_exact": round(mean("mx6"), 6)} if r["mx6"] else {})}


def time_ms(torch, fn, reps):
    """Mean launch time of fn() over reps back-to-back calls, HIP events on the current stream."""
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def config_summary(name, vc, torch):
    """One other workload at its full size, outside the timed region: grouping, demean/quantise and
    attention each timed over a few launches, and V-Smooth's cost relative to attention.  For the
    permutation-reuse workload, also the 4-step schedule with a cold and with a warm-started
    regroup (3 rounds from the previous grouping's centroids, the steady state of a schedule that
    regroups every 4 steps)."""
    import synth
    cfg = synth.get_config(name)
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    to = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    if cfg.steps > 1:
        Q, K, Vs = synth.make_reuse_steps(cfg)
        V = Vs[0]
    else:
        Q, K, V = synth.make_qkv(cfg)
    Qd, Kd, Vd = to(Q), to(K), to(V)
    g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
    ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
    O = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
    t_group = time_ms(torch, lambda: vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters), 3)
    t_dq = time_ms(torch, lambda: vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"]), 5)
    reps = max(3, int(300.0 / max(1e-3, attn_flops(B, H, N, d) / 2.5e12)))   # ~0.3 s of attention
    t_attn = time_ms(torch, lambda: vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"],
                                                   out=O), min(reps, 200))
    tf = attn_flops(B, H, N, d) / (t_attn * 1e-3) / 1e12
    out = {"workload": f"{name}: B={B} H={H} N={N} d={d} k={cfg.k}", "attn_ms": round(t_attn, 4),
           "attn_tflops": round(tf, 2), "frac": round(tf / FP8_PEAK_TFLOPS, 4), "group_ms": round(t_group, 4),
           "demean_quant_ms": round(t_dq, 4),
           "vsmooth_over_attn": {"grouping_step": round((t_group + t_dq) / t_attn, 4),
                                 "schedule_40_steps": round((3 * t_group + 10 * t_dq) / (40 * t_attn), 4)}}
    if cfg.steps > 1:
        Vds = [to(v) for v in Vs]
        t_warm = time_ms(torch, lambda: vc.vc_vsmooth_group(Vds[1], cfg.k, 3, C_init=g["C"]), 3)
        J_warm = vc.vc_vsmooth_group(Vds[1], cfg.k, 3, C_init=g["C"])["J"].double().mean().item()
        J_cold = vc.vc_vsmooth_group(Vds[1], cfg.k, cfg.iters)["J"].double().mean().item()
        S = cfg.steps
        out["reuse"] = {"steps": S, "warm_regroup_3_rounds_ms": round(t_warm, 4),
                        "window_cold_regroup": round((t_group + S * t_dq) / (S * t_attn), 4),
                        "window_warm_regroup": round((t_warm + S * t_dq) / (S * t_attn), 4),
                        "J_warm_3_over_J_cold_10": round(J_warm / J_cold, 6)}
        del Vds
    del Qd, Kd, Vd, ops, O, g
    torch.cuda.empty_cache()
    return out


def diagnostics():
    """The pages' error diagnostics on sampled heads of the medium, video and long workloads, of the
    Q/K channel-outlier workload (where a QK rotation has something to remove) and the reuse
    workload's warm start, computed by the oracle alone on the CPU: Eq. 2's split of the
    output error, the block-mean energy share and the value error by token order (Eq. 5, Fig. 4,
    Table 1), and the row total variation of ExpCast (Sec. 3.3).  One JSON line."""
    import synth
    from oracle import diagnostics as D
    from oracle import vsmooth as S
    plan = {"medium": [0, 4], "video": [0, 20], "long": [0, 12], "qk_outlier": [0, 2]}
    res = {}
    for name, heads in plan.items():
        cfg = synth.get_config(name)
        log(f"diagnostics: {name} heads {heads}")
        Qb, Kb, Vb = synth.make_qkv(cfg, heads)
        acc = {}
        for i, h in enumerate(heads):
            Q, K, V = (synth.bits_to_f32(x[0, i]).astype(np.float64) for x in (Qb, Kb, Vb))
            perm = S.vsmooth_group(V, cfg.k, cfg.iters)["perm"]
            cube = D.static_cube_order(cfg.grid, cfg.N)
            seq = np.arange(cfg.N)
            rows = np.sort(np.random.default_rng([cfg.cfg_id, h, 9]).choice(cfg.N, 256, replace=False))
            r = {"mean_share_sequence": D.block_mean_share(V[seq]),
                 "mean_share_static_cube": D.block_mean_share(V[cube]),
                 "mean_share_kmeans": D.block_mean_share(V[perm]),
                 "value_rmse_sequence": D.value_rel_mse(V, seq),
                 "value_rmse_hadamard_on_v": D.value_rel_mse(V, seq, rotate=True),
                 "value_rmse_static_cube": D.value_rel_mse(V, cube),
                 "value_rmse_kmeans": D.value_rel_mse(V, perm)}
            for tag, p_, dm in (("unsmoothed", None, False), ("vc", perm, True)):
                for rot in (False, True):
                    t = D.output_error_terms(Q, K, V, p_, rows, demean=dm, hadamard_qk=rot)
                    key = f"eq2_{tag}{'_qk_rotated' if rot else ''}"
                    for k2 in ("prob_term", "value_term", "value_share"):
                        r[f"{key}_{k2}"] = t[k2]
            tvr = D.row_tv(Q, K, rows)
            clean = tvr["tau"] < 1e-9
            r.update({"tv_expcast_mean": float(tvr["tv_expcast"].mean()), "tv_expcast_max": float(tvr["tv_expcast"].max()),
                      "tv_expcast_mean_no_underflow": float(tvr["tv_expcast"][clean].mean()) if clean.any() else None,
                      "tv_expcast_max_no_underflow": float(tvr["tv_expcast"][clean].max()) if clean.any() else None,
                      "tv_exp_then_cast_mean": float(tvr["tv_exp_then_cast"].mean()),
                      "rows_with_underflow": int((~clean).sum()),
                      "rows_over_0.0364_plus_tau": int((tvr["tv_expcast"] >= 0.0364 + tvr["tau"]).sum())})
            for k2, v in r.items():
                acc.setdefault(k2, []).append(v)
            log(f"  head {h}: " + json.dumps({k2: (round(v, 6) if isinstance(v, float) else v) for k2, v in r.items()}))
        agg = {}
        for k2, v in acc.items():
            v = [x for x in v if x is not None]
            if not v:
                agg[k2] = None
            elif k2.endswith("_max") or k2.endswith("_max_no_underflow"):
                agg[k2] = round(float(max(v)), 6)
            elif k2.startswith("rows_"):
                agg[k2] = int(sum(v))
            else:
                agg[k2] = round(float(np.mean(v)), 6)
        res[name] = {"workload": f"{name}: H={cfg.H} N={cfg.N} k={cfg.k}", "heads": heads, "rows_per_head": 256, **agg}
    # warm start (Table 1's warm-started row): step 1 of the reuse workload grouped by 3 rounds from
    # step 0's centroids, against a cold 10-round grouping of step 1
    cfg = synth.get_config("reuse")
    log("diagnostics: reuse head 0, warm start")
    Qb, Kb, Vs = synth.make_reuse_steps(cfg, [0])
    V0, V1 = (synth.bits_to_f32(v[0, 0]).astype(np.float64) for v in Vs[:2])
    g0 = S.vsmooth_group(V0, cfg.k, cfg.iters)
    warm = S.vsmooth_group(V1, cfg.k, 3, C_init=g0["C"])
    cold = S.vsmooth_group(V1, cfg.k, cfg.iters)
    res["reuse"] = {"workload": f"reuse: H={cfg.H} N={cfg.N} k={cfg.k}, step 1 of head 0",
                    "value_rmse_sequence": round(D.value_rel_mse(V1, None), 6),
                    "value_rmse_kmeans": round(D.value_rel_mse(V1, cold["perm"]), 6),
                    "value_rmse_kmeans_warm_3_rounds": round(D.value_rel_mse(V1, warm["perm"]), 6),
                    "value_rmse_previous_step_pi": round(D.value_rel_mse(V1, g0["perm"]), 6)}
    print(json.dumps({"diagnostics": res, "data": "synthetic", "kind": "oracle (CPU)"}), flush=True)


def reuse_schedule(args, cfg, vc, torch):
    """The permutation-reuse workload: V drifts over cfg.steps steps; grouping runs on the
    first step only and pi is reused (the pages' amortisation, Sec. 3.4).  Also times a
    warm-started 3-round regrouping of each later step from the previous centroids."""
    import synth
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    log(f"generating {cfg.name}: B={B} H={H} N={N} d={d} k={cfg.k}, {cfg.steps} steps")
    Q, K, Vs = synth.make_reuse_steps(cfg)
    to = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    Qd, Kd = to(Q), to(K)
    Vds = [to(v) for v in Vs]
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def schedule(rec):
        t = {"group": [], "dq": [], "attn": []}
        g = None
        for s_i, Vd in enumerate(Vds):
            e = [ev() for _ in range(4)]
            e[0].record()
            if s_i == 0:
                g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
            e[1].record()
            ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
            e[2].record()
            vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
            e[3].record()
            rec.append(e)
        return g

    for _ in range(args.warmup):
        schedule([])
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g = schedule(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_sched = args.steps
    ms_sched = wall * 1e3 / n_sched
    t_group = float(np.mean([r[0].elapsed_time(r[1]) for r in recs[0::cfg.steps]]))
    t_dq = float(np.mean([r[1].elapsed_time(r[2]) for r in recs]))
    t_attn = float(np.mean([r[2].elapsed_time(r[3]) for r in recs]))
    # warm start: regroup a later step from the previous step's centroids in 3 rounds
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(3):
        gw = vc.vc_vsmooth_group(Vds[1], cfg.k, 3, C_init=g["C"])
    e1.record()
    torch.cuda.synchronize()
    t_warm = e0.elapsed_time(e1) / 3
    J_cold = vc.vc_vsmooth_group(Vds[1], cfg.k, cfg.iters)["J"].double().mean().item()
    J_warm = gw["J"].double().mean().item()
    log(f"schedule {ms_sched:.2f} ms for {cfg.steps} steps: group {t_group:.2f} ms (step 1), "
        f"demean_quant {t_dq:.3f} ms, attn {t_attn:.2f} ms; warm regroup {t_warm:.2f} ms")
    fl = attn_flops(B, H, N, d)
    out = {
        "metric": "FP8 VC-attn fwd TFLOP/s at N=70K,H=40,d=128; % of FP8 MFMA peak",
        "value": round(fl * cfg.steps / (ms_sched * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_sched / cfg.steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} N={N} d={d}, {cfg.steps} steps with V drifting, "
                               f"grouping (k={cfg.k}, {cfg.iters} rounds) on the first step only, pi reused; "
                               f"one bench step = the {cfg.steps}-step schedule",
                   "B": B, "H": H, "N": N, "d": d, "k": cfg.k, "iters": cfg.iters, "reuse_steps": cfg.steps},
        "roofline": {"bound": "mfma", "achieved": round(fl / (t_attn * 1e-3) / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fl / (t_attn * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "k_attn_fwd", "avg_launch_ms": round(t_attn, 4)},
        "attn_ms": round(t_attn, 4), "group_ms": round(t_group, 4), "demean_quant_ms": round(t_dq, 4),
        "reuse": {
            "vsmooth_over_attn_reuse_window": round((t_group + cfg.steps * t_dq) / (cfg.steps * t_attn), 4),
            "warm_regroup_3_rounds_ms": round(t_warm, 4),
            "warm_over_cold_group_time": round(t_warm / t_group, 4),
            "J_warm_3_over_J_cold_10": round(J_warm / J_cold, 6),
            "vsmooth_over_attn_reuse_window_warm": round((t_warm + cfg.steps * t_dq) / (cfg.steps * t_attn), 4),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, Q, K, Vs[0], np.random.default_rng(0).permutation(N))
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="video")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true", help="skip the oracle accuracy report")
    ap.add_argument("--no-configs", action="store_true", help="skip the medium, reuse and long summaries")
    ap.add_argument("--diagnostics", action="store_true",
                    help="only the oracle's error diagnostics on sampled heads (CPU, no GPU)")
    ap.add_argument("--attn-only-iters", type=int, default=0,
                    help="extra back-to-back vc_attn_fwd launches timed alone (for profiling)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.diagnostics:
        return diagnostics()
    if args.copy_calib_mib:
        import torch
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import bit_attention_video_amd as vc
    import synth

    cfg = synth.get_config(args.config)
    if cfg.steps > 1:
        return reuse_schedule(args, cfg, vc, torch)
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    log(f"generating {cfg.name}: B={B} H={H} N={N} d={d} k={cfg.k}")
    t0 = time.perf_counter()
    Q, K, V = synth.make_qkv(cfg)
    log(f"generated in {time.perf_counter() - t0:.1f} s")
    dev = "cuda:0"
    to = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    Qd, Kd, Vd = to(Q), to(K), to(V)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev: ev[0].record()
        g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
        if ev: ev[1].record()
        ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
        if ev: ev[2].record()
        O = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
        if ev: ev[3].record()
        return g, ops, O

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        g, ops, O = step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    t_group = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_dq = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_attn = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    log(f"step {ms_step:.2f} ms: group {t_group:.2f} ms, demean_quant {t_dq:.3f} ms, attn {t_attn:.2f} ms")
    assert torch.isfinite(O.float()).all(), "non-finite attention output"

    # the same attention with P by exp-then-cast (v_exp_f32 + FP8 conversion) instead of ExpCast,
    # the comparator of the pages' Table 4, timed the same way on the same operands
    def time_attn(reps, **kw):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], out=O, **kw)
        e0.record()
        for _ in range(reps):
            vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], out=O, **kw)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    t_etc = time_attn(3, exp_then_cast=True)
    log(f"attention with exp-then-cast P: {t_etc:.2f} ms (ExpCast {t_attn:.2f} ms)")

    # the fused QK Hadamard rotation (App. B): rotated key codes, then attention rotating Q
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ops_rot = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"], hadamard=True)
    e0.record()
    for _ in range(3):
        ops_rot = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"], hadamard=True)
    e1.record()
    torch.cuda.synchronize()
    t_dq_rot = e0.elapsed_time(e1) / 3
    vc.vc_attn_fwd(Qd, ops_rot["Kq"], ops_rot["sK"], ops_rot["Rq"], ops_rot["mu"], ops_rot["sV"], out=O,
                   hadamard=True)
    e0.record()
    for _ in range(3):
        vc.vc_attn_fwd(Qd, ops_rot["Kq"], ops_rot["sK"], ops_rot["Rq"], ops_rot["mu"], ops_rot["sV"], out=O,
                       hadamard=True)
    e1.record()
    torch.cuda.synchronize()
    t_attn_rot = e0.elapsed_time(e1) / 3
    assert torch.isfinite(O.float()).all(), "non-finite attention output (rotated)"
    del ops_rot
    log(f"QK rotation: demean_quant {t_dq_rot:.3f} ms, attention {t_attn_rot:.2f} ms")

    # the 4-bit path (MX E2M1 operands, P by exp2): its quantisers and attention on the same pi
    ops4 = vc.vc_vsmooth_demean_quant_mx4(Kd, Vd, g["perm"])
    e0.record()
    for _ in range(3):
        ops4 = vc.vc_vsmooth_demean_quant_mx4(Kd, Vd, g["perm"])
    e1.record()
    torch.cuda.synchronize()
    t_dq4 = e0.elapsed_time(e1) / 3
    attn4 = lambda: vc.vc_attn_fwd_mx4(Qd, ops4["Kq4"], ops4["sK4"], ops4["Rq4"], ops4["sR4"], ops4["mu"], out=O)
    attn4()
    e0.record()
    for _ in range(3):
        attn4()
    e1.record()
    torch.cuda.synchronize()
    t_attn4 = e0.elapsed_time(e1) / 3
    assert torch.isfinite(O.float()).all(), "non-finite attention output (4-bit)"
    del ops4
    log(f"4-bit path: demean_quant {t_dq4:.3f} ms, attention {t_attn4:.2f} ms")

    # the 6-bit path (MX E2M3 operands, P by exp2), the same way
    ops6 = vc.vc_vsmooth_demean_quant_mx6(Kd, Vd, g["perm"])
    e0.record()
    for _ in range(3):
        ops6 = vc.vc_vsmooth_demean_quant_mx6(Kd, Vd, g["perm"])
    e1.record()
    torch.cuda.synchronize()
    t_dq6 = e0.elapsed_time(e1) / 3
    attn6 = lambda: vc.vc_attn_fwd_mx6(Qd, ops6["Kq6"], ops6["sK6"], ops6["Rq6"], ops6["sR6"], ops6["mu"], out=O)
    attn6()
    e0.record()
    for _ in range(3):
        attn6()
    e1.record()
    torch.cuda.synchronize()
    t_attn6 = e0.elapsed_time(e1) / 3
    assert torch.isfinite(O.float()).all(), "non-finite attention output (6-bit)"
    del ops6
    log(f"6-bit path: demean_quant {t_dq6:.3f} ms, attention {t_attn6:.2f} ms")

    if args.attn_only_iters:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.attn_only_iters):
            vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], out=O)
        e1.record()
        torch.cuda.synchronize()
        log(f"attn alone x{args.attn_only_iters}: {e0.elapsed_time(e1) / args.attn_only_iters:.3f} ms")

    fl = attn_flops(B, H, N, d)
    attn_tflops = fl / (t_attn * 1e-3) / 1e12
    value = fl / (ms_step * 1e-3) / 1e12
    # attention alone under the pages' timing protocol: 20 warm-up launches, then the median of
    # 50 individually event-timed launches
    for _ in range(20):
        vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], out=O)
    proto = []
    for _ in range(50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], out=O)
        e1.record()
        e1.synchronize()
        proto.append(e0.elapsed_time(e1))
    t_attn_med = float(np.median(proto))
    log(f"attention alone, median of 50 after 20 warm-up launches: {t_attn_med:.3f} ms")
    probe_ms, kernel_ghz = attn_clock_probe(vc, torch, Qd, ops, O)
    log(f"attention clock probe: {probe_ms:.3f} ms per launch at a {kernel_ghz:.3f} GHz shader clock")
    fp8_peak_meas, clock_ghz = measured_fp8_peak(vc, torch)
    log(f"measured dense FP8 rate {fp8_peak_meas:.0f} TFLOP/s at a {clock_ghz:.2f} GHz shader clock "
        f"(vendor figure {FP8_PEAK_TFLOPS:.0f})")
    # the HBM bandwidth a plain device-to-device copy reaches on this part (read + write bytes),
    # the practical ceiling beside which the V-Smooth kernels' GB/s read
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    t_copy = time_ms(torch, lambda: dst.copy_(src), 10)
    copy_gbs = 2.0 * (1 << 30) / (t_copy * 1e-3) / 1e9
    del src, dst
    log(f"plain device copy of 1 GiB: {t_copy:.3f} ms = {copy_gbs:.0f} GB/s (read + write)")
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            tr = json.load(f)
        if tr.get("config") == cfg.name and tr.get("kernel_source_sha256_16") == attn_source_hash():
            traffic = tr.get("bytes_per_launch")
    # V-Smooth cost relative to attention (the pages' schedule: 40 steps, grouping at steps 0, 4, 8,
    # demeaning on the first 25% of steps; the reuse window: group once, demean each of 4 steps)
    amort = {
        "grouping_step": (t_group + t_dq) / t_attn,
        "reuse_window_4": (t_group + 4 * t_dq) / (4 * t_attn),
        "schedule_40_steps": (3 * t_group + 10 * t_dq) / (40 * t_attn),
    }
    dq_bytes = 10.0 * B * H * N * d          # K, V read twice (bf16), Kq and Rq written
    out = {
        "metric": "FP8 VC-attn fwd TFLOP/s at N=70K,H=40,d=128; % of FP8 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} N={N} d={d}, full V-Smooth (k-means k={cfg.k}, "
                               f"{cfg.iters} Lloyd iters, sort, demean/quantise) + ExpCast FP8 attention",
                   "B": B, "H": H, "N": N, "d": d, "k": cfg.k, "iters": cfg.iters},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "k_attn_fwd", "avg_launch_ms": round(t_attn, 4),
                     "measured_peak": round(fp8_peak_meas, 1),
                     "measured_peak_clock_ghz": round(clock_ghz, 3),
                     "frac_of_measured_peak": round(attn_tflops / fp8_peak_meas, 4),
                     "kernel_clock_ghz": round(kernel_ghz, 3), "clock_probe_ms": round(probe_ms, 4),
                     "clock_probe_frac": round(fl / (probe_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                     "frac_of_clock_peak": round(fl / (probe_ms * 1e-3) / (256 * 8192 * kernel_ghz * 1e9), 4)},
        "attn_protocol": {"warmup_launches": 20, "launches": 50, "median_ms": round(t_attn_med, 4),
                          "tflops": round(fl / (t_attn_med * 1e-3) / 1e12, 2),
                          "frac": round(fl / (t_attn_med * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)},
        "attn_ms": round(t_attn, 4), "attn_tflops": round(attn_tflops, 2),
        "group_ms": round(t_group, 4), "demean_quant_ms": round(t_dq, 4),
        "demean_quant_gbs": round(dq_bytes / (t_dq * 1e-3) / 1e9, 1),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "vsmooth_over_attn": {k2: round(v2, 4) for k2, v2 in amort.items()},
        "p_path": {"expcast_ms": round(t_attn, 4), "exp_then_cast_ms": round(t_etc, 4),
                   "expcast_speedup": round(t_etc / t_attn, 4)},
        "mx4": {"demean_quant_ms": round(t_dq4, 4), "attn_ms": round(t_attn4, 4),
                "attn_tflops": round(attn_flops(B, H, N, d) / (t_attn4 * 1e-3) / 1e12, 2),
                "attn_frac_of_fp4_peak": round(attn_flops(B, H, N, d) / (t_attn4 * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4),
                "attn_over_8bit": round(t_attn4 / t_attn, 4)},
        "mx6": {"demean_quant_ms": round(t_dq6, 4), "attn_ms": round(t_attn6, 4),
                "attn_tflops": round(attn_flops(B, H, N, d) / (t_attn6 * 1e-3) / 1e12, 2),
                "attn_frac_of_fp6_peak": round(attn_flops(B, H, N, d) / (t_attn6 * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4),
                "attn_over_8bit": round(t_attn6 / t_attn, 4)},
        "qk_rotation": {"demean_quant_ms": round(t_dq_rot, 4), "attn_ms": round(t_attn_rot, 4),
                        "attn_over_unrotated": round(t_attn_rot / t_attn, 4),
                        "demean_quant_over_unrotated": round(t_dq_rot / t_dq, 4)},
    }
    if not args.no_configs:
        out["configs"] = {}
        for name in ("medium", "reuse", "long"):
            log(f"workload {name} (outside the timed region)")
            out["configs"][name] = config_summary(name, vc, torch)
            log(f"{name}: {json.dumps(out['configs'][name])}")
    if not args.no_accuracy:
        log("accuracy on sampled heads (oracle, outside the timed region)")
        base = vc.vc_vsmooth_demean_quant(Kd, Vd, None, no_demean=True)
        bargs = (Qd, base["Kq"], base["sK"], base["Rq"], None, base["sV"])
        Ob = vc.vc_attn_fwd(*bargs, no_mean=True)
        Oe = vc.vc_attn_fwd(*bargs, no_mean=True, exp_then_cast=True)
        O = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
        O4 = vc.vc_attention_mx4(Qd, Kd, Vd, g["perm"])
        O6 = vc.vc_attention_mx6(Qd, Kd, Vd, g["perm"])
        out["accuracy"] = accuracy(cfg, Q, K, V, g, O, Ob, Oe, heads=sorted({0, H // 2, H - 1}), O4=O4, O6=O6)
        del base, Ob, Oe, O4, O6
        log(f"accuracy: {json.dumps(out['accuracy'])}")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        perm0 = np.random.default_rng(0).permutation(N)   # any permutation: the cost does not depend on it
        out["cpu_baseline"] = cpu_baseline(cfg, Q, K, V, perm0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
