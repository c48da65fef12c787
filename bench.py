"""Benchmark of the verify path on one MI355X.

A step is one pass of the whole path over one batch: rva_schedule_and_pack (stages 1
and 2, one launch) -> rva_verify_attention -> rva_accept_and_commit (with the TV labels
fused), on the mixed-traffic workload (B = 64, gamma = 8, GQA 32/8 D = 128 bf16 paged KV,
contexts U[512, 8K], V = 151936 bf16 logits), compact mode.  With --overlap-schedule the
scheduling call of each step is for the next step and runs on a second stream beside the
acceptance kernels (zero-overhead scheduling, as the SGLang integration runs it), and the
serial step is reported beside it.  Inputs are resident in HBM
before the timed region; between steps context_lens is restored (a 256-byte device copy,
inside the timed region) so every step redoes the same work.

Prints ONE JSON line: packed verify tokens/s for the step, plus the achieved HBM GB/s of
verify attention + acceptance, the roofline of the dominant kernel (verify attention,
timed with HIP events on the stream it runs on) and the CPU oracle's rate on a bounded
sample of the same workload.  The default (compact) run also times static full-block
verify on the same inputs (`static`), and compares the step's commits and labels with the
oracle's on the sample (`parity_sample`: mismatches, and how many sit in the flip band).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "packed verify tokens/s + achieved HBM GB/s (% peak), verify attn + accept, B=64"


def algorithmic_bytes(wl, context_lens, windows):
    """Bytes each stage must move at minimum (one read of every input byte it needs,
    one write of every output byte)."""
    s_kv = 2 if wl.kv_dtype == "bf16" else 4
    s_lg = 2 if wl.logit_dtype == "bf16" else 4
    L = context_lens.astype(np.int64)
    w = windows.astype(np.int64)
    kvrow = wl.Hkv * wl.D * s_kv
    attn = int(np.sum(2 * (L + w) * kvrow      # read context K/V + window K/V
                      + 2 * w * kvrow          # append window K/V to the cache
                      + 2 * w * wl.Hq * wl.D * s_kv))  # read Q, write O
    accept = int(np.sum((2 * w - 1) * wl.V * s_lg))   # every target and draft row once
    flops = int(np.sum(4 * w * wl.Hq * wl.D * (L + (w + 1) / 2)))
    return attn, accept, flops


def profile_fields(name):
    """Fields ("key: value" lines) of a committed rocprofv3 summary under profiles/, or None
    when it is missing or the attention source changed since its counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", name)
    src = os.path.join(ROOT, "ragged_verify_acceptance_amd", "csrc", "attention.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "*", "cd ", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return fields if fields.get("attention_source_sha256") == sha else None


def counter_traffic(workload):
    """HBM bytes per launch of rva_verify_attention from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE passes, each scaled by the copy calibration), or None."""
    f = profile_fields(f"verify_attention_{workload}_hbm_counters.md")
    return float(f["traffic_bytes_per_launch"]) if f and "traffic_bytes_per_launch" in f else None


def counter_mfma(workload):
    """MFMA utilisation of attn_sk_kernel from the committed rocprofv3 counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs; MFMA ops x 512 over the
    dispatch time), or None."""
    f = profile_fields(f"verify_attention_{workload}_mfma_counters.md")
    if not f or "mfma_util_pct" not in f:
        return None
    return {"mfma_busy_pct": float(f["mfma_util_pct"]), "mfma_TFLOPs": float(f["mfma_tflops"]),
            "mfma_flops_per_launch": float(f["mfma_flops_per_launch"]),
            "source": f"profiles/verify_attention_{workload}_mfma_counters.md"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(inp, windows, n_req):
    """The oracle, single-threaded, on the first n_req requests of the same workload."""
    from threadpoolctl import threadpool_limits

    import oracle
    from tests.reference import sub_pool

    wl = inp.wl
    reqs = list(range(n_req))
    # inputs prepared outside the timed region
    k_pool, v_pool, bt, _ = sub_pool(inp, reqs)
    ws = [int(windows[b]) for b in reqs]
    cu = np.concatenate([[0], np.cumsum(ws)]).astype(np.int32)
    R = int(cu[-1])
    q = np.zeros((R, wl.Hq, wl.D))
    kn = np.zeros((R, wl.Hkv, wl.D))
    vn = np.zeros((R, wl.Hkv, wl.D))
    logits = []
    for j, b in enumerate(reqs):
        qb, kb, vb = inp.request_qkv(b)
        q[cu[j]:cu[j + 1]] = qb[: ws[j]].double().numpy()
        kn[cu[j]:cu[j + 1]] = kb[: ws[j]].double().numpy()
        vn[cu[j]:cu[j + 1]] = vb[: ws[j]].double().numpy()
        tl, dl, toks = inp.request_logits(b)
        logits.append((tl[: ws[j]].double().numpy(), dl[: ws[j] - 1].double().numpy(), toks))
    ua, ur = inp.uniforms()
    conf = inp.conf()
    bias, alpha, theta = inp.cost_tables()
    reps, dt = 0, 0.0
    results = {}
    with threadpool_limits(1):
        # the sample is repeated until about 10 s of CPU work (at most 5 passes)
        while reps < 5 and dt < 10.0:
            t0 = time.perf_counter()
            a = oracle.survival(conf)
            oracle.schedule_windows(a, wl.gamma, bias, alpha, theta)
            oracle.pack_ragged(windows, inp.context_lens, wl.tiers)
            oracle.verify_attention(q, kn, vn, k_pool, v_pool, bt, inp.context_lens[reqs], cu, R,
                                    np.float32(1.0 / np.sqrt(wl.D)))
            for j, b in enumerate(reqs):
                tl, dl, toks = logits[j]
                results[b] = oracle.accept_request(tl, dl, toks[: ws[j] - 1], ua[b, : ws[j] - 1],
                                                   ur[b])
            dt += time.perf_counter() - t0
            reps += 1
    return results, {"value": reps * R / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_req} of {inp.B} requests of {wl.name} ({R} packed verify rows): "
                      f"full-batch scheduling + pack, then attention and acceptance+labels of the "
                      f"sample, float64 NumPy, 1 thread, {reps} pass(es) in {dt:.1f} s on "
                      f"{cpu_model()} ({len(os.sched_getaffinity(0))} cores visible)"}


def stage_times(ds, n_ev, stream, capped=False):
    """Mean HIP-event durations (ms) of schedule + pack, attention and acceptance inside
    whole steps, on the stream the kernels are launched on."""
    import torch

    wl = ds.wl
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]
    for i in range(n_ev):
        ds.restore()
        ev[i][0].record(stream)
        if capped:
            ds.schedule()
            ds.cap_windows.copy_(ds.windows)
            ds.windows.fill_(wl.gamma)
            ds.pack()
        else:
            ds.schedule_pack()
        ev[i][1].record(stream)
        ds.attention()
        ev[i][2].record(stream)
        if capped:
            ds.accept_capped(None)
        else:
            ds.accept(labels=True)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    return tuple(float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n_ev)]))
                 for j in range(3))


def time_steps(step, steps, warmup, stream):
    """Mean ms per step over exactly `steps` back-to-back steps after `warmup` untimed ones."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def static_arm(inp, steps, warmup, stream):
    """Static full-block verify on the same inputs: every request verifies its whole block
    (window gamma), the arm the compact mode is compared with."""
    from workloads.device import DeviceStep

    wl = inp.wl
    ds = DeviceStep(inp, mode="static")
    ds.prepare()

    def step():
        ds.restore()
        ds.step()

    ms = time_steps(step, steps, warmup, stream)
    t_front, t_attn, t_acc = stage_times(ds, max(10, steps // 2), stream)
    windows = ds.windows.cpu().numpy()
    M = int(ds.total_tier[0].item())
    attn_b, acc_b, _ = algorithmic_bytes(wl, inp.context_lens, windows)
    committed = int(ds.accept_len.sum().item()) + inp.B
    gbs = (attn_b + acc_b) / ((t_attn + t_acc) * 1e-3) / 1e9
    return {"ms_per_step": ms, "packed_rows_M": M, "tokens_per_s": M / (ms * 1e-3),
            "committed_tokens_per_step": committed,
            "goodput_committed_tokens_per_s": committed / (ms * 1e-3),
            "attn_ms": t_attn, "accept_ms": t_acc, "schedule_pack_ms": t_front,
            "verify_attn_accept_GBps": gbs, "pct_peak": 100.0 * gbs / PEAK_HBM_GBS,
            "device_status": int(ds.status.item())}


def sample_parity(ds, results, windows):
    """The GPU step's commits and labels against the oracle's on the baseline sample:
    requests whose commit differs, and how many of those sit in the flip band (an accept
    test within 1e-6 of its threshold, or a draw within 1e-9 of a bin edge)."""
    committed = ds.committed.cpu().numpy()
    accept_len = ds.accept_len.cpu().numpy()
    labels = ds.labels.cpu().numpy()
    mism = band = 0
    lab_err = 0.0
    for b, r in results.items():
        w = int(windows[b])
        n = int(accept_len[b])
        same = n == r["n"] and list(committed[b, : n + 1]) == list(r["committed"])
        near = any(m < 1e-6 for m in r["margins"]) or r["draw_margin"] < 1e-9
        if not same:
            mism += 1
            band += int(near)
        if w > 1:
            lab_err = max(lab_err, float(np.max(np.abs(labels[b, : w - 1] - np.asarray(r["labels"])))))
    return {"requests_checked": len(results), "commit_mismatches": mism,
            "mismatches_in_flip_band": band, "labels_max_abs_err": lab_err}


def cost_table(inp, reps, warm):
    """T(bs, M) of the verify calls measured by graph replay on the first bs requests, the
    additive fit, and the windows the scheduler picks on the fitted tier-aware tables."""
    import torch

    from ragged_verify_acceptance_amd.costmodel import (fit_additive, fit_linear,
                                                        scheduler_tables)
    from workloads.costgrid import measure
    from workloads.device import DeviceStep

    wl = inp.wl
    ds = DeviceStep(inp)
    ds.prepare()
    bs_list = sorted({b for b in (1, 2, 4, 8, 16, 32, 48, 64, 128, 256) if b <= inp.B} | {inp.B})
    samples, sched = measure(ds, bs_list, reps=reps, warm=warm)
    fit = fit_additive(samples, ds.tiers)
    _, alpha_lin, theta1, rms_lin = fit_linear(samples)
    bias, alpha, theta = scheduler_tables(fit, inp.B, wl.gamma, ds.tiers)
    # the whole step's floor adds the scheduling call at the full batch
    alpha = (alpha + np.float32(np.interp(np.arange(inp.B + 1), list(sched), list(sched.values()))))
    windows_pages = ds.windows.cpu().numpy()  # scheduled on the pages' cost line at prepare()
    ds.bias = float(bias)
    ds.alpha = torch.from_numpy((alpha * 1e-3).astype(np.float32)).cuda()
    ds.theta = torch.from_numpy((theta * 1e-3).astype(np.float32)).cuda()
    ds.restore()
    ds.schedule()
    ds.pack()
    torch.cuda.synchronize()
    w = ds.windows.cpu().numpy()
    M, tier = (int(x) for x in ds.total_tier.cpu().numpy())
    return {
        "metric": "verify step cost T(bs, M) by graph replay (us) and the scheduler on it",
        "unit": "us", "n_gpus": 1, "data": "synthetic", "workload": wl.name,
        "reps_per_point": reps,
        "grid": [[b, m, round(t, 2)] for b, m, t in samples],
        "schedule_us": {str(b): round(t, 2) for b, t in sched.items()},
        "fit_tier_aware": {"bs": fit.bs.tolist(), "alpha_us": np.round(fit.alpha, 2).tolist(),
                           "tiers": fit.tiers.tolist(), "theta_us": np.round(fit.theta, 2).tolist(),
                           "rms_us": fit.rms, "max_abs_us": fit.max_abs},
        "fit_linear": {"alpha_us": np.round(alpha_lin, 2).tolist(), "theta_us_per_token": theta1,
                       "rms_us": rms_lin},
        "scheduler_on_measured_tables": {"mean_window": float(w.mean()), "M": M, "tier": tier,
                                         "K": int(ds.K_out.item())},
        "scheduler_on_pages_cost_line": {"mean_window": float(windows_pages.mean()),
                                         "M": int(windows_pages.sum())},
    }


def markov_bench(wl, steps, warmup, cpu):
    """Markov sequential head over the workload's batch: G1 positions drawn in order, each
    an int8-MFMA vocabulary pass and a per-request draw; HIP events on the launch stream."""
    import torch

    from ragged_verify_acceptance_amd import rva
    from workloads.generate import markov_inputs

    B, G1, V, r = wl.B, wl.G1, wl.V, 256
    inp = markov_inputs(wl.seed, B, G1, V, r=r, dtype=wl.logit_dtype)
    dev = "cuda"
    t = lambda x, d: torch.as_tensor(np.ascontiguousarray(x)).to(d).to(dev)
    U = inp["U"].to(dev)
    anchor, u = t(inp["anchor"], torch.int32), t(inp["u"], torch.float32)
    q1, s1 = t(inp["q1"], torch.int8), t(inp["s1"], torch.float32)
    q2, s2 = t(inp["q2"], torch.int8), t(inp["s2"], torch.float32)
    out = torch.empty_like(U)
    tokens = torch.empty((B, G1), dtype=torch.int32, device=dev)
    p_at = torch.empty((B, G1), dtype=torch.float32, device=dev)
    ws = torch.empty(rva.markov_workspace_size(B, V), dtype=torch.uint8, device=dev)

    def call():
        rva.markov_sample(B, G1, V, r, U, anchor, u, q1, s1, q2, s2, out, tokens, p_at, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s_lg = 2 if wl.logit_dtype == "bf16" else 4
    # per position: the q2 factor once, U in, logits out, the gathered q1 rows, the scales
    per_pos = V * r + 2 * B * V * s_lg + B * r + 2 * V * 4
    bytes_call = G1 * per_pos
    gbs = bytes_call / (ms * 1e-3) / 1e9
    res = {
        "metric": "Markov sequential head: drafted tokens/s (B requests x gamma-1 positions)",
        "value": B * G1 / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "i8 x i8 -> i32, f64",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} Markov head", "B": B, "G1": G1, "V": V, "r": r,
                   "logit_dtype": wl.logit_dtype},
        "roofline": {"kernel": "rva_markov_sample (markov_logits_kernel + markov_sample_kernel)",
                     "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None, "algorithmic_bytes": bytes_call},
        "int8_TOPs": 2.0 * B * r * V * G1 / (ms * 1e-3) / 1e12,
    }
    if cpu:
        import time

        from threadpoolctl import threadpool_limits

        import oracle

        n = 2
        with threadpool_limits(1):
            t0 = time.perf_counter()
            oracle.markov_sample(inp["U"][:n], inp["anchor"][:n], inp["u"][:n], inp["q1"],
                                 inp["s1"], inp["q2"], inp["s2"])
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n * G1 / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {B} requests x {G1} positions, float64 NumPy, "
                                         f"1 thread, {dt:.1f} s"}
    return res


def sts_bench(wl, steps, reps, cpu):
    """Acceptance trace from the acceptance call itself (full blocks, so every position is
    observed), an over-confident head on it, then the STS fit and ECE calls, timed."""
    import torch

    from ragged_verify_acceptance_amd import rva

    B, gamma, G1, V = wl.B, wl.gamma, wl.G1, 4096
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    sig = torch.tensor([wl.classes[b % len(wl.classes)].sigma for b in range(B)], device=dev)
    cu = torch.arange(0, B * gamma + 1, gamma, dtype=torch.int32, device=dev)
    acc_ws = torch.zeros(rva.accept_workspace_size(B, gamma, V, B * gamma), dtype=torch.uint8, device=dev)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    committed = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    ctx = torch.zeros(B, dtype=torch.int32, device=dev)
    labels = torch.empty((steps, B, G1), dtype=torch.float32, device=dev)
    n_all = torch.empty((steps, B), dtype=torch.int32, device=dev)
    for s in range(steps):
        # the drafter's side (outside the path): logits and tokens sampled from the draft
        target = 2.0 * torch.randn((B * gamma, V), generator=g, device=dev)
        draft = (target.view(B, gamma, V)[:, :G1]
                 + sig[:, None, None] * torch.randn((B, G1, V), generator=g, device=dev)).contiguous()
        gum = -torch.log(-torch.log(torch.rand((B, G1, V), generator=g, device=dev).clamp_min(1e-30)))
        tokens = torch.argmax(draft + gum, dim=-1).to(torch.int32).contiguous()
        u_acc = torch.rand((B, G1), generator=g, device=dev)
        u_res = torch.rand(B, generator=g, device=dev)
        rva.accept_and_commit(B, gamma, V, B * gamma, target, draft, tokens, u_acc, u_res, cu,
                              accept_len, committed, ctx, None, None, labels[s], acc_ws)
        n_all[s].copy_(accept_len)
    # an over-confident head that tracks the label: z = T* logit(c*) + noise
    T_star = torch.tensor([1.5 + 0.1 * k for k in range(G1)], device=dev)
    q = labels.clamp(1e-6, 1 - 1e-6)
    z = (T_star * torch.log(q / (1 - q))
         + 0.3 * torch.randn(q.shape, generator=g, device=dev)).reshape(-1, G1).contiguous()
    n = n_all.reshape(-1).contiguous()
    N = z.shape[0]
    T = torch.empty(G1, dtype=torch.float32, device=dev)
    nll = torch.empty(G1, dtype=torch.float64, device=dev)
    ws = torch.empty(rva.sts_fit_workspace_size(N), dtype=torch.uint8, device=dev)
    ece_before = torch.empty(G1 + 1, dtype=torch.float64, device=dev)
    ece_after = torch.empty(G1 + 1, dtype=torch.float64, device=dev)
    ews = torch.empty(rva.calibration_ece_workspace_size(N, G1, 15), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    rva.sts_fit(N, G1, z, n, None, 0.05, 20.0, T, nll, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_fit, t_ece = [], []
    for _ in range(reps):
        ev[0].record(stream)
        rva.sts_fit(N, G1, z, n, None, 0.05, 20.0, T, nll, ws)
        ev[1].record(stream)
        rva.calibration_ece(N, G1, z, n, None, T, 15, ece_after, None, ews)
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_fit.append(ev[0].elapsed_time(ev[1]))
        t_ece.append(ev[1].elapsed_time(ev[2]))
    rva.calibration_ece(N, G1, z, n, None, None, 15, ece_before, None, ews)
    torch.cuda.synchronize()
    ms_fit, ms_ece = float(np.median(t_fit)), float(np.median(t_ece))
    nn = n.cpu().numpy()
    res = {
        "metric": "STS fit + ECE on an acceptance trace from the acceptance call",
        "value": N / ((ms_fit + ms_ece) * 1e-3), "unit": "trace samples/s", "n_gpus": 1,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{wl.name} classes, V={V} f32 logits, full blocks",
                   "B": B, "gamma": gamma, "trace_steps": steps, "N": N, "n_bins": 15,
                   "T_bracket": [0.05, 20.0]},
        "sts_fit_ms": ms_fit, "ece_ms": ms_ece,
        "head_T_true": [round(float(x), 3) for x in T_star.cpu()],
        "T_fit": [round(float(x), 4) for x in T.cpu()],
        "ece_before": {"pooled": float(ece_before[0]), "per_position": ece_before[1:].cpu().tolist()},
        "ece_after": {"pooled": float(ece_after[0]), "per_position": ece_after[1:].cpu().tolist()},
        "mean_accept_len": float(nn.mean()),
        "mean_tv_label": float(labels.mean()),
    }
    if cpu:
        import time

        from threadpoolctl import threadpool_limits

        import oracle

        zc, nc = z.cpu().numpy(), nn
        with threadpool_limits(1):
            t0 = time.perf_counter()
            r = oracle.sts_fit(zc, nc, grid=513)
            oracle.ece(zc, nc, T=r["T"], n_bins=15)
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": N / dt, "unit": "trace samples/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the whole trace ({N} samples x {G1} positions): "
                                         f"sts_fit (513-point scan + bounded refinement) and ECE, "
                                         f"float64 NumPy, 1 thread, {dt:.1f} s"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed-b64")
    ap.add_argument("--mode", default="compact",
                    choices=["compact", "static", "cap-accept", "cost-table", "sts", "markov"],
                    help="cap-accept: whole blocks verified, commits capped at the scheduled windows; "
                         "cost-table: measure T(bs, M) by graph replay and fit the scheduler's tables")
    ap.add_argument("--trace-steps", type=int, default=200,
                    help="sts mode: verify steps (of B requests) in the acceptance trace")
    ap.add_argument("--overlap-schedule", action="store_true",
                    help="run each step's scheduling call for the next step on a second stream, "
                         "beside the acceptance kernels (the serial step is reported beside it)")
    ap.add_argument("--graph", action="store_true",
                    help="time each step as one replay of the captured step graph")
    ap.add_argument("--cpu-sample", type=int, default=64, help="requests in the oracle sample (0: skip)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="touch 1 GiB before every timed step (working sets under the 256 MB "
                         "Infinity Cache); each step is then timed alone and the median reported")
    ap.add_argument("--no-static", action="store_true",
                    help="skip the static full-block arm of the default run (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the verify path shards by request: each GPU runs its own batch with this library)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from __graft_entry__ import _ensure_built
    _ensure_built()
    from workloads import Inputs, get
    from workloads.device import DeviceStep

    torch.cuda.set_device(0)
    wl = get(args.workload)
    if args.mode == "markov":
        print(json.dumps(markov_bench(wl, steps=args.steps, warmup=args.warmup,
                                      cpu=args.cpu_sample > 0)))
        return
    if args.mode == "sts":
        print(json.dumps(sts_bench(wl, args.trace_steps, reps=max(3, args.steps),
                                   cpu=args.cpu_sample > 0)))
        return
    inp = Inputs(wl)
    if args.mode == "cost-table":
        print(json.dumps(cost_table(inp, reps=max(5, args.steps), warm=max(1, args.warmup))))
        return
    capped = args.mode == "cap-accept"
    ds = DeviceStep(inp, mode="compact" if capped else args.mode)
    ds.prepare()
    if capped:
        from workloads.device import prepare_with_windows
        caps = ds.windows.cpu().numpy()
        prepare_with_windows(ds, np.full(inp.B, wl.gamma))
    torch.cuda.synchronize()
    windows = ds.windows.cpu().numpy()
    M, tier = (int(x) for x in ds.total_tier.cpu().numpy())
    attn_b, acc_b, attn_flops = algorithmic_bytes(wl, inp.context_lens, windows)

    stream = torch.cuda.current_stream()
    # a plain 1 GiB device-to-device copy on this GPU, for scale (and the counter calibration)
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(3):
        y.copy_(x)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    flush = x if args.flush_mall else None
    del y
    if flush is None:
        del x

    graph = None
    if args.graph:
        if capped:
            sys.exit("bench.py: --graph times the compact and static steps only")
        from ragged_verify_acceptance_amd.graph import CallGraph
        ds.restore()
        graph = CallGraph(ds.step)

    overlap = args.overlap_schedule and not (capped or graph is not None)
    side = torch.cuda.Stream() if overlap else None  # default priority
    ev_attn = torch.cuda.Event() if overlap else None
    ev_sched = torch.cuda.Event() if overlap else None

    def step():
        ds.restore()
        if capped:
            ds.step_capped()
        elif graph is not None:
            graph.replay()
        elif overlap:
            ds.step_overlapped(side, ev_attn, ev_sched)
        else:
            ds.step()

    def serial_step():
        ds.restore()
        ds.step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` whole steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if flush is None:
        e0.record(stream)
        t_host = time.perf_counter()
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t_host
        ms_step = e0.elapsed_time(e1) / args.steps
    else:
        # the cache is flushed before each step, outside its own event pair
        per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t_host = time.perf_counter()
        for a0, a1 in per:
            flush.add_(1)
            a0.record(stream)
            step()
            a1.record(stream)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t_host
        ms_step = float(np.median([a0.elapsed_time(a1) for a0, a1 in per]))

    # the same number of steps with the scheduling call in line, for comparison
    ms_serial = None
    if overlap:
        for _ in range(3):
            serial_step()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(stream)
        for _ in range(args.steps):
            serial_step()
        s1.record(stream)
        torch.cuda.synchronize()
        ms_serial = s0.elapsed_time(s1) / args.steps

    # ---- per-stage durations inside whole steps (HIP events on the launch stream)
    t_front, t_attn, t_acc = stage_times(ds, max(10, args.steps // 2), stream, capped)
    status = int(ds.status.item())

    attn_gbs = attn_b / (t_attn * 1e-3) / 1e9
    acc_gbs = acc_b / (t_acc * 1e-3) / 1e9
    path_gbs = (attn_b + acc_b) / ((t_attn + t_acc) * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": M / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": args.mode, "B": wl.B, "gamma": wl.gamma,
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "page": wl.page, "V": wl.V,
                   "packed_rows_M": M, "tier": tier, "mean_window": float(windows.mean()),
                   "mean_context": float(inp.context_lens.mean()), "graph": bool(args.graph),
                   "schedule_overlapped": overlap},
        "ms_per_step_serial_schedule": ms_serial,
        "verify_attn_accept": {
            "achieved_GBps": path_gbs, "pct_peak": 100.0 * path_gbs / PEAK_HBM_GBS,
            "tokens_per_s": M / ((t_attn + t_acc) * 1e-3),
            "attn_ms": t_attn, "accept_ms": t_acc, "schedule_pack_ms": t_front,
            "attn_bytes": attn_b, "accept_bytes": acc_b,
            "attn_GBps": attn_gbs, "accept_GBps": acc_gbs,
            "attn_TFLOPs": attn_flops / (t_attn * 1e-3) / 1e12,
        },
        "roofline": {"kernel": "rva_verify_attention (attn_sk_kernel + attn_merge_kernel)",
                     "bound": "hbm", "achieved": attn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": attn_gbs / PEAK_HBM_GBS, "traffic": counter_traffic(wl.name),
                     "algorithmic_bytes": attn_b, "mfma_counters": counter_mfma(wl.name)},
        "device_status": status,
        "committed_tokens_per_step": int(ds.accept_len.sum().item()) + inp.B,
        "goodput_committed_tokens_per_s": (int(ds.accept_len.sum().item()) + inp.B) / (ms_step * 1e-3),
        "copy_1GiB_GBps": copy_gbs,
        "device": {"name": torch.cuda.get_device_name(0),
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
                   "cus": torch.cuda.get_device_properties(0).multi_processor_count},
        "flush_mall": bool(args.flush_mall),
        "host_wall_s": t_host,
    }
    if capped:
        acc = int(ds.accept_len.sum().item())
        full = int(ds.accept_len_full.sum().item())
        res["cap_accept"] = {"accepted_drafts_capped": acc, "accepted_drafts_uncapped": full,
                             "utilisation": acc / max(1, full),
                             "mean_cap_window": float(caps.mean())}
    # windows per traffic class (requests are assigned to classes round-robin)
    hist = {}
    for ci, cl in enumerate(wl.classes):
        ws = windows[np.asarray(inp.classes) == ci]
        hist[f"class{ci} Beta({cl.a:g},{cl.b:g})"] = [int((ws == w).sum()) for w in range(1, wl.gamma + 1)]
    res["window_histogram"] = {"windows": list(range(1, wl.gamma + 1)), "per_class": hist}
    if args.mode == "compact" and graph is None and flush is None and not args.no_static:
        res["static"] = static_arm(inp, args.steps, args.warmup, stream)
    if args.cpu_sample > 0:
        results, res["cpu_baseline"] = cpu_baseline(inp, windows, min(args.cpu_sample, inp.B))
        if not capped:
            res["parity_sample"] = sample_parity(ds, results, windows)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
