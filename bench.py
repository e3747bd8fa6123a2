#!/usr/bin/env python3
"""Benchmark of the shared-INT4 speculative-decoding hot path on one MI355X.

One step = one QSPEC round over a Llama-3-8B-shaped model's projections and vocabulary head (32
layers of qkv 4096->6144, o 4096->4096, gate+up 4096->2x14336, down 14336->4096, each layer with
its own shared INT4 group-128 weights: 3.65 GB, far beyond the 256 MB last-level cache; the head
4096->128256, 275 MB), batch B (default 16) and gamma = 4:
  draft   gamma x (per layer and projection: qspec_quantize_act + qspec_gemm_w4a4 at M = B; then
          the head: qspec_quantize_act + qspec_gemm_w4a4 at M = B writing that step's fp32 draft
          logits, and qspec_draft_sample drawing each sequence's draft token from them into the
          draft-token buffer the verification reads; the rows are kept as q_j)
  verify  per layer and projection qspec_gemm_w4a16 at M = B (gamma + 1), then the head at
          M = B (gamma + 1) writing the [B][gamma + 1][V] fp32 target logits
  accept  qspec_verify_accept (speculative sampling) on those target and draft logits
  commit  qspec_kv_overwrite of the accepted rows in a 32-layer x 8-head x 4096 x 128 bf16 cache
Attention, norms and activation functions are not on this path: every projection reads fixed
synthetic activations, and the head reads fixed hidden rows (draft step j and verify position j
read the same row, so draft and target logits differ only by the W4A4 / W4A16 arithmetic on the
shared weights).

Each phase of each draft step is captured once as a HIP graph and replayed; HIP events between
phase replays time each phase.  The value is verify tokens/s: B (gamma + 1) positions per round
over the measured round time.  The dominant GEMM phase's graphs hold only that GEMM's launches,
so its event time divided by the launch count is the kernel's average launch duration; with the
algorithmic bytes per launch it gives the roofline figure.
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

METRIC = "shared-INT4 GEMM HBM TB/s (% of peak) at M=1..16; verify tokens/s at gamma=4"
HBM_PEAK_GBS = 8000.0
GROUP = 128
VOCAB = 128256
KV_HEADS, HEAD_DIM, CONTEXT = 8, 128, 4096


def w4_bytes(K, N):
    """Algorithmic bytes of the shared weights: 4-bit codes plus a binary16 scale and an 8-bit zero
    point per (column, 128-group), 0.5234375 B per weight.  (The store's meta word pads the pair to
    4 bytes, 0.53125 B per weight; the padding is the store's, not the method's.)"""
    return K * N // 2 + 3 * N * (K // GROUP)


def w4a4_alg_bytes(M, K, N):
    return w4_bytes(K, N) + M * K // 2 + 4 * M * (K // GROUP) + 2 * M * N


def w4a16_alg_bytes(M, K, N):
    return w4_bytes(K, N) + 2 * M * K + 2 * M * N


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "pmc_traffic.json")
COPY_MIB = 256


# How the summaries under profiles/ are made (OUT = an output folder, REPO = this repository).
PROFILE_COMMAND = ('cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o bench -- python3 REPO/bench.py --steps 3 --warmup 1 --no-cpu-baseline ; rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/prof_fetch -o bench -- python3 REPO/bench.py --steps 1 --warmup 0 --no-cpu-baseline --copy-calibration-mib 256 ; (the same with --pmc WRITE_SIZE -d OUT/prof_write) ; python3 REPO/bench.py --summarize OUT/prof_trace OUT/prof_fetch OUT/prof_write')


def kernel_source_hash() -> str:
    """Hash of the HIP sources; counter figures are only reused while it is unchanged."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_speculative_decoding_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def summarize(args):
    """rocprofv3 CSVs -> profiles/*.md and profiles/pmc_traffic.json."""
    import collections
    import csv
    import glob

    def find(d, suffix):
        hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
        if not hits:
            raise SystemExit(f"no *{suffix} under {d}")
        return hits[0]

    trace_dir, fetch_dir, write_dir = args.summarize
    stats = list(csv.DictReader(open(find(trace_dir, "kernel_stats.csv"))))
    os.makedirs(PROFILES, exist_ok=True)
    lines = ["# rocprofv3 kernel statistics: one QSPEC round, Llama-3-8B-shaped projections (32 layers) and "
             "vocabulary head, B=16, gamma=4",
             "", "Command (run from /tmp with TMPDIR=/tmp):", "", "```", args.summary_command or "(not recorded)", "```",
             "", "| kernel | calls | avg us | total % |", "|---|---:|---:|---:|"]
    for r in stats[:16]:
        name = r["Name"].split("(")[0]
        lines.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # per kernel family (template instantiations together): the figure bench.py's roofline uses
    fam = collections.defaultdict(lambda: [0, 0.0])
    for r in stats:
        base = r["Name"].split("(")[0].split("<")[0].replace("void ", "")
        if base.startswith("qspec::"):
            fam[base][0] += int(r["Calls"])
            fam[base][1] += float(r["TotalDurationNs"])
    lines += ["", "Per kernel family (all template instantiations):", "",
              "| kernel | calls | avg us |", "|---|---:|---:|"]
    for k, (c, t) in sorted(fam.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{k}` | {c} | {t / c / 1e3:.2f} |")
    lines += ["", "Attention over one layer of the cache, outside the timed round (B=16, 32 query heads, 8 KV "
              "heads, d 128, T=4096; k_attn_partial<1> serves the draft step Q=1, <2> the verify pass Q=5):", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        if "k_attn" in r["Name"]:
            lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "FP8 parent, outside the timed round (Qwen2.5-7B qkv, o, gate+up, down, lm_head at M=5; "
              "the split-K reduce it shares with W4A16 is in the table above):", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        if "w8a8" in r["Name"] or "fp8" in r["Name"]:
            lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    open(os.path.join(PROFILES, "kernel_trace_llama3_8b_round_with_head_B16_g4.md"), "w").write("\n".join(lines) + "\n")

    def per_dispatch(d):
        rows = list(csv.DictReader(open(find(d, "counter_collection.csv"))))
        agg = collections.defaultdict(list)
        calib = None
        for r in rows:
            key = r["Kernel_Name"].split("(")[0]
            agg[(key, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
            if "copyBuffer" in r["Kernel_Name"]:
                # the calibration copy is by far the largest copy of the run
                calib = max(calib or 0.0, float(r["Counter_Value"]))
        return agg, calib

    fetch, fcal = per_dispatch(fetch_dir)
    write, wcal = per_dispatch(write_dir)
    known_kib = COPY_MIB * 1024.0
    ffac = known_kib / fcal if fcal else None
    wfac = known_kib / wcal if wcal else None
    out = {"src_hash": kernel_source_hash(), "copy_mib": COPY_MIB, "fetch_factor": ffac, "write_factor": wfac,
           "kernels": {}}
    md = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE; separate runs)", "",
          f"Copy calibration: a {COPY_MIB} MiB device-to-device copy reads {fcal} KiB on FETCH_SIZE and writes "
          f"{wcal} KiB on WRITE_SIZE, so FETCH_SIZE is scaled by {ffac:.4f} and WRITE_SIZE by {wfac:.4f}.", "",
          "Command:", "", "```", args.summary_command or "(not recorded)", "```", "",
          "| kernel | grid | dispatches | fetch MB (scaled) | write MB (scaled) |", "|---|---:|---:|---:|---:|"]
    for (k, grid), v in sorted(fetch.items(), key=lambda kv: -sum(kv[1])):
        if not k.startswith("void qspec::") and not k.startswith("qspec::"):
            continue
        f = sum(v) / len(v) * 1024 * ffac
        w = write.get((k, grid))
        wb = (sum(w) / len(w) * 1024 * wfac) if w else 0.0
        md.append(f"| `{k}` | {grid} | {len(v)} | {f / 1e6:.3f} | {wb / 1e6:.3f} |")
        ent = out["kernels"].setdefault(k, {"fetch_bytes": 0.0, "write_bytes": 0.0, "dispatches": 0})
        ent["fetch_bytes"] += f * len(v)
        ent["write_bytes"] += wb * len(v)
        ent["dispatches"] += len(v)
    for k, e in out["kernels"].items():
        e["bytes_per_dispatch"] = (e["fetch_bytes"] + e["write_bytes"]) / e["dispatches"]
    open(os.path.join(PROFILES, "pmc_traffic_llama3_8b_round_with_head.md"), "w").write("\n".join(md) + "\n")
    json.dump(out, open(TRAFFIC_JSON, "w"), indent=1)
    print(f"wrote profiles/ (src_hash {out['src_hash']})")


def traffic_for(kernel_prefix: str):
    """Counter-measured HBM bytes per dispatch of a kernel, if taken on the current sources."""
    try:
        d = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    if d.get("src_hash") != kernel_source_hash():
        return None
    hits = [e for k, e in d["kernels"].items() if kernel_prefix in k]
    if not hits:
        return None
    disp = sum(e["dispatches"] for e in hits)
    return (sum(e["fetch_bytes"] + e["write_bytes"] for e in hits)) / disp


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--gamma", type=int, default=4)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this size (for counter scaling)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output and exit (no GPU needed)")
    ap.add_argument("--shape-table", metavar="OUT_MD",
                    help="time every GEMM shape of the workloads (W4A4 and W4A16, graph-replayed, weight copies "
                         "rotated beyond the last-level cache), write a markdown table to OUT_MD and exit")
    ap.add_argument("--probe", metavar="LAYER:K:N:M",
                    help="run one GEMM shape (LAYER w4a4 or w4a16) --probe-reps times on fresh weight copies "
                         "and exit: a short program for rocprofv3 counter passes; attention:Q runs one "
                         "layer's attention (B = 16, 4096 positions) for Q query tokens instead")
    ap.add_argument("--probe-reps", type=int, default=4)
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="OUT_MD LABEL=DIR [LABEL=DIR ...]: summarize rocprofv3 --pmc runs of --probe (one "
                         "directory per probe and counter pass) into a markdown table and exit")
    ap.add_argument("--summary-command", default=PROFILE_COMMAND,
                    help="the command that produced the profiles (recorded in the summaries)")
    return ap.parse_args()


class Round:
    """Device buffers and per-phase launch closures of one QSPEC round."""

    def __init__(self, args, dev):
        import torch

        import quantized_speculative_decoding_amd as q
        import synthetic_inputs as si

        self.q, self.torch = q, torch
        B, g, L = args.batch, args.gamma, args.layers
        self.B, self.gamma, self.L = B, g, L
        self.projs = list(si.LLAMA3_8B_PROJ.items())
        self.weights = [[si.weights_device(K, N, seed=l * 8 + i, device=dev) for i, (_, (K, N)) in
                         enumerate(self.projs)] for l in range(L)]
        self.x_draft = [si.activations_device(B, K, seed=10 + i, device=dev) for i, (_, (K, N)) in enumerate(self.projs)]
        self.x_verify = [si.activations_device(B * (g + 1), K, seed=20 + i, device=dev)
                         for i, (_, (K, N)) in enumerate(self.projs)]
        # activation codes / scales and outputs per (layer, projection): distinct buffers
        self.codes = [[torch.empty((B, K // 2), dtype=torch.uint8, device=dev) for _, (K, N) in self.projs]
                      for _ in range(L)]
        self.ascales = [[torch.empty((B, K // GROUP), dtype=torch.float32, device=dev) for _, (K, N) in self.projs]
                        for _ in range(L)]
        self.y_draft = [torch.empty((B, N), dtype=torch.bfloat16, device=dev) for _, (K, N) in self.projs]
        self.y_verify = [torch.empty((B * (g + 1), N), dtype=torch.bfloat16, device=dev) for _, (K, N) in self.projs]
        self.ws_verify = [q.gemm_w4a16_workspace(B * (g + 1), K, N, dev) for _, (K, N) in self.projs]
        self.ws_plain = [q.gemm_w4a16_workspace(B, K, N, dev) for _, (K, N) in self.projs]
        # the vocabulary projection, shared by the draft (W4A4, fp32 logits per step) and the
        # verifier (W4A16, fp32 logits of the gamma + 1 positions).  Draft step j reads hidden rows
        # h_j [B][H]; the verifier reads the same rows at positions j < gamma (row b (gamma + 1) + j)
        # and one more row at position gamma, so target and draft logits differ only by the W4A4 vs
        # W4A16 arithmetic on the shared weights.
        Kh, V = si.LLAMA3_8B_HEAD
        self.V = V
        self.w_head = si.weights_device(Kh, V, seed=7777, device=dev)
        hid = si.activations_device(B * (g + 1), Kh, seed=30, device=dev).view(B, g + 1, Kh)
        self.x_head_verify = hid.reshape(B * (g + 1), Kh).contiguous()
        self.x_head_draft = [hid[:, j, :].contiguous() for j in range(g)]
        self.head_codes = torch.empty((B, Kh // 2), dtype=torch.uint8, device=dev)
        self.head_scales = torch.empty((B, Kh // GROUP), dtype=torch.float32, device=dev)
        self.q_step = torch.empty((B, V), dtype=torch.float32, device=dev)          # one step's draft logits
        self.draft_logits = torch.empty((B, g, V), dtype=torch.float32, device=dev)
        self.target_logits = torch.empty((B, g + 1, V), dtype=torch.float32, device=dev)
        self.ws_head_verify = q.gemm_w4a16_workspace(B * (g + 1), Kh, V, dev)
        self.ws_head_plain = q.gemm_w4a16_workspace(B, Kh, V, dev)
        self.draft_tokens = torch.zeros((B, g), dtype=torch.int32, device=dev)
        self.head_u = si.uniforms_device((g, B), seed=200, device=dev)               # draft-side draws
        self.u_accept = si.uniforms_device((B, g), seed=201, device=dev)
        self.u_resample = si.uniforms_device((B,), seed=202, device=dev)
        self.ws_head = torch.empty((q.qspec_draft_sample_workspace_bytes(q.QSPEC_SAMPLE, B, V),),
                                   dtype=torch.uint8, device=dev)
        self.accept = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.out_tokens = torch.zeros((B, g + 1), dtype=torch.int32, device=dev)
        self.ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_SAMPLE, B, g, V),), dtype=torch.uint8,
                              device=dev)
        # KV cache and the verifier's staging rows
        self.cache = torch.zeros((L, B, 2, KV_HEADS, CONTEXT, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.stage = torch.randn((L, B, 2, KV_HEADS, g + 1, HEAD_DIM), device=dev).to(torch.bfloat16)
        self.start = torch.from_numpy(si.start_positions(B, CONTEXT, g, seed=0)).to(dev)

    # ---- phases (draft step j: quantize, W4A4 layers and head, draft-side sampling head)
    def quant(self, j):
        for l in range(self.L):
            for i in range(len(self.projs)):
                self.q.qspec_quantize_act(self.x_draft[i], self.codes[l][i], self.ascales[l][i])
        self.q.qspec_quantize_act(self.x_head_draft[j], self.head_codes, self.head_scales)

    def draft_gemm(self, j):
        for l in range(self.L):
            for i in range(len(self.projs)):
                wc, wm = self.weights[l][i]
                self.q.qspec_gemm_w4a4(self.codes[l][i], self.ascales[l][i], wc, wm, self.y_draft[i])
        self.q.qspec_gemm_w4a4(self.head_codes, self.head_scales, *self.w_head, self.q_step)

    def draft_head(self, j):
        self.q.qspec_draft_sample(self.q.QSPEC_SAMPLE, self.q_step, self.draft_tokens[:, j], self.head_u[j],
                                  self.ws_head)
        self.draft_logits[:, j, :].copy_(self.q_step)        # q_j for the verification

    def verify_gemm(self):
        for l in range(self.L):
            for i in range(len(self.projs)):
                wc, wm = self.weights[l][i]
                self.q.qspec_gemm_w4a16(self.x_verify[i], wc, wm, self.y_verify[i], self.ws_verify[i])
        self.q.qspec_gemm_w4a16(self.x_head_verify, *self.w_head, self.target_logits.view(-1, self.V),
                                self.ws_head_verify)

    def plain_gemm(self):
        """One plain W4A16 decoding step (M = B) over the same layers and the head: T_target."""
        for l in range(self.L):
            for i in range(len(self.projs)):
                wc, wm = self.weights[l][i]
                self.q.qspec_gemm_w4a16(self.x_draft[i], wc, wm, self.y_draft[i], self.ws_plain[i])
        self.q.qspec_gemm_w4a16(self.x_head_draft[0], *self.w_head, self.q_step, self.ws_head_plain)

    def accept_phase(self):
        self.q.qspec_verify_accept(self.q.QSPEC_SAMPLE, self.target_logits, self.draft_logits, self.draft_tokens,
                                   self.u_accept, self.u_resample, self.accept, self.out_tokens, self.ws)

    def commit(self):
        self.q.qspec_kv_overwrite(self.cache, self.stage, self.start, self.accept)

    # ---- algorithmic work per phase
    def draft_gemm_bytes(self):
        """One draft step's W4A4 launches: the layers' projections and the head (fp32 logits)."""
        Kh, V = self.w_head_shape()
        return (self.L * sum(w4a4_alg_bytes(self.B, K, N) for _, (K, N) in self.projs)
                + w4a4_alg_bytes(self.B, Kh, V) + 2 * self.B * V)

    def verify_gemm_bytes(self):
        Kh, V = self.w_head_shape()
        M = self.B * (self.gamma + 1)
        return (self.L * sum(w4a16_alg_bytes(M, K, N) for _, (K, N) in self.projs)
                + w4a16_alg_bytes(M, Kh, V) + 2 * M * V)

    def w_head_shape(self):
        import synthetic_inputs as si

        return si.LLAMA3_8B_HEAD

    def launches_per_gemm_phase(self):
        return self.L * len(self.projs) + 1


def capture(fn, torch):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    return g


def gpu_leg(args):
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = Round(args, dev)
    torch.cuda.synchronize()

    def eager_round():
        for j in range(R.gamma):
            R.quant(j); R.draft_gemm(j); R.draft_head(j)
        R.verify_gemm(); R.accept_phase(); R.commit()

    # eager reference outputs, then the captured phases
    eager_round()
    torch.cuda.synchronize()
    ref = (R.y_draft[2].clone(), R.y_verify[3].clone(), R.draft_tokens.clone(), R.accept.clone(),
           R.out_tokens.clone(), R.target_logits[:, :, :64].clone())
    g_quant = [capture(lambda j=j: R.quant(j), torch) for j in range(R.gamma)]
    g_draft = [capture(lambda j=j: R.draft_gemm(j), torch) for j in range(R.gamma)]
    g_head = [capture(lambda j=j: R.draft_head(j), torch) for j in range(R.gamma)]
    g_verify = capture(R.verify_gemm, torch)
    g_accept = capture(R.accept_phase, torch)
    g_commit = capture(R.commit, torch)

    phases = ["quantize_act", "gemm_w4a4", "draft_head", "gemm_w4a16", "verify_accept", "kv_overwrite"]
    n_ev = R.gamma * 3 + 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]

    def step(ev):
        k = 0
        if ev: ev[k].record(); k += 1
        for j in range(R.gamma):
            g_quant[j].replay()
            if ev: ev[k].record(); k += 1
            g_draft[j].replay()
            if ev: ev[k].record(); k += 1
            g_head[j].replay()
            if ev: ev[k].record(); k += 1
        g_verify.replay()
        if ev: ev[k].record(); k += 1
        g_accept.replay()
        if ev: ev[k].record(); k += 1
        g_commit.replay()
        if ev: ev[k].record(); k += 1

    # one untimed round of replays (the captures above ran each phase once, out of round order),
    # then the warm-up rounds
    for i in range(1 + args.warmup):
        step(None)
    torch.cuda.synchronize()
    # replays reproduce the eager outputs (every round recomputes the same inputs)
    same = (torch.equal(R.y_draft[2], ref[0]) and torch.equal(R.y_verify[3], ref[1])
            and torch.equal(R.draft_tokens, ref[2]) and torch.equal(R.accept, ref[3])
            and torch.equal(R.out_tokens, ref[4]) and torch.equal(R.target_logits[:, :, :64], ref[5]))
    if not same:
        raise SystemExit("graph replay differs from the eager run")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-phase times from the events (ms), and each round's own time
    ph = {p: 0.0 for p in phases}
    per_round = []
    for ev in evs:
        k = 0
        for _ in range(R.gamma):
            ph["quantize_act"] += ev[k].elapsed_time(ev[k + 1]); k += 1
            ph["gemm_w4a4"] += ev[k].elapsed_time(ev[k + 1]); k += 1
            ph["draft_head"] += ev[k].elapsed_time(ev[k + 1]); k += 1
        ph["gemm_w4a16"] += ev[k].elapsed_time(ev[k + 1]); k += 1
        ph["verify_accept"] += ev[k].elapsed_time(ev[k + 1]); k += 1
        ph["kv_overwrite"] += ev[k].elapsed_time(ev[k + 1]); k += 1
        per_round.append(ev[0].elapsed_time(ev[n_ev - 1]))
    ph = {p: v / args.steps for p, v in ph.items()}
    event_ms = sum(ph.values())

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    R.per_round_ms = per_round
    R.model = round_model(R, ph, torch)
    R.verify_tps = verify_tokens_per_s(R, torch)
    R.speckv_us = speckv_controller_us(R, torch)
    R.attention = attention_us(R, torch)
    R.fp8 = fp8_parent_us(R, torch)
    R.verify_commit = verify_commit_us(R, torch)
    return R, ph, wall, event_ms


def round_model(R, ph, torch):
    """Outside the timed round: the speedup model S = E[L] T_target / (T_draft + T_verify +
    T_overhead) with every time measured here (T_target = one plain W4A16 decoding step at M = B
    over the same layers and the head, graph-replayed), E[L] as the round's accept counts give it
    (mean A + 1 over the B sequences) and as the round's logits imply it (the per-position
    acceptance probabilities, free of the sampling noise of B = 16 draws), and S at a few
    acceptance rates a through E[L] = (1 - a^(gamma+1)) / (1 - a)."""
    graph = capture(R.plain_gemm, torch)
    graph.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    t_target = a.elapsed_time(b) / 5
    acc = R.accept.cpu().double()
    e_l = float(acc.mean()) + 1.0
    # the acceptance probability of each drafted position, sum_v min(p, q) with p and q the
    # softmaxes of that position's target and draft logits (the rule's expected acceptance for a
    # token drawn from q), and the expected committed length it implies for each sequence:
    # E[L_b] = 1 + sum_k prod_{j<k} alpha_{b,j}.  Computed once in float64 on the round's logits.
    p = torch.softmax(R.target_logits[:, :R.gamma, :].double(), dim=-1)
    q = torch.softmax(R.draft_logits.double(), dim=-1)
    alpha = torch.minimum(p, q).sum(-1)                                     # [B][gamma]
    e_l_exp = float((1.0 + torch.cumprod(alpha, dim=1).sum(1)).mean())
    del p, q
    t_draft = ph["quantize_act"] + ph["gemm_w4a4"] + ph["draft_head"]
    t_verify = ph["gemm_w4a16"]
    t_over = ph["verify_accept"] + ph["kv_overwrite"]
    t_round = t_draft + t_verify + t_over
    g = R.gamma
    at = {al: (1 - al ** (g + 1)) / (1 - al) * t_target / t_round for al in (0.6, 0.8, 0.9)}
    return {"T_target_ms": round(t_target, 4), "T_draft_ms": round(t_draft, 4), "T_verify_ms": round(t_verify, 4),
            "T_overhead_ms": round(t_over, 4), "accept_counts": [int(v) for v in R.accept.cpu().tolist()],
            "E_L_measured": round(e_l, 4), "S_measured_E_L": round(e_l * t_target / t_round, 3),
            "alpha_per_position_mean": round(float(alpha.mean()), 4),
            "E_L_expected_from_logits": round(e_l_exp, 4), "S_expected_E_L": round(e_l_exp * t_target / t_round, 3),
            "S_at_alpha": {str(k): round(v, 3) for k, v in at.items()}}


def verify_tokens_per_s(R, torch, batches=(1, 4, 16)):
    """Outside the timed round: verify tokens/s at this gamma as the verify GEMMs alone bound it,
    B (gamma + 1) / (sum of the four projections' W4A16 times at M = B (gamma + 1)), per layer and
    for the whole stack, with the HBM roofline bound from the algorithmic bytes at 8 TB/s.  One
    graph over all layers' projections (each layer its own weights, beyond the last-level cache),
    replayed 5 x 3 times; median."""
    import synthetic_inputs as si

    q, dev, g = R.q, R.accept.device, R.gamma
    out = {}
    for B in batches:
        M = B * (g + 1)
        xs = [si.activations_device(M, K, seed=40 + i, device=dev) for i, (_, (K, N)) in enumerate(R.projs)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, (K, N) in R.projs]
        wss = [q.gemm_w4a16_workspace(M, K, N, dev) for _, (K, N) in R.projs]

        def fn():
            for l in range(R.L):
                for i in range(len(R.projs)):
                    wc, wm = R.weights[l][i]
                    q.qspec_gemm_w4a16(xs[i], wc, wm, ys[i], wss[i])

        graph = capture(fn, torch)
        graph.replay()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(3):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 3)
        t_layer_us = sorted(ts)[2] * 1e3 / R.L
        roof_us = sum(w4a16_alg_bytes(M, K, N) for _, (K, N) in R.projs) / (HBM_PEAK_GBS * 1e9) * 1e6
        out[f"B{B}"] = {"M": M, "layer_us": round(t_layer_us, 2), "tokens_per_s_per_layer": round(M / (t_layer_us * 1e-6), 1),
                        "tokens_per_s_32_layers": round(M / (t_layer_us * 1e-6) / 32, 1),
                        "roofline_tokens_per_s_per_layer": round(M / (roof_us * 1e-6), 1),
                        "fraction_of_roofline": round(roof_us / t_layer_us, 4)}
        del graph, xs, ys, wss
    return out


def speckv_controller_us(R, torch):
    """Outside the timed round: the adaptive-gamma controller (draft confidence and entropy over
    one draft row per sequence, then its MLP) on the round's draft logits (the W4A4 head's rows of
    each draft step), graph-replayed; random controller weights (the trained ones are not
    published).  Returns microseconds per draft step for: the controller alone
    (qspec_speckv_gamma), the draft-side sampling head alone (qspec_draft_sample), and both on
    the same rows with the head's softmax statistics shared (qspec_draft_sample_speckv)."""
    q, B, V = R.q, R.B, R.V
    dev = R.accept.device
    rows = [R.draft_logits[:, j, :] for j in range(R.gamma)]            # one row set per draft step
    crows = [r.contiguous() for r in rows]
    gen = torch.Generator(device=dev).manual_seed(900)
    w1, b1 = torch.randn((64, 3), device=dev, generator=gen), torch.randn((64,), device=dev, generator=gen)
    w2, b2 = torch.randn((9, 64), device=dev, generator=gen), torch.randn((9,), device=dev, generator=gen)
    g = torch.empty((B,), dtype=torch.int32, device=dev)
    toks = torch.empty((B, R.gamma), dtype=torch.int32, device=dev)
    ws = torch.empty((q.qspec_speckv_workspace_bytes(B, V),), dtype=torch.uint8, device=dev)
    ws_h = torch.empty((q.qspec_draft_sample_workspace_bytes(q.QSPEC_SAMPLE, B, V),), dtype=torch.uint8, device=dev)
    ws_b = torch.empty((q.qspec_draft_sample_speckv_workspace_bytes(q.QSPEC_SAMPLE, B, V),), dtype=torch.uint8,
                       device=dev)

    def per_step(fn):
        graph = capture(fn, torch)
        graph.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(5):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (5 * len(rows))

    ctrl = per_step(lambda: [q.qspec_speckv_gamma(r, 0.0, w1, b1, w2, b2, g, None, ws) for r in crows])
    head = per_step(lambda: [q.qspec_draft_sample(q.QSPEC_SAMPLE, r, toks[:, j], R.head_u[j], ws_h)
                             for j, r in enumerate(rows)])
    both = per_step(lambda: [q.qspec_draft_sample_speckv(q.QSPEC_SAMPLE, r, toks[:, j], R.head_u[j], 0.0, w1, b1, w2,
                                                         b2, g, None, ws_b) for j, r in enumerate(rows)])
    return {"controller_alone": round(ctrl, 1), "draft_head_alone": round(head, 1),
            "draft_head_and_controller_shared_stats": round(both, 1)}


def attention_us(R, torch):
    """Outside the timed round: one layer's attention over a full 4096-position cache (B
    sequences, 32 query heads, 8 KV heads, d 128) for a draft step (Q = 1) and a verify pass
    (Q = gamma + 1), graph-replayed; the bfloat16 cache (qspec_attention) and the quantized FP8
    cache (qspec_attention_fp8: E4M3 codes, one scale per row), each rotated over enough copies to
    exceed the 256 MB last-level cache.  Returns {(kind, Q): microseconds per call}."""
    import math

    import synthetic_inputs as si

    q, B, dev = R.q, R.B, R.accept.device
    Hq = 32
    res = {}
    for Q in (1, R.gamma + 1):
        qd, cache = si.attention_inputs_device(B, Q, Hq, KV_HEADS, CONTEXT, HEAD_DIM, 1, dev)
        pos = torch.full((B,), CONTEXT - Q, dtype=torch.int32, device=dev)
        out = torch.empty((B, Q, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, KV_HEADS, CONTEXT),), dtype=torch.uint8,
                         device=dev)
        codes = torch.empty((B, 2, KV_HEADS, CONTEXT, HEAD_DIM), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, 2, KV_HEADS, CONTEXT), dtype=torch.float32, device=dev)
        q.qspec_quantize_act_fp8(cache.view(-1, HEAD_DIM), codes.view(-1, HEAD_DIM), scales.view(-1))
        bf_copies = [cache, cache.clone()]                                  # 2 x 268 MB
        f8_copies = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(3)]   # 4 x 136 MB
        for kind, fn, n in (
                ("bf16", lambda: [q.qspec_attention(qd, bf_copies[i % 2], pos, 1.0 / math.sqrt(HEAD_DIM), out, ws)
                                  for i in range(8)], 8),
                ("fp8", lambda: [q.qspec_attention_fp8(qd, *f8_copies[i % 4], pos, 1.0 / math.sqrt(HEAD_DIM), out, ws)
                                 for i in range(8)], 8)):
            graph = capture(fn, torch)
            graph.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(3):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            res[(kind, Q)] = a.elapsed_time(b) * 1e3 / (3 * n)
            del graph
        del qd, cache, codes, scales, bf_copies, f8_copies
        torch.cuda.empty_cache()
    return res


def verify_commit_us(R, torch, B=32, gamma=4, sets=4):
    """Outside the timed round: the verify-and-commit stage at B = 32, gamma = 4 over a
    128256-word vocabulary (target logits N(0, 3), draft = target + N(0, 0.5)), in greedy mode
    (argmax-match drafts) and sampling mode (drafts sampled from softmax(draft)): qspec_verify_accept
    and then qspec_kv_overwrite of the accepted rows into a 32-layer x 32-sequence x 8-head x 4096 x
    128 bf16 cache, graph-replayed over `sets` logit sets (beyond the last-level cache).  Returns
    {mode: (accept us, kv us, mean committed rows per sequence)}."""
    import synthetic_inputs as si

    q, dev, V = R.q, R.accept.device, VOCAB
    cache = torch.empty((R.L, B, 2, KV_HEADS, CONTEXT, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    stage = torch.randn((R.L, B, 2, KV_HEADS, gamma + 1, HEAD_DIM), device=dev).to(torch.bfloat16)
    start = torch.from_numpy(si.start_positions(B, CONTEXT, gamma, seed=1)).to(dev)
    acc = torch.zeros((B,), dtype=torch.int32, device=dev)
    out = torch.zeros((B, gamma + 1), dtype=torch.int32, device=dev)
    res = {}
    for mode, name in ((q.QSPEC_GREEDY, "greedy"), (q.QSPEC_SAMPLE, "sample")):
        inputs = []
        for s_ in range(sets):
            t, d = si.logits_device(B, gamma, V, seed=50 + s_, device=dev)
            toks = (d.argmax(dim=-1).to(torch.int32) if mode == q.QSPEC_GREEDY
                    else si.draft_tokens_sampled_device(d, seed=50 + s_))
            inputs.append((t, d if mode == q.QSPEC_SAMPLE else None, toks,
                           si.uniforms_device((B, gamma), seed=60 + s_, device=dev),
                           si.uniforms_device((B,), seed=70 + s_, device=dev)))
        ws = torch.empty((q.qspec_verify_workspace_bytes(mode, B, gamma, V),), dtype=torch.uint8, device=dev)

        def accept(i):
            t, d, toks, u, v = inputs[i]
            q.qspec_verify_accept(mode, t, d, toks, u if d is not None else None, v if d is not None else None,
                                  acc, out, ws)

        rows = 0.0
        for i in range(sets):
            accept(i)
            rows += float((acc.double() + 1).mean())
        times = []
        for fn in (lambda: [accept(i) for i in range(sets)],
                   lambda: [q.qspec_kv_overwrite(cache, stage, start, acc) for _ in range(sets)]):
            graph = capture(fn, torch)
            graph.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(5):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / (5 * sets))
        res[name] = (times[0], times[1], rows / sets)
        del inputs, ws
    del cache, stage
    torch.cuda.empty_cache()
    return res


QWEN25_7B = {"qkv": (3584, 4608), "o": (3584, 3584), "gate_up": (3584, 2 * 18944), "down": (18944, 3584),
             "lm_head": (3584, 152064)}


def fp8_parent_us(R, torch, gamma=4):
    """Outside the timed round: the FP8 parent (per-token E4M3 activations, E4M3 weights with column
    scales) verifying gamma = 4 drafts of one sequence (M = 5) on Qwen2.5-7B's shapes: per projection,
    qspec_quantize_act_fp8 + qspec_gemm_w8a8, graph-replayed over 4 weight copies of the layer (beyond
    the last-level cache); returns {projection: (layer us, quantize us, weight+scale bytes)}."""
    import synthetic_inputs as si

    q, dev, M = R.q, R.accept.device, gamma + 1
    res = {}
    for name, (K, N) in QWEN25_7B.items():
        copies = 1 if name == "lm_head" else 4
        W = [si.fp8_weights_device(K, N, seed=c, device=dev) for c in range(copies)]
        x = si.activations_device(M, K, seed=1, device=dev)
        codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((max(1, q.qspec_gemm_w8a8_workspace_bytes(M, K, N)),), dtype=torch.uint8, device=dev)
        times = []
        for fn in (lambda: [q.qspec_gemm_w8a8(codes, sa, *W[c], y, ws) for c in range(copies)],
                   lambda: [q.qspec_quantize_act_fp8(x, codes, sa) for c in range(copies)]):
            graph = capture(lambda: [fn() for _ in range(8 // copies if copies < 8 else 1)], torch)
            graph.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(4):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / (4 * 8))
        res[name] = (times[0], times[1], K * N + 4 * N)
        del W
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_leg(args, repeats: int = 5):
    """The oracle, as written, on a bounded sample of one round, scaled to a whole round: timed on
    one host thread, and with the sample's GEMM columns split over the host's threads (the oracle's
    calls release the GIL, so a thread pool runs them in parallel on disjoint column tiles); the
    median of `repeats` passes of each."""
    import concurrent.futures

    import numpy as np

    import oracle
    import synthetic_inputs as si

    B, g, L = args.batch, args.gamma, args.layers
    frac, frac_head = 64, 256      # projections on 1/64 of their columns, the head on 1/256
    Kh, V = si.LLAMA3_8B_HEAD
    threads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()))
    def cols(N, fr):                # whole 16-column tiles, about N / fr columns
        return 16 * max(1, N // 16 // fr)

    items = []        # (layers, draft steps, column scale, weights, draft rows, verify rows)
    for i, (name, (K, N)) in enumerate(si.LLAMA3_8B_PROJ.items()):
        n = cols(N, frac)
        items.append((L, g, N / n, si.weights(K, n, seed=i), si.activations(B, K, seed=10 + i),
                      si.activations(B * (g + 1), K, seed=20 + i)))
    n = cols(V, frac_head)
    items.append((1, g, V / n, si.weights(Kh, n, seed=99), si.activations(B, Kh, seed=30),
                  si.activations(B * (g + 1), Kh, seed=31)))
    t_logits, d_logits = si.logits(B, g, V, seed=0)
    hu = si.uniforms((g, B), 2)
    u, v = si.uniforms((B, g), 0), si.uniforms((B,), 1)
    kv_cache = si.kv_canary(1, B, KV_HEADS, 64, HEAD_DIM).reshape(1, B, 2, KV_HEADS, 64, HEAD_DIM)
    kv_stage = si.kv_staging(1, B, KV_HEADS, g, HEAD_DIM, seed=0)
    kv_start = si.start_positions(B, 64, g, seed=0)

    def gemms(w, c, s, xv, pool):
        """W4A4 at M = B and W4A16 at M = B (gamma + 1) on the slice's column tiles; with a pool, the
        tiles are split into one contiguous range per thread."""
        T = w["codes"].shape[0]
        if pool is None:
            parts = [np.arange(T)]
        else:
            parts = [p for p in np.array_split(np.arange(T), threads) if len(p)]
        subs = [si.slice_tiles(w, p) for p in parts]
        f4 = lambda sub: oracle.gemm_w4a4(c, s, sub["codes"], sub["meta"], want_dots=False)
        f16 = lambda sub: oracle.gemm_w4a16(xv, sub["codes"], sub["meta"])
        t0 = time.perf_counter()
        if pool is None:
            f4(subs[0])
        else:
            list(pool.map(f4, subs))
        t1 = time.perf_counter()
        if pool is None:
            f16(subs[0])
        else:
            list(pool.map(f16, subs))
        return t1 - t0, time.perf_counter() - t1

    def one_pass(pool):
        est = 0.0
        for (layers, steps, fr, w, xd, xv) in items:
            t0 = time.perf_counter()
            c, s = oracle.quantize_act(xd)
            tq = time.perf_counter() - t0
            t4, t16 = gemms(w, c, s, xv, pool)
            est += layers * (steps * (tq + fr * t4) + fr * t16)
        t0 = time.perf_counter()
        toks = np.empty((B, g), np.int32)
        for j in range(g):          # the draft-side head: verification with gamma = 0 on step j's rows
            _, o, _ = oracle.verify_sample(d_logits[:, j:j + 1, :], np.zeros((B, 0, V), np.float32),
                                           np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32), hu[j],
                                           with_diag=False)
            toks[:, j] = o[:, 0]
        acc, _, _ = oracle.verify_sample(t_logits, d_logits, toks, u, v, with_diag=False)
        est += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.kv_overwrite(kv_cache.copy(), kv_stage, kv_start, acc)
        est += L * (time.perf_counter() - t0)
        return est

    t_start = time.perf_counter()
    single = sorted(one_pass(None) for _ in range(repeats))[repeats // 2]
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        multi = sorted(one_pass(pool) for _ in range(repeats))[repeats // 2]
    spent = time.perf_counter() - t_start
    tok = B * (g + 1)
    return {
        "value": round(tok / multi, 4),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "single_thread_tokens_per_s": round(tok / single, 5),
        "round_s_single_thread": round(single, 1),
        "round_s_threads": round(multi, 1),
        "sample": (f"one layer of each projection on 1/{frac} of its columns and the vocabulary head on "
                   f"1/{frac_head} (quantize + W4A4 at M={B}, W4A16 at M={B * (g + 1)}), {g} full draft-side "
                   f"heads and the full verify_accept (sampling, B={B}, V={V}), one KV layer; scaled x{L} layers, "
                   f"x{g} draft steps and by the column fractions; median of {repeats} passes on 1 thread and on "
                   f"{threads} threads (GEMM column tiles split over a thread pool); {spent:.1f} s of CPU work "
                   f"in all"),
    }


SHAPE_TABLE_COMMAND = "python3 bench.py --shape-table OUT.md"


def shape_table(args):
    """Per-shape GEMM times: Llama-3-8B projections and the Qwen2.5-7B vocabulary projection at the
    decode / verify batch sizes, and the Llama-70B-shaped FFN at its large batches.  Each (shape, M)
    is one graph of launches over rotating weight copies (at least 600 MB, beyond the 256 MB
    last-level cache), replayed 5 x 5 times; the median per launch is reported with the HBM rate
    of its algorithmic bytes and, for the large batches, its MFMA rate."""
    import torch

    import quantized_speculative_decoding_amd as q
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = [("512 x 512 layer", 512, 512, (1,), (5,))]
    shapes += [(f"Llama-3-8B {n}", K, N, (1, 4, 16), (1, 5, 16, 20, 80)) for n, (K, N) in si.LLAMA3_8B_PROJ.items()]
    shapes += [(f"Qwen2.5-7B {n}", K, N, (1,), (3, 5, 9, 17)) for n, (K, N) in QWEN25_7B.items() if n != "lm_head"]
    shapes.append(("Qwen2.5-7B lm_head (fp32 out)", 3584, 152064, (1, 16), (1, 3, 5, 9, 17, 80)))
    shapes += [(f"Llama-70B FFN {n}", K, N, (256,), (1280,)) for n, (K, N) in si.LLAMA3_70B_FFN.items()]

    def timed(fn, reps):
        graph = capture(fn, torch)
        graph.replay()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(5):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / (5 * reps))
        return sorted(ts)[2]

    # a read-only streaming reference on this machine: torch's sum over 2 GiB of fp32, timed eagerly
    # (a multi-block reduction is kept out of graph capture); median of 5 x 5 calls
    big = torch.ones((1 << 29,), dtype=torch.float32, device=dev)
    torch.sum(big)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            torch.sum(big)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / 5)
    read_tbs = big.numel() * 4 / (sorted(ts)[2] * 1e-6) / 1e12
    del big
    torch.cuda.empty_cache()
    rows = []
    for name, K, N, m4, m16 in shapes:
        wc, wm = si.weights_device(K, N, seed=1, device=dev)
        wbytes = w4_bytes(K, N)
        R = max(2, int(600e6 // wbytes) + 1)
        copies = [(wc, wm)] + [(wc.clone(), wm.clone()) for _ in range(R - 1)]
        out = torch.float32 if "lm_head" in name else torch.bfloat16
        for kind, Ms in (("W4A4", m4), ("W4A16", m16)):
            for M in Ms:
                x = si.activations_device(M, K, seed=3, device=dev)
                y = torch.empty((M, N), dtype=out, device=dev)
                if kind == "W4A4":
                    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
                    sc = torch.empty((M, K // GROUP), dtype=torch.float32, device=dev)
                    q.qspec_quantize_act(x, codes, sc)
                    us = timed(lambda: [q.qspec_gemm_w4a4(codes, sc, c, m, y) for c, m in copies], R)
                    alg = w4a4_alg_bytes(M, K, N) + (2 * M * N if out == torch.float32 else 0)
                    peak_ops = 5.0e15
                else:
                    ws = q.gemm_w4a16_workspace(M, K, N, dev)
                    us = timed(lambda: [q.qspec_gemm_w4a16(x, c, m, y, ws) for c, m in copies], R)
                    alg = w4a16_alg_bytes(M, K, N) + (2 * M * N if out == torch.float32 else 0)
                    peak_ops = 2.5e15
                tbs = alg / (us * 1e-6) / 1e12
                ops = 2.0 * M * K * N / (us * 1e-6)
                rows.append((name, f"{K} -> {N}", kind, M, us, tbs, tbs * 1e3 / HBM_PEAK_GBS, ops / 1e12, ops / peak_ops))
                print(rows[-1], flush=True)
        del copies, wc, wm
        torch.cuda.empty_cache()
    lines = ["# Per-shape GEMM times on one MI355X (graph-replayed, weight copies rotated beyond the LLC)", "",
             "Command (from the repository root):", "", "```", SHAPE_TABLE_COMMAND, "```", "",
             "HBM rate = algorithmic bytes (4-bit codes + per-group fp16 scale and zero, activations in, outputs "
             "out) / time; its fraction is of 8 TB/s.  Op rate = 2 M K N / time, as a fraction of the dense "
             "int8 (W4A4, 5.0 POP/s) or bf16 (W4A16, 2.5 PFLOP/s) MFMA peak.", "",
             f"Read-only reference on the same box: torch.sum over 2 GiB of fp32 streams at {read_tbs:.2f} TB/s "
             f"({read_tbs * 1e3 / HBM_PEAK_GBS:.0%} of 8 TB/s).", "",
             "| shape | K -> N | layer | M | us per launch | HBM TB/s | of 8 TB/s | T(FL)OP/s | of MFMA peak |",
             "|---|---|---|---:|---:|---:|---:|---:|---:|"]
    for name, kn, kind, M, us, tbs, hf, top, mf in rows:
        lines.append(f"| {name} | {kn} | {kind} | {M} | {us:.2f} | {tbs:.2f} | {hf:.0%} | {top:.0f} | {mf:.1%} |")
    open(args.shape_table, "w").write("\n".join(lines) + "\n")
    print("wrote", args.shape_table)


PMC_COMMAND = ("cd /tmp && export TMPDIR=/tmp && for each probe P in the table and each pass C: "
               "timeout -s KILL 120 rocprofv3 --pmc C --output-format csv -d OUT/P_pass -o probe -- "
               "python3 REPO/bench.py --probe P --probe-reps 4 ; then python3 REPO/bench.py --summarize-pmc "
               "OUT.md LABEL=OUT/P_pass ...")
PMC_PASSES = {
    "pass1": "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA "
             "SQ_BUSY_CYCLES SQ_WAVES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
    "pass2": "SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT "
             "SQ_ACTIVE_INST_VMEM SQ_INST_CYCLES_VMEM_RD SQ_CYCLES GRBM_GUI_ACTIVE",
    "pass3": "FETCH_SIZE",
    "pass4": "WRITE_SIZE",
}


def summarize_pmc(args):
    """Per-dispatch averages of the counters of --probe runs (the qspec kernels only; the passes of
    one probe merged), with the derived ratios named in the table."""
    import collections
    import csv
    import glob

    out_md, specs = args.summarize_pmc[0], args.summarize_pmc[1:]
    per = collections.OrderedDict()      # probe -> kernel -> counter -> [values]
    dur = collections.defaultdict(list)  # (probe, kernel) -> dispatch durations (ns)
    for spec in specs:
        label, d = spec.split("=", 1)
        probe_name = label.rsplit("_pass", 1)[0]
        hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no counter_collection.csv under {d}")
        seen = set()
        for r in csv.DictReader(open(hits[0])):
            k = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if "qspec::" not in k:
                continue
            per.setdefault(probe_name, collections.OrderedDict()).setdefault(k, collections.defaultdict(list))[
                r["Counter_Name"]].append(float(r["Counter_Value"]))
            if (k, r["Dispatch_Id"]) not in seen:
                seen.add((k, r["Dispatch_Id"]))
                dur[(probe_name, k)].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    lines = ["# rocprofv3 counters of single probed launches (--probe: one GEMM shape, or one layer's attention), per dispatch", "",
             "Command:", "", "```", PMC_COMMAND, "```", "",
             "Passes (one rocprofv3 run each; a probe's passes are merged per kernel): "
             + "; ".join(f"{k}: {v}" for k, v in PMC_PASSES.items()), "",
             "Calibration: SQ_VALU_MFMA_BUSY_CYCLES equals 16 x SQ_INSTS_MFMA for the bf16 16x16x32 MFMA kernels "
             "(16 cycles of a SIMD's matrix core per instruction); SQ_BUSY_CYCLES sums the 32 shader engines "
             "(8 XCDs x 4), so C = SQ_BUSY_CYCLES / 32 is the dispatch's cycle count (C / duration gives the "
             "clock; GRBM_GUI_ACTIVE / 8 agrees on long dispatches but also counts the profiler's window around "
             "short ones); SQ_WAVE_CYCLES and SQ_WAIT_* count in units of 4 cycles.  "
             "Derived over 1024 SIMDs: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 C); VALU busy = "
             "4 (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (1024 C) (SQ_INSTS_VALU counts MFMA instructions too; a wave64 "
             "VALU instruction occupies a 16-lane SIMD for 4 cycles); co-execution = SQ_VALU_MFMA_COEXEC_CYCLES / "
             "SQ_VALU_MFMA_BUSY_CYCLES; wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS wait share = "
             "SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES.", ""]
    lines += ["| probe | kernel | us | clock GHz | MFMA busy | VALU busy | co-exec | wait share | LDS wait share | "
              "VALU per MFMA | waves |", "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    raw = ["", "Raw counters per dispatch:", "", "| probe | kernel | counter | per dispatch |", "|---|---|---|---:|"]
    for probe_name, kernels in per.items():
        for k, cs in kernels.items():
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            for c in sorted(avg):
                raw.append(f"| {probe_name} | `{k[:60]}` | {c} | {avg[c]:.4g} |")
            ds = dur[(probe_name, k)]
            us = sum(ds) / len(ds) / 1e3 if ds else float("nan")
            C = avg.get("SQ_BUSY_CYCLES", 0) / 32
            f = lambda v: f"{v:.3f}" if v == v else "-"
            nan = float("nan")
            mb = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", nan) / (1024 * C) if C else nan
            vb = 4 * (avg.get("SQ_INSTS_VALU", nan) - avg.get("SQ_INSTS_MFMA", nan)) / (1024 * C) if C else nan
            co = (avg.get("SQ_VALU_MFMA_COEXEC_CYCLES", nan) / avg["SQ_VALU_MFMA_BUSY_CYCLES"]
                  if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") else nan)
            wc = avg.get("SQ_WAVE_CYCLES")
            ws = avg.get("SQ_WAIT_INST_ANY", nan) / wc if wc else nan
            wl = avg.get("SQ_WAIT_INST_LDS", nan) / wc if wc else nan
            vpm = ((avg.get("SQ_INSTS_VALU", nan) - avg["SQ_INSTS_MFMA"]) / avg["SQ_INSTS_MFMA"]
                   if avg.get("SQ_INSTS_MFMA") else nan)
            clock = C / (us * 1e3) if us == us and us > 0 else nan
            lines.append(f"| {probe_name} | `{k[:60]}` | {us:.1f} | {f(clock)} | {f(mb)} | {f(vb)} | {f(co)} | {f(ws)} | "
                         f"{f(wl)} | {f(vpm)} | {avg.get('SQ_WAVES', 0):.0f} |")
    open(out_md, "w").write("\n".join(lines + raw) + "\n")
    print("wrote", out_md)


def probe_attention(args, Q):
    """One layer's attention over the bfloat16 cache (the shape of the benchmark's attention
    figure: B = 16, 32 query heads, 8 KV heads, d 128, a full 4096-position cache) for Q query
    tokens, launched eagerly --probe-reps times over two cache copies; prints and exits."""
    import math

    import torch

    import quantized_speculative_decoding_amd as q
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    B, Hq = 16, 32
    qd, cache = si.attention_inputs_device(B, Q, Hq, KV_HEADS, CONTEXT, HEAD_DIM, 1, dev)
    pos = torch.full((B,), CONTEXT - Q, dtype=torch.int32, device=dev)
    out = torch.empty((B, Q, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((q.qspec_attention_workspace_bytes(B, Q, Hq, KV_HEADS, CONTEXT),), dtype=torch.uint8, device=dev)
    copies = [cache, cache.clone()]
    for i in range(args.probe_reps):
        q.qspec_attention(qd, copies[i % 2], pos, 1.0 / math.sqrt(HEAD_DIM), out, ws)
    torch.cuda.synchronize()
    print(f"probe attention B={B} Q={Q} T={CONTEXT} x{args.probe_reps}", flush=True)


def probe(args):
    """One GEMM shape, launched eagerly --probe-reps times over distinct weight copies (each read
    from HBM), for counter collection; prints the shape and exits.  attention:Q probes the
    attention kernel instead (probe_attention)."""
    import torch

    import quantized_speculative_decoding_amd as q
    import synthetic_inputs as si

    if args.probe.startswith("attention:"):
        probe_attention(args, int(args.probe.split(":")[1]))
        return
    layer, K, N, M = args.probe.split(":")
    K, N, M = int(K), int(N), int(M)
    dev = torch.device("cuda:0")
    W = [si.weights_device(K, N, seed=c, device=dev) for c in range(args.probe_reps)]
    x = si.activations_device(M, K, seed=3, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if layer == "w4a4":
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((M, K // GROUP), dtype=torch.float32, device=dev)
        q.qspec_quantize_act(x, codes, sc)
        for wc, wm in W:
            q.qspec_gemm_w4a4(codes, sc, wc, wm, y)
    elif layer == "w4a16":
        ws = q.gemm_w4a16_workspace(M, K, N, dev)
        for wc, wm in W:
            q.qspec_gemm_w4a16(x, wc, wm, y, ws)
    else:
        raise SystemExit(f"unknown layer {layer!r}")
    torch.cuda.synchronize()
    print(f"probe {layer} K={K} N={N} M={M} x{args.probe_reps}", flush=True)


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.probe:
        probe(args)
        return
    if args.summarize:
        summarize(args)
        return
    if args.shape_table:
        shape_table(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: every box here has one MI355X and this build has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    R, ph, wall, event_ms = gpu_leg(args)
    B, g = args.batch, args.gamma
    ms_per_step = wall * 1e3 / args.steps
    value = B * (g + 1) / (ms_per_step / 1e3)
    rounds = sorted(R.per_round_ms)
    pct = lambda p: rounds[min(len(rounds) - 1, int(round(p * (len(rounds) - 1))))]
    nl = R.launches_per_gemm_phase()
    draft_ms = ph["gemm_w4a4"]                     # gamma draft passes per round
    verify_ms = ph["gemm_w4a16"]
    # The dominant GEMM phase: its graph holds only that GEMM's launches, so the phase's event time
    # over the timed region divided by its launch count is the kernel's average launch duration
    # (the rocprofv3 kernel statistics of the same command give the same figure).
    dom = "gemm_w4a4" if draft_ms >= verify_ms else "gemm_w4a16"
    if dom == "gemm_w4a4":
        bytes_per_launch = R.draft_gemm_bytes() / nl
        n_launch = g * nl
        avg_launch_ms = draft_ms / n_launch
        kernel = "k_w4a4_decode"
    else:
        bytes_per_launch = R.verify_gemm_bytes() / nl
        n_launch = nl
        avg_launch_ms = verify_ms / n_launch
        kernel = "k_w4a16_mid"           # plus k_w4a16_splitk_reduce on split-K shapes
    achieved = bytes_per_launch / (avg_launch_ms / 1e3) / 1e9
    tb = traffic_for(kernel)
    traffic = None if tb is None else round(tb)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+bf16",
        "data": "synthetic",
        "config": {"workload": f"llama3-8b-projections-{args.layers}L-and-head-qspec-round-B{B}-gamma{g}",
                   "batch": B, "gamma": g, "layers": args.layers, "draft_M": B, "verify_M": B * (g + 1),
                   "vocab": R.V, "head": "4096x128256 shared INT4: W4A4 draft logits per step, W4A16 target logits",
                   "kv_cache": f"{args.layers}x{B}x2x{KV_HEADS}x{CONTEXT}x{HEAD_DIM} bf16",
                   "verify_mode": "sample"},
        "round_ms": {"median": round(pct(0.5), 4), "p10": round(pct(0.1), 4), "p90": round(pct(0.9), 4)},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(bytes_per_launch), "us_per_launch": round(avg_launch_ms * 1e3, 3),
                     "launches_per_round": n_launch},
        "phases_ms_per_round": {k: round(v, 4) for k, v in ph.items()},
        "event_ms_per_round": round(event_ms, 4),
        "gemm_hbm_tbs": {"gemm_w4a4_M%d" % B: round(R.draft_gemm_bytes() * g / (draft_ms / 1e3) / 1e12, 3),
                         "gemm_w4a16_M%d" % (B * (g + 1)): round(R.verify_gemm_bytes() / (verify_ms / 1e3) / 1e12, 3)},
        # outside the timed round: the round-time and speedup model from these measurements
        # (projections and head only: attention and norms are not in T_target)
        "round_model": R.model,
        # outside the timed round: the adaptive-gamma controller on one draft row per sequence
        "speckv_us_per_draft_step": R.speckv_us,
        # outside the timed round: one layer's attention over the full cache; every key and value
        # (B x 8 heads x 4096 positions x 2 rows of 256 bytes in bfloat16, of 128 code bytes and a
        # 4-byte scale in the quantized FP8 cache) is read once per call
        "attention": {"workload": f"B{B}-Hq32-Hkv{KV_HEADS}-d{HEAD_DIM}-T{CONTEXT}-one-layer",
                      **{f"us_Q{Qa}": round(u, 1) for (k, Qa), u in R.attention.items() if k == "bf16"},
                      **{f"hbm_frac_Q{Qa}": round(B * KV_HEADS * CONTEXT * 2 * HEAD_DIM * 2 / (u * 1e-6) / 1e9
                                                  / HBM_PEAK_GBS, 4) for (k, Qa), u in R.attention.items() if k == "bf16"},
                      "fp8_cache": {
                          **{f"us_Q{Qa}": round(u, 1) for (k, Qa), u in R.attention.items() if k == "fp8"},
                          **{f"hbm_frac_Q{Qa}": round(B * KV_HEADS * CONTEXT * 2 * (HEAD_DIM + 4) / (u * 1e-6) / 1e9
                                                      / HBM_PEAK_GBS, 4) for (k, Qa), u in R.attention.items()
                             if k == "fp8"}}},
        # outside the timed round: the FP8 parent (W8A8, E4M3) verifying gamma = 4 drafts of one
        # sequence (M = 5) on Qwen2.5-7B's projections; HBM fraction of the weight bytes alone
        "fp8_parent_qwen25_7b_M5": {
            **{f"{k}_us": round(v[0], 2) for k, v in R.fp8.items()},
            **{f"{k}_hbm_frac": round(v[2] / (v[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 3) for k, v in R.fp8.items()},
            "quantize_act_fp8_us": {k: round(v[1], 2) for k, v in R.fp8.items()},
            "layer_projections_us": round(sum(v[0] + v[1] for k, v in R.fp8.items() if k != "lm_head"), 1)},
        # outside the timed round: the verify-and-commit stage at B = 32, gamma = 4, V = 128256:
        # tokens/s = B (gamma + 1) / (T_accept + T_kv); HBM fractions of the algorithmic bytes
        # (greedy: the B (gamma + 1) target rows; sampling: those and the B gamma draft rows; KV:
        # each committed row read from the staging rows and written to the cache, all layers)
        "verify_commit_B32_g4": {
            name: {"accept_us": round(ta, 2), "kv_us": round(tk, 2), "committed_rows_per_seq": round(rows, 3),
                   "tokens_per_s": round(32 * 5 / ((ta + tk) * 1e-6), 1),
                   "accept_hbm_frac": round(4 * 32 * (5 if name == "greedy" else 9) * VOCAB / (ta * 1e-6) / 1e9
                                            / HBM_PEAK_GBS, 4),
                   "kv_hbm_frac": round(2 * rows * 32 * args.layers * 2 * KV_HEADS * HEAD_DIM * 2 / (tk * 1e-6) / 1e9
                                        / HBM_PEAK_GBS, 4)}
            for name, (ta, tk, rows) in R.verify_commit.items()},
        # verify tokens/s at gamma = 4: B (gamma + 1) / (sum of one layer's four W4A16 projections at
        # M = B (gamma + 1)), measured over all layers at B = 1, 4, 16, with the HBM roofline bound
        "verify_tokens_per_s": R.verify_tps,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_leg(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
