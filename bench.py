"""Benchmark of the Medusa tree-verification step on one MI355X.

One step = the whole hot path on one batch of synthetic input, already resident in HBM:
Medusa heads (residual block + vocabulary projection with top-k) -> candidate-tree assembly
-> tree-masked GQA attention -> acceptance -> commit of the accepted path into the KV cache.
The default workload is the Llama-3-8B-shaped layer: batch 1, 32 query / 8 KV heads of 128
dims, a 4096-token prefix, the 64-node (4,3,2,1) tree, 4 Medusa heads over d=4096 and a
32000-token vocabulary, bf16, greedy acceptance against target logits whose argmax matches a
child token with probability 0.6.

Prints one JSON line: steps/s (and verified tree tokens/s), the roofline of the dominant
kernel (the vocabulary-streaming head projection) timed with HIP events on the stream it
runs on, and the CPU oracle timed on the host cores on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload c3] [--no-cpu-baseline]
    python bench.py --workload c3 --tau 1024   # mean accepted length over a decode loop
    python bench.py --copy-calibration      # plain device copy of known size (for counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
F32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20         # Infinity Cache

DESCR = {
    "c1": "tiny-fp32: B=1, Hq=Hkv=4, dh=64, prefix 128, 8-node tree (two depth-4 chains), "
          "heads d=256 V=1000 K=3, greedy",
    "c2": "llama3-8b-layer: B=1, Hq=32, Hkv=8, dh=128, prefix 4096, 64-node (4,3,2,1) tree, "
          "heads d=4096 V=32000 K=4 bf16, greedy (planted p=0.6)",
    "c3": "70b-share-b8: B=8, Hq=64, Hkv=8, dh=128, prefix U[8192,32768], 64-node (4,3,2,1) tree, "
          "heads d=8192 V=32000 K=4 bf16, greedy (planted p=0.6)",
    "c4": "long-ctx-131k: B=1, Hq=64, Hkv=8, dh=128, prefix 131072, 212-node (4,4,4,2) tree, "
          "attention only, bf16",
    "c5": "spec-serving-b64: B=64, Hq=32, Hkv=8, dh=128, prefix U[512,8192], 64-node (4,3,2,1) "
          "tree, speculative acceptance over V=128256 (fp32 probabilities)",
    "c7": "spec-serving-b64-multicand: the spec-serving-b64 attention with 4/3/2/1 independent "
          "draft samples per node and sibling-recursive (lossless) acceptance over V=128256",
    "c8": "llama3-8b-layer-dyntree: the llama3-8b-layer step with 10 candidates per head and a "
          "per-sequence dynamic tree of the 64 most probable candidate paths",
    "c6": "llama3-8b-layer-lmhead: the llama3-8b-layer step with the greedy target computed by "
          "the target LM head (W_lm 32000 x 4096 bf16 over the 65 verify rows, argmax fused)",
    "c9": "llama3-8b-layer-lmhead-spec: the llama3-8b-layer step with speculative acceptance, "
          "the target from the LM head (W_lm 32000 x 4096 bf16, LSE per verify row) and the "
          "draft of depth k from Medusa head k's logits; no [N+1, V] probabilities",
    "c10": "spec-serving-b64-lmhead: the spec-serving-b64 attention (B=64, prefix U[512,8192]) "
           "with speculative acceptance driven by the target LM head (W_lm 128256 x 4096 bf16 "
           "over 64 x 65 verify rows, LSE per row) and a draft's per-depth logits [64, 4, 128256] "
           "(candidates = their top tokens); no [B, N+1, V] probabilities",
}


def _kernel_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel_key, workload, src_path):
    """HBM traffic per launch from the committed counter record of this kernel on this
    workload, if there is one and the kernel's source is still the one it was taken on."""
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not (name.startswith(f"traffic_{kernel_key}_") and name.endswith(".json")):
            continue
        with open(os.path.join(ROOT, "profiles", name)) as f:
            t = json.load(f)
        if t.get("workload") == workload and t.get("kernel_src_sha") == _kernel_sha(src_path):
            return t.get("hbm_bytes_per_launch")
    return None


# --------------------------------------------------------------------------- inputs
def make_inputs(wl, seed):
    from medusa_tree_attention_verify_amd import workloads as W
    x = {}
    if wl.has_heads:
        x.update(W.gen_heads(wl, seed))
    x.update(W.gen_attention(wl, seed))
    if wl.target_head:
        x.update(W.gen_target_head(wl, seed))
        if wl.accept == "speculative":
            x["uniforms"] = W.gen_uniforms(wl, seed)
            if not wl.has_heads:
                x["draft_logits"] = W.gen_draft_logits(wl, seed)
    elif wl.accept == "greedy":
        x["target"] = W.gen_target_logits(wl, seed)
    elif wl.accept in ("speculative", "multicand"):
        x.update(W.gen_speculative(wl, seed))
    return x


def step_bytes(wl, x):
    """Algorithmic bytes / FLOPs of one step (weights, K/V and rows read once)."""
    esz = 2 if wl.dtype == "bf16" else 4
    parts = {}
    if wl.has_heads:
        res = wl.K * wl.d * wl.d * esz + wl.B * wl.d * esz + wl.B * wl.K * wl.d * 4
        head = wl.K * wl.V * wl.d * esz + wl.B * wl.K * wl.d * 4
        parts["heads_residual"] = (res, 2.0 * wl.B * wl.K * wl.d * wl.d)
        parts["heads_projection"] = (head, 2.0 * wl.B * wl.K * wl.V * wl.d)
    L = x["prefix_len"].astype(np.int64)
    N = wl.N
    kv = int(np.sum((L + N) * wl.Hkv * wl.dh * esz * 2))
    qo = 2 * wl.B * N * wl.Hq * wl.dh * esz
    depth = []
    for p in wl.parents:
        depth.append(1 if p < 0 else depth[p] + 1)
    flops = float(np.sum(4.0 * wl.dh * wl.Hq * (N * L + sum(depth))))
    parts["attention"] = (kv + qo, flops)
    if wl.target_head and wl.accept == "speculative" and not wl.has_heads:
        # candidates and LSE of the draft's per-depth rows
        parts["heads_select"] = (wl.B * wl.D * wl.accept_V * 2, 0.0)
    if wl.target_head:
        T = wl.B * (N + 1)
        parts["target_head"] = (wl.accept_V * wl.d * 2 + T * wl.d * 2, 2.0 * T * wl.accept_V * wl.d)
        if wl.accept == "speculative":
            # per node: its W_lm row and its parent's hidden state; the terminal's target row
            # is one more pass over W_lm; the draft row and the two rows' residual passes
            parts["accept"] = (wl.B * N * 4 * wl.d + wl.accept_V * wl.d * 2
                               + wl.B * wl.accept_V * (2 + 3 * 2 * 4),
                               2.0 * wl.B * (N + wl.accept_V) * wl.d)
        else:
            parts["accept"] = (T * 4, 0.0)
    elif wl.accept == "greedy":
        parts["accept"] = (wl.B * (N + 1) * wl.accept_V * esz, 0.0)
    elif wl.accept in ("speculative", "multicand"):
        # the extra token's pass over the terminal rows (P_t, P_d) and the 2N gathers; the
        # multi-candidate walk adds one such row pass per rejection followed by a sibling
        parts["accept"] = (wl.B * (2 * N * 4 + 2 * wl.accept_V * 4), 0.0)
    return parts


# --------------------------------------------------------------------------- CPU oracle
def _host_info():
    """CPU model (first /proc/cpuinfo entry), usable cores and the BLAS thread count."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return model, cores, blas


def _oracle_step(wl, x, seed, attn_rows=None):
    """One oracle step of the workload on its inputs; returns seconds per part.

    attn_rows = (b, h, i) query rows: the attention is computed for those rows only (None:
    every row).  Planting the target is input generation and is not timed."""
    from medusa_tree_attention_verify_amd import workloads as W
    from oracle import medusa_oracle as O

    parents = list(wl.parents)
    t = {}
    t0 = time.perf_counter()
    cand = []
    if wl.has_heads:
        heads = O.medusa_heads(x["h"], x["w_res"], x["w_head"], list(wl.head_widths))
        if wl.lm_width:
            cand.append(np.stack([O.topk_rows(x["target"][b, 0], wl.lm_width)["ids"]
                                  for b in range(wl.B)]))
        cand += [heads["topk_ids"][:, k, :wl.head_widths[k]] for k in range(wl.K)]
    elif "draft_logits" in x:    # a draft's per-depth logits: their top tokens are the candidates
        cand = [np.stack([O.topk_rows(x["draft_logits"][b, k], wl.depth_widths[k])["ids"]
                          for b in range(wl.B)]) for k in range(wl.D)]
    t1 = time.perf_counter()
    if wl.dynamic_nodes:         # one tree per sequence: its most probable head paths
        dyn = O.dynamic_tree(heads["topk_ids"], heads["topk_vals"], heads["lse"],
                             list(wl.head_widths), wl.dynamic_nodes)
        trees = [{"parents": dyn["parents"][b], "anc": dyn["anc"][b],
                  "tokens": np.array([dyn["tokens"][b]])} for b in range(wl.B)]
    else:
        tree = (O.build_tree(parents, cand, list(wl.depth_widths)) if cand
                else O.build_tree(parents))
        trees = [{"parents": parents, "anc": tree["anc"],
                  "tokens": tree["tokens"][b:b + 1] if "tokens" in tree else None}
                 for b in range(wl.B)]
    t2 = time.perf_counter()
    t["heads"], t["tree"] = t1 - t0, t2 - t1
    target = None
    x_t = None
    if wl.target_head:
        x_t = x["x_t"].copy()
        if wl.plant_p > 0:
            x_t = W.plant_target_head(x_t, x["w_lm"], parents, tree["tokens"], seed, wl.plant_p)
    elif wl.accept == "greedy":
        target = x["target"].copy()
        if wl.plant_p > 0 and wl.dynamic_nodes:
            for b, tr in enumerate(trees):
                target[b:b + 1] = W.plant_greedy(target[b:b + 1], tr["parents"], tr["tokens"],
                                                 seed + b, wl.plant_p)
        elif wl.plant_p > 0:
            target = W.plant_greedy(target, parents, tree["tokens"], seed, wl.plant_p)
        if wl.dtype == "bf16":
            target = W.round_bf16(target)
    t3 = time.perf_counter()
    if wl.dynamic_nodes:
        for b, tr in enumerate(trees):
            sl = slice(b, b + 1)
            O.tree_attention(x["q"][sl], x["k_cache"][sl], x["v_cache"][sl],
                             x["prefix_len"][sl], tr["anc"])
    else:
        O.tree_attention(x["q"], x["k_cache"], x["v_cache"], x["prefix_len"], tree["anc"],
                         select=attn_rows)
    t4 = time.perf_counter()
    if wl.target_head and wl.accept == "speculative":
        draft = heads["logits"] if wl.has_heads else x["draft_logits"]
        acc = O.accept_speculative_lm(x_t, x["w_lm"], draft, tree["tokens"], parents,
                                      x["uniforms"], wl.D)
    elif wl.target_head:
        z = O.lm_head_argmax(x_t.reshape(-1, wl.d), x["w_lm"])["logits"]
        target = z.reshape(wl.B, wl.N + 1, wl.accept_V)
    if wl.target_head and wl.accept == "speculative":
        pass
    elif wl.accept == "greedy" and wl.dynamic_nodes:
        per = [O.accept_greedy(target[b:b + 1], tr["tokens"], tr["parents"], wl.D)
               for b, tr in enumerate(trees)]
        acc = {k: np.concatenate([a[k] for a in per]) for k in ("accept_len", "path_nodes")}
    elif wl.accept == "greedy":
        acc = O.accept_greedy(target, tree["tokens"], parents, wl.D)
    elif wl.accept == "multicand":
        acc = O.accept_multicandidate(x["p_target"], x["p_draft"], x["node_tokens"], parents,
                                      x["uniforms"], wl.D)
    elif wl.accept == "speculative":
        acc = O.accept_speculative(x["p_target"], x["p_draft"], x["node_tokens"], parents,
                                   x["uniforms"], wl.D)
    if wl.accept != "none":     # commit, on each sequence's tree block
        for b in range(wl.B):
            Lb = int(x["prefix_len"][b])
            blk = slice(Lb, Lb + wl.N)
            O.kv_commit(x["k_cache"][b:b + 1, :, blk], x["v_cache"][b:b + 1, :, blk],
                        np.zeros(1, np.int64), acc["path_nodes"][b:b + 1],
                        acc["accept_len"][b:b + 1], wl.N)
    t5 = time.perf_counter()
    t["attention"], t["accept_commit"] = t4 - t3, t5 - t4
    return t


# query-row x key products above which one oracle step is sampled instead of run whole, and
# the products of the sampled attention (whole (sequence, KV head) slices: the 70B share's whole
# attention, ~10 s of the oracle on a 16-core host)
ORACLE_FULL_STEP_WORK = 5e7
ORACLE_SAMPLE_WORK = 1e9


def cpu_baseline(wl, x, seed, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Small steps run whole, repeatedly, until ``budget_s`` seconds of oracle work.  Larger ones
    run one step in which every part is whole except the attention, which is computed for the
    query rows of whole (sequence, KV head) slices, longest sequences first, until about
    ORACLE_SAMPLE_WORK row x key products, and scaled to the whole batch by its share of row x
    key products (the oracle's attention costs one pass over the visible keys per query row)."""
    model, cores, blas = _host_info()
    N, G = wl.N, wl.Hq // wl.Hkv
    keys = x["prefix_len"].astype(np.int64) + N
    work = float(np.sum(keys)) * wl.Hq * N
    res = {"unit": "steps/s", "cores": int(blas), "kind": "oracle", "cpu_model": model,
           "host_cores": int(cores), "blas_threads": int(blas)}
    if work <= ORACLE_FULL_STEP_WORK:
        t_total, steps = 0.0, 0
        while True:
            t_total += sum(_oracle_step(wl, x, seed).values())
            steps += 1
            if t_total >= budget_s or steps >= 100:
                break
        res.update(value=steps / t_total,
                   sample=f"{steps} full oracle step(s) of the same workload (seed {seed}), "
                          f"{t_total:.1f} s, NumPy fp64")
        return res
    rows, sampled, slices = [], 0.0, []
    for b in np.argsort(-keys, kind="stable"):   # whole slices, longest sequences first
        for g in range(wl.Hkv):
            if sampled >= ORACLE_SAMPLE_WORK:
                break
            rows += [(int(b), g * G + j, i) for j in range(G) for i in range(N)]
            sampled += float(keys[b]) * G * N
            slices.append((int(b), g))
    parts = _oracle_step(wl, x, seed, attn_rows=rows)
    scale = work / sampled
    t_step = parts["heads"] + parts["tree"] + parts["accept_commit"] + parts["attention"] * scale
    res.update(value=1.0 / t_step,
               sample=f"one oracle step (seed {seed}, NumPy fp64) with heads, tree, acceptance "
                      f"and commit whole and the attention of {len(rows)} of {wl.B * wl.Hq * N} "
                      f"query rows ({len(slices)} whole (sequence, KV head) slices, longest "
                      f"sequences first), scaled x{scale:.2f} by query-row x key products; "
                      f"measured {sum(parts.values()):.1f} s",
               parts_s={k: round(v * (scale if k == "attention" else 1.0), 3)
                        for k, v in parts.items()})
    return res


def cpu_single_thread(names=("c1", "c2"), budget_s=5.0):
    """Whole oracle steps of the small workloads with one BLAS thread (steps/s)."""
    from threadpoolctl import threadpool_limits

    from medusa_tree_attention_verify_amd import workloads as W
    out = {}
    for n in names:
        wl = W.WORKLOADS[n]
        seed = int(n[1:])
        x = make_inputs(wl, seed)
        with threadpool_limits(limits=1):
            t_total, steps = 0.0, 0
            while t_total < budget_s and steps < 100:
                t_total += sum(_oracle_step(wl, x, seed).values())
                steps += 1
        out[DESCR[n].split(":")[0]] = round(steps / t_total, 3)
        del x
    return out


# --------------------------------------------------------------------------- main
def hbm_copy_probe(nbytes=1 << 30, reps=5):
    """GB/s of a plain device-to-device copy (read + write bytes), best of `reps`."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    best = 0.0
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (e0.elapsed_time(e1) / 1000.0) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return best


def copy_calibration(nbytes=1 << 30, reps=5):
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def tau_loop(n_seq_steps, wl, seed, step, inputs, x):
    """Committed decode loop for the mean accepted length (tau) of the planted generator.

    Every step verifies the same candidate tree (the heads' input is fixed) against a target
    planted afresh (its own seed): each parent row's greedy token is one of its children with
    probability p, independently.  The step commits its accepted path and the next step starts
    from the grown prefix (the prefixes start D x steps below the drawn ones, so they stay
    inside the cache).  On a tree that is full to depth D this gives P(accepted >= k) = p^k
    and a mean accepted length of sum_{k=1..D} p^k (the page's tau with one extra token per
    step is that plus one).  Prints one JSON line; nothing here is timed."""
    import torch

    from medusa_tree_attention_verify_amd import workloads as W
    if wl.accept != "greedy" or wl.plant_p <= 0 or wl.target_head or wl.dynamic_nodes:
        raise SystemExit("--tau needs a greedy workload with a planted target and a fixed tree")
    parents = list(wl.parents)
    depth = []
    for p_ in parents:
        depth.append(1 if p_ < 0 else depth[p_] + 1)
    has_kids = {p_ for p_ in parents}
    full = all(i in has_kids for i, dd in enumerate(depth) if dd < wl.D)
    steps = -(-n_seq_steps // wl.B)
    calls = step.sequence(step.bind(inputs))
    toks = step.tree["node_tokens"].cpu().numpy()
    pl = inputs["prefix_len"]
    start = np.maximum(0, x["prefix_len"].astype(np.int64) - wl.D * steps).astype(np.int32)
    pl.copy_(torch.from_numpy(start))
    lens = []
    for it in range(steps):
        tgt = W.plant_greedy(x["target"].copy(), parents, toks, seed * 100003 + it + 1,
                             wl.plant_p)
        if wl.dtype == "bf16":
            tgt = W.round_bf16(tgt)
        inputs["target"].copy_(torch.from_numpy(tgt))
        for c in calls:
            c()
        torch.cuda.synchronize()
        lens.append(step.acc["accept_len"].cpu().numpy().copy())
        pl.copy_(step.prefix_next)
    torch.cuda.synchronize()
    if int(step.status.item()) != 0:
        raise RuntimeError(f"device status flags {int(step.status.item())}")
    a = np.concatenate(lens).astype(np.float64)
    n = a.size
    mean, se = float(a.mean()), float(a.std(ddof=1) / np.sqrt(n))
    p = wl.plant_p
    cf = sum(p ** k for k in range(1, wl.D + 1)) if full else None
    grew = (pl.cpu().numpy().astype(np.int64) - start).tolist()
    print(json.dumps({
        "metric": "mean accepted length per verify step (tau, planted greedy target)",
        "value": round(mean, 4), "unit": "tokens", "sequence_steps": int(n), "steps": steps,
        "std_err": round(se, 4), "ci95": [round(mean - 1.96 * se, 4), round(mean + 1.96 * se, 4)],
        "closed_form": None if cf is None else round(cf, 4),
        "z_vs_closed_form": None if cf is None else round((mean - cf) / se, 2),
        "emitted_per_step": round(mean + 1.0, 4),
        "emitted_closed_form": None if cf is None else round(cf + 1.0, 4),
        "p_len_ge_k": {str(k): [round(float((a >= k).mean()), 4), round(p ** k, 4)]
                       for k in range(1, wl.D + 1)},
        "prefix_growth_per_sequence": grew,
        "config": {"workload": DESCR[wl_key(wl)], "plant_p": p, "seed": seed},
    }), flush=True)


def wl_key(wl):
    from medusa_tree_attention_verify_amd import workloads as W
    return next(k for k, v in W.WORKLOADS.items() if v == wl)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps before each timed pass (the clocks settle after ~600)")
    ap.add_argument("--workload", default="c3", choices=sorted(DESCR))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single-thread", action="store_true",
                    help="skip the one-thread oracle timings of the two small workloads")
    ap.add_argument("--tau", type=int, default=0,
                    help="instead of timing: run a committed decode loop of this many "
                         "sequence-steps with freshly planted targets and report the mean "
                         "accepted length against the planted closed form")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work timed for cpu_baseline (whole steps, at least one)")
    ap.add_argument("--fork", default="auto", choices=["auto", "on", "off"],
                    help="graph launch: run the attention branch beside the heads (a parallel "
                         "branch of the graph, the attention on half of the CUs) or after them; "
                         "auto = beside them for steps with Medusa heads over a batch (the 70B "
                         "share: 1360 against 1187 steps/s; one-sequence steps, whose attention "
                         "is a short latency-bound call, lose 2-4%%)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="time the step replayed as one HIP graph (default) or as eager launches")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for {args.gpus}); "
              "the path would shard per sequence / KV head / vocabulary slice, but the library "
              "has no multi-GPU code", file=sys.stderr)
        sys.exit(2)

    import torch

    from medusa_tree_attention_verify_amd import _lib, ops
    from medusa_tree_attention_verify_amd import workloads as W
    from medusa_tree_attention_verify_amd.step import VerifyStep

    if args.copy_calibration:
        copy_calibration()
        return
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    _lib.lib()
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.workload]
    seed = args.seed or int(args.workload[1:])
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    t0 = time.time()
    x = make_inputs(wl, seed)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    parts = step_bytes(wl, x)
    step_total = sum(b for b, _ in parts.values())

    max_L = int(x["prefix_len"].max())
    spec = wl.accept in ("speculative", "multicand") and not wl.target_head
    step = VerifyStep(parents=wl.parents, depth_widths=wl.depth_widths, dtype=dt, B=wl.B,
                      Hq=wl.Hq, Hkv=wl.Hkv, dh=wl.dh, max_L=max_L,
                      heads={"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)}
                      if wl.has_heads else None,
                      lm_width=wl.lm_width, accept=wl.accept, V=wl.accept_V,
                      tokens_given=not wl.has_heads and not wl.target_head,
                      target_head=wl.d if wl.target_head else None,
                      commit=wl.accept != "none", dynamic_nodes=wl.dynamic_nodes or None)
    d = lambda a, t=dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    static = {}
    if wl.has_heads:
        static.update(h=d(x["h"]), w_res=d(x["w_res"]), w_head=d(x["w_head"]))
    if wl.target_head:
        static["w_lm"] = d(x["w_lm"], torch.bfloat16)
    # Rotating copies of the per-step activations so that the 256 MB Infinity Cache cannot
    # serve them as "HBM" reads: only needed when one step moves less than 2x the cache.
    rot_bytes = parts["attention"][0] + (parts["accept"][0] if "accept" in parts else 0)
    R = 1 if step_total >= 2 * MALL_BYTES else int(np.ceil(2 * MALL_BYTES / max(rot_bytes, 1)))
    R = min(R, 64)
    base = {"q": d(x["q"]), "k_cache": d(x["k_cache"]), "v_cache": d(x["v_cache"]),
            "prefix_len": d(x["prefix_len"], torch.int32)}
    if spec:
        base.update(target=d(x["p_target"], torch.float32), draft=d(x["p_draft"], torch.float32),
                    uniforms=d(x["uniforms"], torch.float32),
                    node_tokens=d(x["node_tokens"], torch.int32))
    elif wl.target_head:
        # the target rows' hidden states are planted against the node tokens this step
        # produces (the heads and the tree run once, untimed, to get them)
        base["x_t"] = d(x["x_t"], torch.bfloat16)
        if "uniforms" in x:
            base["uniforms"] = d(x["uniforms"], torch.float32)
        if "draft_logits" in x:
            base["draft_logits"] = d(x["draft_logits"], torch.bfloat16)
        if wl.plant_p > 0:
            c = step.bind(dict(static, **base))
            for part in ("heads_residual", "heads_projection", "heads_select", "tree"):
                c[part]()
            torch.cuda.synchronize()
            toks = step.tree["node_tokens"].cpu().numpy()
            xt = W.plant_target_head(x["x_t"].copy(), x["w_lm"], list(wl.parents), toks, seed,
                                     wl.plant_p)
            base["x_t"] = d(xt, torch.bfloat16)
    elif wl.accept == "greedy":
        # the greedy target is planted against the node tokens this step produces: run the
        # heads and the tree once (untimed) to get them
        base["target"] = d(W.round_bf16(x["target"]) if wl.dtype == "bf16" else x["target"])
        if wl.plant_p > 0:
            c = step.bind(dict(static, **base))
            for part in ("heads_residual", "heads_projection", "heads_select", "tree"):
                c[part]()
            torch.cuda.synchronize()
            toks = step.tree["node_tokens"].cpu().numpy()
            if step.dynamic:         # each sequence planted against its own tree
                par = step.parents.cpu().numpy()
                tgt = x["target"].copy()
                for b in range(wl.B):
                    tgt[b:b + 1] = W.plant_greedy(tgt[b:b + 1], par[b].tolist(), toks[b:b + 1],
                                                  seed + b, wl.plant_p)
            else:
                tgt = W.plant_greedy(x["target"].copy(), list(wl.parents), toks, seed, wl.plant_p)
            base["target"] = d(W.round_bf16(tgt) if wl.dtype == "bf16" else tgt)
    if args.tau:
        tau_loop(args.tau, wl, seed, step, dict(static, **base), x)
        return
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    seqs = [step.sequence(step.bind(dict(static, **s))) for s in sets]
    present = [p for p in step.PARTS if p in step.bind(dict(static, **base))]

    def one_step(i, ev=None):
        for j, call in enumerate(seqs[i % R]):
            if ev is not None:
                ev[j].record()
            call()
        if ev is not None:
            ev[len(present)].record()

    for i in range(max(args.warmup, 1)):
        one_step(i)
    torch.cuda.synchronize()
    if step.commit:
        # the commit moves 2 (K, V) x Hkv x dh elements per accepted token, read and written,
        # and reads the path, its length and the prefix, and writes the next prefix
        esz = 2 if wl.dtype == "bf16" else 4
        n_acc = int(step.acc["accept_len"].sum().item())
        parts["commit"] = (4 * wl.Hkv * wl.dh * esz * n_acc + 4 * wl.B * (wl.D + 3), 0.0)
        step_total = sum(b for b, _ in parts.values())
    K = args.steps
    # Pass 1 (eager, per-part HIP events on the launch stream): per-kernel durations.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(present) + 1)]
           for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        one_step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(stop) / K
    # Pass 2 (the timed region of the metric): the same K steps, each replayed as one graph.
    t_wall = None
    ms = ms_eager
    fork = (args.fork == "on" or (args.fork == "auto" and wl.has_heads and wl.B > 1)) and step.can_fork()
    if args.launch == "graph":
        graphs = [step.capture(dict(static, **s_), fork=fork) for s_ in sets]
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record()
        for i in range(K):
            graphs[i % R].replay()
        stop.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms = start.elapsed_time(stop) / K
    if int(step.status.item()) != 0:
        raise RuntimeError(f"device status flags {int(step.status.item())}")
    ms = start.elapsed_time(stop) / K
    steps_per_s = 1000.0 / ms
    # Spread: four more regions of the same K steps after the timed one (not part of `value`).
    repeats = [steps_per_s]
    for _ in range(4):
        start.record()
        for i in range(K):
            if args.launch == "graph":
                graphs[i % R].replay()
            else:
                one_step(i)
        stop.record()
        torch.cuda.synchronize()
        repeats.append(1000.0 * K / start.elapsed_time(stop))
    probe = hbm_copy_probe()
    seg = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(present))] for e in evs])
    seg_mean = dict(zip(present, seg.mean(axis=0)))  # ms per part
    parts_ms = {n: round(float(v), 4) for n, v in seg_mean.items()}

    # dominant kernel: the vocabulary-streaming head projection (one kernel launch)
    roof = None
    if wl.has_heads:
        b_head = parts["heads_projection"][0]
        dur_s = seg_mean["heads_projection"] / 1000.0
        ach = b_head / dur_s / 1e9
        src = os.path.join(ROOT, "medusa_tree_attention_verify_amd", "csrc", "heads.hip")
        kname = "gemv_bf16_kernel" if wl.dtype == "bf16" else "gemv_f32_kernel"
        roof = {"kernel": f"{kname}<head projection>", "bound": "hbm",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": _traffic("head_projection", DESCR[args.workload].split(":")[0], src),
                "algorithmic_bytes": int(b_head), "avg_launch_us": round(seg_mean["heads_projection"] * 1000, 2)}
    elif wl.target_head:
        # dominant: the target LM head over all verify rows (tiled kernel + merge, one call);
        # at B*(N+1) = 4160 rows it is bound by the matrix cores
        b_lm, f_lm = parts["target_head"]
        dur_s = seg_mean["target_head"] / 1000.0
        src = os.path.join(ROOT, "medusa_tree_attention_verify_amd", "csrc", "lmhead.hip")
        traffic = _traffic("lm_head", DESCR[args.workload].split(":")[0], src)
        if f_lm / b_lm > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            ach = f_lm / dur_s / 1e12
            roof = {"kernel": "lm_head_gemm_kernel + lm_head_merge_kernel", "bound": "mfma",
                    "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "algorithmic_flops": f_lm}
        else:
            ach = b_lm / dur_s / 1e9
            roof = {"kernel": "lm_head_kernel + lm_head_merge_kernel", "bound": "hbm",
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
        roof["algorithmic_bytes"] = int(b_lm)
        roof["avg_launch_us"] = round(seg_mean["target_head"] * 1000, 2)
    else:
        # dominant: the tree-attention call (attention kernel, plus the combine when the keys
        # are split and the length ordering for batches), timed as one part
        b_att, f_att = parts["attention"]
        dur_s = seg_mean["attention"] / 1000.0
        src = os.path.join(ROOT, "medusa_tree_attention_verify_amd", "csrc", "attention.hip")
        traffic = _traffic("tree_attention", DESCR[args.workload].split(":")[0], src)
        if f_att / b_att > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            ach = f_att / dur_s / 1e12
            roof = {"kernel": "tree_attn_bf16_kernel + combine", "bound": "mfma",
                    "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "algorithmic_flops": f_att}
        else:
            ach = b_att / dur_s / 1e9
            roof = {"kernel": "tree_attn_bf16_kernel + combine", "bound": "hbm",
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
        roof["algorithmic_bytes"] = int(b_att)
        roof["avg_launch_us"] = round(seg_mean["attention"] * 1000, 2)
    t_roof = sum(max(b / (HBM_PEAK_GBS * 1e9), f / (BF16_PEAK_TFLOPS * 1e12))
                 for b, f in parts.values())
    out = {
        "metric": "tree-verify steps/s & verified tree tokens/s; % of HBM/MFMA roofline",
        "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,s) weights/activations, planted target argmax)",
        "config": {"workload": DESCR[args.workload], "global_batch": wl.B, "tree_nodes": wl.N,
                   "seq_len": max_L, "rotating_input_sets": R},
        "verified_tree_tokens_per_s": round(steps_per_s * wl.B * wl.N, 1),
        # acceptance of the last timed step: one draw of the planted target per sequence (every
        # replay accepts the same path); a many-step mean is what `--tau` measures
        "last_step_accept_len": ({"mean": round(float(step.acc["accept_len"].float().mean().item()), 3),
                                  "sequences": wl.B}
                                 if wl.accept != "none" else None),
        # accepted tokens + one bonus token per sequence, per second of replayed steps
        "last_step_emitted_tokens_per_s": (round(steps_per_s * float((step.acc["accept_len"] + 1)
                                                                      .sum().item()), 1)
                                           if wl.accept != "none" else None),
        "step_roofline_frac": round(t_roof / (ms / 1000.0), 4),
        "step_algorithmic_bytes": int(step_total),
        "parts_ms": parts_ms,
        # each part's roofline fraction: its algorithmic bytes / 8 TB/s or FLOPs / bf16 peak,
        # whichever is larger, over its eager HIP-event time
        "parts_roofline_frac": {n: round(max(parts[n][0] / (HBM_PEAK_GBS * 1e9),
                                             parts[n][1] / (BF16_PEAK_TFLOPS * 1e12))
                                         / (seg_mean[n] / 1000.0), 4)
                                for n in parts if n in seg_mean and seg_mean[n] > 0},
        "roofline": roof,
        "launch": args.launch,
        "graph_fork": bool(fork and args.launch == "graph"),
        "eager_steps_per_s": round(1000.0 / ms_eager, 2),
        "wall_s_timed_region": None if t_wall is None else round(t_wall, 4),
        "repeats_steps_per_s": [round(v, 1) for v in repeats],
        "repeats_p10_p50_p90": [round(float(np.percentile(repeats, q)), 1) for q in (10, 50, 90)],
        # context for the 8 TB/s denominator: a plain 1 GiB device copy on this GPU (bytes read
        # + written per second, best of 5)
        "hbm_copy_probe_GBs": round(probe, 1),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(wl, x, seed, args.cpu_budget)
        if not args.no_single_thread:
            del x
            out["cpu_baseline"]["single_thread_steps_per_s"] = cpu_single_thread()
        print(f"# cpu baseline took {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
