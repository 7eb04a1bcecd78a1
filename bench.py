"""Benchmark of the tree speculative-decoding verify step on one MI355X.

One step = the whole verify hot path over one batch of seeded synthetic input:
jt_build_tree -> jt_tree_meta -> jt_tree_attention -> jt_accept, all through
the C ABI on the current stream.  The workload is the Qwen3-30B-A3B-shaped
attention layer (32 query heads, 4 KV heads, head_dim 128, bf16), batch 8,
32768-token prefixes in a paged cache (16-token pages, permuted), trees of
budget B = 256 (W = 8, N = 16) drafted from [16, 151936] fp32 logits, and
acceptance over [257, 151936] fp32 target logits per sequence.

Printed: one JSON line.  ``value`` is tree-node tokens per second of the whole
step (sum of n_nodes over the batch / step time); the attention kernel is
additionally reported as KV GB/s and against the bf16 MFMA roofline.  The
same run also times the step on the pages' other settings (budget 16 and 256
at batch 1, batch 16/32 serving; ``configs``) and two probes of this box's
practical ceilings (a device copy and a large bf16 GEMM; ``probes``).
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

WORKLOAD = "qwen3_30b_a3b_b8"
# the other settings timed in the same run (shorter: they are secondary lines)
SECONDARY = ("tiny_f32", "qwen3_8b_b16", "qwen3_8b_b256", "serving_b16", "serving_b32")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=8,
                    help="sequences of the workload the CPU oracle is timed on")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the main workload, not the secondary settings")
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device --steps times (a plain copy of known "
                         "size, the reference that HBM byte counters are scaled by)")
    return ap.parse_args()


ATTN_SRC = os.path.join(ROOT, "tree_causal_attention_amd", "csrc", "tree_attention.hip")
PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(workload):
    """HBM bytes per jt_tree_attention launch from the committed counter summary.

    The summary records the sha256 of the attention source it was measured on;
    when the source has changed since, the figure no longer applies (None).
    """
    import hashlib
    path = os.path.join(PROFILES, f"tree_attention_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    with open(ATTN_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel source sha256") != sha:
        return None
    try:
        return int(fields["HBM traffic per launch (bytes)"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes, steps):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_probe_bytes": nbytes, "ms_per_copy": ms,
                      "GBps": 2 * nbytes / ms / 1e6}))


def algorithmic_work(w, prefix, n_nodes, depth):
    """Attention bytes and flops the method must move / compute.

    bytes = sum_s (P_s + n_s) * Hkv * D * 2 * e   (K and V read once)
          + sum_s n_s * Hq * D * 2 * e           (Q read, O written)
    flops = 4 * D * Hq * sum_s sum_{i < n_s} (P_s + depth_i + 1)
    (masked tail entries do not count).
    """
    e = 2 if w.dtype == "bf16" else 4
    kv = q = fl = 0
    for s in range(len(prefix)):
        P, n = int(prefix[s]), int(n_nodes[s])
        kv += (P + n) * w.hkv * w.head_dim * 2 * e
        q += n * w.hq * w.head_dim * 2 * e
        vis = n * P + int(sum(int(d) + 1 for d in depth[s][:n]))
        fl += 4 * w.head_dim * w.hq * vis
    return kv, q, fl


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def probes():
    """Practical ceilings measured on this machine: a 1 GiB device copy (read +
    write bytes) and an 8192^3 bf16 GEMM through the vendor library."""
    import torch
    out = {}
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["copy_gbps"] = 2 * (1 << 30) * 10 / e0.elapsed_time(e1) / 1e6
    del a, b
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    y = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):
        torch.matmul(x, y)
    e0.record()
    for _ in range(10):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    out["gemm_bf16_tflops"] = 2 * n ** 3 * 10 / e0.elapsed_time(e1) / 1e9
    return out


def cpu_baseline(w, x, seqs):
    """The CPU oracle, untouched, on the first ``seqs`` sequences of the batch."""
    import numpy as np
    from oracle import tree_oracle as O
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    kf = x.k_pool.float().numpy()
    vf = x.v_pool.float().numpy()
    t0 = time.perf_counter()
    nodes = 0
    for s in range(seqs):
        tr = O.build_tree(x.draft[s].numpy(), w.width_w, w.budget_b, int(x.root_token[s]),
                          check_exact=False)
        n = tr["n_nodes"]
        O.ancestor_mask(tr["parent"], n)
        O.tree_attention_seq_fast(x.q[s].float().numpy(), kf, vf, x.page_table[s].numpy(),
                                  int(x.prefix_len[s]), tr["parent"], n, w.scale)
        O.accept(x.target[s].numpy(), tr["parent"], tr["token"], tr["depth"], n, w.depth_n)
        nodes += n
    dt = time.perf_counter() - t0
    return {"value": nodes / dt, "unit": "tree-node tok/s", "cores": int(threads),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{seqs} of {w.batch} sequences of the same workload, whole verify step "
                      f"(build, mask, attention, accept) in fp64 NumPy; {dt:.2f} s"}


class Verify:
    """One workload's inputs in HBM, its outputs and workspaces (allocated
    once, outside any timed region) and the verify step on the current stream."""

    def __init__(self, B, w, dev):
        import torch
        self.B, self.w = B, w
        x = self.x = make_inputs_for(w)
        self.d_draft = x.draft.to(dev)
        self.d_target = x.target.to(dev)
        self.d_q, self.d_k, self.d_v = x.q.to(dev), x.k_pool.to(dev), x.v_pool.to(dev)
        self.d_prefix, self.d_table = x.prefix_len.to(dev), x.page_table.to(dev)
        self.d_root = x.root_token.to(dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        b, T = w.batch, w.max_nodes
        lib = B.load()
        self.ws_build = torch.empty(max(1, lib.jt_build_tree_workspace(
            b, w.depth_n, w.vocab, w.width_w, w.budget_b)), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(1, lib.jt_tree_attention_workspace(
            b, T, w.hq, w.hkv, w.head_dim, x.page_table.shape[1], 16,
            B.JT_BF16 if w.dtype == "bf16" else B.JT_F32)), dtype=torch.uint8, device=dev)
        self.ws_acc = torch.empty(max(1, lib.jt_accept_workspace(b, T, w.vocab)),
                                  dtype=torch.uint8, device=dev)
        self.anc = torch.empty((b, T, (T + 31) // 32), dtype=torch.int32, device=dev)
        self.tree_out = B._tree_outputs(b, T, dev, True)
        self.acc_out = B._accept_outputs(b, w.depth_n, dev, None)
        self.out = torch.empty_like(self.d_q)
        self.lse = torch.empty((b, T, w.hq), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        self.ev = {k: [] for k in ("s0", "s1", "s2", "s3", "s4")}

    def step(self, record):
        import torch
        B, w, ev, st = self.B, self.w, self.ev, self.stream

        def mark(k):
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(st)
                ev[k].append(e)
        mark("s0")
        tree = B.jt_build_tree(self.d_draft, w.width_w, w.budget_b, self.d_root, err=self.err,
                               workspace=self.ws_build, out=self.tree_out)
        mark("s1")
        B.jt_tree_meta(tree["parent"], tree["n_nodes"], err=self.err, out=self.anc)
        mark("s2")
        B.jt_tree_attention(self.d_q, self.d_k, self.d_v, tree["n_nodes"], self.d_prefix,
                            self.d_table, self.x.num_pages, self.anc, w.scale, err=self.err,
                            out=self.out, lse=self.lse, workspace=self.ws_attn)
        mark("s3")
        res = B.jt_accept(self.d_target, w.depth_n, tree["parent"], tree["token"],
                          tree["depth"], tree["n_nodes"], err=self.err, workspace=self.ws_acc,
                          out=self.acc_out)
        mark("s4")
        return tree, res

    def run(self, steps, warmup):
        """Warm up, then two passes of `steps` steps.  The timed pass has the
        wall clock around it (synchronised on both sides) and nothing but the
        steps inside; it gives the step time.  The breakdown pass right after
        records HIP events between the stages; each event costs the stream a
        few microseconds (≈ 3 µs on MI355X), so its stages add up to a little
        more than the timed step."""
        import torch
        for _ in range(warmup):
            self.step(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            tree, res = self.step(False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for k_ in self.ev:
            self.ev[k_].clear()
        for _ in range(steps):
            self.step(True)
        torch.cuda.synchronize()
        if int(self.err.item()) != 0:
            raise RuntimeError(f"{self.w.name}: device error bits {int(self.err.item())}")
        return wall * 1000.0 / steps, tree, res

    def avg(self, a, b_):
        ev = self.ev
        return sum(x_.elapsed_time(y_) for x_, y_ in zip(ev[a], ev[b_])) / len(ev[a])

    def pct(self, a, b_):
        import numpy as np
        ev = self.ev
        v = np.sort([x_.elapsed_time(y_) for x_, y_ in zip(ev[a], ev[b_])])
        return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
                "p90": float(np.percentile(v, 90))}

    def stage_ms(self):
        return {"build_tree": self.avg("s0", "s1"), "tree_meta": self.avg("s1", "s2"),
                "tree_attention": self.avg("s2", "s3"), "accept": self.avg("s3", "s4")}

    def attention_figures(self, tree, t_attn_ms):
        w = self.w
        n_nodes = tree["n_nodes"].cpu().numpy()
        depth = tree["depth"].cpu().numpy()
        kv_bytes, qo_bytes, flops = algorithmic_work(w, self.x.prefix_len.numpy(), n_nodes,
                                                     depth)
        t = t_attn_ms / 1000.0
        return {"tokens": int(n_nodes.sum()), "kv_bytes": kv_bytes, "qo_bytes": qo_bytes,
                "flops": flops, "tflops": flops / t / 1e12, "kv_gbps": kv_bytes / t / 1e9}


def make_inputs_for(w):
    from tree_causal_attention_amd import workloads as WL
    return WL.make_inputs(w)


def secondary_line(B, name, dev, steps, warmup, peaks):
    """Step time, stage times and the attention's rates for one more setting."""
    import torch
    from tree_causal_attention_amd import workloads as WL
    w = WL.WORKLOADS[name]
    v = Verify(B, w, dev)
    ms_step, tree, res = v.run(steps, warmup)
    st = v.stage_ms()
    fig = v.attention_figures(tree, st["tree_attention"])
    line = {
        "workload": f"batch {w.batch}, prefix {w.prefix}, {w.hq}q/{w.hkv}kv heads, head_dim "
                    f"{w.head_dim}, {w.dtype}, B={w.budget_b}, W={w.width_w}, N={w.depth_n}, "
                    f"vocab {w.vocab}",
        "ms_per_step": ms_step,
        "tree_nodes_per_step": fig["tokens"],
        "tok_per_s": fig["tokens"] / (ms_step / 1000.0),
        "stage_ms": st,
        "attention": {
            "tflops": fig["tflops"],
            "frac_mfma_peak": fig["tflops"] / PEAK_BF16_TFLOPS,
            "frac_gemm_probe": fig["tflops"] / peaks["gemm_bf16_tflops"],
            "kv_gbps": fig["kv_gbps"],
            "frac_hbm_peak": fig["kv_gbps"] / PEAK_HBM_GBPS,
            "frac_copy_probe": fig["kv_gbps"] / peaks["copy_gbps"],
        },
        "accept_len": res[0].cpu().tolist()[:8],
    }
    del v
    torch.cuda.empty_cache()
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; the library has no multi-GPU path, so --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe > 0:
        copy_probe(args.copy_probe, args.steps)
        return
    import torch
    from tree_causal_attention_amd import binding as B
    from tree_causal_attention_amd import workloads as WL

    w = WL.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    v = Verify(B, w, dev)
    ms_step, tree, res = v.run(args.steps, args.warmup)
    stage_ms = v.stage_ms()
    stage_pct = {"step": v.pct("s0", "s4"), "tree_attention": v.pct("s2", "s3")}

    # the same step with the 256 MB last-level cache and L2 flushed before each
    # step (an untimed 1 GiB write), timed step by step with events
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for k_ in v.ev:
        v.ev[k_].clear()
    for _ in range(args.steps):
        flush.fill_(1)
        v.step(True)
    torch.cuda.synchronize()
    flushed = {"step": v.pct("s0", "s4"), "tree_attention": v.pct("s2", "s3")}
    del flush
    fig = v.attention_figures(tree, stage_ms["tree_attention"])
    peaks = probes()
    achieved_tflops = fig["tflops"]
    tokens = fig["tokens"]
    result = {
        "metric": "tree-attn verify tree-node tok/s + KV GB/s at B=256; % of HBM/MFMA peak",
        "value": tokens / (ms_step / 1000.0),
        "unit": "tree-node tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded draws with the workload's shapes; no datasets or weights)",
        "config": {
            "workload": f"{w.name}: full verify step (build tree, tree meta, paged tree attention, "
                        f"accept), batch {w.batch}, prefix {w.prefix}, {w.hq}q/{w.hkv}kv heads, "
                        f"head_dim {w.head_dim}, B={w.budget_b}, W={w.width_w}, N={w.depth_n}, "
                        f"vocab {w.vocab}, page 16",
            "tree_nodes_per_step": tokens,
        },
        "roofline": {
            "kernel": "jt_tree_attention (tree_attn_mfma + tree_attn_combine)",
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(w.name),
            "algorithmic_flops": fig["flops"],
            "algorithmic_bytes": fig["kv_bytes"] + fig["qo_bytes"],
            "frac_gemm_probe": achieved_tflops / peaks["gemm_bf16_tflops"],
        },
        "kv_gbps": fig["kv_gbps"],
        "kv_hbm_frac": fig["kv_gbps"] / PEAK_HBM_GBPS,
        "kv_copy_probe_frac": fig["kv_gbps"] / peaks["copy_gbps"],
        "probes": peaks,
        "stage_ms": stage_ms,
        "stage_ms_pct": stage_pct,
        "flushed_ms_pct": flushed,
        "accept_len": res[0].cpu().tolist(),
    }
    result["next_rows"] = time_next_rows(B, w, v.x, tree, v.d_draft, v.d_target, v.d_k, v.d_v,
                                         v.d_prefix, v.d_table, v.d_root, v.ws_build, v.ws_acc,
                                         v.err, v.stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, v.x, min(args.cpu_seqs, w.batch))
    if not args.no_configs:
        del v
        torch.cuda.empty_cache()
        result["configs"] = {
            name: secondary_line(B, name, dev, args.config_steps, max(3, args.warmup // 2), peaks)
            for name in SECONDARY if name != w.name}
    print(json.dumps(result))


def time_next_rows(B, w, x, tree, d_draft, d_target, d_k, d_v, d_prefix, d_table, d_root,
                   ws_build, ws_acc, err, stream, iters=20):
    """Average device time (HIP events on the launch stream) of the calls that
    extend the verify step, on the same batch, after the timed region."""
    import numpy as np
    import torch
    dev = d_draft.device
    b, T = w.batch, w.max_nodes

    def timed(fn, before=None):
        fn()  # warm-up
        tot = 0.0
        for _ in range(iters):
            if before is not None:
                before()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / iters * 1000.0  # us

    par, tok, dep, nn = tree["parent"], tree["token"], tree["depth"], tree["n_nodes"]
    out = {}
    # margin acceptance: one pass over the target rows, like the greedy rule
    us = timed(lambda: B.jt_accept_margin(d_target, w.depth_n, par, tok, dep, nn, 0.5, 1.0,
                                          err=err, workspace=ws_acc))
    tb = b * T * w.vocab * 4
    out["accept_margin"] = {"us": us, "target_bytes": tb, "gbps": tb / us / 1e3,
                            "hbm_frac": tb / us / 1e3 / PEAK_HBM_GBPS}
    # stochastic verification at T = 1 with seeded uniforms, on the build's
    # top-W trees (point-mass proposals; mostly rejections on these
    # independent target rows), and the i.i.d.-proposal rule for comparison
    # (up to W residual passes per sequence)
    g = torch.Generator().manual_seed(17)
    ua = torch.rand((b, T), generator=g).to(dev)
    usamp = torch.rand((b,), generator=g).to(dev)
    out["accept_stochastic_us"] = timed(lambda: B.jt_accept_stochastic(
        d_target, w.depth_n, par, tok, dep, nn, 1.0, ua, usamp, err=err))
    out["accept_stochastic_sampled_us"] = timed(lambda: B.jt_accept_stochastic(
        d_target, w.depth_n, par, tok, dep, nn, 1.0, ua, usamp, draft_logits=d_draft,
        draft_mode="sampled", err=err))
    # KV commit of each tree's deepest path (prefix_len restored before each call)
    depth_h, par_h = dep.cpu().numpy(), par.cpu().numpy()
    anodes = np.full((b, w.depth_n), -1, dtype=np.int32)
    alen = np.zeros(b, dtype=np.int32)
    for s_ in range(b):
        v = int(np.argmax(depth_h[s_][:int(nn[s_])]))
        path = []
        while v > 0:
            path.append(v)
            v = int(par_h[s_][v])
        path.reverse()
        alen[s_] = len(path)
        anodes[s_, :len(path)] = path
    d_alen = torch.from_numpy(alen).to(dev)
    d_anodes = torch.from_numpy(anodes).to(dev)
    pref = d_prefix.clone()
    out["commit_kv_us"] = timed(
        lambda: B.jt_commit_kv(d_k, d_v, d_table, x.num_pages, nn, T, d_alen, d_anodes, pref,
                               parent=par, err=err),
        before=lambda: pref.copy_(d_prefix))
    out["commit_kv_rows"] = int(alen.sum())
    # build-mode variants (sequential best-first) next to the default build
    out["build_default_us"] = timed(lambda: B.jt_build_tree(d_draft, w.width_w, w.budget_b,
                                                            d_root, err=err, workspace=ws_build))
    out["build_node_block_us"] = timed(lambda: B.jt_build_tree_variant(
        d_draft, w.width_w, w.budget_b, d_root, "node_block", 0.0, err=err, workspace=ws_build))
    out["build_candidate_mixed_us"] = timed(lambda: B.jt_build_tree_variant(
        d_draft, w.width_w, w.budget_b, d_root, "candidate", 0.5, err=err, workspace=ws_build))
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error bits {int(err.item())} in the extension calls")
    return out


if __name__ == "__main__":
    main()
