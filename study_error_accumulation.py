"""Synthetic probe of quantisation-error accumulation in autoregressive decoding.

The pages ([HYPHO] section "论文的核心发现：推理场景的误差累积") state that in decoding every step
re-reads the whole KV cache, so a wrongly estimated token scale keeps perturbing every later step,
and that the joint row/column normalisation of KVarN removes most of that accumulation.  Without a
model or weights, this script builds a small seeded recurrence and runs it in lockstep:

    state x_t (1024 = 8 heads x 128, RMS-normalised)
    q_t = Wq x_t (8 query heads), k_t = (Wk x_t) * ch * tau_t, v_t = (Wv x_t) * ch' * tau'_t (1 kv head)
    o_t = attention(q_t, K_<=t, V_<=t)                      (8 heads x 128)
    x_{t+1} = rmsnorm(x_t + f Wo o_t + 0.5 eps_t)     (f = feedback gain)

with fixed outlier channels (ch: 4 channels x20, as in the synthetic KV generator) and log-normal
per-token scales tau_t = exp(0.5 n_t), all drawn from seeded streams shared by every run.  The
reference run keeps K/V in fp16 and attends in fp32 (plain PyTorch); each quantised run keeps the
same prefix quantised by kvarn_quantize_tiles and appends / decodes through kvarn_append_token and
kvarn_decode_attention.  "free" runs feed their own output back (errors can compound); "forced" runs
attend over a cache filled with the reference run's tokens and queries (one-step error only).
Sinkhorn iterations 0 (rotation + per-token RTN only) against 8 isolate the normalisation step.

Reports, per run, the relative L2 error of o_t and of x_t against the reference run at a few steps
(median over a window of 64 steps).  This is a toy recurrence, not a language model: it shows how the
kernels' error behaves under feedback, not task accuracy.
"""
import argparse
import json
import math
import sys

import numpy as np


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--prefix", type=int, default=2048, help="prefill tokens (multiple of 128)")
    p.add_argument("--steps", type=int, default=4096, help="decode steps")
    p.add_argument("--seeds", type=str, default="11,12,13")
    p.add_argument("--report", type=str, default="256,1024,2048,4096")
    p.add_argument("--feedback", type=float, default=0.02,
                   help="gain of the attention output in the state update (at 0.1 and above the fp16 recurrence "
                        "itself amplifies any perturbation, 8-bit included)")
    p.add_argument("--out", type=str, default="", help="also write the JSON summary to this file")
    return p.parse_args(argv)


def run(args, seed):
    import torch

    import kv_cache_quantization_pipeline_amd as kv

    assert args.prefix % 128 == 0 and args.prefix > 0
    dev = torch.device("cuda:0")
    D, HQ, HKV, DM = 128, 8, 1, 1024
    sm = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(seed)

    def mat(rows, cols):
        return torch.from_numpy((rng.standard_normal((rows, cols)) / math.sqrt(cols)).astype(np.float32)).to(dev)

    Wq, Wk, Wv, Wo = mat(HQ * D, DM), mat(D, DM), mat(D, DM), mat(DM, HQ * D)
    ch_k = np.ones(D, np.float32)
    ch_k[rng.choice(D, 4, replace=False)] = 20.0
    ch_v = np.ones(D, np.float32)
    ch_v[rng.choice(D, 4, replace=False)] = 20.0
    ch_k, ch_v = torch.from_numpy(ch_k).to(dev), torch.from_numpy(ch_v).to(dev)
    n_tok = args.prefix + args.steps
    tau_k = torch.from_numpy(np.exp(0.5 * rng.standard_normal(n_tok)).astype(np.float32)).to(dev)
    tau_v = torch.from_numpy(np.exp(0.5 * rng.standard_normal(n_tok)).astype(np.float32)).to(dev)
    eps = torch.from_numpy(rng.standard_normal((args.steps, DM)).astype(np.float32)).to(dev)

    def rmsnorm(x):
        return x / x.pow(2).mean().sqrt()

    # prefix: a trajectory of the recurrence without attention feedback, shared by every run
    x = rmsnorm(torch.from_numpy(rng.standard_normal(DM).astype(np.float32)).to(dev))
    pre_k, pre_v = [], []
    for t in range(args.prefix):
        pre_k.append(((Wk @ x) * ch_k * tau_k[t]).half())
        pre_v.append(((Wv @ x) * ch_v * tau_v[t]).half())
        x = rmsnorm(x + 0.5 * torch.from_numpy(rng.standard_normal(DM).astype(np.float32)).to(dev))
    x0 = x.clone()
    pre_k = torch.stack(pre_k)            # [prefix, 128] fp16
    pre_v = torch.stack(pre_v)

    def step_tokens(x, t):
        q = (Wq @ x).half().view(1, HQ, D)
        k = ((Wk @ x) * ch_k * tau_k[t]).half().view(1, HKV, D)
        v = ((Wv @ x) * ch_v * tau_v[t]).half().view(1, HKV, D)
        return q, k, v

    def advance(x, o, i):
        return rmsnorm(x + args.feedback * (Wo @ o.float().reshape(-1)) + 0.5 * eps[i])

    class Ref:
        def __init__(self):
            self.K = torch.zeros(n_tok, D, dtype=torch.float16, device=dev)
            self.V = torch.zeros_like(self.K)
            self.K[:args.prefix] = pre_k
            self.V[:args.prefix] = pre_v
            self.L = args.prefix
            self.x = x0.clone()

        def attend(self, q, k, v):
            self.K[self.L] = k[0, 0]
            self.V[self.L] = v[0, 0]
            self.L += 1
            K = self.K[:self.L].float().contiguous()
            V = self.V[:self.L].float().contiguous()
            qq = q[0].float()                                  # [HQ, D]
            s = (K @ qq.t().contiguous()) * sm                 # [L, HQ]
            p = torch.softmax(s, dim=0)
            return (p.t().contiguous() @ V).view(1, HQ, D)     # [1, HQ, D]

    class Quant:
        def __init__(self, name, iters):
            self.fmt = kv.format_parse(name)
            self.fmt.sinkhorn_iters = iters
            R = kv.record_bytes(self.fmt)
            self.stride = HKV * R
            self.maxp = n_tok // 128 + 1
            self.cache = torch.zeros(self.maxp * self.stride, dtype=torch.uint8, device=dev)
            self.pt = torch.arange(self.maxp, dtype=torch.int32, device=dev).view(1, -1).contiguous()
            npre = args.prefix // 128
            kv.quantize_tiles(self.fmt, pre_k.view(npre, 128, HKV, D).contiguous(),
                              pre_v.view(npre, 128, HKV, D).contiguous(), self.pt[0, :npre].contiguous(),
                              self.cache, self.stride)
            self.lens = torch.full((1,), args.prefix, dtype=torch.int32, device=dev)
            self.tk = torch.zeros(1, HKV, 128, D, dtype=torch.float16, device=dev)
            self.tv = torch.zeros_like(self.tk)
            self.ws = kv.decode_workspace(self.fmt, 1, HQ, HKV, self.maxp, dev)
            self.x = x0.clone()

        def attend(self, q, k, v):
            kv.append_token(self.fmt, k.contiguous(), v.contiguous(), self.lens, self.tk, self.tv, self.pt,
                            self.cache, self.stride)
            out = torch.empty(1, HQ, D, dtype=torch.float16, device=dev)
            kv.decode_attention(self.fmt, q.contiguous(), self.cache, self.stride, self.pt, self.lens, self.tk,
                                self.tv, sm, out, self.ws, HKV)
            return out

    configs = CONFIGS
    ref = Ref()
    free = [Quant(n, it) for n, it in configs]
    forced = [Quant(n, it) for n, it in configs]
    err_o = {("free",) + c: [] for c in configs}
    err_o.update({("forced",) + c: [] for c in configs})
    err_x = {("free",) + c: [] for c in configs}

    for i in range(args.steps):
        t = args.prefix + i
        q, k, v = step_tokens(ref.x, t)
        o_ref = ref.attend(q, k, v)
        for c, run in zip(configs, forced):
            o = run.attend(q, k, v)
            err_o[("forced",) + c].append(o.float() - o_ref.float())
        for c, run in zip(configs, free):
            qr, kr, vr = step_tokens(run.x, t)
            o = run.attend(qr, kr, vr)
            err_o[("free",) + c].append(o.float() - o_ref.float())
            run.x = advance(run.x, o, i)
        ref.x = advance(ref.x, o_ref.half(), i)
        if (i + 1) % 512 == 0:
            print(f"seed {seed}: step {i + 1} of {args.steps}", file=sys.stderr, flush=True)
        for c, run in zip(configs, free):
            err_x[("free",) + c].append(torch.linalg.vector_norm(run.x - ref.x) / torch.linalg.vector_norm(ref.x))
        # keep the reference outputs' norms next to the differences (relative error per step)
        ref_norm = torch.linalg.vector_norm(o_ref.float())
        for key in err_o:
            d = err_o[key][-1]
            err_o[key][-1] = torch.linalg.vector_norm(d) / ref_norm
    torch.cuda.synchronize()

    report = [int(s) for s in args.report.split(",") if int(s) <= args.steps]
    out = {}
    for key, series in err_o.items():
        e = torch.stack(series).cpu().numpy()
        ex = torch.stack(err_x[key]).cpu().numpy() if key in err_x else None
        row = {"o": [float(np.median(e[max(0, s - 64):s])) for s in report],
               "o_all": float(np.median(e[min(256, len(e) - 1):]))}
        if ex is not None:
            row["x"] = [float(np.median(ex[max(0, s - 64):s])) for s in report]
            row["x_all"] = float(np.median(ex[min(256, len(ex) - 1):]))
        out[key] = row
    return report, out


CONFIGS = [("kvarn_k4v2_g128", 8), ("kvarn_k4v2_g128", 0), ("kvarn_k8v8_g128", 8), ("kvarn_k4v8_g128", 8),
           ("kvarn_k8v2_g128", 8), ("kvarn_k2v2_g128", 8), ("kvarn_k2v2_g128", 0)]


def summarise(args, seeds, per_seed):
    """One row per (run, format, Sinkhorn iterations): each statistic averaged over the seeds."""
    report = per_seed[0][0]
    rows = []
    for key in per_seed[0][1]:
        rs = [ps[1][key] for ps in per_seed]
        row = {"run": key[0], "format": key[1], "sinkhorn_iters": key[2],
               "o_rel_l2": dict(zip(report, np.mean([r["o"] for r in rs], axis=0).tolist())),
               "o_rel_l2_steps_after_256": float(np.mean([r["o_all"] for r in rs]))}
        if "x" in rs[0]:
            row["x_rel_l2"] = dict(zip(report, np.mean([r["x"] for r in rs], axis=0).tolist()))
            row["x_rel_l2_steps_after_256"] = float(np.mean([r["x_all"] for r in rs]))
        rows.append(row)
    return {"study": "error accumulation (synthetic recurrence)", "prefix": args.prefix,
            "steps": args.steps, "seeds": seeds, "feedback": args.feedback, "q_heads": 8, "kv_heads": 1,
            "window": 64, "statistic": "median over the window (or over steps > 256), mean over seeds",
            "rows": rows}


def main(argv=None):
    args = parse(argv)
    seeds = [int(x) for x in args.seeds.split(",")]
    per_seed = [run(args, sd) for sd in seeds]
    summary = summarise(args, seeds, per_seed)
    print(json.dumps(summary), flush=True)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(summary, f, indent=1)
            f.write("\n")
    for r in summary["rows"]:
        o = " ".join(f"{v:.3e}" for v in r["o_rel_l2"].values())
        xx = " ".join(f"{v:.3e}" for v in r.get("x_rel_l2", {}).values())
        print(f"{r['run']:6s} {r['format']:16s} it={r['sinkhorn_iters']}  o: {o} | all {r['o_rel_l2_steps_after_256']:.3e}"
              f"   x: {xx} | all {r.get('x_rel_l2_steps_after_256', float('nan')):.3e}", file=sys.stderr)
    return summary


if __name__ == "__main__":
    main()
