"""ISD step benchmark on one MI355X.

One step = the whole hot path over one batch of 64 requests at stride N=4 (7 query rows
each), on synthetic inputs already resident in HBM:
  1. R-ISD gated projection  448 x 4096 -> 4096, rank-128 delta on the 4 [MASK] rows
  2. attention               Qwen3-8B shapes (32 q / 8 kv heads, D=128), contexts ~ U[512,4096]
  3. verification            vocab 151936, anchor ~ N(0,3), proposal = anchor + N(0,0.3)
Prints ONE JSON line: ISD steps/s (value), accepted tokens/s, per-kernel times, the
attention kernel against the HBM roofline, and the CPU oracle on a bounded sample.

The attention stream (~600 MB) exceeds the 256 MB last-level cache, so every kernel of a
step starts cold with respect to the previous step's data.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ISD steps/s and accepted tokens/s at N=4, C=64 (1 GPU); % HBM roofline"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--verify-sets", type=int, default=3,
                    help="distinct seeded verification inputs rotated over the steps")
    ap.add_argument("--proj-sets", type=int, default=12,
                    help="distinct seeded projection inputs (activations and weights) rotated over "
                         "the steps, so that every step reads its weights from HBM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--proj-row-major", action="store_true",
                    help="run the projection on row-major weights instead of the packed layout")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager steps instead of HIP-graph replays of the same steps")
    ap.add_argument("--steps-per-graph", type=int, default=0,
                    help="consecutive steps captured in one HIP graph (default: the least common "
                         "multiple of the verification and projection set counts, so each graph holds "
                         "every set); 1 replays one graph per step")
    ap.add_argument("--workload", choices=["qwen3_8b", "qwen3_32b"], default="qwen3_8b")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="concurrency sweep instead of the single benchmark line: one JSON line "
                         "per (N, C) point, contexts fixed at 2048, inputs generated on the device")
    ap.add_argument("--sweep-c", default="1,4,16,64,128,256")
    ap.add_argument("--closed-loop", action="store_true",
                    help="closed decoding loop on the device instead of the single benchmark line")
    ap.add_argument("--layer", action="store_true",
                    help="R-ISD decoder layer (Qwen3-8B shapes): gated against base-only time")
    ap.add_argument("--sweep-n", default="2,3,4")
    ap.add_argument("--sweep-p", default="0.9,0.5",
                    help="acceptance targets of the sweep (proposal noise bisected on the oracle)")
    ap.add_argument("--lm-head", action="store_true",
                    help="the LM head fused with verification (Qwen3-8B shapes) against the unfused pair")
    return ap.parse_args()


def tpf_closed_form(N, p):
    """Tokens per forward of ISD at acceptance rate p (「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor Explorer")."""
    return (2 + sum(p ** k for k in range(1, N - 1))) / (2 - p ** (N - 1))


def attention_bytes(ctx_lens, R, Hq, Hkv, D, s=2):
    """Algorithmic bytes of one attention launch: K and V of every token read once
    (cached tokens and the block), the block's K/V written to the cache, Q read, O written,
    and the page-table entries used."""
    L = np.asarray(ctx_lens, np.int64)
    kv_read = int(np.sum(L + R)) * Hkv * D * 2 * s
    append = len(L) * R * Hkv * D * 2 * s
    qo = 2 * len(L) * R * Hq * D * s
    pages = int(np.sum((L + R + 15) // 16)) * 4
    return kv_read + append + qo + pages


def verify_bytes(B, N, V, n_rejected_sampled, s=2):
    """Logit rows + draft rows once, the two rows of each rejected request once more,
    one 1024-entry sub-chunk per sampled row."""
    R = 2 * N - 1
    return B * R * V * s + B * (N - 1) * V * s + n_rejected_sampled * 2 * V * s + B * N * 1024 * s


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              f"(requests shard by data parallelism with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.closed_loop:
        closed_loop(args)
        return
    if args.layer:
        layer_alpha(args)
        return
    if args.lm_head:
        lm_head_bench(args)
        return
    import torch

    from strided_verify_propose_amd import isd, synth
    from strided_verify_propose_amd.profsum import read_attention_traffic, read_mfma

    dev = torch.device("cuda:0")

    def dt(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    scfg = synth.QWEN3_8B if args.workload == "qwen3_8b" else synth.QWEN3_32B
    pcfg = synth.PROJ
    t0 = time.time()
    # ---- inputs (seeded, generated on the host once, then resident in HBM)
    att = synth.attention_inputs(scfg)
    maxctx = int(att.ctx_lens.max())
    vsets = []
    vsets_host = []
    ver0 = None
    for k in range(args.verify_sets):
        v = synth.verify_inputs(scfg, seed=scfg.seed + 100 * k)
        ver0 = v if ver0 is None else ver0
        vsets_host.append(v)
    pin = synth.proj_inputs(pcfg)
    pool = None
    if not args.no_cpu_baseline:
        # worker processes for the all-core oracle baseline, forked now -- before anything
        # touches the GPU -- so they inherit the host inputs and never share GPU state
        pool = oracle_pool(att, ver0, pin, scfg)
    torch.cuda.set_device(dev)
    A = dict(q=dt(att.q), k_new=dt(att.k_new), v_new=dt(att.v_new),
             k_cache=dt(synth.k_tile_layout(att.k_pages)), v_cache=dt(synth.v_tile_layout(att.v_pages)),
             page_table=dt(att.page_table), ctx_lens=dt(att.ctx_lens))
    for v in vsets_host:
        vsets.append(dict(logits=dt(v.logits), draft_logits=dt(v.draft_logits),
                          draft_ids=dt(v.draft_ids), uniforms=dt(v.uniforms)))
    P = dict(x=dt(pin.x), w=dt(pin.w), a=dt(pin.a), b=dt(pin.b), gate=dt(pin.gate))
    # weights are packed once, outside the timed region, as a serving system would at load
    packed = None if args.proj_row_major else isd.pack_proj_weights(P["w"], P["a"], P["b"])
    # the projection's input sets: the seeded host set first, then sets drawn on the device
    # with the same shapes and distributions (x ~ N(0, 1); w, a, b ~ N(0, w_sd)).  A step
    # takes set i mod proj_sets: between two uses of a set the other sets' 480 MB and more
    # pass through the 256 MB last-level cache, as the other layers' weights do in a model
    # (the attention pages and the logits are read non-temporally and do not evict them).
    psets = [dict(x=P["x"], w=P["w"], a=P["a"], b=P["b"], packed=packed)]
    pg = torch.Generator(device=dev)
    pg.manual_seed(pcfg.seed + 1)
    for _ in range(1, max(1, args.proj_sets)):
        ps = dict(x=torch.randn((pcfg.M, pcfg.K), generator=pg, device=dev).to(torch.bfloat16),
                  w=(torch.randn((pcfg.Nout, pcfg.K), generator=pg, device=dev) * pcfg.w_sd).to(torch.bfloat16),
                  a=(torch.randn((pcfg.r, pcfg.K), generator=pg, device=dev) * pcfg.w_sd).to(torch.bfloat16),
                  b=(torch.randn((pcfg.Nout, pcfg.r), generator=pg, device=dev) * pcfg.w_sd).to(torch.bfloat16))
        if not args.proj_row_major:
            ps["packed"] = isd.pack_proj_weights(ps["w"], ps["a"], ps["b"])
            del ps["w"], ps["a"], ps["b"]
        psets.append(ps)
    gen_s = time.time() - t0

    att_out = torch.empty_like(A["q"])
    y = torch.empty((pcfg.M, pcfg.Nout), dtype=torch.bfloat16, device=dev)
    vouts = [None] * len(vsets)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        ps = psets[i % len(psets)]
        if packed is None:
            isd.gated_lora_proj(ps["x"], ps["w"], ps["a"], ps["b"], P["gate"], out=y)
        else:
            isd.gated_lora_proj_packed(ps["x"], ps["packed"], P["gate"], out=y)
        if ev is not None:
            ev[1].record()
        isd.attention_step(A["q"], A["k_new"], A["v_new"], A["k_cache"], A["v_cache"],
                           A["page_table"], A["ctx_lens"], maxctx, out=att_out)
        if ev is not None:
            ev[2].record()
        k = i % len(vsets)
        vs = vsets[k]
        vouts[k] = isd.verify(vs["logits"], vs["draft_logits"], vs["draft_ids"], vs["uniforms"],
                              with_diagnostics=False, out=vouts[k])
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- per-call times: eager steps with events around each call on the launch stream
    n_ev = min(args.steps, 100)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    t_ev = time.perf_counter()
    for i in range(n_ev):
        step(i, evs[i])
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t_ev) / n_ev
    proj_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    att_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ver_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    # ---- timed region: K whole steps, replayed from HIP graphs holding the same launches
    # as the eager step, so the steps run back to back without host launch gaps;
    # --no-graph times the eager steps instead.
    # A graph launch costs the GPU some 20 us between graphs, so G consecutive steps go into
    # one graph (by default one period of the input rotation: every verification and every
    # projection set once); the steps past a multiple of G replay one-step graphs.  Every
    # step runs the same launches either way.
    graphs = []
    multi = None
    period = math.lcm(len(vsets), len(psets))
    G = args.steps_per_graph or period
    if not args.no_graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for k in range(period):
                step(k)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for k in range(period):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        if G > 1:
            multi = torch.cuda.CUDAGraph()
            with torch.cuda.graph(multi):
                for k in range(G):
                    step(k)
            multi.replay()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if multi is not None:
        for _ in range(args.steps // G):
            multi.replay()
        for i in range(args.steps % G):
            graphs[i % len(graphs)].replay()
    else:
        for i in range(args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    # ---- acceptance statistics from the kernel's own outputs
    n_acc = np.concatenate([vouts[k]["n_accept"].cpu().numpy() for k in range(len(vsets))])
    N = scfg.N
    rej = n_acc < N - 1
    tpf_hat = float((np.mean(n_acc + 1) + rej.mean()) / (1 + rej.mean()))
    evaluated = np.sum(n_acc + rej)
    p_hat = float(np.sum(n_acc) / evaluated)
    steps_per_s = args.steps / elapsed
    ms_per_step = 1e3 * elapsed / args.steps

    a_bytes = attention_bytes(att.ctx_lens, scfg.R, scfg.Hq, scfg.Hkv, scfg.D)
    # the attention step (its two kernels), timed with events on the launch stream
    a_us = float(np.mean(att_ms)) * 1e3
    traffic = read_attention_traffic(os.path.join(ROOT, "profiles", f"attention_step_{scfg.name}_hbm.txt"))
    a_gbps = a_bytes / (a_us * 1e-6) / 1e9
    v_bytes = verify_bytes(scfg.B, N, scfg.V, int(rej.sum() / len(vsets)))
    v_us = float(np.mean(ver_ms)) * 1e3
    m_g = int(pin.gate.sum())
    p_flops = 2 * pcfg.M * pcfg.K * pcfg.Nout + 2 * m_g * pcfg.K * pcfg.r + 2 * m_g * pcfg.r * pcfg.Nout
    p_us = float(np.mean(proj_ms)) * 1e3

    # the projection alone: back to back on one input set (weights warm in the last-level
    # cache) and rotated over PROJ_SETS sets of activations and packed weights (cold), with
    # hipBLASLt's time for the base product (torch.nn.functional.linear) as a reference
    proj_alone = projection_alone(P, packed, pcfg, m_g, dev)
    carried_q = verify_carried(vsets, vouts, N, dev)

    # measured device copy ceiling: a 512 MiB device-to-device copy, timed with events
    src = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * 5 * (1 << 29) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    ceilings = attainable_bandwidth(dev)
    kv_sweep = kv_read_sweep_rate(A, att, scfg, maxctx, a_us, dev)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"isd_step_{scfg.name}_plus_rlora_proj",
            "batch": scfg.B, "stride_N": N, "query_rows": scfg.R, "q_heads": scfg.Hq,
            "kv_heads": scfg.Hkv, "head_dim": scfg.D, "page_size": 16,
            "context": f"U[{scfg.ctx[1]},{scfg.ctx[2]}]" if scfg.ctx[0] == "uniform" else scfg.ctx[1],
            "vocab": scfg.V, "proj": f"{pcfg.M}x{pcfg.K}->{pcfg.Nout} r{pcfg.r}",
            "proj_weights": "row-major" if packed is None else "packed (MFMA fragment order)",
            "verify_input_sets": len(vsets),
            "proj_input_sets": len(psets),
            "seeds": {"attention": scfg.seed, "verify": [scfg.seed + 100 * k for k in range(len(vsets))],
                      "proj": pcfg.seed,
                      "proj_device_sets": f"torch.Generator(cuda).manual_seed({pcfg.seed + 1})"},
        },
        "accepted_tokens_per_s": round(steps_per_s * scfg.B * tpf_hat, 1),
        "hot_tokens_per_step": round(float(np.mean(n_acc + 1)) * scfg.B, 2),
        "tpf_meas": round(tpf_hat, 4),
        "p_hat": round(p_hat, 4),
        "tpf_closed_form_at_p_hat": round(tpf_closed_form(N, p_hat), 4),
        "kernels_us": {"gated_lora_proj": round(p_us, 2), "attention": round(a_us, 2),
                       "verify": round(v_us, 2)},
        "kernels_us_p10_p50_p90": {k: [round(float(np.percentile(x, q)) * 1e3, 2) for q in (10, 50, 90)]
                                   for k, x in (("gated_lora_proj", proj_ms), ("attention", att_ms),
                                                ("verify", ver_ms))},
        "device_copy_GBps": round(copy_gbps, 1),
        "attainable_GBps": ceilings,
        "kv_read_sweep": kv_sweep,
        "verify_hbm_frac": round(v_bytes / (v_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "proj_mfma_frac": round(p_flops / (p_us * 1e-6) / 2.5e15, 4),
        "proj_alone": proj_alone,
        "verify_with_carried_q_stats": carried_q,
        # MFMA busy share and bf16 flops from rocprofv3 counters (profiles/), when they were
        # taken on the current projection sources
        "proj_mfma_counters": read_mfma(os.path.join(ROOT, "profiles", f"isd_step_{scfg.name}_mfma.txt"),
                                        ("base_kernel_packed", "lora_kernel")),
        "roofline": {"bound": "hbm",
                     "kernel": "isd_attention_step (attn_bf16_kernel + attn_combine_kernel)",
                     "achieved": round(a_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(a_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": a_bytes,
                     "traffic_ratio": None if traffic is None else round(traffic / a_bytes, 4)},
        "timing": ((f"hip graph replay of whole steps, {G} per graph" if multi is not None
                    else "hip graph replay of whole steps, one per graph") if graphs else "eager launches"),
        "eager_ms_per_step": round(1e3 * eager_s, 4),
        "input_generation_s": round(gen_s, 1),
    }
    # the timed verification outputs against the oracle, draw by draw (the oracle runs on
    # the host here; its time is not part of any figure)
    line["verify_parity"] = verify_parity_counts(vsets_host, vouts, scfg.N)
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(scfg, att, ver0, pin, pool)
        line["cpu_host"] = cpu_host_info(pool)
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------- concurrency sweep
def sweep(args):
    """Steps/s and tokens/s of the whole step against the number of concurrent requests C
    (one request = one 2N-1 row block), for each stride N and acceptance target (0.9 and
    0.5, the proposal noise calibrated on the oracle): where the block stops being
    memory-bound.  Qwen3-8B attention shapes with every context at 2048 tokens, the
    151936-entry vocabulary, the 4096 x 4096 r128 projection on C (2N-1) rows with the
    [MASK] rows gated.  Inputs are drawn on the device (torch generator seeded per point),
    the verification inputs in four rotated sets and the projection weights in twelve;
    each point times 48 steps replayed from one HIP graph holding one period of that
    rotation, after an eager pass that times each call with events."""
    import torch

    from strided_verify_propose_amd import isd
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Hq, Hkv, D, V, L, PAGE = 32, 8, 128, 151936, 2048, 16
    K, Nout, r = 4096, 4096, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(1300)
    # PROJ_SETS weight sets rotated over the steps, so that the projection reads its
    # weights from HBM every step, as in a model whose other layers' weights pass between
    # two uses (the attention pages and the logits are read non-temporally and would not
    # evict a single set)
    packs = []
    for _ in range(PROJ_SETS):
        w = (torch.randn((Nout, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        a = (torch.randn((r, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        b = (torch.randn((Nout, r), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        packs.append(isd.pack_proj_weights(w, a, b))
        del w, a, b
    from strided_verify_propose_amd import synth
    Cs = [int(c) for c in args.sweep_c.split(",")]
    Ns = [int(n) for n in args.sweep_n.split(",")]
    Ps = [float(p) for p in args.sweep_p.split(",")]
    for pi, (p_target, N, C) in enumerate([(p, n, c) for p in Ps for n in Ns for c in Cs]):
        sigma = synth.SWEEP_SIGMA[p_target]
        gen.manual_seed(1400 + pi)
        R = 2 * N - 1
        bf = torch.bfloat16

        def randn(*shape, sd=1.0):
            return torch.randn(shape, generator=gen, device=dev) * sd

        npg = (L + R + PAGE - 1) // PAGE
        perm = torch.randperm(C * npg, generator=gen, device=dev).to(torch.int32)
        A = dict(q=randn(C, R, Hq, D).to(bf), k_new=randn(C, R, Hkv, D).to(bf), v_new=randn(C, R, Hkv, D).to(bf),
                 k_cache=randn(C * npg, Hkv, D // 8, PAGE, 8).to(bf),
                 v_cache=randn(C * npg, Hkv, D // 16, 4, PAGE, 4).to(bf),
                 page_table=perm.view(C, npg).contiguous(),
                 ctx_lens=torch.full((C,), L, dtype=torch.int32, device=dev))
        vsets = []
        for _ in range(4):
            anchor = randn(C, R, V, sd=3.0)
            prop = anchor + randn(C, R, V, sd=sigma)
            logits = torch.cat([anchor[:, :N - 1], prop[:, N - 1:]], dim=1).to(bf).contiguous()
            draft = prop[:, :N - 1].to(bf).contiguous()
            del anchor, prop
            u01 = torch.rand(draft.shape, generator=gen, device=dev, dtype=torch.float64)
            ids = torch.argmax(draft.double() - torch.log(-torch.log(u01)), dim=-1).to(torch.int32).contiguous()
            del u01
            u = (torch.randint(0, 1 << 24, (C, R), generator=gen, device=dev) / float(1 << 24)).to(torch.float32)
            vsets.append((logits, draft, ids, u))
        M = C * R
        x = randn(M, K).to(bf)
        gate = torch.tensor(([0] * (N - 1) + [1] * N) * C, dtype=torch.uint8, device=dev)
        y = torch.empty((M, Nout), dtype=bf, device=dev)
        att_out = torch.empty_like(A["q"])
        vouts = [None] * len(vsets)

        def step(i, ev=None):
            if ev is not None:
                ev[0].record()
            isd.gated_lora_proj_packed(x, packs[i % len(packs)], gate, out=y)
            if ev is not None:
                ev[1].record()
            isd.attention_step(A["q"], A["k_new"], A["v_new"], A["k_cache"], A["v_cache"],
                               A["page_table"], A["ctx_lens"], L, out=att_out)
            if ev is not None:
                ev[2].record()
            k = i % len(vsets)
            vouts[k] = isd.verify(*vsets[k], with_diagnostics=False, out=vouts[k])
            if ev is not None:
                ev[3].record()

        for i in range(8):
            step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(20)]
        for i, e in enumerate(evs):
            step(i, e)
        torch.cuda.synchronize()
        us = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3 for j in range(3)]
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for k in range(len(vsets)):
                step(k)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        # one graph holds one period of the rotation, every verification and projection
        # set in turn (a graph launch costs the GPU some 20 us, a large share of a step at
        # small C)
        G = math.lcm(len(vsets), len(packs))
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi):
            for k in range(G):
                step(k)
        steps = 4 * G
        multi.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // G):
            multi.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        n_acc = np.concatenate([vo["n_accept"].cpu().numpy() for vo in vouts])
        rej = n_acc < N - 1
        p_hat = float(np.sum(n_acc) / max(1, np.sum(n_acc + rej))) if N > 1 else 1.0
        tpf = tpf_closed_form(N, p_hat) if N > 1 else 1.0
        sps = steps / el
        a_bytes = attention_bytes(np.full(C, L), R, Hq, Hkv, D)
        v_bytes = verify_bytes(C, N, V, int(rej.sum() / len(vsets)))
        p_flops = 2 * M * K * Nout + 2 * (C * N) * K * r + 2 * (C * N) * r * Nout
        print(json.dumps({
            "sweep": "concurrency", "stride_N": N, "C": C, "context": L, "query_rows": R,
            "acceptance_target": p_target, "proposal_noise_sd": sigma,
            "ms_per_step": round(1e3 * el / steps, 4), "steps_per_s": round(sps, 1),
            "tokens_per_s": round(sps * C * tpf, 1), "p_hat": round(p_hat, 4),
            "tpf_closed_form_at_p_hat": round(tpf, 4),
            "us": {"gated_lora_proj": round(us[0], 2), "attention": round(us[1], 2), "verify": round(us[2], 2)},
            "attention_hbm_frac": round(a_bytes / (us[1] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "verify_hbm_frac": round(v_bytes / (us[2] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "proj_mfma_frac": round(p_flops / (us[0] * 1e-6) / 2.5e15, 4),
            "timing": f"hip graph replay of whole steps, {G} per graph; per-call times from an eager pass",
            "data": "synthetic"}), flush=True)
        del A, vsets, vouts, multi, x, y, att_out
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- closed loop
def closed_loop(args):
    """Closed-loop decoding of the benchmark workload (64 requests, N = 4, contexts from
    U[512, 4096], the projection on the block's rows): each step's outputs feed the next
    step on the device (contexts, drafts, draft rows), one HIP graph per step replayed
    `--steps` times.  Reports the tokens kept per forward against the closed form at the
    measured acceptance rate, the hot path's time per step (events around the library's
    calls in an eager pass), the synthetic model's time apart, and graph against eager
    launch.  One JSON line."""
    import torch

    from strided_verify_propose_amd.loop import ClosedLoop, LoopConfig
    steps = max(args.steps, 20)
    cfg = LoopConfig(B=64, N=4, steps=steps + 40 + args.warmup)
    lp = ClosedLoop(cfg)
    for _ in range(args.warmup):
        lp.step()
    torch.cuda.synchronize()
    # eager pass: events around the model, the hot path's calls and the bookkeeping
    n_ev = 20
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(n_ev)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        lp.model()
        lp.hot_path(e[1:6])
        lp.keep_draft_rows()
        e[6].record()
    torch.cuda.synchronize()
    eager_ms = 1e3 * (time.perf_counter() - t0) / n_ev
    seg = lambda i, j: float(np.mean([e[i].elapsed_time(e[j]) for e in evs])) * 1e3
    model_us = seg(0, 1) + seg(5, 6)
    proj_us, att_us, ver_us, commit_us = seg(1, 2), seg(2, 3), seg(3, 4), seg(4, 5)
    hot_us = seg(1, 5)
    # reset the totals, then time graph replays
    for t in (lp.kept, lp.accepted, lp.evaluated, lp.hot_steps):
        t.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lp.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    if hasattr(g, "register_generator_state"):
        g.register_generator_state(lp.gen)
    with torch.cuda.graph(g):
        lp.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = lp.stats(steps + 2)     # the capture-stream step and the captured step ran too
    tpf = st["tpf_meas"]
    print(json.dumps({
        "closed_loop": "isd_qwen3_8b_b64_n4", "steps": steps, "data": "synthetic",
        "q_stats_carried": bool(cfg.carry_q_stats),
        "graph_ms_per_step": round(1e3 * el / steps, 4), "eager_ms_per_step": round(eager_ms, 4),
        "hot_path_us": {"gated_lora_proj": round(proj_us, 2), "attention": round(att_us, 2),
                        "verify": round(ver_us, 2), "commit": round(commit_us, 2), "total": round(hot_us, 2)},
        "synthetic_model_and_tallies_us": round(model_us, 2),
        "tpf_meas": round(tpf, 4), "tpf_se": round(st["tpf_se"], 4), "p_hat": round(st["p_hat"], 4),
        "tpf_closed_form_at_p_hat": round(st["tpf_closed_form_at_p_hat"], 4),
        "kept_tokens_per_s_hot_path": round(cfg.B * tpf / (hot_us * 1e-6), 1),
        "kept_tokens_per_s_with_model": round(cfg.B * tpf * steps / el, 1),
    }), flush=True)


# ---------------------------------------------------------------- R-ISD layer
def layer_alpha(args):
    """The R-ISD overhead alpha at the scale of a decoder layer: one Qwen3-8B-shaped layer
    (seven linears with rank-128 deltas on the gated rows, attention over contexts from
    U[512, 4096]) on 64 requests x 7 rows, gated against base-only, each as a HIP graph
    replayed `--steps` times; the linears are timed one by one with events."""
    import torch

    from strided_verify_propose_amd import isd
    from strided_verify_propose_amd.layer import LayerConfig, RIsdLayer
    lay = RIsdLayer(LayerConfig())
    res = {}
    for gated in (False, True):
        for _ in range(3):
            lay.forward(gated)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            lay.forward(gated)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward(gated)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        res[gated] = 1e6 * (time.perf_counter() - t0) / args.steps
        del g
    per = {}
    gate = lay.gate
    for name, pk in lay.packed.items():
        x = torch.randn((lay.M, pk.K), device="cuda").to(torch.bfloat16)
        us = []
        for gt in (None, gate):
            for _ in range(3):
                isd.gated_lora_proj_packed(x, pk, gt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                isd.gated_lora_proj_packed(x, pk, gt)
            e1.record()
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) / 20 * 1e3)
        per[name] = {"K": pk.K, "Nout": pk.Nout, "base_us": round(us[0], 2), "gated_us": round(us[1], 2)}
    print(json.dumps({"layer": "r_isd_qwen3_8b_b64_n4", "rows": lay.M, "rank": lay.cfg.r, "data": "synthetic",
                      "base_only_us": round(res[False], 2), "gated_us": round(res[True], 2),
                      "alpha": round(res[True] / res[False], 4), "linears": per,
                      "timing": "hip graph replay of the layer; linears with events (warm weights)"}), flush=True)


def lm_head_bench(args):
    """The LM head in front of verification at Qwen3-8B's shapes: 64 requests x 7 rows,
    hidden 4096, vocabulary 151936 (hidden ~ N(0,1), weights ~ N(0, 3/64), so logits have
    sd ~3); --workload qwen3_32b takes hidden 5120.  The previous step's proposal rows
    stand in as the verify rows' own logits plus N(0, 0.3) noise, with drafts drawn from
    them by the Gumbel-max trick, so acceptance is that of the verification workload.
    Times, with events over --steps calls each: the LM head alone, the LM head then
    verification, and the fused call."""
    import torch

    from strided_verify_propose_amd import isd, synth
    cfg = synth.LM_HEAD_32B if args.workload == "qwen3_32b" else synth.LM_HEAD_8B
    B, N, R, Dm, V = cfg.B, cfg.N, cfg.R, cfg.Dm, cfg.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    h = torch.randn((cfg.M, Dm), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((V, Dm), generator=g, device=dev) * cfg.w_sd).to(torch.bfloat16)
    logits = isd.lm_head(h, w).view(B, R, V)
    draft = (logits[:, :N - 1].float() + 0.3 * torch.randn((B, N - 1, V), generator=g, device=dev))
    gum = -torch.log(-torch.log(torch.rand(draft.shape, generator=g, device=dev).clamp_min(1e-30)))
    ids = torch.argmax(draft + gum, dim=-1).to(torch.int32).contiguous()
    draft = draft.to(torch.bfloat16).contiguous()
    del gum
    u = (torch.randint(0, 1 << 24, (B, R), generator=g, device=dev).float() / float(1 << 24)).contiguous()
    torch.cuda.synchronize()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3

    out_l = torch.empty((cfg.M, V), dtype=torch.bfloat16, device=dev)
    t_head = timed(lambda: isd.lm_head(h, w, out=out_l))
    vout = {}

    def unfused():
        isd.lm_head(h, w, out=out_l)
        vout["r"] = isd.verify(out_l.view(B, R, V), draft, ids, u, with_diagnostics=False,
                               out=vout.get("r"))
    t_unfused = timed(unfused)
    fout = {}

    def fused():
        fout["r"] = isd.lm_head_verify(h, w, draft, ids, u, with_diagnostics=False, out=fout.get("r"))
    t_fused = timed(fused)
    # reference only: the vendor GEMM (hipBLASLt through torch) on the same product
    t_lib = timed(lambda: torch.nn.functional.linear(h, w))
    if args.copy_calibration:  # a 1 GiB device copy for the HBM counters' scale
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    n_acc = fout["r"]["n_accept"].float().mean().item()
    flops = 2.0 * cfg.M * Dm * V
    w_bytes = V * Dm * 2
    print(json.dumps({
        "lm_head": cfg.name, "rows": cfg.M, "hidden": Dm, "vocab": V, "data": "synthetic",
        "steps": args.steps, "lm_head_us": round(t_head, 2), "lm_head_then_verify_us": round(t_unfused, 2),
        "fused_us": round(t_fused, 2), "fusion_saving_us": round(t_unfused - t_fused, 2),
        "lm_head_tflops": round(flops / (t_head * 1e-6) / 1e12, 1),
        "lm_head_mfma_frac": round(flops / (t_head * 1e-6) / 2.5e15, 4),
        "lm_head_weight_GBps": round(w_bytes / (t_head * 1e-6) / 1e9, 1),
        "reference_torch_linear_us": round(t_lib, 2),
        "mean_n_accept": round(n_acc, 3),
        "timing": f"events around --steps back-to-back calls (weights {w_bytes / 1e9:.2f} GB, streamed "
                  f"from HBM each call)"}),
        flush=True)


# ---------------------------------------------------------------- helpers of the main bench
PROJ_SETS = 12   # rotated activation + weight sets for the cold projection timing


def verify_carried(vsets, vouts, N, dev, reps=30):
    """Verification of the same input sets with the draft rows' statistics carried from
    the previous step (isd_verify_carry), as a decoding loop runs it: the statistics come
    from a real call on a previous step whose rows N..2N-2 are this set's draft rows, made
    before the timing; the timed calls also hand their own on.  Eager calls with events on
    the launch stream.  Context beside the main line, which reduces every row itself."""
    import torch
    from strided_verify_propose_amd import isd
    B, R, V = vsets[0]["logits"].shape
    nb = isd.verify_carry_bytes(B, N, V)
    if nb == 0 or vsets[0]["draft_logits"] is None:
        return None
    carried, nxt = [], torch.empty(nb, dtype=torch.uint8, device=dev)
    for vs in vsets:
        prev = vs["logits"].clone()
        prev[:, N:] = vs["draft_logits"]
        q = torch.empty(nb, dtype=torch.uint8, device=dev)
        isd.verify(prev, vs["draft_logits"], vs["draft_ids"], vs["uniforms"], with_diagnostics=False,
                   q_stats_next=q)
        carried.append(q)
        del prev
    outs = [None] * len(vsets)
    for k, vs in enumerate(vsets):   # warm-up, and the outputs to compare
        outs[k] = isd.verify(vs["logits"], vs["draft_logits"], vs["draft_ids"], vs["uniforms"],
                             with_diagnostics=False, q_stats_prev=carried[k], q_stats_next=nxt)
    torch.cuda.synchronize()
    same = all(torch.equal(outs[k][n], vouts[k][n]) for k in range(len(vsets)) for n in vouts[k])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(evs):
        k = i % len(vsets)
        vs = vsets[k]
        e0.record()
        isd.verify(vs["logits"], vs["draft_logits"], vs["draft_ids"], vs["uniforms"], with_diagnostics=False,
                   out=outs[k], q_stats_prev=carried[k], q_stats_next=nxt)
        e1.record()
    torch.cuda.synchronize()
    us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
    return {"verify_us": round(us, 2), "outputs_identical_to_verify": bool(same), "calls": reps}


def projection_alone(P, packed, pcfg, m_g, dev, reps=48):
    """The R-ISD projection alone: back to back on one input set (the 43 MB of operands
    stay in the 256 MB last-level cache: warm) and rotated over PROJ_SETS sets of
    activations and packed weights (cold), HIP events around `reps` calls each.  The
    base product through hipBLASLt (torch.nn.functional.linear, 448 x 4096 -> 4096, no
    delta) is timed the same two ways as a reference."""
    import torch

    from strided_verify_propose_amd import isd
    M, K, Nout, r = pcfg.M, pcfg.K, pcfg.Nout, pcfg.r
    flops = 2 * M * K * Nout + 2 * m_g * K * r + 2 * m_g * r * Nout
    g = torch.Generator(device=dev)
    g.manual_seed(pcfg.seed + 7)
    sets = []
    for _ in range(PROJ_SETS):
        x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        w = (torch.randn((Nout, K), generator=g, device=dev) * pcfg.w_sd).to(torch.bfloat16)
        a = (torch.randn((r, K), generator=g, device=dev) * pcfg.w_sd).to(torch.bfloat16)
        b = (torch.randn((Nout, r), generator=g, device=dev) * pcfg.w_sd).to(torch.bfloat16)
        sets.append((x, w, isd.pack_proj_weights(w, a, b)))
        del a, b
    y = torch.empty((M, Nout), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for i in range(4):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    gate = P["gate"]
    warm = timed(lambda i: isd.gated_lora_proj_packed(P["x"], packed, gate, out=y))
    cold = timed(lambda i: isd.gated_lora_proj_packed(sets[i % PROJ_SETS][0], sets[i % PROJ_SETS][2], gate, out=y))
    lib_warm = timed(lambda i: torch.nn.functional.linear(P["x"], P["w"]))
    lib_cold = timed(lambda i: torch.nn.functional.linear(sets[i % PROJ_SETS][0], sets[i % PROJ_SETS][1]))
    del sets
    torch.cuda.empty_cache()
    frac = lambda us, f: round(f / (us * 1e-6) / 2.5e15, 4)
    base_flops = 2 * M * K * Nout
    return {"gated_warm_us": round(warm, 2), "gated_cold_us": round(cold, 2),
            "mfma_frac_warm": frac(warm, flops), "mfma_frac_cold": frac(cold, flops),
            "rotated_sets": PROJ_SETS, "alg_flops": flops,
            "reference_hipblaslt_base_only_warm_us": round(lib_warm, 2),
            "reference_hipblaslt_base_only_cold_us": round(lib_cold, 2),
            "reference_hipblaslt_mfma_frac_cold": frac(lib_cold, base_flops)}


def kv_read_sweep_rate(A, att, scfg, maxctx, a_us, dev, reps=20):
    """The cached K/V tiles one attention step reads, read by isd_kv_read_sweep (each once,
    spread evenly over the GPU, nothing computed), timed with events: the rate this GPU
    reads those bytes at, against the attention step's own rate for the same bytes."""
    import torch
    from strided_verify_propose_amd import isd

    pages = (att.ctx_lens.astype(np.int64) + 15) // 16
    kv_bytes = int(pages.sum()) * scfg.Hkv * 2 * 16 * scfg.D * 2
    cs = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        isd.kv_read_sweep(A["k_cache"], A["v_cache"], A["page_table"], A["ctx_lens"], maxctx, checksum=cs)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3

    # the same kernel over one request whose pages are consecutive (identity page table,
    # one head): a streaming read of two contiguous 96 MiB buffers, the verification
    # pass's volume, as that pass's ceiling
    pages = (96 << 20) // 4096
    ks = torch.zeros((pages, 1, 16, 16, 8), dtype=torch.bfloat16, device=dev)
    vs = torch.zeros((pages, 1, 8, 4, 16, 4), dtype=torch.bfloat16, device=dev)
    ident = torch.arange(pages, dtype=torch.int32, device=dev).reshape(1, pages)
    lens = torch.full((1,), pages * 16, dtype=torch.int32, device=dev)

    def stream():
        isd.kv_read_sweep(ks, vs, ident, lens, pages * 16, checksum=cs)

    for _ in range(3):
        stream()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        stream()
    e1.record()
    torch.cuda.synchronize()
    s_us = e0.elapsed_time(e1) / reps * 1e3
    s_bytes = 2 * pages * 4096
    del ks, vs
    return {"us": round(us, 2), "GBps": round(kv_bytes / (us * 1e-6) / 1e9, 1), "kv_bytes": kv_bytes,
            "attention_kv_GBps": round(kv_bytes / (a_us * 1e-6) / 1e9, 1),
            "attention_rate_frac_of_sweep": round(us / a_us, 4),
            "contiguous": {"us": round(s_us, 2), "bytes": s_bytes,
                           "GBps": round(s_bytes / (s_us * 1e-6) / 1e9, 1)}}


def attainable_bandwidth(dev):
    """What the machine's HBM delivers to torch's own kernels, as context for the rooflines: a
    gather of randomly placed 4 KB rows (index_select over 512 MiB of rows, read + write
    counted) -- the access pattern of paged K/V tiles -- next to the plain device copy.
    HIP events around 5 calls, after one warm-up."""
    import torch

    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    rows = torch.empty((1 << 17, 2048), dtype=torch.bfloat16, device=dev).normal_()   # 4 KB rows
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    perm = torch.randperm(rows.shape[0], generator=g, device=dev)
    out = torch.empty_like(rows)
    t_gather = timed(lambda: torch.index_select(rows, 0, perm, out=out))
    nbytes = rows.numel() * 2
    del rows, out, perm
    torch.cuda.empty_cache()
    return {"gather_4k_rows_read_write": round(2 * nbytes / t_gather / 1e9, 1)}


def verify_parity_counts(vsets_host, vouts, N):
    """The timed verification outputs of every input set against the oracle on the same
    inputs: draws the oracle flags as within 1e-6 of a threshold (and what follows them
    in the request) are excluded and counted; every other decision and id is compared.
    Returns the counts; `mismatches` must be 0."""
    import oracle
    compared = excluded = mism = 0
    for v, out in zip(vsets_host, vouts):
        ref = oracle.verify_step(v.logits, v.draft_logits, v.draft_ids, v.uniforms, N)
        g = {k: t.cpu().numpy() for k, t in out.items()}
        mism += int(np.count_nonzero(g["argmax_ids"] != ref["argmax_ids"]))
        compared += g["argmax_ids"].size
        for b in range(ref["n_accept"].shape[0]):
            n_ref = int(ref["n_accept"][b])
            evaluated = min(n_ref + 1, N - 1)
            flagged = [i for i in range(evaluated) if ref["accept_flag"][b, i]]
            upto = flagged[0] if flagged else evaluated
            mism += int(np.count_nonzero(g["accept"][b, :upto] != ref["accept"][b, :upto]))
            compared += upto
            if flagged:
                excluded += 1
            else:
                mism += int(g["n_accept"][b] != n_ref) + int(np.any(g["accept"][b] != ref["accept"][b]))
                compared += 1
                if ref["residual_flag"][b]:
                    excluded += 1
                else:
                    mism += int(g["next_token"][b] != ref["next_token"][b])
                    compared += 1
            for j in range(N):
                if ref["sample_flag"][b, j]:
                    excluded += 1
                else:
                    mism += int(g["sampled_ids"][b, j] != ref["sampled_ids"][b, j])
                    compared += 1
    return {"sets": len(vsets_host), "compared": compared, "excluded_draws": excluded,
            "excluded_frac": round(excluded / max(1, compared + excluded), 6), "mismatches": mism}


# The all-core oracle baseline: worker processes forked before the GPU is touched, each
# holding the host inputs (inherited at the fork) and one BLAS thread.
_POOL_DATA = None


def _pool_init():
    from threadpoolctl import threadpool_limits
    global _POOL_LIMIT
    _POOL_LIMIT = threadpool_limits(1)


def _w_proj(rows):
    import oracle
    att, ver, pin, scfg = _POOL_DATA
    oracle.gated_lora_proj(pin.x[rows], pin.w, pin.a, pin.b, pin.gate[rows])
    return len(rows)


def _w_attention(b):
    """One request: its own pages, under a page table that numbers them 0, 1, ..."""
    import oracle
    att, ver, pin, scfg = _POOL_DATA
    s = slice(b, b + 1)
    n = (int(att.ctx_lens[b]) + scfg.R + 15) // 16
    pages = att.page_table[b, :n]
    oracle.attention_step(att.q[s], att.k_new[s], att.v_new[s], att.k_pages[pages], att.v_pages[pages],
                          np.arange(n, dtype=np.int32)[None], att.ctx_lens[s], att.scale)
    return b


def _w_verify(b):
    import oracle
    att, ver, pin, scfg = _POOL_DATA
    s = slice(b, b + 1)
    oracle.verify_step(ver.logits[s], ver.draft_logits[s], ver.draft_ids[s], ver.uniforms[s], scfg.N)
    return b


def _w_info(_):
    from threadpoolctl import threadpool_info
    return [{k: i.get(k) for k in ("internal_api", "version", "num_threads")} for i in threadpool_info()]


def pool_workers() -> int:
    """Worker count: the cores this process may run on, capped at 16 (a one-GPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_pool(att, ver, pin, scfg):
    import multiprocessing as mp
    global _POOL_DATA
    _POOL_DATA = (att, ver, pin, scfg)
    return mp.get_context("fork").Pool(pool_workers(), initializer=_pool_init)


def cpu_baseline(scfg, att, ver, pin, pool, one_core_steps=1, all_core_steps=4):
    """The oracle, as it is, on the host: whole steps of the benchmark workload (the
    projection, attention and verification of all 64 requests, first verification input
    set).  One core: in this process with one BLAS thread.  All cores: the same step
    spread over a pool of worker processes, one BLAS thread each -- the projection by
    row blocks, attention and verification by request.  `value` is the all-core rate."""
    import oracle
    from threadpoolctl import threadpool_limits
    t_proj = t_att = t_ver = 0.0
    with threadpool_limits(1):
        for _ in range(one_core_steps):
            t0 = time.perf_counter()
            oracle.gated_lora_proj(pin.x, pin.w, pin.a, pin.b, pin.gate)
            t1 = time.perf_counter()
            oracle.attention_step(att.q, att.k_new, att.v_new, att.k_pages, att.v_pages,
                                  att.page_table, att.ctx_lens, att.scale)
            t2 = time.perf_counter()
            oracle.verify_step(ver.logits, ver.draft_logits, ver.draft_ids, ver.uniforms, scfg.N)
            t3 = time.perf_counter()
            t_proj, t_att, t_ver = t_proj + t1 - t0, t_att + t2 - t1, t_ver + t3 - t2
    one = t_proj + t_att + t_ver
    nw = pool._processes
    blocks = [np.arange(i, min(i + 28, pin.x.shape[0])) for i in range(0, pin.x.shape[0], 28)]
    pool.map(_w_info, range(nw))                      # workers up and initialised
    t0 = time.perf_counter()
    for _ in range(all_core_steps):
        pool.map(_w_proj, blocks, chunksize=1)
        pool.map(_w_attention, range(scfg.B), chunksize=1)
        pool.map(_w_verify, range(scfg.B), chunksize=1)
    allc = time.perf_counter() - t0
    return {"value": round(all_core_steps / allc, 4), "unit": "steps/s", "cores": nw, "kind": "oracle",
            "sample": (f"{all_core_steps} whole steps of the benchmark workload ({scfg.B} requests: projection, "
                       f"attention, verification) over {nw} worker processes, {allc:.1f} s; one core: "
                       f"{one_core_steps} step(s), {one:.1f} s"),
            "one_core": {"value": round(one_core_steps / one, 4), "unit": "steps/s", "cores": 1,
                         "seconds_per_step": {"proj": round(t_proj / one_core_steps, 3),
                                              "attention": round(t_att / one_core_steps, 3),
                                              "verify": round(t_ver / one_core_steps, 3)}},
            "all_cores_seconds_per_step": round(allc / all_core_steps, 3)}


def cpu_host_info(pool):
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "workers": pool._processes, "numpy": np.__version__, "blas": pool.map(_w_info, [0])[0]}


if __name__ == "__main__":
    main()
