"""Benchmark of the KVarN hot path on one MI355X: quantize + packed decode attention.

One step = one pass of the whole path over one batch of synthetic input:
quantise every 128-token block of K and V of the workload into packed pages,
then one decode-attention step of every sequence over the packed cache.  The
default (headline) workload is the largest single-GPU step: a Qwen2.5-1.5B-shaped
model, 28 layers of 64 sequences x 4096 tokens, 12 query / 2 KV heads,
head_dim 128 (28 quantise and 28 decode launches per step).  The other workloads
(tiny, one Llama-3-8B layer, one 131,072-token sequence, the paged mix of 128
sequences) are timed the same way and reported in the same line under
"configs".  Inputs are resident in HBM before the timed region starts.

Prints one JSON line (rank 0).  Throughput is algorithmic bytes / time:
  quantize: 65536 B of fp16 in + 15360 B of pages out per (block, KV head)
  decode:   15360 B of pages per attended (block, KV head) + q, out, table
Outside the timed steps it also times, after a last-level-cache flush, the
packed decode and the same decode over uncompressed fp16 pages (65536 B per
attended (block, KV head)), and reports their ratio.
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

METRIC = "quantize GB/s + packed decode-attn GB/s & tok/s, % of MI355X HBM peak"


# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE x2 + WRITE_SIZE x1, the factors a plain 1 GiB
# copy needs to read back its own size), keyed by kernel and workload.  Each entry holds a digest of the
# kernel source it was measured on; once the source changes the figure no longer applies and is reported
# as null.
MEASURED_TRAFFIC = {
    ("quantize_kernel", "llama3_8b_layer_16x8192"): ("9fdbec7513ad9de4", 663418347),
    ("quantize_kernel", "qwen25_1p5b_28layer_64x4096"): ("9fdbec7513ad9de4", 332141624),
    ("decode_kernel", "qwen25_1p5b_28layer_64x4096"): ("f710cd0b8e1bd9f5", 67394583),
    ("decode_kernel", "llama3_8b_layer_16x8192"): ("f710cd0b8e1bd9f5", 128996384),
}
# the sources each kernel's measurements depend on: its own file, and for the decode the code conversion
# helpers and the host plan that picks its launch shape and instance
KERNEL_SOURCE = {"quantize_kernel": ("kvarn_quantize.hip",),
                 "decode_kernel": ("kvarn_decode.hip", "kvarn_codes.h", "kvarn_host.h")}
# VALU instructions per launch (rocprofv3 SQ_INSTS_VALU, wave64), keyed like MEASURED_TRAFFIC.
MEASURED_VALU = {
    ("quantize_kernel", "llama3_8b_layer_16x8192"): ("9fdbec7513ad9de4", 111398912),
    ("quantize_kernel", "qwen25_1p5b_28layer_64x4096"): ("9fdbec7513ad9de4", 56650476),
    ("decode_kernel", "qwen25_1p5b_28layer_64x4096"): ("f710cd0b8e1bd9f5", 5836098),
    ("decode_kernel", "llama3_8b_layer_16x8192"): ("f710cd0b8e1bd9f5", 9665216),
}
# Issue rate of non-packed fp32 VALU lane operations: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12



def source_digest(kernel):
    """Digest of the kernel's source code with comments and blank space removed, and of its compiler
    flags, so that a comment edit keeps the measurement while any change to the code drops it."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "kv_cache_quantization_kvarn_amd", "csrc")
    data = ""
    for f in KERNEL_SOURCE[kernel] + ("kvarn_common.h",):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            data += fh.read()
    data = re.sub(r"/\*.*?\*/", " ", data, flags=re.S)
    data = re.sub(r"//[^\n]*", " ", data)
    data = " ".join(data.split())
    # the compiler flags of that source are part of what was measured
    from kv_cache_quantization_kvarn_amd import build
    data += " flags: " + " ".join(build.FLAGS)
    return hashlib.sha256(data.encode()).hexdigest()[:16]


def measured_traffic(kernel, workload, table=None):
    entry = (MEASURED_TRAFFIC if table is None else table).get((kernel, workload))
    if entry is None or entry[0] != source_digest(kernel):
        return None
    return entry[1]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen25_1p5b_28layer_64x4096",
                    help="the headline workload (the largest single-GPU step by default)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload summaries of the other configurations")
    ap.add_argument("--no-head-dims", action="store_true",
                    help="skip the layers with heads of 64 and 256 channels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time for each of the two CPU-baseline legs (one thread, all cores)")
    ap.add_argument("--flush-reps", type=int, default=20, help="decode-only repetitions after a cache flush")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the step")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the other formats (code widths k4v4, k8v2, k8v4; group size 64)")
    ap.add_argument("--prefill-workload", default="prefill_llama3_8b_16x7680p512")
    ap.add_argument("--no-tail", action="store_true", help="skip the decode with fp16 tails")
    ap.add_argument("--no-fp16-baseline", action="store_true",
                    help="skip the fp16 paged decode baseline (measured outside the timed steps)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (calibrates HBM byte counters) and exit")
    return ap.parse_args()


def copy_probe(mib):
    """Plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE counters scale the kernels' readings."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each": n * 4, "copies": 5}), flush=True)


class Case:
    """Device buffers and the two launches of one workload."""

    def __init__(self, K, w, cfg):
        import torch
        from kv_cache_quantization_kvarn_amd import synth
        self.K, self.w, self.cfg = K, w, cfg
        pm = synth.make_page_map(w)
        self.pm = pm
        n_prefix = synth.total_prefix_blocks(w)
        self.layers = []
        for layer in range(w.layers):
            if w.append_blocks:
                # paged mixed: the prefix is filled once outside the timed region; a step
                # quantises the appended block of every sequence and decodes over prefix + append
                k, v = synth.layer_kv(w, layer, n_prefix * 128, "cuda")
                ka, va = synth.layer_kv(w, layer, w.batch * 128, "cuda", append=True)
                kp, vp = K.alloc_pools(cfg, pm.num_pages, w.hkv)
                K.kvarn_quantize_blocks(cfg, k, v, pm.prefix_pages.cuda(), kp, vp)
                del k, v
                qk, qv, dst = ka, va, pm.append_pages.cuda()
            else:
                qk, qv = synth.layer_kv(w, layer, n_prefix * 128, "cuda")
                kp, vp = K.alloc_pools(cfg, pm.num_pages, w.hkv)
                dst = pm.prefix_pages.cuda()
            q = synth.make_q(w, layer, "cuda")
            self.layers.append(dict(k=qk, v=qv, dst=dst, kp=kp, vp=vp, q=q))
        self.bt = pm.block_table.cuda()
        self.sl = pm.seq_lens.cuda()
        self.ws = K.alloc_workspace(cfg, w.batch, w.hq, w.hkv, pm.block_table.shape[1])
        self.out = torch.empty(w.batch, w.hq, w.head_dim, dtype=torch.float32, device="cuda")
        self.flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        from kv_cache_quantization_kvarn_amd import accounting as acc
        kb, vb = K.kvarn_page_bytes(cfg, False), K.kvarn_page_bytes(cfg, True)
        qblocks = self.layers[0]["dst"].numel()
        attended = int(pm.seq_lens.sum().item()) // 128
        d = w.head_dim
        self.q_bytes = acc.quantize_bytes(qblocks, w.hkv, kb, vb, d) * w.layers
        self.d_bytes = acc.decode_bytes(attended, w.hkv, w.batch, w.hq, kb, vb, head_dim=d) * w.layers
        self.q_bytes_launch = acc.quantize_bytes(qblocks, w.hkv, kb, vb, d)
        self.d_bytes_launch = acc.decode_bytes(attended, w.hkv, w.batch, w.hq, kb, vb, head_dim=d)
        self.q_tokens = qblocks * 128 * w.layers
        self.ctx_tokens = attended * 128

    def quantize(self, L):
        self.K.kvarn_quantize_blocks(self.cfg, L["k"], L["v"], L["dst"], L["kp"], L["vp"], self.flags)

    def decode(self, L):
        self.K.kvarn_decode_attention(self.cfg, L["q"], L["kp"], L["vp"], self.bt, self.sl, self.w.hkv, self.out,
                                      self.ws, dev_flags=self.flags)

    def step(self, stream, events=None):
        """One step: quantise every layer, then one decode step of every layer.  `events` maps a layer
        index to four timing events recorded around that layer's quantise and decode launches; the
        layers it names are the timed sample."""
        events = events or {}
        for li, L in enumerate(self.layers):
            ev = events.get(li)
            if ev:
                ev[0].record(stream)
            self.quantize(L)
            if ev:
                ev[1].record(stream)
        for li, L in enumerate(self.layers):
            ev = events.get(li)
            if ev:
                ev[2].record(stream)
            self.decode(L)
            if ev:
                ev[3].record(stream)


def event_layers(n_layers):
    """Layers whose launches carry timing events in every timed step: four evenly spaced layers (all
    of a workload with fewer), so that the markers do not perturb the step they time."""
    return sorted(set(range(0, n_layers, max(1, n_layers // 4))))


def time_steps(case, stream, steps, warmup):
    """Warm-up steps, then `steps` timed steps bracketed by device synchronisation.  Returns the wall
    time of the timed steps and the average quantise and decode launch times (HIP events around the
    sampled layers' launches of every timed step)."""
    import torch
    for _ in range(warmup):
        case.step(stream)
    torch.cuda.synchronize()
    sample = event_layers(len(case.layers))
    evs = [{li: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for li in sample} for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        case.step(stream, evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert case.K.kvarn_read_flags(case.flags) == 0, "device flags set during the benchmark"
    q_ms = [e[0].elapsed_time(e[1]) for st in evs for e in st.values()]
    d_ms = [e[2].elapsed_time(e[3]) for st in evs for e in st.values()]
    return elapsed, sum(q_ms) / len(q_ms) / 1e3, sum(d_ms) / len(d_ms) / 1e3


def config_summary(K, cfg, name, stream, steps, warmup, reps, flush, sink, workloads=None):
    """Step rate, per-launch quantise and decode rates and the cache-flushed decode of one workload."""
    import torch
    from kv_cache_quantization_kvarn_amd import accounting as acc
    from kv_cache_quantization_kvarn_amd import synth
    w = (workloads or synth.WORKLOADS)[name]
    case = Case(K, w, cfg)
    elapsed, q_s, d_s = time_steps(case, stream, steps, warmup)
    d_flush = timed_after_flush(lambda: case.decode(case.layers[0]), reps, stream, flush, sink)
    step_bytes = case.q_bytes + case.d_bytes
    pk = lambda gbps: round(gbps / acc.HBM_PEAK_GBPS, 4)
    qg, dg, fg = case.q_bytes_launch / q_s / 1e9, case.d_bytes_launch / d_s / 1e9, case.d_bytes_launch / d_flush / 1e9
    res = {"ms_per_step": round(elapsed / steps * 1e3, 4), "value": round(step_bytes / (elapsed / steps) / 1e9, 1),
           "layers": w.layers, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
           "seq_len": w.seq_len or list(w.seq_len_range),
           "quantize": {"us_per_launch": round(q_s * 1e6, 2), "gbps": round(qg, 1), "frac": pk(qg),
                        "bytes_per_launch": case.q_bytes_launch,
                        "tokens_per_s": round(case.q_tokens / (q_s * w.layers), 1)},
           "decode": {"us_per_launch": round(d_s * 1e6, 2), "gbps": round(dg, 1), "frac": pk(dg),
                      "bytes_per_launch": case.d_bytes_launch, "tokens_per_s": round(w.batch / (d_s * w.layers), 1),
                      "context_tokens_per_s": round(case.ctx_tokens / d_s, 1),
                      "after_cache_flush": {"us_median": round(d_flush * 1e6, 2), "gbps": round(fg, 1),
                                            "frac": pk(fg)}},
           "steps": steps}
    if w.append_blocks:
        res["quantize"]["what"] = "append: one 128-token block per sequence, into pages of a permuted pool"
    del case
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_pass(C, acc, w, kh, vh, blocks, kp, vp, q, bt, sl, seconds, threads, qblocks_per_call):
    """Repeated C++-oracle quantise calls (qblocks_per_call blocks of every KV head, K and V) for half of
    `seconds`, then repeated whole decode calls over `bt` for the other half.  Returns bytes and times."""
    kb, vb = kp.shape[2], vp.shape[2]
    t0 = time.perf_counter()
    nq = 0
    while time.perf_counter() - t0 < seconds / 2 or nq < 1:
        lo = (nq * qblocks_per_call) % (blocks - qblocks_per_call + 1)
        C.quantize_blocks(kh[128 * lo:128 * (lo + qblocks_per_call)], vh[128 * lo:128 * (lo + qblocks_per_call)],
                          np.arange(qblocks_per_call, dtype=np.int32), kp, vp, threads=threads)
        nq += 1
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    nd = 0
    while time.perf_counter() - t0 < seconds / 2 or nd < 1:
        C.decode(q, kp, vp, bt, sl, w.hkv, threads=threads)
        nd += 1
    td = time.perf_counter() - t0
    qbytes = nq * acc.quantize_bytes(qblocks_per_call, w.hkv, kb, vb)
    attended = int(sl.sum()) // 128
    dbytes = nd * acc.decode_bytes(attended, w.hkv, q.shape[0], w.hq, kb, vb)
    return qbytes, tq, dbytes, td, nq, nd


def cpu_baseline(w, seconds):
    """The C++ oracle (double precision, FWHT mode, the one the parity tests use at full size) on a
    bounded sample of the same workload, in the same GB/s units: one thread, then one thread per
    available core (at most 16).  The sample: layer 0's first blocks quantised (K and V of every KV
    head), and decode steps of sequences of the workload's length over those pages."""
    from kv_cache_quantization_kvarn_amd import accounting as acc
    from kv_cache_quantization_kvarn_amd import synth
    from oracle import kvarn_oracle_cpp as C

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    n = max(1, min(16, avail))
    pm = synth.make_page_map(w)
    nb_seq = int(pm.seq_lens[0]) // 128
    blocks = 16 * n
    k, v = synth.layer_kv(w, 0, blocks * 128, "cpu")
    kh, vh = k.numpy(), v.numpy()
    kp = np.zeros((blocks, w.hkv, 9728), np.uint8)
    vp = np.zeros((blocks, w.hkv, 5632), np.uint8)
    C.quantize_blocks(kh, vh, np.arange(blocks, dtype=np.int32), kp, vp)
    res = {"unit": "GB/s", "kind": "oracle", "cpu_model": cpu_model()}
    for threads, key in ((1, "one_thread"), (n, "all_cores")):
        seqs = threads  # one sequence per thread per decode call
        bt = (np.arange(seqs * nb_seq, dtype=np.int32) % blocks).reshape(seqs, nb_seq)
        sl = np.full(seqs, nb_seq * 128, np.int32)
        q = synth.make_q(w, 0, "cpu").numpy()[:1].repeat(seqs, axis=0)
        qb, tq, db, td, nq, nd = _oracle_pass(C, acc, w, kh, vh, blocks, kp, vp, q, bt, sl, seconds, threads,
                                              max(1, threads))
        res[key] = {"value": round((qb + db) / (tq + td) / 1e9, 6), "cores": threads,
                    "quantize_gbps": round(qb / tq / 1e9, 6), "decode_gbps": round(db / td / 1e9, 6),
                    "sample": "%d quantise calls of %d block(s) x %d KV heads (K and V) + %d decode calls of %d "
                              "sequence(s) x %d query heads over %d blocks each; C++ oracle, %d thread(s)"
                              % (nq, max(1, threads), w.hkv, nd, seqs, w.hq, nb_seq, threads)}
    top = res["all_cores"]
    res.update(value=top["value"], cores=top["cores"], sample=top["sample"])
    return res


def timed_after_flush(fn, reps, stream, flush, sink):
    """Median time (s) of fn() launches, each after reading 512 MB (evicts the 256 MB last-level cache)."""
    import torch
    ms = []
    for _ in range(reps):
        torch.sum(flush, dim=0, out=sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2] / 1e3


def fp16_baseline(case, K, synth, acc, stream, reps, flush, sink, kvarn_flush_s):
    """The same decode over uncompressed fp16 pages (layer 0), cache-flushed like the packed decode."""
    import torch
    w, pm = case.w, case.pm
    n_prefix = synth.total_prefix_blocks(w)
    k, v = synth.layer_kv(w, 0, n_prefix * 128, "cuda")
    kc = synth.fp16_pages(k, pm.prefix_pages, pm.num_pages)
    vc = synth.fp16_pages(v, pm.prefix_pages, pm.num_pages)
    del k, v
    if w.append_blocks:
        ka, va = synth.layer_kv(w, 0, w.batch * 128, "cuda", append=True)
        synth.fp16_pages(ka, pm.append_pages, pm.num_pages, pool=kc)
        synth.fp16_pages(va, pm.append_pages, pm.num_pages, pool=vc)
        del ka, va
    q = case.layers[0]["q"]

    def run():
        K.kvarn_fp16_decode_attention(case.cfg, q, kc, vc, case.bt, case.sl, w.hkv, case.out, case.ws,
                                      dev_flags=case.flags)

    run()
    torch.cuda.synchronize()
    t = timed_after_flush(run, reps, stream, flush, sink)
    assert K.kvarn_read_flags(case.flags) == 0, "device flags set by the fp16 baseline"
    page = K.kvarn_fp16_page_bytes(case.cfg)
    attended = int(pm.seq_lens.sum().item()) // 128
    nbytes = acc.decode_bytes(attended, w.hkv, w.batch, w.hq, page, page)
    gbps = nbytes / t / 1e9
    del kc, vc
    torch.cuda.empty_cache()
    return {"us_median": round(t * 1e6, 2), "gbps": round(gbps, 1),
            "pct_peak": round(100 * gbps / acc.HBM_PEAK_GBPS, 2), "bytes_per_launch": nbytes,
            "tokens_per_s": round(w.batch / t, 1),
            "packed_decode_speedup": round(t / kvarn_flush_s, 3),
            "protocol": "both decodes timed after a 512 MB read that evicts the last-level cache; median of %d" % reps}


def tail_measure(case, K, synth, acc, stream, reps, flush, sink, packed_flush_s, tail_tokens=127):
    """Decode over the layer-0 packed cache plus an fp16 tail of `tail_tokens` per sequence (127 is the
    longest a tail gets), cache-flushed like the packed decode it is compared with."""
    import torch
    w, pm = case.w, case.pm
    L0 = case.layers[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.stream_seed(w, 9))
    kt = torch.zeros(w.batch, 128, w.hkv, 128, dtype=torch.float16, device="cuda")
    vt = torch.zeros_like(kt)
    kt[:, :tail_tokens] = torch.randn(w.batch, tail_tokens, w.hkv, 128, generator=g, device="cuda").half()
    vt[:, :tail_tokens] = torch.randn(w.batch, tail_tokens, w.hkv, 128, generator=g, device="cuda").half()
    sl = (pm.seq_lens + tail_tokens).to(torch.int32).cuda()

    def run():
        K.kvarn_decode_attention_tail(case.cfg, L0["q"], L0["kp"], L0["vp"], case.bt, sl, kt, vt, w.hkv, case.out,
                                      case.ws, dev_flags=case.flags, stream=stream)

    run()
    torch.cuda.synchronize()
    t = timed_after_flush(run, reps, stream, flush, sink)
    assert K.kvarn_read_flags(case.flags) == 0, "device flags set by the tail decode"
    kb, vb = K.kvarn_page_bytes(case.cfg, False), K.kvarn_page_bytes(case.cfg, True)
    attended = int(pm.seq_lens.sum().item()) // 128
    nbytes = acc.tail_decode_bytes(attended, w.hkv, w.batch, w.hq, kb, vb, w.batch * tail_tokens)
    gbps = nbytes / t / 1e9
    del kt, vt
    torch.cuda.empty_cache()
    return {"tail_tokens": tail_tokens, "us_median": round(t * 1e6, 2), "gbps": round(gbps, 1),
            "pct_peak": round(100 * gbps / acc.HBM_PEAK_GBPS, 2), "bytes_per_launch": nbytes,
            "vs_packed_only": round(t / packed_flush_s, 3),
            "protocol": "median of %d launches, each after a 512 MB read that evicts the last-level cache" % reps}


def prefill_measure(K, synth, acc, cfg, name, stream, reps, flush, sink):
    """Chunked prefill over packed pages plus fp16 rows (a matrix-core bound kernel), cache-flushed."""
    import torch
    w = synth.PREFILL_WORKLOADS[name]
    x = synth.prefill_inputs(w, "cuda")
    kp, vp = K.alloc_pools(cfg, x.num_pages, w.hkv)
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    K.kvarn_quantize_blocks(cfg, x.k_prefix, x.v_prefix, x.pages, kp, vp, fl)
    out = torch.empty(tuple(x.q.shape), dtype=torch.float32, device="cuda")

    def run():
        K.kvarn_prefill_attention(cfg, x.q, kp, vp, x.block_table, x.prefix_lens, x.k_new, x.v_new, x.new_lens,
                                  x.q_lens, w.hkv, out, dev_flags=fl, stream=stream)

    run()
    torch.cuda.synchronize()
    t = timed_after_flush(run, reps, stream, flush, sink)
    assert K.kvarn_read_flags(fl) == 0, "device flags set by the prefill"
    pairs = acc.prefill_pairs(x.prefix_lens.tolist(), x.new_lens.tolist(), x.q_lens.tolist(), w.hq)
    flops = acc.prefill_flops(pairs)
    nbytes = acc.prefill_bytes(w.batch * (w.prefix // 128), w.hkv, K.kvarn_page_bytes(cfg, 0), K.kvarn_page_bytes(cfg, 1),
                               w.batch * w.chunk, w.batch * w.chunk, w.hq)
    tflops = flops / t / 1e12
    del kp, vp, out, x
    torch.cuda.empty_cache()
    return {"workload": w.name, "us_median": round(t * 1e6, 2), "tflops": round(tflops, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": acc.MFMA_FP16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / acc.MFMA_FP16_PEAK_TFLOPS, 4)},
            "flops_per_launch": flops, "attended_pairs": pairs, "bytes_per_launch": nbytes,
            "gbps": round(nbytes / t / 1e9, 1), "query_tokens_per_s": round(w.batch * w.chunk / t, 1),
            "protocol": "median of %d launches, each after a 512 MB read that evicts the last-level cache" % reps}


def formats_measure(K, w, case, stream, reps, flush, sink):
    """Quantise and decode launches of the workload's first layer in the other code widths.  Decode in
    these formats runs on the matrix-core decode kernel instantiated for their code widths."""
    import torch
    from kv_cache_quantization_kvarn_amd import accounting as acc
    res = {}
    L0 = case.layers[0]
    for name in ("kvarn_k4v4_g128", "kvarn_k8v2_g128", "kvarn_k8v4_g128", "kvarn_k4v2_g64", "kvarn_k4v4_g64",
                 "kvarn_k8v2_g64", "kvarn_k8v4_g64"):
        cfg = K.kvarn_config_parse(name)
        kp, vp = K.alloc_pools(cfg, case.pm.num_pages, w.hkv)
        if w.append_blocks:
            from kv_cache_quantization_kvarn_amd import synth
            k, v = synth.layer_kv(w, 0, synth.total_prefix_blocks(w) * 128, "cuda")
            K.kvarn_quantize_blocks(cfg, k, v, case.pm.prefix_pages.cuda(), kp, vp, case.flags)
            del k, v

        def quant():
            K.kvarn_quantize_blocks(cfg, L0["k"], L0["v"], L0["dst"], kp, vp, case.flags)

        def dec():
            K.kvarn_decode_attention(cfg, L0["q"], kp, vp, case.bt, case.sl, w.hkv, case.out, case.ws,
                                     dev_flags=case.flags)

        quant()
        dec()
        torch.cuda.synchronize()
        tq = timed_after_flush(quant, reps, stream, flush, sink)
        td = timed_after_flush(dec, reps, stream, flush, sink)
        assert K.kvarn_read_flags(case.flags) == 0, "device flags set in format " + name
        kb, vb = K.kvarn_page_bytes(cfg, False), K.kvarn_page_bytes(cfg, True)
        qb = acc.quantize_bytes(L0["dst"].numel(), w.hkv, kb, vb)
        db = acc.decode_bytes(int(case.pm.seq_lens.sum().item()) // 128, w.hkv, w.batch, w.hq, kb, vb)
        res[name] = {"quantize_us": round(tq * 1e6, 2), "quantize_gbps": round(qb / tq / 1e9, 1),
                     "decode_us": round(td * 1e6, 2), "decode_gbps": round(db / td / 1e9, 1),
                     "page_bytes": [kb, vb]}
        del kp, vp
        torch.cuda.empty_cache()
    return res


def progress(msg):
    """A phase of the run, on stderr (stdout carries only the result line)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (run with --gpus 1)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import torch

    from kv_cache_quantization_kvarn_amd import accounting as acc
    from kv_cache_quantization_kvarn_amd import synth

    w = synth.WORKLOADS[args.workload]
    # the oracle baseline runs first, before the GPU work (it uses the host's cores only)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    progress("cpu baseline done" if cpu else "cpu baseline skipped")
    from kv_cache_quantization_kvarn_amd import kvarn as K

    cfg = K.kvarn_config_parse("kvarn_k4v2_g128")
    case = Case(K, w, cfg)
    stream = torch.cuda.current_stream()

    def step():
        case.step(stream)

    elapsed, q_avg_s, d_avg_s = time_steps(case, stream, args.steps, args.warmup)
    progress("%s: %d steps timed, %.3f ms per step" % (w.name, args.steps, elapsed / args.steps * 1e3))

    # the same step captured once in a HIP graph and replayed (one launch of the whole step; for the
    # 28-layer workload that is 56 kernels)
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0g = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0g) / args.steps * 1e3
        assert K.kvarn_read_flags(case.flags) == 0, "device flags set during the graph replays"
        del graph
        progress("graph replays timed")

    # decode alone after reading 512 MB (evicts the 256 MB last-level cache, leaving clean lines, so
    # the decode pays no write-back of the flush), timed per launch
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty(1, dtype=torch.float32, device="cuda")
    L0 = case.layers[0]
    d_flush_s = timed_after_flush(lambda: case.decode(L0), args.flush_reps, stream, flush, flush_sink)
    fp16 = None
    if not args.no_fp16_baseline:
        fp16 = fp16_baseline(case, K, synth, acc, stream, args.flush_reps, flush, flush_sink, d_flush_s)

    tail = None
    if not args.no_tail:
        tail = tail_measure(case, K, synth, acc, stream, args.flush_reps, flush, flush_sink, d_flush_s)

    progress("cache-flushed decode, fp16 baseline and tail done")
    formats = None
    if not args.no_formats:
        formats = formats_measure(K, w, case, stream, max(5, args.flush_reps // 2), flush, flush_sink)
    prefill = None
    if formats is not None:
        progress("formats done")
    if not args.no_prefill:
        prefill = prefill_measure(K, synth, acc, cfg, args.prefill_workload, stream, args.flush_reps, flush, flush_sink)
        g64 = prefill_measure(K, synth, acc, K.kvarn_config_parse("kvarn_k4v2_g64"), args.prefill_workload, stream,
                              max(5, args.flush_reps // 2), flush, flush_sink)
        prefill["group64"] = {"format": "kvarn_k4v2_g64", "us_median": g64["us_median"], "tflops": g64["tflops"],
                              "frac": g64["roofline"]["frac"]}

    # heads of 64 and 256 channels: one full-size layer each, quantise and decode launches
    head_dims = None
    if not args.no_head_dims:
        head_dims = {}
        for name, hw in synth.HEAD_DIM_WORKLOADS.items():
            if name.startswith("tiny"):
                continue
            hcfg = K.kvarn_config_parse("kvarn_k4v2_g128", hw.head_dim)
            head_dims[name] = config_summary(K, hcfg, name, stream, args.steps, args.warmup, args.flush_reps, flush,
                                             flush_sink, workloads=synth.HEAD_DIM_WORKLOADS)
            head_dims[name]["head_dim"] = hw.head_dim
            progress(name + " done")

    # the other workloads, each timed like the headline step (a summary object per workload)
    configs = None
    if not args.no_configs:
        configs = {}
        for name in synth.WORKLOADS:
            if name != w.name:
                configs[name] = config_summary(K, cfg, name, stream, args.steps, args.warmup, args.flush_reps, flush,
                                               flush_sink)
                progress(name + " done")

    step_bytes = case.q_bytes + case.d_bytes
    ms_per_step = elapsed / args.steps * 1e3
    value = step_bytes / (elapsed / args.steps) / 1e9
    q_gbps = case.q_bytes_launch / q_avg_s / 1e9
    d_gbps = case.d_bytes_launch / d_avg_s / 1e9
    d_flush_gbps = case.d_bytes_launch / d_flush_s / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: K N(0,1) with outlier channels, V N(0,1) x per-token lognormal scale, q N(0,1); fp16)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len or list(w.seq_len_range),
                   "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": 128, "layers": w.layers,
                   "format": "kvarn_k4v2_g128", "parallelism": "single GPU"},
        "pct_hbm_peak": round(100.0 * value / acc.HBM_PEAK_GBPS, 2),
        "quantize": {"gbps": round(q_gbps, 1), "pct_peak": round(100 * q_gbps / acc.HBM_PEAK_GBPS, 2),
                     "us_per_launch": round(q_avg_s * 1e6, 2), "tokens_per_s": round(case.q_tokens / (q_avg_s * w.layers), 1),
                     "bytes_per_launch": case.q_bytes_launch},
        "decode": {"gbps": round(d_gbps, 1), "pct_peak": round(100 * d_gbps / acc.HBM_PEAK_GBPS, 2),
                   "us_per_launch": round(d_avg_s * 1e6, 2),
                   "tokens_per_s": round(w.batch / (d_avg_s * w.layers), 1),
                   "context_tokens_per_s": round(case.ctx_tokens / d_avg_s, 1),
                   "bytes_per_launch": case.d_bytes_launch,
                   "after_cache_flush": {"gbps": round(d_flush_gbps, 1),
                                         "pct_peak": round(100 * d_flush_gbps / acc.HBM_PEAK_GBPS, 2),
                                         "us_median": round(d_flush_s * 1e6, 2)}},
    }
    if fp16 is not None:
        line["fp16_baseline"] = fp16
    if tail is not None:
        line["tail"] = tail
    if graph_ms is not None:
        line["graph"] = {"ms_per_step": round(graph_ms, 4), "value": round(step_bytes / (graph_ms / 1e3) / 1e9, 3),
                         "kernels_per_step": 2 * w.layers,
                         "protocol": "the timed step captured once in a HIP graph, %d replays timed like the eager steps"
                                     % args.steps}
    if prefill is not None:
        line["prefill"] = prefill
    if formats is not None:
        line["formats"] = formats
    if configs is not None:
        line["configs"] = configs
    if head_dims is not None:
        line["head_dims"] = head_dims
    # dominant kernel by time: the one whose launches take longer in the step
    if q_avg_s >= d_avg_s:
        dom, ach = "quantize_kernel", q_gbps
    else:
        dom, ach = "decode_kernel", d_gbps
    traffic = measured_traffic(dom, w.name)
    units = case.layers[0]["dst"].numel() * w.hkv if dom == "quantize_kernel" else int(case.pm.seq_lens.sum()) // 128 * w.hkv
    line["roofline"] = {"kernel": "kvarn " + dom, "bound": "hbm", "achieved": round(ach, 1), "peak": acc.HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(ach / acc.HBM_PEAK_GBPS, 4), "traffic": traffic,
                        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                        "algorithmic_bytes_per_launch": case.q_bytes_launch if dom == "quantize_kernel" else case.d_bytes_launch,
                        "units_per_launch": units,
                        "unit_of_work": "(128-token block, KV head)",
                        "us_per_launch": round((q_avg_s if dom == "quantize_kernel" else d_avg_s) * 1e6, 2)}
    valu = measured_traffic(dom, w.name, MEASURED_VALU)
    if valu is not None:
        # the same launches seen as ALU work: VALU lane operations issued per second (wave64 -> 64 lanes)
        avg_s = q_avg_s if dom == "quantize_kernel" else d_avg_s
        t = valu * 64 / avg_s / 1e12
        line["roofline"]["valu"] = {"achieved": round(t, 2), "peak": round(VALU_PEAK_TLANEOPS, 2),
                                    "unit": "T lane-ops/s", "frac": round(t / VALU_PEAK_TLANEOPS, 4),
                                    "insts_per_launch": valu,
                                    "source": "rocprofv3 SQ_INSTS_VALU of the same kernel source"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
