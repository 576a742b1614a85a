#!/usr/bin/env python3
"""Decode-attention benchmark over a calibrated E4M3 paged KV cache (one MI355X).

One step is one layer's decode hot path over the batch: quantise-write the new
token of every sequence into the E4M3 cache, split-context attention over the
whole context, and the FP32 split reduce. For decode the attention kernel
appends the new tokens itself (paged_attn_e4m3_decode_append: the same cache
bytes and output as the write kernel followed by attention); the step time
with the separate write kernel is reported beside it. The headline workload is batch 32 at
a 4,096-token context (32 query / 4 KV heads, head_dim 128, page 16); the 32k
(batch 32, context 32,768) and 256k (batch 4, context 262,144, page 64, 64
splits, outlier channels) points are reported beside it.

Timing: the caches are rotated over enough copies that every step reads its KV
from HBM (the 256 MB Infinity Cache cannot hold them). Each point's steps are
captured in HIP graphs and the timed region replays exactly --steps of them,
bracketed by device synchronisation and HIP events. The attention kernel's own
average duration comes from a graph of back-to-back attention launches timed
with HIP events on the stream the kernels run on.

Prints one JSON line. --gpus above 1 is refused: the library runs on one GPU.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E datasheet peak

# HBM bytes per launch of the 4k decode attention kernel from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs (`bench.py --counter-pass`), scaled by the same
# counters' reading of a 1 GiB device copy. Valid only for the kernel source
# they were taken on (sha256 prefix); otherwise the traffic is reported as null.
MEASURED_TRAFFIC = {"source_sha256_prefix": "58c927dbd5d8d8ee", "read_bytes": 137039137,
                    "write_bytes": 1081344}


TRAFFIC_SOURCES = ("attn_split.hip", "split_plan.h", "kvfp8_internal.h")  # the sources the counted kernel is built from


def measured_traffic():
    import hashlib
    csrc = os.path.join(ROOT, "fp8_quantised_paged_amd", "csrc")
    h = hashlib.sha256()
    try:
        for name in TRAFFIC_SOURCES:
            h.update(open(os.path.join(csrc, name), "rb").read())
    except OSError:
        return None
    sha = h.hexdigest()[:16]
    if sha != MEASURED_TRAFFIC["source_sha256_prefix"]:
        return None
    return MEASURED_TRAFFIC["read_bytes"] + MEASURED_TRAFFIC["write_bytes"]
METRIC = "decode attention KV GB/s & % of HBM peak; tokens/s per layer at 4k/32k/256k"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(seq_lens, n_q_heads, n_kv_heads, head_dim, max_pages, q_rows=None, kv_elem_bytes=1):
    """Bytes one decode (or verify) step must move at minimum: every cached K
    and V byte (kv_elem_bytes per element: 1 for E4M3, 2 for the fp16 arm),
    Q in, O out (fp16, q_rows query rows, one per sequence unless given), the
    block table and the sequence lengths."""
    B = len(seq_lens)
    rows = B if q_rows is None else int(q_rows)
    kv = int(np.sum(seq_lens, dtype=np.int64)) * n_kv_heads * head_dim * 2 * kv_elem_bytes
    qo = 2 * rows * n_q_heads * head_dim * 2
    meta = B * max_pages * 4 + B * 4
    return kv, kv + qo + meta


class Point:
    """One decode workload resident on the GPU with `nsets` cache copies."""

    def __init__(self, K, torch, name, layout, k_src, v_src, calib, num_splits, nsets, scales=None, f16=False):
        self.K, self.torch, self.name, self.bt = K, torch, name, layout
        bt = layout
        dev = "cuda"
        self.S = num_splits
        self.f16 = f16  # the fp16-cache arm of the format comparison
        if f16:
            scales = (1.0, 1.0)
        self.B, self.Hq, self.Hkv, self.D, self.P = bt.batch, bt.n_q_heads, bt.n_kv_heads, bt.head_dim, bt.page_size
        if scales is None:
            amax, scale, _ = K.kv_calibrate_amax(calib)
            scales = (float(scale[0].item()), float(scale[1].item()))
        self.ks, self.vs = scales
        self.verify = bool((bt.q_lens != 1).any())
        self.max_q = int(bt.q_lens.max())
        self.rows = bt.total_q
        self.cu_q = torch.from_numpy(bt.cu_q_lens).to(dev)
        self.sm = float(np.float32(1.0 / np.sqrt(self.D)))
        self.q = torch.from_numpy(bt.q).to(dev)
        self.block_table = torch.from_numpy(bt.block_table).to(dev)
        self.seq_lens = torch.from_numpy(bt.seq_lens).to(dev)
        slots = torch.from_numpy(bt.slot_mapping).to(dev)
        self.slots_all = slots
        new_rows = torch.from_numpy(bt.new_token_rows()).to(dev)
        self.k_new = k_src[new_rows].contiguous()
        self.v_new = v_src[new_rows].contiguous()
        self.slots_new = slots[new_rows].contiguous()
        self.sets = []
        for _ in range(nsets):
            if f16:
                # cache fill (setup): fp16 values scattered to their slots, NaN elsewhere
                kc = torch.full((bt.num_pages, self.Hkv, self.P, self.D), float("nan"), dtype=torch.float16,
                                device=dev)
                vc = torch.full((bt.num_pages, self.Hkv, self.D, self.P), float("nan"), dtype=torch.float16,
                                device=dev)
                pg, off = slots // self.P, slots % self.P
                kc[pg, :, off, :] = k_src
                vc[pg, :, :, off] = v_src
            else:
                kc = torch.full((bt.num_pages, self.Hkv, self.P, self.D), 0x7F, dtype=torch.uint8, device=dev)
                vc = torch.full((bt.num_pages, self.Hkv, self.D, self.P), 0x7F, dtype=torch.uint8, device=dev)
                K.kv_quant_write(k_src, v_src, slots, self.ks, self.vs, kc, vc)
            self.sets.append((kc, vc))
        self.ws = K.workspace(self.rows, self.Hq, self.D, self.S)
        self.ws_o, self.ws_m, self.ws_l = K.workspace_views(self.ws, self.rows, self.Hq, self.D, self.S)
        self.out = torch.empty_like(self.q)
        self.kv_bytes, self.alg_bytes = algorithmic_bytes(bt.seq_lens, self.Hq, self.Hkv, self.D,
                                                          bt.max_pages, q_rows=self.rows,
                                                          kv_elem_bytes=2 if f16 else 1)
        torch.cuda.synchronize()

    def _call(self, i, out):
        kc, vc = self.sets[i % len(self.sets)]
        kw = dict(num_splits=self.S, workspace=self.ws)
        kw.update(out=out) if out is not None else kw.update(partials_only=True)
        if self.f16 and self.verify:
            self.K.paged_attn_f16_verify(self.q, self.cu_q, self.max_q, kc, vc, self.block_table, self.seq_lens,
                                         self.sm, **kw)
        elif self.f16:
            self.K.paged_attn_f16_decode(self.q, kc, vc, self.block_table, self.seq_lens, self.sm, **kw)
        elif self.verify:
            self.K.paged_attn_e4m3_verify(self.q, self.cu_q, self.max_q, kc, vc, self.block_table,
                                          self.seq_lens, self.ks, self.vs, self.sm, **kw)
        else:
            self.K.paged_attn_e4m3_decode(self.q, kc, vc, self.block_table, self.seq_lens, self.ks,
                                          self.vs, self.sm, **kw)

    def attend(self, i):
        """The attention kernel alone (partials only; unsplit calls write out)."""
        self._call(i, self.out if self.S == 1 else None)

    def step(self, i):
        """Write kernel, then attention (and the reduce when split). The fp16
        arm has no write kernel: its step is attention and reduce."""
        kc, vc = self.sets[i % len(self.sets)]
        if not self.f16:
            self.K.kv_quant_write(self.k_new, self.v_new, self.slots_new, self.ks, self.vs, kc, vc)
        self._call(i, self.out)

    def step_fused(self, i):
        """Decode or verify with the new tokens appended by the attention kernel
        itself (and the reduce when split): the same cache bytes and output as step."""
        kc, vc = self.sets[i % len(self.sets)]
        if self.verify:
            self.K.paged_attn_e4m3_verify_append(self.q, self.k_new, self.v_new, self.cu_q, self.max_q, kc, vc,
                                                 self.block_table, self.seq_lens, self.ks, self.vs, self.sm,
                                                 num_splits=self.S, workspace=self.ws, out=self.out)
        else:
            self.K.paged_attn_e4m3_decode_append(self.q, self.k_new, self.v_new, kc, vc, self.block_table,
                                                 self.seq_lens, self.ks, self.vs, self.sm, num_splits=self.S,
                                                 workspace=self.ws, out=self.out)

    def capture(self, fn, count):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)  # warm the launch path outside the capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(count):
                    fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def time_steps(self, steps, warmup, fused=False):
        """Exactly `steps` graph-replayed steps; returns (seconds per step, out).
        The steps are captured as whole rotations of the cache copies, up to
        STEPS_PER_GRAPH steps in one graph (as a captured multi-layer decode
        would run them); the rest run as one-rotation graphs and, for a last
        partial rotation, single-step graphs."""
        torch = self.torch
        n = len(self.sets)
        fn = self.step_fused if fused else self.step
        per_graph = n * max(1, min(steps // n, STEPS_PER_GRAPH // n))
        full = self.capture(fn, per_graph)
        rotation = self.capture(fn, n) if per_graph > n else full
        singles = [self.capture(lambda i, j=j: fn(j), 1) for j in range(n)]
        for w in range(warmup):
            singles[w % n].replay()
        torch.cuda.synchronize()
        # the graphs must reproduce the eager result exactly
        fn(0)
        torch.cuda.synchronize()
        eager = self.out.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        done = 0
        while done + per_graph <= steps:
            full.replay()
            done += per_graph
        while done + n <= steps:
            rotation.replay()
            done += n
        while done < steps:
            singles[done % n].replay()
            done += 1
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu = e0.elapsed_time(e1) / 1e3
        singles[0].replay()
        torch.cuda.synchronize()
        replay_matches = bool(torch.equal(self.out, eager))
        return max(gpu, 0.0) / steps, wall / steps, replay_matches

    def time_attention_kernel(self, launches, replays=5):
        """Average attention-kernel duration from HIP events around `replays`
        back-to-back replays of a graph of `launches` attention launches."""
        torch = self.torch
        g = self.capture(self.attend, launches)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (launches * replays)


    def _time_graph(self, fn, launches, replays=5):
        """Average duration of fn(i) from HIP events around `replays` replays of
        a graph of `launches` back-to-back calls."""
        torch = self.torch
        g = self.capture(fn, launches)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (launches * replays)

    def time_reduce(self, launches=60):
        """The split reduce on its own (the partials of the last attention call
        stay in the workspace)."""
        if self.S == 1:
            return None
        self._call(0, None)
        return self._time_graph(lambda i: self.K.split_reduce_fp32(self.ws_o, self.ws_m, self.ws_l, out=self.out),
                                launches)

    def saturated_codes(self):
        """Cache codes at +-448 (0x7E / 0xFE) over the workload's slots, K and V."""
        if self.f16:
            return None
        kc, vc = self.sets[0]
        pg = self.slots_all // self.P
        off = self.slots_all % self.P
        k = kc[pg, :, off, :]
        v = vc[pg, :, :, off]
        sat = int(((k & 0x7F) == 0x7E).sum().item() + ((v & 0x7F) == 0x7E).sum().item())
        return {"saturated": sat, "codes": int(k.numel() + v.numel()),
                "fraction": sat / float(k.numel() + v.numel())}

    def verify_flops(self):
        """4 * head_dim flops per visible (query token, key) pair and query head."""
        pairs = sum(causal_pairs(int(L), int(T)) for L, T in zip(self.bt.seq_lens, self.bt.q_lens))
        return 4 * self.D * self.Hq * pairs

    def time_buckets(self, launches=12):
        """The verify kernel on the sequences of each context length alone (the
        same pages, queries and cache sets), with its own split count."""
        torch, K, bt = self.torch, self.K, self.bt
        out = {}
        lens = bt.seq_lens.astype(np.int64)
        for L in sorted(set(int(x) for x in lens)):
            idx = np.nonzero(lens == L)[0]
            rows = np.concatenate([np.arange(bt.cu_q_lens[b], bt.cu_q_lens[b + 1]) for b in idx])
            ql = bt.q_lens[idx]
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)).cuda()
            q = self.q[torch.from_numpy(rows).cuda()].contiguous()
            btab = self.block_table[torch.from_numpy(idx).cuda()].contiguous()
            sl = self.seq_lens[torch.from_numpy(idx).cuda()].contiguous()
            S = K.default_splits(len(idx), self.Hkv, L, seq_lens=lens[idx], n_q_heads=self.Hq, q_len=int(ql.max()))
            ws = K.workspace(len(rows), self.Hq, self.D, S)
            o = torch.empty_like(q)
            n = len(self.sets)

            def call(i, q=q, cu=cu, btab=btab, sl=sl, S=S, ws=ws, o=o, mq=int(ql.max()), full=False):
                kc, vc = self.sets[i % n]
                kw = dict(num_splits=S, workspace=ws)
                kw.update(partials_only=True) if (S > 1 and not full) else kw.update(out=o)
                K.paged_attn_e4m3_verify(q, cu, mq, kc, vc, btab, sl, self.ks, self.vs, self.sm, **kw)

            nl = max(launches // n, 1) * n
            sec = self._time_graph(call, nl)
            step = self._time_graph(lambda i, c=call: c(i, full=True), nl)
            kv = int(L) * len(idx) * self.Hkv * self.D * 2
            out[str(L)] = {"sequences": int(len(idx)), "query_rows": int(len(rows)), "num_splits": int(S),
                           "kernel_us": sec * 1e6, "kv_gbs": kv / sec / 1e9,
                           "step_us": step * 1e6, "query_tokens_per_s_per_layer": len(rows) / step,
                           "step": "verify + reduce over this bucket's sequences alone"}
        return out

    def time_fill(self, k_src, v_src, launches=12, replays=3):
        """The cache-fill write (every token of the workload in one
        kv_quant_write launch, as a prefill writes its prompt): average duration
        from HIP events around graph replays of `launches` back-to-back fills
        rotated over the point's cache sets. Algorithmic bytes per launch: fp16
        K and V in, one E4M3 code each out, 8 slot bytes per token."""
        torch = self.torch
        n = len(self.sets)
        launches = max(launches // n, 1) * n

        def fill(i):
            kc, vc = self.sets[i % n]
            self.K.kv_quant_write(k_src, v_src, self.slots_all, self.ks, self.vs, kc, vc)

        g = self.capture(fill, launches)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / (launches * replays)
        tokens = int(k_src.shape[0])
        nbytes = tokens * self.Hkv * self.D * (2 + 2 + 1 + 1) + 8 * tokens
        return {"tokens": tokens, "launches": launches * replays, "kernel_us": sec * 1e6,
                "algorithmic_bytes": nbytes, "gbs": nbytes / sec / 1e9,
                "frac_of_hbm_peak": nbytes / sec / 1e9 / HBM_PEAK_GBS}


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA


def causal_pairs(seq_len, q_len):
    """(query token, visible key) pairs of one sequence's q_len query tokens."""
    return sum(seq_len - q_len + i + 1 for i in range(q_len))


class MixedLayer:
    """One layer of the mixed workload: 8 decode sequences at 8,192 keys plus one
    2,048-token chunk over 30,000 prior keys, sharing one cache."""

    def __init__(self, K, torch, scales, nsets=2):
        from synth import make_config
        self.K, self.torch = K, torch
        bt = make_config(5, layer=0)
        self.bt = bt
        dev = "cuda"
        self.ks, self.vs = scales
        self.sm = float(np.float32(1.0 / np.sqrt(bt.head_dim)))
        self.q_dec = torch.from_numpy(bt.q[:8]).to(dev)
        self.q_chunk = torch.from_numpy(bt.q[8:]).to(dev)
        bt_t = torch.from_numpy(bt.block_table).to(dev)
        sl = torch.from_numpy(bt.seq_lens).to(dev)
        self.bt_dec, self.bt_chunk = bt_t[:8].contiguous(), bt_t[8:].contiguous()
        self.sl_dec, self.sl_chunk = sl[:8].contiguous(), sl[8:].contiguous()
        self.cu_chunk = torch.tensor([0, 2048], dtype=torch.int32, device=dev)
        k_src = torch.from_numpy(bt.k).to(dev)
        v_src = torch.from_numpy(bt.v).to(dev)
        slots = torch.from_numpy(bt.slot_mapping).to(dev)
        new_rows = torch.from_numpy(bt.new_token_rows()).to(dev)
        self.k_new, self.v_new = k_src[new_rows].contiguous(), v_src[new_rows].contiguous()
        self.slots_new = slots[new_rows].contiguous()
        self.sets = []
        for _ in range(nsets):
            kc = torch.full((bt.num_pages, 4, 16, 128), 0x7F, dtype=torch.uint8, device=dev)
            vc = torch.full((bt.num_pages, 4, 128, 16), 0x7F, dtype=torch.uint8, device=dev)
            K.kv_quant_write(k_src, v_src, slots, self.ks, self.vs, kc, vc)
            self.sets.append((kc, vc))
        del k_src, v_src
        self.S = K.default_splits(8, 4, 8192)
        self.ws = K.workspace(8, 32, 128, self.S)
        self.ws_o, self.ws_m, self.ws_l = K.workspace_views(self.ws, 8, 32, 128, self.S)
        self.out_dec = torch.empty_like(self.q_dec)
        self.out_chunk = torch.empty_like(self.q_chunk)
        self.chunk_flops = 4 * 128 * 32 * causal_pairs(32048, 2048)
        self.dec_kv_bytes = 8 * 8192 * 4 * 128 * 2
        torch.cuda.synchronize()

    def chunk(self, i):
        kc, vc = self.sets[i % len(self.sets)]
        self.K.paged_attn_e4m3_verify(self.q_chunk, self.cu_chunk, 2048, kc, vc, self.bt_chunk,
                                      self.sl_chunk, self.ks, self.vs, self.sm, out=self.out_chunk)

    def step(self, i):
        kc, vc = self.sets[i % len(self.sets)]
        self.K.kv_quant_write(self.k_new, self.v_new, self.slots_new, self.ks, self.vs, kc, vc)
        self.K.paged_attn_e4m3_decode(self.q_dec, kc, vc, self.bt_dec, self.sl_dec, self.ks, self.vs, self.sm,
                                      num_splits=self.S, workspace=self.ws, out=self.out_dec)
        self.chunk(i)

    capture = Point.capture

    def time(self, steps):
        torch = self.torch
        n = len(self.sets)
        g = self.capture(self.step, n)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // n)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        step_s = e0.elapsed_time(e1) / 1e3 / (reps * n)
        gc = self.capture(self.chunk, n)
        gc.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            gc.replay()
        e1.record()
        torch.cuda.synchronize()
        chunk_s = e0.elapsed_time(e1) / 1e3 / (reps * n)
        return {
            "layer_step_us": step_s * 1e6, "steps": reps * n, "chunk_kernel_us": chunk_s * 1e6,
            "chunk_tflops": self.chunk_flops / chunk_s / 1e12,
            "chunk_mfma_util": self.chunk_flops / chunk_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "chunk_flops": self.chunk_flops, "decode_splits": self.S,
            "tokens_per_s_per_layer": (8 + 2048) / step_s,
            "24_layer_step_ms": 24 * step_s * 1e3,
        }



def dense_f16_gemm_rate(torch, n=8192, launches=20):
    """Achievable dense fp16 matrix-core rate on this GPU: torch.mm of two
    contiguous n x n fp16 matrices (the vendor GEMM library), HIP events around
    a graph of back-to-back products. A reference for the chunk kernel's
    matrix-core rate beside the 2.5 PFLOP/s datasheet figure."""
    a = torch.randn((n, n), dtype=torch.float16, device="cuda")
    b = torch.randn((n, n), dtype=torch.float16, device="cuda")
    c = torch.empty((n, n), dtype=torch.float16, device="cuda")
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / launches
    del a, b, c
    torch.cuda.empty_cache()
    return {"tflops": 2.0 * n ** 3 / sec / 1e12, "n": n, "us": sec * 1e6,
            "method": f"torch.mm fp16 {n}x{n}x{n}, mean of {launches} back-to-back launches"}


def cpu_baseline(seconds_target=10.0):
    """The fp64 oracle timed on host cores over sampled sequences of the 4k
    decode workload (same seeded inputs as the GPU run)."""
    from oracle import calibrate_amax, new_caches, paged_attention, quant_write
    from synth import make_config
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    bt = make_config(2)
    _, sc, _ = calibrate_amax(np.stack([bt.calib_k.reshape(-1), bt.calib_v.reshape(-1)]))
    sample = [0, 1, 2, 3]
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    for b in sample:
        s0, s1 = int(bt.cu_seq_lens[b]), int(bt.cu_seq_lens[b + 1])
        quant_write(bt.k[s0:s1], bt.v[s0:s1], bt.slot_mapping[s0:s1], sc[0], sc[1], kc, vc)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    reps = 0
    t0 = time.perf_counter()
    while True:
        paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm,
                        rows=sample)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds_target:
            break
    kv_bytes = reps * len(sample) * 4096 * bt.n_kv_heads * bt.head_dim * 2
    return {
        "value": kv_bytes / el / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle attention over {len(sample)} of the 32 sequences of the 4k decode "
                  f"workload, repeated {reps}x ({el:.1f} s); host os.cpu_count()={os.cpu_count()}",
        "tokens_per_s_per_layer": reps * len(sample) / el,
    }


# GPU clock cycles the stream is held before a timed calibration call (well
# over the host's time to queue the call's three kernels and its readback)
HOLD_CYCLES = 2_000_000


def _scan_call_seconds(K, torch, x, amax, scale):
    """One synchronous kv_calibrate_amax call, timed with HIP events on its
    stream. A spin kernel holds the stream first, so the call's kernels and its
    status readback are all queued before the start event is reached and run
    back to back: the interval holds them plus the host's return, not the
    host's launch latency, which would otherwise overlap a long scan but not a
    short one."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(HOLD_CYCLES)
    e0.record()
    K.kv_calibrate_amax(x, amax, scale)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


def streaming_read_ceiling(K, torch, elems_per_tensor=1 << 30, reps=15):
    """HBM streaming-read rate of committed code: the library's calibration
    scan (kv_calibrate_amax: contiguous fp16, 16-byte non-temporal loads, a
    packed max per element), timed as in _scan_call_seconds over two tensors
    of `elems_per_tensor` fp16 values each (4 GiB in all by default) and over
    the first half of the same memory (two tensors of half the length). The
    rate is the byte difference over the time difference, so every part of
    the call that does not grow with its input (the small kernels, the
    readback, the host's return, the scan's start-up and tail) cancels. The
    two sizes alternate for `reps` rounds and each takes its median, so that
    drift and single outliers move both alike."""
    big = torch.ones((2, elems_per_tensor), dtype=torch.float16, device="cuda")
    half = big.view(-1)[: elems_per_tensor].view(2, elems_per_tensor // 2)
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    scale = torch.empty(2, dtype=torch.float32, device="cuda")
    _scan_call_seconds(K, torch, big, amax, scale)  # warm-up
    tb, th = [], []
    for _ in range(reps):
        tb.append(_scan_call_seconds(K, torch, big, amax, scale))
        th.append(_scan_call_seconds(K, torch, half, amax, scale))
    t_big, t_half = float(np.median(tb)), float(np.median(th))
    nbytes, hbytes = big.numel() * 2, half.numel() * 2
    del big, half
    torch.cuda.empty_cache()
    return {"gbs": (nbytes - hbytes) / (t_big - t_half) / 1e9, "bytes": nbytes, "call_us": t_big * 1e6,
            "half_bytes": hbytes, "half_call_us": t_half * 1e6,
            "method": "kv_calibrate_amax over 2 x %d fp16 and over the first half of it (HIP events after a stream "
                      "hold), alternating for %d rounds; rate = byte difference / difference of the median times"
                      % (elems_per_tensor, reps)}


def same_size_scan(K, torch, nbytes, nsets=6, reps=12):
    """The calibration scan (as in streaming_read_ceiling) over exactly
    `nbytes` of fp16 in two tensors, rotated over `nsets` separate copies so
    that, like the attention points, no call finds its bytes in the caches
    (6 x 134 MB exceeds the 256 MB Infinity Cache): a plain contiguous read of
    the 4k decode's size, start-up and tail included. Its kernel's duration is
    read from a kernel trace of the run (rocprofv3), beside the attention
    kernel's; HIP events around the synchronous call cannot separate the scan
    kernel from the call's fixed part at this size (a few tens of microseconds
    either way), so no rate is derived here."""
    n = nbytes // 4
    bufs = [torch.ones((2, n), dtype=torch.float16, device="cuda") for _ in range(nsets)]
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    scale = torch.empty(2, dtype=torch.float32, device="cuda")
    for b in bufs:
        _scan_call_seconds(K, torch, b, amax, scale)  # warm-up, and evicts the first copies before the timed calls
    t = min(_scan_call_seconds(K, torch, bufs[i % nsets], amax, scale) for i in range(reps))
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": 4 * n, "copies": nsets, "calls": nsets + reps, "fastest_call_us": t * 1e6,
            "method": f"kv_calibrate_amax over 2 x {n} fp16 rotated over {nsets} copies; the call includes its "
                      f"readback and the host's return, the scan kernel's own duration is in a kernel trace"}


COPY_BYTES = 1 << 30
# steps captured in one graph by Point.time_steps (whole rotations of the cache copies)
STEPS_PER_GRAPH = 60


def counter_pass(K, torch, make_config, point="4k"):
    """Eager, unprofiled-timing launches for `rocprofv3 --pmc` runs. The copy
    reads and writes exactly COPY_BYTES, so its FETCH_SIZE / WRITE_SIZE readings
    give the scale from counter units to bytes. Then 12 attention launches of
    the 4k decode point (or the MTP3 verify point)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if point == "chunk":
        # the mixed workload's 2,048-token chunk over 30,000 prior keys (layer 0's scales)
        from synth.workloads import make_mixed_calibration
        _, scale, _ = K.kv_calibrate_amax(torch.from_numpy(make_mixed_calibration()[:2]).cuda())
        ml = MixedLayer(K, torch, (float(scale[0].item()), float(scale[1].item())))
        for i in range(12):
            ml.chunk(i)
        torch.cuda.synchronize()
        log(f"counter pass: copy {COPY_BYTES} B x3, 12 chunk attention launches ({ml.chunk_flops} flops each)")
        return
    bt = make_config(2 if point == "4k" else 3)
    k_src = torch.from_numpy(bt.k).cuda()
    v_src = torch.from_numpy(bt.v).cuda()
    calib = torch.from_numpy(np.stack([bt.calib_k.reshape(-1), bt.calib_v.reshape(-1)])).cuda()
    if point == "4k":
        S, nsets = K.default_splits(bt.batch, bt.n_kv_heads, 4096), 6
    else:
        S = K.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                             n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()))
        nsets = 3
    pt = Point(K, torch, point, bt, k_src, v_src, calib, S, nsets)
    for i in range(12):
        pt.attend(i)
    torch.cuda.synchronize()
    log(f"counter pass: copy {COPY_BYTES} B x3, 12 {point} attention launches (splits {S}, "
        f"algorithmic bytes {pt.alg_bytes})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--points", default="4k,32k,256k,mtp3,mixed,4k_p4,4k_tp4,4k_f16,mtp3_f16")
    ap.add_argument("--splits", type=int, default=0, help="splits of the 4k point (0: heuristic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-launches", type=int, default=60)
    ap.add_argument("--counter-pass", action="store_true",
                    help="eager launches for hardware-counter runs: a 1 GiB device copy "
                         "(reference for the byte counters), then 4k decode attention launches")
    ap.add_argument("--counter-point", default="4k", choices=("4k", "mtp3", "chunk"),
                    help="workload of the counter pass's attention launches")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the library runs on one GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_quantised_paged_amd import kvfp8 as K
    from synth import make_config
    from synth.device import normal_kv

    torch.cuda.set_device(0)
    if args.counter_pass:
        counter_pass(K, torch, make_config, args.counter_point)
        return
    points = [p for p in args.points.split(",") if p]
    results = {}

    for p in points:
        log(f"setting up point {p}")
        if p == "4k":
            bt = make_config(2)
            k_src = torch.from_numpy(bt.k).cuda()
            v_src = torch.from_numpy(bt.v).cuda()
            calib = torch.from_numpy(np.stack([bt.calib_k.reshape(-1), bt.calib_v.reshape(-1)])).cuda()
            S = args.splits or K.default_splits(bt.batch, bt.n_kv_heads, 4096)
            nsets, steps = 6, args.steps
        elif p == "32k":
            bt = make_config(2, seq_len_override=32768, values=False)
            total = int(bt.cu_seq_lens[-1])
            k_src = normal_kv(total, 4, 128, bt.seed * 10 + 1)
            v_src = normal_kv(total, 4, 128, bt.seed * 10 + 2)
            cal = normal_kv(2 * 2048, 4, 128, bt.seed * 10 + 3)
            calib = cal.view(2, -1)
            S = K.default_splits(bt.batch, bt.n_kv_heads, 32768)
            nsets, steps = 2, max(10, args.steps // 3)
        elif p == "4k_tp4":
            # one GPU's share of the 4k decode under four-way head parallelism: one kv-head and its
            # 8 query heads of every sequence (the other kv-heads live on the other GPUs)
            from synth import make_batch
            bt = make_batch([4096] * 32, [1] * 32, 8, 1, 128, 16, seed=20260002, name="decode_4k_tp4_share",
                            calib_tokens=2048, values=False)
            total = int(bt.cu_seq_lens[-1])
            k_src = normal_kv(total, 1, 128, bt.seed * 10 + 1)
            v_src = normal_kv(total, 1, 128, bt.seed * 10 + 2)
            cal = normal_kv(2 * 2048, 1, 128, bt.seed * 10 + 3)
            calib = cal.view(2, -1)
            S = K.default_splits(bt.batch, bt.n_kv_heads, 4096)
            nsets, steps = 12, args.steps
        elif p == "4k_p4":
            # derived: the 4k decode shape with the pages' grouped page-size-4 layout
            bt = make_config(2, values=False, page_size_override=4)
            total = int(bt.cu_seq_lens[-1])
            k_src = normal_kv(total, 4, 128, bt.seed * 10 + 1)
            v_src = normal_kv(total, 4, 128, bt.seed * 10 + 2)
            cal = normal_kv(2 * 2048, 4, 128, bt.seed * 10 + 3)
            calib = cal.view(2, -1)
            S = K.default_splits(bt.batch, bt.n_kv_heads, 4096)
            nsets, steps = 6, args.steps
        elif p in ("4k_f16", "mtp3_f16"):
            # the fp16-cache arm of the format comparison, on the 4k decode and MTP3 shapes
            bt = make_config(2 if p == "4k_f16" else 3, values=False)
            total = int(bt.cu_seq_lens[-1])
            k_src = normal_kv(total, 4, 128, bt.seed * 10 + 1)
            v_src = normal_kv(total, 4, 128, bt.seed * 10 + 2)
            calib = None
            S = (K.default_splits(bt.batch, bt.n_kv_heads, 4096, kv_elem_bytes=2) if p == "4k_f16" else
                 K.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                                  n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()), kv_elem_bytes=2))
            nsets, steps = (6, args.steps) if p == "4k_f16" else (3, max(10, args.steps // 3))
        elif p == "mtp3":
            bt = make_config(3)
            k_src = torch.from_numpy(bt.k).cuda()
            v_src = torch.from_numpy(bt.v).cuda()
            calib = torch.from_numpy(np.stack([bt.calib_k.reshape(-1), bt.calib_v.reshape(-1)])).cuda()
            S = K.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                                 n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()))
            nsets, steps = 3, max(10, args.steps // 3)  # 3 x 189 MB of KV: no set stays in the 256 MB MALL
        elif p == "mixed":
            from synth.workloads import make_mixed_calibration
            calib = torch.from_numpy(make_mixed_calibration()).cuda()
            # kv_calibrate_amax is synchronous (it reads the status back), so this
            # is host-inclusive: the fastest of five calls
            cal_us = float("inf")
            for _ in range(5):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                amax, scale, _ = K.kv_calibrate_amax(calib)
                cal_us = min(cal_us, (time.perf_counter() - t0) * 1e6)
            scales = (float(scale[0].item()), float(scale[1].item()))
            del calib
            ml = MixedLayer(K, torch, scales)
            r = ml.time(max(10, args.steps // 3))
            gemm = dense_f16_gemm_rate(torch)
            r["dense_f16_gemm_reference"] = gemm
            r["chunk_frac_of_dense_gemm_rate"] = r["chunk_tflops"] / gemm["tflops"]
            r["calibration_us_48_tensors_host_inclusive"] = cal_us
            r["calibration_gbs"] = 48 * 4096 * 512 * 2 / (cal_us * 1e-6) / 1e9
            results[p] = r
            log(f"{p}: {json.dumps(r)}")
            del ml
            torch.cuda.empty_cache()
            continue
        elif p == "256k":
            bt = make_config(4, values=False)
            total = int(bt.cu_seq_lens[-1])
            k_src = normal_kv(total, 4, 128, bt.seed * 10 + 1, bt.outlier_channels_k)
            v_src = normal_kv(total, 4, 128, bt.seed * 10 + 2, bt.outlier_channels_v)
            ck = normal_kv(2048, 4, 128, bt.seed * 10 + 3, bt.outlier_channels_k)
            cv = normal_kv(2048, 4, 128, bt.seed * 10 + 4, bt.outlier_channels_v)
            calib = torch.stack([ck.reshape(-1), cv.reshape(-1)])
            S = 64
            nsets, steps = 2, max(10, args.steps // 3)
        else:
            raise SystemExit(f"unknown point {p}")
        pt = Point(K, torch, p, bt, k_src, v_src, calib, S, nsets, f16=p.endswith("_f16"))
        fill = pt.time_fill(k_src, v_src) if p == "4k" else None
        if fill is not None:
            log(f"{p}: cache-fill write {json.dumps(fill)}")
        del k_src, v_src
        torch.cuda.empty_cache()
        log(f"{p}: batch {pt.B} splits {S} kv bytes {pt.kv_bytes}; timing {steps} steps")
        sec_sep, wall_sep, same_sep = pt.time_steps(steps, args.warmup)
        if pt.f16:
            sec, wall, same = sec_sep, wall_sep, same_sep
        else:
            sec, wall, same = pt.time_steps(steps, args.warmup, fused=True)
            same = same and same_sep
        launches = args.kernel_launches if p == "4k" else max(6, args.kernel_launches // 6)
        launches = max(launches // nsets, 1) * nsets
        kern = pt.time_attention_kernel(launches)
        results[p] = {
            "batch": pt.B, "seq_len": int(bt.seq_lens.max()), "num_splits": S, "page_size": pt.P,
            "query_rows": pt.rows,
            "steps": steps, "ms_per_step": sec * 1e3, "host_ms_per_step": wall * 1e3,
            "kv_bytes_per_step": pt.kv_bytes, "algorithmic_bytes_per_step": pt.alg_bytes,
            "kv_gbs": pt.kv_bytes / sec / 1e9, "tokens_per_s_per_layer": pt.rows / sec,
            "ms_per_step_separate_write": sec_sep * 1e3,
            "step": ("attention + reduce over fp16 pages (no write)" if pt.f16 else
                     "attention with the new tokens appended"),
            "kv_cache": "fp16" if pt.f16 else "e4m3",
            "attn_kernel_us": kern * 1e6, "attn_kernel_gbs": pt.alg_bytes / kern / 1e9,
            "attn_kernel": K.kvfp8_attn_kernel_name(pt.B, pt.Hq, pt.Hkv, pt.D, pt.P, bt.max_pages, pt.max_q, S,
                                                    pt.f16),
            "graph_replay_matches_eager": same, "cache_sets": nsets,
        }
        if fill is not None:
            results[p]["cache_fill_write"] = fill
        red = pt.time_reduce()
        if red is not None:
            results[p]["reduce_us"] = red * 1e6
        sat = pt.saturated_codes()
        if sat is not None:
            results[p]["saturated_codes"] = sat
        if p == "mtp3":
            fl = pt.verify_flops()
            results[p]["mfma_tflops"] = fl / kern / 1e12
            results[p]["mfma_util"] = fl / kern / 1e12 / MFMA_F16_PEAK_TFLOPS
            results[p]["buckets"] = pt.time_buckets()
        log(f"{p}: {json.dumps(results[p])}")
        del pt
        torch.cuda.empty_cache()

    main = results.get("4k")
    if main is None:  # the headline is the 4k decode point; report what was measured
        print(json.dumps({"metric": METRIC, "note": "headline needs the 4k point", "points": results}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline()
    achieved = main["attn_kernel_gbs"]
    log("measuring the streaming-read ceiling")
    ceiling = streaming_read_ceiling(K, torch)
    log(f"streaming-read ceiling: {json.dumps(ceiling)}")
    # the same scan over the 4k decode's K/V bytes: a plain read of that size (kernel duration from a trace)
    same = same_size_scan(K, torch, main["kv_bytes_per_step"])
    log(f"same-size scan: {json.dumps(same)}")
    tps = {}
    for p, key in (("4k", "4k"), ("32k", "32k_derived_decode_b32"), ("256k", "256k")):
        if p in results:
            tps[key] = results[p]["tokens_per_s_per_layer"]
    bucket = results.get("mtp3", {}).get("buckets", {}).get("32768")
    if bucket is not None:
        tps["32k_mtp3_bucket_query_tokens"] = bucket["query_tokens_per_s_per_layer"]
    line = {
        "metric": METRIC,
        "value": main["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": main["steps"],
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_b32_ctx4096_h32kv4_d128_p16_e4m3", "batch": main["batch"],
                   "seq_len": main["seq_len"], "n_q_heads": 32, "n_kv_heads": 4, "head_dim": 128,
                   "page_size": main["page_size"], "num_splits": main["num_splits"],
                   "kv_cache": "e4m3 (OCP), per-layer K/V scales", "accumulate": "f32"},
        "pct_hbm_peak": 100.0 * main["kv_gbs"] / HBM_PEAK_GBS,
        "tokens_per_s_per_layer": tps,
        "tokens_per_s_note": ("4k and 256k: the decode workloads; 32k_derived_decode_b32: the 4k decode shape at "
                              "32,768 keys (derived, not one of the five workloads); "
                              "32k_mtp3_bucket_query_tokens: the MTP3 workload's 32,768-key sequences alone "
                              "(query tokens through verify + reduce)"),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": main["attn_kernel"], "kernel_us": main["attn_kernel_us"],
                     "measured_streaming_read_gbs": ceiling["gbs"],
                     "frac_of_measured_streaming_read": achieved / ceiling["gbs"],
                     "streaming_read": ceiling,
                     "same_size_scan": same},
        "cpu_baseline": cpu,
        "points": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
