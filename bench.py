"""Benchmark of the paged-KV attention hot path on one MI355X.

Default run: the five workloads of the build's contract, each timed, checked and set
against its roofline, in one JSON line:
  single  - single-request decode, kv_len 1024, 32/32 heads, fp16, contiguous KV;
  decode  - batch paged decode, 64 requests, kv_len U[512, 4096], 32/8 heads, fp16,
            16-token pages (the headline: `value` is its HBM throughput);
  prefill - batch paged causal prefill, 16 requests, qo U[128, 1024] after a prefix
            U[0, 2048], 32/8 heads, bf16;
  cascade - 128 decode requests sharing an 8192-token prefix, suffix U[64, 1024], fp16;
  long    - long-context split-KV decode, 4 x 131072 tokens, 64/8 heads, bf16, P = 64.
A step is one run of the workload's planned pass (every kernel of it) over the whole
batch; the host plan is made once before timing and reused, as the plan/run split
intends, and its host time is reported as plan_us (median of 20 plan calls).

Timing: W warm-up steps, then K timed steps. Before every step a 512 MiB buffer is read
(outside the timed events) so the 256 MB Infinity Cache holds no KV and no dirty lines;
each step is bracketed by HIP events on the stream the kernels run on, and the whole pass
by a device synchronize. `value` and `ms_per_step` use the median step (the mean is
reported beside it). The attention kernel alone (the roofline figure) is timed in a second
pass of K steps by a pair of events its own dispatch carries (hipExtLaunchKernel), the
interval rocprofv3's kernel trace reports; those events lengthen a step by a few
microseconds, so step times come from the first pass.

After timing, the output buffers of the last timed step are compared with the fp64
oracle on every row (max |dO| and max |dLSE| in the line, against the tolerances), and
the oracle is timed on the host cores on a bounded sample of the same workload
(`cpu_baseline`). Neither touches the timed region.

`--workload X` measures one workload (also append, block_sparse, pod, decode_variants,
prefill_variants); `--all` adds those five to the default five.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA, TFLOP/s

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources the decode kernel and its plan come from; a traffic figure in profiles/
# is used only while their hash matches the one recorded next to it.
DECODE_SOURCES = ["paged_kv_cache_173_amd/csrc/decode.hip",
                  "paged_kv_cache_173_amd/csrc/decode_item.h",
                  "paged_kv_cache_173_amd/csrc/device_common.h",
                  "paged_kv_cache_173_amd/csrc/kernels.h",
                  "paged_kv_cache_173_amd/csrc/planner.cpp",
                  "paged_kv_cache_173_amd/csrc/api.cpp"]
TRAFFIC_PROFILE = "profiles/decode_kernel_batch64_fp16_hbm_traffic.md"


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic():
    """HBM bytes per decode-kernel launch measured by rocprofv3 counters, or None
    when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip().strip("`- ")] = v.strip().strip("`")
    if fields.get("source_sha256") != decode_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# algorithmic work per run: bytes that must cross HBM, flops of visible pairs
# ----------------------------------------------------------------------------
def decode_bytes(kv_lens, Hkv, D, elem, B, Hq):
    """K + V rows read once per (request, KV head), plus q, o and LSE."""
    kv = int(np.sum(kv_lens)) * Hkv * D * elem * 2
    return kv + B * Hq * D * elem * 2 + B * Hq * 4


def prefill_flops(qo_lens, kv_lens, Hq, D, causal, window_left=-1):
    """4 * D * Hq * (number of visible (query, key) pairs); with a sliding window the
    query at position p sees keys max(0, p - W) .. p (causal) or .. L - 1."""
    pairs = 0
    for Q, L in zip(qo_lens, kv_lens):
        Q, L = int(Q), int(L)
        if window_left < 0:
            pairs += Q * (L - Q) + Q * (Q + 1) // 2 if causal else Q * L
            continue
        p = np.arange(Q, dtype=np.int64) + (L - Q)
        hi = np.minimum(p, L - 1) if causal else np.full(Q, L - 1, np.int64)
        lo = np.maximum(p - window_left, 0)
        pairs += int(np.sum(np.maximum(hi - lo + 1, 0)))
    return 4.0 * D * Hq * pairs


def prefill_bytes(w):
    q = w.q.size * 2
    kv = int(np.sum(w.kv.kv_lens)) * w.num_kv_heads * w.head_dim * 2 * 2
    return q * 2 + kv + w.q.shape[0] * w.num_qo_heads * 4


# ----------------------------------------------------------------------------
# runners
# ----------------------------------------------------------------------------
class Runner:
    """Uploads one workload, plans once, and exposes step() = one run."""

    def __init__(self, name, w, pkv, torch):
        self.name, self.w, self.pkv, self.torch = name, w, pkv, torch
        dt = torch.float16 if w.dtype == "f16" else torch.bfloat16

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to("cuda")

        def dev_i32(a):
            a = np.asarray(a, np.int32)
            return torch.from_numpy(a if a.size else np.zeros(1, np.int32)).to("cuda")

        if w.kind == "block_sparse":
            self.q, self.k, self.v = dev(w.q), dev(w.k), dev(w.v)
            self.ip, self.ix = dev_i32(w.bsr_indptr), dev_i32(w.bsr_indices)
            self.ws = pkv.Workspace()
            self.dt = dt
            self.o = torch.empty_like(self.q)
            self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
            self.plan_us = self._time_plan()
            return
        if w.kind == "pod":
            wp, wd = w.prefill, w.decode
            self.k, self.v = dev(wp.kv.k_cache), dev(wp.kv.v_cache)
            self.q_p, self.q_d = dev(wp.q), dev(wd.q)
            self.qo = dev_i32(wp.qo_indptr)
            self.ip, self.ix = dev_i32(wp.kv.kv_indptr), dev_i32(wp.kv.kv_indices)
            self.dp, self.dx = dev_i32(wd.kv.kv_indptr), dev_i32(wd.kv.kv_indices)
            self.o_p, self.o_d = torch.empty_like(self.q_p), torch.empty_like(self.q_d)
            self.l_p = torch.empty(self.q_p.shape[:2], dtype=torch.float32, device="cuda")
            self.l_d = torch.empty(self.q_d.shape[:2], dtype=torch.float32, device="cuda")
            self.ws, self.ws_p, self.ws_d = pkv.Workspace(), pkv.Workspace(), pkv.Workspace()
            self.dt = dt
            self.sequential = False     # True: the same parts as separate prefill + decode runs
            self.plan_us = self._time_plan()
            return
        if w.kind == "append":
            self.ak, self.av = dev(w.append_k), dev(w.append_v)
            self.k, self.v = dev(w.kv.k_cache), dev(w.kv.v_cache)
            bi, pos = pkv.pkv_append_positions(w.append_indptr, w.kv.kv_indptr,
                                               w.kv.last_page_len, w.kv.page_size)
            self.bi, self.pos = dev_i32(bi), dev_i32(pos)
            self.kv_indptr, self.kv_indices = dev_i32(w.kv.kv_indptr), dev_i32(w.kv.kv_indices)
            self.lpl = dev_i32(w.kv.last_page_len)
            self.plan_us = 0.0
            return
        self.q = dev(w.q)
        self.ws = pkv.Workspace()
        var = w.meta.get("variant") or {}
        self.window_left = int(var.get("window_left", -1))
        self.soft_cap = float(var.get("logits_soft_cap", 0.0))
        self.sinks = (torch.from_numpy(np.asarray(var["sinks"], np.float32)).to("cuda")
                      if var.get("sinks") is not None else None)
        if w.kind == "single_decode":
            self.k, self.v = dev(w.k), dev(w.v)
            self.o = torch.empty_like(self.q)
            self.lse = torch.empty(self.q.shape[:1], dtype=torch.float32, device="cuda")
        else:
            self.k, self.v = dev(w.kv.k_cache), dev(w.kv.v_cache)
            self.kv_indptr, self.kv_indices = dev_i32(w.kv.kv_indptr), dev_i32(w.kv.kv_indices)
            self.o = torch.empty_like(self.q)
            self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
            if w.kind == "prefill":
                self.qo_indptr = dev_i32(w.qo_indptr)
            if w.kind == "cascade":
                self.prefix = dev_i32(w.prefix_indices)
        self.dt = dt
        self.plan_us = self._time_plan()

    def _time_plan(self, calls=20):
        """Steady-state host time of one plan call (the median of `calls` calls after two
        untimed ones, each on an idle stream): the host rule, the table writes and queuing
        the table copy; the copy itself runs on the stream after the call returns."""
        torch = self.torch
        self._plan()
        self._plan(timing_only=True)
        times = []
        for _ in range(calls):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            self._plan(timing_only=True)
            times.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        return float(np.median(times)) * 1e6

    def _plan(self, timing_only=False):
        w, pkv, torch, dt = self.w, self.pkv, self.torch, self.dt
        if w.kind == "pod":
            wp, wd = w.prefill, w.decode
            Hq, Hkv, P = wp.num_qo_heads, wp.num_kv_heads, wp.kv.page_size
            self.plan = pkv.pkv_pod_plan(wp.qo_indptr, wp.kv.kv_indptr, wp.kv.last_page_len,
                                         wp.causal, wd.kv.kv_indptr, wd.kv.last_page_len, Hq, Hkv,
                                         wp.head_dim, P, dt, self.ws)
            if timing_only:   # the timed plan is the one-launch plan alone
                return
            self.plan_p = pkv.pkv_prefill_plan(wp.qo_indptr, wp.kv.kv_indptr, wp.kv.last_page_len,
                                               Hq, Hkv, wp.head_dim, P, dt, wp.causal, self.ws_p)
            self.plan_d = pkv.pkv_decode_plan(wd.kv.kv_indptr, wd.kv.last_page_len, Hq, Hkv,
                                              wd.head_dim, P, dt, self.ws_d)
        elif w.kind == "block_sparse":
            self.plan = pkv.pkv_block_sparse_plan(w.bsr_indptr, w.bsr_indices, w.q.shape[0],
                                                  w.k.shape[0], w.row_block, w.col_block,
                                                  w.num_qo_heads, w.num_kv_heads, w.head_dim, dt,
                                                  self.ws)
        elif w.kind == "single_decode":
            need = pkv._I64(0)
            pkv._lib_single_decode(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                   w.k.shape[0], w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                   pkv.dtype_code(dt), w.sm_scale, None, None, 0,
                                   pkv.ctypes.byref(need), None, None, None)
            self.fws = torch.empty(max(need.value, 16), dtype=torch.uint8, device="cuda")
            self.plan = None
        elif w.kind == "decode":
            self.plan = pkv.pkv_decode_plan(w.kv.kv_indptr, w.kv.last_page_len, w.num_qo_heads,
                                            w.num_kv_heads, w.head_dim, w.kv.page_size, dt,
                                            self.ws, window_left=self.window_left)
        elif w.kind == "prefill":
            self.plan = pkv.pkv_prefill_plan(w.qo_indptr, w.kv.kv_indptr, w.kv.last_page_len,
                                             w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                             w.kv.page_size, dt, w.causal, self.ws,
                                             window_left=self.window_left)
        else:
            self.plan = pkv.pkv_cascade_plan(len(w.prefix_indices), w.prefix_last_page_len,
                                             w.kv.kv_indptr, w.kv.last_page_len, w.num_qo_heads,
                                             w.num_kv_heads, w.head_dim, w.kv.page_size, dt,
                                             self.ws)

    def step(self, kernel_events=None):
        """One run; `kernel_events` (decode / prefill / mixed: a (start, done) pair of
        torch.cuda.Events, or None) ride on the attention kernel's own dispatch and take
        its begin and end timestamps (the merge of split chunks is not included)."""
        p, w = self.pkv, self.w
        attention_start, attention_done = kernel_events or (None, None)
        if w.kind == "pod" and self.sequential:
            p.pkv_prefill_run(self.plan_p, self.q_p, self.k, self.v, self.qo, self.ip, self.ix,
                              w.prefill.sm_scale, o=self.o_p, lse=self.l_p)
            p.pkv_decode_run_timed(self.plan_d, self.q_d, self.k, self.v, self.dp, self.dx,
                                   w.decode.sm_scale, attention_start, attention_done,
                                   o=self.o_d, lse=self.l_d)
        elif w.kind == "pod":
            p.pkv_pod_run(self.plan, self.k, self.v, self.q_p, self.qo, self.ip, self.ix, self.q_d,
                          self.dp, self.dx, w.prefill.sm_scale, o_p=self.o_p, lse_p=self.l_p,
                          o_d=self.o_d, lse_d=self.l_d, attention_start=attention_start,
                          attention_done=attention_done)
        elif w.kind == "block_sparse":
            p.pkv_block_sparse_run(self.plan, self.q, self.k, self.v, self.ip, self.ix,
                                   w.sm_scale, o=self.o, lse=self.lse)
        elif w.kind == "append":
            p.pkv_append_paged_kv(self.ak, self.av, self.bi, self.pos, self.k, self.v,
                                  self.kv_indptr, self.kv_indices, self.lpl)
        elif w.kind == "single_decode":
            p.pkv_single_decode(self.q, self.k, self.v, w.sm_scale, float_ws=self.fws, o=self.o,
                                lse=self.lse)
        elif w.kind == "decode":
            p.pkv_decode_run_timed(self.plan, self.q, self.k, self.v, self.kv_indptr,
                                   self.kv_indices, w.sm_scale, attention_start, attention_done,
                                   o=self.o,
                                   lse=self.lse, window_left=self.window_left,
                                   logits_soft_cap=self.soft_cap, sinks=self.sinks)
        elif w.kind == "prefill":
            p.pkv_prefill_run_timed(self.plan, self.q, self.k, self.v, self.qo_indptr,
                                    self.kv_indptr, self.kv_indices, w.sm_scale, attention_start,
                                    attention_done, o=self.o, lse=self.lse,
                                    window_left=self.window_left, logits_soft_cap=self.soft_cap,
                                    sinks=self.sinks)
        else:
            p.pkv_cascade_run(self.plan, self.q, self.k, self.v, self.prefix, self.kv_indptr,
                              self.kv_indices, w.sm_scale, o=self.o, lse=self.lse)

    def work(self):
        """(algorithmic bytes, algorithmic flops, tokens) of one step."""
        w = self.w
        if w.kind == "pod":
            wp, wd = w.prefill, w.decode
            fp = prefill_flops(wp.meta["qo_lens"], wp.kv.kv_lens, wp.num_qo_heads, wp.head_dim,
                               wp.causal)
            B = len(wd.kv.kv_lens)
            bd = decode_bytes(wd.kv.kv_lens, wd.num_kv_heads, wd.head_dim, 2, B, wd.num_qo_heads)
            fd = 4.0 * wd.num_qo_heads * wd.head_dim * float(np.sum(wd.kv.kv_lens))
            return prefill_bytes(wp) + bd, fp + fd, int(np.sum(wp.meta["qo_lens"])) + B
        if w.kind == "block_sparse":
            R, C, Nq, Nkv = w.row_block, w.col_block, w.q.shape[0], w.k.shape[0]
            pairs = 0
            for i in range(len(w.bsr_indptr) - 1):
                rows = min(R, Nq - i * R)
                cols = w.bsr_indices[w.bsr_indptr[i]:w.bsr_indptr[i + 1]]
                pairs += rows * int(np.sum(np.minimum(C, Nkv - cols * C)))
            f = 4.0 * w.head_dim * w.num_qo_heads * pairs
            b = w.q.size * 2 * 2 + w.k.size * 2 * 2 + Nq * w.num_qo_heads * 4
            return b, f, Nq
        if w.kind == "append":
            nnz = w.append_k.shape[0]
            row = w.append_k.shape[1] * w.append_k.shape[2] * 2      # bytes of one K (or V) row
            # K and V rows read once and written once, plus the two int32 index arrays
            return 4 * nnz * row + 8 * nnz, 0.0, nnz
        if w.kind == "single_decode":
            L = w.k.shape[0]
            b = decode_bytes([L], w.num_kv_heads, w.head_dim, 2, 1, w.num_qo_heads)
            return b, 4.0 * w.num_qo_heads * w.head_dim * L, 1
        if w.kind == "decode":
            B = len(w.kv.kv_lens)
            # with a sliding window a request needs only its last W + 1 keys
            seen = (w.kv.kv_lens if self.window_left < 0 else
                    np.minimum(w.kv.kv_lens, self.window_left + 1))
            b = decode_bytes(seen, w.num_kv_heads, w.head_dim, 2, B, w.num_qo_heads)
            return b, 4.0 * w.num_qo_heads * w.head_dim * float(np.sum(seen)), B
        if w.kind == "prefill":
            f = prefill_flops(w.meta["qo_lens"], w.kv.kv_lens, w.num_qo_heads, w.head_dim,
                              w.causal, self.window_left)
            return prefill_bytes(w), f, int(np.sum(w.meta["qo_lens"]))
        B = len(w.kv.kv_lens)
        pre = w.meta["prefix_len"]
        suf = w.kv.kv_lens
        b = (pre + int(np.sum(suf))) * w.num_kv_heads * w.head_dim * 2 * 2 + \
            B * w.num_qo_heads * w.head_dim * 2 * 2 + B * w.num_qo_heads * 4
        f = 4.0 * w.num_qo_heads * w.head_dim * B * pre + \
            4.0 * w.num_qo_heads * w.head_dim * float(np.sum(suf))
        return b, f, B


def time_steps(torch, runner, steps, warmup, flush):
    """Returns (step ms list, attention-kernel ms list or None, wall s of the step pass).

    The K timed steps carry only the step's own pair of events. The attention kernel's
    time comes from a second pass of K steps in which the kernel's dispatch also carries
    a pair of events (its begin and end timestamps); those events lengthen a step by a few
    microseconds, so they stay out of the pass that gives the step time."""
    def evict():
        return flush.view(torch.int64).sum()

    timed_kernel = runner.w.kind in ("decode", "prefill", "pod")

    def event():
        return torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        evict()
        runner.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [event() for _ in range(steps)]
    ends = [event() for _ in range(steps)]
    for ev in starts + ends:                 # create the events before the timed loop
        ev.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evict()                              # evicts the Infinity Cache, outside the events
        starts[i].record(stream)
        runner.step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern = None
    if timed_kernel:
        k_begin = [event() for _ in range(steps)]
        k_end = [event() for _ in range(steps)]
        for ev in k_begin + k_end:
            ev.record(stream)
        torch.cuda.synchronize()
        for i in range(steps):
            evict()
            runner.step((k_begin[i], k_end[i]))
        torch.cuda.synchronize()
        kern = [b.elapsed_time(e) for b, e in zip(k_begin, k_end)]
    return ms, kern, wall


# fp16: O <= 2e-3, LSE <= 1e-3; bf16: O <= 1e-2, LSE <= 2e-3 (max abs error against the oracle)
TOL = {"f16": (2e-3, 1e-3), "bf16": (1e-2, 2e-3)}


def _errors(o, lse, O, LSE):
    """(max |dO|, max |dLSE| over rows the oracle gives a finite LSE, -inf rows agree)."""
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    inf_ref = np.isneginf(LSE)
    agree = bool(np.array_equal(np.isneginf(lse), inf_ref)) and not np.isnan(o).any()
    d_o = float(np.max(np.abs(o - O))) if o.size else 0.0
    fin = ~inf_ref
    d_l = float(np.max(np.abs(lse[fin] - LSE[fin]))) if fin.any() else 0.0
    return d_o, d_l, agree


def parity(runner):
    """The output buffers of the last timed step against the fp64 oracle, on every row
    (append: every byte of both page pools)."""
    import oracle
    torch, w = runner.torch, runner.w

    def host(t):
        return t.float().cpu().numpy().astype(np.float64)

    if torch.cuda.is_available():
        torch.cuda.synchronize()
    if w.kind == "append":
        kv = w.kv
        bi, pos = oracle.append_positions(w.append_indptr, kv.kv_indptr, kv.last_page_len,
                                          kv.page_size)
        K, V = oracle.append_paged_kv(kv.k_cache, kv.v_cache, w.append_k, w.append_v, bi, pos,
                                      kv.kv_indptr, kv.kv_indices, kv.last_page_len)
        same = (np.array_equal(runner.k.view(torch.int16).cpu().numpy().view(np.uint16), K) and
                np.array_equal(runner.v.view(torch.int16).cpu().numpy().view(np.uint16), V))
        return {"bit_exact": bool(same), "bytes_compared": int(K.nbytes + V.nbytes), "ok": same}
    var = w.meta.get("variant", {}) if w.kind in ("decode", "prefill") else {}
    win = int(var.get("window_left", -1))
    cap = float(var.get("logits_soft_cap", 0.0))
    sinks = var.get("sinks")
    pairs = []
    if w.kind == "pod":
        wp, wd = w.prefill, w.decode
        pairs.append((runner.o_p, runner.l_p, oracle.batch_prefill(
            wp.q, wp.kv.k_cache, wp.kv.v_cache, wp.qo_indptr, wp.kv.kv_indptr,
            wp.kv.kv_indices, wp.kv.last_page_len, wp.dtype, wp.sm_scale, wp.causal)))
        pairs.append((runner.o_d, runner.l_d, oracle.batch_decode(
            wd.q, wd.kv.k_cache, wd.kv.v_cache, wd.kv.kv_indptr, wd.kv.kv_indices,
            wd.kv.last_page_len, wd.dtype, wd.sm_scale)))
    elif w.kind == "single_decode":
        pairs.append((runner.o, runner.lse, oracle.single_decode(w.q, w.k, w.v, w.dtype,
                                                                 w.sm_scale)))
    elif w.kind == "block_sparse":
        pairs.append((runner.o, runner.lse, oracle.block_sparse_attention(
            w.q, w.k, w.v, w.dtype, w.bsr_indptr, w.bsr_indices, w.row_block, w.col_block,
            w.sm_scale)))
    elif w.kind == "cascade":
        kv = w.kv
        pairs.append((runner.o, runner.lse, oracle.cascade_decode(
            w.q, kv.k_cache, kv.v_cache, w.prefix_indices, w.prefix_last_page_len,
            kv.kv_indptr, kv.kv_indices, kv.last_page_len, w.dtype, w.sm_scale)))
    elif w.kind == "decode":
        kv = w.kv
        if win >= 0 or cap > 0 or sinks is not None:
            ref = oracle.batch_decode_variant(w.q, kv.k_cache, kv.v_cache, kv.kv_indptr,
                                              kv.kv_indices, kv.last_page_len, w.dtype,
                                              w.sm_scale, win, cap, sinks)
        else:
            ref = oracle.batch_decode(w.q, kv.k_cache, kv.v_cache, kv.kv_indptr, kv.kv_indices,
                                      kv.last_page_len, w.dtype, w.sm_scale)
        pairs.append((runner.o, runner.lse, ref))
    else:
        kv = w.kv
        if win >= 0 or cap > 0 or sinks is not None:
            ref = oracle.batch_prefill_variant(w.q, kv.k_cache, kv.v_cache, w.qo_indptr,
                                               kv.kv_indptr, kv.kv_indices, kv.last_page_len,
                                               w.dtype, w.sm_scale, w.causal, win, cap, sinks)
        else:
            ref = oracle.batch_prefill(w.q, kv.k_cache, kv.v_cache, w.qo_indptr, kv.kv_indptr,
                                       kv.kv_indices, kv.last_page_len, w.dtype, w.sm_scale,
                                       w.causal)
        pairs.append((runner.o, runner.lse, ref))
    to, tl = TOL[w.dtype]
    d_o = d_l = 0.0
    agree = True
    rows = 0
    for o, lse, (O, LSE) in pairs:
        e_o, e_l, a = _errors(host(o), lse.cpu().numpy(), O, LSE)
        d_o, d_l, agree = max(d_o, e_o), max(d_l, e_l), agree and a
        rows += int(np.prod(LSE.shape))
    return {"max_abs_dO": d_o, "max_abs_dLSE": d_l, "tol_O": to, "tol_LSE": tl,
            "rows": rows, "neg_inf_rows_agree": agree,
            "ok": bool(agree and d_o <= to and d_l <= tl)}


def roofline_of(name, runner, step_ms, kernel_ms):
    """The workload's bound and its fraction: HBM bytes or MFMA flops per attention-kernel
    time, or (the cascade) the combined floor of its prefix and suffix passes per step."""
    nbytes, flops, _ = runner.work()
    t_s = (kernel_ms if kernel_ms is not None else step_ms) * 1e-3
    timed = "attention kernel (events on its dispatch)" if kernel_ms is not None else "step"
    if name == "cascade":
        w = runner.w
        pre = w.meta["prefix_len"] * w.num_kv_heads * w.head_dim * 2 * 2
        pre_flops = 4.0 * w.num_qo_heads * w.head_dim * len(w.kv.kv_lens) * w.meta["prefix_len"]
        floor_us = (nbytes / (HBM_PEAK_GBS * 1e9) + pre_flops / (MFMA_PEAK_TFLOPS * 1e12)) * 1e6
        return {"bound": "hbm+mfma", "achieved": floor_us / (step_ms * 1e3), "peak": 1.0,
                "unit": "fraction of the combined floor (all KV bytes at 8 TB/s + the prefix "
                        "pass's flops at 2.5 PFLOP/s)", "frac": floor_us / (step_ms * 1e3),
                "floor_us": floor_us, "kernel_us": step_ms * 1e3, "timed": "step",
                "prefix_bytes": pre, "traffic": None}
    if name in PREFILL_LIKE:
        a = flops / t_s / 1e12
        return {"bound": "mfma", "achieved": a, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a / MFMA_PEAK_TFLOPS, "traffic": None, "kernel_us": t_s * 1e6,
                "timed": timed}
    a = nbytes / t_s / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a / HBM_PEAK_GBS, "traffic": profiled_traffic() if name == "decode" else None,
            "kernel_us": t_s * 1e6, "timed": timed}


def host_threads():
    """(threads the oracle's BLAS uses, CPUs this process may run on). The BLAS thread
    count follows OMP_NUM_THREADS where the environment sets it."""
    cpus = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return int(blas), int(cpus)


def oracle_units(runner):
    """The oracle's work for one step of the runner's workload, cut into units (one request,
    or one KV head for block-sparse attention), each with its share of the step's algorithmic
    work (bytes for HBM-bound workloads, flops for MFMA-bound ones)."""
    import oracle
    w = runner.w
    var = w.meta.get("variant", {}) if w.kind in ("decode", "prefill") else {}
    win = int(var.get("window_left", -1))
    cap = float(var.get("logits_soft_cap", 0.0))
    sinks = var.get("sinks")
    units = []
    if w.kind == "single_decode":
        units.append((lambda: oracle.single_decode(w.q, w.k, w.v, w.dtype, w.sm_scale), 1.0))
    elif w.kind == "append":
        kv = w.kv
        bi, pos = oracle.append_positions(w.append_indptr, kv.kv_indptr, kv.last_page_len,
                                          kv.page_size)
        units.append((lambda: oracle.append_paged_kv(kv.k_cache, kv.v_cache, w.append_k,
                                                     w.append_v, bi, pos, kv.kv_indptr,
                                                     kv.kv_indices, kv.last_page_len), 1.0))
    elif w.kind == "decode":
        kv = w.kv
        seen = kv.kv_lens if win < 0 else np.minimum(kv.kv_lens, win + 1)
        total = float(np.sum(seen))
        for b in range(len(seen)):
            if win >= 0 or cap > 0 or sinks is not None:
                fn = (lambda b=b: oracle.batch_decode_variant(
                    w.q, kv.k_cache, kv.v_cache, kv.kv_indptr, kv.kv_indices, kv.last_page_len,
                    w.dtype, w.sm_scale, win, cap, sinks, requests=[b]))
            else:
                fn = (lambda b=b: oracle.batch_decode(
                    w.q, kv.k_cache, kv.v_cache, kv.kv_indptr, kv.kv_indices, kv.last_page_len,
                    w.dtype, w.sm_scale, requests=[b]))
            units.append((fn, float(seen[b]) / total if total else 0.0))
    elif w.kind == "prefill":
        kv = w.kv
        qo = w.meta["qo_lens"]
        fl = [prefill_flops([qo[b]], [kv.kv_lens[b]], w.num_qo_heads, w.head_dim, w.causal, win)
              for b in range(len(qo))]
        total = float(sum(fl))
        for b in range(len(qo)):
            if win >= 0 or cap > 0 or sinks is not None:
                fn = (lambda b=b: oracle.batch_prefill_variant(
                    w.q, kv.k_cache, kv.v_cache, w.qo_indptr, kv.kv_indptr, kv.kv_indices,
                    kv.last_page_len, w.dtype, w.sm_scale, w.causal, win, cap, sinks,
                    requests=[b]))
            else:
                fn = (lambda b=b: oracle.batch_prefill(
                    w.q, kv.k_cache, kv.v_cache, w.qo_indptr, kv.kv_indptr, kv.kv_indices,
                    kv.last_page_len, w.dtype, w.sm_scale, w.causal, requests=[b]))
            units.append((fn, fl[b] / total if total else 0.0))
    elif w.kind == "cascade":
        kv = w.kv
        B = len(kv.kv_lens)
        for b in range(B):
            units.append((lambda b=b: oracle.cascade_decode(
                w.q, kv.k_cache, kv.v_cache, w.prefix_indices, w.prefix_last_page_len,
                kv.kv_indptr, kv.kv_indices, kv.last_page_len, w.dtype, w.sm_scale,
                requests=[b]), 1.0 / B))
    elif w.kind == "block_sparse":
        G = w.num_qo_heads // w.num_kv_heads
        for g in range(w.num_kv_heads):
            qs = np.ascontiguousarray(w.q[:, g * G:(g + 1) * G])
            ks, vs = np.ascontiguousarray(w.k[:, g:g + 1]), np.ascontiguousarray(w.v[:, g:g + 1])
            units.append((lambda qs=qs, ks=ks, vs=vs: oracle.block_sparse_attention(
                qs, ks, vs, w.dtype, w.bsr_indptr, w.bsr_indices, w.row_block, w.col_block,
                w.sm_scale), 1.0 / w.num_kv_heads))
    elif w.kind == "pod":
        wp, wd = w.prefill, w.decode
        fp = [prefill_flops([wp.meta["qo_lens"][b]], [wp.kv.kv_lens[b]], wp.num_qo_heads,
                            wp.head_dim, wp.causal) for b in range(len(wp.meta["qo_lens"]))]
        fd = [4.0 * wd.num_qo_heads * wd.head_dim * float(L) for L in wd.kv.kv_lens]
        total = float(sum(fp) + sum(fd))
        for b in range(len(fp)):
            units.append((lambda b=b: oracle.batch_prefill(
                wp.q, wp.kv.k_cache, wp.kv.v_cache, wp.qo_indptr, wp.kv.kv_indptr,
                wp.kv.kv_indices, wp.kv.last_page_len, wp.dtype, wp.sm_scale, wp.causal,
                requests=[b]), fp[b] / total))
        for b in range(len(fd)):
            units.append((lambda b=b: oracle.batch_decode(
                wd.q, wd.kv.k_cache, wd.kv.v_cache, wd.kv.kv_indptr, wd.kv.kv_indices,
                wd.kv.last_page_len, wd.dtype, wd.sm_scale, requests=[b]), fd[b] / total))
    return units


def oracle_timing(runner, prefill_like, min_s=3.0, max_s=10.0):
    """The oracle on the host cores over a bounded sample of one step's work (whole units in
    order: at least one pass and `min_s` seconds, stopping once past `max_s`), in the
    workload's roofline unit."""
    cores, cpus = host_threads()
    nbytes, flops, _ = runner.work()
    units = oracle_units(runner)
    t0 = time.perf_counter()
    share, n = 0.0, 0
    while units:                      # at least one pass, then until min_s (or past max_s)
        for fn, sh in units:
            fn()
            share += sh
            n += 1
            if time.perf_counter() - t0 > max_s:
                break
        elapsed = time.perf_counter() - t0
        if elapsed >= min_s or elapsed > max_s:
            break
    dt = time.perf_counter() - t0
    work = (flops if prefill_like else nbytes) * share
    return {"value": work / dt / (1e12 if prefill_like else 1e9),
            "unit": "TFLOP/s" if prefill_like else "GB/s", "cores": cores,
            "affinity_cpus": cpus, "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {n} unit evaluations ({len(units)} units make one "
                      f"step; {share:.3f} steps' work) in {dt:.1f} s, {cores} BLAS threads"}


# workloads whose roofline is the MFMA peak (the rest are bound by HBM)
PREFILL_LIKE = ("prefill", "block_sparse", "pod", "prefill_variants")

WORKLOADS = {"single": 0, "decode": 1, "prefill": 2, "cascade": 3, "long": 4, "append": 5,
             "block_sparse": 6, "pod": 7, "decode_variants": 8, "prefill_variants": 9}


def with_variants(w, window_left, soft_cap, seed):
    """The workload with a sliding window, a logit soft cap and seeded N(0, 2) sinks."""
    rng = np.random.default_rng(seed)
    w.meta["variant"] = {"window_left": window_left, "logits_soft_cap": soft_cap,
                         "sinks": (rng.standard_normal(w.num_qo_heads) * 2).astype(np.float32)}
    return w


def make_workload(name, wl):
    if name == "append":
        return wl.append_kv()
    if name == "block_sparse":
        return wl.block_sparse()
    if name == "pod":
        return wl.pod()
    if name == "decode_variants":
        return with_variants(wl.FULL[1](), 1023, 30.0, 173008)
    if name == "prefill_variants":
        return with_variants(wl.FULL[2](), 1023, 50.0, 173009)
    return wl.FULL[WORKLOADS[name]]()


DEFAULT_FIVE = ("single", "decode", "prefill", "cascade", "long")
EXTRA = ("append", "block_sparse", "pod", "decode_variants", "prefill_variants")

DESCRIPTION = {
    "single": "single-request decode, kv_len 1024, 32/32 heads, fp16, contiguous",
    "decode": "batch paged decode, 64 requests, kv_len U[512,4096], 32/8 heads, P=16, fp16",
    "prefill": "batch paged causal prefill, 16 requests, qo U[128,1024] after prefix "
               "U[0,2048], 32/8 heads, P=16, bf16",
    "cascade": "cascade, 128 requests, 8192-token shared prefix, suffix U[64,1024], "
               "32/8 heads, P=16, fp16",
    "long": "long-context split-KV decode, 4 x 131072 tokens, 64/8 heads, P=64, bf16",
    "append": "append of the prefill workload's 10420 new tokens' K/V into the paged "
              "cache, 8 KV heads, P=16, bf16",
    "block_sparse": "block-sparse attention, 8192 x 8192 tokens, 64 x 64 blocks, "
                    "density 0.25 + diagonal, 32/8 heads, bf16",
    "pod": "mixed batch in one launch: the causal prefill workload's 16 requests and "
           "64 decode requests with kv_len U[512,4096], 32/8 heads, P=16, bf16",
    "decode_variants": "batch paged decode, 64 requests, kv_len U[512,4096], 32/8 heads, "
                       "P=16, fp16, sliding window 1023, logit soft cap 30, sinks",
    "prefill_variants": "batch paged causal prefill, 16 requests, qo U[128,1024] after "
                        "prefix U[0,2048], 32/8 heads, P=16, bf16, sliding window 1023, "
                        "logit soft cap 50, sinks",
}


def measure(name, wl, pkv, torch, args, flush, headline):
    """Times one workload, checks its timed outputs against the oracle, sets it against its
    roofline and times the oracle on a bounded sample; returns (result dict, runner)."""
    t0 = time.perf_counter()
    w = make_workload(name, wl)
    r = Runner(name, w, pkv, torch)
    log(f"[bench] {name}: generated and planned in {time.perf_counter() - t0:.1f} s "
        f"(plan {r.plan_us:.0f} us); timing {args.steps} steps")
    ms, kern, wall = time_steps(torch, r, args.steps, args.warmup, flush)
    med, mean = float(np.median(ms)), float(np.mean(ms))
    kern_med = float(np.median(kern)) if kern else None
    nbytes, flops, tokens = r.work()
    prefill_like = name in PREFILL_LIKE
    res = {"config": DESCRIPTION[name], "ms_per_step": med, "ms_per_step_mean": mean,
           "attention_kernel_ms": kern_med, "plan_us": r.plan_us,
           "value": flops / (med * 1e-3) / 1e12 if prefill_like else nbytes / (med * 1e-3) / 1e9,
           "unit": "TFLOP/s" if prefill_like else "GB/s",
           "tokens_per_s": tokens / (med * 1e-3), "bytes": nbytes, "flops": flops,
           "timed_pass_wall_s": wall}
    res["roofline"] = roofline_of(name, r, med, kern_med)
    if name == "pod":
        # the same two parts as separate prefill and decode runs, timed the same way
        r.sequential = True
        s_ms, _, _ = time_steps(torch, r, args.steps, args.warmup, flush)
        r.sequential = False
        res["sequential_ms_per_step"] = float(np.median(s_ms))
        res["pod_speedup"] = res["sequential_ms_per_step"] / med
        r.step()                       # the outputs checked below are the mixed launch's
    log(f"[bench] {name}: {med * 1e3:.1f} us/step (mean {mean * 1e3:.1f}), {res['value']:.4g} "
        f"{res['unit']}; roofline {res['roofline']['bound']} frac {res['roofline']['frac']:.3f}")
    if not args.no_parity:
        t1 = time.perf_counter()
        res["parity"] = parity(r)
        log(f"[bench] {name}: parity {res['parity']} ({time.perf_counter() - t1:.1f} s)")
    if not args.no_cpu_baseline:
        lo, hi = (10.0, 30.0) if headline else (3.0, 8.0)
        res["cpu_baseline"] = oracle_timing(r, prefill_like, min_s=lo, max_s=hi)
        log(f"[bench] {name}: oracle {res['cpu_baseline']['value']:.4g} "
            f"{res['cpu_baseline']['unit']} ({res['cpu_baseline']['sample']})")
    return res, r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="measure this workload alone (default: the five contract workloads)")
    ap.add_argument("--all", action="store_true", help="also measure the extra workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed outputs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path would shard requests, or one request's KV chunks, across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_173_amd import pkv
    from paged_kv_cache_173_amd import workloads as wl

    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    if args.workload is not None:
        names = [args.workload]
    else:
        names = list(DEFAULT_FIVE) + (list(EXTRA) if args.all else [])
    head_name = "decode" if "decode" in names else names[0]
    results = {}
    head_runner = None
    for name in names:
        res, r = measure(name, wl, pkv, torch, args, flush, headline=name == head_name)
        results[name] = res
        if name == head_name:
            head_runner = r
        else:
            del r
        torch.cuda.empty_cache()

    res = results[head_name]
    w = head_runner.w
    prefill_like = head_name in PREFILL_LIKE
    line = {
        "metric": "paged decode HBM GB/s (% peak); prefill TFLOPS (% MFMA peak); tokens/s",
        "value": res["value"], "unit": res["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"], "ms_per_step_mean": res["ms_per_step_mean"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTION[head_name], "head_dim": 128,
                   "tokens_per_step": head_runner.work()[2],
                   "tokens_per_s": res["tokens_per_s"], "plan_us": res["plan_us"]},
        "roofline": res["roofline"],
    }
    if "parity" in res:
        line["parity"] = res["parity"]
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    if len(results) > 1:
        line["workloads"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
