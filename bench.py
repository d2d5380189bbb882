#!/usr/bin/env python3
"""Benchmark of the SSM layer's hot path on one MI355X.

Default workload (`hybrid_decode`): the decode step of a hybrid model's 24 SSM layers for
32 sequences (32 heads, P = 128, expanded state N = 256, 8 B/C groups, bf16 token inputs,
fp32 state, 4 GiB of caches in all), each sequence with a 1024-token context prefilled on
the GPU.  One step is, for every layer, verify K = 4 drafts -> commit j ~ min(Geom(0.3)-1, 4).
The same line carries the long prefill (`llama8b_long_prefill`: one 8192-token prompt of
the Llama-3-8B layer shape, chunk 256) under "prefill", with its own roofline over the
whole prefill and its own CPU baseline.  Inputs and caches rotate so that every step reads
them from HBM, not the 256 MB Infinity Cache.

Printed JSON line:
  value                verified tokens/s = batch*K / (time per step)
  hbm_gbs              verify's algorithmic bytes / verify kernel time
  ms_per_step          whole step, HIP events; the steps are queued behind a spin kernel so
                       that they run back to back and the events time the device, not the
                       Python launch loop
  host_us_per_step     the host's launch time per step (Python + C ABI calls)
  roofline             for the kernel with the largest time per step (HIP events around
                       its launches, recorded by the library's trace hook), against the
                       published peaks and against ceilings measured in the same run (a
                       512 MiB copy, an 8192^3 bf16 matrix product), with the fraction of
                       the attainable roofline max(bytes/8 TB/s, flops/peak) / time
  prefill              the long prefill: prefill tokens/s, its roofline over all its
                       launches (bytes and flops of the whole prefill over the time of one
                       prefill, prefills back to back), its kernels, its CPU baseline
  cpu_baseline         the CPU oracle on a bounded sample of the same step
Other workloads: --workload llama8b_single | llama8b_batched | llama8b_long_prefill |
llama8b_batched_greedy | llama8b_batched_project | llama8b_batched_tree.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector
ACCEPT_DRAWS = 8  # accepted-length draws a multi-layer step rotates through
KERNELS = ["prefill_state", "prefill_pass", "prefill_out", "verify", "commit", "accept", "project", "prefill_scan"]
PREFILL_KERNELS = ["prefill_state", "prefill_pass", "prefill_out", "prefill_scan"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")


# the sources each kernel family is compiled from (besides the shared headers): a stored
# traffic figure stays valid while these are unchanged
SHARED_SOURCES = ["ssm_internal.h", "../../include/mil_ssm.h"]
FAMILY_SOURCES = {
    "verify": ["verify_kernel.h", "verify.hip", "verify_bf16.hip", "verify_f32.hip"],
    "commit": ["commit.hip"], "accept": ["commit.hip"],
    "project": ["project.hip"],
    "prefill_state": ["prefill_mfma.hip", "prefill.hip"], "prefill_pass": ["prefill_mfma.hip", "prefill.hip"],
    "prefill_out": ["prefill_mfma.hip", "prefill.hip"], "prefill_scan": ["prefill_mfma.hip"],
}


def source_hash(family: str | None = None) -> str:
    """Hash of the kernel sources: of one family's files (and the shared headers), or of
    every file under csrc/ when family is None."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "speculative_decode_amd", "csrc")
    files = sorted(os.listdir(d)) if family is None else SHARED_SOURCES + FAMILY_SOURCES[family]
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------- algorithmic work

def elt(dtype):
    return 2 if dtype == "bf16" else 4


def prefill_work(w, L):
    """Algorithmic bytes and flops of one sequence's prefill, per phase.
    Bytes count what the method must move (inputs, fp32 y, final state); the chunk
    states in the workspace are the implementation's, not the method's."""
    e = elt(w.dtype)
    hpg = w.H // w.G
    inp_state = L * (w.H * w.P + w.G * w.N + w.H) * e           # x, B, dt
    inp_out = L * (w.H * w.P + 2 * w.G * w.N + w.H) * e         # x, B, C, dt
    y = L * w.H * w.P * 4
    st = w.H * w.N * w.P * 4
    fl_state = fl_out = 0
    for c0 in range(0, L, w.chunk):
        q = min(w.chunk, L - c0)
        fl_state += w.H * 2 * q * w.N * w.P                    # B^T (w X)
        fl_out += w.H * (q * q * w.N / hpg + q * q * w.P + 2 * q * w.N * w.P)  # causal C B^T, M X, C h_in
    return {"prefill_state": (inp_state, fl_state), "prefill_pass": (st, 2 * (L // w.chunk + 1) * w.H * w.N * w.P),
            "prefill_out": (inp_out + y, fl_out), "all": (inp_out + y + st, fl_state + fl_out)}


def verify_work(w, batch, K, pend_mean, write_frac):
    """Algorithmic bytes and flops of one verify launch: every slot's state read once,
    written once where rows are folded (fraction write_frac of the slots), the token rows
    of the folded (pend_mean per slot on average) and draft tokens, fp32 y."""
    e = elt(w.dtype)
    S = w.H * w.N * w.P * 4
    byt = batch * S * (1.0 + write_frac)
    byt += batch * (pend_mean + K) * (w.H * w.P + w.G * w.N + w.H) * e + batch * K * w.G * w.N * e
    byt += batch * K * w.H * w.P * 4
    fl = batch * w.H * w.N * w.P * (3 * pend_mean + 5 * K)
    return byt, fl


def commit_work(w, j):
    e = elt(w.dtype)
    return sum(2 * a * (w.H * w.P + w.G * w.N + w.H) * e for a in j) + 4 * 3 * len(j), 0


# --------------------------------------------------------------------------- GPU run

def _to_dev_factory(torch, synth, dev):
    def to_dev(t):
        if t.dtype == synth.BF16:
            return torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(t.store)).to(dev)
    return to_dev


def step_kind(w):
    if w.name == "llama8b_long_prefill":
        return "prefill"
    if w.name in ("llama8b_batched", "hybrid_decode", "llama8b_batched_greedy", "llama8b_batched_project",
                  "llama8b_batched_tree"):
        return "verify"
    return "full"


def accept_work(w, batch, K):
    """Greedy acceptance: every logit read once, drafts in, accepted lengths and tokens out."""
    le = 2  # bf16 logits
    return batch * K * w.vocab * le + batch * K * 4 * 2 + batch * 4, 0


def path_lengths(parent, node):
    """Length of the root path of node[b] in draft tree parent[b] (0 for node -1)."""
    out = np.zeros(len(node), dtype=np.int64)
    for b, a in enumerate(node):
        a = int(a)
        while a >= 0:
            out[b] += 1
            a = int(parent[b, a])
    return out


def project_work(w, T):
    """Input projections of T rows: every weight element and input row read once, the
    projected x, B, C, dt written once (bf16); 2 flops per weight element per row."""
    cols = w.H * w.P + 2 * w.G * w.N + w.H
    return cols * w.d_model * 2 + T * w.d_model * 2 + T * cols * 2 + w.H * 4, 2 * T * cols * w.d_model


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it
    skips the system-scope release (an L2 writeback and invalidate) that a default event
    performs, which on this GPU adds about 2.5 us inside an interval and disturbs the
    kernel after it.  Timestamps are read only after a device synchronize.  Calls go to
    the HIP runtime already loaded in the process (torch's), so the handle is valid for
    the library's trace hook as well."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            cls._hip = ctypes.CDLL(path)
        return cls._hip

    def __init__(self):
        import ctypes
        self._h = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    @property
    def cuda_event(self):
        return self._h.value

    def record(self):
        import ctypes
        import torch
        if self.hip().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def sleep_cycles_per_s():
    """Rate of the clock that torch.cuda._sleep counts, measured with events."""
    import torch
    a, b = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(4_000_000)
    b.record()
    torch.cuda.synchronize()
    return 4_000_000 / (a.elapsed_time(b) * 1e-3)


def run_gpu(args, w):
    """Times `args.steps` steps.  Step kinds: "full" = prefill + verify + commit on a fresh
    slot; "verify" = verify + commit on prefilled caches (every layer for the hybrid
    workload); "prefill" = one long prefill."""
    import ctypes

    import torch

    from speculative_decode_amd import _lib as L
    from speculative_decode_amd import synth
    from speculative_decode_amd.ssm import SSMCache, commit_layers, project, project_workspace_bytes

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    to_dev = _to_dev_factory(torch, synth, dev)
    rng = np.random.default_rng(w.seed)
    kind = step_kind(w)
    Bt, K = w.batch, w.K
    kcap = w.kmax or K  # pending rows each cache holds
    nlayers = w.layers
    layers = [synth.draw_layer(rng, w.H) for _ in range(nlayers)]
    AD = [(to_dev(l.A), to_dev(l.D)) for l in layers]
    lib = L.lib()
    sets = []

    if kind == "full":
        Lp = w.L
        nch = (Lp + w.chunk - 1) // w.chunk
        per_set = Bt * (prefill_work(w, Lp)["all"][0] + nch * w.H * w.N * w.P * 4)
        R = args.rotate or max(2, min(64, int(np.ceil(320e6 / per_set))))
        for r in range(R):
            pre = synth.draw_tokens(rng, Bt, Lp, w.H, w.P, w.N, w.G, w.dtype)
            drf = synth.draw_tokens(rng, Bt, K, w.H, w.P, w.N, w.G, w.dtype)
            j = synth.draw_accept_uniform(rng, Bt, K)
            cache = SSMCache(Bt, w.H, w.P, w.N, w.G, K, w.dtype, device=dev)
            sets.append(dict(caches=[cache], pre=[to_dev(t) for t in (pre.x, pre.B, pre.C, pre.dt)],
                             drf=[[to_dev(t) for t in (drf.x, drf.B, drf.C, drf.dt)]],
                             j=[torch.from_numpy(j).to(dev)], jn=[j],
                             ws=torch.empty(cache.workspace_bytes(Bt, Lp, w.chunk) + 256, dtype=torch.uint8,
                                            device=dev),
                             y=torch.empty((Bt, Lp, w.H, w.P), dtype=torch.float32, device=dev),
                             yv=[torch.empty((Bt, K, w.H, w.P), dtype=torch.float32, device=dev)],
                             m=np.zeros((1, Bt), np.int64), base=np.zeros((1, Bt), np.int64)))
    elif kind == "prefill":
        Lp = w.L
        nch = (Lp + w.chunk - 1) // w.chunk
        per_set = Bt * (prefill_work(w, Lp)["all"][0] + nch * w.H * w.N * w.P * 4)
        R = args.rotate or max(1, min(16, int(np.ceil(320e6 / per_set))))
        for r in range(R):
            pre = synth.draw_tokens(rng, Bt, Lp, w.H, w.P, w.N, w.G, w.dtype)
            cache = SSMCache(Bt, w.H, w.P, w.N, w.G, 4, w.dtype, device=dev)
            sets.append(dict(caches=[cache], pre=[to_dev(t) for t in (pre.x, pre.B, pre.C, pre.dt)],
                             ws=torch.empty(cache.workspace_bytes(Bt, Lp, w.chunk) + 256, dtype=torch.uint8,
                                            device=dev),
                             y=torch.empty((Bt, Lp, w.H, w.P), dtype=torch.float32, device=dev)))
    else:
        # prior contexts: per-slot lengths (batched) or a fixed 1024 (hybrid), prefilled once
        # on the GPU; every other cache is a byte copy of that one (a snapshot)
        if w.ctx_range:
            ctx = rng.integers(w.ctx_range[0], w.ctx_range[1] + 1, size=Bt)
        else:
            ctx = np.full(Bt, w.L)
        state_bytes = Bt * w.H * w.N * w.P * 4
        if w.accept == "greedy":
            state_bytes += Bt * K * w.vocab * 2  # the logits are rotated with the caches
        if w.d_model:
            state_bytes += project_work(w, Bt * K)[0]  # and so are the projection weights
        R = args.rotate or (1 if nlayers > 1 else max(2, min(64, int(np.ceil(320e6 / state_bytes)))))
        proto = SSMCache(Bt, w.H, w.P, w.N, w.G, kcap, w.dtype, device=dev)
        for b in range(Bt):
            pre = synth.draw_tokens(rng, 1, int(ctx[b]), w.H, w.P, w.N, w.G, w.dtype)
            proto.prefill(*[to_dev(t) for t in (pre.x, pre.B, pre.C, pre.dt)], *AD[0], slot0=b,
                          chunk=128 if w.N > 128 else w.chunk, want_y=False)
        torch.cuda.synchronize()
        for r in range(R):
            caches, drfs, js, jns, yvs, greedy, proj, trees = [], [], [], [], [], [], [], []
            # a round accepts the same drafts in every layer (the verifier decides from the
            # last layer's output), so a multi-layer step uses one j for all its layers; the
            # steps rotate through ACCEPT_DRAWS such draws (each verify folds the rows the step
            # before accepted)
            j_round, j_rounds = None, []
            if nlayers > 1:
                j_rounds = [(synth.draw_accept_geometric(rng, Bt, K) if w.accept == "geometric"
                             else synth.draw_accept_uniform(rng, Bt, K)) for _ in range(ACCEPT_DRAWS)]
                j_round = j_rounds[0]
            for li in range(nlayers):
                c = SSMCache(Bt, w.H, w.P, w.N, w.G, kcap, w.dtype, device=dev)
                c.buffer.copy_(proto.buffer)
                drf = synth.draw_tokens(rng, Bt, K, w.H, w.P, w.N, w.G, w.dtype)
                if j_round is not None:
                    j = j_round
                else:
                    j = (synth.draw_accept_geometric(rng, Bt, K) if w.accept == "geometric"
                         else synth.draw_accept_uniform(rng, Bt, K))
                if w.tree:
                    # a random tree per sequence and one accepted node; j = its path length
                    par = synth.draw_tree(rng, Bt, K, w.tree)
                    node = rng.integers(-1, K, size=Bt).astype(np.int32)
                    j = path_lengths(par, node).astype(np.int32)
                    trees.append(dict(par=torch.from_numpy(par).to(dev), node=torch.from_numpy(node).to(dev)))
                if w.accept == "greedy":
                    # logits planted so that greedy verification accepts j[b] drafts
                    dtok, lg = synth.draw_greedy(rng, Bt, K, w.vocab, synth.BF16, j)
                    greedy.append(dict(dtok=torch.from_numpy(dtok).to(dev), logits=to_dev(lg),
                                       acc=torch.empty(Bt, dtype=torch.int32, device=dev),
                                       ws=torch.empty(c.greedy_workspace_bytes(K, w.vocab) + 256,
                                                      dtype=torch.uint8, device=dev)))
                    del lg
                if w.d_model:
                    # the drafts come from input rows through this set's own weights
                    pr = synth.draw_projection(rng, Bt * K, w.d_model, w.H, w.P, w.N, w.G)
                    wsb = project_workspace_bytes(w.H, w.P, w.N, w.G, Bt * K, w.d_model)
                    proj.append(dict(u=to_dev(pr.u).view(Bt, K, w.d_model),
                                     w=[to_dev(t) for t in (pr.w_x, pr.w_B, pr.w_C, pr.w_dt)], bias=to_dev(pr.bias),
                                     ws=torch.empty(wsb + 256, dtype=torch.uint8, device=dev)))
                    del pr
                caches.append(c)
                drfs.append([to_dev(t) for t in (drf.x, drf.B, drf.C, drf.dt)])
                js.append(torch.from_numpy(j).to(dev))
                jns.append(j)
                yvs.append(torch.empty((Bt, K, w.H, w.P), dtype=torch.float32, device=dev))
            if j_rounds:
                jns = j_rounds  # the draws the steps use
            sets.append(dict(caches=caches, drf=drfs, j=js, jn=jns, yv=yvs, greedy=greedy, proj=proj, tree=trees,
                             jr=[torch.from_numpy(jr).to(dev) for jr in j_rounds], jrn=j_rounds,
                             # host mirror of every layer's pending counts (the caches start
                             # with none pending) and of where the next commit appends
                             m=np.zeros((nlayers, Bt), np.int64), base=np.zeros((nlayers, Bt), np.int64),
                             round=0))
        del proto
        torch.cuda.synchronize()
    R = len(sets)

    # rows folded and state write-backs of the verifies issued while recording (the
    # library's rule, mirrored on the host: write back when pending + K > k_max)
    vstats = dict(on=False, rows=0, writes=0, slots=0)

    def verify_part(s, mark=True, project_too=True):
        st = sets[s % R]
        for li, c in enumerate(st["caches"]):
            m = st["m"][li]
            wb = (m > 0) & (m + K > kcap)
            st["base"][li] = np.where(wb | (m == 0), 0, m)
            if vstats["on"]:
                vstats["rows"] += int(m.sum())
                vstats["writes"] += int(wb.sum())
                vstats["slots"] += Bt
            dx, dB, dC, ddt = st["drf"][li]
            if st.get("proj") and project_too:
                # the drafts' x, B, C, dt projected from the input rows into the same buffers
                pj = st["proj"][li]
                tr = mark and li == 0 and trace_project[0]
                if tr:
                    evs["ta"][s].record()
                project(pj["u"], *pj["w"], w.H, w.P, w.N, w.G, dt_bias=pj["bias"], out=(dx, dB, dC, ddt),
                        ws=pj["ws"])
                if tr:
                    evs["tb"][s].record()
            if st.get("tree"):
                c.verify_tree(st["tree"][li]["par"], dx, dB, dC, ddt, *AD[li], y=st["yv"][li])
            else:
                c.verify(dx, dB, dC, ddt, *AD[li], y=st["yv"][li])

    def commit_part(s):
        st = sets[s % R]
        if nlayers > 1 and not st.get("tree") and not st.get("greedy"):
            # every layer's commit of the round in one call (one launch per 32 layers)
            d = st["drf"]
            # the round's draw: one running count per set, so that every pass (warm-up,
            # timed, traced, back to back) continues the same sequence of pending counts
            r = st["round"] % len(st["jr"])
            st["round"] += 1
            commit_layers(st["caches"], st["jr"][r], [t[0] for t in d], [t[1] for t in d], [t[3] for t in d])
            st["m"][:] = st["base"] + st["jrn"][r][None, :]
            return
        for li in range(nlayers):
            st["m"][li] = st["base"][li] + st["jn"][li]
        for li, c in enumerate(st["caches"]):
            dx, dB, dC, ddt = st["drf"][li]
            if st.get("tree"):
                tr = st["tree"][li]
                c.commit_tree(tr["par"], tr["node"], dx, dB, ddt)
            elif st.get("greedy"):
                gr = st["greedy"][li]
                c.commit_greedy(gr["dtok"], gr["logits"], dx, dB, ddt, accepted=gr["acc"], ws=gr["ws"])
            else:
                c.commit(st["j"][li], dx, dB, ddt)

    def step(s, mark=True):
        st = sets[s % R]
        if kind in ("full", "prefill"):
            x, B, C, dt = st["pre"]
            st["caches"][0].prefill(x, B, C, dt, *AD[0], y=st["y"], chunk=w.chunk, ws=st["ws"])
            if "m" in st:
                st["m"][:] = 0  # a fresh prefill leaves nothing pending
        if kind in ("full", "verify"):
            # every layer's verify, then every layer's commit: the accepted lengths are known
            # only once the last layer has run
            verify_part(s, mark)
            commit_part(s)

    def verify_pass():
        """Time per verify launch from launches back to back: the verifies of n whole steps
        (distinct caches: every layer of n rotating sets) between two timing events, then
        their commits.  No event sits between the verify launches, so no dispatch latency is
        added.  A multi-layer step rotates through ACCEPT_DRAWS accepted-length draws: one whole
        cycle of them runs under one hold, step after step as a decode loop would (the
        commits between the timed spans), and the spans are summed."""
        n = max(1, min(args.steps, R))
        rounds = ACCEPT_DRAWS if nlayers > 1 else 1
        marks = [(TimingEvent(), TimingEvent()) for _ in range(rounds)]
        vstats.update(on=True, rows=0, writes=0, slots=0)
        hold(n * rounds)
        for r in range(rounds):
            marks[r][0].record()
            for s in range(n):
                verify_part(r * R + s, mark=False, project_too=False)
            marks[r][1].record()
            for s in range(n):
                commit_part(r * R + s)
        torch.cuda.synchronize()
        vstats["on"] = False
        tot = sum(a.elapsed_time(b) for a, b in marks)
        return tot / (rounds * n * nlayers)

    trace_project = [False]  # the projection is traced with events on torch's stream, around the call

    def set_trace(s, name):
        st = sets[s % R]
        trace_project[0] = name == "project"
        if name == "project":
            return
        for c in st["caches"]:
            if name is None:
                lib.mil_ssm_cache_trace(ctypes.byref(c.desc), 0, None, None)
        if name is not None:
            # trace one cache per step (the first layer's)
            a, b = evs["ta"][s], evs["tb"][s]
            lib.mil_ssm_cache_trace(ctypes.byref(st["caches"][0].desc), L.TRACE[name],
                                    ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event))

    kernels = {"full": KERNELS[3:5], "prefill": [], "verify": KERNELS[3:5]}[kind]
    if kind in ("full", "prefill"):
        # the prefill kernels this shape launches (one launch, or three phases)
        mask = lib.mil_ssm_prefill_kernels(ctypes.byref(sets[0]["caches"][0].desc), Bt, w.L, w.chunk)
        kernels = [k for k in PREFILL_KERNELS if mask & (1 << L.TRACE[k])] + kernels
    if w.accept == "greedy":
        # a greedy commit is one launch (argmax, accepted lengths, copies), traced as accept
        kernels = [k for k in kernels if k != "commit"] + ["accept"]
    if w.d_model:
        kernels = kernels + ["project"]
    n_ev = max(args.steps, len(kernels) * 4)
    evs = {k: [TimingEvent() for _ in range(n_ev)] for k in ("ta", "tb")}
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()

    # warmup (which also gives the host's launch time per step), then one pass per kernel
    # to find the one with the largest time per launch.  The Python launch loop can be
    # slower than the device (a short step is a few calls of tens of microseconds of host
    # work each), and every event interval would then include the device idling for the
    # host; so before each measured pass the device is held by a spin kernel long enough
    # for the host to queue the whole pass, and the events measure the device alone.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup):
        step(s)
    host_step = (time.perf_counter() - t0) / max(args.warmup, 1)
    torch.cuda.synchronize()
    cps = sleep_cycles_per_s()

    def hold(nsteps):
        torch.cuda._sleep(int((1.5 * host_step * nsteps + 2e-3) * cps))

    ktime = {}
    for i, name in enumerate(kernels):
        hold(4)
        for rep in range(4):
            s = i * 4 + rep
            set_trace(s, name)
            step(s)
            set_trace(s, None)
        torch.cuda.synchronize()
        ktime[name] = float(np.mean([evs["ta"][i * 4 + r].elapsed_time(evs["tb"][i * 4 + r]) for r in range(4)]))
    dominant = max(ktime, key=ktime.get)

    eager_ms = None
    if args.graph:
        # verify rounds as HIP graphs: eager steps timed first for comparison, then each
        # rotating set's whole step (every layer's verify + commit) captured once and
        # replayed; the dominant kernel's time per launch is the traced one found above
        torch.cuda.synchronize()
        hold(args.steps)
        e0.record()
        for s in range(args.steps):
            step(s, mark=False)
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / args.steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(r, mark=False)
            graphs.append(g)
        torch.cuda.synchronize()
        for s in range(args.warmup):
            graphs[s % R].replay()
        torch.cuda.synchronize()
        hold(args.steps)
        t0 = time.perf_counter()
        e0.record()
        for s in range(args.steps):
            graphs[s % R].replay()
        e1.record()
        torch.cuda.synchronize()
        wall = host_launch = time.perf_counter() - t0
        step_ms = vc_ms = e0.elapsed_time(e1) / args.steps
        pre_ms = 0.0
        dom_ms = traced_ms = ktime[dominant]
        if dominant == "verify":
            dom_ms = verify_pass()
    else:
        # The timed region: K whole steps back to back between two events, queued behind
        # the hold as above (`host_us_per_step` reports the host's own launch rate).  Even
        # a fence-free event costs the device ~2 us of dispatch, so none is recorded
        # inside the steps here.
        torch.cuda.synchronize()
        hold(args.steps)
        t0 = time.perf_counter()
        e0.record()
        for s in range(args.steps):
            step(s, mark=False)
        e1.record()
        host_launch = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = e0.elapsed_time(e1) / args.steps
        # The dominant kernel's time per launch: the same K steps again, with events right
        # around that kernel's launches (recorded by the library's trace hook on the
        # stream the kernel runs on).
        hold(args.steps)
        for s in range(args.steps):
            set_trace(s, dominant)
            step(s)
        torch.cuda.synchronize()
        for s in range(args.steps):
            set_trace(s, None)
        dom_ms = traced_ms = float(np.mean([evs["ta"][s].elapsed_time(evs["tb"][s]) for s in range(args.steps)]))
        if kind == "verify" and dominant == "verify":
            dom_ms = verify_pass()
        if kind == "full":
            # The prefill alone, K launches back to back between two events; verify +
            # commit take the rest of the step.
            hold(args.steps)
            e0.record()
            for s in range(args.steps):
                st = sets[s % R]
                st["caches"][0].prefill(*st["pre"], *AD[0], y=st["y"], chunk=w.chunk, ws=st["ws"])
            e1.record()
            torch.cuda.synchronize()
            pre_ms = e0.elapsed_time(e1) / args.steps
            vc_ms = step_ms - pre_ms
            if dominant == "prefill_scan":
                # one launch per prefill: the pass just timed is that kernel alone, launched
                # back to back, so its time per launch carries no event's dispatch latency
                traced_ms, dom_ms = dom_ms, pre_ms
        elif kind == "prefill":
            pre_ms, vc_ms = step_ms, 0.0
        else:
            pre_ms, vc_ms = 0.0, step_ms

    # algorithmic work per launch of each kernel
    work = {}
    if kind in ("full", "prefill"):
        pw = prefill_work(w, w.L)
        work.update({k: (pw[k][0] * Bt, pw[k][1] * Bt) for k in ("prefill_state", "prefill_pass", "prefill_out")})
        work["prefill_scan"] = (pw["all"][0] * Bt, pw["all"][1] * Bt)
        work["prefill_all"] = work["prefill_scan"]
    if kind in ("full", "verify"):
        # rows pending at a verify: none after a prefill ("full"); else the previous
        # commit's accepted lengths, whose mean is that of the j distribution
        jall = np.concatenate([jn for st in sets for jn in st["jn"]])
        if kind == "full":
            work["verify"] = verify_work(w, Bt, K, 0.0, 0.0)
        elif vstats["slots"]:
            # the verifies the back-to-back pass timed: rows they folded, states they wrote
            work["verify"] = verify_work(w, Bt, K, vstats["rows"] / vstats["slots"],
                                         vstats["writes"] / vstats["slots"])
        else:
            work["verify"] = verify_work(w, Bt, K, float(jall.mean()), float((jall > 0).mean()))
        work["commit"] = commit_work(w, [float(jall.mean())] * Bt)
        if nlayers > 1 and not w.tree and w.accept != "greedy":
            # one commit launch covers every layer of the round
            work["commit"] = (work["commit"][0] * nlayers, 0)
        if w.accept == "greedy":
            # the greedy commit's one launch: every logit read, the accepted rows copied
            a, c = accept_work(w, Bt, K), work.pop("commit")
            work["accept"] = (a[0] + c[0], 0)
        if w.d_model:
            work["project"] = project_work(w, Bt * K)
    jmean = float(jall.mean()) if kind in ("full", "verify") else 0.0
    return dict(R=R, kind=kind, wall=wall, host_us=host_launch / args.steps * 1e6, pre_ms=pre_ms, vc_ms=vc_ms, step_ms=step_ms, dominant=dominant, jmean=jmean,
                dom_ms=dom_ms, traced_ms=traced_ms, ktime=ktime, work=work, device=torch.cuda.get_device_name(dev), eager_ms=eager_ms)


# --------------------------------------------------------------------------- CPU baseline

def measured_peaks():
    """Measured ceilings on this GPU, beside the published peaks: a plain 512 MiB
    device-to-device copy (read + write bytes / time) and a large bf16 matrix product
    through torch (hipBLASLt / rocBLAS) for the matrix-core rate."""
    import torch
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return copy_gbs, gemm_tflops


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def run_cpu_baseline(w, kind, budget_s=10.0, max_steps=200):
    """The oracle, as it stands, on a bounded sample of the same step, repeated until
    about budget_s seconds of CPU work.  "full": prefill + verify + commit of the whole
    step.  "prefill": the whole prefill (one repetition may exceed the budget).  "verify":
    single layers of the step (verify K drafts + commit of every sequence, from a random
    fp64 state of the layer's shape; the oracle's cost does not depend on the values),
    scaled to the step's layer count."""
    import oracle
    from speculative_decode_amd import synth
    rng = np.random.default_rng(w.seed + 77)
    layer = synth.draw_layer(rng, w.H)
    threads = oracle.default_threads()
    A, D = layer.A.f64, layer.D.f64
    if kind == "prefill":
        pre = synth.draw_tokens(rng, w.batch, w.L, w.H, w.P, w.N, w.G, w.dtype)
        t, reps = 0.0, 0
        while reps < max_steps and t < budget_s:
            a = time.perf_counter()
            oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, A, D, nthreads=threads)
            t += time.perf_counter() - a
            reps += 1
        return dict(value=w.batch * w.L * reps / t, unit="prefill tokens/s", cores=threads, kind="oracle",
                    cpu=_cpu_model(), sample=f"{reps} whole prefills of {w.batch} x {w.L} tokens, same shapes, "
                                             f"fp64 oracle, {t:.1f} s")
    if kind == "verify":
        state = rng.normal(0.0, 0.1, size=(w.batch, w.H, w.N, w.P))
        drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
        j = (synth.draw_accept_geometric(rng, w.batch, w.K) if w.accept == "geometric"
             else synth.draw_accept_uniform(rng, w.batch, w.K))
        t, reps = 0.0, 0
        while reps < max_steps and t < budget_s:
            a = time.perf_counter()
            oracle.verify(state, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, A, D, nthreads=threads)
            oracle.commit(state, drf.x.f64, drf.B.f64, drf.dt.f64, A, D, j, nthreads=threads)
            t += time.perf_counter() - a
            reps += 1
        per_step = t / reps * w.layers
        return dict(value=w.batch * w.K / per_step, unit="verified tokens/s", cores=threads, kind="oracle",
                    cpu=_cpu_model(),
                    sample=f"{reps} single layers (verify {w.K} + commit, {w.batch} sequences) of the "
                           f"{w.layers}-layer step, fp64 oracle, {t:.1f} s, scaled to {w.layers} layers")
    pre = synth.draw_tokens(rng, w.batch, w.L, w.H, w.P, w.N, w.G, w.dtype)
    drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
    j = synth.draw_accept_uniform(rng, w.batch, w.K)
    t_pre = t_vc = 0.0
    steps = 0
    while steps < max_steps and (t_pre + t_vc) < budget_s:
        a = time.perf_counter()
        _, h = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, A, D, nthreads=threads)
        b = time.perf_counter()
        oracle.verify(h, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, A, D, nthreads=threads)
        oracle.commit(h, drf.x.f64, drf.B.f64, drf.dt.f64, A, D, j, nthreads=threads)
        c = time.perf_counter()
        t_pre += b - a
        t_vc += c - b
        steps += 1
    return dict(value=w.batch * w.K * steps / t_vc, unit="verified tokens/s", cores=threads, kind="oracle",
                prefill_tokens_per_s=w.batch * w.L * steps / t_pre, cpu=_cpu_model(),
                sample=f"{steps} whole steps (prefill {w.L} + verify {w.K} + commit) of the same shapes, "
                       f"fp64 oracle, {t_pre + t_vc:.1f} s")


# --------------------------------------------------------------------------- rocprofv3 summaries

KERNEL_PATTERNS = {  # kernel family -> substring of its symbol
    "prefill_state": "chunk_state_", "prefill_pass": "state_pass", "prefill_out": "chunk_out_",
    "prefill_scan": "chunk_scan_",
    "verify": "ssm_verify_kernel", "commit": ("_commit_kernel", "_commit_tree_kernel", "_commit_layers_kernel"),
    "accept": "greedy_accept",
    "project": "project_",
    "copy": "MulFunctor",  # the calibration copy: torch.mul(src, 1.0, out=dst)
}


def _family(name):
    for k, pat in KERNEL_PATTERNS.items():
        if any(q in name for q in ((pat,) if isinstance(pat, str) else pat)):
            return k
    return None


def summarize(dbs):
    """Per-kernel durations from rocprofv3 --kernel-trace databases, as a text table."""
    import sqlite3
    rows = {}
    for db in dbs:
        con = sqlite3.connect(db)
        for name, dur in con.execute("select name, duration from kernels"):
            rows.setdefault(name, []).append(dur)
    tot = sum(sum(v) for v in rows.values())
    lines = [f"{'calls':>6} {'mean_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for name, v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):6d} {np.mean(v) / 1e3:10.3f} {np.min(v) / 1e3:10.3f} {np.max(v) / 1e3:10.3f} "
                     f"{100 * sum(v) / tot:6.2f}  {name[:110]}")
    return "\n".join(lines)


def per_call(per_kernel):
    """One call's value of a kernel family from per-dispatch counter values grouped by
    kernel: each kernel's mean, counted as often per call as it was launched relative to
    the family's most launched kernel (a projection launches its product and its
    reduction once each; kernels launched only while setting up count zero times)."""
    cmax = max(len(v) for v in per_kernel.values())
    return float(sum(np.mean(v) * round(len(v) / cmax) for v in per_kernel.values()))


def traffic(fetch_db, write_db, workload, copy_mib):
    """HBM bytes per launch of each kernel family from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain elementwise copy of
    copy_mib MiB (which reads and writes exactly that many bytes) in the same process."""
    import sqlite3

    def per_family(db, counter):
        con = sqlite3.connect(db)
        acc = {}
        for name, v in con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                                   (counter,)):
            f = _family(name)
            if f:
                acc.setdefault(f, {}).setdefault(name, []).append(v * 1024.0)
        return {k: per_call(per) for k, per in acc.items()}

    fe = per_family(fetch_db, "FETCH_SIZE")
    wr = per_family(write_db, "WRITE_SIZE")
    known = copy_mib * 1024 * 1024
    kf, kw = known / fe["copy"], known / wr["copy"]
    out = {"_calibration": {"copy_bytes": known, "fetch_counter_bytes": fe["copy"],
                            "write_counter_bytes": wr["copy"], "fetch_scale": kf, "write_scale": kw}}
    for k in fe:
        if k != "copy" and k in wr:
            out[f"{k}/{workload}"] = {"fetch_bytes": fe[k] * kf, "write_bytes": wr[k] * kw,
                                      "bytes_per_launch": fe[k] * kf + wr[k] * kw, "source_sha": source_hash(k)}
    return out


def mfma_counters(db, workload):
    """Issued matrix-core work per launch of each kernel family from a rocprofv3 --pmc run
    of SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA flops / 512) and MfmaUtil (rocprofv3's
    derived busy percentage of the matrix cores over the dispatch)."""
    import sqlite3
    con = sqlite3.connect(db)
    acc = {}
    for name, cname, v in con.execute("select kernel_name, counter_name, value from counters_collection"):
        f = _family(name)
        if f in FAMILY_SOURCES:
            acc.setdefault(f, {}).setdefault(cname, {}).setdefault(name, []).append(v)
    out = {}
    for f, c in acc.items():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in c or "MfmaUtil" not in c:
            continue
        out[f"{f}/{workload}"] = {"issued_bf16_flops": per_call(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512,
                                  "mfma_busy_frac": float(np.mean([x for v in c["MfmaUtil"].values() for x in v])) / 100.0,
                                  "source_sha": source_hash(f)}
    return out


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # multiples of ACCEPT_DRAWS: every phase of a multi-layer run covers whole cycles of the
    # accepted-length draws, so each phase's verifies fold and write the same mix
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="hybrid_decode")
    ap.add_argument("--prefill-workload", default="llama8b_long_prefill",
                    help="with a verify workload: also run this prefill workload and report it in the same "
                         "line under \"prefill\" ('none' to skip)")
    ap.add_argument("--rotate", type=int, default=0, help="independent cache/input sets (0: enough for >320 MB)")
    ap.add_argument("--chunk", type=int, default=0, help="prefill chunk length (0: the workload's)")
    ap.add_argument("--kmax", type=int, default=0,
                    help="verify workloads: pending rows each cache holds (0: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="verify workloads: replay each round as a HIP graph (launches included in the time)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, time a plain elementwise copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar="DB",
                    help="print a per-kernel summary of rocprofv3 --kernel-trace databases and exit")
    ap.add_argument("--mfma", metavar="DB",
                    help="turn a SQ_INSTS_VALU_MFMA_MOPS_BF16 / MfmaUtil --pmc database into "
                         "profiles/mfma.json entries for --workload, then exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn FETCH_SIZE / WRITE_SIZE --pmc databases (run with --copy-mib) into "
                         "profiles/traffic.json entries for --workload, then exit")
    args = ap.parse_args()
    if args.summarize:
        print(summarize(args.summarize))
        return
    if args.mfma:
        t = mfma_counters(args.mfma, args.workload)
        old = json.load(open(MFMA_FILE)) if os.path.exists(MFMA_FILE) else {}
        old.update(t)
        with open(MFMA_FILE, "w") as fh:
            json.dump(old, fh, indent=1, sort_keys=True)
        print(json.dumps(t, indent=1))
        return
    if args.traffic:
        if not args.copy_mib:
            ap.error("--traffic needs the --copy-mib value the counter runs used")
        t = traffic(args.traffic[0], args.traffic[1], args.workload, args.copy_mib)
        old = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
        old.update(t)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(old, fh, indent=1, sort_keys=True)
        print(json.dumps(t, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(nothing in the SSM path runs across GPUs)", file=sys.stderr)
        sys.exit(2)
    from speculative_decode_amd import synth
    w = synth.WORKLOADS[args.workload]
    if args.chunk or args.kmax:
        import dataclasses
        w = dataclasses.replace(w, chunk=args.chunk or w.chunk, kmax=args.kmax or w.kmax)
    args.steps = max(1, args.steps)
    if args.graph and step_kind(w) != "verify":
        ap.error("--graph applies to the verify workloads (llama8b_batched, llama8b_batched_greedy, "
                 "llama8b_batched_project, llama8b_batched_tree, hybrid_decode)")
    out = report(args, w, args.workload)
    if args.prefill_workload != "none" and step_kind(w) == "verify":
        # the long prefill of the same line: its own roofline over the whole prefill and its
        # own CPU baseline
        wp = synth.WORKLOADS[args.prefill_workload]
        if step_kind(wp) != "prefill":
            ap.error("--prefill-workload must name a prefill workload (llama8b_long_prefill)")
        args.graph = False
        args.copy_mib = 0
        p = report(args, wp, args.prefill_workload)
        out["prefill"] = {k: p[k] for k in ("value", "unit", "ms_per_step", "config", "roofline", "kernels",
                                             "cpu_baseline") if k in p}
        out["prefill_tokens_per_s"] = p["value"]
    print(json.dumps(out))


def report(args, w, name):
    """Run one workload on the GPU and build its JSON report (value, roofline, kernels,
    CPU baseline)."""
    g = run_gpu(args, w)
    kind = g["kind"]

    if args.copy_mib:
        import torch
        n = args.copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    K, Bt, L = w.K, w.batch, w.L
    dom = g["dominant"]
    if kind == "prefill":
        # the whole prefill (every launch it makes), as one unit: its bytes and flops over
        # the time of one prefill measured back to back
        byt, fl = g["work"]["prefill_all"]
        t = g["pre_ms"] * 1e-3
    else:
        byt, fl = g["work"][dom]
        t = g["dom_ms"] * 1e-3
    bf16 = w.dtype == "bf16"
    if kind == "prefill" or dom in ("prefill_out", "prefill_state", "prefill_scan"):
        mfma_bound = bf16 and fl / byt > (BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3)
    else:
        mfma_bound = False
    if mfma_bound:
        roof = dict(bound="mfma", achieved=fl / t / 1e12, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=byt / t / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "prefill (all launches)" if kind == "prefill" else dom
    roof["kernel_ms"] = t * 1e3
    if kind != "prefill":
        roof["kernel_ms_traced"] = g["traced_ms"]  # events right around its launches (dispatch latency included)
    roof["flops_per_launch"] = fl
    roof["bytes_per_launch"] = byt
    roof["mfma_frac_bf16"] = fl / t / 1e12 / BF16_PEAK_TFLOPS
    roof["hbm_frac"] = byt / t / 1e9 / HBM_PEAK_GBS
    fams = [k for k in g["ktime"]] if kind == "prefill" else [dom]
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ents = [tr.get(f"{k}/{name}") for k in fams]
            if all(e and e.get("source_sha") == source_hash(k) for e, k in zip(ents, fams)):
                roof["traffic"] = sum(e["bytes_per_launch"] for e in ents)
        except (OSError, ValueError, KeyError):
            pass
    # issued matrix-core work (counters): the hi / lo splits issue about twice the
    # algorithmic flops of the products they feed
    roof["issued_mfma_tflops"] = None
    roof["mfma_busy_frac"] = None
    if os.path.exists(MFMA_FILE) and (kind == "prefill" or dom in PREFILL_KERNELS):
        try:
            mf = json.load(open(MFMA_FILE))
            ents = [mf.get(f"{k}/{name}") for k in fams]
            if all(e and e.get("source_sha") == source_hash(k) for e, k in zip(ents, fams)):
                issued = sum(e["issued_bf16_flops"] for e in ents)
                roof["issued_mfma_tflops"] = issued / t / 1e12
                roof["issued_mfma_frac_bf16"] = roof["issued_mfma_tflops"] / BF16_PEAK_TFLOPS
                # busy fraction of the whole prefill: each launch's, weighted by its time
                kt = [g["ktime"][k] for k in fams]
                roof["mfma_busy_frac"] = float(sum(e["mfma_busy_frac"] * x for e, x in zip(ents, kt)) / sum(kt))
        except (OSError, ValueError, KeyError):
            pass
    # measured ceilings and the fraction of the attainable roofline: the larger of the
    # byte time and the flop time at the published peaks, over the kernel's time
    copy_gbs, gemm_tflops = measured_peaks()
    roof["measured_copy_gbs"] = copy_gbs
    roof["measured_bf16_gemm_tflops"] = gemm_tflops
    roof["frac_of_measured"] = (byt / t / 1e9 / copy_gbs if roof["bound"] == "hbm"
                                else fl / t / 1e12 / gemm_tflops)
    t_attain = max(byt / (HBM_PEAK_GBS * 1e9), fl / (BF16_PEAK_TFLOPS * 1e12 if bf16 else F32_PEAK_TFLOPS * 1e12))
    roof["attainable_frac"] = t_attain / t
    kern = {k: dict(ms=g["ktime"][k], GBps=g["work"][k][0] / (g["ktime"][k] * 1e-3) / 1e9,
                    TFLOPs=g["work"][k][1] / (g["ktime"][k] * 1e-3) / 1e12) for k in g["ktime"]}
    cfg = {"workload": w.name, "batch": Bt, "heads": w.H, "headdim": w.P, "dstate": w.N, "groups": w.G,
           "layers": w.layers, "chunk": w.chunk, "rotating_sets": g["R"], "parallelism": "single GPU",
           "step": {"full": f"prefill {L} + verify {K} + commit", "prefill": f"prefill {L}",
                    "verify": f"{w.layers} x (" + ("project + " if w.d_model else "")
                              + ("tree " if w.tree else "") + f"verify {K} + "
                              + {"greedy": "greedy commit)", "tree": "tree commit)"}.get(w.accept, "commit)")}[kind]}
    if w.d_model:
        cfg["d_model"] = w.d_model
    if kind != "prefill":
        cfg.update({"drafts_K": K, "accept": {"geometric": "j ~ min(Geom(0.3)-1, K)", "uniform": "j ~ U{0..K}",
                                              "greedy": f"greedy on the device, bf16 logits over {w.vocab} tokens "
                                                        "planted for j ~ U{0..K}",
                                              "tree": f"{w.tree} draft tree (parent ~ U{{-1..k-1}}), accepted node "
                                                      "~ U{-1..K-1}, j = its root path's length"}[w.accept]})
    if kind != "prefill":
        cfg["pending_rows"] = w.kmax or K  # the caches' k_max: accepted rows they can hold unfolded
    if kind != "verify":
        cfg["prefill_len"] = L
    if w.ctx_range:
        cfg["context"] = f"U{{{w.ctx_range[0]}..{w.ctx_range[1]}}} per sequence"
    elif kind == "verify":
        cfg["context"] = f"{w.L} tokens per sequence, prefilled on the GPU"
    cfg["launch"] = "HIP graph per round (capture once, replay)" if g["eager_ms"] is not None else "eager"
    out = {
        "metric": "verified tokens/s + HBM GB/s (K-step SSM verify); prefill scan tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": g["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, f32 state/accumulate" if bf16 else "f32",
        "data": "synthetic (seeded numpy PCG64; random layer parameters, no trained weights)",
        "config": cfg,
    }
    if kind == "prefill":
        out["value"] = Bt * L / (g["pre_ms"] * 1e-3)
        out["unit"] = "prefill tokens/s"
        out["prefill_tokens_per_s"] = out["value"]
    else:
        out["value"] = Bt * K / (g["vc_ms"] * 1e-3)
        out["unit"] = "verified tokens/s"
        vb, _ = g["work"]["verify"]
        out["hbm_gbs"] = vb / (g["ktime"]["verify"] * 1e-3) / 1e9
        out["verify_commit_ms"] = g["vc_ms"]
        out["accepted_tokens_per_s"] = Bt * g["jmean"] / (g["vc_ms"] * 1e-3)
        if g["eager_ms"] is not None:
            out["eager_step_ms"] = g["eager_ms"]
            out["eager_tokens_per_s"] = Bt * K / (g["eager_ms"] * 1e-3)
        if kind == "full":
            out["prefill_tokens_per_s"] = Bt * L / (g["pre_ms"] * 1e-3)
            out["prefill_ms"] = g["pre_ms"]
    out.update({"roofline": roof, "kernels": kern, "wall_s_timed": g["wall"], "host_us_per_step": g["host_us"],
                "device": g["device"],
                "source_sha": source_hash()})
    out["cpu_baseline"] = None if args.no_cpu_baseline else run_cpu_baseline(w, kind)
    return out


if __name__ == "__main__":
    main()
