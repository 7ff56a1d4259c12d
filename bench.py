"""Benchmark of the W8A8 rollout linear on one MI355X.

Default workload: one 7B-shaped decoder layer's quantized linears at decode
size, INT8, M = 256 tokens: QKV 4608x3584, O 3584x3584, gate and up stacked
into one 37888x3584 GEMM (the same outputs as two 18944-row GEMMs, bit for
bit), down 3584x18944 (N x K), with per-token activation quantization in front
of each: 4 quantizations + 4 GEMMs per step.
A "step" is one such layer pass over one batch; successive steps walk through
distinct copies of the layer's weights (more bytes than the 256 MB Infinity
Cache), like a decode pass walks a model's layers.

The timed region is K steps between device synchronizations. Each weight
copy's whole step (quantizations and GEMMs) is captured as one HIP graph, and
the K steps are K replays walking the copies (what a rollout engine that
captures its decode step runs). The roofline object's kernel time comes from
a second graph of 20 back-to-back launches of the dominant GEMM, replayed
between events on its own stream, so no host launch gap is counted. Inputs
are seeded synthetic tensors generated on the device. The roofline "traffic"
(HBM bytes per launch) comes from the committed rocprofv3 counter summary in
profiles/hbm_traffic.md and is null when the GEMM sources changed since.
Where the dominant GEMM runs on a tiling the copy-stream probe replays (192x128,
192x256 or 256x256 tiles without split K), "copy_stream_us" is that probe's time over
the same weights and codes, timed the same way: the GEMM's operand copies,
LDS ring, waits and barriers without the matrix work.

The default run adds, beside the 7B line: the peaks this GPU reaches (HBM
read, dense INT8 / FP8 MFMA, the shader clock under MFMA load; every roofline
object then also carries its fraction of the measured peak), the 32B-shaped
decode layer at 512 tokens in INT8 and FP8, and the 32B prefill gate
projection at 4096 tokens.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS & HBM GB/s vs roofline; decode-layer µs at 7B/32B shapes"
HBM_PEAK_GBS = 8000.0
MFMA8_PEAK_TOPS = 5000.0  # dense INT8 / FP8 MFMA

DOM_BATCH = 20  # dominant-GEMM launches per timing graph
EPS = 1e-6  # RMSNorm epsilon of the producer workloads

WORKLOADS = {
    # gate and up run as one GEMM over the stacked [W_gate; W_up] (as rollout
    # engines merge them; the same outputs bit for bit), QKV fused likewise
    "7b_decode_int8": dict(M=256, qt="int8", chain="7b_gateup", sets=4, kind="outliers"),
    "7b_decode_fp8": dict(M=256, qt="fp8", chain="7b_gateup", sets=4, kind="outliers"),
    # the same layer with one launch per linear: qr_w8a8_gemm_quant (fuse
    # override 1) adds split-K partial sums and quantizes the next linear's
    # input inside the GEMM launch behind grid-wide barriers
    "7b_decode_int8_one_launch": dict(M=256, qt="int8", chain="7b", sets=4, kind="outliers",
                                      one_launch=True),
    # gate and up as two GEMMs of 18944 rows each
    "7b_decode_int8_separate": dict(M=256, qt="int8", chain="7b", sets=4, kind="outliers"),
    # with the producers of the linears' inputs (two RMSNorms, SiLU x up), fused
    # into the quantizers or run as separate torch ops before them
    "7b_decode_int8_fused": dict(M=256, qt="int8", chain="7b_producers", sets=4, kind="outliers",
                                 fused=True),
    "7b_decode_int8_unfused": dict(M=256, qt="int8", chain="7b_producers", sets=4,
                                   kind="outliers", fused=False),
    # q, k and v stacked into one 7168-row projection (the merged QKV rollout
    # engines run; the 7B layer's QKV is merged the same way)
    "32b_decode_int8": dict(M=512, qt="int8", chain="32b_qkv", sets=2, kind="normal"),
    "32b_decode_fp8": dict(M=512, qt="fp8", chain="32b_qkv", sets=2, kind="normal"),
    # q, k and v as three GEMMs
    "32b_decode_int8_separate": dict(M=512, qt="int8", chain="32b", sets=2, kind="normal"),
    "32b_decode_fp8_separate": dict(M=512, qt="fp8", chain="32b", sets=2, kind="normal"),
    "32b_prefill_int8": dict(M=4096, qt="int8", chain="32b_prefill", sets=2, kind="heavy"),
    # one small linear (X[16, 512] x W[512, 512], INT8): launch-bound, timed for
    # its latency, with no roofline claim behind its fraction
    "single_int8_16x512x512": dict(M=16, qt="int8", chain="single", sets=4, kind="normal"),
}


# Per-RL-step weight refresh of a whole model's layer stack: every stored
# parameter matrix W' (fp32) is requantized into its codes, counting the codes
# the last update changed. One step = one refresh of the whole stack.
REFRESH = {
    "refresh_7b_int8": dict(stack="7b", qt="int8"),
    "refresh_7b_fp8": dict(stack="7b", qt="fp8"),
    "refresh_32b_int8": dict(stack="32b", qt="int8"),
}
REFRESH_METRIC = "per-RL-step weight refresh (requantize + flip count) GB/s vs HBM roofline"

# Block-wise FP8 (power-of-two scales per 32 elements): the 7B gate projection.
MX = {"mx_7b_gate_m256": dict(M=256, N=18944, K=3584), "mx_7b_gate_m32": dict(M=32, N=18944, K=3584)}
MX_METRIC = "block-wise FP8 GEMM (E8M0 per-32 scales) GB/s / TOPS vs roofline"

# Trainer-side ACR / TIS loss over one batch of response tokens.
ACR = {"acr_tis_512x8192": dict(n_seq=512, max_len=8192)}
ACR_METRIC = "ACR/TIS per-token loss + gradient GB/s vs HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def chain_spec(name):
    from w8a8_gemm_rl_amd import inputs as I

    if name == "7b":
        return I.CHAIN_7B, I.LINEARS_7B, I.W_SIGMA_7B
    if name == "7b_gateup":
        return I.CHAIN_7B_GATEUP, I.LINEARS_7B, I.W_SIGMA_7B
    if name == "7b_producers":
        return I.CHAIN_7B_PRODUCERS, I.LINEARS_7B, I.W_SIGMA_7B
    if name == "32b":
        return I.CHAIN_32B, I.LINEARS_32B, I.W_SIGMA_32B
    if name in ("32b_prefill", "32b_qkv"):
        return I.CHAIN_32B_PREFILL, I.LINEARS_32B, I.W_SIGMA_32B
    if name == "single":
        return I.CHAIN_SINGLE, I.LINEARS_SINGLE, I.SINGLE["w_sigma"]
    raise ValueError(name)


def linear_bytes(M, N, K):
    """Algorithmic bytes of one GEMM: weight codes, activation codes, scales, bf16 out."""
    return N * K + M * K + 4 * (M + N) + 2 * M * N


def fused_linear_bytes(M, N, K):
    """Algorithmic bytes of one linear that quantizes its bf16 input itself:
    weight codes, bf16 input, weight scales, bf16 out."""
    return N * K + 2 * M * K + 4 * N + 2 * M * N


SMALL_M_MK = 8192  # qr_linear_fused runs as one launch (input quantized in the kernel) up to M K


def small_m_linears(chain, shapes, M, one_launch):
    """Linears that run as one qr_linear_fused launch: up to M K = 8192, no
    producer before them (the library's own choice for qr_linear_fused)."""
    if one_launch:
        return set()
    return {L["name"] for L in chain
            if not L.get("prod") and M <= 4 and M * shapes[L["name"]][1] <= SMALL_M_MK}


def sum_quant_linears(B, chain, shapes, M, qt, small, one_launch):
    """Linears run as qr_w8a8_gemm_quant's separate launches: the GEMM writes
    split-K partial sums and one kernel adds them and quantizes the next
    linear's input (its output read next with no producer in between, by a
    linear that does not quantize its own input; a plan that splits K; N a
    multiple of 8 up to 16384). Their readers need no quantizer launch."""
    if one_launch:
        return set()
    key, epi = chain_keys(chain)
    needed = {key[L["name"]] for L in chain if L["name"] not in small}
    out = set()
    for name, k in epi.items():
        N, K = shapes[name]
        if (name not in small and k in needed and N % 8 == 0 and N <= 16384
                and B.gemm_plan(M, N, K, qt)[1] > 1):
            out.add(name)
    return out


def small_m_rf(N):
    """Block height (16-row fragments) the library picks for the one-launch
    path: the fewest, 1-5, that keep the grid within 256 blocks."""
    for rf in range(1, 5):
        if -(-N // (16 * rf)) <= 256:
            return rf
    return 5


def quant_bytes(M, K, prod=None):
    """Algorithmic bytes of one input quantization: bf16 rows in, codes and
    scales out; a fused norm also reads its gain, SiLU x up two inputs."""
    if prod == "norm":
        return 3 * M * K + 4 * M + 4 * K
    if prod == "silu":
        return 5 * M * K + 4 * M
    return 3 * M * K + 4 * M


def chain_keys(chain):
    """Input key of each linear (its source, column slice and producer) and,
    for one launch per linear, the key each GEMM quantizes in its epilogue:
    the first later linear that reads its output with no producer in between."""
    key = {L["name"]: (L["src"], L["cols"], L.get("prod")) for L in chain}
    epi = {}
    for L in chain:
        if L["src"] != "x0" and not L.get("prod") and L["src"] not in epi:
            epi[L["src"]] = key[L["name"]]
    return key, epi


class Layer:
    """One set of quantized weights for the chain, plus the ops of one step.

    one_launch: every GEMM is one qr_w8a8_gemm_quant launch that also
    quantizes the next linear's input (and adds split-K partial sums) in its
    epilogue; only the layer input (and inputs with a producer) keep a
    quantizer launch. Otherwise: a quantizer before every distinct input and
    qr_w8a8_gemm (with its split-K kernel)."""

    def __init__(self, chain, shapes, M, qt, sigma, seed, dev, x0, bufs, ws, s, fused=True,
                 one_launch=False, wsq=None, small=(), sum_quant=()):
        import torch

        from w8a8_gemm_rl_amd import binding as B

        self.B = B
        self.qt = qt
        self.W, self.gamma = {}, {}
        g = torch.Generator(device=dev)
        for i, L in enumerate(chain):
            N, K = shapes[L["name"]]
            g.manual_seed(seed + i)
            Wf = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * sigma
            gam = None
            if L.get("prod") == "norm":
                gam = 1.0 + 0.1 * torch.randn(K, generator=g, device=dev, dtype=torch.float32)
            # UAQ: W' = W / s, and s folded into the producing norm's gain
            self.W[L["name"]] = B.quantize_weights_uaq(Wf, s, qt, gamma=gam)
            if gam is not None:
                self.gamma[L["name"]] = (gam, gam.to(torch.bfloat16))
            del Wf
        self.x0, self.bufs, self.ws, self.s = x0, bufs, ws, s
        self.chain, self.M, self.fused = chain, M, fused
        self.one_launch, self.wsq, self.shapes = one_launch, wsq, shapes
        self.small = set(small)  # linears run as one qr_linear_fused launch
        # linears whose split-K sum also quantizes the next input (separate launches)
        self.sum_quant = set(sum_quant)

    def ops(self):
        """The step as a list of (kind, name, thunk): per-token quantizations
        (one per distinct input not quantized by a GEMM epilogue) and GEMMs,
        in chain order."""
        B, bufs = self.B, self.bufs
        key, epi = chain_keys(self.chain)
        if not self.one_launch:
            epi = {k: v for k, v in epi.items() if k in self.sum_quant}
        key_buf = {}
        for L in self.chain:
            key_buf.setdefault(key[L["name"]], bufs["q_" + L["name"]])
        by_epilogue = set(epi.values())
        # inputs whose every reader quantizes them itself need no quantizer
        needed = {key[L["name"]] for L in self.chain if L["name"] not in self.small}
        out, done = [], set()
        for L in self.chain:
            k = key[L["name"]]
            if L["name"] in self.small:
                src = self.x0 if L["src"] == "x0" else bufs["y_" + L["src"]]
                if L["cols"] is not None:
                    src = src[:, L["cols"][0]:L["cols"][1]]
                Wq, sw = self.W[L["name"]]
                y = bufs["y_" + L["name"]]

                def fl(src=src, Wq=Wq, sw=sw, y=y):
                    B.linear_fused(src, self.s, Wq, sw, self.qt, Y=y, ws=self.ws)

                out.append(("gemm", L["name"], fl))
                continue
            if k not in done and k not in by_epilogue and k in needed:
                xq, sx = key_buf[k]

                def q(L=L, xq=xq, sx=sx):
                    import torch.nn.functional as Fn

                    src = self.x0 if L["src"] == "x0" else bufs["y_" + L["src"]]
                    if L["cols"] is not None:
                        src = src[:, L["cols"][0]:L["cols"][1]]
                    prod = L.get("prod")
                    if prod == "norm":
                        g32, g16 = self.gamma[L["name"]]
                        if self.fused:
                            B.norm_quant(src, g32, self.qt, eps=EPS, Xq=xq, scale_x=sx)
                        else:
                            h = Fn.rms_norm(src, (src.shape[1],), g16, EPS)
                            B.quantize_act_per_token(h, 1.0, self.qt, Xq=xq, scale_x=sx)
                    elif prod == "silu":
                        n = src.shape[1] // 2
                        if self.fused:
                            B.silu_mul_quant(src[:, :n], src[:, n:], self.s, self.qt, Xq=xq,
                                             scale_x=sx)
                        else:
                            a = Fn.silu(src[:, :n]) * src[:, n:]
                            B.quantize_act_per_token(a, self.s, self.qt, Xq=xq, scale_x=sx)
                    else:
                        B.quantize_act_per_token(src, self.s, self.qt, Xq=xq, scale_x=sx)

                out.append(("quant", L["name"], q))
            done.add(k)
            xq, sx = key_buf[k]
            Wq, sw = self.W[L["name"]]
            y = bufs["y_" + L["name"]]
            if self.one_launch or L["name"] in self.sum_quant:
                nk = epi.get(L["name"])
                cols = None
                xn = sn = None
                if nk is not None:
                    cols = nk[1] if nk[1] is not None else (0, self.shapes[L["name"]][0])
                    xn, sn = key_buf[nk]

                def gm(xq=xq, sx=sx, Wq=Wq, sw=sw, y=y, cols=cols, xn=xn, sn=sn):
                    B.w8a8_gemm_quant(xq, sx, Wq, sw, self.qt, Y=y, q_cols=cols, q_act_mult=self.s,
                                      Xq_next=xn, scale_x_next=sn, ws=self.wsq)
            else:
                def gm(xq=xq, sx=sx, Wq=Wq, sw=sw, y=y):
                    B.w8a8_gemm(xq, sx, Wq, sw, self.qt, out="bf16", Y=y, ws=self.ws)

            out.append(("gemm", L["name"], gm))
        return out

    def run(self, per_linear=None):
        """Enqueue one layer step; per_linear = {name: (start, end)} events around each GEMM."""
        for kind, name, f in self.ops():
            e = per_linear.get(name) if (per_linear and kind == "gemm") else None
            if e:
                e[0].record()
            f()
            if e:
                e[1].record()


KERNEL_SOURCES = {
    "mx": ("mx_kernels.hip", "qr_device.h"),
    "acr": ("acr_kernels.hip",),
    "gemm": ("gemm_kernels.hip", "gemm_plan.hip", "qr_gemm.h", "qr_device.h", "qr_copy.h"),
    "refresh": ("quant_kernels.hip", "qr_device.h"),
    "small": ("small_m_kernels.hip", "qr_device.h", "qr_small_m.h"),
}


def kernel_source_sha256(kind="gemm"):
    """Hash of the sources that define a kernel family (GEMM or refresh) and its launch."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w8a8_gemm_rl_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def committed_traffic(key, kind="gemm"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, or None if there is none for `key` or the kernel's sources
    changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = kernel_source_sha256(kind)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 4 and cells[0] == key:
                if cells[1] != sha[:16]:
                    return None
                return int(cells[2])
    return None


KERNEL_PATTERNS = {
    "mx": r"mx_dma_kernel",
    "acr": r"acr_(tis|sum)_kernel",  # one pass: the per-token kernel and the ordered sum
    "gemm": r"gemm_\w*kernel",  # the main GEMM kernels (any tile family), not the split-K reduction
    "refresh": r"weight_quant_kernel<[^>]*true>",  # the weight quantizer with flip counting
    "small": r"small_m_linear_kernel",  # the one-launch linear of one or two tokens
}


def is_kernel(name, kind="gemm"):
    import re

    return re.search(KERNEL_PATTERNS[kind], name) is not None


def summarize_rocprof(paths, grid, kind="gemm"):
    """Print the figures used from rocprofv3 CSV outputs (kernel trace, or a
    --pmc counter collection) for dispatches of the given grid size."""
    import csv
    import statistics

    for path in paths:
        rows = list(csv.DictReader(open(path)))
        if rows and "Counter_Name" in rows[0]:
            by = {}
            for r in rows:
                if int(r["Grid_Size"]) == grid and is_kernel(r["Kernel_Name"], kind):
                    by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for c, v in by.items():
                unit = " KiB" if c in ("FETCH_SIZE", "WRITE_SIZE") else ""
                print(f"{path}: {c} per dispatch (grid {grid}): mean {statistics.mean(v):.1f}{unit}, "
                      f"n={len(v)}")
            if not by:
                for r in rows:
                    print(f"{path}: {r['Kernel_Name'][:50]} grid {r['Grid_Size']} "
                          f"{r['Counter_Name']} {float(r['Counter_Value']):.1f}")
        else:
            ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in rows
                  if int(r["Grid_Size_X"]) == grid and is_kernel(r["Kernel_Name"], kind)]
            if ds:
                print(f"{path}: {kind} dispatches of grid {grid}: n={len(ds)} mean {statistics.mean(ds):.2f} us "
                      f"median {statistics.median(ds):.2f} us min {min(ds):.2f} us")


def cpu_model():
    """The host CPU's model name (first processor of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(chain, shapes, M, qt, sigma, kind, s, bytes_step, name):
    """Time the CPU oracle on whole layer steps of the same workload on the
    host's cores: about 10 s with every BLAS thread, then one step with one
    thread."""
    import numpy as np

    import oracle as O
    from w8a8_gemm_rl_amd import inputs as I

    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count()
    log("cpu baseline: preparing oracle weights ...")
    layers = []
    for i, L in enumerate(chain):
        N, K = shapes[L["name"]]
        W = I.weights(N, K, sigma, seed=I.matrix_seed(9, i))
        q = O.quantize_weights_uaq(W, s, qt)
        del W
        layers.append(dict(L, Wq=q["Wq"], scale_w=q["scale_w"], act_mult=s))
    K0 = shapes[chain[0]["name"]][1]
    x0 = I.activations(M, K0, seed=I.matrix_seed(9, 99), kind=kind)
    log("cpu baseline: timing oracle layer steps (about 10 s) ...")
    t0 = time.perf_counter()
    steps = 0
    while True:
        O.decode_chain(x0, layers, qt)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or steps >= 30:
            break
    dt /= steps
    one = None
    if threadpool_limits is not None:
        log("cpu baseline: one layer step on one thread ...")
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.decode_chain(x0, layers, qt)
            one = time.perf_counter() - t0
    return {"value": round(bytes_step / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} {name} layer steps (M={M}, all {len(chain)} linears and their "
                      f"per-token quantizations, exact accumulation) by the numpy oracle on "
                      f"{threads} BLAS threads, {dt:.3f} s per step; then one step on 1 thread",
            "seconds_per_step": round(dt, 4),
            "one_thread": None if one is None else {"value": round(bytes_step / one / 1e9, 3),
                                                   "unit": "GB/s", "seconds_per_step": round(one, 4)},
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def refresh_bytes(N, K):
    """Algorithmic bytes of one refresh launch: fp32 parameters read, previous
    codes read, new codes written, scales and per-row change counts written."""
    return 6 * N * K + 8 * N


def refresh_cpu_baseline(qt, N, K, sigma, s):
    """Time the CPU oracle's refresh (requantize + flip count) of one matrix."""
    import numpy as np

    import oracle as O
    from w8a8_gemm_rl_amd import inputs as I

    try:
        from threadpoolctl import threadpool_info

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    s32 = np.float32(s)
    Wp = (I.weights(N, K, sigma, seed=I.matrix_seed(9, 0)) / s32).astype(np.float32)
    c0, _, _ = O.requantize_weights(Wp, qt)
    Wp += (I.normal_f32((N, K), I.DW_SIGMA, seed=I.matrix_seed(9, 1)) * s32).astype(np.float32)
    log("cpu baseline: timing oracle refreshes (about 10 s) ...")
    t0 = time.perf_counter()
    n = 0
    while True:
        O.requantize_weights(Wp, qt, codes_old=c0)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or n >= 30:
            break
    return dt / n, n, threads


def run_refresh(args, dev):
    """Per-RL-step refresh of a whole layer stack (one step = every matrix of
    every layer requantized, with the codes each update changed counted).

    Layout: the stored parameters of all matrices with the same row length K
    live in one [rows, K] fp32 slab (every layer's matrices are row ranges of
    it, as a flat parameter buffer holds them), with codes, scales and change
    counts in matching slabs. A refresh is one launch per slab: 2 for the
    7B/32B stacks (K = hidden: QKV, O, gate+up of every layer; K =
    intermediate: down), instead of one per matrix with a kernel drain and
    fill between each.
    """
    import numpy as np
    import torch

    from w8a8_gemm_rl_amd import binding as B
    from w8a8_gemm_rl_amd import inputs as I

    wl = REFRESH[args.workload]
    stack = I.STACK_7B if wl["stack"] == "7b" else I.STACK_32B
    qt, s, nl = wl["qt"], args.uaq_s, stack["layers"]
    names = stack["names"]
    shapes = {n: stack["linears"][n] for n in names}
    sigma_p = stack["sigma"] / s  # stored parameters W' = W / s
    upd = s * I.DW_SIGMA  # the update on W' (the pages' size, grown by s)
    log(f"bench: {args.workload}: {nl} layers x {', '.join(f'{n} {shapes[n][0]}x{shapes[n][1]}' for n in names)}")

    # Slabs by row length; (layer, matrix) -> (K, first row, end row).
    where, rows = {}, {}
    for l in range(nl):
        for n in names:
            N, K = shapes[n]
            r0 = rows.get(K, 0)
            where[l, n] = (K, r0, r0 + N)
            rows[K] = r0 + N
    CH = 1 << 28  # elements per generation / update chunk
    g = torch.Generator(device=dev)
    slab = {}
    for gi, K in enumerate(sorted(rows)):
        R = rows[K]
        Wp = torch.empty((R, K), dtype=torch.float32, device=dev)
        g.manual_seed(7000 + gi)
        step = max(1, CH // K)
        for a in range(0, R, step):
            Wp[a:a + step].normal_(0.0, sigma_p, generator=g)
        slab[K] = dict(Wp=Wp, Wq=torch.empty((R, K), dtype=B.code_dtype(qt), device=dev),
                       Sw=torch.empty(R, dtype=torch.float32, device=dev),
                       rf=torch.zeros(R, dtype=torch.int32, device=dev), step=step)
    params = sum(R * K for K, R in rows.items())
    bytes_step = sum(refresh_bytes(R, K) for K, R in rows.items())

    def refresh_all():
        for K, d in slab.items():
            B.requantize_weights(d["Wp"], qt, d["Wq"], d["Sw"], row_flips=d["rf"])

    def update():
        for K, d in slab.items():
            W, step = d["Wp"], d["step"]
            for a in range(0, W.shape[0], step):
                c = W[a:a + step]
                c.add_(torch.randn(c.shape, generator=g, device=dev), alpha=upd)

    # The whole refresh as one HIP graph; the dominant launch (the largest
    # slab) alone in a graph of a few launches.
    domK = max(rows, key=lambda K: refresh_bytes(rows[K], K))
    dom_batch = 3
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    whole, dom_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    d = slab[domK]
    with torch.cuda.stream(st):
        refresh_all()  # untimed: codes now match the parameters
        with torch.cuda.graph(whole, stream=st):
            refresh_all()
        with torch.cuda.graph(dom_graph, stream=st):
            for _ in range(dom_batch):
                B.requantize_weights(d["Wp"], qt, d["Wq"], d["Sw"], row_flips=d["rf"])
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        whole.replay()
    torch.cuda.synchronize()

    # Timed: K refreshes, each after an untimed update of every parameter.
    g.manual_seed(99)
    steps = args.steps
    log(f"bench: timing {steps} refresh steps (updates between them untimed)")
    total = 0.0
    acc = {K: torch.zeros(rows[K], dtype=torch.int64, device=dev) for K in rows}
    for _ in range(steps):
        update()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        whole.replay()
        torch.cuda.synchronize()
        total += time.perf_counter() - t0
        for K in rows:
            acc[K] += slab[K]["rf"]
    sec_step = total / steps

    reps = 5
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        dom_graph.replay()
        b.record()
    torch.cuda.synchronize()
    dom_us = 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / (reps * dom_batch)

    acc = {K: v.cpu().numpy() for K, v in acc.items()}
    fl = np.array([[acc[where[l, n][0]][where[l, n][1]:where[l, n][2]].sum() for n in names]
                   for l in range(nl)], dtype=float) / max(steps, 1)
    flip_stats = {
        n: dict(N=shapes[n][0], K=shapes[n][1], mean_flips=round(float(fl[:, j].mean()), 1),
                frac=float(f"{fl[:, j].mean() / (shapes[n][0] * shapes[n][1]):.3e}"),
                min_layer=round(float(fl[:, j].min()), 1), max_layer=round(float(fl[:, j].max()), 1))
        for j, n in enumerate(names)}
    per_layer = [round(float(v), 1) for v in fl.sum(axis=1)]

    Nd = rows[domK]
    dbytes = refresh_bytes(Nd, domK)
    achieved = dbytes / (dom_us * 1e-6) / 1e9
    key = f"{args.workload}:slab:N{Nd}:K{domK}"
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(key, "refresh"),
        "traffic_key": key,
        "kernel": f"refresh of the K={domK} slab ({Nd} rows: every layer's "
                  f"{', '.join(n for n in names if shapes[n][1] == domK)}; {qt}, per-row change counts)",
        "kernel_us": round(dom_us, 2), "alg_bytes_per_launch": dbytes,
    }
    cpu = None
    if not args.no_cpu_baseline:
        Nq, Kq = shapes["qkv"]
        dt, n, threads = refresh_cpu_baseline(qt, Nq, Kq, stack["sigma"], s)
        cpu = {"value": round(refresh_bytes(Nq, Kq) / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{n} refreshes of one {Nq}x{Kq} QKV matrix (requantize + per-row change "
                         f"counts) by the numpy oracle, {dt:.3f} s each",
               "seconds_per_refresh": round(dt, 4), "host_cpus": os.cpu_count()}
    code_bytes = params + 4 * sum(rows.values())
    out = {
        "metric": REFRESH_METRIC,
        "value": round(bytes_step / sec_step / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(sec_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: refresh of {nl} layers x ({', '.join(f'{n} {shapes[n][0]}x{shapes[n][1]}' for n in names)}) "
                        f"= {params / 1e9:.2f} B parameters into {qt} codes, after an update "
                        f"N(0, ({s} x 1e-7)^2) of every stored W' = W / {s}; one launch per "
                        f"row-length slab ({len(rows)})",
            "layers": nl, "qtype": qt, "uaq_s": s, "params": params, "timing": "hip_graph",
            "slabs": {str(K): [R, K] for K, R in sorted(rows.items())},
            "parallelism": "none (1 GPU)",
        },
        "params_per_s": float(f"{params / sec_step:.4e}"),
        "alg_bytes_per_step": bytes_step,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "flips": flip_stats,
        "flips_per_layer": per_layer,
        "broadcast_bytes": {"codes_and_scales": code_bytes, "bf16": 2 * params,
                            "ratio": round(code_bytes / (2 * params), 4)},
    }
    print(json.dumps(out), flush=True)


def run_mx(args, dev):
    """One block-wise FP8 GEMM (activation quantization excluded), timed as a
    graph of launches walking four weight copies, beside the per-channel FP8
    GEMM of the same shape."""
    import torch

    from w8a8_gemm_rl_amd import binding as B

    wl = MX[args.workload]
    M, N, K = wl["M"], wl["N"], wl["K"]
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    X = (torch.randn((M, K), generator=g, device=dev)).to(torch.bfloat16)
    xq, xs = B.mx_quantize(X)
    sets = []
    for j in range(4):
        W = torch.randn((N, K), generator=g, device=dev) * 0.02
        sets.append(B.mx_quantize(W) + B.quantize_weights_uaq(W, 1.5, "fp8"))
        del W
    pxq, psx = B.quantize_act_per_token(X, 1.5, "fp8")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws, _ = B.workspace(B.workspace_size("qr_w8a8_gemm", M, N, K, "fp8"), dev)

    def timed(fn, batch=20):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            fn(0)
            with torch.cuda.graph(gph, stream=st):
                for i in range(batch):
                    fn(i)
        torch.cuda.synchronize()
        gph.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, e in evs:
            a.record()
            gph.replay()
            e.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(e) * 1000.0 / batch for a, e in evs)[2]

    mx_us = timed(lambda i: B.mx_gemm(xq, xs, sets[i % 4][0], sets[i % 4][1], Y=Y))
    pc_us = timed(lambda i: B.w8a8_gemm(pxq, psx, sets[i % 4][2], sets[i % 4][3], "fp8", Y=Y, ws=ws))
    alg = N * K + M * K + (N + M) * (K // 32) + 2 * M * N
    ops = 2 * M * N * K
    bound = "hbm" if ops / alg < MFMA8_PEAK_TOPS / HBM_PEAK_GBS * 1000 else "mfma"
    achieved = alg / (mx_us * 1e-6) / 1e9 if bound == "hbm" else ops / (mx_us * 1e-6) / 1e12
    peak = HBM_PEAK_GBS if bound == "hbm" else MFMA8_PEAK_TOPS
    out = {
        "metric": MX_METRIC, "value": round(alg / (mx_us * 1e-6) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": 100, "warmup": 1, "ms_per_step": round(mx_us / 1000, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3/e8m0",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: Y[{M}, {N}] = X[{M}, {K}] W^T, E4M3FN with one "
                               f"E8M0 scale per 32 elements on both operands",
                   "timing": "hip_graph", "parallelism": "none (1 GPU)"},
        "tops": round(ops / (mx_us * 1e-6) / 1e12, 1),
        "per_channel_fp8_us": round(pc_us, 2),
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": committed_traffic(f"{args.workload}:mx:M{M}:N{N}:K{K}", "mx"),
                     "kernel": "mx_dma_kernel", "kernel_us": round(mx_us, 2),
                     "alg_bytes_per_launch": alg, "alg_ops_per_launch": ops},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def run_acr(args, dev):
    """The ACR / TIS loss and gradient over one batch of response tokens
    (one step = one pass over the batch), timed as a graph of launches."""
    import numpy as np
    import torch

    from w8a8_gemm_rl_amd import binding as B
    from w8a8_gemm_rl_amd import inputs as I

    wl = ACR[args.workload]
    b = I.acr_batch(wl["n_seq"], wl["max_len"], seed=11)
    d = {k: torch.from_numpy(v).to(dev) for k, v in b.items()}
    n = d["logp"].numel()
    loss = torch.empty(n, dtype=torch.float32, device=dev)
    grad = torch.empty(n, dtype=torch.float32, device=dev)
    args_ = (d["logp"], d["logp_prox"], d["logp_behav"], d["adv"], d["mask"], I.ACR_EPS, I.ACR_C)

    def step():
        return B.acr_tis_loss(*args_, loss=loss, grad=grad)

    step()
    torch.cuda.synchronize()
    batch = 20
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        step()
        with torch.cuda.graph(gph, stream=st):
            for _ in range(batch):
                step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        gph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // batch)
    t0 = time.perf_counter()
    for _ in range(reps):
        gph.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / (reps * batch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
    for a, e in evs:
        a.record()
        gph.replay()
        e.record()
    torch.cuda.synchronize()
    k_us = 1000.0 * sum(a.elapsed_time(e) for a, e in evs) / (3 * batch)
    per_tok = 4 * 4 + 1 + 2 * 4  # four fp32 inputs, the mask, loss and gradient out
    alg = per_tok * n
    _, _, sums = step()
    sums = sums.cpu().numpy()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        m = 64 * wl["max_len"]
        sl = {k: v[:m] for k, v in b.items()}
        t1 = time.perf_counter()
        k = 0
        while time.perf_counter() - t1 < 10.0 and k < 30:
            O.acr_tis_loss(sl["logp"], sl["logp_prox"], sl["logp_behav"], sl["adv"], sl["mask"],
                           I.ACR_EPS, I.ACR_C)
            k += 1
        dt = (time.perf_counter() - t1) / k
        cpu = {"value": round(per_tok * m / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{k} passes of the numpy oracle over 64 of the 512 responses "
                         f"({m} tokens), {dt:.3f} s each"}
    out = {
        "metric": ACR_METRIC, "value": round(alg / sec / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": reps * batch, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl['n_seq']} responses x {wl['max_len']} "
                               f"tokens (ragged lengths, {int(sums[1])} valid), eps {I.ACR_EPS}, "
                               f"C {I.ACR_C}; loss, gradient and float64 sums",
                   "timing": "hip_graph", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(alg / (k_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": committed_traffic(f"{args.workload}:acr:pass", "acr"),
                     "kernel": "acr_tis_kernel + acr_sum_kernel",
                     "kernel_us": round(k_us, 2), "alg_bytes_per_launch": alg},
        "cpu_baseline": cpu,
        "mean_loss": float(sums[0] / max(sums[1], 1)), "clipped_frac": float(sums[2] / max(sums[1], 1)),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="7b_decode_int8",
                    choices=sorted(WORKLOADS) + sorted(REFRESH) + sorted(ACR) + sorted(MX))
    ap.add_argument("--m", type=int, default=None, help="override the token count M")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip the 32B decode / prefill lines and the measured peaks")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--no-small-m", action="store_true",
                    help="run every linear as quantizer + GEMM launches, also at 1-2 tokens")
    ap.add_argument("--no-sum-quant", action="store_true",
                    help="keep a quantizer launch after every split-K sum (instead of the sum "
                         "kernel that also quantizes the next linear's input)")
    ap.add_argument("--summarize-rocprof", nargs="+", metavar="CSV",
                    help="print the figures used from rocprofv3 CSV files (with --grid) and exit")
    ap.add_argument("--grid", type=int, default=0, help="grid size (threads) of the dispatches to summarize")
    ap.add_argument("--kernel-kind", default="gemm", choices=sorted(KERNEL_PATTERNS),
                    help="kernel family for --summarize-rocprof and --source-sha")
    ap.add_argument("--source-sha", action="store_true", help="print the kernel family's source hash and exit")
    ap.add_argument("--uaq-s", type=float, default=1.5,
                    help="refresh workloads: UAQ factor s (stored W' = W / s, update s * dW)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    ap.add_argument("--copy-stream-variants", action="store_true",
                    help="only time the copy-stream probe's variants (row strides padded by a line, "
                         "weights as K panels, no barrier per K step) beside the GEMM on the 7B and "
                         "32B gate shapes, print one JSON line and exit")
    ap.add_argument("--gemm-bound-sweeps", action="store_true",
                    help="only time the 7B gate GEMM at 256 tokens and its copy stream over fewer "
                         "blocks and fewer owned rows per tile, print one JSON line and exit")
    args = ap.parse_args()

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.grid, args.kernel_kind)
        return
    if args.source_sha:
        print(kernel_source_sha256(args.kernel_kind)[:16])
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py: this library runs on one GPU only (got --gpus {args.gpus}, "
            f"WORLD_SIZE {world}); the path has no multi-GPU mode")
        sys.exit(2)

    import torch

    from w8a8_gemm_rl_amd import binding as B

    if not torch.cuda.is_available():
        log("bench.py needs a HIP device")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return
    B.lib()
    if args.copy_stream_variants:
        print(json.dumps(copy_stream_variants(dev)))
        return
    if args.gemm_bound_sweeps:
        print(json.dumps(gemm_bound_sweeps(dev)))
        return
    if args.workload in REFRESH:
        run_refresh(args, dev)
        return
    if args.workload in ACR:
        run_acr(args, dev)
        return
    if args.workload in MX:
        run_mx(args, dev)
        return

    wl = dict(WORKLOADS[args.workload])
    if args.m is not None:
        wl["M"] = args.m
    if args.no_small_m:
        wl["no_small_m"] = True
    if args.no_sum_quant:
        wl["no_sum_quant"] = True
    r = run_chain(args.workload, wl, dev, args.steps, args.warmup, args.eager)
    M, qt, s = wl["M"], wl["qt"], 1.5
    chain, shapes, sigma = chain_spec(wl["chain"])

    extra = {}
    if not args.no_extras and args.workload == "7b_decode_int8" and args.m is None:
        # The 32B half of the metric (decode layer at 512 tokens, INT8 and
        # FP8; the prefill gate projection at 4096 tokens) and the peaks the
        # chip reaches, beside the headline 7B line.
        extra["peaks_measured"] = measure_peaks(dev)
        for name in ("32b_decode_int8", "32b_decode_fp8"):
            x = run_chain(name, dict(WORKLOADS[name]), dev, 50, 5, False, breakdown=False)
            extra[name] = {k: x[k] for k in ("layer_us", "tops", "value_gbs", "roofline", "config")}
            add_measured_fraction(extra[name]["roofline"], extra["peaks_measured"])
        extra["32b_prefill_gate_int8"] = prefill_gate(dev)
        add_measured_fraction(extra["32b_prefill_gate_int8"]["roofline"], extra["peaks_measured"])
        extra["gemm_source_sha16"] = kernel_source_sha256("gemm")[:16]
        add_measured_fraction(r["roofline"], extra["peaks_measured"])

    cpu = None
    if any(L.get("prod") for L in chain):
        log("bench: no CPU baseline for chains with producers (the oracle chain has none)")
    elif not args.no_cpu_baseline:
        cpu = cpu_baseline(chain, shapes, M, qt, sigma, wl["kind"], s, r["bytes_step"], args.workload)

    out = {
        "metric": METRIC,
        "value": r["value_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["layer_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": qt,
        "data": "synthetic",
        "config": r["config"],
        "layer_us": r["layer_us"],
        "tops": r["tops"],
        "alg_bytes_per_step": r["bytes_step"],
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "linears": r["linears"],
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


def run_chain(name, wl, dev, steps, warmup, eager, breakdown=True):
    """Time one decoder layer's chain of quantized linears (the workload
    `name`): whole-step HIP graphs over distinct weight sets, the dominant
    GEMM alone in a graph of back-to-back launches, and (breakdown) eager
    per-linear times."""
    import torch

    from w8a8_gemm_rl_amd import binding as B

    M, qt, s = wl["M"], wl["qt"], 1.5
    chain, shapes, sigma = chain_spec(wl["chain"])
    K0 = shapes[chain[0]["name"]][1]

    # ---- buffers: activations, per-linear codes and outputs, one workspace
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    x = torch.randn((M, K0), generator=g, device=dev)
    if wl["kind"] == "outliers":
        n_out = int(round(0.01 * K0))
        ch = torch.randperm(K0, generator=g, device=dev)[:n_out]
        x[:, ch] *= 20.0
    elif wl["kind"] == "heavy":
        x = x * torch.exp(torch.randn((1, K0), generator=g, device=dev))
    x0 = x.to(torch.bfloat16)
    del x
    bufs = {}
    need = needq = 0
    for L in chain:
        N, K = shapes[L["name"]]
        bufs["y_" + L["name"]] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        bufs["q_" + L["name"]] = (torch.empty((M, K), dtype=B.code_dtype(qt), device=dev),
                                  torch.empty(M, dtype=torch.float32, device=dev))
        need = max(need, B.workspace_size("qr_w8a8_gemm", M, N, K, qt),
                   B.workspace_size("qr_linear_fused", M, N, K, qt))
        needq = max(needq, B.workspace_size("qr_w8a8_gemm_quant", M, N, K, qt))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    # one launch per linear: its own workspace, zeroed once (barrier words)
    wsq = torch.zeros(max(needq, 256), dtype=torch.uint8, device=dev)
    one_launch = wl.get("one_launch", False)

    small = set() if wl.get("no_small_m") else small_m_linears(chain, shapes, M, one_launch)
    sum_quant = (set() if wl.get("no_sum_quant") else
                 sum_quant_linears(B, chain, shapes, M, qt, small, one_launch))
    log(f"bench: {name} M={M} qt={qt}: building {wl['sets']} weight sets ...")
    layers = [Layer(chain, shapes, M, qt, sigma, 1000 * (j + 1), dev, x0, bufs, ws, s,
                    fused=wl.get("fused", True), one_launch=one_launch, wsq=wsq, small=small,
                    sum_quant=sum_quant)
              for j in range(wl["sets"])]
    torch.cuda.synchronize()
    # qr_w8a8_gemm_quant's one-launch path for the one-launch workload (the
    # mode is read when each call is made, so also while graphs are captured)
    B.set_fuse_override(1 if one_launch else 0)
    try:
        res = _time_chain(name, wl, layers, bufs, ws, chain, shapes, M, qt, s, small, sum_quant,
                          one_launch, steps, warmup, eager, breakdown)
    finally:
        B.set_fuse_override(0)
    del layers, bufs, ws, wsq
    torch.cuda.empty_cache()
    return res


def _time_chain(name, wl, layers, bufs, ws, chain, shapes, M, qt, s, small, sum_quant, one_launch,
                steps, warmup, eager, breakdown):
    import torch

    from w8a8_gemm_rl_amd import binding as B

    # ---- per-step algorithmic work
    gemm_bytes = {L["name"]: (fused_linear_bytes if L["name"] in small else linear_bytes)(
        M, *shapes[L["name"]]) for L in chain}
    ops_step = sum(2 * M * shapes[L["name"]][0] * shapes[L["name"]][1] for L in chain)
    quant_keys, qbytes = set(), 0
    for L in chain:
        if L["name"] in small:
            continue
        k = (L["src"], L["cols"], L.get("prod"))
        if k not in quant_keys:
            quant_keys.add(k)
            qbytes += quant_bytes(M, shapes[L["name"]][1], L.get("prod"))
    bytes_step = sum(gemm_bytes.values()) + qbytes
    n_epi = len(set(chain_keys(chain)[1].values())) if one_launch else 0
    n_sq = len(sum_quant)
    dom = max(chain, key=lambda L: (gemm_bytes[L["name"]], -chain.index(L)))["name"]
    Nd, Kd = shapes[dom]
    dom_ops = 2 * M * Nd * Kd
    dom_intensity = dom_ops / gemm_bytes[dom]
    dom_bound = "hbm" if dom_intensity < MFMA8_PEAK_TOPS / HBM_PEAK_GBS * 1000 else "mfma"

    # ---- warmup (eager)
    log(f"bench: warmup {warmup} steps")
    for i in range(warmup):
        layers[i % len(layers)].run()
    torch.cuda.synchronize()

    K = steps
    mode = "eager" if eager else "hip_graph"
    copy_us = None
    if eager:
        # Every op launched from the host; events around the dominant GEMM.
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        log(f"bench: timing {K} steps ({mode})")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            layers[i % len(layers)].run(per_linear={dom: evs[i]})
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dom_us = 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / K
    else:
        # One HIP graph per weight set holds the whole step (what a rollout
        # engine that captures its decode step replays); K replays, walking
        # the weight sets, between two synchronizations.
        log("bench: capturing one graph per weight set")
        whole = []
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        for L in layers:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                with torch.cuda.graph(gph, stream=st):
                    L.run()
            whole.append(gph)
        # The dominant GEMM alone: a graph of DOM_BATCH back-to-back launches
        # over the weight sets, replayed on stream `st` between events recorded
        # on `st`, so they measure the kernels with no host launch gap.
        dom_graph = torch.cuda.CUDAGraph()
        dom_fns = [next(f for kind, n, f in L.ops() if kind == "gemm" and n == dom) for L in layers]
        with torch.cuda.stream(st):
            with torch.cuda.graph(dom_graph, stream=st):
                for j in range(DOM_BATCH):
                    dom_fns[j % len(dom_fns)]()
        torch.cuda.synchronize()
        for gph in whole:  # one untimed replay each
            gph.replay()
        dom_graph.replay()
        torch.cuda.synchronize()

        log(f"bench: timing {K} steps ({mode})")
        t0 = time.perf_counter()
        for i in range(K):
            whole[i % len(whole)].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()

        reps = max(3, min(20, K // DOM_BATCH))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        with torch.cuda.stream(st):
            for a, b in evs:
                a.record(st)
                dom_graph.replay()
                b.record(st)
        torch.cuda.synchronize()
        dom_us = 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / (reps * DOM_BATCH)
        copy_us = copy_stream_us(B, layers, bufs, chain, dom, M, Nd, Kd, qt, small, one_launch,
                                 st, reps)
        del whole, dom_graph
    sec_step = (t1 - t0) / K

    # ---- per-linear breakdown (eager, events around every GEMM; not timed)
    linears = {}
    if breakdown:
        per = {L["name"]: [] for L in chain}
        reps = min(20, K)
        for i in range(reps):
            e = {L["name"]: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for L in chain}
            layers[i % len(layers)].run(per_linear=e)
            torch.cuda.synchronize()
            for n, (a, b) in e.items():
                per[n].append(a.elapsed_time(b) * 1000.0)
        for L in chain:
            n = L["name"]
            N_, K_ = shapes[n]
            us = sorted(per[n])[len(per[n]) // 2]
            # host-launched: at small M the host's own launch time between the
            # events is counted too, so these are upper bounds on the kernels
            linears[n] = dict(N=N_, K=K_, eager_us=round(us, 2),
                              eager_gbs=round(gemm_bytes[n] / us / 1e3, 1),
                              eager_tops=round(2 * M * N_ * K_ / us / 1e6, 1),
                              plan=(["small_m", 16 * small_m_rf(N_)] if n in small
                                    else list(B.gemm_plan(M, N_, K_, qt))))

    dom_plan = B.gemm_plan(M, Nd, Kd, qt)
    if dom in small:
        rf = small_m_rf(Nd)
        traffic_key = f"{name}:{dom}:M{M}:N{Nd}:K{Kd}:small_m:rows{16 * rf}"
        kernel = (f"{dom} linear {Nd}x{Kd} M={M} (small_m_linear_kernel: input quantized in the "
                  f"kernel, {16 * rf}-row blocks, K split over the waves)")
    else:
        traffic_key = (f"{name}:{dom}:M{M}:N{Nd}:K{Kd}:tile{dom_plan[0]}:split{dom_plan[1]}"
                       f":rows{dom_plan[2]}")
        kernel = f"{dom} GEMM {Nd}x{Kd} M={M} ({B.tile_name(dom_plan[0])}, splitk {dom_plan[1]})"
    roofline = roofline_object(dom_bound, gemm_bytes[dom], dom_ops, dom_us, qt)
    roofline.update({
        "traffic": committed_traffic(traffic_key, "small" if dom in small else "gemm"),
        "traffic_key": traffic_key,
        "kernel": kernel,
    })
    if copy_us:
        # the same tiling's operand copies, ring, waits and barriers without
        # the matrix work: the kernel's time against its copy pipeline's
        roofline["copy_stream_us"] = round(copy_us, 2)
        roofline["copy_stream_over_kernel"] = round(copy_us / dom_us, 4)
    config = {
        "workload": f"{name}: one decoder layer's W8A8 linears, M={M} tokens, "
                    + ", ".join(f"{L['name']} {shapes[L['name']][0]}x{shapes[L['name']][1]}"
                                for L in chain)
                    + f"; {len(quant_keys) + len(small)} per-token quantizations + {len(chain)} GEMMs"
                    + (f" in {len(chain) + len(quant_keys) - n_epi} launches ({n_epi} quantizations and "
                       f"the split-K sums in the GEMM epilogues)" if one_launch else
                       " as separate launches (quantizers, GEMMs, split-K sum kernels)"
                       + ("" if not n_sq else
                          f"; the split-K sums of {', '.join(L['name'] for L in chain if L['name'] in sum_quant)} "
                          f"also quantize the next linear's input ({n_sq} quantizer launches fewer)")
                       + ("" if not small else
                          f"; {', '.join(L['name'] for L in chain if L['name'] in small)} each as one "
                          f"launch that quantizes its own input"))
                    + ("" if not any(L.get("prod") for L in chain) else
                       (", producers (RMSNorm x2, SiLU x up) "
                        + ("fused into the quantizers" if wl.get("fused", True)
                           else "as separate torch ops"))),
        "M": M, "qtype": qt, "uaq_s": s, "weight_sets": len(layers), "timing": mode,
        "launches": "one per linear" if one_launch else "separate", "parallelism": "none (1 GPU)",
    }
    res = {
        "layer_us": round(sec_step * 1e6, 2),
        "value_gbs": round(bytes_step / sec_step / 1e9, 1),
        "tops": round(ops_step / sec_step / 1e12, 1),
        "bytes_step": bytes_step,
        "roofline": roofline,
        "linears": linears,
        "config": config,
    }
    return res


def copy_stream_us(B, layers, bufs, chain, dom, M, N, K, qt, small, one_launch, st, reps):
    """Mean time of qr_probe_copy_stream over the dominant GEMM's tiling (its
    plan's tile and rows, the same weight sets and input codes), timed like
    the GEMM: a graph of DOM_BATCH launches replayed between events on `st`.
    None where the probe does not replay the plan (other tiles, split K)."""
    import torch

    tile, split, rows = B.gemm_plan(M, N, K, qt)
    if dom in small or one_launch or split != 1 or tile not in (4, 8, 10) or K % 128:
        return None
    key = chain_keys(chain)[0]
    xq = next(bufs["q_" + L["name"]][0] for L in chain if key[L["name"]] == key[dom])
    bm = 128 if tile == 8 else 256
    sink = torch.empty(-(-N // rows) * -(-M // bm), dtype=torch.int32, device=xq.device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            for j in range(DOM_BATCH):
                B.probe_copy_stream(tile, layers[j % len(layers)].W[dom][0], xq, rows, sink=sink)
    graph.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    with torch.cuda.stream(st):
        for a, b in evs:
            a.record(st)
            graph.replay()
            b.record(st)
    torch.cuda.synchronize()
    del graph
    return 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / (reps * DOM_BATCH)


def copy_stream_variants(dev, rounds=7):
    """The copy-stream probe's variants on the 7B gate at 256 tokens (tile 8,
    K = 3584) and the 32B gate at 512 tokens (tile 4, K = 5120), INT8, each a
    graph of DOM_BATCH launches walking enough weight copies to exceed the
    256 MB Infinity Cache, replayed round-robin with the GEMM itself on the
    same codes: row-major codes as the GEMM reads them, row strides padded
    by one 128-byte line (weights and tokens), the weights read as K panels,
    no barrier per K step (alone and with panels), and every K step
    re-reading the first step's bytes (the operands resident in L2: the copy
    pipeline's rate when no miss reaches HBM). Median per-launch us."""
    import statistics

    import torch

    from w8a8_gemm_rl_amd import binding as B

    out = []
    for name, M, N, K in (("7b_gate_m256", 256, 18944, 3584), ("32b_gate_m512", 512, 27648, 5120)):
        tile, split, rows = B.gemm_plan(M, N, K, "int8")
        if split != 1 or tile not in (4, 8):
            continue
        ncopy = max(2, int(600e6 // (N * K)) + 1)
        g = torch.Generator(device=dev)
        g.manual_seed(N + K)
        W = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g) for _ in range(ncopy)]
        Wp = [torch.randint(-127, 128, (N, K + 128), dtype=torch.int8, device=dev, generator=g)[:, :K]
              for _ in range(ncopy)]
        X = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        Xp = torch.randint(-127, 128, (M, K + 128), dtype=torch.int8, device=dev, generator=g)[:, :K]
        sx = torch.rand(M, device=dev) * 1e-3
        sw = torch.rand(N, device=dev) * 1e-3
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.zeros(max(B.workspace_size("qr_w8a8_gemm", M, N, K, "int8"), 256), dtype=torch.uint8,
                         device=dev)
        bm = 256 if tile == 4 else 128
        sink = torch.empty(-(-N // rows) * -(-M // bm), dtype=torch.int32, device=dev)
        cases = {
            "gemm": lambda j: B.w8a8_gemm(X, sx, W[j], sw, "int8", Y=Y, ws=ws),
            "copies": lambda j: B.probe_copy_stream(tile, W[j], X, rows, sink=sink),
            "copies_padded_rows": lambda j: B.probe_copy_stream(tile, Wp[j], Xp, rows, sink=sink),
            "copies_k_panels": lambda j: B.probe_copy_stream(tile, W[j], X, rows, sink=sink, panel=True),
            "copies_no_barrier": lambda j: B.probe_copy_stream(tile, W[j], X, rows, sink=sink, barrier=False),
            "copies_k_panels_no_barrier": lambda j: B.probe_copy_stream(tile, W[j], X, rows, sink=sink,
                                                                        panel=True, barrier=False),
            "copies_l2_resident": lambda j: B.probe_copy_stream(tile, W[j], X, rows, sink=sink,
                                                                resident=True),
        }
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        graphs = {}
        with torch.cuda.stream(st):
            for key, fn in cases.items():
                fn(0)
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph, stream=st):
                    for j in range(DOM_BATCH):
                        fn(j % ncopy)
                graphs[key] = gph
        torch.cuda.synchronize()
        ts = {key: [] for key in graphs}
        with torch.cuda.stream(st):
            for gph in graphs.values():
                gph.replay()
            for _ in range(rounds):
                for key, gph in graphs.items():
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(st)
                    gph.replay()
                    b.record(st)
                    b.synchronize()
                    ts[key].append(a.elapsed_time(b) * 1000.0 / DOM_BATCH)
        out.append({"shape": name, "M": M, "N": N, "K": K, "tile": B.tile_name(tile), "rows": rows,
                    "weight_copies": ncopy,
                    "us": {key: round(statistics.median(v), 2) for key, v in ts.items()}})
        del graphs, W, Wp, X, Xp, Y, ws
        torch.cuda.empty_cache()
    return {"copy_stream_variants": out, "gemm_source_sha16": kernel_source_sha256()[:16]}


def gemm_bound_sweeps(dev, rounds=7):
    """What bounds the 7B gate GEMM at 256 tokens (INT8, 192 x 128 tiles,
    K = 3584): the GEMM and its copy stream alone (qr_probe_copy_stream)
    timed (1) at a fixed 192 weight rows per block while the number of
    blocks, 2 per weight tile, shrinks from the gate's 198 to 24 (N cut to
    fewer rows), and (2) on the gate's 18944 rows with 192 down to 152 rows
    owned per tile (198 to 250 blocks; the copies of the rows a tile does not
    own still issue and read zeros). Every case is a graph of launches
    walking 720 MB of weight codes (past the 256 MB Infinity Cache), replayed
    round-robin with the others; median per-launch us."""
    import statistics

    import torch

    from w8a8_gemm_rl_amd import binding as B

    M, K, NFULL, TILE, BN = 256, 3584, 18944, 8, 192
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    total = (720 << 20) // K
    Wall = torch.randint(-127, 128, (total, K), dtype=torch.int8, device=dev, generator=g)
    X = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
    sx = torch.rand(M, device=dev) * 1e-3
    sw = torch.rand(NFULL, device=dev) * 1e-3
    Y = torch.empty((M, NFULL), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    sink = torch.empty(2 * -(-NFULL // 152), dtype=torch.int32, device=dev)
    cases = {}  # key -> (N, rows, gemm?)
    for tiles in (99, 74, 50, 25, 12):
        N = min(tiles * BN, NFULL)
        cases[f"blocks{2 * tiles}_gemm"] = (N, BN, True)
        cases[f"blocks{2 * tiles}_copies"] = (N, BN, False)
    for rows in (176, 160, 152):
        cases[f"rows{rows}_gemm"] = (NFULL, rows, True)
        cases[f"rows{rows}_copies"] = (NFULL, rows, False)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graphs = {}
    try:
        with torch.cuda.stream(st):
            for key, (N, rows, gemm) in cases.items():
                sets = total // N
                launches = max(DOM_BATCH, sets)

                def fn(j, N=N, rows=rows, gemm=gemm, sets=sets):
                    Wj = Wall[(j % sets) * N:(j % sets + 1) * N]
                    if gemm:
                        B.w8a8_gemm(X, sx, Wj, sw[:N], "int8", Y=Y[:, :N], ws=ws)
                    else:
                        B.probe_copy_stream(TILE, Wj, X, rows, sink=sink)

                B.set_plan_override(TILE, 1, rows)
                assert B.gemm_plan(M, N, K, "int8") == (TILE, 1, rows)
                fn(0)
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph, stream=st):
                    for j in range(launches):
                        fn(j)
                graphs[key] = (gph, launches)
    finally:
        B.set_plan_override(-1)
    torch.cuda.synchronize()
    ts = {key: [] for key in graphs}
    with torch.cuda.stream(st):
        for gph, _ in graphs.values():
            gph.replay()
        for _ in range(rounds):
            for key, (gph, launches) in graphs.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                gph.replay()
                b.record(st)
                b.synchronize()
                ts[key].append(a.elapsed_time(b) * 1000.0 / launches)
    us = {key: round(statistics.median(v), 2) for key, v in ts.items()}
    blocks = [{"blocks": 2 * t, "rows": BN, "gemm_us": us[f"blocks{2 * t}_gemm"],
               "copies_us": us[f"blocks{2 * t}_copies"],
               "copy_bytes_per_block": (BN + 128) * K} for t in (99, 74, 50, 25, 12)]
    rows = [{"rows": BN, "blocks": 198, "gemm_us": us["blocks198_gemm"],
             "copies_us": us["blocks198_copies"], "copy_bytes_per_block": (BN + 128) * K}]
    rows += [{"rows": r, "blocks": 2 * -(-NFULL // r), "gemm_us": us[f"rows{r}_gemm"],
              "copies_us": us[f"rows{r}_copies"], "copy_bytes_per_block": (r + 128) * K}
             for r in (176, 160, 152)]
    del graphs, Wall
    torch.cuda.empty_cache()
    return {"gemm_bound_sweeps": {"shape": "7b_gate_m256 (M=256, N=18944, K=3584, INT8)",
                                  "tile": B.tile_name(TILE), "by_blocks": blocks, "by_rows": rows},
            "gemm_source_sha16": kernel_source_sha256()[:16]}


def roofline_object(bound, alg_bytes, alg_ops, us, qt):
    """Roofline of one kernel launch of `us` microseconds: algorithmic bytes
    per second against HBM peak, or operations per second against the dense
    8-bit MFMA peak (TOP/s for INT8, TFLOP/s for FP8)."""
    if bound == "hbm":
        achieved, peak, unit = alg_bytes / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak = alg_ops / (us * 1e-6) / 1e12, MFMA8_PEAK_TOPS
        unit = "TOP/s" if qt == "int8" else "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "kernel_us": round(us, 2),
            "alg_bytes_per_launch": alg_bytes, "alg_ops_per_launch": alg_ops}


def add_measured_fraction(roof, peaks):
    """Add the fraction against the peak measured on this GPU (same run)."""
    if not peaks:
        return
    if roof["bound"] == "hbm":
        p = peaks["hbm_read_gbs"]
    else:
        p = peaks["mfma_int8_tops"] if roof["unit"] == "TOP/s" else peaks["mfma_fp8_tflops"]
    roof["measured_peak"] = p
    roof["frac_of_measured_peak"] = round(roof["achieved"] / p, 4)


def measure_peaks(dev):
    """Peaks this GPU reaches (the library's measurement kernels): HBM read
    rate over a 4 GiB buffer, dense INT8 / FP8 MFMA rate, and the shader clock
    the matrix cores ran at (from the kernel's clock counters)."""
    import statistics

    import torch

    from w8a8_gemm_rl_amd import binding as B

    log("bench: measuring the HBM read and MFMA peaks")
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(2048, dtype=torch.int32, device=dev)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[reps // 2]

    t = timed(lambda: B.probe_read(buf, sink))
    hbm = buf.numel() / t / 1e9
    del buf
    out = {"hbm_read_gbs": round(hbm, 1), "hbm_read_buffer_bytes": 4 << 30}
    blocks, iters = 256, 4000  # one block of 8 waves per CU, all resident at once
    for qt, key, ops_per in (("int8", "mfma_int8_tops", 65536), ("fp8", "mfma_fp8_tflops", 131072)):
        res = {}
        t = timed(lambda: res.update(r=B.probe_mfma(qt, blocks, iters, dev)))
        _, ticks, khz = res["r"]
        tk = ticks.view(-1, 4).cpu().tolist()
        mhz = statistics.median((c1 - c0) / (w1 - w0) * khz / 1e3 for c0, c1, w0, w1 in tk if w1 > w0)
        out[key] = round(blocks * 8 * iters * 8 * ops_per / t / 1e12, 1)
        out["sclk_mhz_" + qt] = round(mhz, 0)
    out["kernels"] = "read_probe_kernel (16-byte non-temporal loads, 4 GiB once), mfma_probe_kernel (256 blocks x 8 waves, " \
                     "8 independent 32x32 MFMAs per round, 4000 rounds)"
    torch.cuda.empty_cache()
    return out


def prefill_gate(dev):
    """The 32B prefill gate projection (27648x5120, INT8, 4096 tokens with
    heavy-tailed channels): a graph of 20 launches over two weight copies."""
    import torch

    from w8a8_gemm_rl_amd import binding as B
    from w8a8_gemm_rl_amd import inputs as I

    M, (N, K) = 4096, I.LINEARS_32B["gate"]
    qt = "int8"
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    x = torch.randn((M, K), generator=g, device=dev) * torch.exp(torch.randn((1, K), generator=g, device=dev))
    xq, sx = B.quantize_act_per_token(x.to(torch.bfloat16), 1.5, qt)
    del x
    sets = []
    for j in range(2):
        W = torch.randn((N, K), generator=g, device=dev) * I.W_SIGMA_32B
        sets.append(B.quantize_weights_uaq(W, 1.5, qt))
        del W
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(B.workspace_size("qr_w8a8_gemm", M, N, K, qt), 256), dtype=torch.uint8,
                     device=dev)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        B.w8a8_gemm(xq, sx, *sets[0], qt, Y=Y, ws=ws)
        with torch.cuda.graph(gph, stream=st):
            for i in range(DOM_BATCH):
                B.w8a8_gemm(xq, sx, *sets[i % 2], qt, Y=Y, ws=ws)
    torch.cuda.synchronize()
    ts = []
    with torch.cuda.stream(st):
        gph.replay()
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            gph.replay()
            b.record(st)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1000.0 / DOM_BATCH)
    us = sorted(ts)[2]
    plan = B.gemm_plan(M, N, K, qt)
    roof = roofline_object("mfma", linear_bytes(M, N, K), 2 * M * N * K, us, qt)
    roof["kernel"] = f"gate GEMM {N}x{K} M={M} ({B.tile_name(plan[0])}, splitk {plan[1]})"
    if plan[1] == 1 and plan[0] in (4, 8):
        # the tiling's operand copies alone (qr_probe_copy_stream), timed alike
        bm = 256 if plan[0] == 4 else 128
        sink = torch.empty(-(-N // plan[2]) * -(-M // bm), dtype=torch.int32, device=dev)
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(cg, stream=st):
                for i in range(DOM_BATCH):
                    B.probe_copy_stream(plan[0], sets[i % 2][0], xq, plan[2], sink=sink)
        torch.cuda.synchronize()
        cts = []
        with torch.cuda.stream(st):
            cg.replay()
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                cg.replay()
                b.record(st)
                b.synchronize()
                cts.append(a.elapsed_time(b) * 1000.0 / DOM_BATCH)
        del cg
        roof["copy_stream_us"] = round(sorted(cts)[2], 2)
        roof["copy_stream_over_kernel"] = round(sorted(cts)[2] / us, 4)
    del sets, Y, ws, xq, sx, gph
    torch.cuda.empty_cache()
    return {"us": round(us, 2), "tops": round(2 * M * N * K / us / 1e6, 1), "roofline": roof,
            "config": "32B prefill gate projection, INT8, X[4096, 5120] (heavy-tailed channels) x "
                      "W[27648, 5120], 2 weight copies, graph of 20 launches"}


if __name__ == "__main__":
    main()
