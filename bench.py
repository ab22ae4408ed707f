"""Benchmark of the MC2 per-rank hot path on one MI355X.

One step runs every operator once on its full-size synthetic workload, in
this order (names as in the JSON "rows"):

  ag_bf16_tp   AllGatherMatmul, 8 x bf16 (512, 4096) shards @ (4096, 1792), + gather_out
  ag_arrival   the same in arrival-emulation mode: a side-stream copy kernel lands the
               shards in gather_out chunk by chunk and the GEMM waits per chunk
  colpar_dx    column-parallel backward dX = dY (8192, 1792) @ W (1792, 4096)
  colpar_dw    column-parallel backward dW = dY^T (1792, 8192) @ AG(X) (8192, 4096)
  rs_fwd       MatmulReduceScatter, rank 0 of 8: row-parallel forward partial x (4096, 1792) @
               w^T (w (4096, 1792)), its own (512, 4096) block reduced with 7 received blocks
  rs_dx        MatmulReduceScatter completing dX: dY (8192, 1792) @ W (1792, 4096), own
               (1024, 4096) block reduced with 7 received blocks
  a16w8        AlltoAllQuantMatmul A16W8: permute+quant of bf16 (8192, 4096) on 8 ranks,
               then int8 (1024, 32768) @ (32768, 7168) with per-token x per-channel dequant + bias
  a8w8         AlltoAllQuantMatmul, full quantisation: int8 (8192, 4096) on 8 ranks with
               per-token scales, the permute folded into the int8 GEMM's loads, same GEMM
  a16w4        AlltoAllQuantMatmul A16W4: the a16w8 chain with an int4 weight (32768, 7168), two codes per byte
  a4w4         AlltoAllQuantMatmul A4W4 (full quantisation): int4 (8192, 4096) on 8 ranks with per-token
               scales, int4 weight (32768, 7168)
  qar_int8     QuantAllReduce, 8 ranks x int8 (4, 2048, 7168) + fp32 group-128 scales -> fp32
  qar_mx       QuantAllReduce, 8 ranks x E4M3FN (4, 2048, 7168) + E8M0 mx scales -> bf16
  qrs_int8     QuantReduceScatter, rank 3's share of the qar_int8 workload: 1024 of 8192 rows -> fp32
  ag_tiny      the AllGatherMatmul page's example: 8 x fp16 (16, 512) @ (512, 64) (launch-latency bound;
               its microseconds per call are the figure)

Inputs are generated on the host, copied to HBM before timing, and stay
resident.  --copy-calib adds a plain 256 MiB device copy to every step (the
reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters to bytes);
--summarize DIR turns a directory of rocprofv3 CSV output into the summary
kept under profiles/.  W warm-up steps (default 5), then exactly K timed steps
(default 50) between two synchronisations.  Per-call durations come from HIP
events recorded on the stream the kernels run on (torch's current stream,
which libmc2 is handed); each row reports their mean (the roofline figure),
minimum and median.  Every step runs all rows, so each call finds the caches
holding the other rows' data (largely dirty outputs), not its own inputs.
The headline value is the AllGatherMatmul's TFLOP/s; every row's figure and
its roofline fraction are in "rows".  The oracle (CPU) is timed on bounded
samples of the AllGatherMatmul, A16W8, backward and QuantAllReduce workloads
and on the page's example for the "cpu_baseline" entry (with the CPU model,
thread count and GPU / oracle ratios).
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

PEAK_BF16 = 2500.0     # TFLOP/s, dense MFMA, MI355X
PEAK_INT8 = 5000.0     # TOP/s, dense MFMA, MI355X
PEAK_HBM = 8000.0      # GB/s, MI355X HBM3E

ALL_ROWS = ["ag_bf16_tp", "ag_arrival", "colpar_dx", "colpar_dw", "rs_fwd", "rs_dx", "a16w8", "a8w8", "a16w4",
            "a4w4", "qar_int8", "qar_mx", "qrs_int8", "ag_tiny"]
EXTRA_ROWS = ["copy_calib"]
COPY_CALIB_BYTES = 256 << 20

# Kernel sources whose hash keys the stored traffic counters of the dominant kernel.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_bf16_ag.json")
TRAFFIC_SOURCES = ["comm_matmul_tensor_amd/csrc/gemm_mfma.hpp", "comm_matmul_tensor_amd/csrc/gemm16.hpp",
                   "comm_matmul_tensor_amd/csrc/gemm_bf16.hip", "comm_matmul_tensor_amd/csrc/device.hpp",
                   "comm_matmul_tensor_amd/csrc/kernels.hpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rows", default=",".join(ALL_ROWS), help="comma-separated subset of rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the sampled oracle check")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle work for the CPU baseline")
    ap.add_argument("--copy-calib", action="store_true", help="add a plain 256 MiB device copy to every step")
    ap.add_argument("--summarize", metavar="DIR", help="summarise rocprofv3 CSV output in DIR and exit")
    ap.add_argument("--write-traffic", action="store_true",
                    help="with --summarize: store the dominant kernel's scaled traffic for later bench lines")
    return ap.parse_args()


class Row:
    """One operator on its workload: setup -> callables run each step."""

    def __init__(self, name, unit, bound, peak, work, launches):
        self.name, self.unit, self.bound, self.peak, self.work = name, unit, bound, peak, work
        self.launches = launches  # list of (kernel label, fn)
        self.ms = []


def setup_rows(names, mc2, torch):
    import numpy as np

    import mc2_inputs
    T = mc2_inputs.to_torch
    rows = {}
    if "ag_bf16_tp" in names:
        seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
        t = mc2_inputs.make("ag_bf16_tp")
        shards = [T(t[f"shard{i}"], "bf16") for i in range(d["r"])]
        x2 = T(t["x2"], "bf16")
        m, k, n = d["r"] * d["m_local"], d["k"], d["n"]
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        g = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
        row = Row("ag_bf16_tp", "TFLOP/s", "mfma", PEAK_BF16, 2.0 * m * n * k,
                  [("gemm_bf16", lambda shards=shards, x2=x2, out=out, g=g:
                    mc2.mc2_allgather_matmul(shards, x2, out=out, gather_out=g))])
        row.bytes = 2 * (m * k + k * n + m * n + m * k)
        row.check = lambda t=t, d=d, out=out, g=g: check_ag(t, d, out, g)
        rows[row.name] = row
    if "ag_arrival" in names:
        seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
        t = mc2_inputs.make("ag_bf16_tp")
        shards = [T(t[f"shard{i}"], "bf16") for i in range(d["r"])]
        x2 = T(t["x2"], "bf16")
        m, k, n = d["r"] * d["m_local"], d["k"], d["n"]
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        g = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
        row = Row("ag_arrival", "TFLOP/s", "mfma", PEAK_BF16, 2.0 * m * n * k,
                  [("arrive_copy+gemm_bf16", lambda shards=shards, x2=x2, out=out, g=g:
                    mc2.mc2_allgather_matmul(shards, x2, out=out, gather_out=g, mode=mc2.MC2_AG_ARRIVAL,
                                             rank_id=0))])
        row.bytes = 2 * (m * k + k * n + m * n + m * k)
        row.check = lambda t=t, d=d, out=out, g=g, mc2=mc2: (check_ag(t, d, out, g) and
                                                            mc2.mc2_allgather_arrival_fallbacks() == 0)
        rows[row.name] = row
    if "colpar_dx" in names or "colpar_dw" in names:
        seed, d, specs = mc2_inputs.CONFIGS["colpar_bwd"]
        t = mc2_inputs.make("colpar_bwd")
        dy, w, x = T(t["dy"], "bf16"), T(t["w"], "bf16"), T(t["ag_x"], "bf16")
        m, nl, k = d["m"], d["n_local"], d["k"]
        dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((nl, k), dtype=torch.bfloat16, device="cuda")
        if "colpar_dx" in names:
            row = Row("colpar_dx", "TFLOP/s", "mfma", PEAK_BF16, 2.0 * m * nl * k,
                      [("gemm_bf16", lambda dy=dy, w=w, dx=dx: mc2.mc2_matmul_grad_input(dy, w, out=dx))])
            row.bytes = 2 * (m * nl + nl * k + m * k)
            row.check = lambda t=t, dx=dx: check_bwd(t, dx, "dx")
            rows[row.name] = row
        if "colpar_dw" in names:
            row = Row("colpar_dw", "TFLOP/s", "mfma", PEAK_BF16, 2.0 * m * nl * k,
                      [("gemm_bf16", lambda dy=dy, x=x, dw=dw: mc2.mc2_matmul_grad_weight(dy, x, out=dw))])
            row.bytes = 2 * (m * nl + m * k + nl * k)
            row.check = lambda t=t, dw=dw: check_bwd(t, dw, "dw")
            rows[row.name] = row
    for name in ("rs_fwd", "rs_dx"):
        if name not in names:
            continue
        seed, d, specs = mc2_inputs.CONFIGS[name]
        t = mc2_inputs.make(name)
        r, rank, m, k, n, tr = d["r"], d["rank"], d["m"], d["k"], d["n"], d["x2_trans"]
        x, x2 = T(t["x"], "bf16"), T(t["x2"], "bf16")
        recv = [None if j == rank else T(t[f"recv{j}"], "bf16") for j in range(r)]
        out = torch.empty((m // r, n), dtype=torch.bfloat16, device="cuda")
        part = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        row = Row(name, "TFLOP/s", "mfma", PEAK_BF16, 2.0 * m * k * n,
                  [("gemm_bf16_rs", lambda x=x, x2=x2, recv=recv, rank=rank, tr=tr, out=out, part=part:
                    mc2.mc2_matmul_reduce_scatter(x, x2, recv, rank, x2_trans=tr, out=out, partial_out=part))])
        rows_ = m // r
        row.bytes = 2 * (m * k + k * n + (m - rows_) * n + (r - 1) * rows_ * n + rows_ * n)
        row.check = lambda t=t, d=d, out=out, part=part: check_rs(t, d, out, part)
        rows[row.name] = row
    if "a16w8" in names:
        seed, d, specs = mc2_inputs.CONFIGS["a16w8"]
        t = mc2_inputs.make("a16w8")
        r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
        x1, x2 = T(t["x1"], "bf16"), T(t["x2"], "i8")
        s2, sm, bias = T(t["x2_scale"], "f32"), T(t["x1_smooth"], "bf16"), T(t["bias"], "bf16")
        rows_, cols = bs // r, r * h
        out = torch.empty((rows_, n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mc2.mc2_alltoall_quant_matmul_workspace_size(r, bs, h, n), dtype=torch.uint8, device="cuda")
        row = Row("a16w8", "TOP/s", "mfma", PEAK_INT8, 2.0 * rows_ * cols * n,
                  [("permute_quant+gemm_i8", lambda x1=x1, r=r, x2=x2, s2=s2, sm=sm, bias=bias, out=out, ws=ws:
                    mc2.mc2_alltoall_quant_matmul(x1, r, x2, s2, sm, bias, out=out, workspace=ws))])
        row.bytes = 2 * bs * h + 2 * cols + cols * n + 4 * n + 2 * n + 2 * rows_ * n
        row.check = lambda t=t, d=d, out=out: check_a16w8(t, d, out, mc2, torch)
        rows[row.name] = row
    if "a8w8" in names:
        seed, d, specs = mc2_inputs.CONFIGS["a8w8"]
        t = mc2_inputs.make("a8w8")
        r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
        x1, s1, x2 = T(t["x1"], "i8"), T(t["x1_scale"], "f32"), T(t["x2"], "i8")
        s2, bias = T(t["x2_scale"], "f32"), T(t["bias"], "bf16")
        rows_, cols = bs // r, r * h
        out = torch.empty((rows_, n), dtype=torch.bfloat16, device="cuda")
        row = Row("a8w8", "TOP/s", "mfma", PEAK_INT8, 2.0 * rows_ * cols * n,
                  [("gemm_i8", lambda x1=x1, r=r, s1=s1, x2=x2, s2=s2, bias=bias, out=out:
                    mc2.mc2_alltoall_quant_matmul_static(x1, r, s1, x2, s2, bias, out=out))])
        row.bytes = bs * h + 4 * rows_ + cols * n + 4 * n + 2 * n + 2 * rows_ * n
        row.check = lambda t=t, d=d, out=out: check_a8w8(t, d, out)
        rows[row.name] = row
    if "a16w4" in names:
        seed, d, specs = mc2_inputs.CONFIGS["a16w4"]
        t = mc2_inputs.make("a16w4")
        r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
        x1 = T(t["x1"], "bf16")
        x2 = torch.from_numpy(mc2_inputs.pack_int4(t["x2"])).cuda()
        s2, sm, bias = T(t["x2_scale"], "f32"), T(t["x1_smooth"], "bf16"), T(t["bias"], "bf16")
        rows_, cols = bs // r, r * h
        out = torch.empty((rows_, n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mc2.mc2_alltoall_quant_matmul_a16w4_workspace_size(r, bs, h, n), dtype=torch.uint8,
                         device="cuda")
        row = Row("a16w4", "TOP/s", "mfma", PEAK_INT8, 2.0 * rows_ * cols * n,
                  [("widen_int4+permute_quant+gemm_i8", lambda x1=x1, r=r, x2=x2, s2=s2, sm=sm, bias=bias, out=out,
                    ws=ws: mc2.mc2_alltoall_quant_matmul_a16w4(x1, r, x2, s2, sm, bias, out=out, workspace=ws))])
        row.bytes = 2 * bs * h + 2 * cols + cols * n // 2 + 4 * n + 2 * n + 2 * rows_ * n
        row.check = lambda t=t, d=d, out=out: check_w4(t, d, out, "a16w4")
        rows[row.name] = row
    if "a4w4" in names:
        seed, d, specs = mc2_inputs.CONFIGS["a4w4"]
        t = mc2_inputs.make("a4w4")
        r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
        x1 = torch.from_numpy(mc2_inputs.pack_int4(t["x1"])).cuda()
        x2 = torch.from_numpy(mc2_inputs.pack_int4(t["x2"])).cuda()
        s1, s2, bias = T(t["x1_scale"], "f32"), T(t["x2_scale"], "f32"), T(t["bias"], "bf16")
        rows_, cols = bs // r, r * h
        out = torch.empty((rows_, n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mc2.mc2_alltoall_quant_matmul_a4w4_workspace_size(r, bs, h, n), dtype=torch.uint8,
                         device="cuda")
        row = Row("a4w4", "TOP/s", "mfma", PEAK_INT8, 2.0 * rows_ * cols * n,
                  [("widen_int4+gemm_i8", lambda x1=x1, r=r, s1=s1, x2=x2, s2=s2, bias=bias, out=out, ws=ws:
                    mc2.mc2_alltoall_quant_matmul_a4w4(x1, r, s1, x2, s2, bias, out=out, workspace=ws))])
        row.bytes = bs * h // 2 + 4 * rows_ + cols * n // 2 + 4 * n + 2 * n + 2 * rows_ * n
        row.check = lambda t=t, d=d, out=out: check_w4(t, d, out, "a4w4")
        rows[row.name] = row
    for name, xdt, sdt, odt in (("qar_int8", "i8", "f32", torch.float32), ("qar_mx", "e4m3fn", "e8m0", torch.bfloat16)):
        if name not in names:
            continue
        seed, d, specs = mc2_inputs.CONFIGS[name]
        t = mc2_inputs.make(name)
        xs = [T(t[f"x{i}"], xdt) for i in range(d["r"])]
        sc = [T(t[f"scale{i}"], sdt) for i in range(d["r"])]
        out = torch.empty(d["shape"], dtype=odt, device="cuda")
        elems = int(np.prod(d["shape"]))
        sbytes = (4 * elems // 128) if sdt == "f32" else elems // 32
        nbytes = d["r"] * (elems + sbytes) + elems * out.element_size()
        row = Row(name, "GB/s", "hbm", PEAK_HBM, float(nbytes),
                  [("dequant_sum", (lambda xs=xs, sc=sc, out=out, odt=odt:
                                    mc2.mc2_quant_all_reduce(xs, sc, out_dtype=odt, out=out)))])
        row.bytes = nbytes
        row.check = (lambda t=t, d=d, out=out, xdt=xdt, sdt=sdt: check_qar(t, d, out, xdt, sdt))
        rows[name] = row
    if "qrs_int8" in names:
        seed, d, specs = mc2_inputs.CONFIGS["qar_int8"]
        t = mc2_inputs.make("qar_int8")
        r, rank = d["r"], 3
        xs = [T(t[f"x{i}"], "i8") for i in range(r)]
        sc = [T(t[f"scale{i}"], "f32") for i in range(r)]
        h = d["shape"][-1]
        nrows = int(np.prod(d["shape"][:-1]))
        out = torch.empty((nrows // r, h), dtype=torch.float32, device="cuda")
        elems = nrows // r * h
        nbytes = r * (elems + 4 * elems // 128) + 4 * elems
        row = Row("qrs_int8", "GB/s", "hbm", PEAK_HBM, float(nbytes),
                  [("dequant_sum", lambda xs=xs, sc=sc, out=out, rank=rank:
                    mc2.mc2_quant_reduce_scatter(xs, sc, rank, out_dtype=torch.float32, out=out))])
        row.bytes = nbytes
        row.check = lambda t=t, d=d, out=out, rank=rank: check_qrs(t, d, out, rank)
        rows[row.name] = row
    if "ag_tiny" in names:
        seed, d, specs = mc2_inputs.CONFIGS["ag_tiny"]
        t = mc2_inputs.make("ag_tiny")
        shards = [T(t[f"shard{i}"], "f16") for i in range(d["r"])]
        x2 = T(t["x2"], "f16")
        m, k, n = d["r"] * d["m_local"], d["k"], d["n"]
        out = torch.empty((m, n), dtype=torch.float16, device="cuda")
        g = torch.empty((m, k), dtype=torch.float16, device="cuda")
        row = Row("ag_tiny", "TFLOP/s", "latency", PEAK_BF16, 2.0 * m * n * k,
                  [("gemm_f16", lambda shards=shards, x2=x2, out=out, g=g:
                    mc2.mc2_allgather_matmul(shards, x2, out=out, gather_out=g))])
        row.bytes = 2 * (m * k + k * n + m * n + m * k)
        row.check = lambda t=t, d=d, out=out, g=g: check_ag_tiny(t, d, out, g)
        rows[row.name] = row
    if "copy_calib" in names:
        src = torch.empty(COPY_CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        row = Row("copy_calib", "GB/s", "hbm", PEAK_HBM, 2.0 * COPY_CALIB_BYTES,
                  [("copy", lambda src=src, dst=dst: dst.copy_(src))])
        row.bytes = 2 * COPY_CALIB_BYTES
        row.check = lambda src=src, dst=dst: bool(torch.equal(src, dst))
        rows[row.name] = row
    return [rows[n] for n in ALL_ROWS + EXTRA_ROWS if n in rows]


# ---------------------------------------------------------------- sampled parity against the oracle
def _tol16(got, want, dtype):
    import numpy as np
    dec = (lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) if dtype == "bf16" else \
        (lambda a: a.view(np.float16).astype(np.float64))
    g, w = dec(got), dec(want)
    rms = np.sqrt(np.mean(w ** 2))
    return bool(np.all(np.abs(g - w) <= 1e-2 * np.abs(w) + 1e-2 * rms))


def check_ag(t, d, out, g):
    import numpy as np

    import mc2_inputs
    import oracle
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(d["r"] * d["m_local"], 24, replace=False))
    G = np.concatenate([t[f"shard{i}"] for i in range(d["r"])])
    want = oracle.matmul(np.ascontiguousarray(G[rows]), t["x2"], "bf16")
    got = mc2_inputs.from_torch(out)[rows]
    gat_ok = np.array_equal(mc2_inputs.from_torch(g), G)
    return bool(gat_ok and _tol16(got, want, "bf16"))


def check_ag_tiny(t, d, out, g):
    import mc2_inputs
    import oracle
    want, want_g = oracle.allgather_matmul([t[f"shard{i}"] for i in range(d["r"])], t["x2"], "f16")
    import numpy as np
    return bool(np.array_equal(mc2_inputs.from_torch(g).view(np.uint16), want_g.view(np.uint16)) and
                _tol16(mc2_inputs.from_torch(out), want, "f16"))


def check_bwd(t, res, which):
    import numpy as np

    import mc2_inputs
    import oracle
    rng = np.random.default_rng(1)
    got = mc2_inputs.from_torch(res)
    if which == "dx":
        rows = np.sort(rng.choice(t["dy"].shape[0], 24, replace=False))
        want = oracle.matmul(np.ascontiguousarray(t["dy"][rows]), t["w"], "bf16")
    else:
        rows = np.sort(rng.choice(t["dy"].shape[1], 24, replace=False))
        want = oracle.matmul(np.ascontiguousarray(t["dy"][:, rows]), t["ag_x"], "bf16", a_trans=True)
    return _tol16(got[rows], want, "bf16")


def check_rs(t, d, out, part):
    import numpy as np

    import mc2_inputs
    import oracle
    r, rank, m, k, tr = d["r"], d["rank"], d["m"], d["k"], d["x2_trans"]
    rows = m // r
    rng = np.random.default_rng(6)
    others = np.sort(rng.choice(np.arange(rows * (rank + 1), m), 6, replace=False))
    want = oracle.matmul(np.ascontiguousarray(t["x"][others]), t["x2"], "bf16", b_trans=tr)
    ok = _tol16(mc2_inputs.from_torch(part)[others], want, "bf16")
    ts = np.sort(rng.choice(rows, 4, replace=False))
    xsub = np.zeros((r * 4, k), dtype=t["x"].dtype)
    xsub[rank * 4:(rank + 1) * 4] = t["x"][rank * rows + ts]
    rsub = [None if j == rank else np.ascontiguousarray(t[f"recv{j}"][ts]) for j in range(r)]
    ref = oracle.matmul_reduce_scatter(xsub, t["x2"], rsub, rank, "bf16", tr)
    return bool(ok and _tol16(mc2_inputs.from_torch(out)[ts], ref["out"], "bf16"))


def check_a16w8(t, d, out, mc2, torch):
    import numpy as np

    import mc2_inputs
    import oracle
    r = d["r"]
    p = oracle.permute(t["x1"], r)
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(p.shape[0], 6, replace=False))
    q, s1 = oracle.smooth_quant(np.ascontiguousarray(p[toks]), t["x1_smooth"])
    acc = oracle.int8_matmul(q, t["x2"])
    want = oracle.dequant(acc, s1, t["x2_scale"], t["bias"])
    return _tol16(mc2_inputs.from_torch(out)[toks], want, "bf16")


def check_a8w8(t, d, out):
    import numpy as np

    import mc2_inputs
    import oracle
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(d["bs"] // d["r"], 6, replace=False))
    p = oracle.permute_i8(t["x1"], d["r"])
    acc = oracle.int8_matmul(np.ascontiguousarray(p[toks]), t["x2"])
    want = oracle.dequant(acc, t["x1_scale"][toks], t["x2_scale"], t["bias"])
    return _tol16(mc2_inputs.from_torch(out)[toks], want, "bf16")


def check_w4(t, d, out, kind):
    import numpy as np

    import mc2_inputs
    import oracle
    r = d["r"]
    rng = np.random.default_rng(5)
    toks = np.sort(rng.choice(d["bs"] // r, 6, replace=False))
    if kind == "a16w4":
        q, s1 = oracle.smooth_quant(np.ascontiguousarray(oracle.permute(t["x1"], r)[toks]), t["x1_smooth"])
    else:
        q = np.ascontiguousarray(t["x1"].reshape(r, d["bs"] // r, d["h"]).transpose(1, 0, 2)
                                 .reshape(d["bs"] // r, r * d["h"])[toks])
        s1 = t["x1_scale"][toks]
    acc = oracle.int8_matmul(q, oracle.unpack_int4(mc2_inputs.pack_int4(t["x2"])))
    want = oracle.dequant(acc, s1, t["x2_scale"], t["bias"])
    return _tol16(mc2_inputs.from_torch(out)[toks], want, "bf16")


def check_qar(t, d, out, xdt, sdt):
    import numpy as np

    import mc2_inputs
    import oracle
    r = d["r"]
    h = d["shape"][-1]
    rows = d["shape"][0] * d["shape"][1]
    rng = np.random.default_rng(3)
    sel = np.sort(rng.choice(rows, 16, replace=False))
    per = h // 128 if sdt == "f32" else h // 32
    xs = [np.ascontiguousarray(t[f"x{i}"].reshape(rows, h)[sel]) for i in range(r)]
    sc = [np.ascontiguousarray(t[f"scale{i}"].reshape(rows, per)[sel]) for i in range(r)]
    want = oracle.quant_all_reduce(xs, sc, xdt, sdt, "f32" if out.dtype.itemsize == 4 else "bf16")
    got = mc2_inputs.from_torch(out).reshape(rows, h)[sel]
    view = np.uint32 if want.dtype == np.float32 else np.uint16
    return bool(np.array_equal(got.view(view), want.view(view)))


def check_qrs(t, d, out, rank):
    import numpy as np

    import mc2_inputs
    import oracle
    r = d["r"]
    h = d["shape"][-1]
    rows = int(np.prod(d["shape"][:-1]))
    blk = rows // r
    rng = np.random.default_rng(7)
    sel = np.sort(rng.choice(blk, 16, replace=False))
    xs = [np.ascontiguousarray(t[f"x{i}"].reshape(rows, h)[rank * blk + sel]) for i in range(r)]
    sc = [np.ascontiguousarray(t[f"scale{i}"].reshape(rows, h // 128)[rank * blk + sel]) for i in range(r)]
    want = oracle.quant_all_reduce(xs, sc, "i8", "f32", "f32")
    got = mc2_inputs.from_torch(out)[sel]
    return bool(np.array_equal(got.view(np.uint32), want.view(np.uint32)))


# ---------------------------------------------------------------- CPU baseline (the oracle)
def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def _scaled_run(run, full, target_s, probe):
    """Times run(n) on a prefix of n of `full` units: a probe, then the size that takes
    about target_s (the whole workload, repeated, if that is quicker).  Returns
    (units per run, runs, seconds)."""
    dt = run(probe)
    n = int(min(full, max(probe, probe * target_s / max(dt, 1e-3))))
    reps = 1
    if n == full:
        reps = max(1, int(target_s / max(run(n), 1e-3)))
    total = sum(run(n) for _ in range(reps))
    return n, reps, total


def cpu_baseline(target_s, gpu_rows):
    """The oracle, as it stands, on the host cores: the AllGatherMatmul workload (the
    headline object), plus the A16W8, column-parallel backward and QuantAllReduce
    workloads and the API page's example, each on a bounded sample scaled to the
    metric's unit, with the GPU / oracle ratio."""
    import numpy as np

    import mc2_inputs
    import oracle

    # AllGatherMatmul (8 x (512, 4096) @ (4096, 1792)): a prefix of each shard's rows
    seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
    t = mc2_inputs.make("ag_bf16_tp")
    r, k, n = d["r"], d["k"], d["n"]
    x2 = t["x2"]
    run = lambda rows: _timed(lambda: oracle.allgather_matmul(
        [np.ascontiguousarray(t[f"shard{i}"][:rows]) for i in range(r)], x2, "bf16"))
    per, reps, tot = _scaled_run(run, d["m_local"], target_s * 0.4, 64)
    ag = 2.0 * r * per * k * n * reps / tot / 1e12
    res = {"value": round(ag, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"AllGatherMatmul oracle (fp64 accumulation) on {per} of {d['m_local']} rows of each of the "
                     f"{r} bf16 shards, k={k}, n={n}, run {reps} time(s): {tot:.1f} s wall",
           "cpu_model": _cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS", "unset")}
    configs = {}

    # A16W8 (permute + quant + int8 GEMM + dequant): a prefix of the tokens
    seed, d, specs = mc2_inputs.CONFIGS["a16w8"]
    t = mc2_inputs.make("a16w8")
    ra, bs, h, na = d["r"], d["bs"], d["h"], d["n"]
    rows_all = bs // ra
    p_all = oracle.permute(t["x1"], ra)

    def a16(tok):
        q, s1 = oracle.smooth_quant(np.ascontiguousarray(p_all[:tok]), t["x1_smooth"])
        oracle.dequant(oracle.int8_matmul(q, t["x2"]), s1, t["x2_scale"], t["bias"])
    per, reps, tot = _scaled_run(lambda tok: _timed(lambda: a16(tok)), rows_all, target_s * 0.25, 16)
    v = 2.0 * per * ra * h * na * reps / tot / 1e12
    configs["a16w8"] = {"value": round(v, 5), "unit": "TOP/s", "sample": f"{per} of {rows_all} tokens, {reps} run(s), "
                        f"{tot:.1f} s (quantisation, exact int8 GEMM, exact dequant)"}

    # column-parallel backward dX = dY @ W and dW = dY^T @ AG(X): a prefix of the rows / columns
    seed, d, specs = mc2_inputs.CONFIGS["colpar_bwd"]
    t = mc2_inputs.make("colpar_bwd")
    m, nl, kk = d["m"], d["n_local"], d["k"]
    per, reps, tot = _scaled_run(lambda rows: _timed(lambda: oracle.matmul(
        np.ascontiguousarray(t["dy"][:rows]), t["w"], "bf16")), m, target_s * 0.15, 256)
    configs["colpar_dx"] = {"value": round(2.0 * per * nl * kk * reps / tot / 1e12, 5), "unit": "TFLOP/s",
                            "sample": f"{per} of {m} rows of dY, {reps} run(s), {tot:.1f} s"}
    per, reps, tot = _scaled_run(lambda cols: _timed(lambda: oracle.matmul(
        np.ascontiguousarray(t["dy"][:, :cols]), t["ag_x"], "bf16", a_trans=True)), nl, target_s * 0.1, 64)
    configs["colpar_dw"] = {"value": round(2.0 * per * m * kk * reps / tot / 1e12, 5), "unit": "TFLOP/s",
                            "sample": f"{per} of {nl} rows of dW, {reps} run(s), {tot:.1f} s"}

    # QuantAllReduce int8 + fp32 groups -> fp32: a prefix of the rows (bytes as the GPU row counts them)
    for name, xdt, sdt, odt, ob in (("qar_int8", "i8", "f32", "f32", 4), ("qar_mx", "e4m3fn", "e8m0", "bf16", 2)):
        seed, d, specs = mc2_inputs.CONFIGS[name]
        t = mc2_inputs.make(name)
        rq, hq = d["r"], d["shape"][-1]
        nrows = int(np.prod(d["shape"][:-1]))
        per_s = hq // 128 if sdt == "f32" else hq // 32
        xs = [t[f"x{i}"].reshape(nrows, hq) for i in range(rq)]
        sc = [t[f"scale{i}"].reshape(nrows, per_s) for i in range(rq)]
        sb = 4 * per_s if sdt == "f32" else per_s
        per, reps, tot = _scaled_run(lambda rows: _timed(lambda: oracle.quant_all_reduce(
            [np.ascontiguousarray(x[:rows]) for x in xs], [np.ascontiguousarray(s[:rows]) for s in sc], xdt, sdt,
            odt)), nrows, target_s * 0.05, 512)
        nbytes = per * (rq * (hq + sb) + hq * ob) * reps
        configs[name] = {"value": round(nbytes / tot / 1e9, 3), "unit": "GB/s",
                         "sample": f"{per} of {nrows} rows, {reps} run(s), {tot:.2f} s"}

    # the API page's example (8 x fp16 (16, 512) @ (512, 64)): median of 5, in us
    seed, d, specs = mc2_inputs.CONFIGS["ag_tiny"]
    t = mc2_inputs.make("ag_tiny")
    times = sorted(_timed(lambda: oracle.allgather_matmul([t[f"shard{i}"] for i in range(d["r"])], t["x2"], "f16"))
                   for _ in range(5))
    configs["ag_tiny"] = {"value": round(times[2] * 1e6, 1), "unit": "us per call", "sample": "median of 5 runs"}

    for key, c in configs.items():
        g = gpu_rows.get(key)
        if g is not None and c["value"] > 0:
            gv = g["us_per_call"] if c["unit"] == "us per call" else g["achieved"]
            c["gpu_over_oracle"] = round((c["value"] / gv) if c["unit"] == "us per call" else (gv / c["value"]), 1)
    res["gpu_over_oracle"] = round(gpu_rows["ag_bf16_tp"]["achieved"] / res["value"], 1) \
        if "ag_bf16_tp" in gpu_rows else None
    res["configs"] = configs
    return res


# ---------------------------------------------------------------- profile summaries and stored traffic
def _source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void mc2::", "")
    return name.split("(")[0]


def summarize(d, write_traffic):
    """Markdown summary of rocprofv3 CSV output under d: kernel-trace stats
    (*kernel_stats.csv) and per-dispatch counters (*counter_collection.csv in
    sub-directories named after the counter).  FETCH_SIZE and WRITE_SIZE are
    scaled by the ratio of the copy kernel's known bytes to what the same
    counter reads for it."""
    import csv
    import glob
    from collections import defaultdict
    lines = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        lines.append(f"Kernel trace ({os.path.relpath(f, d)}):\n")
        lines.append("| kernel | calls | avg us | min us | max us |")
        lines.append("|---|---|---|---|---|")
        for r in csv.DictReader(open(f)):
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        lines.append("")
    counters = defaultdict(lambda: defaultdict(list))
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            counters[_short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    scale = {}
    copy_names = [k for k in counters if "copy" in k.lower() or "elementwise_kernel" in k]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [v for k in copy_names for v in counters[k].get(c, []) if v * 1024 > COPY_CALIB_BYTES / 2]
        if vals:
            scale[c] = COPY_CALIB_BYTES / (1024.0 * sum(vals) / len(vals))
    mfma_names = ("MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_I8")
    if counters:
        names = sorted({c for k in counters for c in counters[k] if c not in mfma_names})
        lines.append("Counters, average per dispatch (FETCH_SIZE / WRITE_SIZE in KiB as read, and in MB after "
                     "scaling by the 256 MiB copy):\n")
        lines.append("| kernel | dispatches | " + " | ".join(names) + " | fetch MB (scaled) | write MB (scaled) |")
        lines.append("|---|---|" + "---|" * len(names) + "---|---|")
        for k, cs in sorted(counters.items()):
            if not any(c in cs for c in names):
                continue
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            n = max(len(v) for c, v in cs.items() if c in names)
            fm = avg.get("FETCH_SIZE", 0) * 1024 * scale.get("FETCH_SIZE", 1.0) / 1e6
            wm = avg.get("WRITE_SIZE", 0) * 1024 * scale.get("WRITE_SIZE", 1.0) / 1e6
            lines.append(f"| {k} | {n} | " + " | ".join(f"{avg.get(c, 0):.0f}" for c in names) +
                         f" | {fm:.1f} | {wm:.1f} |")
        lines.append("")
        lines.append("Copy-kernel scale factors (known bytes / counted bytes): " +
                     ", ".join(f"{c} {v:.4f}" for c, v in scale.items()) + "\n")
    mf = {k: cs for k, cs in counters.items() if "MfmaUtil" in cs}
    if mf:
        lines.append("MFMA counters, average per dispatch (MfmaUtil: MFMA-busy cycles over the dispatch's active "
                     "cycles x SIMDs, in %; MFMA ops: the MOPS counters x 512):\n")
        lines.append("| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP | int8 MFMA GOP |")
        lines.append("|---|---|---|---|---|")
        for k, cs in sorted(mf.items()):
            avg = {c: sum(v) / len(v) for c, v in cs.items()}
            if avg.get("MfmaUtil", 0) < 0.05:
                continue
            lines.append(f"| {k} | {len(cs['MfmaUtil'])} | {avg['MfmaUtil']:.1f} | "
                         f"{avg.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0) * 512 / 1e9:.2f} | "
                         f"{avg.get('SQ_INSTS_VALU_MFMA_MOPS_I8', 0) * 512 / 1e9:.2f} |")
        lines.append("")
    print("\n".join(lines))
    if write_traffic:
        # the fused AllGatherMatmul: bf16, 128 x 224 tiles, B N-contiguous, gather_out written by
        # the copy wavefronts
        ag = [k for k in counters if k.startswith("gemm16_gather_kernel<128, 224, false, 2>")]
        if not ag or not all(c in counters[ag[0]] for c in ("FETCH_SIZE", "WRITE_SIZE")):
            raise SystemExit("no FETCH_SIZE / WRITE_SIZE for the AllGatherMatmul kernel in " + d)
        cs = counters[ag[0]]
        fetch = sum(cs["FETCH_SIZE"]) / len(cs["FETCH_SIZE"]) * 1024 * scale.get("FETCH_SIZE", 1.0)
        write = sum(cs["WRITE_SIZE"]) / len(cs["WRITE_SIZE"]) * 1024 * scale.get("WRITE_SIZE", 1.0)
        rec = {"kernel": ag[0], "source_hash": _source_hash(), "fetch_bytes": round(fetch),
               "write_bytes": round(write), "scale": scale}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"wrote {TRAFFIC_FILE}: {rec}")


def stored_traffic():
    """HBM bytes per launch of the AllGatherMatmul kernel from the stored
    counters, or None if they are missing or the kernel changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != _source_hash():
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.write_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus above 1 is not supported "
                                   "(the r ranks are simulated as r buffers on one device)"}))
        sys.exit(2)
    import torch

    import comm_matmul_tensor_amd as mc2
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    names = [s for s in args.rows.split(",") if s]
    if args.copy_calib:
        names.append("copy_calib")
    for s in names:
        if s not in ALL_ROWS + EXTRA_ROWS:
            raise SystemExit(f"unknown row {s}")
    t0 = time.time()
    rows = setup_rows(names, mc2, torch)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f} s; rows: {[r.name for r in rows]}")

    stream = torch.cuda.current_stream()

    def step(record):
        for row in rows:
            if record:
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
            for _, fn in row.launches:
                fn()
            if record:
                ev1.record(stream)
                row.events.append((ev0, ev1))

    for row in rows:
        row.events = []
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log("warm-up done")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f} s")

    out_rows = {}
    for row in rows:
        ms = [a.elapsed_time(b) for a, b in row.events]
        avg_ms = sum(ms) / len(ms)
        achieved = row.work / (avg_ms * 1e-3) / (1e12 if row.unit != "GB/s" else 1e9)
        out_rows[row.name] = {"achieved": round(achieved, 2), "unit": row.unit, "bound": row.bound,
                              "peak": row.peak, "frac": round(achieved / row.peak, 4),
                              "us_per_call": round(avg_ms * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
                              "median_us": round(sorted(ms)[len(ms) // 2] * 1e3, 2),
                              "kernels": [k for k, _ in row.launches]}
    if not args.no_parity:
        for row in rows:
            t1 = time.time()
            out_rows[row.name]["parity"] = "pass" if row.check() else "FAIL"
            log(f"parity {row.name}: {out_rows[row.name]['parity']} ({time.time() - t1:.1f} s)")

    head = "ag_bf16_tp" if "ag_bf16_tp" in out_rows else rows[0].name
    h = out_rows[head]
    res = {
        "metric": "TFLOPS/TOPS (% MFMA peak) for AG-GEMM & A16W8; GB/s for dequant-sum",
        "value": h["achieved"], "unit": h["unit"], "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8" if head in ("a16w8", "a8w8") else "bf16", "data": "synthetic",
        "config": {"workload": {"ag_bf16_tp": "AllGatherMatmul bf16 TP layer: 8 x (512, 4096) shards @ (4096, 1792)",
                                }.get(head, head),
                   "rows_in_step": [r.name for r in rows], "seeds": "workload number (1..8)"},
        "roofline": {"bound": h["bound"], "achieved": h["achieved"], "peak": h["peak"],
                     "unit": "TFLOP/s" if h["unit"] == "TFLOP/s" else h["unit"], "frac": h["frac"],
                     "traffic": stored_traffic() if head == "ag_bf16_tp" else None,
                     "kernel": h["kernels"][0]},
        "rows": out_rows,
    }
    if not args.no_cpu_baseline:
        t1 = time.time()
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds, out_rows)
        log(f"cpu baseline {time.time() - t1:.1f} s")
    print(json.dumps(res))


if __name__ == "__main__":
    main()
