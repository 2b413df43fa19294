"""Throughput of Ozaki scheme II DGEMM/ZGEMM emulation on INT8 MFMA, one MI355X.

Default workload (the headline): square DGEMM M = N = K = 8192, op = N/N,
alpha = 1, beta = 0, entries (u - 1/2) exp(0.5 g), u ~ U(0,1), g ~ N(0,1),
seeded; one "step" is one emulated DGEMM at each s in {8, 12, 16} (three
calls, every phase of the method inside each).  Inputs are resident in HBM
before timing starts.

Other workloads (--workload), each printing the same kind of JSON line:
  wide4096   DGEMM 4096^3, op T/N, alpha 1.5, beta -0.5, random C, entries
             with exp(4 g) spread, s in {20, 24} (extended-width residues)
  zgemm4096  ZGEMM 4096^3 via the integer 3M form, op(A) = C (conjugate
             transpose), op(B) = N, alpha (0.7, -0.3), beta (0.2, 0.1),
             random C, s = 16; 8 MNK flops per call
  chain      Y = X x1 A x2 B x3 C for 32768 tensors of 16^3 with shared
             16 x 16 operators, one emulated product per mode (s = 16);
             metric GDoF/s = tensor entries per second of whole chains
  reuse8192  the headline product with op(A) prepared once and reused; each
             call re-encodes B (oz2_operand_update) and runs
             oz2_gemm_prepared (phase times: GEMM and reconstruct only)
  chain_rbe  the same chain by OzII-RescaleBE ("You Only Convert Twice",
             Algorithm 7): one kernel per chain, residues persist across the
             modes (rescaling + base extension), reconstruction once
  chain_sizes  OzII-RescaleBE over tensor sides n = 8 .. 256 at about 2^24
             entries per chain, s = 15 (the chain page's Sec. 6 throughput
             test): LDS kernel for n <= 16, HBM-resident kernels above
  nonsquare  the eight m x k x n shapes of the Arc page's Table 10 (k from
             256 to 65536, m or n from 1024 to 65536), N/N, U(-1,1) entries,
             s = 8 and 16; one step = the 16 calls, all inputs resident
  tiled8192  the headline product under a 1 GiB workspace cap: memory-aware
             tiling in blocks of C; reports each s's blocking and the
             slowdown against the same calls untiled
  datapower  the headline product at s = 16 on zero, constant, random-integer
             and headline operands: the residue GEMM's rate by operand data
  perfmodel  the performance model (the Arc page's Sec. 9.2 form: GEMM
             blocks + memory bytes + launches) fitted to square DGEMMs and
             checked on the non-square shapes of Table 10
  accuracy   the Arc page's accuracy protocol (Tables 6 and 8): 512 x 512 x
             4096 products of U(-1,1), phi = 2, sin/cos, spike, cancellation
             and 1 - 2^-53 data at s = 16, 20, 24; max ulp, correctly rounded
             share, componentwise and normwise error on 256 sampled entries
             against the exact products

Printed: ONE JSON line with the metric, per-call phase times (HIP events
recorded on the stream the kernels run on), the median and best step, the
memory phases against HBM ceilings measured on the same GPU with this
library's own stream kernels, the roofline of the dominant kernel, the
oracle's rate on a bounded sample on the host cores and on one core
(cpu_baseline), and how many of that sample's entries differ from one GPU
call at the same s (parity_sample).

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload dgemm8192]
       python bench.py --copy-calibration ...   (also runs a plain device copy of
       known size first, so that hardware byte counters taken over the same
       process can be scaled to bytes)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
# MI355X vector ALU in 32-bit lane operations per second: the published
# fp32 vector rate, 157.3 TFLOP/s, counts an FMA as two flops, so one
# operation of any kind per lane is 78.6 T/s (256 CUs x 128 lanes x 2.4 GHz)
PEAK_VALU_TOPS = 157.3 / 2
GEMM_SOURCE = os.path.join(ROOT, "complex_gemm_emulation_amd", "csrc", "oz2_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "residue_gemm_traffic.json")
SMALL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "small_gemm_traffic.json")
COPY_CAL_BYTES = 1 << 30     # bytes read (and written) by the calibration copy
METRIC = "emulated DGEMM TFLOP/s at N=8192, s=8/12/16 (+ INT8 MFMA util, HBM GB/s)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(m, n, k, s, cplx=False, beta_nonzero=False):
    """Minimum work of one call (each operand read once, INT8 intermediates).
    Complex: 3 residue sets per operand (re, im, re+im), 3s products, 2 outputs."""
    w = 2 if cplx else 1           # doubles per element
    sets = 3 if cplx else 1
    outs = 2 if cplx else 1
    return dict(
        int8_ops=2.0 * m * n * k * s * sets,
        scan_bytes=8.0 * w * (m * k + k * n),
        encode_bytes=(8.0 * w + sets * s) * (m * k + k * n),
        gemm_bytes=sets * s * (m * k + k * n) + outs * s * m * n,
        recon_bytes=(outs * s + 8.0 * w) * m * n + (8.0 * w * m * n if beta_nonzero else 0.0),
    )


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, traffic_file=TRAFFIC_FILE):
    """HBM bytes per launch of the bench's dominant kernel from the committed
    counter runs of this workload, or None when the kernel's sources changed
    since they were taken (or none were taken for this workload).  A record
    names its sources (several files hashed in order) or, for the residue
    GEMM, hashes oz2_gemm.hip."""
    try:
        with open(traffic_file) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if "sources" in rec:
        h = hashlib.sha256()
        for rel in rec["sources"]:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        digest = h.hexdigest()[:16]
    else:
        digest = source_digest(GEMM_SOURCE)
    if rec.get("source_sha256_16") != digest or rec.get("bench_workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(torch):
    """A plain device copy of COPY_CAL_BYTES bytes, three times: the
    reference against which FETCH_SIZE / WRITE_SIZE counters are scaled."""
    n = COPY_CAL_BYTES // 8
    src = torch.empty(n, dtype=torch.float64, device="cuda").uniform_(-1, 1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


STREAM_LIB = os.path.join(ROOT, "complex_gemm_emulation_amd", "liboz2_stream.so")


def hbm_ceilings(torch, nbytes=1 << 30, reps=3):
    """Measured HBM ceilings on this GPU: the best rate over launch shapes of
    this library's own read-only, write-only and copy stream kernels
    (liboz2_stream.so) on `nbytes` buffers, each shape timed `reps` times
    with events on the current stream after one untimed run.  Copy counts
    the bytes read plus the bytes written."""
    import ctypes
    lib = ctypes.CDLL(STREAM_LIB)
    lib.oz2_stream_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.oz2_stream_run.restype = ctypes.c_int
    src = torch.empty(nbytes // 8, dtype=torch.float64, device="cuda").uniform_(-1, 1)
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    best = {}
    for kind, name in ((0, "read"), (1, "write"), (2, "copy")):
        moved = nbytes * (2 if kind == 2 else 1)
        for blocks in (1024, 2048, 4096, 8192):
            for unroll in (2, 4, 8):
                for nt in (0, 1):
                    args = (kind, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                            blocks, unroll, nt, ctypes.c_void_p(st.cuda_stream))
                    if lib.oz2_stream_run(*args) != 0:
                        raise RuntimeError("oz2_stream_run failed")
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        lib.oz2_stream_run(*args)
                    e1.record()
                    torch.cuda.synchronize()
                    gbs = moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
                    if gbs > best.get(name, (0.0,))[0]:
                        best[name] = (gbs, f"{blocks}x256 threads, {unroll} x 16 B per trip"
                                           + (", nontemporal" if nt else ""))
    del src, dst
    out = {f"{k}_gbs": round(v[0], 1) for k, v in best.items()}
    out["shapes"] = {k: v[1] for k, v in best.items()}
    out["how"] = (f"best over 24 launch shapes of this library's stream kernels on {nbytes >> 20} MiB, "
                  "events on the stream; copy counts read + write bytes")
    return out


def sample_entries(m, n, side, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, min(side, m), replace=False)]))[:side]
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(side, n), replace=False)]))[:side]
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    return ii.reshape(-1), jj.reshape(-1), rows.size, cols.size


def cpu_baseline_gemm(spec, ops_a, A, B, C, s, side, label, got=None, single_side=64):
    """The oracle (as it stands) on a seeded side x side sample of output
    entries of the same workload, on all host cores, then on a smaller
    single_side^2 sample on one core.  got: the GPU's output of one call at
    this s (column-major, flat); the sample's entries are compared with it
    bit for bit and the count that differ is returned with the rates."""
    import oracle
    m, n, k = spec["m"], spec["n"], spec["k"]
    ii, jj, nr, nc = sample_entries(m, n, side, 12345)
    nt = oracle.max_threads()
    lda, ldb = ops_a
    t0 = time.perf_counter()
    r = oracle.gemm_entries(spec["cplx"], spec["transa"], spec["transb"], m, n, k, spec["alpha"], A, lda,
                            B, ldb, spec["beta"], C, m, s, rows=ii, cols=jj, nthreads=nt, chat_ints=False)
    dt = time.perf_counter() - t0
    flops_per_entry = (8.0 if spec["cplx"] else 2.0) * k
    i1, j1, _, _ = sample_entries(m, n, single_side, 54321)
    t1 = time.perf_counter()
    oracle.gemm_entries(spec["cplx"], spec["transa"], spec["transb"], m, n, k, spec["alpha"], A, lda,
                        B, ldb, spec["beta"], C, m, s, rows=i1, cols=j1, nthreads=1, chat_ints=False)
    dt1 = time.perf_counter() - t1
    out = dict(value=flops_per_entry * ii.size / dt / 1e12, unit="TFLOP/s", cores=nt, kind="oracle",
               sample=f"{nr}x{nc} sampled output entries of the {label} s={s} workload "
                      f"(exact wide-integer products), {dt:.1f} s",
               cpu_model=cpu_model(),
               single_thread=dict(value=flops_per_entry * i1.size / dt1 / 1e12, unit="TFLOP/s",
                                  sample=f"{i1.size} sampled entries, {dt1:.1f} s"))
    parity = None
    if got is not None:
        w = np.ascontiguousarray(r["out"])
        g = np.ascontiguousarray(got[ii + jj * m])
        wb, gb = w.view(np.uint64).reshape(w.size, -1), g.view(np.uint64).reshape(g.size, -1)
        parity = dict(s=s, entries=int(ii.size), not_bit_identical=int(np.count_nonzero(np.any(wb != gb, axis=1))),
                      how="one GPU call at this s on a fresh C, against the oracle at the sampled entries")
    return out, parity


GEMM_SPECS = {
    "dgemm8192": dict(cplx=False, m=8192, n=8192, k=8192, s=[8, 12, 16], transa="N", transb="N",
                      alpha=1.0, beta=0.0, phi=0.5, seedw=2, cpu_side=1024),
    "wide4096": dict(cplx=False, m=4096, n=4096, k=4096, s=[20, 24], transa="T", transb="N",
                     alpha=1.5, beta=-0.5, phi=4.0, seedw=3, cpu_side=640),
    "zgemm4096": dict(cplx=True, m=4096, n=4096, k=4096, s=[16], transa="C", transb="N",
                      alpha=complex(0.7, -0.3), beta=complex(0.2, 0.1), phi=0.5, seedw=4,
                      cpu_side=512),
    # the headline product with op(A) prepared once (oz2_operand_create) and
    # reused by every call: each call re-encodes B into a prepared op(B)
    # (oz2_operand_update) and runs oz2_gemm_prepared
    "reuse8192": dict(cplx=False, m=8192, n=8192, k=8192, s=[8, 12, 16], transa="N", transb="N",
                      alpha=1.0, beta=0.0, phi=0.5, seedw=2, cpu_side=1024, prepared_a=True),
    # the headline product under a 1 GiB workspace cap (memory-aware tiling):
    # the untiled workspace is 1.5 / 2.25 / 3 GiB at s = 8 / 12 / 16
    "tiled8192": dict(cplx=False, m=8192, n=8192, k=8192, s=[8, 12, 16], transa="N", transb="N",
                      alpha=1.0, beta=0.0, phi=0.5, seedw=2, cpu_side=1024, mem_limit=1 << 30),
}


def _dyadic(x):
    """integer mantissas and exponents: x = q 2^e exactly (finite doubles)"""
    mant, ex = np.frexp(np.asarray(x, dtype=np.float64))
    return (mant * 2.0 ** 53).astype(np.int64), ex.astype(np.int64) - 53


def _int_to_double(v, e):
    """v 2^e rounded once to double (CPython's integer true division rounds
    correctly)"""
    return float(v << e) if e >= 0 else v / (1 << -e)


def exact_dot(a, b):
    """sum_p a_p b_p of two double vectors, exact in integers, rounded once"""
    qa, ea = _dyadic(a)
    qb, eb = _dyadic(b)
    e = ea + eb
    e0 = int(e.min())
    tot = 0
    for x, y, z in zip(qa.tolist(), qb.tolist(), (e - e0).tolist()):
        tot += (x * y) << z
    return _int_to_double(tot, e0)


def exact_dot_fraction(a, b):
    """sum_p a_p b_p of two double vectors as an exact Fraction"""
    from fractions import Fraction
    qa, ea = _dyadic(a)
    qb, eb = _dyadic(b)
    e = ea + eb
    e0 = int(e.min())
    tot = 0
    for x, y, z in zip(qa.tolist(), qb.tolist(), (e - e0).tolist()):
        tot += (x * y) << z
    return Fraction(tot) * (Fraction(2) ** e0)


def entry_accuracy(got, Am, Bm, rows, cols):
    """Accuracy of computed entries against the exact products (Arc page
    Sec. 7: maximum error in ulps of the exact result, the share of correctly
    rounded entries, the componentwise error |c~ - c| / (|A||B|)_ij and the
    normwise relative error).  Am[i] is row i of op(A), Bm[j] column j of
    op(B) (real); got[q] the computed entry (rows[q], cols[q])."""
    from fractions import Fraction
    max_ulp = comp = 0.0
    cr = 0
    num = den = Fraction(0)
    for q, (i, j) in enumerate(zip(rows, cols)):
        a, b = Am[i], Bm[j]
        ex = exact_dot_fraction(a, b)
        g = float(got[q])
        rn = float(ex) if ex != 0 else 0.0   # CPython rounds a Fraction once, to nearest even
        cr += int(g == rn)
        err = abs(Fraction(g) - ex)
        if rn != 0.0:
            ulp = Fraction(2) ** (int(np.frexp(rn)[1]) - 53)
            max_ulp = max(max_ulp, float(err / ulp))
        elif err != 0:
            max_ulp = float("inf")
        aabb = float(np.dot(np.abs(a), np.abs(b)))
        if aabb > 0:
            comp = max(comp, float(err) / aabb)
        num += err * err
        den += ex * ex
    normwise = float((num / den) ** 0.5) if den != 0 else 0.0
    return dict(max_ulp=max_ulp, cr_pct=100.0 * cr / len(rows), componentwise=comp, normwise=normwise)


ACCURACY_DATA = ("uniform", "phi2", "sincos", "spike", "cancel", "one_minus_ulp")


def accuracy_operands(data, m, n, k, seed_base):
    """op(A) (m x k) and op(B) (k x n), N/N column-major, of one data family
    of the Arc page's Sec. 7 and Sec. 8.3"""
    import workloads
    if data == "uniform":
        return workloads.real_matrix(m, k, seed_base), workloads.real_matrix(k, n, seed_base + 1)
    if data == "phi2":
        return (workloads.real_matrix(m, k, seed_base, "phi", 2.0),
                workloads.real_matrix(k, n, seed_base + 1, "phi", 2.0))
    if data == "sincos":
        return workloads.sincos_matrix(m, k, seed_base), workloads.sincos_matrix(k, n, seed_base + 1)
    if data == "spike":
        # one element per row of A 2^40 times larger than the rest
        return workloads.spike_matrix(m, k, seed_base), workloads.real_matrix(k, n, seed_base + 1)
    if data == "cancel":
        return workloads.cancel_pair(m, n, k, seed_base)
    if data == "one_minus_ulp":
        return np.full(m * k, 1.0 - 2.0 ** -53), np.full(k * n, 1.0 - 2.0 ** -53)
    raise ValueError(data)


def run_accuracy(args):
    """The accuracy protocol of the Arc page (Sec. 7, Sec. 8.2-8.3, Tables 6
    and 8) on this GPU: 512 x 512 x 4096 DGEMM (N/N) for each data family at
    s = 16, 20, 24, the entries of a seeded 16 x 16 sample of rows and
    columns (256 entries, first and last included) compared with the exact
    products."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads
    m = n = 512
    k = 4096
    side = 16
    rng = np.random.default_rng(777)
    ri = np.unique(np.concatenate([[0, m - 1], rng.choice(m, side, replace=False)]))[:side]
    cj = np.unique(np.concatenate([[0, n - 1], rng.choice(n, side, replace=False)]))[:side]
    rows, cols = (x.reshape(-1) for x in np.meshgrid(ri, cj, indexing="ij"))
    h = oz2.Handle(torch.cuda.current_stream())
    table = {}
    t0 = time.perf_counter()
    for q, data in enumerate(ACCURACY_DATA):
        A, B = accuracy_operands(data, m, n, k, workloads.seed(8, 10 * q))
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dC = torch.zeros(m * n, dtype=torch.float64, device="cuda")
        Am, Bm = A.reshape(k, m).T, B.reshape(n, k)
        for s in (16, 20, 24):
            log(f"[bench] accuracy: {data}, s = {s}")
            h.dgemm("N", "N", m, n, k, 1.0, dA, m, dB, k, 0.0, dC, m, s)
            torch.cuda.synchronize()
            got = dC.cpu().numpy()[rows + cols * m]
            st = entry_accuracy(got, Am, Bm, rows, cols)
            st["t"] = oz2.plan_info(s, k)["t"]
            table[f"{data} s={s}"] = {key: (round(v, 4) if key == "cr_pct" else (float(f"{v:.3g}") if isinstance(v, float) else v))
                                      for key, v in st.items()}
    h.close()
    dt = time.perf_counter() - t0
    return {
        "metric": "accuracy of emulated DGEMM against exact products (512 x 512 x 4096, 256 sampled entries)",
        "value": table["uniform s=16"]["cr_pct"],
        "unit": "% correctly rounded (U(-1,1), s = 16)",
        "ms_per_step": round(dt * 1e3, 1),
        "dtype": "i8",
        "config": {"workload": "dgemm_512_512_4096_accuracy", "m": m, "n": n, "k": k, "s": [16, 20, 24],
                   "data": list(ACCURACY_DATA), "sample": f"{side} x {side} rows x columns"},
        "per_data": table,
    }


def general_accuracy(h, spec, A, B, C, s, count=32, seed=4242):
    """Normwise relative error of one call C <- alpha op(A) op(B) + beta C on
    a fresh copy of C (the timed steps overwrite C) at `count` seeded entries
    (first and last included), against alpha op(A) op(B) + beta C formed
    exactly in rationals and rounded once; complex entries count both parts."""
    import torch
    from fractions import Fraction
    m, n, k, cplx = spec["m"], spec["n"], spec["k"], spec["cplx"]
    ta, tb = spec["transa"], spec["transb"]
    ra = m if ta == "N" else k
    rb = k if tb == "N" else n
    dC = torch.from_numpy(C.copy()).cuda()
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    if cplx:
        h.zgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
    else:
        h.dgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
    torch.cuda.synchronize()
    got_all = dC.cpu().numpy()
    rng = np.random.default_rng(seed)
    ii = np.concatenate([[0, m - 1], rng.choice(m, count - 2)])
    jj = np.concatenate([[0, n - 1], rng.choice(n, count - 2)])
    Am = A.reshape(k, m).T if ta == "N" else A.reshape(m, k)   # Am[i] = row i of op(A) before conj
    Bm = B.reshape(n, k) if tb == "N" else B.reshape(k, n).T   # Bm[j] = column j of op(B) before conj
    al, be = complex(spec["alpha"]), complex(spec["beta"])
    Far, Fai, Fbr, Fbi = (Fraction(x) for x in (al.real, al.imag, be.real, be.imag))
    got, ref = [], []
    for i, j in zip(ii, jj):
        a, b = Am[i], Bm[j]
        c = C[i + j * m]
        if cplx:
            if ta == "C":
                a = np.conj(a)
            if tb == "C":
                b = np.conj(b)
            pr = exact_dot_fraction(a.real, b.real) - exact_dot_fraction(a.imag, b.imag)
            pi = exact_dot_fraction(a.real, b.imag) + exact_dot_fraction(a.imag, b.real)
            cr, ci = Fraction(c.real), Fraction(c.imag)
            ref += [float(Far * pr - Fai * pi + Fbr * cr - Fbi * ci), float(Far * pi + Fai * pr + Fbr * ci + Fbi * cr)]
            g = got_all[i + j * m]
            got += [g.real, g.imag]
        else:
            ref.append(float(Far * exact_dot_fraction(a, b) + Fbr * Fraction(float(c))))
            got.append(got_all[i + j * m])
    return normwise_error(got, ref), f"{count} seeded entries of one call on a fresh C vs alpha op(A) op(B) + beta C formed exactly"


def normwise_error(got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    return float(np.sqrt(np.sum((got - ref) ** 2) / np.sum(ref ** 2)))


def gemm_accuracy(dC, A, B, m, n, k, ta, tb, count=32, seed=4242):
    """Normwise relative error of C = op(A) op(B) (beta = 0) on `count`
    seeded entries (first and last included) against the exact product"""
    rng = np.random.default_rng(seed)
    ii = np.concatenate([[0, m - 1], rng.choice(m, count - 2)])
    jj = np.concatenate([[0, n - 1], rng.choice(n, count - 2)])
    C = dC.cpu().numpy()
    Am = A.reshape(k, m).T if ta == "N" else A.reshape(m, k)   # Am[i] = row i of op(A)
    Bm = B.reshape(n, k) if tb == "N" else B.reshape(k, n).T   # Bm[j] = column j of op(B)
    got = np.array([C[i + j * m] for i, j in zip(ii, jj)])
    ref = np.array([exact_dot(Am[i], Bm[j]) for i, j in zip(ii, jj)])
    return normwise_error(got, ref), f"{count} seeded entries vs the exact product"


def chain_accuracy(Y, X, ops, n, count):
    """Normwise relative error of the first `count` chains
    Y = X x1 A1 x2 A2 x3 A3 x1 A4 ... (operator i along direction i mod 3)
    against the exact chain, in integers"""
    n3 = n ** 3
    mats = []
    for a in ops:
        q, e = _dyadic(a)
        e0 = int(e.min())
        M = np.array([int(v) << int(z) for v, z in zip(q.tolist(), (e - e0).tolist())], dtype=object)
        mats.append((M.reshape(n, n).T, e0))   # M[i, j] = a[i + n j]
    errs_num = errs_den = 0.0
    for t in range(count):
        x = X[t * n3:(t + 1) * n3]
        q, e = _dyadic(x)
        nz = x != 0
        e0 = int(e[nz].min()) if nz.any() else 0
        T = np.array([int(v) << int(z - e0) if f else 0 for v, z, f in zip(q.tolist(), e.tolist(), nz.tolist())],
                     dtype=object).reshape(n, n, n).transpose(2, 1, 0)   # T[k1, k2, k3]
        esum = e0
        for i, (M, em) in enumerate(mats):
            m = i % 3
            T = np.moveaxis(np.tensordot(M, T, axes=([1], [m])), 0, m)
            esum += em
        ref = np.array([_int_to_double(int(v), esum) for v in T.transpose(2, 1, 0).reshape(-1)])
        got = Y[t * n3:(t + 1) * n3]
        errs_num += float(np.sum((got - ref) ** 2))
        errs_den += float(np.sum(ref ** 2))
    return float(np.sqrt(errs_num / errs_den)), f"first {count} tensors vs the exact chain"


def run_gemm(args, name):
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads

    spec = dict(GEMM_SPECS[name])
    if args.s:
        spec["s"] = [int(x) for x in args.s.split(",")]
    if args.n and name == "dgemm8192":
        spec["m"] = spec["n"] = spec["k"] = args.n
    m, n, k, cplx = spec["m"], spec["n"], spec["k"], spec["cplx"]
    ta, tb = spec["transa"], spec["transb"]
    w = workloads.seed
    ra, ca = workloads.stored_shape(ta, m, k)
    rb, cb = workloads.stored_shape(tb, k, n)
    log(f"[bench] {name}: generating inputs (seeded)")
    if cplx:
        A = workloads.complex_matrix(ra, ca, w(spec["seedw"], 0), w(spec["seedw"], 3), "phi", spec["phi"])
        B = workloads.complex_matrix(rb, cb, w(spec["seedw"], 1), w(spec["seedw"], 4), "phi", spec["phi"])
        C = workloads.complex_matrix(m, n, w(spec["seedw"], 2), w(spec["seedw"], 5), "uniform")
    else:
        A = workloads.real_matrix(ra, ca, w(spec["seedw"], 0), "phi", spec["phi"])
        B = workloads.real_matrix(rb, cb, w(spec["seedw"], 1), "phi", spec["phi"])
        C = workloads.real_matrix(m, n, w(spec["seedw"], 2), "uniform") if spec["beta"] != 0 else None
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    # beta != 0: C starts as the seeded random matrix; later calls update it in
    # place (|beta| < 1 keeps it bounded), the same work every call
    if C is not None:
        dC = torch.from_numpy(C.copy()).cuda()
    else:
        dC = torch.zeros(m * n, dtype=torch.complex128 if cplx else torch.float64, device="cuda")
    stream = torch.cuda.current_stream()
    s_list = spec["s"]
    handles = {s: oz2.Handle(stream) for s in s_list}
    for h in handles.values():
        h.set_timing(True)
        if spec.get("mem_limit"):
            h.set_memory_limit(spec["mem_limit"])

    prepared = {}
    if spec.get("prepared_a"):
        for s in s_list:
            prepared[s] = (handles[s].prepare("A", ta, m, k, dA, ra, s, cplx),
                           handles[s].prepare("B", tb, n, k, dB, rb, s, cplx))
        torch.cuda.synchronize()

    def step(record):
        for s in s_list:
            if prepared:
                pa, pb = prepared[s]
                handles[s].update(pb, dB, rb)
                handles[s].gemm_prepared(pa, pb, spec["alpha"], spec["beta"], dC, m)
            elif cplx:
                handles[s].zgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
            else:
                handles[s].dgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
        if record is not None:
            for s in s_list:
                record[s].append(handles[s].phase_times())

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    phases = {s: [] for s in s_list}
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for q in range(args.steps):
        step(phases)
        ev[q + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = [ev[q].elapsed_time(ev[q + 1]) for q in range(args.steps)]
    ms_per_step = dt / args.steps * 1e3
    fl = (8.0 if cplx else 2.0) * m * n * k
    value = fl * len(s_list) / (dt / args.steps) / 1e12

    per_s = {}
    gemm_ops = gemm_ms = 0.0
    beta_nz = spec["beta"] != 0
    for s in s_list:
        ph = np.mean(np.array(phases[s]), axis=0)  # ms: scan, encode, gemm, reconstruct
        wk = algorithmic(m, n, k, s, cplx, beta_nz)
        call_ms = float(np.sum(ph))
        if spec.get("mem_limit"):
            # a tiled call times only its whole duration
            per_s[str(s)] = dict(tflops=fl / (call_ms * 1e-3) / 1e12, ms=dict(call=round(call_ms, 4)))
            continue
        per_s[str(s)] = dict(
            tflops=fl / (call_ms * 1e-3) / 1e12,
            ms=dict(scan=round(float(ph[0]), 4), encode=round(float(ph[1]), 4),
                    gemm=round(float(ph[2]), 4), reconstruct=round(float(ph[3]), 4)),
            gemm_int8_tops=wk["int8_ops"] / (ph[2] * 1e-3) / 1e12,
            gemm_int8_util=wk["int8_ops"] / (ph[2] * 1e-3) / 1e12 / PEAK_INT8_TOPS,
            scan_gbs=wk["scan_bytes"] / (ph[0] * 1e-3) / 1e9,
            encode_gbs=wk["encode_bytes"] / (ph[1] * 1e-3) / 1e9,
            reconstruct_gbs=wk["recon_bytes"] / (ph[3] * 1e-3) / 1e9,
        )
        gemm_ops += wk["int8_ops"]
        gemm_ms += float(ph[2])
    tiling = None
    if spec.get("mem_limit"):
        # the same calls untiled, for the slowdown (own handles, no cap)
        plans = {str(s): handles[s].tile_plan() for s in s_list}
        free = {s: oz2.Handle(stream) for s in s_list}
        for _ in range(2):
            for s in s_list:
                free[s].dgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
        torch.cuda.synchronize()
        reps = max(3, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for s in s_list:
                free[s].dgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC, m, s)
        e1.record()
        torch.cuda.synchronize()
        untiled_ms = e0.elapsed_time(e1) / reps
        for h2 in free.values():
            h2.close()
        tiling = dict(mem_limit=spec["mem_limit"], plans=plans,
                      workspace_bytes={str(s): handles[s].workspace_size() for s in s_list},
                      untiled_ms_per_step=round(untiled_ms, 3),
                      slowdown=round(float(np.median(step_ms)) / untiled_ms, 4),
                      how="median tiled step over the untiled step of the same calls without a cap")

    # residue GEMM: one launch per call; the mean launch of a step does the
    # mean of the calls' INT8 ops, timed by HIP events on its stream
    achieved = gemm_ops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else 0.0
    roofline = dict(kernel="residue_gemm_kernel (INT8 MFMA, fused mod m)", bound="mfma",
                    achieved=round(achieved, 2), peak=PEAK_INT8_TOPS, unit="TOP/s",
                    frac=round(achieved / PEAK_INT8_TOPS, 4), traffic=measured_traffic(name),
                    ops_per_launch=gemm_ops / len(s_list),
                    launch_ms=round(gemm_ms / len(s_list), 4))
    if tiling:
        # a tiled call records only its whole duration (reported as the GEMM
        # phase), so the GEMM's own rate is not separable here
        roofline = None

    ceil = None
    if not args.no_ceiling:
        log("[bench] HBM ceilings: this library's read, write and copy stream kernels")
        ceil = hbm_ceilings(torch)
        for s in s_list:
            rec = per_s[str(s)]
            if "scan_gbs" not in rec:
                continue
            rec["scan_frac_of_read_ceiling"] = round(rec["scan_gbs"] / ceil["read_gbs"], 4)
            rec["encode_frac_of_copy_ceiling"] = round(rec["encode_gbs"] / ceil["copy_gbs"], 4)
            rec["reconstruct_frac_of_copy_ceiling"] = round(rec["reconstruct_gbs"] / ceil["copy_gbs"], 4)
            for ph in ("scan", "encode", "reconstruct"):
                rec[f"{ph}_frac_of_peak"] = round(rec[f"{ph}_gbs"] / PEAK_HBM_GBS, 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        s_cpu = s_list[-1]
        side = args.cpu_side or spec["cpu_side"]
        got = None
        if not prepared:
            log(f"[bench] one s={s_cpu} call on a fresh C for the sample's parity")
            dC2 = (torch.from_numpy(C.copy()).cuda() if C is not None else
                   torch.zeros(m * n, dtype=torch.complex128 if cplx else torch.float64, device="cuda"))
            h = handles[s_cpu]
            if cplx:
                h.zgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC2, m, s_cpu)
            else:
                h.dgemm(ta, tb, m, n, k, spec["alpha"], dA, ra, dB, rb, spec["beta"], dC2, m, s_cpu)
            torch.cuda.synchronize()
            got = dC2.cpu().numpy()
            del dC2
        log(f"[bench] oracle cpu baseline on a {side}^2 entry sample, s={s_cpu}")
        cpu, parity = cpu_baseline_gemm(spec, (ra, rb), A, B, C, s_cpu, side, f"{m}x{n}x{k}", got)

    accuracy = None
    if not cplx and spec["beta"] == 0:
        log(f"[bench] accuracy of the s={s_list[-1]} result on sampled entries")
        err, how = gemm_accuracy(dC, A, B, m, n, k, ta, tb)
        accuracy = {"normwise_rel_err": err, "s": s_list[-1], "sample": how}
    elif not prepared:
        accuracy = {}
        for s in s_list:
            log(f"[bench] accuracy of one s={s} call on sampled entries")
            err, how = general_accuracy(handles[s], spec, A, B, C, s)
            accuracy[str(s)] = err
        accuracy["sample"] = how

    for pa, pb in prepared.values():
        pa.close()
        pb.close()
    for h in handles.values():
        h.close()
    kind = "zgemm" if cplx else "dgemm"
    return {
        "metric": METRIC if name == "dgemm8192" else
                  f"emulated {'ZGEMM' if cplx else 'DGEMM'} TFLOP/s ({'8' if cplx else '2'}MNK/t)"
                  + (", op(A) prepared once and reused" if prepared else ""),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms_per_step, 3),
        "dtype": "i8",
        "config": {"workload": f"{kind}_{m}_{ta}{tb}_phi{spec['phi']}_s{'_'.join(map(str, s_list))}"
                               + ("_prepared_a" if prepared else "") + ("_cap1GiB" if spec.get("mem_limit") else ""),
                   "m": m, "n": n, "k": k, "s": s_list, "ops": f"{ta}/{tb}",
                   "alpha": str(spec["alpha"]), "beta": str(spec["beta"])},
        "step_ms": dict(median=round(float(np.median(step_ms)), 3), best=round(float(np.min(step_ms)), 3),
                        how="HIP events on the stream around each timed step"),
        "per_s": per_s,
        "hbm_ceiling": ceil,
        "tiling": tiling,
        "accuracy": accuracy,
        "parity_sample": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


def run_nonsquare(args):
    """The non-square shapes at s = 8 and 16: value = all calls' 2mnk flops
    over their total time; per shape and s the phase times."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads

    W = workloads.NONSQUARE
    s_list = list(W["s"])
    shapes = [tuple(x) for x in W["shapes"]]
    dev = []
    for q, (m, k, n) in enumerate(shapes):
        log(f"[bench] nonsquare: generating {m}x{k}x{n} (seeded)")
        A = workloads.real_matrix(m, k, workloads.nonsquare_seed(q, 0), W["dist"])
        B = workloads.real_matrix(k, n, workloads.nonsquare_seed(q, 1), W["dist"])
        dev.append((torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                    torch.zeros(m * n, dtype=torch.float64, device="cuda")))
        del A, B
    stream = torch.cuda.current_stream()
    handles = {s: oz2.Handle(stream) for s in s_list}
    for h in handles.values():
        h.set_timing(True)
    phases = {(q, s): [] for q in range(len(shapes)) for s in s_list}

    def step(record):
        for q, (m, k, n) in enumerate(shapes):
            dA, dB, dC = dev[q]
            for s in s_list:
                handles[s].dgemm("N", "N", m, n, k, 1.0, dA, m, dB, k, 0.0, dC, m, s)
                if record:
                    phases[(q, s)].append(handles[s].phase_times())

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    flops = sum(2.0 * m * n * k for (m, k, n) in shapes) * len(s_list)
    value = flops / (dt / args.steps) / 1e12
    per_shape = {}
    gemm_ops = gemm_ms = 0.0
    for q, (m, k, n) in enumerate(shapes):
        rec = {}
        for s in s_list:
            ph = np.mean(np.array(phases[(q, s)]), axis=0)
            wk = algorithmic(m, n, k, s)
            rec[str(s)] = dict(tflops=round(2.0 * m * n * k / (float(np.sum(ph)) * 1e-3) / 1e12, 2),
                               ms=dict(scan=round(float(ph[0]), 4), encode=round(float(ph[1]), 4),
                                       gemm=round(float(ph[2]), 4), reconstruct=round(float(ph[3]), 4)),
                               gemm_int8_tops=round(wk["int8_ops"] / (ph[2] * 1e-3) / 1e12, 1))
            gemm_ops += wk["int8_ops"]
            gemm_ms += float(ph[2])
        per_shape[f"{m}x{k}x{n}"] = rec
    achieved = gemm_ops / (gemm_ms * 1e-3) / 1e12
    calls = len(shapes) * len(s_list)
    roofline = dict(kernel="residue_gemm_kernel (INT8 MFMA, fused mod m)", bound="mfma",
                    achieved=round(achieved, 2), peak=PEAK_INT8_TOPS, unit="TOP/s",
                    frac=round(achieved / PEAK_INT8_TOPS, 4), traffic=None,
                    ops_per_launch=gemm_ops / calls, launch_ms=round(gemm_ms / calls, 4))
    cpu = None
    if not args.no_cpu_baseline:
        q = 1  # 8192 x 1024 x 8192
        m, k, n = shapes[q]
        A = workloads.real_matrix(m, k, workloads.nonsquare_seed(q, 0), W["dist"])
        B = workloads.real_matrix(k, n, workloads.nonsquare_seed(q, 1), W["dist"])
        spec = dict(m=m, n=n, k=k, cplx=False, transa="N", transb="N", alpha=1.0, beta=0.0)
        side = args.cpu_side or 1024
        log(f"[bench] oracle cpu baseline on a {side}^2 entry sample of {m}x{k}x{n}, s=16")
        cpu, _ = cpu_baseline_gemm(spec, (m, k), A, B, None, 16, side, f"{m}x{k}x{n}")
    for h in handles.values():
        h.close()
    return {
        "metric": "emulated DGEMM TFLOP/s over the Table 10 non-square shapes (2mnk/t)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(dt / args.steps * 1e3, 3),
        "dtype": "i8",
        "config": {"workload": "dgemm_nonsquare_table10_s8_16", "shapes_mkn": [list(x) for x in shapes],
                   "s": s_list, "ops": "N/N", "dist": W["dist"]},
        "per_shape": per_shape,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


RBE_OPS_BASIS = ("the page's steps per entry (repeated RnsDrop, mixed-radix BaseExtend, one elimination for the "
                 "final digits: rbe_valu_ops_per_entry); the kernels reach the same integers with fewer (drops at "
                 "once, CRT base extension, final digits in two blocks), so this is an effective rate")


def rbe_valu_ops_per_entry(s, g):
    """Vector-ALU operations per tensor entry that the modular steps of an
    OzII-RescaleBE chain of depth d = len(g) take, counting one per 32-bit
    lane operation and two per fp64 one: a centred reduction [x]_m is 3
    (fma, floor, fma), a mixed-radix or drop step [(x - y) c]_m is 5.  Per
    product, the s products of an entry are reduced; after every product but
    the last, with k = s - g kept moduli, RnsDrop takes sum_j (s - 1 - j)
    steps, the digits k (k - 1) / 2 steps and BaseExtend g sums of k
    products plus a reduction; ReconstructFP64 takes s (s - 1) / 2 digit
    steps, s - 1 fp64 Horner FMAs and one scaling.  The encode and the
    integer MFMA products are not counted."""
    g = list(g)
    ops = 3 * s * len(g)
    for gi in g[:-1]:
        k = s - gi
        ops += 5 * sum(s - 1 - j for j in range(gi)) + 5 * k * (k - 1) // 2 + gi * (k + 3)
    ops += 5 * s * (s - 1) // 2 + 2 * (s - 1) + 2
    return ops


def rbe_product_ops_per_entry(s, gi):
    """The part of rbe_valu_ops_per_entry that one non-final product takes:
    the reduction of the s products of an entry, gi drops, the digits of the
    k = s - gi kept moduli and the base extension to the gi dropped ones."""
    k = s - gi
    return 3 * s + 5 * sum(s - 1 - j for j in range(gi)) + 5 * k * (k - 1) // 2 + gi * (k + 3)


def run_chain_rbe(args):
    """The 32768 x 16^3 chain by OzII-RescaleBE: one kernel per chain, the
    tensor in residue form from encode to reconstruction."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads

    w = workloads.WORKLOADS[5]
    n, batch, s = w["n"], w["batch"], w["s"][0]
    n3 = n ** 3
    log(f"[bench] chain_rbe: generating {batch} tensors of {n}^3 (seeded)")
    X = workloads.tensor_batch(n, batch, workloads.seed(5, 0))
    depth = args.chain_depth
    ops = [workloads.real_matrix(n, n, workloads.seed(5, q)) for q in range(1, depth + 1)]
    dX = torch.from_numpy(X).cuda()
    dY = torch.empty_like(dX)
    h = oz2.Handle(torch.cuda.current_stream())
    h.set_timing(True)
    plan = h.chain_plan(ops, n, s)
    launch_ms = []

    def step(record):
        h.chain_rescale_be(plan, dX, dY, batch)
        if record is not None:
            launch_ms.append(h.phase_times()[2])

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(launch_ms)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    value = n3 * batch / (dt / args.steps) / 1e9
    lm = float(np.mean(launch_ms))
    ops_per_launch = float(rbe_valu_ops_per_entry(s, plan.g)) * n3 * batch
    achieved = ops_per_launch / (lm * 1e-3) / 1e12
    bytes_per_launch = 16.0 * n3 * batch  # each input entry read and each output entry written once
    roofline = dict(kernel="chain_kernel (OzII-RescaleBE, whole chain)", bound="alu",
                    achieved=round(achieved, 2), peak=round(PEAK_VALU_TOPS, 2), unit="TOP/s",
                    frac=round(achieved / PEAK_VALU_TOPS, 4), traffic=None,
                    ops_per_launch=ops_per_launch, launch_ms=round(lm, 4),
                    ops_basis=RBE_OPS_BASIS,
                    hbm_GBs=round(bytes_per_launch / (lm * 1e-3) / 1e9, 1))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nt = args.chain_rbe_cpu_tensors
        log(f"[bench] oracle cpu baseline on {nt} tensors")
        t0 = time.perf_counter()
        rplan = oracle.rescale_be.prepare_chain(ops, n, s)
        for t in range(nt):
            oracle.rescale_be.chain_tensor(X[t * n3:(t + 1) * n3], rplan)
        cdt = time.perf_counter() - t0
        cpu = dict(value=n3 * nt / cdt / 1e9, unit="GDoF/s", cores=1, kind="oracle",
                   sample=f"first {nt} of the {batch} tensors, whole chain, {cdt:.1f} s", cpu_model=cpu_model())
    log("[bench] accuracy against the exact chain")
    err, how = chain_accuracy(dY.cpu().numpy(), X, ops, n, args.chain_acc_tensors)
    accuracy = {"normwise_rel_err": err, "sample": how}
    info = dict(b=plan.b, g=list(plan.g))
    plan.close()
    h.close()
    return {
        "metric": ("tensor-mode chain GDoF/s (Y = X x1 A x2 B x3 C, OzII-RescaleBE persistent residues)"
                   if depth == 3 else
                   f"tensor-mode chain GDoF/s (depth {depth}: operator i along direction i mod 3, "
                   "OzII-RescaleBE persistent residues)"),
        "value": round(value, 3),
        "unit": "GDoF/s",
        "ms_per_step": round(dt / args.steps * 1e3, 3),
        "dtype": "i8",
        "config": {"workload": f"tensor_chain_rescale_be_n{n}_b{batch}_s{s}" + (f"_d{depth}" if depth != 3 else ""),
                   "n": n, "batch": batch, "s": s, "depth": depth,
                   "plan": info},
        "accuracy": accuracy,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


CHAIN_SIZES = (8, 12, 16, 32, 64, 128, 256)
CHAIN_SIZES_DOF = 1 << 24


def run_chain_sizes(args):
    """OzII-RescaleBE over tensor sides (the chain page's Sec. 6 throughput
    test, Fig. 7): depth 3, the directions in turn, U(-1, 1) tensors and
    operators, s = 15 unless --s, batch floor(2^24 / n^3) so that every chain
    processes about 2^24 entries.  8 < n <= 16 runs the LDS kernel (and the
    HBM kernels as well, for comparison), other n the HBM kernels.  Per
    side: GDoF/s over whole chains (encode to reconstruction), the phase
    times, the algorithmic vector-ALU rate (rbe_valu_ops_per_entry per real
    entry); for n <= 64 one tensor bit for bit against the oracle, for
    n <= 32 the normwise error of one tensor against the exact chain.  The
    line's value is all sides' entries over all sides' chain times."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import oracle
    import workloads

    s = int(args.s) if args.s else 15
    only = [int(x) for x in args.chain_sizes.split(",")] if args.chain_sizes else None
    sizes = [(n, "auto") for n in CHAIN_SIZES] + [(n, "hbm") for n in CHAIN_SIZES if 8 < n <= 16]
    if only:
        sizes = [(n, "auto") for n in only]
    h = oz2.Handle(torch.cuda.current_stream())
    h.set_timing(True)
    rows, tot_dof, tot_ms, parity_bad, parity_n = {}, 0, 0.0, 0, 0
    roofline = None
    for n, kern in sizes:
        batch = CHAIN_SIZES_DOF // n ** 3
        n3 = n ** 3
        log(f"[bench] chain_sizes: n={n} batch={batch} kernel={kern}")
        X = workloads.tensor_batch(n, batch, workloads.seed(8, n))
        ops = [workloads.real_matrix(n, n, workloads.seed(8, 1000 + 10 * n + q)) for q in range(3)]
        dX = torch.from_numpy(X).cuda()
        dY = torch.empty_like(dX)
        h.set_chain_kernel(kern)
        plan = h.chain_plan(ops, n, s)
        for _ in range(args.warmup):
            h.chain_rescale_be(plan, dX, dY, batch)
        torch.cuda.synchronize()
        ph, t0 = [], time.perf_counter()
        for _ in range(args.steps):
            h.chain_rescale_be(plan, dX, dY, batch)
            ph.append(h.phase_times())
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        phm = [float(x) for x in np.mean(np.array(ph), axis=0)]
        dof = n3 * batch
        lds = 8 < n <= 16 and kern == "auto"
        valu = float(rbe_valu_ops_per_entry(s, plan.g)) * dof / (sum(phm) * 1e-3) / 1e12
        row = dict(batch=batch, kernel="lds" if lds else "hbm", gdofs=round(dof / (ms * 1e-3) / 1e9, 3),
                   ms=round(ms, 4), b=plan.b, g=list(plan.g),
                   phases_ms=(dict(chain=round(phm[2], 4)) if lds else
                              dict(scan=round(phm[0], 4), encode=round(phm[1], 4), rescaling_products=round(phm[2], 4),
                                   last_product=round(phm[3], 4))),
                   valu_tops=round(valu, 2))
        if n <= 64:
            Y = dY[:n3].cpu().numpy()
            rplan = oracle.rescale_be.prepare_chain(ops, n, s)
            want = oracle.rescale_be.chain_tensor(X[:n3], rplan)
            bad = int(np.count_nonzero(Y.view(np.int64) != want.view(np.int64)))
            row["parity_first_tensor_not_bit_identical"] = bad
            parity_bad += bad
            parity_n += n3
        if n <= 32:
            row["normwise_rel_err"] = chain_accuracy(dY[:n3].cpu().numpy(), X, ops, n, 1)[0]
        rows[f"{n}" if kern == "auto" else f"{n}_{kern}"] = row
        if kern == "auto":
            tot_dof += dof
            tot_ms += ms
        if n == max(CHAIN_SIZES) and not lds:
            # the dominant kernel: the rescaling products (d - 1 launches,
            # timed together by the phase events on the library's stream)
            gr = list(plan.g)[:-1]
            per_launch = phm[2] / len(gr)
            ops_launch = np.mean([rbe_product_ops_per_entry(s, gi) for gi in gr]) * dof
            ach = ops_launch / (per_launch * 1e-3) / 1e12
            roofline = dict(kernel=f"chain_step_staged_kernel (OzII-RescaleBE product and rescaling, residues "
                                   f"in HBM), n = {n}",
                            bound="alu", achieved=round(ach, 2), peak=round(PEAK_VALU_TOPS, 2), unit="TOP/s",
                            frac=round(ach / PEAK_VALU_TOPS, 4), traffic=None, launch_ms=round(per_launch, 4),
                            ops_per_launch=float(ops_launch), ops_basis=RBE_OPS_BASIS)
        plan.close()
        del dX, dY
    h.set_chain_kernel("auto")
    h.close()
    value = tot_dof / (tot_ms * 1e-3) / 1e9
    return {
        "metric": "OzII-RescaleBE tensor-mode chain GDoF/s over tensor sides n = 8 .. 256 (about 2^24 entries per chain)",
        "value": round(value, 3),
        "unit": "GDoF/s",
        "ms_per_step": round(tot_ms, 3),
        "dtype": "i8",
        "config": {"workload": f"tensor_chain_rescale_be_sizes_dof2^24_s{s}_d3", "sizes": list(CHAIN_SIZES),
                   "dof_per_chain": CHAIN_SIZES_DOF, "s": s, "depth": 3, "dist": "uniform"},
        "per_shape": rows,
        "parity_sample": dict(entries=parity_n, not_bit_identical=parity_bad,
                              how="the first tensor of each side n <= 64 against the oracle"),
        "roofline": roofline,
    }


def oracle_chain(X, Aop, Bop, Cop, n, nt, s):
    """The three emulated modes of nt tensors with the oracle, as the library
    decomposes them (mode 1 over all nt tensors at once)."""
    import oracle
    n2, n3 = n * n, n ** 3
    z1 = oracle.gemm_entries(False, "N", "N", n, n2 * nt, n, 1.0, Aop, n, X[:n3 * nt], n, 0.0, None,
                             n, s, nthreads=oracle.max_threads())["out"]
    z2 = np.zeros(n3 * nt)
    for q in range(n * nt):
        z2[q * n2:(q + 1) * n2] = oracle.gemm_entries(False, "N", "T", n, n, n, 1.0, z1[q * n2:],
                                                      n, Bop, n, 0.0, None, n, s, nthreads=1)["out"]
    y = np.zeros(n3 * nt)
    for b in range(nt):
        y[b * n3:(b + 1) * n3] = oracle.gemm_entries(False, "N", "T", n2, n, n, 1.0, z2[b * n3:], n2,
                                                     Cop, n, 0.0, None, n2, s, nthreads=1)["out"]
    return y


def run_chain(args):
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads

    w = workloads.WORKLOADS[5]
    n, batch, s = w["n"], w["batch"], w["s"][0]
    n3 = n ** 3
    log(f"[bench] chain: generating {batch} tensors of {n}^3 (seeded)")
    X = workloads.tensor_batch(n, batch, workloads.seed(5, 0))
    ops = [workloads.real_matrix(n, n, workloads.seed(5, q)) for q in (1, 2, 3)]
    dX = torch.from_numpy(X).cuda()
    dops = [torch.from_numpy(o).cuda() for o in ops]
    dY = torch.empty_like(dX)
    work = torch.empty_like(dX)
    h = oz2.Handle(torch.cuda.current_stream())
    h.set_timing(True)
    launch_ms = []

    def step(record):
        h.tensor_mode_chain(dX, dops[0], dops[1], dops[2], n, batch, s, Y=dY, work=work)
        if record is not None:
            launch_ms.append(h.phase_times()[2])  # the last mode's fused launch

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(launch_ms)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / args.steps * 1e3
    dofs = float(n3 * batch)
    value = dofs / (dt / args.steps) / 1e9
    # the fused kernel reads each input entry and writes each output entry once
    lm = float(np.mean(launch_ms))
    bytes_per_launch = 16.0 * n3 * batch
    achieved = bytes_per_launch / (lm * 1e-3) / 1e9
    roofline = dict(kernel="small_gemm_kernel (fused short-k Ozaki II, mode 3)", bound="hbm",
                    achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic("chain", SMALL_TRAFFIC_FILE),
                    bytes_per_launch=bytes_per_launch, launch_ms=round(lm, 4))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nt = args.chain_cpu_tensors
        log(f"[bench] oracle cpu baseline on {nt} tensors")
        t0 = time.perf_counter()
        oracle_chain(X, ops[0], ops[1], ops[2], n, nt, s)
        cdt = time.perf_counter() - t0
        cpu = dict(value=n3 * nt / cdt / 1e9, unit="GDoF/s", cores=oracle.max_threads(), kind="oracle",
                   sample=f"first {nt} of the {batch} tensors, all three modes, {cdt:.1f} s", cpu_model=cpu_model())
    log("[bench] accuracy against the exact chain")
    err, how = chain_accuracy(dY.cpu().numpy(), X, ops, n, args.chain_acc_tensors)
    accuracy = {"normwise_rel_err": err, "sample": how}
    h.close()
    return {
        "metric": "tensor-mode chain GDoF/s (Y = X x1 A x2 B x3 C, per-mode Ozaki II)",
        "value": round(value, 3),
        "unit": "GDoF/s",
        "ms_per_step": round(ms_per_step, 3),
        "dtype": "i8",
        "config": {"workload": f"tensor_chain_n{n}_b{batch}_s{s}", "n": n, "batch": batch, "s": s,
                   "modes": 3, "emulated_tflops": round(3 * 2.0 * n * dofs / (dt / args.steps) / 1e12, 3)},
        "accuracy": accuracy,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


def run_datapower(args):
    """The headline product at s = 16 on four operand data sets with the
    same shapes and hence the same kernels, loads and instruction streams:
    all zeros, one constant, random integers and the headline's data.  The
    residue bytes are then all zero, constant per modulus, or random; the
    GEMM phase times (HIP events on the stream) show how much of the
    residue GEMM's rate depends on its operand data."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads
    n, s = 8192, 16
    h = oz2.Handle(torch.cuda.current_stream())
    h.set_timing(True)
    dC = torch.zeros(n * n, dtype=torch.float64, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(workloads.seed(2, 7))
    cases = [("zeros", torch.zeros(n * n, dtype=torch.float64, device="cuda")),
             ("constant 0.75", torch.full((n * n,), 0.75, dtype=torch.float64, device="cuda")),
             ("integers in [-2^15, 2^15)",
              torch.randint(-2 ** 15, 2 ** 15, (n * n,), device="cuda", generator=gen).double()),
             ("headline (u - 1/2) exp(0.5 g)",
              torch.from_numpy(workloads.real_matrix(n, n, workloads.seed(2, 0), "phi", 0.5)).cuda())]
    out = {}
    t_all = time.perf_counter()
    for name, X in cases:
        log(f"[bench] datapower: {name}")
        for _ in range(args.warmup):
            h.dgemm("N", "N", n, n, n, 1.0, X, n, X, n, 0.0, dC, n, s)
        torch.cuda.synchronize()
        g = []
        for _ in range(args.steps):
            h.dgemm("N", "N", n, n, n, 1.0, X, n, X, n, 0.0, dC, n, s)
            g.append(h.phase_times()[2])
        ms = float(np.median(g))
        out[name] = dict(gemm_ms=round(ms, 4), int8_tops=round(2.0 * n ** 3 * s / (ms * 1e-3) / 1e12, 1),
                         frac_of_peak=round(2.0 * n ** 3 * s / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4))
    dt = time.perf_counter() - t_all
    h.close()
    head = out[cases[-1][0]]
    return {
        "metric": "residue GEMM INT8 TOP/s on the headline product at s = 16, by operand data",
        "value": head["int8_tops"],
        "unit": "TOP/s",
        "ms_per_step": round(dt / (len(cases) * (args.steps + args.warmup)) * 1e3, 3),
        "dtype": "i8",
        "config": {"workload": "dgemm_8192_NN_s16_operand_data", "m": n, "n": n, "k": n, "s": s},
        "per_data": out,
    }


def gemm_block_terms(m, n, k, s, cplx=False):
    """The residue GEMM's time terms under the per-block model, for the tile
    the library launches: (waves, waves x k steps x passes) of the 256 x 256
    tile and of the 128 x 128 tile (one of the two pairs is zero).  A wave is
    one block per CU on 256 CUs (256 x 256), or four per CU (128 x 128);
    k runs of at most 130816 positions are separate launches."""
    pad = lambda x, q: (x + q - 1) // q * q
    mp, np_, kp = pad(m, 256), pad(n, 256), pad(k, 256)
    passes = 3 if cplx else 1
    big = [0.0, 0.0]
    small = [0.0, 0.0]
    for k0 in range(0, kp, 130816):
        steps = (min(kp, k0 + 130816) - k0) // 64
        nb256 = (mp // 256) * (np_ // 256) * s
        if nb256 >= 512 and steps * 64 > 512:
            w = -(-nb256 // 256)
            big[0] += w
            big[1] += w * steps * passes
        else:
            w = -(-((mp // 128) * (np_ // 128) * s) // 1024)
            small[0] += w
            small[1] += w * steps * passes
    return big + small


def model_terms(m, n, k, s):
    """Regressors of the performance model of one real N/N call (the Arc
    page's Sec. 9.2 model, re-derived for this design): the four GEMM block
    terms; the memory bytes, scan and encode (8 + 8 + s)(mk + kn) and
    reconstruct (s + 8) mn, the GEMM's own s mn written counted in its block
    time; and the launches (two fills, two scans, two encodes, one GEMM per
    k run, one reconstruct)."""
    runs = -(-((k + 255) // 256 * 256) // 130816)
    mem = (16.0 + s) * (m * k + k * n) + (s + 8.0) * m * n
    return gemm_block_terms(m, n, k, s) + [mem, 7.0 + runs]


def run_perfmodel(args):
    """Fit T = waves x (c0 + c1 k steps) [per tile kind] + bytes / beta + launches x tau
    to measured call times of square DGEMMs (N = 1024 .. 8192, s = 8, 16, 24:
    the grid of the Arc page's Table 17 and the headline's size) and check it
    on the held-out non-square shapes of Table 10 (s = 8, 16)."""
    import torch
    import complex_gemm_emulation_amd as oz2
    import workloads
    h = oz2.Handle(torch.cuda.current_stream())
    h.set_timing(True)

    def measure(m, n, k, s, A, B):
        dC = torch.zeros(m * n, dtype=torch.float64, device="cuda")
        for _ in range(2):
            h.dgemm("N", "N", m, n, k, 1.0, A, m, B, k, 0.0, dC, m, s)
        torch.cuda.synchronize()
        tot, ph = [], []
        for _ in range(max(3, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            h.dgemm("N", "N", m, n, k, 1.0, A, m, B, k, 0.0, dC, m, s)
            e1.record()
            torch.cuda.synchronize()
            tot.append(e0.elapsed_time(e1))
            ph.append(h.phase_times())
        return float(np.median(tot)), [float(x) for x in np.median(np.array(ph), axis=0)]

    fit_pts, test_pts = [], []
    for N in (1024, 2048, 3072, 4096, 8192):
        A = torch.from_numpy(workloads.real_matrix(N, N, workloads.seed(10, 0), "phi", 0.5)).cuda()
        B = torch.from_numpy(workloads.real_matrix(N, N, workloads.seed(10, 1), "phi", 0.5)).cuda()
        for s_ in (8, 16, 24):
            log(f"[bench] perfmodel: {N}^3, s = {s_}")
            t, ph = measure(N, N, N, s_, A, B)
            fit_pts.append(((N, N, N, s_), t, ph))
        del A, B
    W = workloads.NONSQUARE
    for q, (m, k, n) in enumerate(W["shapes"]):
        A = torch.from_numpy(workloads.real_matrix(m, k, workloads.nonsquare_seed(q, 0), W["dist"])).cuda()
        B = torch.from_numpy(workloads.real_matrix(k, n, workloads.nonsquare_seed(q, 1), W["dist"])).cuda()
        for s_ in W["s"]:
            log(f"[bench] perfmodel: {m} x {k} x {n}, s = {s_}")
            t, ph = measure(m, n, k, s_, A, B)
            test_pts.append(((m, n, k, s_), t, ph))
        del A, B
    h.close()
    X = np.array([model_terms(*p[0]) for p in fit_pts])
    y = np.array([p[1] for p in fit_pts])
    used = [j for j in range(X.shape[1]) if np.any(X[:, j])]
    coef = np.zeros(X.shape[1])
    coef[used] = np.linalg.lstsq(X[:, used] / y[:, None], np.ones(len(y)), rcond=None)[0]  # relative errors
    params = dict(c0_256_us=coef[0] * 1e3, c1_256_us=coef[1] * 1e3, c0_128_us=coef[2] * 1e3,
                  c1_128_us=coef[3] * 1e3, beta_mem_GBs=(1e-6 / coef[4]) if coef[4] > 0 else None,
                  tau_us=coef[5] * 1e3)

    def rows(pts):
        out = []
        for (m, n, k, s_), t, ph in pts:
            pred = float(np.dot(model_terms(m, n, k, s_), coef))
            out.append(dict(shape=f"{m}x{k}x{n}", s=s_, measured_ms=round(t, 4), model_ms=round(pred, 4),
                            deviation=round(pred / t - 1.0, 4),
                            phases_ms=dict(scan=round(ph[0], 4), encode=round(ph[1], 4), gemm=round(ph[2], 4),
                                           reconstruct=round(ph[3], 4))))
        return out
    fit_rows, test_rows = rows(fit_pts), rows(test_pts)
    worst = max(abs(r["deviation"]) for r in test_rows)
    return {
        "metric": "performance model: largest |model / measured - 1| on the held-out non-square shapes",
        "value": round(worst, 4),
        "unit": "relative deviation",
        "ms_per_step": None,
        "dtype": "i8",
        "config": {"workload": "dgemm_perf_model", "fit": "square N = 1024..8192, s = 8, 16, 24",
                   "check": "Table 10 non-square shapes, s = 8, 16"},
        "per_shape": {"params": {k_: (round(v, 4) if v is not None else None) for k_, v in params.items()},
                      "fit": fit_rows, "check": test_rows},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="dgemm8192",
                    choices=["dgemm8192", "wide4096", "zgemm4096", "chain", "chain_rbe", "chain_sizes", "nonsquare",
                             "reuse8192", "tiled8192", "datapower", "accuracy", "perfmodel"])
    ap.add_argument("--s", type=str, default="")
    ap.add_argument("--n", type=int, default=0)
    ap.add_argument("--cpu-side", type=int, default=0)
    ap.add_argument("--chain-cpu-tensors", type=int, default=256)
    ap.add_argument("--chain-rbe-cpu-tensors", type=int, default=384)
    ap.add_argument("--chain-acc-tensors", type=int, default=8)
    ap.add_argument("--chain-depth", type=int, default=3, help="chain_rbe: operators (3 = one pass)")
    ap.add_argument("--chain-sizes", type=str, default="", help="chain_sizes: only these sides (comma list)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip timing the HBM stream ceilings")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the emulated GEMM on one GPU (got --gpus {args.gpus}); "
              f"multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        log(f"[bench] calibration copy of {COPY_CAL_BYTES} bytes x 3")
        copy_calibration(torch)
    if args.workload == "chain":
        out = run_chain(args)
    elif args.workload == "chain_rbe":
        out = run_chain_rbe(args)
    elif args.workload == "chain_sizes":
        out = run_chain_sizes(args)
    elif args.workload == "nonsquare":
        out = run_nonsquare(args)
    elif args.workload == "datapower":
        out = run_datapower(args)
    elif args.workload == "accuracy":
        out = run_accuracy(args)
    elif args.workload == "perfmodel":
        out = run_perfmodel(args)
    else:
        out = run_gemm(args, args.workload)
    line = {"metric": out["metric"], "value": out["value"], "unit": out["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": out["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": out["dtype"],
            "data": "synthetic", "config": out["config"]}
    for key in ("step_ms", "per_s", "per_shape", "per_data", "hbm_ceiling", "tiling", "accuracy", "parity_sample",
                "roofline", "cpu_baseline"):
        if key in out:
            line[key] = out[key]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
