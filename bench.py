#!/usr/bin/env python3
"""Throughput of the fused D3Q19 BGK step on one MI355X, with its HBM roofline.

    python bench.py [--steps K] [--warmup W] [--workload porous256] [--scheme aa] [--layout compact]

A "step" is one lattice time step: one fused collide-and-stream kernel over
the whole box (alternating the even and odd kernels of the in-place pattern).
Default workload: 256^3 periodic porous medium (overlapping spheres,
r ~ U(6, 12), 2400 spheres -> porosity ~0.61), tau = 0.65, body force 1e-6
along +x, fp32, one-lattice AA scheme, fluid-compacted SoA layout (populations of
fluid cells only).  Inputs are resident in HBM
before timing starts.  Prints ONE JSON line.

value = MLUPS over all cells (cells x steps / seconds / 1e6) over the K timed
steps.  The timed region is cut into `reps` equal segments (10 by default,
each an even number of steps) with HIP events between them; `reps_mlups`
gives the median, minimum and maximum over the segments (the PortLBM page's
Results section reports the median of 10 runs with their range).
roofline: the dominant kernel's algorithmic bytes per launch (152 B per fluid
cell for fp32, 304 B for fp64, + 1 B per cell for the mask) over its mean
launch time from HIP events on the launch stream, against 8 TB/s; also
against the measured ceilings of two probe kernels (libprobes.so): a float4
copy and the 19-plane in-place swap of the AA even step without arithmetic.
cpu_baseline: the fp64 CPU oracle, single-threaded, on three steps of the same
box; also the 32^3 seeded case in full (100 steps).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "MLUPS (million lattice updates/s) and % of HBM roofline, D3Q19 fp32, 1 GPU"


def workload(name):
    import numpy as np
    import lbm_inputs as li
    if name == "porous256":
        mask, ns = li.porous_mask(256)
        return dict(shape=(256, 256, 256), periodic=(1, 1, 1), tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask,
                    rho=None, u=None, precision="f32", extra={"n_spheres": ns})
    if name == "porous256_300":
        # the porous recipe taken literally: 300 spheres in the 256^3 box
        # (porosity ~0.94; the headline box scales the count to keep ~0.6)
        mask, ns = li.porous_mask(256, n_spheres=300)
        return dict(shape=(256, 256, 256), periodic=(1, 1, 1), tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask,
                    rho=None, u=None, precision="f32", extra={"n_spheres": ns})
    if name == "porous256_f64":
        # the same medium in double precision (304 B per fluid-cell update)
        mask, ns = li.porous_mask(256)
        return dict(shape=(256, 256, 256), periodic=(1, 1, 1), tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask,
                    rho=None, u=None, precision="f64", extra={"n_spheres": ns})
    if name == "porous512":
        mask, ns = li.porous_mask(512)
        return dict(shape=(512, 512, 512), periodic=(1, 1, 1), tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask,
                    rho=None, u=None, precision="f32", extra={"n_spheres": ns})
    if name == "random32":
        # the small seeded case: 32^3 periodic, tau 0.8, random fields (launch-bound)
        rho, u = li.random_fields(32, 32, 32, seed=1)
        return dict(shape=(32, 32, 32), periodic=(1, 1, 1), tau=0.8, force=(0.0, 0.0, 0.0), mask=None,
                    rho=rho.astype(np.float32), u=u.astype(np.float32), precision="f32", extra={})
    if name == "tgv128":
        rho, u = li.taylor_green(128, u0=0.04)
        return dict(shape=(128, 128, 128), periodic=(1, 1, 1), tau=0.6, force=(0.0, 0.0, 0.0), mask=None,
                    rho=rho, u=u, precision="f32", extra={})
    if name == "sphere128":
        return dict(shape=(128, 128, 128), periodic=(1, 1, 1), tau=0.7, force=(1e-6, 0.0, 0.0),
                    mask=li.sphere_mask(128, radius=16), rho=None, u=None, precision="f32", extra={})
    if name == "channel_f64":
        return dict(shape=(64, 64, 256), periodic=(1, 0, 1), tau=0.9, force=(0.0, 0.0, 1e-6), mask=None,
                    rho=None, u=None, precision="f64", extra={})
    if name == "karman":
        # open channel along x, PortLBM's boundary set: an equilibrium
        # (Dirichlet) inlet at rho 1, u 0.05 along x on -x, a Zou-He pressure
        # outlet at rho 1 on +x, walls in y, periodic z; a cylinder of radius
        # 20 a quarter-cell off the centre line, Re = u D / nu = 100 (tau 0.56)
        nx, ny, nz = 768, 192, 96
        u_in = (0.05, 0.0, 0.0)
        return dict(shape=(nx, ny, nz), periodic=(0, 0, 1), tau=0.56, force=(0.0, 0.0, 0.0),
                    mask=li.cylinder_mask(nx, ny, nz, 2 * 160, 2 * 96 + 1, 20), rho=None,
                    u=np.tile(np.array(u_in, np.float32)[:, None], (1, nx * ny * nz)), precision="f32",
                    open_faces={"-x": (1.0, u_in), "+x": (1.0, (0.0, 0.0, 0.0), "zou_he_pressure")}, extra={})
    if name == "periodic256_mask0":
        import numpy as np
        return dict(shape=(256, 256, 256), periodic=(1, 1, 1), tau=0.65, force=(1e-6, 0.0, 0.0),
                    mask=np.zeros(256 ** 3, np.uint8), rho=None, u=None, precision="f32", extra={})
    if name == "periodic256":
        return dict(shape=(256, 256, 256), periodic=(1, 1, 1), tau=0.65, force=(0.0, 0.0, 0.0), mask=None,
                    rho=None, u=None, precision="f32", extra={})
    raise SystemExit(f"unknown workload {name}")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lattice_boltzmann_cfd_d3q19_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".hpp", ".cpp")) and fn != "probes.hip":
            h.update(fn.encode())
            h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(name, scheme, layout, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{scheme}_{layout}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != kernel_source_hash():
        return None
    key = f"bytes_per_launch_{kernel}"
    return float(vals[key]) if key in vals else None


def state_check(rho, u, mask=None):
    """(finite, bounded) for moments rho[N], u[3][N] (numpy or torch): every
    fluid value finite, and every fluid cell with rho > 0 and |u| below the
    lattice speed 1 (a run past that bound has gone unstable)."""
    import numpy as np
    rho = rho.detach().cpu().numpy() if hasattr(rho, "detach") else np.asarray(rho)
    u = u.detach().cpu().numpy() if hasattr(u, "detach") else np.asarray(u)
    rho, u = rho.reshape(-1).astype(np.float64), u.reshape(3, -1).astype(np.float64)
    if mask is not None:
        fluid = np.asarray(mask).reshape(-1) == 0
        rho, u = rho[fluid], u[:, fluid]
    finite = bool(np.isfinite(rho).all() and np.isfinite(u).all())
    with np.errstate(invalid="ignore", over="ignore"):
        bounded = finite and bool((rho > 0).all() and (np.sqrt((u * u).sum(axis=0)) < 1.0).all())
    return finite, bounded


def _oracle_mlups(wl, steps):
    import oracle
    box = oracle.Box(*wl["shape"], periodic=wl["periodic"], tau=wl["tau"], force=wl["force"],
                     open_faces=wl.get("open_faces"))
    f = oracle.init_equilibrium(box, wl["mask"], wl["rho"], wl["u"])
    t0 = time.perf_counter()
    f = oracle.run(box, f, steps, wl["mask"])
    dt = time.perf_counter() - t0
    del f
    return box.n * steps / dt / 1e6, dt


def cpu_baseline(wl, steps=3):
    """Time the single-threaded fp64 oracle on a few steps of the same box,
    and on the 32^3 seeded case in full."""
    value, dt = _oracle_mlups(wl, steps)
    c1, dt1 = _oracle_mlups(workload("random32"), 100)
    return {"value": round(value, 3), "unit": "MLUPS", "cores": 1, "kind": "oracle",
            "sample": f"{steps} steps of the full {'x'.join(map(str, wl['shape']))} box, fp64, "
                      f"single thread, {dt:.1f} s",
            "c1_32cubed_100_steps": {"value": round(c1, 3), "unit": "MLUPS", "seconds": round(dt1, 2)},
            "host_cpu": _cpu_model(), "host_threads": os.cpu_count()}


def _cpu_model():
    """Model name as /proc/cpuinfo gives it, with family, model and stepping
    (a virtualised host may print only the vendor's series name)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                info.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    extra = [f"{info['cpu MHz']} MHz"] if "cpu MHz" in info else []
    extra += [f"cache {info['cache size']}"] if "cache size" in info else []
    return f"{name} ({', '.join(ids + extra)})" if ids or extra else name


def probe_ceilings(n_cells, reps=20):
    """Bandwidth (GB/s, bytes read + written) of the two probe kernels on the
    launch stream: a float4 copy of 1 GiB (the best of plain and nontemporal
    accesses with 1, 2, 4 or 8 elements per work-item) and the 19-plane
    in-place swap over n_cells cells (the better of plain and nontemporal),
    each also with its workgroups per CU capped at 4, 3 and 2; and the swap in
    64-cell blocks of 19 planes (the compact layout's store)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "lattice_boltzmann_cfd_d3q19_amd", "libprobes.so"))
    lib.probe_copy_f4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_size_t, ctypes.c_void_p]
    lib.probe_swap19.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_size_t, ctypes.c_void_p]
    lib.probe_swap19_blocked.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_size_t,
                                         ctypes.c_void_p]
    # workgroups per CU: all that fit, or 4, 3, 2 (reserved, unused LDS; the
    # step kernels cap theirs the same way)
    caps = [0] + [2 * 160 * 1024 // (2 * w + 1) for w in (4, 3, 2)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn, nbytes):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed: hip error {rc}")

    out = {}
    src = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    n4 = src.numel() // 4
    out["copy_float4_GBps"] = max(
        timed(lambda nt=nt, per=per, lds=lds: check(lib.probe_copy_f4(src.data_ptr(), dst.data_ptr(), n4, nt, per,
                                                                      lds, sp)), 2 * n4 * 16)
        for nt in (0, 1) for per in (1, 2, 4, 8) for lds in caps)
    del src, dst
    stride = (n_cells + 63) // 64 * 64
    buf = torch.zeros(19 * stride, dtype=torch.float32, device="cuda")
    out["swap19_inplace_GBps"] = max(
        timed(lambda nt=nt, lds=lds: check(lib.probe_swap19(buf.data_ptr(), stride, n_cells, nt, 1, lds, sp)),
              2 * 19 * 4 * n_cells)
        for nt in (0, 1) for lds in caps)
    # the same pattern with 2 and 4 cells per work-item (8- and 16-byte
    # accesses per plane), over the largest multiple of 4 cells
    n4c = n_cells // 4 * 4
    for per in (2, 4):
        out[f"swap19_{per}cells_GBps"] = max(
            timed(lambda nt=nt, per=per, lds=lds: check(lib.probe_swap19(buf.data_ptr(), stride, n4c, nt, per, lds,
                                                                         sp)), 2 * 19 * 4 * n4c)
            for nt in (0, 1) for lds in caps)
    # the same swap in the compact layout's store (64-cell blocks, each with
    # its 19 planes side by side)
    out["swap19_blocked_GBps"] = max(
        timed(lambda nt=nt, lds=lds: check(lib.probe_swap19_blocked(buf.data_ptr(), n_cells, nt, lds, sp)),
              2 * 19 * 4 * n_cells)
        for nt in (0, 1) for lds in caps)
    del buf
    out["swap19_cells"] = n_cells
    return {k: (round(v, 1) if isinstance(v, float) else v) for k, v in out.items()}


def segments(steps, want=10):
    """Largest r <= want that cuts `steps` into r equal even segments."""
    for r in range(min(want, steps // 2), 0, -1):
        if steps % r == 0 and (steps // r) % 2 == 0:
            return r
    return 1


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="porous256")
    ap.add_argument("--scheme", default="aa", choices=["aa", "ab", "eso", "twist"])
    ap.add_argument("--layout", default="compact", choices=["stream", "bundle", "collision", "compact"])
    ap.add_argument("--per-kernel-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=10, help="segments of the timed region (median, min, max)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the probe-kernel ceilings (profiling runs): their keys are then absent")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.steps < 2 or args.steps % 2:
        raise SystemExit("--steps must be even and >= 2 (the in-place scheme alternates two kernels)")

    import numpy as np
    import torch
    from lattice_boltzmann_cfd_d3q19_amd import Lattice

    wl = workload(args.workload)
    shape = wl["shape"]
    n = shape[0] * shape[1] * shape[2]
    mask = wl["mask"]
    n_fluid = n if mask is None else int(n - np.count_nonzero(mask))
    prec = wl["precision"]
    esize = 4 if prec == "f32" else 8

    lat = Lattice(*shape, precision=prec, layout=args.layout, scheme=args.scheme, tau=wl["tau"],
                  force=wl["force"])
    lat.set_geometry(None if mask is None else torch.from_numpy(mask), wl["periodic"])
    if wl.get("open_faces"):
        lat.set_open_faces(wl["open_faces"])
    lat.init(None if wl["rho"] is None else torch.from_numpy(wl["rho"]),
             None if wl["u"] is None else torch.from_numpy(wl["u"]))
    stream = lat.stream

    # warm-up
    lat.step(args.warmup if args.warmup % 2 == 0 else args.warmup + 1)
    torch.cuda.synchronize()

    # timed region: exactly K steps, in `reps` equal segments between HIP
    # events on the launch stream
    reps = segments(args.steps, args.reps)
    seg = args.steps // reps
    evs_t = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs_t[0].record(stream)
    for r in range(reps):
        lat.step(seg)
        evs_t[r + 1].record(stream)
    torch.cuda.synchronize()
    seg_ms = [evs_t[r].elapsed_time(evs_t[r + 1]) for r in range(reps)]
    ms_total = evs_t[0].elapsed_time(evs_t[reps])
    sec = ms_total / 1e3
    mlups = n * args.steps / sec / 1e6
    seg_mlups = sorted(n * seg / (m / 1e3) / 1e6 for m in seg_ms)

    # per-kernel launch durations (events around single steps on the launch stream)
    per = {}
    if args.scheme == "aa":
        names = ["aa_even", "aa_odd"]
    elif args.scheme == "eso":
        names = ["eso_even", "eso_odd"]
    elif args.scheme == "twist":
        names = ["twist_even", "twist_odd"]
    else:
        names = ["ab", "ab"]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.per_kernel_steps)]
    for i in range(args.per_kernel_steps):
        evs[i][0].record(stream)
        lat.step(1)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t_parity = lat.t - args.per_kernel_steps
    for i, (a, b) in enumerate(evs):
        per.setdefault(names[(t_parity + i) % 2], []).append(a.elapsed_time(b))
    per_ms = {k: float(np.mean(v)) for k, v in per.items()}
    dominant = max(per_ms, key=per_ms.get)
    alg_bytes = 2 * 19 * esize * n_fluid + (n if mask is not None else 0)
    achieved = alg_bytes / (per_ms[dominant] / 1e3) / 1e9
    step_gbps = alg_bytes * args.steps / sec / 1e9

    traffic = read_traffic(args.workload, args.scheme, args.layout, dominant)

    # state sanity after the run: finite, and below the lattice speed
    rho, u = lat.moments()
    torch.cuda.synchronize()
    finite, bounded = state_check(rho, u, mask)
    del rho, u

    # measured ceilings: the probe kernels
    ceilings = None if args.no_probes else probe_ceilings(n_fluid)

    # plain copy reference (torch copy kernel, 2 GiB moved)
    src = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    # one plain streaming kernel of known size for the HBM counters: reads
    # 1 GiB, writes 1 GiB (torch's elementwise negation)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del src, dst

    out = {
        "metric": METRIC,
        "value": round(mlups, 1),
        "unit": "MLUPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}_{args.scheme}_{args.layout}_{prec}",
                   "box": list(shape), "scheme": args.scheme, "layout": args.layout, "tau": wl["tau"],
                   "force": list(wl["force"]), "periodic": list(wl["periodic"]),
                   "porosity": round(n_fluid / n, 4), **wl["extra"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "traffic_over_alg": None if traffic is None else round(traffic / alg_bytes, 4),
                     "kernel": dominant, "alg_bytes_per_launch": alg_bytes,
                     "kernel_ms": {k: round(v, 5) for k, v in per_ms.items()},
                     **({} if ceilings is None else {
                         "frac_of_copy_float4": round(achieved / ceilings["copy_float4_GBps"], 4),
                         "frac_of_swap19": round(achieved / ceilings["swap19_inplace_GBps"], 4),
                         "frac_of_swap19_blocked": round(achieved / ceilings["swap19_blocked_GBps"], 4)})},
        "reps": reps,
        "steps_per_rep": seg,
        "reps_mlups": {"median": round(float(np.median(seg_mlups)), 1), "min": round(seg_mlups[0], 1),
                       "max": round(seg_mlups[-1], 1)},
        "mflups": round(n_fluid * args.steps / sec / 1e6, 1),
        "step_hbm_frac": round(step_gbps / PEAK_HBM_GBPS, 4),
        **({} if ceilings is None else {
            "step_frac_of_copy_float4": round(step_gbps / ceilings["copy_float4_GBps"], 4), **ceilings}),
        "copy_GBps": round(copy_gbps, 1),
        "state_finite": finite,
        "state_bounded": bounded,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
