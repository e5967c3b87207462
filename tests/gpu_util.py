"""Helpers shared by the GPU parity tests: error metrics, tolerances and
oracle comparisons, head by head.

Every comparison prints its margins; with FA_PARITY_RECORD=<path> in the
environment each one is also appended to that file as a JSON line (test,
case, tensor, max-abs and its bar, relative RMS, representation floor), so
that one GPU run leaves a complete table of margins.
"""

import concurrent.futures
import json
import math
import os

import numpy as np
import torch

import oracle.attention as orc

# Tolerances on O (and dQ, dK, dV): fp32 max-abs 1e-5; half precision
# max-abs 2e-2 and relative RMS 5e-3. LSE (fp32 for every dtype) is held to
# 1e-4 absolute: its error comes from fp32 score accumulation and fp32
# exp2/log2/sum over at most 2^17 keys (relative ~1e-6 .. 1e-5 on values of
# order 10), independent of the dtype.
TOL = {
    "fp32": dict(max_abs=1e-5, rel_rms=None),
    "bf16": dict(max_abs=2e-2, rel_rms=5e-3),
    "fp16": dict(max_abs=2e-2, rel_rms=5e-3),
}
LSE_TOL = 1e-4
# The half-precision max-abs bar is only widened where rounding the exact
# result to the dtype alone costs more than half of it (bf16 outputs of
# magnitude >= 4, whose half-ulp is 2^-6): there a correct fp32 value one
# rounding step away lands a whole ulp from the exact result, so the bar
# becomes 2e-2 plus that ulp (twice the floor).
FLOOR_WIDEN_AT = 1e-2

TORCH_DTYPE = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}

# Host threads for the oracle: one head per thread, BLAS single-threaded
# (numpy releases the interpreter lock inside its array loops).
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def to64(t):
    return t.detach().to(torch.float32).cpu().to(torch.float64).numpy()


def errors(x, ref):
    d = x - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    den = math.sqrt(float(np.mean(ref * ref))) if d.size else 1.0
    rel_rms = math.sqrt(float(np.mean(d * d))) / den if den > 0 else float(np.abs(d).max())
    return max_abs, rel_rms


def rep_floor(ref, dtype):
    """max |cast(ref) - ref|: what rounding the exact result to dtype costs."""
    if dtype == "fp32" or ref.size == 0:
        return 0.0
    t = torch.from_numpy(np.ascontiguousarray(ref)).to(TORCH_DTYPE[dtype]).to(torch.float64)
    return float(np.abs(t.numpy() - ref).max())


def max_abs_bar(dtype, floor, strict=False):
    """The max-abs bar; strict (the named workloads) never widens."""
    bar = TOL[dtype]["max_abs"]
    if not strict and dtype != "fp32" and floor > FLOOR_WIDEN_AT:
        bar += 2 * floor
    return bar


def record(entry):
    path = os.environ.get("FA_PARITY_RECORD")
    if not path:
        return
    entry = dict(entry, test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0])
    with open(path, "a") as f:
        f.write(json.dumps(entry) + "\n")


def _judge(name, max_abs, rel_rms, floor, dtype, finite, heads=None, strict=False):
    tol = TOL[dtype]
    bar = max_abs_bar(dtype, floor, strict)
    widened = bar != tol["max_abs"]
    msg = (f"{name}: max_abs={max_abs:.3e} (tol {bar:.2e}{', widened' if widened else ''}) "
           f"rel_rms={rel_rms:.3e} (tol {tol['rel_rms']}) floor={floor:.3e}"
           + (f" heads={heads}" if heads is not None else ""))
    print(msg, flush=True)
    record(dict(case=name, dtype=dtype, max_abs=max_abs, max_abs_bar=bar, rel_rms=rel_rms,
                rel_rms_bar=tol["rel_rms"], floor=floor, heads=heads, strict=strict))
    assert finite, name + ": non-finite values"
    assert max_abs <= bar, msg
    if tol["rel_rms"] is not None:
        assert rel_rms <= tol["rel_rms"], msg
    return max_abs, rel_rms


def assert_close(name, x, ref, dtype, strict=False):
    """Element-wise comparison with the oracle: fp32 max-abs 1e-5; half
    precision max-abs 2e-2 (widened only as FLOOR_WIDEN_AT says, never when
    strict) and relative RMS 5e-3 over the whole tensor."""
    max_abs, rel_rms = errors(x, ref)
    return _judge(name, max_abs, rel_rms, rep_floor(ref, dtype), dtype,
                  bool(np.all(np.isfinite(x))), strict=strict)


def assert_lse_close(name, x, ref):
    err = float(np.abs(x - ref).max()) if x.size else 0.0
    print(f"{name}: lse max_abs={err:.3e} (tol {LSE_TOL:.0e})", flush=True)
    record(dict(case=name + " LSE", dtype="fp32", max_abs=err, max_abs_bar=LSE_TOL))
    assert np.all(np.isfinite(x)), name + ": non-finite LSE"
    assert err <= LSE_TOL, f"{name}: lse max_abs {err:.3e} > {LSE_TOL}"


def pick(t, heads):
    """The selected (b, h) slices of a [B, H, ...] tensor as fp64 [1, n, ...]."""
    return to64(torch.stack([t[b, h] for b, h in heads]))[None]


def oracle_forward(q, k, v, scale, causal, heads):
    q64, k64, v64 = (pick(t, heads) for t in (q, k, v))
    return orc.attention_forward(q64, k64, v64, scale, causal)


def oracle_backward(q, k, v, do, scale, causal, heads):
    q64, k64, v64, g64 = (pick(t, heads) for t in (q, k, v, do))
    return orc.attention_backward(q64, k64, v64, g64, scale, causal)


def all_heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


class _Acc:
    """Running max-abs, squared sums and floor of one output over heads."""

    def __init__(self):
        self.max_abs = 0.0
        self.ss_d = 0.0
        self.ss_r = 0.0
        self.n = 0
        self.floor = 0.0
        self.finite = True
        self.worst = None

    def add(self, head, got, ref, dtype):
        d = got - ref
        m = float(np.abs(d).max()) if d.size else 0.0
        if m > self.max_abs or self.worst is None:
            self.max_abs = max(self.max_abs, m)
            self.worst = head
        self.ss_d += float(np.sum(d * d))
        self.ss_r += float(np.sum(ref * ref))
        self.n += d.size
        self.floor = max(self.floor, rep_floor(ref, dtype))
        self.finite = self.finite and bool(np.all(np.isfinite(got)))

    def rel_rms(self):
        return math.sqrt(self.ss_d / self.ss_r) if self.ss_r > 0 else math.sqrt(self.ss_d)


def compare_heads(name, inputs, oracle_fn, outputs, dtype, heads, lse=None, pass_head=False,
                  strict=False):
    """Compare GPU results with the oracle on every listed (b, h), in parallel.

    inputs: GPU tensors [B, H, N, D] handed to the oracle as fp64 [1, 1, N, D];
    oracle_fn(*head_inputs) returns the reference tuple; outputs: list of
    (tag, GPU tensor [B, H, N, D], index into that tuple); lse: optional
    (GPU tensor [B, H, N], index). Max-abs is over every compared element and
    the relative RMS over the whole set of compared heads. With pass_head
    the oracle also receives head=(b, h); strict keeps the fixed bars.
    Returns the per-output (max_abs, rel_rms).
    """
    cpu_in = [t.detach().cpu() for t in inputs]
    cpu_out = [(tag, t.detach().cpu(), i) for tag, t, i in outputs]
    cpu_lse = (lse[0].detach().cpu(), lse[1]) if lse is not None else None

    def f64(t, b, h):
        return t[b:b + 1, h:h + 1].to(torch.float64).numpy()

    def one(bh):
        b, h = bh
        args = [f64(t, b, h) for t in cpu_in]
        ref = oracle_fn(*args, head=bh) if pass_head else oracle_fn(*args)
        res = []
        for tag, t, i in cpu_out:
            got = f64(t, b, h)
            acc = _Acc()
            acc.add(bh, got, ref[i], dtype)
            res.append(acc)
        lerr = None
        if cpu_lse is not None:
            got = cpu_lse[0][b:b + 1, h:h + 1].to(torch.float64).numpy()
            r = ref[cpu_lse[1]]
            lerr = (float(np.abs(got - r).max()), bool(np.all(np.isfinite(got))))
        return bh, res, lerr

    import threadpoolctl
    totals = [_Acc() for _ in cpu_out]
    lse_max, lse_finite = 0.0, True
    with threadpoolctl.threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=WORKERS) as ex:
            for bh, res, lerr in ex.map(one, heads):
                for tot, acc in zip(totals, res):
                    if acc.max_abs >= tot.max_abs:
                        tot.worst = bh
                    tot.max_abs = max(tot.max_abs, acc.max_abs)
                    tot.ss_d += acc.ss_d
                    tot.ss_r += acc.ss_r
                    tot.n += acc.n
                    tot.floor = max(tot.floor, acc.floor)
                    tot.finite = tot.finite and acc.finite
                if lerr is not None:
                    lse_max = max(lse_max, lerr[0])
                    lse_finite = lse_finite and lerr[1]
    out = {}
    for (tag, _, _), tot in zip(cpu_out, totals):
        _judge(f"{name} {tag}", tot.max_abs, tot.rel_rms(), tot.floor, dtype, tot.finite,
               heads=len(heads), strict=strict)
        out[tag] = (tot.max_abs, tot.rel_rms())
    if lse is not None:
        print(f"{name}: lse max_abs={lse_max:.3e} (tol {LSE_TOL:.0e}) heads={len(heads)}",
              flush=True)
        record(dict(case=name + " LSE", dtype="fp32", max_abs=lse_max, max_abs_bar=LSE_TOL,
                    heads=len(heads)))
        assert lse_finite, name + ": non-finite LSE"
        assert lse_max <= LSE_TOL, f"{name}: lse max_abs {lse_max:.3e} > {LSE_TOL}"
    return out


def forward_oracle(scale, causal):
    return lambda q, k, v: orc.attention_forward(q, k, v, scale, causal)


def backward_oracle(scale, causal):
    return lambda q, k, v, do: orc.attention_backward(q, k, v, do, scale, causal)
