"""Comparison helpers for GPU-vs-oracle parity (no method arithmetic here).

Tolerances (rel-L2 = ||x - ref|| / ||ref||):
  * fp32 inputs:  1e-4
  * bf16 inputs with fp32 accumulation: 2e-2
Ratio-normalised outputs are checked in three parts, because den_t is a sum
that changes sign and num_t / den_t amplifies rounding without bound where
|den_t| is small compared with its natural scale |q_t| |u_t|
(u_t = S_t m_t - h_t, so den_t = q_t . u_t):
  (i)   num, rel-L2 over all tokens (from a normalize=0 run),
  (ii)  den, rel-L2 over all tokens (from den_out),
  (iii) the division, on EVERY token, through the conditioning-normalised error
          e_t = |o_t - o*_t| |den*_t| / (|num*_t| + |o*_t| |q_t| |u*_t|)
        (* = oracle).  If num and den carry errors of at most eps_n |num*| and
        eps_d |q| |u*|, then e_t <= max(eps_n, eps_d) to first order, and for a
        well-conditioned token (|den*| ~ |q| |u*|) e_t is about half the relative
        error of o_t.  Asserted, as an aggregate like the rel-L2 tolerances:
        RMS_t e_t <= tol / 2 over all tokens (max_t e_t is reported).
  (iv)  on the benchmark workloads, also the rel-L2 of o over the tokens with
        |den*_t| >= 1e-2 |q_t| |u*_t| (the excluded fraction is reported).  On
        arbitrary shapes this subset check is only reported: with bf16 operands
        it sits at 1.3-2.6e-2 in a CPU emulation of the kernel's rounding points,
        i.e. at the tolerance itself, because the few tokens just above the
        cut-off dominate it.
"""
from __future__ import annotations

import json
import os

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
COND = 1e-2            # conditioning threshold of the ratio check


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (nr if nr > 0 else 1.0))


def tol_for(dtype_name: str) -> float:
    return TOL_F32 if dtype_name in ("f32", "float32") else TOL_BF16


def well_conditioned(den_ref, unorm_ref, q):
    qn = np.linalg.norm(np.asarray(q, dtype=np.float64), axis=-1)
    return np.abs(den_ref) >= COND * qn * unorm_ref


def ratio_report(o_gpu, den_gpu, num_ref, den_ref, unorm_ref, q):
    """den rel-L2 (all tokens), e_t statistics (all tokens), and the reported
    rel-L2 of o over the well-conditioned tokens."""
    q = np.asarray(q, dtype=np.float64)
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    well = well_conditioned(den_ref, unorm_ref, q)
    with np.errstate(divide="ignore", invalid="ignore"):
        o_ref = num_ref / den_ref[..., None]
        e = (np.linalg.norm(o_gpu - o_ref, axis=-1) * np.abs(den_ref)
             / (np.linalg.norm(num_ref, axis=-1) + np.linalg.norm(o_ref, axis=-1) * np.linalg.norm(q, axis=-1)
                * unorm_ref))
    e = np.where(np.isfinite(e), e, np.inf)
    return {
        "den": rel_l2(den_gpu, den_ref),
        "e_max": float(e.max()),
        "e_rms": float(np.sqrt(np.mean(e ** 2))),
        "ratio_well": rel_l2(o_gpu[well], o_ref[well]),
        "excluded": float(1.0 - well.mean()),
    }


def ratio_ok(rep, tol, subset=False) -> bool:
    ok = rep["e_rms"] <= tol / 2
    if subset:
        ok = ok and rep["ratio_well"] <= tol
    return ok


def per_row_rel_l2(x, ref, axes):
    """rel-L2 of every leading index, reducing over `axes` (e.g. per head)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    nr = np.sqrt(np.sum(ref ** 2, axis=axes))
    return num / np.where(nr > 0, nr, 1.0)


def segment_bounds(n: int, nseg: int, lead_chunks: int, seg_chunks: int, kc: int = 64):
    """Token ranges [t0, t1) of the segments of a forward plan (segment 0 holds lead_chunks
    chunks of kc tokens, every later one seg_chunks, the last possibly fewer)."""
    out, t0 = [], 0
    for s in range(nseg):
        c = lead_chunks if s == 0 else seg_chunks
        t1 = min(n, t0 + c * kc)
        out.append((t0, t1))
        t0 = t1
    assert t0 == n, (n, nseg, lead_chunks, seg_chunks)
    return out


# Parity figures of the workload-size tests, written at the end of the session to
# $HLA2_PARITY_DIR (parity_workloads.json and .md) when that variable is set.
RECORDS: dict = {}


def record(name: str, **figures):
    RECORDS[name] = figures


def write_records(path_dir: str):
    if not RECORDS:
        return
    os.makedirs(path_dir, exist_ok=True)
    with open(os.path.join(path_dir, "parity_workloads.json"), "w") as f:
        json.dump(RECORDS, f, indent=1, sort_keys=True)
    keys = ["heads", "tokens", "num", "num_head_max", "num_seg_max", "den", "den_head_max", "den_seg_max",
            "e_rms", "e_rms_head_max", "e_rms_well_head_max", "e_max", "ratio_well", "ratio_well_head_max",
            "excluded", "state", "state_head_max"]
    lines = ["| test | " + " | ".join(keys) + " |", "|---|" + "---|" * len(keys)]

    def fmt(x):
        if x is None:
            return "-"
        if isinstance(x, (int, np.integer)):
            return str(int(x))
        return "%.3g" % x
    for name in sorted(RECORDS):
        r = RECORDS[name]
        lines.append("| %s | " % name + " | ".join(fmt(r.get(k)) for k in keys) + " |")
    with open(os.path.join(path_dir, "parity_workloads.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def ratio_per_head(o_gpu, num_ref, den_ref, unorm_ref, q, head_axes=2):
    """Per-head figures of the ratio criterion: e_rms and e_max over each head's tokens, and the
    rel-L2 of o over each head's well-conditioned tokens (shape: the leading head axes)."""
    q = np.asarray(q, dtype=np.float64)
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    well = well_conditioned(den_ref, unorm_ref, q)
    with np.errstate(divide="ignore", invalid="ignore"):
        o_ref = num_ref / den_ref[..., None]
        e = (np.linalg.norm(o_gpu - o_ref, axis=-1) * np.abs(den_ref)
             / (np.linalg.norm(num_ref, axis=-1) + np.linalg.norm(o_ref, axis=-1) * np.linalg.norm(q, axis=-1)
                * unorm_ref))
    e = np.where(np.isfinite(e), e, np.inf)
    tok_axes = tuple(range(head_axes, e.ndim))
    e_rms = np.sqrt(np.mean(e ** 2, axis=tok_axes))
    e_max = np.max(e, axis=tok_axes)
    # over the well-conditioned tokens only: there e_t is bounded by the relative errors of num and
    # den; where |den*_t| is as small as den's own rounding error it is not, and one such token
    # among 65536 can carry a head's RMS
    cnt = np.maximum(np.sum(well, axis=tok_axes), 1)
    e_rms_well = np.sqrt(np.sum(np.where(well, e, 0.0) ** 2, axis=tok_axes) / cnt)
    diff = np.where(well[..., None], o_gpu - o_ref, 0.0)
    ref = np.where(well[..., None], o_ref, 0.0)
    all_axes = tuple(range(head_axes, diff.ndim))
    nr = np.sqrt(np.sum(ref ** 2, axis=all_axes))
    well_head = np.sqrt(np.sum(diff ** 2, axis=all_axes)) / np.where(nr > 0, nr, 1.0)
    return {"e_rms": e_rms, "e_max": e_max, "e_rms_well": e_rms_well, "ratio_well": well_head,
            "excluded": 1.0 - np.mean(well, axis=tok_axes)}


def ratio_workload_figures(o_gpu, den_gpu, num_gpu, num_ref, den_ref, unorm_ref, q):
    """Every head of a normalised call: num and den rel-L2 overall and per head, and the ratio
    criterion overall and per head.  Returns (figures, message)."""
    num_head = per_row_rel_l2(num_gpu, num_ref, (-2, -1))
    den_head = per_row_rel_l2(den_gpu, den_ref, (-1,))
    rep = ratio_report(o_gpu, den_gpu, num_ref, den_ref, unorm_ref, q)
    ph = ratio_per_head(o_gpu, num_ref, den_ref, unorm_ref, q)
    fig = {"heads": int(np.prod(num_head.shape)), "tokens": int(num_ref.shape[-2]),
           "num": rel_l2(num_gpu, num_ref), "num_head_max": float(num_head.max()),
           "den": rep["den"], "den_head_max": float(den_head.max()),
           "e_rms": rep["e_rms"], "e_rms_head_max": float(ph["e_rms"].max()),
           "e_rms_well_head_max": float(ph["e_rms_well"].max()), "e_max": rep["e_max"],
           "ratio_well": rep["ratio_well"], "ratio_well_head_max": float(ph["ratio_well"].max()),
           "excluded": rep["excluded"]}
    msg = ("num %.3g (head max %.3g) den %.3g (head max %.3g) | e_rms %.3g (head max %.3g) | ratio(well) %.3g "
           "(head max %.3g) excluded %.3f" % (fig["num"], fig["num_head_max"], fig["den"], fig["den_head_max"],
                                              fig["e_rms"], fig["e_rms_head_max"], fig["ratio_well"],
                                              fig["ratio_well_head_max"], fig["excluded"]))
    return fig, msg


def ratio_workload_ok(fig, tol) -> bool:
    """num and den of every head within tol; e_t's RMS over all tokens within tol/2 and, per head, over
    its well-conditioned tokens; the rel-L2 of o over the well-conditioned tokens of the call within tol
    (the per-head figure is reported: a head's few tokens just above the conditioning cut-off carry
    their relative error of up to e_t / 1e-2 into it)."""
    return (fig["num_head_max"] <= tol and fig["den_head_max"] <= tol and fig["e_rms"] <= tol / 2
            and fig["e_rms_well_head_max"] <= tol / 2 and fig["ratio_well"] <= tol)
