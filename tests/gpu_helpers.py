"""Helpers shared by the GPU parity tests: run a synthetic workload through
the HIP library (via the C ABI binding) and bring its codes back to the CPU,
and the oracle-side dequantization / attention on those same codes."""

import json
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import quantized_attention_fa_amd as faq
from oracle import attention as OA
from oracle import formats as F
from oracle import quantize as OQ
from synth import make_inputs

DEV = "cuda:0"

MODE_CFG = {
    "int8_head": lambda spec, br: faq.QConfig("int8", "per_head"),
    "fp8_token": lambda spec, br: faq.QConfig("fp8_e4m3", "per_token"),
    "mxfp4": lambda spec, br: faq.QConfig("mxfp4", "per_block"),
    "rot_fp8_block": lambda spec, br: faq.QConfig(
        "fp8_e4m3", "per_token_block", block_tokens=spec["q_block"] if br == 0 else spec["kv_block"]),
    "fp8_head": lambda spec, br: faq.QConfig("fp8_e4m3", "per_head"),
    "int8_token": lambda spec, br: faq.QConfig("int8", "per_token"),
    "mxfp8": lambda spec, br: faq.QConfig("mxfp8", "per_block"),
    "fp8_block128": lambda spec, br: faq.QConfig("fp8_e4m3", "per_token_block", block_tokens=128),
    "fp8_block256": lambda spec, br: faq.QConfig("fp8_e4m3", "per_token_block", block_tokens=256),
}
P_RULE = {"int8_head": "int8", "fp8_token": "fp8", "mxfp4": "mxfp4", "rot_fp8_block": "fp8",
          "fp8_head": "fp8", "int8_token": "int8", "mxfp8": "mxfp8", "fp8_block128": "fp8", "fp8_block256": "fp8"}
STATIC_DTYPE = {"int8_head": "int8", "fp8_head": "fp8_e4m3"}


class GpuRun:
    """Quantized Q/K/V of one workload produced by the HIP path.  `modes`
    gives each branch's mode (default: the workload's per-branch modes, else
    its mode for all three); "float" leaves a branch unquantized (bf16)."""

    def __init__(self, w, keep_rotated=False, modes=None):
        self.w = w
        mode = w.spec["mode"]
        self.mode = mode
        # explicit modes, else the workload's own per-branch modes, else its mode for all three
        self.modes = list(modes) if modes is not None else list(w.spec.get("modes", [mode] * 3))
        self.x = [t.to(DEV) for t in (w.q, w.k, w.v)]
        self.static = [None, None, None]
        self.amax = [None, None, None]
        for br in range(3):
            if self.modes[br] in STATIC_DTYPE:
                amax = torch.zeros(w.shape[1], dtype=torch.float32, device=DEV)
                # the workload's calibration batch, else the tensor itself
                for c in (w.calib[br] if w.calib else [self.x[br]]):
                    faq.fa_quant_calibrate(c.to(DEV), amax)
                self.amax[br] = amax
                self.static[br] = faq.fa_quant_scales_from_amax(amax, STATIC_DTYPE[self.modes[br]])
        self.rot = w.rot.to(DEV) if w.rot is not None else None
        self.rotated = [None, None, None]
        self.qt = []
        for br in range(3):
            m = self.modes[br]
            if m == "float":
                self.qt.append(faq.float_branch(self.x[br]))
                continue
            cfg = MODE_CFG[m](w.spec, br)
            rot = self.rot if (self.rot is not None and br < 2 and m == "rot_fp8_block") else None
            dbg = None
            if rot is not None and keep_rotated:
                dbg = torch.empty_like(self.x[br])
                self.rotated[br] = dbg
            self.qt.append(faq.fa_quantize(self.x[br], cfg, static_scale=self.static[br], rot=rot,
                                           debug_rotated=dbg))
        torch.cuda.synchronize()

    def codes_np(self, br):
        return self.qt[br].codes.cpu().numpy()

    def scales_np(self, br):
        return self.qt[br].scales.cpu().numpy()

    def attention(self, out_dtype=torch.float32, causal=None, sm_scale=0.0):
        causal = self.w.spec["causal"] if causal is None else causal
        o = faq.fa_quant_attention(self.qt[0], self.qt[1], self.qt[2], sm_scale=sm_scale, causal=causal,
                                   out_dtype=out_dtype)
        torch.cuda.synchronize()
        return o


def dequant(run: GpuRun, br: int):
    """(values fp64 [B,H,S,D], per-key scale [B,H,S] or None) of branch br,
    decoded by the oracle from the GPU's codes and scales."""
    mode = run.modes[br]
    B, H, S, D = run.x[br].shape  # Q may have its own length (decode)
    if mode == "float":
        return run.x[br].to(torch.float64).cpu().numpy(), None
    c, s = run.codes_np(br), run.scales_np(br)
    if mode == "int8_head":
        return OQ.dequantize_per_head(c, s), np.broadcast_to(s.reshape(1, H, 1), (B, H, S))
    if mode == "fp8_head":
        return OQ.dequantize_per_head(c, s, F.e4m3_decode), np.broadcast_to(s.reshape(1, H, 1), (B, H, S))
    if mode == "fp8_token":
        s = s.reshape(B, H, S)
        return OQ.dequantize_per_token(c, s, F.e4m3_decode), s
    if mode == "int8_token":
        s = s.reshape(B, H, S)
        return OQ.dequantize_per_token(c, s, lambda a: a.astype(np.float64)), s
    if mode == "mxfp4":
        return OQ.dequantize_mxfp4(c, s), None
    if mode == "mxfp8":
        return OQ.dequantize_mxfp8(c, s), None
    bt = run.qt[br].cfg.block_tokens
    st = OQ.block_scales_per_token(s.reshape(B, H, -1), bt, S)
    return OQ.dequantize_per_token(c, st, F.e4m3_decode), st


def _oracle_threads():
    """Worker threads for the oracle (numpy releases the GIL in its array
    operations): the host's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_pool_map(fn, items):
    """map over a thread pool of _oracle_threads() workers, with the BLAS
    library held to one thread meanwhile: one multithreaded BLAS call per
    worker would run workers x cores threads (measured 12x slower)."""
    with threadpool_limits(1), ThreadPoolExecutor(_oracle_threads()) as ex:
        return list(ex.map(fn, items))


def oracle_attention(run: GpuRun, rows=None, causal=None, sm_scale=None):
    """The oracle on the GPU run's codes, one (b, h) head per task on a
    thread pool; returns (O, T, n_tie) as oracle.attention does."""
    causal = run.w.spec["causal"] if causal is None else causal
    q, _ = dequant(run, 0)
    k, _ = dequant(run, 1)
    v, vs = dequant(run, 2)
    rule = "bf16" if run.modes[2] == "float" else P_RULE[run.modes[2]]
    B, H = q.shape[:2]

    def one(bh):
        b, h = divmod(bh, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        return OA.attention(q[sl], k[sl], v[sl], rule, v_scale=None if vs is None else vs[sl], causal=causal,
                            rows=rows, allowance=True, sm_scale=sm_scale)

    parts = oracle_pool_map(one, range(B * H))
    R = parts[0][0].shape[2]
    D = q.shape[3]
    o = np.concatenate([p[0] for p in parts], axis=0).reshape(B, H, R, D)
    T = np.concatenate([p[1] for p in parts], axis=0).reshape(B, H, R, D)
    return o, T, sum(p[2] for p in parts)


def _parity_log(rec):
    """Append one parity record (JSON line) to gpurun_out/parity.jsonl."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    d = os.path.join(root, "gpurun_out")
    try:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "parity.jsonl"), "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass


def check_attention(gpu_out: np.ndarray, ref, label=""):
    """Parity bar: relative Frobenius <= 1e-3 and |err| <= 2e-3 + T (tie
    allowance) element by element.  Elements above 2e-3 may only be ones
    the allowance covers: the query rows holding them number at most the
    probability elements near a rounding boundary, and they are at most 1 %
    of the output.  The counts go to the parity log."""
    o, T, n_tie = ref
    g64 = gpu_out.astype(np.float64)
    err = np.abs(g64 - o)
    rel = float(np.linalg.norm(g64 - o) / max(np.linalg.norm(o), 1e-300))
    over = err > 2e-3
    n_over = int(over.sum())
    n_over_rows = int(over.any(axis=-1).sum()) if err.size else 0
    excess = float((err - 2e-3).max()) if err.size else 0.0
    rec = {"case": label, "t": round(time.time(), 1), "outputs": int(err.size), "rel_frobenius": rel,
           "max_abs": float(err.max()) if err.size else 0.0, "tie_p_elements": int(n_tie),
           "outputs_with_T": int((T > 0).sum()), "outputs_over_2e-3": n_over, "rows_over_2e-3": n_over_rows,
           "max_excess_over_2e-3": max(excess, 0.0)}
    _parity_log(rec)
    assert not np.isnan(gpu_out).any(), f"{label}: NaN in output"
    assert rel <= 1e-3, f"{label}: relative Frobenius {rel:.3e} > 1e-3"
    viol = err > 2e-3 + T
    assert not viol.any(), (f"{label}: {int(viol.sum())} elements over 2e-3 + T; max err {err.max():.3e}, "
                            f"worst excess {(err - 2e-3 - T).max():.3e}; tie elements {n_tie}")
    assert n_over_rows <= n_tie and n_over <= 0.01 * err.size, (
        f"{label}: {n_over} elements in {n_over_rows} rows over 2e-3 (tie elements {n_tie}, "
        f"outputs {err.size})")
    return rel, float(err.max()), n_tie


def bf16_of(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def small_workload(cfg, shape, q_len=None):
    return make_inputs(cfg, shape=shape, calib_batch=2, q_len=q_len)
