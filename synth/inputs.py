"""Seeded synthetic Q/K/V workloads.

Each generator is numpy PCG64 ``default_rng([config, tensor_id])`` with
tensor ids Q/K/V = 0/1/2, calibration batches 10/11/12, outlier channel sets
20/21/22 and the rotation matrix 30.  Values are drawn in float32 (float64
for Student-t) and, for bf16 workloads, rounded to bf16 by torch's CPU cast
(round to nearest even).  This module holds no quantization or attention
arithmetic: it only produces inputs.

Workloads (BNSD shapes):
  1  INT8 per-head static, tiny: fp32 N(0,1) [1,2,128,64]; calibrated on the
     same tensors; non-causal.
  2  INT8 per-head static, LLM prefill: bf16 N(0,1) [2,32,4096,128] with
     round(0.005*H*D) (head, channel) pairs scaled x20; per-branch
     calibration batch [4,32,4096,128] from its own seed with the same
     outlier set; causal.
  3  FP8 per-token, video-DiT shape: bf16 z*exp(0.5 g), z ~ N(0,1) per
     element and g ~ N(0,1) per token row (log-normal row magnitude),
     [1,40,32760,128]; non-causal.
  4  MXFP4 per-block, image-edit shape: bf16 Student-t(4) [1,24,8192,128];
     non-causal.
  5  Rotate + FP8 block: bf16 N(0,1) [2,24,16384,128] with round(0.01*H*D)
     (head, channel) pairs x30; one seeded orthogonal R (QR of a Gaussian,
     signs fixed by diag(R_qr)) in bf16 used as both q_rot and k_rot;
     Q block 128, K/V block 256; non-causal.
The sibling modes of the FA mode list run on the recipe and shape of the
workload of their own family:
  6  FP8 per-head static: as 2 (calibration batch, outliers, causal).
  7  INT8 per-token dynamic: as 3 (log-normal row magnitudes).
  8  MXFP8 per-block dynamic: as 4 (Student-t(4)).
Per-branch configurations (an unconfigured branch is not quantized):
  9  FP8 per-token Q and K, V unquantized (bf16): as 3.
  10 no branch quantized (bf16 attention): as 2, without outliers' effect on
     any scale (the tensors are the same recipe).
Decode over a quantized KV cache (a few queries per head against a long
cache; Q has q_len rows, K and V the shape's S):
  11 INT8 per-head static: the recipe of 2, [4,32,16384,128] cache, 16
     queries per head, not causal.
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

CONFIGS: Dict[int, dict] = {
    1: dict(name="int8_per_head_tiny", mode="int8_head", dtype="f32", dist="normal",
            shape=(1, 2, 128, 64), causal=False, calib="self"),
    2: dict(name="int8_per_head_prefill", mode="int8_head", dtype="bf16", dist="normal",
            shape=(2, 32, 4096, 128), causal=True, calib="batch",
            calib_batch=4, outlier_frac=0.005, outlier_gain=20.0),
    3: dict(name="fp8_per_token_video_dit", mode="fp8_token", dtype="bf16", dist="lognormal_rows",
            shape=(1, 40, 32760, 128), causal=False),
    4: dict(name="mxfp4_per_block_image_edit", mode="mxfp4", dtype="bf16", dist="t4",
            shape=(1, 24, 8192, 128), causal=False),
    5: dict(name="rotate_fp8_block", mode="rot_fp8_block", dtype="bf16", dist="normal",
            shape=(2, 24, 16384, 128), causal=False, outlier_frac=0.01,
            outlier_gain=30.0, q_block=128, kv_block=256),
    6: dict(name="fp8_per_head_prefill", mode="fp8_head", dtype="bf16", dist="normal",
            shape=(2, 32, 4096, 128), causal=True, calib="batch",
            calib_batch=4, outlier_frac=0.005, outlier_gain=20.0),
    7: dict(name="int8_per_token_video_dit", mode="int8_token", dtype="bf16", dist="lognormal_rows",
            shape=(1, 40, 32760, 128), causal=False),
    8: dict(name="mxfp8_per_block_image_edit", mode="mxfp8", dtype="bf16", dist="t4",
            shape=(1, 24, 8192, 128), causal=False),
    9: dict(name="fp8_qk_bf16_v_video_dit", mode="fp8_token", dtype="bf16", dist="lognormal_rows",
            shape=(1, 40, 32760, 128), causal=False, modes=("fp8_token", "fp8_token", "float")),
    10: dict(name="bf16_attention_prefill", mode="float", dtype="bf16", dist="normal",
             shape=(2, 32, 4096, 128), causal=True, outlier_frac=0.005, outlier_gain=20.0,
             modes=("float", "float", "float")),
    11: dict(name="int8_per_head_decode", mode="int8_head", dtype="bf16", dist="normal",
             shape=(4, 32, 16384, 128), q_len=16, causal=False, calib="batch", calib_batch=4,
             outlier_frac=0.005, outlier_gain=20.0),
}

TID_Q, TID_K, TID_V = 0, 1, 2
TID_CALIB = 10
TID_OUTLIER = 20
TID_ROT = 30


def rng(cfg: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([cfg, tid])


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def outlier_pairs(cfg: int, branch: int, H: int, D: int, frac: float) -> np.ndarray:
    n = int(round(frac * H * D))
    idx = rng(cfg, TID_OUTLIER + branch).choice(H * D, size=n, replace=False)
    return np.stack([idx // D, idx % D], axis=1)


def _draw(cfg: int, tid: int, shape, spec: dict, branch: int) -> np.ndarray:
    g = rng(cfg, tid)
    dist = spec["dist"]
    if dist == "t4":
        x = g.standard_t(4.0, size=shape).astype(np.float32)
    elif dist == "lognormal_rows":
        z = g.standard_normal(shape, dtype=np.float32)
        lg = g.standard_normal(shape[:3], dtype=np.float32)
        x = z * np.exp(np.float32(0.5) * lg)[..., None]
    else:
        x = g.standard_normal(shape, dtype=np.float32)
    if "outlier_frac" in spec:
        H, D = shape[1], shape[3]
        for h, d in outlier_pairs(cfg, branch, H, D, spec["outlier_frac"]):
            x[:, h, :, d] *= np.float32(spec["outlier_gain"])
    return x


def rotation(cfg: int, D: int) -> torch.Tensor:
    g = rng(cfg, TID_ROT)
    a = g.standard_normal((D, D))
    qm, rm = np.linalg.qr(a)
    r = qm * np.sign(np.diag(rm))[None, :]
    return _to_bf16(r.astype(np.float32))


@dataclass
class Workload:
    cfg: int
    spec: dict
    shape: Tuple[int, int, int, int]
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    calib: List[List[torch.Tensor]] = field(default_factory=list)  # per branch
    rot: Optional[torch.Tensor] = None

    @staticmethod
    def np32(t: torch.Tensor) -> np.ndarray:
        """float32 numpy copy holding the tensor's values exactly."""
        return t.to(torch.float32).numpy()


def make_inputs(cfg: int, shape=None, calib_batch=None, q_len=None) -> Workload:
    """CPU tensors for workload `cfg` (1..11).  `shape` overrides the BNSD
    shape with the same recipe (smaller test cases); `calib_batch` overrides
    the calibration batch size of workloads with a calibration batch;
    `q_len` gives Q its own sequence length (decode), else the workload's
    q_len or the shape's S."""
    spec = dict(CONFIGS[cfg])
    shape = tuple(shape or spec["shape"])
    q_len = q_len or spec.get("q_len")
    if q_len:
        spec["q_len"] = q_len
    bf16 = spec["dtype"] == "bf16"

    def mk(tid, shp, branch):
        x = _draw(cfg, tid, shp, spec, branch)
        return _to_bf16(x) if bf16 else torch.from_numpy(x)

    qshape = (shape[0], shape[1], q_len, shape[3]) if q_len else shape
    q, k, v = mk(TID_Q, qshape, 0), mk(TID_K, shape, 1), mk(TID_V, shape, 2)
    w = Workload(cfg=cfg, spec=spec, shape=shape, q=q, k=k, v=v)
    if spec.get("calib") == "self":
        w.calib = [[q], [k], [v]]
    elif spec.get("calib") == "batch":
        nb = calib_batch or spec["calib_batch"]
        w.calib = [[mk(TID_CALIB + br, (nb,) + (qshape if br == 0 else shape)[1:], br)] for br in range(3)]
    if spec["mode"] == "rot_fp8_block":
        w.rot = rotation(cfg, shape[3])
    return w


def sample_rows(cfg: int, S: int, n: int, edge: int = 128) -> np.ndarray:
    """Seeded sorted sample of query rows: the first and last `edge` rows
    plus n random others."""
    g = np.random.default_rng([cfg, 99])
    base = set(range(min(edge, S))) | set(range(max(0, S - edge), S))
    rest = np.setdiff1d(np.arange(S), np.fromiter(base, dtype=np.int64))
    extra = g.choice(rest, size=min(n, rest.size), replace=False) if rest.size else []
    return np.array(sorted(base | set(int(x) for x in extra)), dtype=np.int64)
