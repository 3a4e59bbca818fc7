"""Helpers shared by the GPU parity tests: device upload of synthetic inputs, readback,
and the error measures the tolerances are stated in."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from synthetic_inputs import WEIGHT_NAMES, host_array, round_to

DEV = "cuda"
TORCH = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
# unit roundoff of each storage format (half an ulp at 1.0)
UNIT = {"fp32": 2.0 ** -24, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    """Name the case before a GPU step, so a fault's last output says what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 array exactly representable in ``dtype`` -> contiguous device tensor."""
    h = host_array(np.ascontiguousarray(a64), dtype)
    if dtype == "bf16":
        return torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(h).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def rnd(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_to(a, dtype)


def dev_layer(w: dict, dtype: str) -> dict:
    return {k: to_dev(w[k], dtype) for k in WEIGHT_NAMES}


def dev_lens(lens) -> torch.Tensor | None:
    if lens is None:
        return None
    return torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)


def err_report(g: np.ndarray, o: np.ndarray) -> dict:
    d = np.abs(g - o)
    return dict(max_abs=float(d.max()), max_rel1=float((d / np.maximum(np.abs(o), 1.0)).max()),
                rms_ref=float(np.sqrt((o ** 2).mean())))


def assert_within(g: np.ndarray, o: np.ndarray, atol: float, rtol: float, what: str) -> dict:
    """|g - o| <= atol + rtol |o| elementwise."""
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    d = np.abs(g - o)
    lim = atol + rtol * np.abs(o)
    bad = d > lim
    rep = err_report(g, o)
    if bad.any():
        idx = np.unravel_index(np.argmax(d - lim), d.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {d.size} outside atol={atol} rtol={rtol}; "
                             f"worst at {idx}: gpu={g[idx]!r} ref={o[idx]!r}; {rep}")
    return rep
