"""Helpers shared by the GPU tests: bf16 rounding on the host, error metrics."""
import numpy as np
import torch


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and back, on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().float().numpy()


def to_dev(x: np.ndarray, dtype: str):
    """numpy float array -> device tensor of the activation type ('bf16' or 'fp32')."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.bfloat16()
    return t.cuda()


def from_dev(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def random_extras(params, cfg, seed):
    """Move the extras' tensors off their start values (which leave the extras inert),
    as training would: S and the value-embedding gate weights G by 0.3 N(0, 1) per
    entry, the value-embedding tables to 0.5 N(0, 1) (the size of v's entries)."""
    if cfg.get("extras", 0) & 15:
        from gpt_pretraining_step_train_amd import inputs
        rng = np.random.default_rng(seed + 1000)
        for i, (name, shape) in enumerate(inputs.tensor_shapes(cfg)):
            if name in ("S", "G"):
                params[i] = (params[i] + 0.3 * rng.standard_normal(shape)).astype(np.float32)
            elif name.endswith(".VE"):
                params[i] = (0.5 * rng.standard_normal(shape)).astype(np.float32)
    return params


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def say(*a):
    print(*a, flush=True)
