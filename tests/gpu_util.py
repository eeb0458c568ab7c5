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


def check_argmax_margin(am, z, margin):
    """am [n] (the GPU's argmax) against the oracle's logits z [n][V]: positions whose
    top logit leads the runner-up by more than `margin` must agree exactly (lowest index
    on ties); elsewhere the GPU's pick must be within `margin` of the maximum.  Returns
    (fraction of positions with a clear maximum, fraction that agree exactly)."""
    from oracle import gpt_oracle as O
    am = np.asarray(am).reshape(-1)
    top2 = np.partition(z, -2, axis=-1)[:, -2:]
    lead = top2[:, 1] - top2[:, 0]
    unique = lead > margin
    ref = O.argmax_lowest(z)
    np.testing.assert_array_equal(am[unique], ref[unique])
    picked = np.take_along_axis(z, am[:, None].astype(np.int64), -1)[:, 0]
    assert np.all(picked >= z.max(axis=-1) - margin)
    return float(unique.mean()), float(np.mean(am == ref))


def check_argmax_on_gpu_logits(am, z_gpu, z_ref):
    """The argmax is integer work on the step's own logits: am must equal the lowest-index
    argmax of z_gpu [n][V] exactly.  Against the oracle's logits z_ref the pick must be
    consistent with the logits' own difference: with d = max_j |z_gpu - z_ref| on a row,
    z_ref[am] >= max z_ref - 2 d (it cannot be further below the oracle's maximum than
    the two rows disagree).  Returns (agreement with the oracle's argmax, largest d)."""
    from oracle import gpt_oracle as O
    am = np.asarray(am).reshape(-1)
    np.testing.assert_array_equal(am, O.argmax_lowest(z_gpu))
    dz = np.max(np.abs(z_gpu - z_ref), axis=-1)
    picked = np.take_along_axis(z_ref, am[:, None].astype(np.int64), -1)[:, 0]
    assert np.all(picked >= z_ref.max(axis=-1) - 2 * dz - 1e-6)
    return float(np.mean(am == O.argmax_lowest(z_ref))), float(dz.max())
