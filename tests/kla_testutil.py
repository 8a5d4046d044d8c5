"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and
measuring the relative L2 error against the fp64 oracle."""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}   # relative L2 bars for fp32 and bf16 inputs


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(x, dtype_name=None, device="cuda:0"):
    """numpy fp32 -> torch on the GPU; q/k/v in the workload dtype (exact: values are representable)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype_name is not None:
        t = t.to(torch_dtype(dtype_name))
    return t.to(device)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def report(name, **errs):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


def host32(t):
    """A device tensor on the host as fp32 (exact for bf16 and fp32 values)."""
    return t.float().cpu().numpy()


def heads_of(x, heads, time_axis=1):
    """[B, T, H, ...] (time_axis 1) or [steps, B, H, ...] (time_axis 0) -> [n, T, ...] for the listed heads."""
    if time_axis == 1:
        return np.stack([x[b, :, h] for b, h in heads])
    return np.stack([x[:, b, h] for b, h in heads])


def states_of(x, heads):
    """[B, H, dk, dv] -> [n, dk, dv] for the listed heads."""
    return np.stack([x[b, h] for b, h in heads])
