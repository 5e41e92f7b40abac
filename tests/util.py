"""Helpers shared by the tests (no method arithmetic here)."""
import numpy as np
import torch


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))


def f64(t) -> np.ndarray:
    """Exact float64 image of a host/device tensor (bf16 and fp32 upcast exactly)."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def i64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.int64).numpy()


def weights_f64(wd: dict, g: int):
    """float64 (w13, w2) of expert g from a weight dict (bf16/f32 values or fp8 codes + scales)."""
    from oracle import dequant_blockwise
    if wd.get("s13") is None:
        return f64(wd["w13"][g]), f64(wd["w2"][g])
    return (dequant_blockwise(wd["w13"][g].cpu().numpy(), wd["s13"][g].cpu().numpy()),
            dequant_blockwise(wd["w2"][g].cpu().numpy(), wd["s2"][g].cpu().numpy()))


def flush(msg: str):
    print(msg, flush=True)
