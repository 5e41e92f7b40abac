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


def unblock16(t, rows: int):
    """Row-major [rows, K] view of a matrix in the 16-row blocked layout (blocks
    of 16 rows x 32 columns stored contiguously, a row group's blocks in column
    order); works on torch tensors and NumPy arrays."""
    r16 = (rows + 15) // 16 * 16
    K = t.shape[1]
    b = t[:r16].reshape(r16 // 16, K // 32, 16, 32)
    b = b.permute(0, 2, 1, 3) if hasattr(b, "permute") else b.transpose(0, 2, 1, 3)
    return b.reshape(r16, K)[:rows]
