"""Input marshalling for the oracle (test infrastructure only)."""
import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact widening of a torch tensor or array (bf16, fp32, fp64) to float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def as_int(x, dtype=np.int64) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").numpy().astype(dtype)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x).astype(dtype)
