"""Shared helpers for the GPU parity tests (host <-> device, comparisons)."""
import numpy as np

# Acceptance bars: bf16 inputs with fp32 accumulation against the fp64 oracle.
ATOL_OUT_BF16 = 2e-2      # outputs (A, A_local, merged out)
ATOL_LSE_BF16 = 1e-2      # log-normalizers (alpha, a, lambda, merged lse)
REL_L2_BF16 = 1e-2        # stricter internal check on read-outs: ||err|| / ||ref||
ATOL_F32 = 1e-4           # fp32 inputs


def dev(x, device="cuda"):
    """numpy float32 / uint16 (bf16 bits) -> torch tensor on the GPU."""
    import torch
    x = np.ascontiguousarray(x)
    t = torch.from_numpy(x)
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def report(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(got - ref))
    mx = float(np.max(diff)) if diff.size else 0.0
    fin = np.isfinite(ref)
    with np.errstate(invalid="ignore"):
        num = float(np.linalg.norm(np.where(fin, got - ref, 0.0)))
    den = float(np.linalg.norm(np.where(fin, ref, 0.0)))
    rel = num / den if den > 0 else num
    print("  %-28s max|err| = %.3e   rel-L2 = %.3e" % (name, mx, rel), flush=True)
    return mx, rel


def check(name, got, ref, atol, rel=None):
    mx, r = report(name, got, ref)
    assert mx <= atol, "%s: max abs err %.3e > %.1e" % (name, mx, atol)
    if rel is not None:
        assert r <= rel, "%s: rel-L2 err %.3e > %.1e" % (name, r, rel)
