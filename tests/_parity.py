"""Shared helpers of the GPU parity tests (not collected by pytest).

Tolerances: indexer scores and top-k indices are compared bit for bit (the
inputs are integer-valued, so every score is exact); attention outputs, bf16
with fp32 accumulation, must be within max-abs 2e-2 and relative L2 5e-3 of
the fp64 oracle per (config, layer, step) tensor; lse within 1e-3 absolute.
"""
import numpy as np
import torch

MAX_ABS = 2e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def dev(t):
    return t.to("cuda", non_blocking=False)


def host(t):
    return t.detach().to("cpu")


def assert_scores_bitwise(S_gpu, S_ref, what=""):
    g = host(S_gpu).numpy()
    assert g.shape == S_ref.shape, what
    same = g.view(np.uint32) == S_ref.view(np.uint32)
    if not same.all():
        bad = np.argwhere(~same)[:5]
        raise AssertionError(f"{what}: {int((~same).sum())} score mismatches, first at "
                             f"{bad.tolist()}: gpu {g[tuple(bad[0])]} ref {S_ref[tuple(bad[0])]}")


def assert_idx_equal(idx_gpu, idx_ref, what=""):
    g = host(idx_gpu).numpy()
    assert g.shape == idx_ref.shape, what
    same = g == idx_ref
    if not same.all():
        rows = np.argwhere(~same.all(axis=-1))[:3]
        r = tuple(rows[0])
        raise AssertionError(f"{what}: {len(np.argwhere(~same.all(axis=-1)))} rows differ; row {r}: "
                             f"gpu {g[r][:12]} ref {idx_ref[r][:12]}")


def attn_errors(out_gpu, ref):
    g = host(out_gpu).double().numpy()
    d = g - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_attn_close(out_gpu, ref, what=""):
    max_abs, rel = attn_errors(out_gpu, ref)
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs {max_abs:.3g} rel_l2 {rel:.3g}"


def assert_lse_close(lse_gpu, ref, what=""):
    g = host(lse_gpu).double().numpy()
    assert g.shape == ref.shape, what
    both_inf = np.isneginf(g) & np.isneginf(ref)
    # -inf on one side only is a mismatch; the difference is taken only where
    # neither value is -inf (so no inf - inf is formed)
    one_inf = (np.isneginf(g) | np.isneginf(ref)) & ~both_inf
    assert not one_inf.any(), f"{what}: lse -inf on one side at {np.argwhere(one_inf)[:3].tolist()}"
    fin = ~both_inf
    d = np.abs(g[fin] - ref[fin])
    assert np.all(np.isfinite(d)) and d.max(initial=0.0) <= LSE_ABS, f"{what}: lse err {d.max(initial=0.0)}"


# Guard canaries: an output tensor is placed between two pads of a known byte
# pattern, and after the kernel has run both pads must still hold it, so a
# write past either end of the tensor fails the test.  The pads keep the
# tensor 256-byte aligned.
GUARD_BYTES = 4096
GUARD_FILL = 0xA5


class Guarded:
    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((n + 2 * GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device="cuda")
        self.tensor = self.buf[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)

    def check(self, what=""):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        lo, hi = b[:GUARD_BYTES], b[GUARD_BYTES + self.n:]
        bad_lo = np.flatnonzero(lo != GUARD_FILL)
        bad_hi = np.flatnonzero(hi != GUARD_FILL)
        assert bad_lo.size == 0, f"{what}: {bad_lo.size} guard bytes before the output overwritten"
        assert bad_hi.size == 0, f"{what}: {bad_hi.size} guard bytes after the output overwritten"


def guarded(shape, dtype):
    """(tensor, guard): a device tensor of shape/dtype between two canary pads."""
    g = Guarded(shape, dtype)
    return g.tensor, g
