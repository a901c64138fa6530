"""Helpers shared by the GPU parity tests."""
import numpy as np
import pytest
import torch

from oracle import MaskMod, ScoreMod

TOL_OUT = {"bf16": 2e-2, "f32": 1e-5}
TOL_LSE = 1e-3
# (what, out max-abs, lse max-abs) of every parity check of the session; the
# session summary (conftest) prints the full-size ones and the worst case
PARITY_LOG = []


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def oracle_mods(w, doc_id=None):
    return (MaskMod(w.mask, window=w.window, sinks=w.sinks, doc_id=doc_id, clauses=w.clauses),
            ScoreMod(w.score, cap=w.cap, alibi_m=w.alibi_m))


def block_mask_arrays(bm):
    """The four device BlockMask tensors as numpy int32 arrays."""
    return {k: getattr(bm, k).cpu().numpy() for k in
            ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")}


def assert_block_mask_equal(gpu_bm, ref):
    got = block_mask_arrays(gpu_bm)
    for k, arr in got.items():
        want = ref[k]
        assert arr.shape == want.shape, (k, arr.shape, want.shape)
        assert np.array_equal(arr, want), f"{k} differs at {np.argwhere(arr != want)[:5].tolist()}"


def assert_attention_close(out, lse, out_ref, lse_ref, dtype: str, what=""):
    """out within the dtype's max-abs bound; lse within 1e-3 and -inf exactly where expected."""
    o = out.float().cpu().numpy().astype(np.float64) if isinstance(out, torch.Tensor) else out
    assert not np.isnan(o).any(), f"{what}: NaN in out"
    err = np.abs(o - out_ref).max() if o.size else 0.0
    assert err <= TOL_OUT[dtype], f"{what}: out max-abs {err:.3e} > {TOL_OUT[dtype]}"
    if lse is not None:
        l = lse.cpu().numpy().astype(np.float64) if isinstance(lse, torch.Tensor) else lse
        assert not np.isnan(l).any(), f"{what}: NaN in lse"
        ref_inf = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(l), ref_inf), f"{what}: -inf pattern of lse differs"
        fin = ~ref_inf
        lerr = np.abs(l[fin] - lse_ref[fin]).max() if fin.any() else 0.0
        print(f"[parity] {what}: out max-abs {err:.3e}, lse max-abs {lerr:.3e}")
        PARITY_LOG.append((what, float(err), float(lerr)))
        assert lerr <= TOL_LSE, f"{what}: lse max-abs {lerr:.3e} > {TOL_LSE}"
    else:
        print(f"[parity] {what}: out max-abs {err:.3e}")
        PARITY_LOG.append((what, float(err), None))
    return err
