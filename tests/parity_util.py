"""Helpers shared by the GPU parity tests: upload a workload, call the HIP path
through the C ABI, and compare with the fp64 oracle."""
import numpy as np
import torch

import varlen_flash_attention_fa_amd as fa

MAX_ABS = 2e-2     # bf16 output vs fp64 oracle, worst element
MEAN_ABS = 2e-3    # mean over all compared elements
# natural-log sum-exp, fp32 vs fp64.  The kernel's row sum adds the probabilities
# after their rounding to the 16-bit type that feeds the PV product (so out is
# normalised by exactly the weights it used); one round-to-nearest bf16 value is
# off by at most 2^-8 of itself, so the sum of non-negative terms is too and
# |d lse| <= -ln(1 - 2^-8) = 3.92e-3, plus fp32 rounding of the scores.  When many
# comparable terms share a row the errors average out; when one term dominates
# (ALiBi's distance penalty) the bound is nearly reached.
LSE_ABS = 4e-3


def to_dev(wl, dev="cuda"):
    d = dict(q=wl.q.to(dev), k=wl.k.to(dev), v=wl.v.to(dev),
             cu_q=torch.from_numpy(wl.cu_seqlens_q).to(dev),
             cu_k=torch.from_numpy(wl.cu_seqlens_k).to(dev),
             bt=None if wl.block_table is None else torch.from_numpy(wl.block_table).to(dev))
    return d


def run_hip(wl, dev_inputs=None, out=None, return_lse=True):
    d = dev_inputs or to_dev(wl)
    res = fa.varlen_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], block_table=d["bt"],
                        page_block_size=wl.page_block_size or None,
                        softmax_scale=wl.softmax_scale, window_left=wl.window_left,
                        window_right=wl.window_right, return_lse=return_lse, out=out)
    torch.cuda.synchronize()
    return res


def assert_close(out_gpu, lse_gpu, ref_out, ref_lse, rows=None, what=""):
    """Element-wise parity against the oracle on the selected token rows."""
    o = out_gpu.float().cpu().double().numpy()
    l = lse_gpu.cpu().double().numpy() if lse_gpu is not None else None
    if rows is not None:
        o, ref_out = o[rows], ref_out[rows]
        if l is not None:
            l, ref_lse = l[:, rows], ref_lse[:, rows]
    assert np.isfinite(o).all(), what + ": non-finite output"
    err = np.abs(o - ref_out)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    msg = "%s: max|d|=%.3g at %s (|o|=%.3g) mean|d|=%.3g" % (
        what, err.max() if err.size else 0, worst, abs(ref_out[worst]) if worst else 0,
        err.mean() if err.size else 0)
    assert (err.max() if err.size else 0) <= MAX_ABS, msg
    assert (err.mean() if err.size else 0) <= MEAN_ABS, msg
    if l is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(l), fin), what + ": lse finiteness differs"
        assert np.all(l[~fin] == ref_lse[~fin]), what + ": lse of empty rows"
        if fin.any():
            le = np.abs(l[fin] - ref_lse[fin])
            assert le.max() <= LSE_ABS, "%s: lse max|d|=%.3g mean|d|=%.3g" % (what, le.max(), le.mean())
    return err
