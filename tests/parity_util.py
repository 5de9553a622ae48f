"""Helpers shared by the GPU parity tests: upload a workload, call the HIP path
through the C ABI, and compare with the fp64 oracle."""
import numpy as np
import torch

import varlen_flash_attention_fa_amd as fa

MAX_ABS = 2e-2     # bf16 output vs fp64 oracle, worst element
MEAN_ABS = 2e-3    # mean over all compared elements


def lse_bound(dtype, n_keys: int) -> float:
    """Largest |lse_gpu - lse_oracle| the kernel's arithmetic allows (natural log).

    No LSE tolerance is stated, so it is derived.  The kernel normalises by
    l = sum of the probabilities p_j = 2^(s_j - m) after rounding each to the
    16-bit type that feeds the PV product, with m placed so that the largest p is
    in [1, 2^8], hence l >= 1.  Relative error of l, term by term:
      * round to nearest of a normal value: u = 2^-8 (bf16) or 2^-11 (fp16);
      * fp16 only: p below 2^-14 is subnormal and rounds with an absolute error
        of at most 2^-25, so at most n_keys * 2^-25 relative to l >= 1 (bf16
        shares fp32's exponent range and has no such loss);
      * fp32 row sum: about n_keys / 32 + 16 sequential additions of 2^-24 each;
      * fp32 exponent arguments, v_exp_f32 and v_log_f32: below 2^-20 together.
    A relative error e of l moves lse by at most -ln(1 - e).  bf16 gives
    3.93e-3 at 4096 keys; fp16 6.2e-4 at 4097 keys.
    """
    import math
    name = str(dtype)
    u = 2.0 ** -11 if ("float16" in name and "bfloat16" not in name) or name == "f16" else 2.0 ** -8
    sub = n_keys * 2.0 ** -25 if u == 2.0 ** -11 else 0.0
    e = u + sub + (n_keys / 32.0 + 16.0) * 2.0 ** -24 + 2.0 ** -20
    return -math.log1p(-e)


# the bf16 bound at the longest key range any test uses (70k keys): 4.06e-3
LSE_ABS = lse_bound("bf16", 1 << 17)


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


def assert_close(out_gpu, lse_gpu, ref_out, ref_lse, rows=None, what="", n_keys=None):
    """Element-wise parity against the oracle on the selected token rows.

    The lse tolerance is ``lse_bound`` for the output's element type at
    ``n_keys`` (the longest key range of the call; default 2^17)."""
    lse_abs = lse_bound(out_gpu.dtype, n_keys if n_keys is not None else 1 << 17)
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
            assert le.max() <= lse_abs, "%s: lse max|d|=%.3g mean|d|=%.3g (bound %.3g)" % (
                what, le.max(), le.mean(), lse_abs)
    return err
