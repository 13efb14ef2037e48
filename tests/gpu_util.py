"""Helpers for the GPU parity tests: move 16-bit bit patterns to and from the
device, call the library through its C ABI, and compare with the oracle."""
import sys

import numpy as np

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs

F16, BF16 = inputs.F16, inputs.BF16

CLASSICAL_TOL = 1e-3
STRASSEN_TOL = 5e-3
STATS_TOL = 1e-3


def say(msg):
    """Name the case before the GPU work starts (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == BF16 else torch.float16


def to_dev(bits, dtype, pad_cols=0):
    """uint16 matrix -> device tensor; pad_cols > 0 gives a larger leading dimension."""
    import torch
    bits = np.ascontiguousarray(bits)
    if pad_cols:
        padded = np.full((bits.shape[0], bits.shape[1] + pad_cols), 0x7FC0, dtype=np.uint16)
        padded[:, :bits.shape[1]] = bits
        t = torch.from_numpy(padded.view(np.int16)).view(torch_dtype(dtype)).cuda()
        return t[:, :bits.shape[1]]
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch_dtype(dtype)).cuda()


def from_dev(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def empty_out(M, N, dtype, fill=0x7FC0):
    """Output tensor pre-filled with NaN bits so unwritten elements are caught."""
    import torch
    return to_dev(np.full((M, N), fill, dtype=np.uint16), dtype)


def rel_err(gpu_bits, ref_Q, dtype):
    return oracle.rel_fro(oracle.decode(gpu_bits, dtype), oracle.decode(ref_Q, dtype))


def check_full(gpu_bits, D, S, K, dtype, tol=CLASSICAL_TOL):
    """Whole-output parity of a classical (fp32-accumulated) product: every element
    inside oracle.elementwise_bound, and the normwise error against the oracle's
    rounded result within `tol`."""
    g = oracle.decode(gpu_bits, dtype)
    bound = oracle.elementwise_bound(D, S, K, dtype)
    bad = ~(np.abs(g - D) <= bound)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside the bound; "
                           f"first at {tuple(np.argwhere(bad)[0])}")
    Q = oracle.encode(D, dtype)
    assert rel_err(gpu_bits, Q, dtype) <= tol


# Per-element cap of the Strassen paths: their rounding error is not bounded element
# by element by |A||B| (the block sums pair k of one half of K with k of the other),
# so each element is held to ELEM_FACTOR times the normwise tolerance, in units of
# the output's RMS.  The error of one element sums thousands of independent
# roundings, so it is near-Gaussian with a deviation of about the normwise error
# (up to ~1.5x in the quadrants fed by the most products); the largest of 2.7e8
# such values is about sqrt(2 ln 2.7e8) = 6.2 deviations, inside 10x the tolerance,
# while a wrong block, sign or tile leaves errors of order |D| = RMS.
ELEM_FACTOR = 10.0


def check_full_strassen(gpu_bits, D, dtype, tol=STRASSEN_TOL):
    g = oracle.decode(gpu_bits, dtype)
    rms = float(np.sqrt(np.mean(D * D)))
    u16 = 2.0 ** -8 if dtype == BF16 else 2.0 ** -11
    bound = u16 * np.abs(D) + ELEM_FACTOR * tol * rms
    err = np.abs(g - D)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside the bound; "
                           f"worst {float(np.max(err / bound)):.3g}x at "
                           f"{tuple(np.unravel_index(np.argmax(err / bound), err.shape))}")
    Q = oracle.encode(D, dtype)
    assert rel_err(gpu_bits, Q, dtype) <= tol
    return float(np.max((err - u16 * np.abs(D)) / rms))


_handle = None


def handle():
    global _handle
    if _handle is None:
        _handle = fgemm.Handle(0)
    return _handle


def run(A_bits, B_bits, dtype, *, transA=False, transB=False, alpha=1.0, beta=0.0, C_bits=None,
        M=None, N=None, plan=None, epilogue=None, pad=0):
    """Run one GEMM on the device; returns the output bits.  `pad` widens the
    leading dimension of every operand by that many elements, or of A, B and C
    separately when it is a triple."""
    import torch
    pa, pb, pc = pad if isinstance(pad, tuple) else (pad, pad, pad)
    A = to_dev(A_bits, dtype, pa)
    B = to_dev(B_bits, dtype, pb)
    if M is None:
        M = A_bits.shape[1] if transA else A_bits.shape[0]
    if N is None:
        N = B_bits.shape[0] if transB else B_bits.shape[1]
    if C_bits is None:
        C_bits = np.full((M, N), 0x7FC0, dtype=np.uint16)  # NaN: unwritten elements show
    C = to_dev(C_bits, dtype, pc)
    handle().gemm(A, B, C, transA=transA, transB=transB, alpha=alpha, beta=beta, plan=plan,
                  epilogue=epilogue)
    torch.cuda.synchronize()
    return from_dev(C)


def check_full_strassen_swiglu(gpu_bits, out, H, d_gate, d_up, dtype, tol=STRASSEN_TOL):
    """Whole-output parity of RMS + SwiGLU over a Strassen product: the error of
    each sum in H is held to ELEM_FACTOR * tol * RMS of its half of H (the cap of
    check_full_strassen) and carried to the output through the exact first-order
    derivatives; then the 16-bit rounding; and normwise."""
    nout = out.shape[1]
    rg = float(np.sqrt(np.mean(H[:, :nout] ** 2)))
    ru = float(np.sqrt(np.mean(H[:, nout:] ** 2)))
    u16 = 2.0 ** -8 if dtype == BF16 else 2.0 ** -11
    bound = u16 * np.abs(out) + ELEM_FACTOR * tol * (np.abs(d_gate) * rg + np.abs(d_up) * ru)
    o = oracle.decode(gpu_bits, dtype)
    err = np.abs(o - out)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside the bound; "
                           f"worst {float(np.max(err / bound)):.3g}x")
    assert rel_err(gpu_bits, oracle.encode(out, dtype), dtype) <= tol
    return float(np.max(err / bound))
