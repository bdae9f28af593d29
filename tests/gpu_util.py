"""Helpers for the GPU parity tests: upload a workload, run an entry point,
compare against the oracle with the tolerances the target states."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from sparse_mla_attention_indices_amd import smla

# Tolerances, applied separately to o and to the finite lse values. nvfp4_ds_mla
# caches are held to the fp8 bounds, as the native-decode pull-request page
# holds its nvfp4 cases to its fp8 tolerance.
TOL = {"bf16": dict(max_abs=1e-2, rel_l2=5e-3), "fp8": dict(max_abs=2e-2, rel_l2=1e-2),
       "nvfp4": dict(max_abs=2e-2, rel_l2=1e-2)}
ORACLE_FORMAT = {"bf16": oracle.BF16_CACHE, "fp8": oracle.FP8_CACHE, "nvfp4": oracle.NVFP4_CACHE}


def entry_point(cache_format: str):
    """The library call that attends over a cache of this format."""
    return {"bf16": smla.smla_prefill_bf16, "fp8": smla.smla_decode_fp8,
            "nvfp4": smla.smla_decode_nvfp4}[cache_format]


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


class DeviceWorkload:
    def __init__(self, w, device="cuda"):
        self.w = w
        self.q = bf16_tensor(w.q, device)
        if w.cache_format == "bf16":
            self.cache = bf16_tensor(w.cache, device)
        else:
            self.cache = torch.from_numpy(np.ascontiguousarray(w.cache)).to(device)
        self.bt = torch.from_numpy(w.block_table).to(device)
        self.req = torch.from_numpy(w.req_id_per_token).to(device)
        self.idx = torch.from_numpy(w.topk_indices).to(device)

    def run(self, num_splits=0, with_phys=False, num_tokens=None, workspace=None):
        """One call over the first num_tokens tokens (default all)."""
        fn = entry_point(self.w.cache_format)
        T = self.w.num_tokens if num_tokens is None else num_tokens
        idx = self.idx[:T]
        phys = torch.full_like(idx, -7) if with_phys else None
        out, lse = fn(self.q[:T], self.cache, self.bt, self.req[:T], idx, self.w.sm_scale,
                      phys_indices_out=phys, num_splits=num_splits, workspace=workspace)
        torch.cuda.synchronize()
        return out, lse, phys


def oracle_run(w, tokens=None):
    fmt = ORACLE_FORMAT[w.cache_format]
    return oracle.attention(fmt, w.q, w.cache, w.block_table, w.req_id_per_token, w.topk_indices,
                            w.sm_scale, tokens=tokens)


def errors(got: np.ndarray, ref: np.ndarray):
    d = got.astype(np.float64) - ref
    denom = np.linalg.norm(ref)
    return float(np.abs(d).max(initial=0.0)), float(np.linalg.norm(d) / denom) if denom > 0 else float(np.linalg.norm(d))


def assert_parity(w, out, lse, tokens=None, label=""):
    """Compare GPU (out bf16 [T,H,512], lse fp32 [T,H]) with the oracle on `tokens`."""
    o_ref, lse_ref = oracle_run(w, tokens)
    sel = slice(None) if tokens is None else torch.as_tensor(np.asarray(tokens), device=out.device)
    o_gpu = out[sel].float().cpu().numpy().astype(np.float64)
    lse_gpu = lse[sel].cpu().numpy().astype(np.float64)
    tol = TOL[w.cache_format]
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{label}: lse finiteness differs"
    assert np.all(np.isneginf(lse_gpu[~fin])), f"{label}: empty rows must have lse = -inf"
    assert np.all(o_gpu[~fin] == 0), f"{label}: empty rows must have o = 0"
    o_max, o_rel = errors(o_gpu, o_ref)
    l_max, l_rel = errors(lse_gpu[fin], lse_ref[fin])
    log(f"[parity] {label}: o max_abs={o_max:.3e} rel_l2={o_rel:.3e}  "
        f"lse max_abs={l_max:.3e} rel_l2={l_rel:.3e}")
    assert o_max <= tol["max_abs"] and o_rel <= tol["rel_l2"], (label, o_max, o_rel)
    assert l_max <= tol["max_abs"] and l_rel <= tol["rel_l2"], (label, l_max, l_rel)
    return o_max, o_rel, l_max, l_rel


def value_bound(w):
    """[T, 512]: the largest |V[r, d]| over each token's valid rows (rows decoded by
    the oracle). Any softmax-weighted sum of those rows has sum_r p_r |v_r[d]| at
    most this."""
    phys = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    flat = w.cache.reshape(-1, w.cache.shape[-1])
    decode = {"bf16": oracle.decode_bf16_rows, "fp8": oracle.decode_fp8_rows,
              "nvfp4": oracle.decode_nvfp4_rows}[w.cache_format]
    vmax = np.zeros((w.num_tokens, 512))
    for t in range(w.num_tokens):
        slots = np.unique(phys[t][phys[t] >= 0])
        if slots.size:
            vmax[t] = np.abs(decode(flat[slots])[:, :512]).max(axis=0)
    return vmax


def assert_parity_up_to_output_rounding(w, out, lse, label="", weights_rounded=False):
    """For outputs that sit on few rows (|o| up to the rows' own magnitude, where half
    a bf16 ulp alone can pass the max-abs bound): error <= half a bf16 ulp of the
    true value + 2e-3 (fp8: one more half ulp, for a bf16 rounding of the dequantised
    rows; nvfp4 values are exact in bf16), the stated rel-L2 bound, and lse within 2e-3. weights_rounded: the
    weights entered PV as single bf16 values (lists past the short-list bound), each
    off by at most 2^-8 of itself (bf16 keeps 8 significant bits), which adds up to
    2^-8 sum_r p_r |v_r[d]| <= 2^-8 max_r |v_r[d]| per element."""
    o_ref, lse_ref = oracle_run(w)
    o = out.float().cpu().numpy().astype(np.float64)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(o_ref))[1] - 9)    # bf16: 8 significant bits
    bound = half_ulp * (2 if w.cache_format == "fp8" else 1) + 2e-3
    if weights_rounded:
        bound = bound + np.ldexp(value_bound(w), -8)[:, None, :]
    excess = np.abs(o - o_ref) - bound
    rel = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    log(f"[parity] {label}: max |o| {np.abs(o_ref).max():.2f}, max error beyond the bound {excess.max():.3e}, "
        f"rel_l2 {rel:.3e}")
    assert excess.max() <= 0 and rel <= TOL[w.cache_format]["rel_l2"], (label, excess.max(), rel)
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=2e-3)
