"""Helpers for the GPU parity tests: move device state and inputs into the
oracle's layout (float64, math orientation) and measure errors the way the
tolerances are stated (per (request, head) unit)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# tolerances (relative, per unit)
TOL_STATE_STEP = 1e-5      # reconstructed state between compressions
TOL_STATE_COMPRESS = 1e-4  # after a compression
TOL_READOUT = 1e-4
TIE_GAP = 1e-4             # (s_R - s_{R+1}) / s_1 below this: the truncation is not unique


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def units_of(t: torch.Tensor, lead: int = 2):
    """Flatten the leading (batch, heads) dims into one unit axis."""
    return t.reshape((-1,) + tuple(t.shape[lead:]))


def state_np(st: binding.ShallowState, units=None, r=None):
    """(a [n, d_k], U [n, d_k, r], V [n, d_v, r], vbar [n, d_v]) in float64."""
    r = st.r if r is None else r
    a = f64(units_of(st.a))
    U = f64(units_of(st.U))[:, :r].transpose(0, 2, 1)
    V = f64(units_of(st.V))[:, :r].transpose(0, 2, 1)
    vb = np.broadcast_to(f64(st.vbar)[None], (st.batch, st.heads, st.d_v)).reshape(-1, st.d_v)
    if units is not None:
        a, U, V, vb = a[units], U[units], V[units], vb[units]
    return a, U, V, vb


def inputs_np(inp: dict, units=None) -> dict:
    out = {}
    for key in ("q", "k", "v", "g", "beta"):
        x = inp.get(key)
        if x is None:
            out[key] = None
            continue
        x = f64(units_of(x))
        out[key] = x if units is None else x[units]
    return out


def rel_err(x, ref, axes):
    num = np.sqrt(np.sum((np.asarray(x) - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(np.asarray(ref) ** 2, axis=axes))
    return num / np.maximum(den, 1e-300)


def state_rel_err(a, U, V, a_ref, U_ref, V_ref, vb):
    S = oracle.reconstruct(a, U, V, vb)
    S_ref = oracle.reconstruct(a_ref, U_ref, V_ref, vb)
    return rel_err(S, S_ref, (-2, -1))


def content_gap(U, V, R):
    """Relative gap (s_R - s_{R+1}) / s_1 of the content U V^T, per unit."""
    s = np.linalg.svd(U @ np.swapaxes(V, -1, -2), compute_uv=False)
    if s.shape[-1] <= R:
        return np.full(s.shape[:-1], np.inf)
    return (s[..., R - 1] - s[..., R]) / np.maximum(s[..., 0], 1e-300)


def make_state(rule, batch, heads, d_k, d_v, R, W, vbar, device="cuda"):
    return binding.ShallowState(rule, batch, heads, d_k, d_v, R, W, vbar, device=device)


def gpu_inputs(rule, batch, heads, d_k, d_v, vbar, seed, t, in_dtype, layer=0):
    return wl.make_step(rule, batch, heads, d_k, d_v, vbar, seed, t, layer, in_dtype, "cuda")


def dense_prefill(rule, batch, heads, d_k, d_v, vbar, seed, steps, in_dtype, layer=0):
    """Dense prefill on the GPU (dense_decode_step), returns S [B, H, d_k, d_v]."""
    S = torch.zeros(batch, heads, d_k, d_v, device="cuda", dtype=torch.float32)
    o = torch.empty(batch, heads, d_v, device="cuda", dtype=torch.float32)
    for t in range(-steps, 0):
        inp = gpu_inputs(rule, batch, heads, d_k, d_v, vbar, seed, t, in_dtype, layer)
        binding.dense_decode_step(rule, S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
    return S


# ---------------------------------------------------------------------------
# Read-back of the lazily decayed forms at true scale.  The stored columns
# are U~ with U = Diag(gam) U~ (gam one float per unit, or one per key
# channel for Kimi Delta Attention); the library only marshals them, so the
# tests apply the scale themselves.  The device only gathers the units asked
# for (a copy); the scale is applied on the host in float64, so no device
# arithmetic outside the library enters a check.

def _gam_rows(st, gam):
    return gam if st.rule == "kda" else gam[..., None]


def _host(x, idx):
    """x [B, H, ...] as float64 on the host: every unit, or the flat unit
    indices idx ([len(idx), ...])."""
    if idx is not None:
        x = x.reshape((-1,) + tuple(x.shape[2:]))[idx]
    return x.detach().to("cpu", torch.float64)


def true_U(st: binding.ShallowState, idx=None) -> torch.Tensor:
    """U at true scale, float64 on the host: [B, H, cap, d_k], or
    [len(idx), cap, d_k] for the flat unit indices idx (st.U itself when
    decayed in place)."""
    U = _host(st.U, idx)
    if not st.lazy:
        return U
    return U * _gam_rows(st, _host(st.gam, idx))[..., None, :]


def true_factors16(st: binding.ShallowState16, idx=None):
    """(U, V) of the 16-bit form over the r columns held, U at true scale,
    float64 on the host ([B, H, r, .], or [len(idx), r, .])."""
    w = st.r - st.R
    U = torch.cat([_host(st.Uk, idx), _host(st.Uw, idx)[..., :w, :]], dim=-2)
    V = torch.cat([_host(st.Vk, idx), _host(st.Vw, idx)[..., :w, :]], dim=-2)
    return U * _gam_rows(st, _host(st.gam, idx))[..., None, :], V


def sched_true_factors(st: binding.ScheduledState, b: int, h: int):
    """(U at true scale [d_k, r], V [d_v, r]) of unit (b, h) of a per-request
    schedule before its next step, fp32 (after st.join()): its kept buffer
    c & 1 and window column numbers c W .. A - 1 in their ring slots."""
    A = st.t - int(st.t_start_host[b])
    R, W, D = st.R, st.W, st.D
    c = 0 if A < W + D else (A - D) // W
    w = max(A, 0) - c * W if A >= 0 else 0
    sel = c & 1
    cols_u = [st.KU[sel, b, h]]
    cols_v = [st.KV[sel, b, h]]
    if w > 0:
        slots = [(c * W + i) % (W + D) for i in range(w)]
        cols_u.append(st.Uw[b, h, slots])
        cols_v.append(st.Vw[b, h, slots])
    U = torch.cat(cols_u, 0).to("cpu", torch.float64)
    V = torch.cat(cols_v, 0).to("cpu", torch.float64)
    gs = (st.gam[b, h] if st.rule == "kda" else st.gam[b, h].reshape(1)).to("cpu", torch.float64)
    return (U * gs[None, :]).T, V.T
