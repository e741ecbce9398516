"""Helpers for the GPU parity tests: uploading workloads and comparing against the oracle."""

from __future__ import annotations

import contextlib
import math

import numpy as np
import torch

import paged_kv_cache_285_amd as P
import workloads as W

ATOL = 1e-2  # max abs error allowed for bf16 outputs against the fp64 oracle
RTOL_L2 = 5e-3  # relative L2 error allowed
LSE_ATOL = 1e-3


def dev16(a: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Distance between adjacent bf16 values around |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


# Largest |value| the rows under test attend over (None: unknown).  Set for every workload that
# DeviceWorkload / the fp8 helpers upload, and by value_range() around other checks.
_VMAX = None


def workload_vmax(wl, fp8: bool = False) -> float:
    """max |v| over a workload's pools and new values (fp8 pools: e4m3 rounding adds up to 2^-4)."""
    arrs = [wl.v_cache] + [st.v for st in wl.steps]
    vmax = max(float(np.nanmax(np.abs((a.astype(np.uint32) << 16).view(np.float32)))) for a in arrs)
    return vmax * (1.0 + 2.0**-4 if fp8 else 1.0)


def set_value_range(wl, fp8: bool = False, vmax=None) -> None:
    global _VMAX
    _VMAX = workload_vmax(wl, fp8) if vmax is None else float(vmax)


@contextlib.contextmanager
def value_range(wl, fp8: bool = False):
    """Checks inside this context use the value range of ``wl``."""
    global _VMAX
    old = _VMAX
    _VMAX = workload_vmax(wl, fp8)
    try:
        yield _VMAX
    finally:
        _VMAX = old


# Inputs whose softmax rows one key dominates (queries 16x N(0,1)) are checked under the same rule.
peaked_tolerance = value_range


def rounding_bound(ref: np.ndarray, gpu: np.ndarray, bf16_out: bool) -> np.ndarray:
    """Per-element error the method's two prescribed roundings can produce.

    * P to bf16 before P.V: each weight p_j carries a relative error e_j up to the bf16 unit
      roundoff u = 2^-8 (8 significant bits, round to nearest even); the output is normalised by
      the sum of those same rounded weights, so it is a convex combination whose weights moved
      by w_j (e_j - e_mean) / (1 + e_mean), and |o_gpu - o| <= 2u / (1 - u) max_j |v_j - o|
      <= 2^-7 (1 + 2^-7) (max|v| + |o|).
    * The output to bf16: half a bf16 spacing at its magnitude.
    Plus 1e-5 of fp32 accumulation."""
    b = np.full(ref.shape, 1e-5)
    if _VMAX is not None:
        b = b + 2.0**-7 * (1.0 + 2.0**-7) * (_VMAX + np.abs(ref))
    if bf16_out:
        b = b + 0.5 * bf16_spacing(np.maximum(np.abs(ref), np.abs(gpu)))
    return b


def check_attention(gpu: np.ndarray, ref: np.ndarray, what: str, bf16_out: bool = True) -> dict:
    """Assert max |gpu - ref| <= ATOL and relative L2 <= RTOL_L2.  An element above ATOL is
    accepted only within rounding_bound() (the bf16 rounding of P and of the output, which the
    method prescribes); such elements are counted and printed."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(ref).all(), f"{what}: oracle produced non-finite values"
    assert np.isfinite(gpu).all(), f"{what}: GPU produced non-finite values at {np.argwhere(~np.isfinite(gpu))[:5]}"
    err = np.abs(gpu - ref)
    bad = err > ATOL
    exempt = 0
    if bad.any():
        bound = rounding_bound(ref, gpu, bf16_out)
        ok = err <= bound
        exempt = int(bad.sum())
        assert ok[bad].all(), (
            f"{what}: {int((bad & ~ok).sum())} elements exceed {ATOL} beyond the rounding bound "
            f"(vmax {_VMAX}); worst {err.max():.4g} at {np.unravel_index(err.argmax(), err.shape)}, worst excess "
            f"{(err - bound).max():.4g}"
        )
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    assert rel <= RTOL_L2, f"{what}: relative L2 {rel:.3g} > {RTOL_L2}"
    res = {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": rel, "above_atol_within_rounding": exempt}
    print(f"[parity] {what}: max_abs {res['max_abs']:.3g} rel_l2 {rel:.3g} above_1e-2_within_rounding {exempt}",
          flush=True)
    return res


# Largest LSE error the bf16 rounding of the weights can cause in a path whose LSE is taken from
# the sum of its rounded weights (the pipelined 256-row tiles and the cascade prefix pass): each
# weight carries a relative error up to the bf16 unit roundoff 2^-8 (8 significant bits, round to
# nearest even), so the sum does too and ln of it moves by at most ln(1 + 2^-8); plus fp32
# accumulation.
LSE_ROUNDING = math.log1p(2.0**-8) + 2e-5


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str) -> float:
    """LSE max abs error <= LSE_ATOL; elements above it are accepted only within LSE_ROUNDING
    (counted and printed)."""
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), f"{what}: LSE finiteness differs"
    err = np.abs(gpu[fin] - ref[fin])
    d = float(err.max()) if err.size else 0.0
    above = int((err > LSE_ATOL).sum())
    assert d <= LSE_ROUNDING, f"{what}: LSE max abs err {d:.3g} > {LSE_ROUNDING:.3g}"
    if above:
        print(f"[parity] {what}: LSE max abs {d:.3g}, {above} above {LSE_ATOL} within the weight rounding",
              flush=True)
    return d


class DeviceWorkload:
    """A workload's pools and per-step metadata on the device, plus the library shape."""

    def __init__(self, wl, scale: float = 0.0):
        self.wl = wl
        set_value_range(wl)
        self.k_cache = dev16(wl.k_cache)
        self.v_cache = dev16(wl.v_cache)
        self.shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride,
                                  block_size=wl.block_size, scale=scale)
        max_seq = max(int(s.seq_lens.max()) for s in wl.steps)
        max_t = max(s.num_tokens for s in wl.steps)
        max_b = max(s.num_seqs for s in wl.steps)
        self.ws = P.alloc_workspace(P.varlen_workspace_size(max_b, max_t, max_seq, self.shape))

    def step_tensors(self, st):
        return dict(
            q=dev16(st.q),
            k=dev16(st.k),
            v=dev16(st.v),
            bt=dev32(st.block_tables),
            qsl=dev32(st.query_start_loc),
            ctx=dev32(st.context_lens),
            seq=dev32(st.seq_lens),
        )

    def run_step(self, st, out_dtype=torch.bfloat16, want_lse=False, t=None):
        t = t or self.step_tensors(st)
        slots = P.compute_slot_mapping(t["bt"], t["qsl"], t["ctx"], self.shape, st.num_tokens)
        P.reshape_and_cache(t["k"], t["v"], self.k_cache, self.v_cache, slots, self.shape)
        plan = P.plan_varlen(self.ws, st.query_start_loc, st.context_lens, st.seq_lens, self.shape)
        lse = torch.empty((st.num_tokens, self.wl.num_q_heads), dtype=torch.float32, device="cuda") if want_lse else None
        out = P.paged_attention_varlen(
            t["q"], self.k_cache, self.v_cache, t["bt"], t["qsl"], t["ctx"], t["seq"], self.shape, plan, self.ws,
            out_dtype=out_dtype, lse=lse,
        )
        return slots, out, lse, plan


def many_requests(seed, num_req, num_kv_heads, head_dim):
    """A one-step batch of `num_req` requests with 1..5 new tokens each, with runs of requests
    that have no new token (query length 0) inserted between them: (workload, step arrays)."""
    rng = np.random.default_rng(seed)
    reqs = [W.RequestSpec(context=int(rng.integers(0, 40)), chunks=[int(rng.integers(1, 6))]) for _ in range(num_req)]
    wl = W.build("many_requests", reqs, num_q_heads=2 * num_kv_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, seed=seed)
    st = wl.steps[0]
    qlen = np.diff(st.query_start_loc)
    ql2, ctx2, bt2 = [], [], []
    for r in range(st.num_seqs):
        # before a fifth of the requests, a run of 1..300 requests with no new token
        for _ in range(int(rng.integers(1, 301)) if rng.random() < 0.2 else 0):
            ql2.append(0)
            ctx2.append(int(rng.integers(0, 40)))
            bt2.append(st.block_tables[int(rng.integers(0, st.num_seqs))])
        ql2.append(int(qlen[r]))
        ctx2.append(int(st.context_lens[r]))
        bt2.append(st.block_tables[r])
    qsl2 = np.zeros(len(ql2) + 1, dtype=np.int32)
    np.cumsum(ql2, out=qsl2[1:])
    return wl, st, qsl2, np.array(ctx2, dtype=np.int32), np.ascontiguousarray(np.stack(bt2).astype(np.int32))

