"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

# Tolerances (per element, |gpu - oracle| <= atol + rtol * |oracle|):
#  - fp16 KV, fp32 accumulate: max-abs 2e-3 / max-rel 1e-2 (the method's stated bound),
#    read as an allclose bound so that outputs near zero are judged by the absolute term;
#  - int8 / E4M3 KV: 5e-2 absolute against the oracle run on the dequantized cache;
#  - fp32 KV: every step is fp32 arithmetic on exact inputs; 1e-5 abs + 1e-5 rel covers
#    fp32 rounding over a few hundred terms (a wrong index or term is off by ~0.1).
TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "i8": (5e-2, 0.0), "e4m3": (5e-2, 0.0)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(gpu, ref: np.ndarray, cache_dtype: str, what: str = "", mag=None):
    """Element-wise |gpu - ref| <= atol * max(1, mag) + rtol * |ref|.

    mag (optional, broadcastable to ref): the magnitude of the V values each
    output element averages, for inputs far from N(0, 1) (see magnitude_ref).
    The stated tolerances hold for unit-scale V; every error term of the
    arithmetic (fp16 rounding of the weights, fp32 accumulation, the int8
    bias) scales with the magnitude of the V rows that carry weight, so the
    absolute term is taken relative to that magnitude when it exceeds 1."""
    g = gpu.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    atol, rtol = TOL[cache_dtype]
    if str(gpu.dtype) == "torch.float16":   # rounding of the output itself: half an fp16 ulp
        rtol = max(rtol, 2.0 ** -10)
    err = np.abs(g - ref)
    abs_term = atol if mag is None else atol * np.maximum(1.0, np.asarray(mag, np.float64))
    bound = abs_term + rtol * np.abs(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    big = np.abs(ref) >= 1e-3
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    say(f"  {what}: max_abs={max_abs:.3e} max_rel={max_rel:.3e}")
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, (f"{what}: {len(bad)} elements out of tolerance, first "
                           f"{bad[:5].tolist()} gpu={g[tuple(bad[0])]} ref={ref[tuple(bad[0])]}")
    return max_abs, max_rel


def pool_bytes(cache):
    k = cache.k.cpu().numpy()
    v = cache.v.cpu().numpy()
    ks = cache.k_scale.view(__import__("torch").int16).cpu().numpy().view(np.uint16) \
        if cache.k_scale is not None else None
    vs = cache.v_scale.view(__import__("torch").int16).cpu().numpy().view(np.uint16) \
        if cache.v_scale is not None else None
    return k, v, ks, vs


def check_pools_equal(cache, pools, what=""):
    k, v, ks, vs = pool_bytes(cache)
    assert np.array_equal(k, pools.k), f"{what}: K pool differs at {np.argwhere(k != pools.k)[:5].ravel().tolist()}"
    assert np.array_equal(v, pools.v), f"{what}: V pool differs at {np.argwhere(v != pools.v)[:5].ravel().tolist()}"
    if ks is not None:
        assert np.array_equal(ks, pools.k_scale), f"{what}: K scales differ"
        assert np.array_equal(vs, pools.v_scale), f"{what}: V scales differ"


def magnitude_ref(pools, q, tables, lens, scale, q_offsets=None):
    """The V magnitude each output element averages, by the oracle: the same
    attention (same weights) over V rows replaced by their magnitudes --
    |v| element by element for fp16 / fp32 caches, every code at the
    format's largest (127 for int8, 448 for E4M3) for quantized ones, i.e.
    127 or 448 times the token's V scale, at least the row's largest
    magnitude (the int8 bias error scales with the row's scale, not with the
    element).  Prefill rows when q_offsets is given."""
    import copy
    import oracle
    p = copy.copy(pools)
    v = pools.v
    dt = pools.cache_dtype
    if dt == "f16":
        p.v = (v.view(np.uint16) & np.uint16(0x7FFF)).view(np.uint8)
    elif dt == "f32":
        p.v = (v.view(np.uint32) & np.uint32(0x7FFFFFFF)).view(np.uint8)
    elif dt == "i8":
        p.v = np.full_like(v, 0x7F)
    else:
        p.v = np.full_like(v, 0x7E)
    if q_offsets is None:
        out, _ = oracle.decode(p, q, tables, lens, np.float32(scale))
    else:
        out, _ = oracle.prefill(p, q, tables, lens, q_offsets, np.float32(scale))
    return np.abs(out)
