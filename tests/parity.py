"""Helpers for the GPU-vs-oracle parity tests: layout conversions and the acceptance rules.

Acceptance (fixed before any kernel was written):
  * int4 codes, {scale, zero}, page bounds and Quest page sets: bit-exact (fp16 metadata
    compared by value, so +0 and -0 are equal);
  * estimated weights: |w_gpu - w_orc| <= 1e-5 * w_orc on valid slots, exactly 0 elsewhere.
    fp32 weights carry 24 significant bits only down to 2^-126, the bottom of fp32's normal
    range; a valid slot whose oracle weight is below that may hold any fp32 value below
    2^-126 (0 included), as the library's header states for the weights it writes;
  * at p = 1 every valid candidate is kept, whatever its weight;
  * kept set: sum of the oracle's W over the GPU's kept set >= p - 1e-6, and the symmetric
    difference with the oracle's nucleus only holds tokens whose oracle W is within 1e-6 of
    the oracle's tau; kept ids strictly ascending;
  * attention output: max |o_gpu - o_orc| <= 2e-3, against the oracle run on the GPU's kept
    set (isolates the decode) and on the oracle's own kept set (end to end).
"""
from __future__ import annotations

import math

import numpy as np

import oracle

PAGE = 16
W_RTOL = 1e-5
W_NORMAL_MIN = 2.0 ** -126  # smallest normal fp32
MASS_TOL = 1e-6
TAU_TOL = 1e-6
OUT_ATOL = 2e-3


def sm_scale_for(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def logical_rows(paged: np.ndarray, page_table_row: np.ndarray, n: int, kvh: int) -> np.ndarray:
    """Rows [n, ...] of one sequence and KV head from a paged [P, Hkv, 16, ...] array."""
    P = -(-n // PAGE)
    blk = paged[page_table_row[:P], kvh]                   # [P, 16, ...]
    return blk.reshape((P * PAGE,) + blk.shape[2:])[:n]


def unpack_codes(packed: np.ndarray, bits: int = 4) -> np.ndarray:
    """[n, d * bits / 8] bytes -> [n, d] codes; a byte holds 8 / bits channels, the lowest
    channel in the lowest bits."""
    per = 8 // bits
    fields = [(packed >> (bits * i)) & ((1 << bits) - 1) for i in range(per)]
    return np.stack(fields, axis=-1).reshape(packed.shape[0], -1)


def oracle_units(w, p: float, units=None, headwise: bool = False, key_bits: int = 4,
                 threads: int = 1):
    """Oracle results per (b, kvh) unit (all units, or the listed ones). With threads > 1
    the units run concurrently (the oracle's C calls release the interpreter lock); each
    unit's result is the same either way."""
    s = w.spec
    G = s.G
    sm = sm_scale_for(s.d)
    if units is None:
        units = [(b, g) for b in range(s.B) for g in range(s.Hkv)]

    def one(u):
        b, g = u
        return oracle.run_unit(w.q[b, g * G:(g + 1) * G], w.k[b][g], w.v[b][g], w.budget, p,
                               sm, headwise=headwise, key_bits=key_bits)

    if threads > 1 and len(units) > 1:
        import concurrent.futures
        oracle.lib()  # loaded (and built if need be) once, before the workers start
        with concurrent.futures.ThreadPoolExecutor(min(threads, len(units))) as ex:
            return dict(zip(units, ex.map(one, units)))
    return {u: one(u) for u in units}


def head_view(res, h: int):
    """One query head of a head-wise oracle unit, shaped like a group-wise unit with G = 1
    (for check_kept and check_out)."""
    return {"weights": res["weights"][h:h + 1], "sel": res["sel"], "valid": res["valid"],
            "kept": res["kept"][h], "tau": res["tau"][h], "out": res["out"][h:h + 1]}


def slot_tokens(sel, n_slots: int, n: int) -> np.ndarray:
    """Logical token of every candidate slot (-1 when invalid)."""
    if sel is None:
        t = np.arange(n_slots)
    else:
        t = np.full(n_slots, -1, np.int64)
        full = (np.repeat(np.asarray(sel, np.int64), PAGE) * PAGE +
                np.tile(np.arange(PAGE), len(sel)))
        t[:full.size] = full
    t = np.where((t >= 0) & (t < n), t, -1)
    return t


def check_weights(w_gpu: np.ndarray, w_orc: np.ndarray, valid: np.ndarray):
    """w_gpu, w_orc: [G, n_slots]; returns the worst relative error on valid slots."""
    assert np.all(w_gpu[:, ~valid] == 0.0), "invalid slots must be exactly 0"
    a = w_gpu[:, valid].astype(np.float64)
    o = w_orc[:, valid]
    if a.size == 0:
        return 0.0
    below = (o < W_NORMAL_MIN) & (a < W_NORMAL_MIN)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(below, 0.0, np.abs(a - o) / o)
    worst = float(rel.max())
    assert worst <= W_RTOL, f"weight rel err {worst:.3e} > {W_RTOL}"
    return worst


def check_kept(kept_gpu: np.ndarray, res, p: float, n: int):
    """Apply the kept-set acceptance rules against one unit's oracle results."""
    kept_gpu = np.asarray(kept_gpu, np.int64)
    assert np.all(np.diff(kept_gpu) > 0), "kept ids must be strictly ascending"
    assert np.all((kept_gpu >= 0) & (kept_gpu < n))
    w = res["weights"]
    W = w.mean(axis=0)
    n_slots = W.shape[0]
    toks = slot_tokens(res["sel"], n_slots, n)
    w_by_tok = {int(t): float(W[j]) for j, t in enumerate(toks) if t >= 0}
    assert all(int(t) in w_by_tok for t in kept_gpu), "kept a non-candidate"
    total = sum(w_by_tok.values())
    mass = sum(w_by_tok[int(t)] for t in kept_gpu)
    if p >= 1.0:
        assert len(kept_gpu) == len(w_by_tok)
        return mass, 0
    assert mass >= p * total - MASS_TOL, f"kept mass {mass:.9f} < p={p}"
    diff = np.setxor1d(kept_gpu, res["kept"])
    tau = res["tau"]
    bad = [int(t) for t in diff if abs(w_by_tok[int(t)] - tau) > TAU_TOL]
    assert not bad, f"{len(bad)} kept-set differences away from tau (tau={tau:.3e})"
    return mass, len(diff)


def check_out(out_gpu: np.ndarray, q_group, k, v, kept_gpu, res, sm: float):
    """Attention output acceptance; returns (err vs GPU kept set, err vs oracle kept set).

    The end-to-end comparison applies when both kept sets are the same set. When they differ
    (only at weights within 1e-6 of tau, which check_kept enforces, e.g. exact ties that the
    threshold keeps together), both sets are valid nuclei and attention over either is a
    correct result; the output is then checked on the GPU's own set only."""
    o_gpu = out_gpu.astype(np.float64)
    o_same = oracle.sparse_attention(q_group, k, v, np.asarray(kept_gpu, np.int32), sm)
    e1 = float(np.abs(o_gpu - o_same).max()) if o_gpu.size else 0.0
    assert e1 <= OUT_ATOL, f"decode err {e1:.3e} on the GPU kept set"
    same = np.array_equal(np.asarray(kept_gpu, np.int64), np.asarray(res["kept"], np.int64))
    e2 = float(np.abs(o_gpu - res["out"]).max()) if (o_gpu.size and same) else 0.0
    assert e2 <= OUT_ATOL, f"end-to-end err {e2:.3e} vs the oracle kept set"
    return e1, e2
