"""Plausible slips planted in the oracle, one at a time, to show that the CPU pins
catch each of them (test_oracle_mutations.py runs the pin suites once per slip).

A slip is a textual replacement in one oracle source file.  It is applied at
import time by a meta-path hook that compiles the replaced source in place of
the file, so every function of the oracle -- including the ones that call the
changed one -- runs the planted code.  Nothing in the oracle knows about it:
the hook lives here and is installed by conftest.py only when the environment
variable ORACLE_MUTATION names a slip.
"""
from __future__ import annotations

import importlib.abc
import importlib.machinery
import sys

# (name, oracle module, text in the source, replacement, occurrence to replace)
MUTATIONS = [
    # --- the quantisation points of the 8-bit layers
    ("fp8 fwd: x not quantised", "oracle.moe",
     "Xd = qdq_rows_fp8(X16) if X16.shape[0] else X16", "Xd = X16", 0),
    ("fp8 fwd: h not quantised", "oracle.moe",
     "Y[lo:hi] = st(qdq_rows_fp8(h) @ Wd[e].T)", "Y[lo:hi] = st(h @ Wd[e].T)", 0),
    ("fp8 bwd: dY not quantised", "oracle.moe",
     "dh = qdq_rows_fp8(dY16[lo:hi]) @ Wd[e]", "dh = dY16[lo:hi] @ Wd[e]", 0),
    ("fp8 bwd: dG|dU not quantised", "oracle.moe",
     "dX[lo:hi] = st(qdq_rows_fp8(dgu) @ np.concatenate([Wg[e], Wu[e]], 0))",
     "dX[lo:hi] = st(dgu @ np.concatenate([Wg[e], Wu[e]], 0))", 0),
    ("MX fwd: x not quantised", "oracle.moe", "Xd = qdq_rows_mx(X16)", "Xd = X16.astype(np.float64)", 0),
    ("MX fwd: h not quantised", "oracle.moe",
     "Y[lo:hi] = st(qdq_rows_mx(h) @ Wd[e].T)", "Y[lo:hi] = st(h @ Wd[e].T)", 0),
    ("MX bwd: dY not quantised", "oracle.moe",
     "dh = qdq_rows_mx(dY16[lo:hi]) @ WdT[e].T", "dh = dY16[lo:hi] @ WdT[e].T", 0),
    ("MX bwd: dG|dU not quantised", "oracle.moe",
     "dX[lo:hi] = st(qdq_rows_mx(dgu) @ np.concatenate([WgT[e], WuT[e]], 1).T)",
     "dX[lo:hi] = st(dgu @ np.concatenate([WgT[e], WuT[e]], 1).T)", 0),
    ("fp8 wgrad: first operand not quantised", "oracle.moe",
     "Pd, Qd = qdq_cols_fp8(P16, ep_recv_counts), qdq_cols_fp8(Q16, ep_recv_counts)",
     "Pd, Qd = np.asarray(P16, np.float64), qdq_cols_fp8(Q16, ep_recv_counts)", 0),
    ("int8 payload dropped (fp8 layer)", "oracle.moe",
     "Yc = qdq_rows_int8(Y) if comm_quant else Y", "Yc = Y", 0),
    ("int8 payload dropped (MX layer)", "oracle.moe",
     "Yc = qdq_rows_int8(Y) if comm_quant else Y", "Yc = Y", 1),
    ("int8 dispatch: smooth scales ignored", "oracle.moe",
     "X = (X * S[experts]).astype(np.float32)", "X = X.astype(np.float32)", 0),
    ("int8 ffn: h not quantised", "oracle.moe",
     "Y[lo:hi] = st(_i8_gemm(hq[lo:hi], hs[lo:hi], dq[e], ds[e]))",
     "Y[lo:hi] = st(h.astype(np.float64) @ (dq[e].astype(np.float64) * ds[e][:, None]).T)", 0),
    # --- the quantisers themselves
    ("e4m3 ties away from even", "oracle.numerics",
     "((dhi == dlo) & (hi != lo) & (hi % 2 == 0))", "((dhi == dlo) & (hi != lo))", 0),
    ("MX scale one binade too large", "oracle.numerics",
     "(p - 1) - 8 + (m > 0.875)", "(p - 1) - 7", 0),
    # --- the bf16 layer
    ("SwiGLU backward: sign of the sigmoid-derivative term", "oracle.moe",
     "dg = st(dh * u * s * (1 + g * (1 - s)))", "dg = st(dh * u * s * (1 - g * (1 - s)))", 0),
    ("SwiGLU backward: dU without the sigmoid", "oracle.moe",
     "du = st(dh * (g * s))", "du = st(dh * g)", 0),
    ("forward: h not rounded to bf16", "oracle.moe",
     "h = st(silu(g) * u)\n            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h\n            Y[lo:hi] = st(h @ Wd[e].T)",
     "h = silu(g) * u\n            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h\n            Y[lo:hi] = st(h @ Wd[e].T)", 0),
    ("forward: up projection with the gate weights", "oracle.moe",
     "            u = X[lo:hi] @ Wu[e].T\n            h = st(silu(g) * u)",
     "            u = X[lo:hi] @ Wg[e].T\n            h = st(silu(g) * u)", 0),
    ("backward: dWd from the transposed product's wrong operand", "oracle.moe",
     "dWd[e] = dY[lo:hi].T @ Hh[lo:hi]", "dWd[e] = dY[lo:hi].T @ U[lo:hi]", 0),
    ("backward: dX without the up-projection term", "oracle.moe",
     "dX[lo:hi] = st(np.concatenate([dg, du], 1) @ np.concatenate([Wg[e], Wu[e]], 0))",
     "dX[lo:hi] = st(dg @ Wg[e])", 0),
    ("combine: shared term weighted by the first weight", "oracle.moe",
     "out = out + decode(shared_expert_x, prec)", "out = out + w[:, :1] * decode(shared_expert_x, prec)", 0),
    ("combine: constant expert without alpha_2 * v", "oracle.moe",
     "return a1[j] * ori_x[t] + a2[j] * v[j]", "return a1[j] * ori_x[t]", 0),
    ("combine backward: dY without the weight", "oracle.moe",
     "dY[c] = w[t, k] * d[t]", "dY[c] = d[t]", 0),
    ("dispatch backward: copy term without the weight", "oracle.moe",
     "dx[t] = dx[t] + w[t, k] * d[t]", "dx[t] = dx[t] + d[t]", 0),
    ("route: rows of an expert in reverse slot order", "oracle.moe",
     "slots = np.nonzero(routed & (flat_id == e))[0]  # increasing slot order",
     "slots = np.nonzero(routed & (flat_id == e))[0][::-1]", 0),
    ("route: duplicates not dropped", "oracle.moe", "ok = act & valid & ~dup", "ok = act & valid", 0),
]


def mutate(module: str, source: str, index: int) -> str:
    name, mod, old, new, occurrence = MUTATIONS[index]
    if mod != module:
        return source
    parts = source.split(old)
    assert len(parts) > occurrence + 1, f"slip {name!r}: text not found in {module}"
    return old.join(parts[:occurrence + 1]) + new + old.join(parts[occurrence + 1:])


class _Loader(importlib.machinery.SourceFileLoader):
    def __init__(self, fullname, path, index):
        super().__init__(fullname, path)
        self.index = index

    def get_code(self, fullname):
        with open(self.path, encoding="utf-8") as f:
            src = f.read()
        return compile(mutate(fullname, src, self.index), self.path, "exec", dont_inherit=True)


class _Finder(importlib.abc.MetaPathFinder):
    def __init__(self, index):
        self.index = index

    def find_spec(self, fullname, path, target=None):
        if fullname != MUTATIONS[self.index][1]:
            return None
        spec = importlib.machinery.PathFinder.find_spec(fullname, path)
        if spec is None:
            return None
        spec.loader = _Loader(fullname, spec.origin, self.index)
        return spec


def install(index: int) -> None:
    """Plant slip `index` in the oracle (before it is first imported)."""
    assert "oracle" not in sys.modules, "the oracle is already imported"
    sys.meta_path.insert(0, _Finder(index))
