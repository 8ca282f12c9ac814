"""The pins must reject plausible mistakes in the oracle.

Each case plants one mistake into a temporary copy of ``oracle/`` (on the
CPU, never touching the real files) and runs the pin suites against it; at
least one pin must fail.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("coarse scale dropped", "S = (Qc @ Kc.T) / math.sqrt(D)", "S = (Qc @ Kc.T)"),
    ("context score over all query rows", "return P[:n_src, n_src:].mean(axis=0)",
     "return P[:, n_src:].mean(axis=0)"),
    ("TopK keeps the smallest", "order = np.lexsort((j, -np.asarray(c)))",
     "order = np.lexsort((j, np.asarray(c)))"),
    ("routing sends the sharpest to Taylor", "order = np.lexsort((i, np.asarray(M)))",
     "order = np.lexsort((i, -np.asarray(M)))"),
    ("Taylor block weight dropped",
     "P = np.exp(S - m) * np.asarray(w_new, dtype=np.float64)[None, :]", "P = np.exp(S - m)"),
    ("sharpness not centred", "return ((P - 1.0 / N_K) ** 2).mean(axis=1)",
     "return (P ** 2).mean(axis=1)"),
    ("K in place of V", "O = (P @ V_new) / l[:, None]", "O = (P @ K_new) / l[:, None]"),
    ("TopK count floors", "k = math.ceil(alpha_s * n_ctx - _GUARD)", "k = math.floor(alpha_s * n_ctx)"),
    ("gather indexes source blocks", "parts += [X[starts[n_src + j]:ends[n_src + j]] for j in sel]",
     "parts += [X[starts[j]:ends[j]] for j in sel]"),
    ("LSE drops the max", "O = (P @ V_new) / l[:, None]\n    return O, m[:, 0] + np.log(l)",
     "O = (P @ V_new) / l[:, None]\n    return O, np.log(l)"),
    ("partial context block overruns", "ends.append(min(L_src + (j + 1) * b, L_src + L_ctx))",
     "ends.append(L_src + (j + 1) * b)"),
    ("Taylor scale 1/D", "S = (Qrows @ Kc_new.T) / math.sqrt(D)", "S = (Qrows @ Kc_new.T) / D"),
    ("Taylor uses the first blocks, not the kept ones",
     "Kc_new = pool_blocks(Kh, starts[kept], ends[kept])",
     "Kc_new = pool_blocks(Kh, starts, ends)[:len(kept)]"),
    ("flat takes the largest M", "flat = np.sort(order[:n_flat]).astype(np.int64)",
     "flat = np.sort(order[-n_flat:] if n_flat else order[:0]).astype(np.int64)"),
    ("masked blocks also enter the Taylor sum", "rep = np.nonzero(~exact)[0]",
     "rep = np.arange(len(w))"),
    ("exact tokens weighted by the block length", "E_tok = np.exp(S_tok - m)\n",
     "E_tok = np.exp(S_tok - m) * w[0]\n"),
    ("mask keeps the smallest coarse scores", "order = np.lexsort((u, -np.asarray(p_row)))",
     "order = np.lexsort((u, np.asarray(p_row)))"),
    ("mask ranks the first blocks, not the kept ones", "top_ns_blocks(P[i, kept], n_ns)",
     "top_ns_blocks(P[i, :len(kept)], n_ns)"),
    ("mask count floors", "n = math.ceil(alpha_ns * n_kv - _GUARD)", "n = math.floor(alpha_ns * n_kv)"),
    ("mixed drops the representative weight", "E_rep = np.exp(S_rep - m) * w[rep][None, :]",
     "E_rep = np.exp(S_rep - m)"),
]

# mistakes in the backward (oracle/isa_oracle_bwd.py)
BWD_MUTATIONS = [
    ("Taylor backward drops the block weight", "Pi = np.exp(S) * w_new[None, :]",
     "Pi = np.exp(S)"),
    ("masked backward drops the representative weight",
     "logw = np.concatenate([np.zeros(len(tok)), np.log(w_new[rep])])",
     "logw = np.zeros(len(tok) + len(rep))"),
    ("masked backward keeps only the last flat block's pooled gradient",
     "            dKc[rep] += dkr\n", "            dKc[rep] = dkr\n"),
]


# mistakes in the rotary embedding (oracle/isa_oracle_rope.py)
ROPE_MUTATIONS = [
    ("rope turns the other way", "out[..., 0::2] = x * c - y * s", "out[..., 0::2] = x * c + y * s"),
    ("rope context positions continue the source",
     "np.concatenate([np.arange(L_src), np.arange(L_ctx)])",
     "np.concatenate([np.arange(L_src), np.arange(L_src, L_src + L_ctx)])"),
    ("rope pairs the two halves instead of neighbours", "x, y = X[..., 0::2], X[..., 1::2]",
     "h = X.shape[-1] // 2\n    x, y = X[..., :h], X[..., h:]"),
    ("rope frequency exponent halved", "return np.power(float(base), -2.0 * i / D)",
     "return np.power(float(base), -i / D)"),
    ("bf16 rounding through fp32", "    if dtype == \"bf16\":\n        return round_to_bf16(x)",
     "    if dtype == \"bf16\":\n        return round_to_bf16(np.asarray(x).astype(np.float32)"
     ".astype(np.float64))"),
    ("bf16 rounding ties away from zero", "return np.ldexp(np.rint(m * 256.0), e - 8)",
     "return np.ldexp(np.trunc(m * 256.0 + np.copysign(0.5, m)), e - 8)"),
    ("rope backward turns the gradient forward, not back",
     "return rotate_pairs(dQr, -theta), rotate_pairs(dKr, -theta), dV",
     "return rotate_pairs(dQr, theta), rotate_pairs(dKr, theta), dV"),
    ("rope backward leaves dK unturned",
     "return rotate_pairs(dQr, -theta), rotate_pairs(dKr, -theta), dV",
     "return rotate_pairs(dQr, -theta), dKr, dV"),
]

ALL = [(n, o, w, "isa_oracle.py") for n, o, w in MUTATIONS] + \
      [(n, o, w, "isa_oracle_rope.py") for n, o, w in ROPE_MUTATIONS] + \
      [(n, o, w, "isa_oracle_bwd.py") for n, o, w in BWD_MUTATIONS]


@pytest.mark.parametrize("name,old,new,fname", ALL, ids=[m[0] for m in ALL])
def test_pins_reject_planted_mistake(tmp_path, name, old, new, fname):
    src = open(os.path.join(ROOT, "oracle", fname)).read()
    assert src.count(old) == 1, f"mutation anchor missing: {old!r}"
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    (tmp_path / "oracle" / fname).write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py",
                        "tests/test_oracle_ns_pins.py", "tests/test_oracle_rope_pins.py"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"no pin caught the planted mistake: {name}\n{r.stdout[-2000:]}"
