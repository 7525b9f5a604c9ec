"""Mutation check of the oracle pins (CPU only; run: python tests/oracle_mutations.py).

Each entry plants one plausible mistake in a scratch copy of oracle/ and
expects at least one oracle pin test to fail.  Not collected by pytest.
"""
import os
import shutil
import subprocess
import sys
import tempfile

MUT = os.path.join(tempfile.gettempdir(), "csa_oracle_mutant")
muts = [
 ("csa.py", "a = z_rows + bias[:, None]", "a = z_rows"),
 ("csa.py", "np.broadcast_to(zb + bias[None, :, None]", "np.broadcast_to(zb"),
 ("csa.py", "np.maximum(dots, 0.0) * w[None, :]", "np.minimum(dots, 0.0) * w[None, :]"),
 ("csa.py", "(int(p) + 1) // int(m)", "int(p) // int(m)"),
 ("csa.py", "lo = max(0, p - n_win + 1, int(swa_pos0))", "lo = max(0, p - n_win, int(swa_pos0))"),
 ("csa.py", "order = np.lexsort((js, -scores))", "order = np.lexsort((-js, -scores))"),
 ("csa.py", "logits = s * (q @ keys.T)", "logits = (q @ keys.T)"),
 ("csa.py", "e = np.exp(a - a.max(axis=1, keepdims=True))\n    w = e / e.sum(axis=1", "e = np.exp(a - a.max(axis=2, keepdims=True))\n    w = e / e.sum(axis=2"),
 ("csa.py", "kI = pooled @ W", "kI = pooled[:, ::-1] @ W"),
 ("csa.py", "o = (e / den) @ keys", "o = (e / den) @ keys[::-1]"),
 ("csa.py", "rope = f32_to_bf16(c32[:, d_nope:])", "rope = f32_to_bf16(c32[:, d_nope - 1:-1])"),
 ("formats.py", "packed = (code[..., 0::2] | (code[..., 1::2] << 4))", "packed = (code[..., 1::2] | (code[..., 0::2] << 4))"),
 ("formats.py", "ex.astype(np.int64) - 1 - 2", "ex.astype(np.int64) - 2"),
 ("formats.py", "_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])", "_E2M1_TIE_UP = np.array([False] * 7)"),
 ("formats.py", "mant / 8.0 * 2.0 ** -6", "mant / 8.0 * 2.0 ** -7"),
 ("formats.py", "(e.astype(np.float64) - 7.0)", "(e.astype(np.float64) - 8.0)"),
 ("formats.py", "np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))", "np.uint64(0x8000)"),
 ("formats.py", "code = _e2m1_round(np.abs(scaled)) | np.where(scaled < 0, 8, 0)", "code = _e2m1_round(np.abs(scaled)) | np.where(scaled < -1e-30, 8, 0) & np.where(np.abs(scaled) > 0.25, 15, 0)"),
 ("formats.py", "x = np.clip(x, -127, 127)", "x = np.clip(x, -126, 127)"),
 ("csa.py", "bmax = np.maximum.reduceat(scores[:V], starts)", "bmax = np.minimum.reduceat(scores[:V], starts)"),
 ("csa.py", "nb = -(-V // block)", "nb = V // block"),
 ("csa.py", "ents = [np.arange(b * block, min((b + 1) * block, V))", "ents = [np.arange(b * block, (b + 1) * block)"),
 ("csa.py", "kept, _ = topk_select(bmax, np.arange(nb), n_blocks)", "kept, _ = topk_select(-bmax, np.arange(nb), n_blocks)"),
 ("csa.py", "            sel = idx\n        elif mode == REUSE:", "            pass\n        elif mode == REUSE:"),
 ("csa.py", "            pool = None\n            if L.get", "            if L.get"),
 ("csa.py", "            full = L[\"cache\"]\n", "            full = full if full is not None else L[\"cache\"]\n"),
 ("csa.py", "src = CAND_POOL if pool is not None else CAND_SELECTION", "src = CAND_SELECTION"),
 ("formats.py", "x = np.where(amax > 0, ex.astype(np.int64) - 1 - 8, -127)", "x = np.where(amax > 0, ex.astype(np.int64) - 1 - 7, -127)"),
 ("formats.py", "np.where(lo % 2 == 0, lo, hi)", "np.where(lo % 2 == 1, lo, hi)"),
 ("formats.py", "code = _e4m3_round(np.abs(scaled)) | np.where(scaled < 0, 0x80, 0)", "code = _e4m3_round(np.abs(scaled)) | np.where(scaled < -2.0 ** -9, 0x80, 0)"),
 ("csa.py", "return dict(codes=codes, scales=scales, rope=x[:, d_nope:].copy())", "return dict(codes=codes, scales=scales, rope=x[:, d_nope - 1:-1].copy())"),
 ("csa.py", "layer_b[\"qI\"], layer_b[\"w\"],\n                                   p, m, n_entries, k_b, cand=idx_a)", "layer_a[\"qI\"], layer_b[\"w\"],\n                                   p, m, n_entries, k_b, cand=idx_a)"),
 ("csa.py", "p, m, n_entries, k_b, cand=idx_a)", "p, m, n_entries, k_b)"),
 ("csa.py", "o_b, lse_b = sparse_attention(layer_b[\"q\"]", "o_b, lse_b = sparse_attention(layer_a[\"q\"]"),
 ("csa.py", "return np.concatenate([mxfp4_decode(nope, nscale), bf16_to_f64(rope)], axis=-1)", "return np.concatenate([bf16_to_f64(rope), mxfp4_decode(nope, nscale)], axis=-1)"),
 ("csa.py", "return np.concatenate([mxfp4_decode(nope, nscale), bf16_to_f64(rope)], axis=-1)", "return np.concatenate([mxfp4_decode(nope, nscale), bf16_to_f64(rope)[..., ::-1]], axis=-1)"),
 ("csa.py", "a, b = x[..., 0::2], x[..., 1::2]", "a, b = x[..., :d // 2], x[..., d // 2:]"),
 ("csa.py", "out[..., 1::2] = a * s + b * c", "out[..., 1::2] = -a * s + b * c"),
 ("csa.py", "theta = float(base) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)", "theta = float(base) ** (-1.0 * np.arange(d // 2, dtype=np.float64) / d)"),
 ("csa.py", "rope[\"base\"], sign=-1.0)", "rope[\"base\"], sign=1.0)"),
 ("csa.py", "pos = np.concatenate([(sel + 1) * m - 1,", "pos = np.concatenate([sel * m,"),
 ("csa.py", "lo + np.arange(win.shape[0], dtype=np.int64)])", "lo + 1 + np.arange(win.shape[0], dtype=np.int64)])"),
 ("csa.py", "out[:, -d_rope:] = bf16_to_f64(f32_to_bf16(rot.astype(np.float32)))", "out[:, -d_rope:] = rot"),
 ("csa.py", "q = _rotated_bf16(q, int(rope[\"p\"]), rope[\"base\"], dr)", "q = _rotated_bf16(q, 0, rope[\"base\"], dr)"),
 ("csa.py", "return _compress_rows(h @ bf16_to_f64(w_kv_u16), h @ bf16_to_f64(w_z_u16),", "return _compress_rows(h @ bf16_to_f64(w_z_u16)[:, :1] + h @ bf16_to_f64(w_kv_u16), h @ bf16_to_f64(w_z_u16),"),
 ("csa.py", "return _compress_rows(h @ bf16_to_f64(w_kv_u16), h @ bf16_to_f64(w_z_u16),", "return _compress_rows(h @ bf16_to_f64(w_kv_u16), h @ bf16_to_f64(w_kv_u16)[:, :bf16_to_f64(w_z_u16).shape[1]],"),
]
missed = 0
root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the oracle's own pins only: the copy holds no library, and a test that
# cannot run there would count every mutant as caught
pins = sorted("tests/" + f for f in os.listdir(os.path.join(root, "tests"))
              if f.startswith("test_oracle_") and f.endswith(".py"))


def run_pins(mutation=None):
    shutil.rmtree(MUT, ignore_errors=True)
    os.makedirs(MUT)
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(root, d), os.path.join(MUT, d))
    if mutation:
        f, a, b = mutation
        p = MUT + "/oracle/" + f
        s = open(p).read()
        assert s.count(a) >= 1, a
        open(p, "w").write(s.replace(a, b, 1))
    return subprocess.run(["python", "-m", "pytest", *pins, "-q", "-x", "-p", "no:cacheprovider"],
                          cwd=MUT, capture_output=True, text=True, timeout=600)


base = run_pins()
if base.returncode:
    print("the unmutated pins fail in the copy:\n" + base.stdout[-2000:])
    sys.exit(2)
for f, a, b in muts:
    r = run_pins((f, a, b))
    last = r.stdout.strip().splitlines()[-1]
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    missed += 0 if r.returncode else 1
    print("CAUGHT" if r.returncode else "MISSED", "|", a[:60], "|", failed[0][7:80] if failed else last)
sys.exit(1 if missed else 0)
