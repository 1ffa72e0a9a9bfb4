"""Planted-mistake check of the oracle's pins (CPU only; not collected by pytest).

Each entry plants one plausible mistake in a temporary copy of oracle/ and
runs the oracle pin tests against that copy; every mutation must make at
least one pin fail. Run: python tests/oracle_mutation_check.py (about five
minutes). Exit status 1 if any mutation survives.
"""
import os, shutil, subprocess, sys, tempfile
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = [
 ("moe.py", "amax / FP8_MAX", "FP8_MAX / amax"),
 ("moe.py", "quot = (xf / scale[:, :, None])", "quot = (xf * (np.float32(1) / scale[:, :, None]))"),
 ("moe.py", "for j in range(k):\n        p = pos[toks, j]", "for j in range(k - 1):\n        p = pos[toks, j]"),
 ("moe.py", "cursor = offsets_e[:E]", "cursor = offsets_e[1:]"),
 ("moe.py", "src_idx[p] = t", "src_idx[p] = t * k + j"),
 ("moe.py", "offsets_r = [offsets_e[r * per] for r in range(R)]", "offsets_r = [offsets_e[r] for r in range(R)]"),
 ("moe.py", "term = w[toks, j]", "term = w[toks, k - 1 - j]"),
 ("moe.py", "quot = np.where(nonzero[:, :, None], quot, xf)", "quot = np.where(nonzero[:, :, None], quot, np.abs(xf))"),
 ("codecs.py", "((codes[hi] & 1) == 0))", "True)"),
 ("codecs.py", "(a > mid) |", "(a >= mid + 1e-300) |"),
 ("codecs.py", "subnormal = np.ldexp(mant.astype(np.float64), -9)", "subnormal = np.ldexp(mant.astype(np.float64), -10)"),
 ("codecs.py", "(expo - 10)", "(expo - 11)"),
 # rank-deduplicated exchange
 ("moe.py", "in_rank[t][e // per] = 1", "in_rank[t][e % R] = 1"),
 ("moe.py", "recv_idx[p, j] = e - r * per", "recv_idx[p, j] = e"),
 ("moe.py", "recv_w[p, j] = w[t, j]", "recv_w[p, j] = w[t, 0]"),
 ("moe.py", "        acc += rows\n        mag += np.abs(rows)", "        acc += rows if r else 0.0\n        mag += np.abs(rows)"),
 # MXFP8
 ("moe.py", "shared = np.clip(e - 1 - E4M3_EMAX, -127, 127)", "shared = np.clip(e - E4M3_EMAX, -127, 127)"),
 ("moe.py", "shared = np.where(nonzero, shared, -127)", "shared = np.where(nonzero, shared, 0)"),
 ("moe.py", "shared = np.clip(e - 1 - E4M3_EMAX, -127, 127)", "shared = np.clip(e - 1 - E4M3_EMAX, -126, 127)"),
 ("moe.py", "prod = vals * e8m0_decode(scales)[:, :, None]", "prod = vals * e8m0_decode(scales + 1)[:, :, None]"),
 # fixed-capacity layout
 ("moe.py", "            if r < C:", "            if r <= C:"),
 ("moe.py", "pos[t][j] = e * C + r", "pos[t][j] = e * C + C - 1 - r"),
 ("moe.py", '"counts": np.minimum(np.asarray(seen, dtype=np.int64), C)', '"counts": np.asarray(seen, dtype=np.int64)'),
 # router
 ("router.py", 'order = np.argsort(-L, axis=1, kind="stable")[:, :k]', 'order = np.argsort(L, axis=1, kind="stable")[:, ::-1][:, :k]'),
 ("router.py", "z = np.exp(sel - sel[:, :1])", "z = np.exp(sel)"),
 ("router.py", "z = 1.0 / (1.0 + np.exp(-sel))", "z = 1.0 / (1.0 + np.exp(sel))"),
 ("router.py", "w = z / z.sum(axis=1, keepdims=True)", "w = z / z[:, :1]"),
]
missed = 0
for fname, old, new in MUTS:
    d = tempfile.mkdtemp()
    for sub in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub))
    p = os.path.join(d, "oracle", fname)
    s = open(p).read()
    assert old in s, old
    open(p, "w").write(s.replace(old, new, 1))
    env = dict(os.environ, PYTHONPATH=d)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_codecs.py", "tests/test_oracle_layout.py", "tests/test_oracle_payload.py",
                        "tests/test_oracle_ranks.py", "tests/test_oracle_mxfp8.py", "tests/test_oracle_router.py",
                        "tests/test_oracle_fixed_capacity.py"],
                       cwd=d, env=env, capture_output=True, text=True)
    last = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else r.stderr[-200:]
    print(("CAUGHT " if r.returncode else "MISSED ") + f"{fname}: {old[:40]!r} -> {new[:40]!r} | {last}",
          flush=True)
    missed += 0 if r.returncode else 1
    shutil.rmtree(d)
print(f"{len(MUTS) - missed} of {len(MUTS)} mutations caught")
sys.exit(1 if missed else 0)
