"""Mutation check of the oracle's pins (CPU, run by hand; pytest does not
collect it): plant one plausible mistake at a time in a scratch copy of
oracle/ (a sign, a dropped scale or term, a transposed operand's stand-in,
a tie rule, an off-by-one causal limit or diagonal, floor for ceil, the GQA
head mapping, the XAttention and MoBA readings) and run
tests/test_oracle_pins.py on it; every mistake must make a pin fail.

    python tests/mutate_oracle.py          # all mutations
    python tests/mutate_oracle.py 3 11     # some of them
"""
import os
import shutil
import subprocess
import sys
import tempfile

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
M = [
 ("attention.py", "        dS = A * (dA - delta[h][:, None])", "        dS = A * (dA + delta[h][:, None])", "dense bwd: sign of D"),
 ("attention.py", "        dq[:, h] = scale * dS @ k[:, g]", "        dq[:, h] = dS @ k[:, g]", "dense dQ: dropped scale"),
 ("attention.py", "        dk[:, g] += scale * dS.T @ q[:, h]", "        dk[:, g] += dS.T @ q[:, h]", "dense dK: dropped scale"),
 ("attention.py", "        dv[:, g] += A.T @ do[:, h]", "        dv[:, g] += dS.T @ do[:, h]", "dense dV: dS for P"),
 ("attention.py", "            dS = A * (dA - delta[h, ri][:, None])", "            dS = A * (dA + delta[h, ri][:, None])", "support bwd: sign of D"),
 ("attention.py", "            dv[ci, g] += A.T @ do[ri, h]", "            dv[ci, g] = A.T @ do[ri, h]", "support dV: overwrite, not sum over heads"),
 ("attention.py", "            dk[ci, g] += scale * dS.T @ q[ri, h]", "            dk[ci, g] += scale * dS.T @ q[ri, h] * (h % 2 == 0)", "support dK: half the group's heads"),
 ("attention.py", "    o = (w1 / tot_safe)[..., None] * o1 + (w2 / tot_safe)[..., None] * o2", "    o = (w1 / tot_safe)[..., None] * o1 + (w1 / tot_safe)[..., None] * o2", "merge: wrong weight"),
 ("attention.py", "mx_safe + np.log(np.where(both_empty, 1.0, tot))", "mx_safe + 0.0 * np.log(np.where(both_empty, 1.0, tot))", "merge: LSE without the log term"),
 ("attention.py", "    return (_f64(o) * _f64(do)).sum(-1).T", "    return (_f64(o) * _f64(do)).mean(-1).T", "delta: mean for sum"),
 ("attention.py", "        g = h * hkv // hq\n        M = dense_mask", "        g = h % hkv\n        M = dense_mask", "dense: GQA head mapping"),
 ("index.py", "    share_v = _ceil_div(v_budget * seg_len, n_total)", "    share_v = (v_budget * seg_len) // n_total", "capacity: floor for ceil (verticals)"),
 ("index.py", "    return min(share_v, seg_len), min(_ceil_div(share_s, block), nb)", "    return min(share_v, seg_len), min(share_s // block, nb)", "capacity: floor for ceil (slash)"),
 ("index.py", "    order = np.lexsort((np.arange(scores.shape[0]), -scores))", "    order = np.lexsort((-np.arange(scores.shape[0]), -scores))", "top-k: ties to the highest index"),
 ("index.py", "    causal = cols[None, :] <= rows[:, None]", "    causal = cols[None, :] < rows[:, None]", "window: strict causal"),
 ("index.py", "        M[np.ix_(ri, ci)] = (m <= n) & (vert | slash | blk | rblk)", "        M[np.ix_(ri, ci)] = (m < n) & (vert | slash | blk | rblk)", "mask: strict causal"),
 ("index.py", "    g = ((rows - a) // block)[:, None] - (np.arange(L) // block)[None, :]", "    g = ((rows - a) // block)[:, None] - (np.arange(L) // block)[None, :] + 1", "slash score: off-by-one diagonal"),
 ("index.py", "    v = probs.sum(axis=0)", "    v = probs.max(axis=0)", "vertical score: max for sum"),
 ("xattn.py", "    ks = k_h[a:e].reshape(nC, S, -1)[:, ::-1]", "    ks = k_h[a:e].reshape(nC, S, -1)", "xattn: main diagonal for anti-diagonal"),
 ("xattn.py", "    causal = np.arange(nC)[None, :] <= np.arange(nC)[:, None]", "    causal = np.arange(nC)[None, :] < np.arange(nC)[:, None]", "xattn: diagonal cell dropped"),
 ("xattn.py", "                order = np.lexsort((np.arange(row.size), -row))", "                order = np.lexsort((-np.arange(row.size), -row))", "xattn: ties to the highest block"),
 ("moba.py", "        sel[r, own] = True", "        sel[r, own] = False", "moba: own block not picked"),
 ("moba.py", "        order = np.lexsort((np.arange(own), -past))", "        order = np.lexsort((-np.arange(own), -past))", "moba: ties to the latest block"),
 ("moba.py", "    return np.stack([k_h[a + b * B:min(a + (b + 1) * B, e)].mean(axis=0) for b in range(nB)])", "    return np.stack([k_h[a + b * B:min(a + (b + 1) * B, e)].sum(axis=0) for b in range(nB)])", "moba: block sums for means"),
]
only = sys.argv[1:]
res = []
for i, (f, old, new, what) in enumerate(M):
    if only and str(i) not in only:
        continue
    tmp = tempfile.mkdtemp(prefix="mut_")
    for d in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(REPO, d), os.path.join(tmp, d))
    shutil.copy(os.path.join(REPO, "pytest.ini"), tmp)
    p = os.path.join(tmp, "oracle", f)
    src = open(p).read()
    assert src.count(old) >= 1, (i, what)
    open(p, "w").write(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=tmp, capture_output=True, text=True, timeout=900)
    caught = r.returncode != 0
    line = [l for l in r.stdout.splitlines() if l.startswith("FAILED")][:1]
    res.append((i, what, caught, line[0][:110] if line else ""))
    print(i, "CAUGHT" if caught else "SURVIVED", what, line[0][:100] if line else "", flush=True)
    shutil.rmtree(tmp)
print(sum(c for _, _, c, _ in res), "of", len(res), "caught")
sys.exit(0 if all(c for _, _, c, _ in res) else 1)
