"""The oracle's pins reject plausible mistakes in it.

Each case copies oracle/fsdp_oracle.c, plants one mistake inside one function (a dropped
term, a wrong sign, index or order, a misplaced step), builds the copy and runs the oracle's
pin tests against it (FSDP_ORACLE_LIB); at least one pin must fail.  Every planted mistake
stays inside the buffers the function is given, so a mutant fails by its values, not by a
crash.  The committed oracle is never modified.
"""
import concurrent.futures
import os
import re
import subprocess
import sys
import tempfile

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "fsdp_oracle.c")
PINS = ["tests/test_oracle_cast.py", "tests/test_oracle_flat.py", "tests/test_oracle_rows.py",
        "tests/test_oracle_reduce.py", "tests/test_oracle_adamw.py", "tests/test_oracle_next.py",
        "tests/test_oracle_stats.py"]

# (name, function, [(text in that function, replacement), ...] applied in order)
MUTANTS = [
    ('bf16 widening shifted by 15', 'orc_bf16_to_f32',
     [('(uint32_t)h << 16', '(uint32_t)h << 15')]),
    ('bf16: ties away from zero', 'orc_bf16',
     [('(dropped == 0x8000u && (kept & 1u))', '(dropped == 0x8000u)')]),
    ('bf16: truncation', 'orc_bf16',
     [('kept += 1u;', 'kept += 0u;')]),
    ('bf16 array: last element dropped', 'orc_bf16_array',
     [('for (int64_t i = 0; i < n; ++i)', 'for (int64_t i = 0; i + 1 < n; ++i)')]),
    ('bf16: NaN not kept quiet', 'orc_bf16',
     [('return (uint16_t)(kept | 0x0040u);', 'return (uint16_t)kept;')]),
    ('flat: padding even when N divides T', 'orc_flat_sizes',
     [('int64_t S = ceil_div(T, N);', 'int64_t S = T / N + 1;')]),
    ('flat: pad value 1', 'build_flat',
     [('while (w < L) F[w++] = 0.0f;', 'while (w < L) F[w++] = 1.0f;')]),
    ('flat: shards in reverse rank order', 'orc_flat_shard',
     [('out[j] = F[k * S + j];', 'out[j] = F[(N - 1 - k) * S + j];')]),
    ('flat: copy-out offset off by one', 'orc_flat_copyout',
     [('off += numel[i];', 'off += numel[i] - (i == 0 && numel[i] > 0);')]),
    ('flat u16: shards in reverse rank order', 'orc_flat_shard_u16',
     [('out[j] = F[k * S + j];', 'out[j] = F[(N - 1 - k) * S + j];')]),
    ('flat u16: copy-out offset off by one', 'orc_flat_copyout_u16',
     [('off += numel[i];', 'off += numel[i] - (i == 0 && numel[i] > 0);')]),
    ('rows: numpy array_split rows instead of torch.chunk', 'orc_rows_shard',
     [('int64_t row_lo = min64(m[i], kk * c);\n            int64_t row_hi = min64(m[i], (kk + 1) * c);', 'int64_t row_lo = kk * (m[i] / N) + min64(kk, m[i] % N);\n            int64_t row_hi = (kk + 1) * (m[i] / N) + min64(kk + 1, m[i] % N);')]),
    ('rows: sizes count one extra row per parameter', 'orc_rows_sizes',
     [('s += ceil_div(m[i], N) * r[i];', 's += (ceil_div(m[i], N) + 1) * r[i];')]),
    ('rows: padding rows hold 1', 'orc_rows_shard',
     [('out[w++] = 0.0f;', 'out[w++] = 1.0f;')]),
    ('rows: copy-out rotated by one row', 'orc_rows_copyout',
     [('outs[i][w++] = orc_bf16(seg[e]);', 'outs[i][w++] = orc_bf16(seg[(e + r[i]) % ((row_hi - row_lo) * r[i])]);')]),
    ('rows u16: numpy array_split rows', 'orc_rows_shard_u16',
     [('int64_t row_lo = min64(m[i], kk * c);\n            int64_t row_hi = min64(m[i], (kk + 1) * c);', 'int64_t row_lo = kk * (m[i] / N) + min64(kk, m[i] % N);\n            int64_t row_hi = (kk + 1) * (m[i] / N) + min64(kk + 1, m[i] % N);')]),
    ('rows u16: copy-out rotated by one row', 'orc_rows_copyout_u16',
     [('outs[i][w++] = seg[e];', 'outs[i][w++] = seg[(e + r[i]) % ((row_hi - row_lo) * r[i])];')]),
    ('reduce: last rank dropped', 'orc_grad_reduce',
     [('for (int64_t r = 1; r < N; ++r)', 'for (int64_t r = 1; r < N - 1; ++r)')]),
    ('reduce: sum starts from +0', 'orc_grad_reduce',
     [('float acc = orc_bf16_to_f32(contribs[0][j]) / pre;\n        for (int64_t r = 1;', 'float acc = 0.0f;\n        for (int64_t r = 0;')]),
    ('reduce: pre as a reciprocal multiply', 'orc_grad_reduce',
     [('/ pre;', '* (1.0f / pre);')]),
    ('reduce: post dropped', 'orc_grad_reduce',
     [('out[j] = acc / post;', 'out[j] = acc;')]),
    ('reduce: pre and post swapped', 'orc_grad_reduce',
     [('/ pre;', '/ PRE_;'), ('out[j] = acc / post;', 'out[j] = acc / pre;'), ('/ PRE_;', '/ post;')]),
    ('adamw: eps inside the square root', 'orc_adamw',
     [('float den = sqrtf(vj) / bc2s + epsf;', 'float den = sqrtf(vj + epsf) / bc2s;')]),
    ('adamw: second-moment bias correction dropped', 'orc_adamw',
     [('float den = sqrtf(vj) / bc2s + epsf;', 'float den = sqrtf(vj) + epsf;')]),
    ('adamw: first-moment bias correction dropped', 'orc_adamw',
     [('float step_size = (float)(lr / (1.0 - pow(beta1, (double)step)));', 'float step_size = (float)lr;')]),
    ('adamw: weight decay after the update', 'orc_adamw',
     [('float pj = p[j] * decay;', 'float pj = p[j];')]),
    ('adamw: L2 penalty instead of decoupled decay', 'orc_adamw',
     [('float pj = p[j] * decay;\n        float gj = g[j];', 'float pj = p[j];\n        float gj = g[j] + (float)wd * p[j];')]),
    ('adamw: betas swapped in m', 'orc_adamw',
     [('float mj = b1 * m[j] + omb1 * gj;', 'float mj = b2 * m[j] + omb2 * gj;')]),
    ('adamw: decay sign', 'orc_adamw',
     [('float decay = (float)(1.0 - lr * wd);', 'float decay = (float)(1.0 + lr * wd);')]),
    ('adamw: bf16 copy of the parameter before the update', 'orc_adamw',
     [('float pj = p[j] * decay;', 'float p0 = p[j];\n        float pj = p0 * decay;'), ('if (pb) pb[j] = orc_bf16(pj);', 'if (pb) pb[j] = orc_bf16(p0);')]),
    ('hybrid: last rank of each group dropped', 'orc_grad_reduce_ex',
     [('r < (g + 1) * group; ++r', 'r < (g + 1) * group - 1; ++r')]),
    ('hybrid: accumulate ignored', 'orc_grad_reduce_ex',
     [('out[j] = accumulate ? out[j] + fresh : fresh;', 'out[j] = fresh;')]),
    ('hybrid: accumulate added before the post divide', 'orc_grad_reduce_ex',
     [('float fresh = total / post;\n        out[j] = accumulate ? out[j] + fresh : fresh;', 'out[j] = accumulate ? (out[j] * post + total) / post : total / post;')]),
    ('accumulate: init ignored', 'orc_grad_accumulate',
     [('acc[j] = init ? g : acc[j] + g;', 'acc[j] = acc[j] + g;')]),
    ('unscale: check after the multiply', 'orc_grad_unscale',
     [('if (!isfinite(x)) *found_inf = 1.0f;\n        g[j] = x * inv_scale;', 'g[j] = x * inv_scale;\n        if (!isfinite(g[j])) *found_inf = 1.0f;')]),
    ('unscale: flag cleared by finite values', 'orc_grad_unscale',
     [('if (!isfinite(x)) *found_inf = 1.0f;', '*found_inf = isfinite(x) ? 0.0f : 1.0f;')]),
    ('sqnorm flat: padding counted for the last parameter', 'orc_flat_sqnorm',
     [('if (g >= T) break; /* padding */', 'if (g >= T) { out[p - 1] += (double)shard[j] * shard[j]; continue; }')]),
    ('sqnorm flat: binary32 sums', 'orc_flat_sqnorm',
     [('double x = (double)shard[j];\n        out[i] = out[i] + x * x;', 'float x = shard[j];\n        out[i] = (float)((float)out[i] + x * x);')]),
    ('sqnorm flat: boundary element given to the previous parameter', 'orc_flat_sqnorm',
     [('while (g >= off + numel[i])', 'while (g > off + numel[i])')]),
    ('sqnorm rows: zero rows counted', 'orc_rows_sqnorm',
     [('int64_t rows = min64(m[i], (k + 1) * c) - min64(m[i], k * c);', 'int64_t rows = c;')]),
]


def _function_span(src, name):
    """Start and end of the C function `name` (its signature line through its closing brace)."""
    m = re.search(r"^[A-Za-z][^\n;]*\b%s\(" % re.escape(name), src, flags=re.M)
    assert m, name
    end = src.index("\n}\n", m.start()) + 3
    return m.start(), end


def _mutate(src, fn, pairs):
    a, b = _function_span(src, fn)
    body = src[a:b]
    for old, new in pairs:
        assert old in body, (fn, old)
        body = body.replace(old, new)
    return src[:a] + body + src[b:]


def _run_mutant(args):
    idx, (name, fn, pairs), src, tmp = args
    path_c = os.path.join(tmp, "mutant%d.c" % idx)
    path_so = os.path.join(tmp, "libmutant%d.so" % idx)
    with open(path_c, "w") as f:
        f.write(_mutate(src, fn, pairs))
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, src=path_c, out=path_so)
    env = dict(os.environ, FSDP_ORACLE_LIB=path_so, PYTHONDONTWRITEBYTECODE="1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    failed = [l.split(" ", 1)[1].split(" - ")[0] for l in p.stdout.splitlines()
              if l.startswith("FAILED ")]
    return name, p.returncode, failed, p.stdout[-1500:]


def test_every_function_has_a_mutant():
    src = open(SRC).read()
    exported = set(re.findall(r"^(?:float|uint16_t|void|int)\s+(orc_\w+)\(", src, flags=re.M))
    mutated = {fn for _, fn, _ in MUTANTS}
    assert exported <= mutated, sorted(exported - mutated)


def test_the_pins_reject_every_planted_mistake():
    src = open(SRC).read()
    for _, fn, pairs in MUTANTS:  # every mutation applies and changes the code
        assert _mutate(src, fn, pairs) != src
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [(i, m, src, tmp) for i, m in enumerate(MUTANTS)]
        workers = max(1, min(6, (os.cpu_count() or 2) - 2))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(_run_mutant, jobs))
    survivors = [(name, rc, out) for name, rc, failed, out in results if rc != 1 or not failed]
    assert not survivors, "\n\n".join("%s (exit %d)\n%s" % s for s in survivors)
