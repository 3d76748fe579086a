"""Planted mistakes in the oracle must fail its pins.

Each case copies one oracle module's source, plants one plausible mistake (a
dropped term, a wrong sign, index or bound, a transposed operand, the wrong
tie-break or comparison), runs the pin tests of tests/test_oracle_*.py against
the planted copy in this process, and requires at least one of them to fail.
The control case runs the same pins against an unchanged copy and requires all
of them to pass, so a failure above is the planted mistake's and not the
runner's. Nothing here touches the HIP library.
"""
import importlib
import inspect
import os
import sys
import types

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

PIN_MODULES = {m: "test_oracle_" + m for m in
               ("attention", "selection", "accept", "round", "dynamic", "model")}

# (case id, oracle module, text in its source, planted replacement, pin modules)
MUTATIONS = [
    # attention (MagicDec notes §3.2: verify reads the whole cache; causal
    # alignment of the gamma + 1 query rows; GQA grouping; paging)
    ("verify-causal-off-by-one", "attention",
     "np.repeat(L - n_q + np.arange(n_q), G)", "np.repeat(L - n_q - 1 + np.arange(n_q), G)",
     ["attention"]),
    ("verify-sees-future-row", "attention",
     "visible = pos[None, :] <= last_visible[:, None]",
     "visible = pos[None, :] <= last_visible[:, None] + 1", ["attention"]),
    ("gqa-interleaved-heads", "attention",
     "        heads = list(range(g * G, (g + 1) * G))\n        # rows ordered",
     "        heads = list(range(g, Hq, Hkv))\n        # rows ordered",
     ["attention"]),
    ("page-table-of-first-sequence", "attention",
     "pages = page_table[b, positions // P]",
     "pages = page_table[0, positions // P]", ["attention"]),
    ("softmax-not-normalised", "attention",
     "o[live] = (e @ values) / l", "o[live] = e @ values", ["attention"]),
    ("lse-drops-max", "attention",
     "lse[live] = m[live, 0] + np.log(l[:, 0])", "lse[live] = np.log(l[:, 0])", ["attention"]),
    ("scale-dropped", "attention",
     "s = scale * (q @ keys.T)", "s = q @ keys.T", ["attention"]),
    ("keys-values-swapped", "attention",
     "o[live] = (e @ values) / l", "o[live] = (e @ keys) / l", ["attention"]),
    ("sparse-shared-set-reads-head-row", "attention",
     "gi = hs[0] if per_query_head else (g if idx_heads > 1 else 0)",
     "gi = hs[0] if per_query_head else 0", ["attention"]),
    # StreamingLLM (sink + recent window)
    ("streaming-overlap-duplicates", "selection",
     "list(range(max(sink, L - recent), L))", "list(range(max(0, L - recent), L))",
     ["selection"]),
    ("streaming-recent-short-by-one", "selection",
     "list(range(max(sink, L - recent), L))", "list(range(max(sink, L - recent + 1), L))",
     ["selection"]),
    # SnapKV (observation-window votes, pooling, top-K, window kept)
    ("snapkv-window-visibility-shift", "selection",
     "np.repeat(L - W + np.arange(W), G)", "np.repeat(L - W + 1 + np.arange(W), G)",
     ["selection"]),
    ("snapkv-raw-weights-not-normalised", "selection",
     "p = e / e.sum(axis=1, keepdims=True)", "p = e", ["selection"]),
    ("snapkv-votes-include-window", "selection",
     "return p[:, :L - W].sum(axis=0)", "return p[:, W:].sum(axis=0)", ["selection"]),
    ("maxpool-window-clipped-short", "selection",
     "v[max(0, j - half):min(n, j + half + 1)]", "v[max(0, j - half):min(n, j + half)]",
     ["selection"]),
    ("topk-tie-break-reversed", "selection",
     "np.lexsort((np.arange(v.shape[0]), -v))", "np.lexsort((-np.arange(v.shape[0]), -v))",
     ["selection"]),
    ("topk-smallest-instead-of-largest", "selection",
     "np.lexsort((np.arange(v.shape[0]), -v))", "np.lexsort((np.arange(v.shape[0]), v))",
     ["selection"]),
    ("snapkv-window-shifted", "selection",
     "chosen = np.concatenate([kept, np.arange(L - W, L)])",
     "chosen = np.concatenate([kept, np.arange(L - W - 1, L - 1)])", ["selection"]),
    ("snapkv-budget-excludes-window", "selection",
     "kept = topk_lowest_index(pooled, K_b - W)", "kept = topk_lowest_index(pooled, K_b - W - 1)",
     ["selection"]),
    # acceptance (modified rejection sampling, the explainer's verification round)
    ("accept-with-less-equal", "accept",
     "if ua[b, i] * qi < pi:", "if ua[b, i] * qi <= pi:", ["accept"]),
    ("accept-ratio-inverted", "accept",
     "if ua[b, i] * qi < pi:", "if ua[b, i] * pi < qi:", ["accept"]),
    ("residual-sign-flipped", "accept",
     "np.maximum(0.0, p[n] - q[n])", "np.maximum(0.0, q[n] - p[n])", ["accept"]),
    ("residual-is-plain-target", "accept",
     "r = np.maximum(0.0, p[n] - q[n])", "r = p[n].copy()", ["accept"]),
    ("bonus-from-last-draft-row", "accept",
     "r = p[gamma].copy()", "r = p[gamma - 1].copy()", ["accept"]),
    ("inverse-cdf-wrong-side", "accept",
     'side="right"', 'side="left"', ["accept"]),
    ("temperature-ignored", "accept",
     "x = f64(z) / temperature", "x = f64(z)", ["accept"]),
    ("no-stop-at-first-reject", "accept",
     "                n += 1\n            else:\n                break",
     "                n += 1\n            else:\n                continue", ["accept"]),
    # correct results inside the flag band (accept_outcomes)
    ("band-ignores-zero-target-mass", "accept",
     "band = pi > 0 and qi > 0 and abs(ua[i] - pi / qi) < flag_eps",
     "band = qi > 0 and abs(ua[i] - pi / qi) < flag_eps", ["accept"]),
    ("zero-weight-tokens-drawable", "accept",
     "    live = r > 0\n", "    live = r >= 0\n", ["accept"]),
    ("draw-band-not-widened", "accept",
     "hit = live & (lo <= thr + eps * Z) & (c >= thr - eps * Z)",
     "hit = live & (lo <= thr) & (c > thr)", ["accept"]),
    ("band-test-decided-by-oracle-only", "accept",
     "can_acc.append(acc or band)", "can_acc.append(acc)", ["accept"]),
    # round bookkeeping
    ("append-one-slot-late", "round",
     "t = int(lens[b]) + j", "t = int(lens[b]) + j + 1", ["round"]),
    ("advance-keeps-rejected", "round",
     "lens = i64(kv_lens) + int(add)", "lens = i64(kv_lens)", ["round"]),
    ("compact-wrong-head", "round",
     "keys = token_rows(K, pt, b, pos, g)\n            vals = token_rows(V, pt, b, pos, g)\n            for t",
     "keys = token_rows(K, pt, b, pos, (g + 1) % Hkv)\n            vals = token_rows(V, pt, b, pos, (g + 1) % Hkv)\n            for t",
     ["round"]),
    ("compact-page-off-by-one", "round",
     "Kc[b * pages_per_seq + t // P, g, t % P] = keys[t]",
     "Kc[b * pages_per_seq + (t + 1) // P, g, (t + 1) % P] = keys[t]", ["round"]),
    ("tail-starts-one-late", "round",
     "np.arange(int(i64(tail_begin)[b]), int(i64(kv_lens)[b]), dtype=np.int64)",
     "np.arange(int(i64(tail_begin)[b]) + 1, int(i64(kv_lens)[b]), dtype=np.int64)", ["round"]),
    # dynamic top-K
    ("topk-attn-keeps-smallest", "dynamic",
     "keep = np.argsort(-s, kind=\"stable\")[:budget]", "keep = np.argsort(s, kind=\"stable\")[:budget]",
     ["dynamic"]),
    ("topk-unstable-ties", "dynamic",
     "keep = np.argsort(-s, kind=\"stable\")[:budget]",
     "keep = (len(s) - 1 - np.argsort(-s[::-1], kind=\"stable\"))[:budget]", ["dynamic"]),
    ("topk-wrong-kv-head", "dynamic",
     "np.arange(L), h // G)", "np.arange(L), h % K.shape[1])", ["dynamic"]),
    # speedup model (Omega of the cited speculative-decoding result)
    ("omega-missing-bonus-token", "model",
     "return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)",
     "return (1.0 - alpha ** gamma) / (1.0 - alpha)", ["model"]),
    ("round-time-drops-verify", "model",
     "return t_select_fixed + gamma * t_select_step + gamma * t_draft + t_verify",
     "return t_select_fixed + gamma * t_select_step + gamma * t_draft", ["model"]),
]


def _planted(modname, old, new):
    """(original module, copy of it executed from source with old -> new)."""
    mod = importlib.import_module("oracle." + modname)
    src = inspect.getsource(mod)
    if old != new:
        assert src.count(old) == 1, f"{old!r} must occur exactly once in oracle.{modname}"
    copy = types.ModuleType(mod.__name__)
    copy.__file__ = mod.__file__
    exec(compile(src.replace(old, new), mod.__file__, "exec"), copy.__dict__)
    return mod, copy


def _install(monkeypatch, mod, copy, spaces):
    """Rebind every name that refers to one of mod's functions to the copy's."""
    for name, obj in list(vars(mod).items()):
        if not (inspect.isfunction(obj) and obj.__module__ == mod.__name__):
            continue
        new = getattr(copy, name)
        for ns in spaces:
            for key, val in list(vars(ns).items()):
                if val is obj:
                    monkeypatch.setattr(ns, key, new)


def _pin_calls(test_mod):
    """(label, callable) for every pin test in a module, parametrize expanded.
    Tests that need fixtures are left out."""
    for name, fn in list(vars(test_mod).items()):
        if not (name.startswith("test_") and inspect.isfunction(fn)):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        params = inspect.signature(fn).parameters
        if not marks:
            if not params:
                yield name, fn
            continue
        assert len(marks) == 1, name
        argnames = [a.strip() for a in marks[0].args[0].split(",")] if isinstance(
            marks[0].args[0], str) else list(marks[0].args[0])
        if set(params) != set(argnames):
            continue
        for values in marks[0].args[1]:
            values = getattr(values, "values", values)
            if len(argnames) == 1:
                values = (values,)
            kwargs = dict(zip(argnames, values))
            yield f"{name}{list(kwargs.values())}", (lambda f=fn, kw=kwargs: f(**kw))


def _first_failing_pin(monkeypatch, modname, old, new, pin_mods):
    mod, copy = _planted(modname, old, new)
    tests = [importlib.import_module(PIN_MODULES[p]) for p in pin_mods]
    spaces = [oracle] + [importlib.import_module("oracle." + m) for m in PIN_MODULES] + tests
    _install(monkeypatch, mod, copy, spaces)
    ran = 0
    for t in tests:
        for label, call in _pin_calls(t):
            ran += 1
            try:
                call()
            except Exception as e:  # an assertion or a crash: the pin caught it
                return label, type(e).__name__, ran
    return None, None, ran


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(case, monkeypatch):
    _, modname, old, new, pin_mods = case
    label, err, ran = _first_failing_pin(monkeypatch, modname, old, new, pin_mods)
    assert label is not None, f"no pin among {ran} caught the planted mistake"


@pytest.mark.parametrize("modname", sorted(PIN_MODULES))
def test_unchanged_copy_passes_every_pin(modname, monkeypatch):
    """Control: the runner above, with nothing planted, passes every pin."""
    label, err, ran = _first_failing_pin(monkeypatch, modname, "", "", [modname])
    assert ran > 0
    assert label is None, f"unchanged oracle.{modname} failed {label} ({err})"
