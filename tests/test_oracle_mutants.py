"""Pin strength: plant plausible mistakes in a copy of the oracle (on the CPU)
and check that the oracle pins reject every one of them."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
 "no_decay": ("p = master * c[\"decay\"]", "p = master * np.float32(1.0)"),
 "sign": ("p = p - c[\"step_size\"] * (m / denom)", "p = p + c[\"step_size\"] * (m / denom)"),
 "swap_b1": ("m = c[\"b1\"] * m + c[\"omb1\"] * g", "m = c[\"omb1\"] * m + c[\"b1\"] * g"),
 "eps_in": ("denom = np.sqrt(v) / c[\"bc2_sqrt\"] + c[\"eps\"]", "denom = np.sqrt(v / c[\"bc2_sqrt\"] + c[\"eps\"])"),
 "no_bc2": ("denom = np.sqrt(v) / c[\"bc2_sqrt\"] + c[\"eps\"]", "denom = np.sqrt(v) + c[\"eps\"]"),
 "no_bc1": ("c[\"step_size\"] = np.float32(float(lr) / (1.0 - p1))", "c[\"step_size\"] = lr"),
 "no_sq": ("v = c[\"b2\"] * v + c[\"omb2\"] * (g * g)", "v = c[\"b2\"] * v + c[\"omb2\"] * g"),
 "bf16_trunc": ("r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)", "r = u >> np.uint64(16)"),
 "grow_off1": ("if good == st.window:", "if good == st.window - 1:"),
 "hyst_noreset": ("return replace(st, good_steps=good, hyst_left=st.hysteresis)", "return replace(st, good_steps=good)"),
 "clip_always": ("if max_norm > 0.0 and norm > max_norm:", "if max_norm > 0.0:"),
 "sumsq_abs": ("total += float(np.sum(xc * xc))", "total += float(np.sum(np.abs(xc)))"),
 "shard_off1": ("out.append((t, a - o, b - a, a - lo))", "out.append((t, a - o, b - a - (1 if b - a > 1 else 0), a - lo))"),
 "layout_noalign": ("pos = align_up(pos + n, align)", "pos = pos + n"),
 "flatten_copy_ignores_start": ("bucket[d:d + n] = srcs[t][s:s + n]", "bucket[d:d + n] = srcs[t][:n]"),
 "flatten_acc_ignores_start": ("x = widen(srcs[t][s:s + n], src_dtype)", "x = widen(srcs[t][:n], src_dtype)"),
 "flatten_dst_off1": ("bucket[d:d + n] = srcs[t][s:s + n]", "bucket[d + 1:d + 1 + n] = srcs[t][s:s + n]"),
 "acc_overwrite":("acc[d:d + n] = acc[d:d + n] + x", "acc[d:d + n] = x"),
 "no_K": ("sk = float(scale) * float(accum_steps)", "sk = float(scale)"),
 "scale_not_halved": ("return replace(st, scale=max(st.scale / 2.0, st.min_scale),", "return replace(st, scale=max(st.scale, st.min_scale),"),
 "t_on_skip": ("return replace(st, hyst_left=st.hyst_left - 1, good_steps=0, last_skip=1)", "return replace(st, hyst_left=st.hyst_left - 1, good_steps=0, last_skip=1, t=st.t+1)"),
 "ovf_mask": ("return (bits & m) == m", "return (bits & m) == m - 1"),
 "widen_bf16": ("return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)", "return (x.astype(np.uint32) << np.uint32(15)).view(np.float32)"),
 "decay_sign": ("c[\"decay\"] = np.float32(1.0 - float(lr) * float(wd))", "c[\"decay\"] = np.float32(1.0 + float(lr) * float(wd))"),
 "reduce_drop_last": ("    for sl in slices[1:]:", "    for sl in slices[1:-1]:"),
 "reduce_ignore_dst": ("        return dst + acc if accumulate else acc", "        return acc"),
 "consolidate_unsorted": ("    shards = sorted(shards, key=lambda s: s[0])\n    pos = 0", "    pos = shards[0][0] if shards else 0"),
 "consolidate_keep_pad": ("return [flat[o:o + n].copy() for o, n in zip(offsets, numels)]", "return [flat[i * n:(i + 1) * n].copy() for i, n in enumerate(numels)]"),
 "onebit_no_err": ("    c = x + np.asarray(err, np.float32)\n", "    c = x.copy()\n"),
 "onebit_lane_order": ("        lane, k = divmod(q, 4)\n", "        k, lane = divmod(q, 64)\n"),
 "onebit_msb_first": ("words[64 * u + lane] |= np.uint32(1) << np.uint32(4 * r + k)", "words[64 * u + lane] |= np.uint32(1) << np.uint32(31 - 4 * r - k)"),
 "onebit_group_major": ("words[64 * u + lane] |= np.uint32(1) << np.uint32(4 * r + k)", "words[64 * u + lane] |= np.uint32(1) << np.uint32(8 * k + r)"),
 "onebit_mean_abs": ("s = np.float32(math.sqrt(sumsq / (b - a)))", "s = np.float32(math.fsum(abs(float(v)) for v in c[a:b]) / (b - a))"),
 "onebit_full_len": ("s = np.float32(math.sqrt(sumsq / (b - a)))", "s = np.float32(math.sqrt(sumsq / chunk))"),
 "onebit_err_sign": ("np.where(pos[a:b], c[a:b] - s, c[a:b] + s)", "np.where(pos[a:b], c[a:b] + s, c[a:b] - s)"),
 "onebit_neg_zero": ("    pos = c >= np.float32(0.0)\n", "    pos = ~np.signbit(c)\n"),
 "onebit_dec_sign": ("return np.where(bit == 1, np.float32(1.0), np.float32(-1.0))", "return np.where(bit == 1, np.float32(-1.0), np.float32(1.0))"),
 "clip_no_eps": ("coef = float(max_norm) / (norm + 1e-6)", "coef = float(max_norm) / norm"),
 "clip_at_or_below_max": ("if max_norm > 0.0 and norm > max_norm:", "if max_norm > 0.0 and norm >= max_norm * 0.999:"),
 "norm_sqrt_of_quotient": ("norm = math.sqrt(sumsq) / sk", "norm = math.sqrt(sumsq / sk)"),
 "grad_scale_no_K": ("grad_scale = np.float32(coef / sk)", "grad_scale = np.float32(coef / float(scale))"),
 "bc2_no_sqrt": ("c[\"bc2_sqrt\"] = np.float32(math.sqrt(1.0 - p2))", "c[\"bc2_sqrt\"] = np.float32(1.0 - p2)"),
 "m_unscaled_grad": ("m = c[\"b1\"] * m + c[\"omb1\"] * g", "m = c[\"b1\"] * m + c[\"omb1\"] * widen(x, dtype)"),
 "decay_after_update": ("    p = master * c[\"decay\"]\n    p = p - c[\"step_size\"] * (m / denom)",
                        "    p = master - c[\"step_size\"] * (m / denom)\n    p = p * c[\"decay\"]"),
 "fp16_truncate": ("return p.astype(np.float16).view(np.uint16)", "return (p.view(np.uint32) >> np.uint32(13)).astype(np.uint16)"),
 "bf16_nan_rounded": ("r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)", "r = r"),
 "beta_pow_skip": ("st = replace(st, t=st.t + 1, beta1_pow=st.beta1_pow * b1, beta2_pow=st.beta2_pow * b2,", "st = replace(st, t=st.t + 1, beta1_pow=st.beta1_pow * b2, beta2_pow=st.beta2_pow * b1,"),
 "ddp_bytes": ("return 2 * psi + 2 * psi + 12 * psi", "return 2 * psi + 12 * psi"),
 "stage1_bytes": ("return Fraction(4 * psi) + Fraction(12 * psi, n)", "return Fraction(2 * psi) + Fraction(14 * psi, n)"),
 "stage2_bytes": ("return Fraction(2 * psi) + Fraction(14 * psi, n)", "return Fraction(4 * psi) + Fraction(12 * psi, n)"),
 "stage3_bytes": ("return Fraction(16 * psi, n)", "return Fraction(14 * psi, n) + 2 * psi"),
 "shard_pad_to_world": ("padded = align_up(flat_total, world * align)", "padded = align_up(flat_total, world)"),
 "shard_no_pad": ("padded = align_up(flat_total, world * align)", "padded = flat_total"),
 "layout_first_offset": ("    pos = 0\n    for n in numels:\n", "    pos = align\n    for n in numels:\n"),
 "entries_abs_dst": ("out.append((t, a - o, b - a, a - lo))", "out.append((t, a - o, b - a, a))"),
 "round_robin_blocks": ("return [list(names[r::world]) for r in range(world)]",
                        "return [list(names[r * len(names) // world:(r + 1) * len(names) // world]) for r in range(world)]"),
 "fp16_widen_as_bf16": ("        return x.view(np.float16).astype(np.float32)",
                        "        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)"),
 "nonfinite_nan_only": ("    return (bits & m) == m\n", "    return ((bits & m) == m) & ((bits & ~m) != 0)\n"),
 "sumsq_fp32": ("        xc = widen(x[a:a + chunk], dtype).astype(np.float64)\n", "        xc = widen(x[a:a + chunk], dtype)\n"),
 "ovf_grad_scale_one": ("                    coef=1.0, grad_scale=np.float32(0.0))",
                        "                    coef=1.0, grad_scale=np.float32(1.0))"),
 "static_no_skip": ("            return replace(st, last_skip=1)\n", "            return replace(st, last_skip=0)\n"),
 "min_scale_ignored": ("scale=max(st.scale / 2.0, st.min_scale)", "scale=st.scale / 2.0"),
 "growth_uncapped": ("scale=min(st.scale * 2.0, 2.0 ** 127)", "scale=st.scale * 2.0"),
 "omb1_in_fp64": ("omb1=np.float32(np.float32(1.0) - b1),", "omb1=np.float32(1.0 - float(hp.beta1)),"),
 "bc_off_corrected": ("        c[\"step_size\"] = lr\n",
                      "        c[\"step_size\"] = np.float32(float(lr) / (1.0 - beta1_pow * float(b1)))\n"),
 "skip_writes_params": ("        return master, m, v, None, scaler_update(state, 1, hp.beta1, hp.beta2), sc",
                        "        return master, m, v, narrow(master, pdtype), scaler_update(state, 1, hp.beta1, hp.beta2), sc"),
 "params_from_perturbed_master": ("    p16 = narrow(master, pdtype)\n", "    p16 = narrow(master * np.float32(1.0000001), pdtype)\n"),
 "reduce_rounds_each_add": ("        acc = acc + widen(sl, src_dtype)\n",
                            "        acc = widen(narrow(acc + widen(sl, src_dtype), src_dtype), src_dtype)\n"),
 "consolidate_gap_ok": ("        if lo != pos or hi < lo or len(a) != hi - lo:", "        if hi < lo or len(a) != hi - lo:"),
 "consolidate_short_ok": ("    if pos < total:\n", "    if pos < total - 64:\n"),
 "onebit_scale_fp32_sum": ("sumsq = math.fsum(float(v) * float(v) for v in c[a:b])", "sumsq = float(np.sum(c[a:b] * c[a:b]))"),
 "onebit_dec_peers_reversed": ("    for words, scales in payloads:\n", "    for words, scales in payloads[::-1]:\n"),
 "onebit_dec_chunk_fixed": ("    j = np.arange(n) // chunk\n", "    j = np.arange(n) // 2048\n"),
 "onebit_dec_ignore_dst": ("    return dst + acc if accumulate else acc\n", "    return acc\n"),
 "onebit_dec_word_index": ("word = 64 * (i // 2048) + (i % 256) // 4", "word = 64 * (i // 2048) + (i % 64)"),
 "onebit_dec_bit_pos": ("pos = 4 * ((i % 2048) // 256) + i % 4", "pos = 8 * (i % 4) + (i % 2048) // 256"),
}


def _pins_on_mutant(name, work):
    """Exit status and output tail of the pins run against the oracle with
    mutant `name` planted, in a copy of the test tree under `work`."""
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "zero_step.py")).read()
    if src.count(old) < 1:
        return None, "the mutated text is not in the oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), work / "oracle")
    shutil.copytree(os.path.join(ROOT, "workloads"), work / "workloads")
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), work / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), work / "tests" / "conftest.py")
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), work / "tests" / "test_oracle_pins.py")
    (work / "oracle" / "zero_step.py").write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=work, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    """Every mutant's pins run, in parallel processes (one per host core)."""
    base = tmp_path_factory.mktemp("mutants")
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        futs = {name: ex.submit(_pins_on_mutant, name, base / name) for name in sorted(MUTANTS)}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, pin_runs):
    rc, out = pin_runs[name]
    assert rc is not None, "mutant %s: %s" % (name, out)
    assert rc != 0, "mutant %s passed every pin:\n%s" % (name, out)
