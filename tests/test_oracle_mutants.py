"""Pin strength: plant plausible mistakes in a copy of the oracle (on the CPU)
and check that the oracle pins reject every one of them."""

import os
import shutil
import subprocess
import sys

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
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "zero_step.py")).read()
    assert src.count(old) >= 1, name
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "workloads"), tmp_path / "workloads")
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), tmp_path / "tests" / "conftest.py")
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), tmp_path / "tests" / "test_oracle_pins.py")
    (tmp_path / "oracle" / "zero_step.py").write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, "mutant %s passed every pin:\n%s" % (name, r.stdout[-2000:])
