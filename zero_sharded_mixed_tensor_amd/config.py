"""A DeepSpeed-style JSON configuration mapped onto the library's step settings.

The pages configure the engine with one JSON file (devpress.csdn.net DeepSpeed
tutorial §3.2 ds_config.json; jwzheng96.github.io DeepSpeed chapter 1, §1.4).
The fields that decide one rank's optimizer step are read here; the others
(scheduler, logging, communication buckets) are left to the caller:

  optimizer.type / params   AdamW (or Adam in its decoupled-decay form):
                            lr, betas, eps, weight_decay -> zds_adamw_hparams
  fp16.enabled + loss_scale 0 -> dynamic scaler with loss_scale_window,
                            initial_scale_power, hysteresis, min_loss_scale;
                            > 0 -> that static scale; fp16 params
  bf16.enabled              bf16 params, static scale 1 (no loss scaling)
  neither                   fp32 params: the step writes no 16-bit copy
  gradient_clipping         max global norm (absent or 0: no clipping)
  gradient_accumulation_steps, train_batch_size, train_micro_batch_size_per_gpu
                            K micro-batches per step; with "auto" or absent, K
                            follows from batch = micro * K * world (the
                            tutorial's §2.3 worked example), else 1
  zero_optimization.stage   0..3, reported (the rank's step is the same)
  zero_optimization.offload_optimizer.device  "cpu" -> offloaded optimizer
                            state (OffloadStep)

Readings where the pages are silent: an absent fp16 field takes the value of
the tutorial's example block (window 1000, power 16, hysteresis 2, floor 1);
an absent or "auto" optimizer parameter takes the library default (lr 1e-3,
betas 0.9 / 0.999, eps 1e-8, weight decay 0.01); fp16 and bf16 both enabled,
an optimizer other than AdamW, and batch sizes that do not multiply out are
refused (the chapter's §1.4 remarks that the fields constrain each other).
The parsing needs no GPU and no built library; `hparams()` and
`scaler_config()` build the C structs.
"""

import json
from dataclasses import dataclass
from typing import Optional


class ConfigError(ValueError):
    pass


# the tutorial's example values of the fp16 block, used for absent fields
FP16_DEFAULTS = dict(loss_scale=0, loss_scale_window=1000, initial_scale_power=16, hysteresis=2,
                     min_loss_scale=1)
ADAMW_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


@dataclass(frozen=True)
class StepConfig:
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    dynamic: bool
    initial_scale_power: int
    window: int
    hysteresis: int
    min_scale: float
    static_scale: float
    max_norm: float
    accum_steps: int
    param_dtype: Optional[str]  # "fp16", "bf16", or None (fp32 training: no 16-bit copy)
    stage: int
    offload: bool

    def hparams(self):
        from . import zds
        return zds.hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay)

    def scaler_config(self):
        from . import zds
        return zds.scaler_config(dynamic=self.dynamic, initial_scale_power=self.initial_scale_power,
                                 window=self.window, hysteresis=self.hysteresis, min_scale=self.min_scale,
                                 static_scale=self.static_scale)


def _is_auto(v):
    return v is None or (isinstance(v, str) and v.strip().lower() == "auto")


def _num(block, key, default, kind=float):
    v = block.get(key, default)
    if _is_auto(v):
        v = default
    try:
        out = kind(v)
    except (TypeError, ValueError):
        raise ConfigError("%s: expected a number, got %r" % (key, v)) from None
    if kind is int and out != v:
        raise ConfigError("%s: expected an integer, got %r" % (key, v))
    return out


def _enabled(cfg, key):
    b = cfg.get(key) or {}
    if not isinstance(b, dict):
        raise ConfigError("%s must be an object" % key)
    return bool(b.get("enabled", False)), b


def _accum_steps(cfg, world):
    gas = cfg.get("gradient_accumulation_steps")
    tb = cfg.get("train_batch_size")
    mb = cfg.get("train_micro_batch_size_per_gpu")
    known = lambda v: not _is_auto(v)  # noqa: E731
    if known(gas):
        k = _num(cfg, "gradient_accumulation_steps", 1, int)
        if k < 1:
            raise ConfigError("gradient_accumulation_steps must be >= 1")
        if known(tb) and known(mb) and int(tb) != int(mb) * k * world:
            raise ConfigError("train_batch_size %s != micro batch %s * %d steps * %d ranks" % (tb, mb, k, world))
        return k
    if known(tb) and known(mb):
        tb, mb = _num(cfg, "train_batch_size", 1, int), _num(cfg, "train_micro_batch_size_per_gpu", 1, int)
        if mb < 1 or tb % (mb * world) != 0:
            raise ConfigError("train_batch_size %d is not a multiple of micro batch %d * %d ranks" % (tb, mb, world))
        return tb // (mb * world)
    return 1


def from_ds_config(cfg, world=1):
    """StepConfig of a parsed JSON object (dict) for a job of `world` ranks."""
    if not isinstance(cfg, dict):
        raise ConfigError("the configuration must be a JSON object")
    if world < 1:
        raise ConfigError("world must be >= 1")
    # optimizer
    opt = cfg.get("optimizer") or {"type": "AdamW", "params": {}}
    typ = str(opt.get("type", "AdamW"))
    p = opt.get("params") or {}
    if typ.lower() == "adam" and p.get("adam_w_mode", True) is False and p.get("weight_decay", 0) not in (0, 0.0):
        raise ConfigError("Adam with L2-coupled weight decay is not this step's update (AdamW)")
    if typ.lower() not in ("adamw", "adam"):
        raise ConfigError("optimizer %r: the step implements AdamW" % typ)
    betas = p.get("betas", ADAMW_DEFAULTS["betas"])
    if _is_auto(betas):
        betas = ADAMW_DEFAULTS["betas"]
    if not isinstance(betas, (list, tuple)) or len(betas) != 2:
        raise ConfigError("betas must be a pair")
    b1, b2 = float(betas[0]), float(betas[1])
    if not (0.0 <= b1 < 1.0 and 0.0 <= b2 < 1.0):
        raise ConfigError("betas must lie in [0, 1)")
    lr = _num(p, "lr", ADAMW_DEFAULTS["lr"])
    eps = _num(p, "eps", ADAMW_DEFAULTS["eps"])
    wd = _num(p, "weight_decay", ADAMW_DEFAULTS["weight_decay"])
    # precision and loss scaling
    fp16, f = _enabled(cfg, "fp16")
    bf16, _ = _enabled(cfg, "bf16")
    if fp16 and bf16:
        raise ConfigError("fp16 and bf16 cannot both be enabled")
    if fp16:
        ls = _num(f, "loss_scale", FP16_DEFAULTS["loss_scale"])
        if ls < 0:
            raise ConfigError("loss_scale must be >= 0")
        dynamic = ls == 0
        power = _num(f, "initial_scale_power", FP16_DEFAULTS["initial_scale_power"], int)
        window = _num(f, "loss_scale_window", FP16_DEFAULTS["loss_scale_window"], int)
        hyst = _num(f, "hysteresis", FP16_DEFAULTS["hysteresis"], int)
        floor = _num(f, "min_loss_scale", FP16_DEFAULTS["min_loss_scale"])
        if window < 1 or hyst < 1 or floor <= 0 or not (0 <= power <= 127):
            raise ConfigError("fp16 block: window and hysteresis >= 1, min_loss_scale > 0, "
                              "initial_scale_power in [0, 127]")
        static = 1.0 if dynamic else float(ls)
        pdt = "fp16"
    else:
        dynamic, power, window, hyst, floor, static = False, 0, 1000, 1, 1.0, 1.0
        pdt = "bf16" if bf16 else None
    # clipping, accumulation, ZeRO
    max_norm = _num(cfg, "gradient_clipping", 0.0)
    if max_norm < 0:
        raise ConfigError("gradient_clipping must be >= 0")
    k = _accum_steps(cfg, world)
    z = cfg.get("zero_optimization") or {}
    stage = _num(z, "stage", 0, int)
    if not 0 <= stage <= 3:
        raise ConfigError("zero_optimization.stage must be 0..3")
    off = z.get("offload_optimizer") or {}
    offload = str(off.get("device", "none")).lower() == "cpu"
    return StepConfig(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, dynamic=dynamic,
                      initial_scale_power=power, window=window, hysteresis=hyst, min_scale=floor,
                      static_scale=static, max_norm=max_norm, accum_steps=k, param_dtype=pdt, stage=stage,
                      offload=offload)


def load_ds_config(path, world=1):
    """StepConfig of a JSON file."""
    with open(path) as f:
        return from_ds_config(json.load(f), world)
