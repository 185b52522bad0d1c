"""The JSON configuration mapping (no GPU): the pages' example blocks, the
batch-size arithmetic of the tutorial's worked example, defaults, refusals."""

import json

import pytest

from zero_sharded_mixed_tensor_amd.config import ConfigError, from_ds_config, load_ds_config

# the fields and values of the tutorial's ds_config.json (§3.2), as JSON
TUTORIAL = {
    "train_batch_size": "auto",
    "train_micro_batch_size_per_gpu": 4,
    "gradient_accumulation_steps": "auto",
    "zero_optimization": {"stage": 2, "allgather_partitions": True, "allgather_bucket_size": 2e8,
                          "overlap_comm": True, "reduce_scatter": True, "reduce_bucket_size": 2e8,
                          "contiguous_gradients": True},
    "fp16": {"enabled": True, "loss_scale": 0, "loss_scale_window": 1000, "initial_scale_power": 16,
             "hysteresis": 2, "min_loss_scale": 1},
    "optimizer": {"type": "AdamW", "params": {"lr": 2e-5, "betas": [0.9, 0.999], "eps": 1e-8,
                                              "weight_decay": 0.01}},
    "scheduler": {"type": "WarmupLR", "params": {"warmup_min_lr": 0, "warmup_max_lr": 2e-5,
                                                 "warmup_num_steps": 1000}},
    "steps_per_print": 10,
    "wall_clock_breakdown": False,
}

# the chapter's typical config (§1.4)
CHAPTER = {
    "train_batch_size": 256,
    "gradient_accumulation_steps": 4,
    "bf16": {"enabled": True},
    "zero_optimization": {"stage": 3, "offload_optimizer": {"device": "cpu"}, "overlap_comm": True},
}


def test_tutorial_block():
    c = from_ds_config(TUTORIAL, world=4)
    assert (c.lr, c.beta1, c.beta2, c.eps, c.weight_decay) == (2e-5, 0.9, 0.999, 1e-8, 0.01)
    assert c.dynamic and c.initial_scale_power == 16 and c.window == 1000 and c.hysteresis == 2
    assert c.min_scale == 1.0 and c.param_dtype == "fp16"
    assert c.stage == 2 and not c.offload and c.accum_steps == 1 and c.max_norm == 0.0


def test_chapter_block():
    c = from_ds_config(CHAPTER, world=8)
    assert c.param_dtype == "bf16" and not c.dynamic and c.static_scale == 1.0
    assert c.accum_steps == 4 and c.stage == 3 and c.offload


def test_worked_accumulation_example():
    # target batch 256 on 4 GPUs with 4 samples per micro-batch: 16 steps
    cfg = {"train_batch_size": 256, "train_micro_batch_size_per_gpu": 4, "gradient_accumulation_steps": "auto"}
    assert from_ds_config(cfg, world=4).accum_steps == 16
    # 64 steps on the same setup make a batch of 1024, not 256
    cfg["gradient_accumulation_steps"] = 64
    with pytest.raises(ConfigError):
        from_ds_config(cfg, world=4)
    cfg["train_batch_size"] = 1024
    assert from_ds_config(cfg, world=4).accum_steps == 64
    with pytest.raises(ConfigError):
        from_ds_config({"train_batch_size": 250, "train_micro_batch_size_per_gpu": 4}, world=4)


def test_defaults_and_auto():
    c = from_ds_config({})
    assert (c.lr, c.beta1, c.beta2, c.eps, c.weight_decay) == (1e-3, 0.9, 0.999, 1e-8, 0.01)
    assert c.param_dtype is None and not c.dynamic and c.static_scale == 1.0 and c.accum_steps == 1
    c = from_ds_config({"optimizer": {"type": "AdamW", "params": {"lr": "auto", "betas": "auto"}},
                        "fp16": {"enabled": True}})
    assert c.lr == 1e-3 and (c.beta1, c.beta2) == (0.9, 0.999)
    # absent fp16 fields: the tutorial's example values
    assert c.dynamic and c.window == 1000 and c.initial_scale_power == 16 and c.hysteresis == 2
    c = from_ds_config({"fp16": {"enabled": True, "loss_scale": 128}, "gradient_clipping": 1.0})
    assert not c.dynamic and c.static_scale == 128.0 and c.max_norm == 1.0


@pytest.mark.parametrize("cfg", [
    {"fp16": {"enabled": True}, "bf16": {"enabled": True}},
    {"optimizer": {"type": "SGD", "params": {"lr": 0.1}}},
    {"optimizer": {"type": "Adam", "params": {"adam_w_mode": False, "weight_decay": 0.1}}},
    {"optimizer": {"type": "AdamW", "params": {"betas": [0.9]}}},
    {"fp16": {"enabled": True, "loss_scale_window": 0}},
    {"fp16": {"enabled": True, "initial_scale_power": 200}},
    {"gradient_clipping": -1.0},
    {"gradient_accumulation_steps": 0},
    {"zero_optimization": {"stage": 4}},
    [],
])
def test_refusals(cfg):
    with pytest.raises(ConfigError):
        from_ds_config(cfg)


def test_adam_in_decoupled_form_is_accepted():
    c = from_ds_config({"optimizer": {"type": "Adam", "params": {"lr": 3e-4, "weight_decay": 0.1}}})
    assert c.lr == 3e-4 and c.weight_decay == 0.1


def test_file_and_structs(tmp_path):
    path = tmp_path / "ds_config.json"
    path.write_text(json.dumps(TUTORIAL))
    c = load_ds_config(str(path), world=2)
    hp, sc = c.hparams(), c.scaler_config()
    assert abs(hp.lr - 2e-5) < 1e-12 and abs(hp.beta2 - 0.999) < 1e-7 and abs(hp.weight_decay - 0.01) < 1e-9
    assert sc.dynamic == 1 and sc.initial_scale_power == 16 and sc.window == 1000 and sc.hysteresis == 2
    assert sc.min_scale == 1.0
