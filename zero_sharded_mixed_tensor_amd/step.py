"""Sequencing of one rank's optimizer step over the C ABI.

engine.backward's gradient handling -> zds_grad_accumulate per micro-batch;
engine.step -> zds_overflow_and_norm, zds_adam_step, zds_loss_scaler_update,
all on one stream with no host synchronisation (devpress.csdn.net DeepSpeed
tutorial §3.3: the engine's backward and step replace the plain ones).
"""

from . import zds


class ShardStep:
    """Device buffers of one rank's step: the 64-byte step state, the 64-byte
    per-step scalars and the norm workspace, plus the step's settings."""

    def __init__(self, n, hp=None, scaler=None, max_norm=1.0, accum_steps=1, t0=0,
                 beta1_pow0=1.0, beta2_pow0=1.0, device="cuda", stream=None):
        self.n = n
        self.hp = hp if hp is not None else zds.hparams()
        self.cfg = scaler if scaler is not None else zds.scaler_config()
        self.max_norm = max_norm
        self.accum_steps = accum_steps
        self.state = zds.new_state(device)
        self.scalars = zds.new_scalars(device)
        self.ws = zds.new_workspace(n, device)
        zds.zds_step_state_init(self.state, self.cfg, t0, beta1_pow0, beta2_pow0, stream)

    def accumulate_norm(self, plan, srcs, dst, mode, ws, stream=None):
        """The step's last micro-batch with the overflow/norm pass fused in."""
        zds.zds_grad_accumulate_norm(plan, srcs, dst, mode, self.accum_steps, self.max_norm, self.state,
                                     self.scalars, ws, stream)

    def norm(self, grads, stream=None):
        zds.zds_overflow_and_norm(grads, self.accum_steps, self.max_norm, self.state, self.scalars,
                                  self.ws, stream, n=self.n)

    def adam(self, grads, master, exp_avg, exp_avg_sq, params_out, stream=None):
        zds.zds_adam_step(self.hp, grads, master, exp_avg, exp_avg_sq, params_out, self.scalars,
                          self.state, stream, n=self.n)

    def scaler(self, stream=None):
        zds.zds_loss_scaler_update(self.state, self.scalars, self.hp, stream)

    def step(self, grads, master, exp_avg, exp_avg_sq, params_out, stream=None):
        self.norm(grads, stream)
        self.adam(grads, master, exp_avg, exp_avg_sq, params_out, stream)
        self.scaler(stream)

    def read_state(self):
        return zds.read_state(self.state)

    def read_scalars(self):
        return zds.read_scalars(self.scalars)
