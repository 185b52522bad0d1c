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
        # (positional order is relied on by OffloadStep)
        self.n = n
        self.hp = hp if hp is not None else zds.hparams()
        self.cfg = scaler if scaler is not None else zds.scaler_config()
        self.max_norm = max_norm
        self.accum_steps = accum_steps
        self.state = zds.new_state(device)
        self.scalars = zds.new_scalars(device)
        self.ws = zds.new_workspace(n, device)
        zds.zds_step_state_init(self.state, self.cfg, t0, beta1_pow0, beta2_pow0, stream)

    @classmethod
    def from_config(cls, n, cfg, t0=0, beta1_pow0=1.0, beta2_pow0=1.0, device="cuda", stream=None):
        """A step with the settings of a config.StepConfig (hyperparameters,
        loss scaler, clip threshold, micro-batches per step)."""
        return cls(n, cfg.hparams(), cfg.scaler_config(), cfg.max_norm, cfg.accum_steps, t0, beta1_pow0,
                   beta2_pow0, device, stream)

    def accumulate_norm(self, plan, srcs, dst, mode, ws, stream=None):
        """The step's last micro-batch with the overflow/norm pass fused in."""
        zds.zds_grad_accumulate_norm(plan, srcs, dst, mode, self.accum_steps, self.max_norm, self.state,
                                     self.scalars, ws, stream)

    def intake_norm(self, peers, dst, mode, ws, stream=None):
        """The Stage-2 intake of the peers' slices with the overflow/norm
        pass fused in."""
        zds.zds_reduce_peer_slices_norm(peers, dst, mode, self.accum_steps, self.max_norm, self.state,
                                        self.scalars, ws, stream, n=self.n)

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

    def capture(self, plan, srcs, dst, mode, ws, master, exp_avg, exp_avg_sq, params_out):
        """Records one whole step (the flatten/accumulate call with the norm
        fused in, AdamW, the scaler) into a HIP graph and returns it;
        graph.replay() then runs a step with one launch from the host. The
        graph reads the grads from srcs' addresses and writes the same
        buffers on every replay: refill the grads in place between replays.
        Nothing but kernels is captured (no memset, copy or event)."""
        import torch
        bound = srcs if isinstance(srcs, zds.SourceSet) else zds.SourceSet(plan, srcs)
        # upload the source pointers in an eager call into a scratch buffer
        # (the step's own buffers are left alone), and let it complete
        scratch = torch.empty_like(dst)
        zds.zds_grad_accumulate(plan, bound, scratch, zds.ZDS_COPY if mode == zds.ZDS_COPY else zds.ZDS_OVERWRITE)
        torch.cuda.synchronize()
        del scratch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.accumulate_norm(plan, bound, dst, mode, ws)
            self.adam(dst, master, exp_avg, exp_avg_sq, params_out)
            self.scaler()
        graph.bound_sources = bound  # keeps the grads' storages alive with the graph
        return graph

    def read_state(self):
        return zds.read_state(self.state)

    def read_scalars(self):
        return zds.read_scalars(self.scalars)


class OffloadStep:
    """A rank whose fp32 optimizer shard lives in pinned host memory
    (ZeRO-Offload): the grads' overflow/norm pass runs on the device, the
    grads stream to the host in chunks, the host updates each chunk as soon
    as it has arrived (zds_cpu_adam_step) and streams its 16-bit params
    back, so downloads, the host update and uploads overlap; the loss scaler
    then runs on the device state.

    master, exp_avg, exp_avg_sq: pinned host fp32 tensors (n elements)."""

    def __init__(self, n, master, exp_avg, exp_avg_sq, grad_dtype, param_dtype, hp=None, scaler=None,
                 max_norm=1.0, accum_steps=1, t0=0, beta1_pow0=1.0, beta2_pow0=1.0, chunk=1 << 25,
                 threads=0, device="cuda"):
        import torch
        self.torch = torch
        self.dev = ShardStep(n, hp, scaler, max_norm, accum_steps, t0, beta1_pow0, beta2_pow0, device)
        self.n = n
        self.master, self.m, self.v = master, exp_avg, exp_avg_sq
        self.gh = torch.empty(n, dtype=grad_dtype, pin_memory=True)
        self.ph = torch.empty(n, dtype=param_dtype, pin_memory=True)
        self.sc_h = torch.empty(zds.SCALARS_BYTES, dtype=torch.uint8, pin_memory=True)
        self.st_h = torch.empty(zds.STATE_BYTES, dtype=torch.uint8, pin_memory=True)
        self.chunk = chunk
        self.threads = threads
        self.down = torch.cuda.Stream(device)
        self.up = torch.cuda.Stream(device)

    def step(self, grads, params_out):
        """grads: device gradient shard (n elements); params_out: device
        16-bit params (n elements), written."""
        torch = self.torch
        d = self.dev
        cur = torch.cuda.current_stream()
        self.up.wait_stream(cur)  # earlier readers of params_out come first
        d.norm(grads)
        ready = torch.cuda.Event()
        ready.record(cur)
        # downloads: the scalars/state first, then the grads chunk by chunk
        self.down.wait_event(ready)
        evs = []
        with torch.cuda.stream(self.down):
            self.sc_h.copy_(d.scalars, non_blocking=True)
            self.st_h.copy_(d.state, non_blocking=True)
            for a in range(0, self.n, self.chunk):
                b = min(self.n, a + self.chunk)
                self.gh[a:b].copy_(grads[a:b], non_blocking=True)
                e = torch.cuda.Event()
                e.record(self.down)
                evs.append((a, b, e))
        if evs:
            evs[0][2].synchronize()
        else:
            self.down.synchronize()
        sc = zds.StepScalars.from_buffer_copy(self.sc_h.numpy().tobytes())
        st = zds.StepState.from_buffer_copy(self.st_h.numpy().tobytes())
        last_up = None
        for a, b, e in evs:
            e.synchronize()
            zds.zds_cpu_adam_step(d.hp, self.gh[a:b], self.master[a:b], self.m[a:b], self.v[a:b],
                                  self.ph[a:b], sc, st, num_threads=self.threads)
            if sc.overflow:
                continue
            with torch.cuda.stream(self.up):
                params_out[a:b].copy_(self.ph[a:b], non_blocking=True)
                last_up = torch.cuda.Event()
                last_up.record(self.up)
        if last_up is not None:
            cur.wait_event(last_up)
        d.scaler()
        return sc
