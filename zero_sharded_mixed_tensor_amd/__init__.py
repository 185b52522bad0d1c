"""ZeRO-sharded mixed-precision optimizer step for AMD MI355X (gfx950).

One data-parallel rank's share of the ZeRO optimizer step, as hand-written
HIP kernels behind the C ABI in include/zds.h. `zds` is the ctypes binding
(same function names as the C ABI); `step` sequences the calls of one
optimizer step; `config` maps a DeepSpeed-style JSON configuration onto the
step's settings. The library is built in-tree by `build.build()`; importing
`zds` fails loudly if it has not been built.
"""

__all__ = ["zds", "step", "config", "build"]
