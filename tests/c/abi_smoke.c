/* C99 client of include/zds.h: compiles without C++, links against
 * libzds.so and calls the entry points that need no GPU (geometry, host
 * twins of the scaler and step constants, clip arithmetic, a host-memory
 * checkpoint round trip). Prints "ok" and exits 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zds.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "failed: %s (%s)\n", #cond, zds_last_error());     \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(int argc, char **argv) {
  const char *dir = argc > 1 ? argv[1] : ".";
  CHECK(zds_abi_version() == ZDS_ABI_VERSION);

  /* three tensors, align 64: offsets 0, 64, 192; total 256 */
  const int64_t numel[3] = {10, 100, 1};
  int64_t offs[3], total = 0;
  CHECK(zds_flat_layout(numel, 3, 64, offs, &total) == ZDS_OK);
  CHECK(offs[0] == 0 && offs[1] == 64 && offs[2] == 192 && total == 256);
  int64_t lo = 0, hi = 0;
  CHECK(zds_shard_range(total, 2, 1, 64, &lo, &hi) == ZDS_OK);
  CHECK(lo == 128 && hi == 256);
  int64_t ent[8];
  int32_t count = 0;
  CHECK(zds_shard_entries(numel, 3, 64, lo, hi, ent, 2, &count) == ZDS_OK && count == 2);
  CHECK(ent[0] == 1 && ent[1] == 64 && ent[2] == 36 && ent[3] == 0);
  CHECK(ent[4] == 2 && ent[5] == 0 && ent[6] == 1 && ent[7] == 64);

  /* scaler: dynamic from 2^4, window 2; overflow halves, two clean steps double */
  zds_scaler_config cfg = {1, 4, 2, 1, 1.0f, 1.0f};
  zds_step_state st;
  CHECK(zds_step_state_init_host(&st, &cfg, 0, 1.0, 1.0) == ZDS_OK && st.scale == 16.0f);
  zds_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f};
  CHECK(zds_loss_scaler_update_host(&st, 1, &hp) == ZDS_OK && st.scale == 8.0f && st.t == 0);
  CHECK(zds_loss_scaler_update_host(&st, 0, &hp) == ZDS_OK && st.t == 1);
  CHECK(zds_loss_scaler_update_host(&st, 0, &hp) == ZDS_OK && st.scale == 16.0f && st.t == 2);

  /* step constants after two applied steps */
  float c5[5];
  CHECK(zds_adam_constants_host(&hp, &st, c5) == ZDS_OK);
  CHECK(c5[2] == (float)(1.0 - (double)1e-3f * (double)0.01f));

  /* clip: sumsq 400 at scale 4, K 1 -> norm 5, coef 1/(5 + 1e-6) */
  zds_step_scalars sc;
  CHECK(zds_clip_scalars_host(400.0, 4.0f, 1, 1.0f, &sc) == ZDS_OK);
  CHECK(sc.overflow == 0 && fabs(sc.norm - 5.0) < 1e-12);

  /* errors come back as statuses with a message */
  CHECK(zds_flat_layout(numel, 3, 0, offs, &total) == ZDS_EINVAL && strlen(zds_last_error()) > 0);
  CHECK(strcmp(zds_status_string(ZDS_EIO), "file error") == 0);

  /* checkpoint of rank 1's shard from host memory, then consolidation */
  zds_checkpoint_meta m0 = {2, 0, 64, 1, 1, 3, 256, 0, 128};
  zds_checkpoint_meta m1 = {2, 1, 64, 1, 1, 3, 256, 128, 256};
  float a[3][128], b[3][128];
  for (int k = 0; k < 3; ++k)
    for (int i = 0; i < 128; ++i) a[k][i] = (float)(1000 * k + i);
  char p0[4096], p1[4096];
  snprintf(p0, sizeof p0, "%s/c_rank0.zckpt", dir);
  snprintf(p1, sizeof p1, "%s/c_rank1.zckpt", dir);
  CHECK(zds_checkpoint_save(p0, &m0, numel, a[0], a[1], a[2], &st, ZDS_ON_HOST, NULL) == ZDS_OK);
  CHECK(zds_checkpoint_save(p1, &m1, numel, a[0], a[1], a[2], &st, ZDS_ON_HOST, NULL) == ZDS_OK);
  zds_step_state st2;
  CHECK(zds_checkpoint_load(p1, &m1, numel, b[0], b[1], b[2], &st2, ZDS_ON_HOST, NULL) == ZDS_OK);
  CHECK(memcmp(a, b, sizeof a) == 0 && memcmp(&st, &st2, sizeof st) == 0);
  CHECK(zds_checkpoint_load(p0, &m1, numel, b[0], b[1], b[2], &st2, ZDS_ON_HOST, NULL) == ZDS_EINVAL);
  const char *paths[2] = {p1, p0};
  float full[111];
  CHECK(zds_consolidate_fp32(paths, 2, 0, full, 111) == ZDS_OK);
  /* tensor 0 = rank 0 [0, 10); tensor 1 = rank 0 [64, 128) + rank 1 [0, 36); tensor 2 = rank 1 [64] */
  CHECK(full[0] == 0.0f && full[9] == 9.0f && full[10] == 64.0f && full[73] == 127.0f && full[74] == 0.0f);
  CHECK(full[109] == 35.0f && full[110] == 64.0f);
  remove(p0);
  remove(p1);
  printf("ok\n");
  return 0;
}
