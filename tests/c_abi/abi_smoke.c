/* A plain C caller of libgdnreplay.so: includes the public header, links the
 * library and exercises the host side of the contract (version, error
 * strings, the size of the counter buffer, synchronous argument validation).
 * Every call here is rejected or is a zero-request no-op, so nothing is
 * enqueued and no GPU is needed. Exit status 0 and "OK" on success. */
#include <stdio.h>
#include <string.h>

#include "gdn_replay.h"

static int fails = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

int main(void) {
  void *fake = (void *)(uintptr_t)0x10000; /* aligned, never dereferenced */
  const int32_t *ifake = (const int32_t *)fake;
  float *ffake = (float *)fake;

  CHECK(gdn_replay_version() == GDN_REPLAY_VERSION);
  CHECK(strlen(gdn_replay_strerror(GDN_OK)) > 0);
  CHECK(strlen(gdn_replay_strerror(GDN_EINVAL)) > 0);
  CHECK(gdn_replay_sync_entries(32, 16) == 32 * 33 + 32 * 16);
  CHECK(gdn_replay_sync_entries(-1, 16) == 0);

  gdn_replay_cache c;
  memset(&c, 0, sizeof c);
  c.num_slots = 4;
  c.num_v_heads = 4;
  c.num_k_heads = 2;
  c.d_k = 64;
  c.d_v = 64;
  c.ring_cap = 32;
  c.in_dtype = GDN_BF16;
  c.state = ffake;
  c.ring_k = c.ring_v = fake;
  c.ring_alpha = c.ring_beta = ffake;
  c.head = c.len = c.sync = c.err = (int32_t *)fake;
  c.sync_len = (int32_t)gdn_replay_sync_entries(c.num_slots, c.num_k_heads);

  /* a counter buffer declared one entry short is refused by every call */
  c.sync_len -= 1;
  CHECK(gdn_replay_verify(&c, 1, ifake, 4, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_flush(&c, 1, ifake, 1, 0) == GDN_EINVAL);
  CHECK(gdn_replay_verify_flush(&c, 1, ifake, 4, 16, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_rollback_verify_flush(&c, 1, ifake, ifake, NULL, 4, NULL, 4, 16, fake, fake,
                                         fake, ffake, ffake, ffake, 0) == GDN_EINVAL);
  c.sync_len += 1;

  /* verify: no cache, bad counts and lengths, zero requests */
  CHECK(gdn_replay_verify(NULL, 1, ifake, 4, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_verify(&c, -1, ifake, 4, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_verify(&c, 1, ifake, 33, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_verify(&c, 1, ifake, 4, fake, fake, fake, ffake, ffake, NULL, 0) ==
        GDN_EINVAL);
  CHECK(gdn_replay_verify(&c, 0, NULL, 4, NULL, NULL, NULL, NULL, NULL, NULL, 0) == GDN_OK);

  /* a head dimension that is not built */
  c.d_k = c.d_v = 48;
  CHECK(gdn_replay_verify(&c, 1, ifake, 4, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EUNSUPPORTED);
  c.d_k = c.d_v = 64;

  /* rollback, flush, the fused calls */
  CHECK(gdn_replay_rollback(&c, 2, ifake, 0, ifake, 0) == GDN_EINVAL);
  CHECK(gdn_replay_rollback(&c, 2, ifake, 4, NULL, 0) == GDN_EINVAL);
  CHECK(gdn_replay_flush(&c, -1, ifake, 1, 0) == GDN_EINVAL);
  CHECK(gdn_replay_flush(&c, 0, NULL, 1, 0) == GDN_OK);
  CHECK(gdn_replay_verify_flush(&c, 5, ifake, 4, 16, fake, fake, fake, ffake, ffake, ffake, 0) ==
        GDN_EINVAL); /* more requests than slots */
  CHECK(gdn_replay_rollback_verify_flush(&c, 2, ifake, NULL, NULL, 4, NULL, 4, 16, fake, fake,
                                         fake, ffake, ffake, ffake, 0) == GDN_EINVAL);
  CHECK(gdn_replay_rollback_verify_flush(&c, 2, ifake, ifake, NULL, 0, NULL, 4, 16, fake, fake,
                                         fake, ffake, ffake, ffake, 0) == GDN_EINVAL);

  /* the step with the norm: eps out of range, a missing norm, a shape the
   * one-kernel path does not take */
  gdn_norm_fp8 n = {fake, ffake, 0.0f, (uint8_t *)fake, ffake};
  CHECK(gdn_replay_step_norm_fp8(&c, 2, ifake, ifake, NULL, 4, NULL, 4, 16, fake, fake, fake,
                                 ffake, ffake, NULL, &n, 0) == GDN_EINVAL);
  n.eps = 1e-6f;
  CHECK(gdn_replay_step_norm_fp8(&c, 2, ifake, ifake, NULL, 4, NULL, 4, 16, fake, fake, fake,
                                 ffake, ffake, NULL, NULL, 0) == GDN_EINVAL);
  c.ring_cap = 40;
  CHECK(gdn_replay_step_norm_fp8(&c, 2, ifake, ifake, NULL, 4, NULL, 4, 16, fake, fake, fake,
                                 ffake, ffake, NULL, &n, 0) == GDN_EUNSUPPORTED);
  c.ring_cap = 32;
  CHECK(gdn_replay_step_norm_fp8(&c, 0, NULL, NULL, NULL, 4, NULL, 4, 16, NULL, NULL, NULL, NULL,
                                 NULL, NULL, &n, 0) == GDN_OK);

  /* the norm and the convolution on their own */
  CHECK(gdn_gated_rmsnorm_fp8(4, 2, 24, ffake, fake, ffake, 1e-6f, (uint8_t *)fake, ffake, 0) ==
        GDN_EUNSUPPORTED);
  CHECK(gdn_gated_rmsnorm_fp8(0, 2, 128, NULL, NULL, NULL, 1e-6f, NULL, NULL, 0) == GDN_OK);
  CHECK(gdn_causal_conv_update(&c, fake, 3, 4, 2, ifake, NULL, NULL, 0, 4, fake, ffake, NULL,
                               fake, 0) == GDN_EINVAL); /* odd channel count */
  CHECK(gdn_causal_conv_update(&c, fake, 4, 4, 2, ifake, ifake, NULL, 0, 4, fake, ffake, NULL,
                               fake, 0) == GDN_EINVAL); /* pending rollback without its length */

  printf("%s\n", fails ? "FAILED" : "OK");
  return fails != 0;
}
