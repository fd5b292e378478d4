/* A plain C caller of the libmoe C ABI.  It makes only calls that return
 * before any GPU work: sizes, status strings, argument validation, and a
 * zero-token forward (a no-op).  Prints "ok" and exits 0 when every result is
 * as include/libmoe.h documents. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libmoe.h"

static int failures = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                \
    }                                                            \
  } while (0)

int main(void) {
  moe_problem_t p;
  memset(&p, 0, sizeof p);
  p.tokens = 4096;
  p.dim = 4096;
  p.hidden = 14336;
  p.n_experts = 8;
  p.top_k = 2;
  p.out_dtype = MOE_F32;
  p.path = MOE_PATH_AUTO;

  /* capacity: T*K + n*(MOE_TILE_M-1), rounded up to MOE_TILE_M */
  const int64_t cap = moe_capacity_rows(&p);
  CHECK(cap == (8192 + 8 * (MOE_TILE_M - 1) + MOE_TILE_M - 1) / MOE_TILE_M * MOE_TILE_M);
  const size_t ws = moe_workspace_bytes(&p);
  CHECK(ws >= (size_t)cap * 14336 * 2);
  CHECK(moe_decode_max_tokens() >= 16);
  CHECK(strcmp(moe_status_string(MOE_OK), moe_status_string(MOE_EINVAL)) != 0);
  CHECK(strcmp(moe_status_string(99), "unknown status") == 0);

  /* invalid problems: size 0, capacity -1 */
  moe_problem_t bad = p;
  bad.top_k = 9;
  CHECK(moe_workspace_bytes(&bad) == 0);
  CHECK(moe_capacity_rows(&bad) == -1);
  bad = p;
  bad.dim = 4100;
  CHECK(moe_workspace_bytes(&bad) == 0);

  /* validation happens before any enqueue; a fake, aligned device address
   * is never dereferenced on these paths */
  void* fake = (void*)(uintptr_t)0x100000;
  CHECK(moe_forward(&bad, fake, fake, fake, fake, fake, fake, NULL, NULL, fake, ws, NULL) ==
        MOE_EINVAL);
  CHECK(moe_forward(&p, fake, fake, fake, fake, fake, fake, NULL, NULL, NULL, ws, NULL) ==
        MOE_EWORKSPACE);
  CHECK(moe_forward(NULL, fake, fake, fake, fake, fake, fake, NULL, NULL, fake, ws, NULL) ==
        MOE_EINVAL);

  /* every enqueueing entry point: bad problems, null or misaligned pointers
   * and missing workspaces are refused before anything is enqueued */
  void* odd = (void*)(uintptr_t)0x100004;
  int32_t* fi = (int32_t*)fake;
  float* ff = (float*)fake;
  CHECK(moe_route_workspace_bytes(&bad) == 0);
  CHECK(moe_route(&bad, fake, fake, fi, ff, NULL, NULL, 0, NULL) == MOE_EINVAL);
  CHECK(moe_route(&p, NULL, fake, fi, ff, NULL, NULL, 0, NULL) == MOE_EINVAL);
  CHECK(moe_route(&p, odd, fake, fi, ff, NULL, NULL, 0, NULL) == MOE_EINVAL);
  /* the slice-wise router (here: 160 experts) takes its partial sums from ws */
  moe_problem_t many = p;
  many.n_experts = 160;
  many.top_k = 8;
  CHECK(moe_route_workspace_bytes(&many) > 0);
  CHECK(moe_route(&many, fake, fake, fi, ff, NULL, NULL, 0, NULL) == MOE_EWORKSPACE);
  CHECK(moe_permute(&p, NULL, fi, fi, fi, fi, NULL) == MOE_EINVAL);
  CHECK(moe_permute(&bad, fi, fi, fi, fi, fi, NULL) == MOE_EINVAL);
  CHECK(moe_grouped_ffn(&p, fake, fi, fi, fi, fake, fake, fake, ff, NULL, 0, NULL) ==
        MOE_EWORKSPACE);
  CHECK(moe_grouped_ffn(&p, fake, fi, fi, fi, odd, fake, fake, ff, fake, ws, NULL) ==
        MOE_EINVAL);
  CHECK(moe_combine(&p, NULL, fi, ff, fake, NULL) == MOE_EINVAL);
  CHECK(moe_combine(&bad, ff, fi, ff, fake, NULL) == MOE_EINVAL);
  CHECK(moe_route_stats(&p, fi, NULL, NULL) == MOE_EINVAL);
  CHECK(moe_forward_timed(&bad, fake, fake, fake, fake, fake, fake, NULL, NULL, fake, ws, NULL,
                          NULL) == MOE_EINVAL);
  /* the allocation-free form serves the streaming batches only */
  CHECK(moe_forward_noalloc(&p, fake, fake, fake, fake, fake, fake, NULL, NULL, NULL) ==
        MOE_ENOTSUP);
  CHECK(moe_forward_noalloc(&p, NULL, fake, fake, fake, fake, fake, NULL, NULL, NULL) ==
        MOE_EINVAL);
  CHECK(strcmp(moe_status_string(MOE_EHIP), "unknown status") != 0);

  /* zero tokens: MOE_OK and nothing is enqueued */
  moe_problem_t empty = p;
  empty.tokens = 0;
  CHECK(moe_forward(&empty, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        MOE_OK);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
