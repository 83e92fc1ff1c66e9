/* Plain-C use of the KDA C ABI: compiled against include/kda.h alone and
 * linked against libkda.so.  Every call here returns from argument checks,
 * so the program runs without a GPU.  Exit status 0 on success. */
#include <stdio.h>
#include <stdint.h>
#include "kda.h"

#define CHECK(expr, want)                                                     \
  do {                                                                        \
    int got_ = (expr);                                                        \
    if (got_ != (want)) {                                                     \
      fprintf(stderr, "%s: got %d want %d (%s)\n", #expr, got_, (want),      \
              kda_status_string(got_));                                       \
      return 1;                                                               \
    }                                                                         \
  } while (0)

int main(void) {
  void* p = (void*)(uintptr_t)64;          /* aligned stand-in, never dereferenced */
  void* odd = (void*)(uintptr_t)66;
  if (kda_version() < 10000) return 1;
  CHECK(kda_chunk_fwd(NULL, p, p, p, p, NULL, p, NULL, 1, 64, 1, 128, 128, KDA_BF16, NULL, 0, NULL), KDA_ERR_NULL);
  CHECK(kda_chunk_fwd(p, p, p, p, p, NULL, p, NULL, 1, 64, 1, 96, 96, KDA_BF16, NULL, 0, NULL), KDA_ERR_SHAPE);
  CHECK(kda_chunk_fwd(odd, p, p, p, p, NULL, p, NULL, 1, 64, 1, 128, 128, KDA_BF16, NULL, 0, NULL), KDA_ERR_ALIGN);
  CHECK(kda_chunk_fwd(p, p, p, p, p, NULL, p, NULL, 0, 64, 1, 128, 128, KDA_BF16, NULL, 0, NULL), KDA_OK);
  CHECK(kda_chunk_fwd_ex(p, p, p, p, NULL, NULL, p, NULL, 1, 64, 1, 128, 128, KDA_BF16, KDA_GATE_SCALAR, NULL, 0,
                         NULL), KDA_ERR_NULL);
  CHECK(kda_chunk_fwd_ex(p, p, p, p, p, NULL, p, NULL, 1, 64, 1, 64, 64, KDA_BF16, KDA_NO_DELTA, NULL, 0, NULL),
        KDA_ERR_ARG);
  CHECK(kda_chunk_fwd_noalloc(p, p, p, NULL, p, NULL, p, NULL, 1, 64, 1, 128, 128, KDA_BF16, NULL), KDA_ERR_NULL);
  CHECK(kda_chunk_fwd_noalloc(p, p, p, p, p, NULL, p, NULL, 0, 64, 1, 128, 128, KDA_BF16, NULL), KDA_OK);
  CHECK(kda_recurrent_step(p, p, p, p, p, NULL, p, 4, 2, 128, 128, KDA_BF16, NULL), KDA_ERR_NULL);
  CHECK(kda_recurrent_step_ex(p, p, p, p, p, p, p, 4, 2, 128, 128, KDA_BF16, 8, NULL), KDA_ERR_ARG);
  CHECK(kda_chunk_fwd_varlen(p, p, p, p, p, NULL, p, NULL, NULL, NULL, 3, 100, 2, 128, 128, KDA_BF16, 0, NULL),
        KDA_ERR_NULL);
  CHECK(kda_varlen_schedule(p, 16385, 100, p, NULL), KDA_ERR_SHAPE);
  CHECK(kda_chunk_bwd(p, p, p, p, p, NULL, p, NULL, p, p, p, p, p, NULL, 1, 64, 1, 64, 64, KDA_BF16, NULL, 0, NULL),
        KDA_ERR_WORKSPACE);   /* d = 64: the token-recurrence backward, workspace missing */
  CHECK(kda_chunk_bwd(p, p, p, p, p, NULL, p, NULL, p, p, p, p, p, NULL, 1, 64, 1, 128, 128, KDA_BF16, NULL, 0, NULL),
        KDA_ERR_WORKSPACE);
  if (kda_chunk_bwd_workspace_size(1, 64, 1, 128, 128, KDA_BF16) != (size_t)131840)
    return 1;
  CHECK(kda_chunk_bwd_ex(p, p, p, p, NULL, NULL, p, NULL, p, p, p, p, NULL, NULL, 1, 64, 1, 128, 128, KDA_BF16,
                         KDA_NO_DELTA, NULL, 0, NULL), KDA_ERR_WORKSPACE);
  CHECK(kda_chunk_bwd_ex(p, p, p, p, p, NULL, p, NULL, p, p, p, p, p, NULL, 1, 64, 1, 128, 128, KDA_BF16,
                         8, NULL, 0, NULL), KDA_ERR_ARG);
  CHECK(kda_chunk_bwd_ex(p, p, p, p, p, NULL, p, NULL, p, p, p, p, p, NULL, 1, 64, 1, 128, 128, KDA_BF16,
                         KDA_STATES_SAVED, NULL, 0, NULL), KDA_ERR_WORKSPACE);
  CHECK(kda_chunk_fwd_save(p, p, p, p, p, NULL, p, NULL, 1, 64, 1, 64, 64, KDA_BF16, 0, NULL, 0, NULL),
        KDA_ERR_ARG);
  CHECK(kda_chunk_bwd_ex(p, p, p, odd, p, NULL, p, NULL, p, p, p, odd, p, NULL, 1, 64, 1, 128, 128, KDA_BF16,
                         KDA_GATE_SCALAR, NULL, 0, NULL), KDA_ERR_WORKSPACE);
  if (kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, KDA_BF16, KDA_GATE_SCALAR) !=
      (size_t)131840 + (size_t)64 * 128 * 6)
    return 1;
  CHECK(kda_chunk_bwd_varlen(p, p, p, p, p, NULL, p, NULL, p, p, p, p, p, NULL, NULL, 2, 100, 1, 128, 128,
                             KDA_BF16, 0, NULL, 0, NULL), KDA_ERR_NULL);
  CHECK(kda_chunk_bwd_varlen(p, p, p, p, NULL, NULL, p, NULL, p, p, p, p, NULL, NULL, p, 2, 100, 1, 128, 128,
                             KDA_BF16, KDA_NO_DELTA, NULL, 0, NULL), KDA_ERR_WORKSPACE);
  if (kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, KDA_BF16, 0) != (size_t)3 * 131840)
    return 1;
  printf("kda C ABI ok (version %d)\n", kda_version());
  return 0;
}
