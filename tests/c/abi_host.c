/* Plain C99 client of libkda's C ABI (include/kda.h), host side only: the library loads and
 * links, reports its ABI version and status names, sizes a workspace, and rejects bad
 * arguments on the host before touching a device. No pointer passed here is dereferenced:
 * every call below fails validation or only inspects shapes. Prints "ok" and returns 0 on
 * success; any mismatch prints what differed and returns 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

#define EXPECT(cond, ...)                 \
  do {                                    \
    if (!(cond)) {                        \
      printf("FAIL line %d: ", __LINE__); \
      printf(__VA_ARGS__);                \
      printf("\n");                       \
      ++failures;                         \
    }                                     \
  } while (0)

static kda_chunk_args base_args(void) {
  /* B=1, T=256, H=4, dk=dv=128, chunk 64, bf16 in, fp32 out; disjoint fake device ranges */
  kda_chunk_args a;
  const uintptr_t fake = (uintptr_t)1 << 40, tok = 256u * 4u;
  memset(&a, 0, sizeof a);
  a.B = 1; a.T = 256; a.H = 4; a.dk = 128; a.dv = 128; a.chunk = 64;
  a.act_dtype = KDA_BF16; a.gate_dtype = KDA_BF16; a.out_dtype = KDA_F32;
  a.q = (const void*)fake;
  a.k = (const void*)(fake + tok * 128 * 2);
  a.v = (const void*)(fake + 2 * tok * 128 * 2);
  a.g = (const void*)(fake + 3 * tok * 128 * 2);
  a.beta = (const void*)(fake + 4 * tok * 128 * 2);
  a.o = (void*)(fake + ((uintptr_t)1 << 30));
  return a;
}

int main(void) {
  EXPECT(kda_abi_version() == KDA_ABI_VERSION, "abi %d vs header %d", kda_abi_version(),
         KDA_ABI_VERSION);
  EXPECT(strcmp(kda_status_string(KDA_ERR_ALIAS), "KDA_ERR_ALIAS") == 0, "status string");

  /* workspace: 4 heads (composed steps): one 163,840-byte block per 128 tokens and head */
  kda_chunk_args a = base_args();
  size_t bytes = kda_chunk_fwd_workspace_bytes(&a);
  EXPECT(bytes != SIZE_MAX, "workspace query: %s", kda_last_error());
  EXPECT(bytes >= (size_t)2 * 4 * 163840, "workspace %zu bytes", bytes);
  a.flags = KDA_FLAG_GENERIC;
  bytes = kda_chunk_fwd_workspace_bytes(&a);
  EXPECT(bytes == 0, "fp32 path workspace %zu", bytes);
  a = base_args();
  a.dk = 96;
  EXPECT(kda_chunk_fwd_workspace_bytes(&a) == SIZE_MAX && strlen(kda_last_error()) > 0,
         "workspace query of a bad shape");

  /* validation before any launch */
  a = base_args();
  a.dk = 96;
  EXPECT(kda_chunk_fwd(&a, NULL) == KDA_ERR_BAD_SHAPE, "dk 96");
  EXPECT(strlen(kda_last_error()) > 0, "no error detail");
  a = base_args();
  a.q = NULL;
  EXPECT(kda_chunk_fwd(&a, NULL) == KDA_ERR_NULL_PTR, "NULL q");
  a = base_args();
  a.o = (void*)a.v;
  EXPECT(kda_chunk_fwd(&a, NULL) == KDA_ERR_ALIAS, "o on v");
  a = base_args();
  EXPECT(kda_chunk_fwd(&a, NULL) == KDA_ERR_WORKSPACE, "missing workspace: %s", kda_last_error());

  kda_decode_args d;
  memset(&d, 0, sizeof d);
  d.N = 0; d.H = 4; d.dk = 128; d.dv = 128;
  EXPECT(kda_decode_step(&d, NULL) == KDA_ERR_BAD_SHAPE, "decode N=0");

  kda_decode_multi_args m;
  memset(&m, 0, sizeof m);
  m.N = 2; m.H = 2; m.dk = 128; m.dv = 128; m.m = 0;
  EXPECT(kda_decode_multi(&m, NULL) == KDA_ERR_BAD_SHAPE, "decode_multi m=0");

  int64_t n_bad = -1;
  EXPECT(kda_check_gates(NULL, 10, NULL, 0, KDA_BF16, NULL, KDA_CHECK_COUNTERS, NULL, &n_bad) ==
             KDA_ERR_NULL_PTR,
         "check_gates NULL g");
  EXPECT(kda_check_gates((const void*)((uintptr_t)1 << 40), 10, NULL, 0, KDA_BF16, NULL,
                         KDA_CHECK_COUNTERS, NULL, &n_bad) == KDA_ERR_NULL_PTR,
         "check_gates NULL counts");
  EXPECT(kda_check_gates((const void*)((uintptr_t)1 << 40), 10, NULL, 0, KDA_BF16,
                         (int64_t*)((uintptr_t)1 << 40), KDA_CHECK_COUNTERS, NULL, &n_bad) ==
             KDA_ERR_ALIAS,
         "check_gates counts on g");

  if (failures == 0) printf("ok\n");
  return failures ? 1 : 0;
}
