/* A plain C client of libdcp: compiled with a C compiler against include/dcp.h and
 * linked to libdcp.so, it calls the host entry points and the argument checks of the
 * device entry points (which fail before any launch), and prints one line per check.
 * Test infrastructure: built and run by tests/test_c_abi.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dcp.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok" : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  /* The contiguous split of a 200,000-token request over 4 ranks in runs of 50,000. */
  const int32_t L[1] = {200000};
  int32_t local[1] = {0};
  int64_t total = 0;
  int32_t mx = 0;
  for (int32_t r = 0; r < 4; ++r) {
    check(dcp_shard_map(L, 1, 4, 50000, r, local, &total, &mx) == DCP_SUCCESS && local[0] == 50000 &&
              total == 50000 && mx == 50000,
          "shard_map 200k over 4 ranks");
  }
  /* Owner and local index of a few positions, and the inverse. */
  const int64_t pos[5] = {0, 49999, 50000, 150001, 199999};
  int32_t owner[5];
  int64_t idx[5], back[5];
  check(dcp_shard_locate(pos, 5, 4, 50000, owner, idx) == DCP_SUCCESS && owner[0] == 0 && owner[1] == 0 &&
            owner[2] == 1 && owner[3] == 3 && owner[4] == 3 && idx[2] == 0 && idx[3] == 1,
        "shard_locate");
  int ok = 1;
  for (int i = 0; i < 5; ++i) {
    ok &= dcp_shard_global(&idx[i], 1, 4, 50000, owner[i], &back[i]) == DCP_SUCCESS && back[i] == pos[i];
  }
  check(ok, "shard_global inverts shard_locate");
  /* Errors. */
  check(dcp_shard_map(L, 1, 0, 1, 0, local, NULL, NULL) == DCP_ERROR_INVALID_VALUE, "N = 0 rejected");
  check(dcp_shard_map(L, 1, 2, 1, 2, local, NULL, NULL) == DCP_ERROR_INVALID_VALUE, "rank >= N rejected");
  check(strcmp(dcp_status_string(DCP_ERROR_WORKSPACE), "DCP_ERROR_WORKSPACE") == 0, "status string");
  /* Workspace sizing and the partial call's checks. */
  dcp_attn_desc_t mla = {DCP_KV_MLA_LATENT, 64, 1, 576, 512, 128, 0.0416667f};
  dcp_attn_desc_t bad = mla;
  bad.qk_dim = 128;
  check(dcp_decode_workspace_size(&mla, 128, 256) > 0, "workspace size");
  check(dcp_decode_workspace_size(&bad, 128, 256) == 0, "unsupported dims give no workspace");
  char fake;
  void* f = (void*)(((uintptr_t)&fake + 4096) & ~(uintptr_t)4095);
  check(dcp_decode_partial(&mla, f, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 2, 2, 1, 0, f,
                           1 << 30, (float*)f, (float*)f, NULL) == DCP_ERROR_INVALID_VALUE,
        "partial: rank >= N rejected before launch");
  check(dcp_decode_partial(&mla, f, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 0, 2, 1, 0, f, 16,
                           (float*)f, (float*)f, NULL) == DCP_ERROR_WORKSPACE,
        "partial: small workspace rejected before launch");
  check(dcp_merge((const float*)f, (const float*)f, 0, 2, 4, 512, (float*)f, (float*)f, NULL) ==
            DCP_ERROR_INVALID_VALUE,
        "merge: zero parts rejected");
  check(dcp_workspace_init(NULL, 4096, NULL) == DCP_ERROR_INVALID_VALUE, "workspace_init: NULL rejected");
  check(dcp_workspace_init((char*)f + 4, 4096, NULL) == DCP_ERROR_INVALID_VALUE,
        "workspace_init: misaligned workspace rejected");
  uint32_t bits = 0;
  check(dcp_workspace_errors(f, 128, &bits, 0, NULL) == DCP_ERROR_INVALID_VALUE,
        "workspace_errors: short workspace rejected");
  check(dcp_workspace_errors(f, 4096, NULL, 0, NULL) == DCP_ERROR_INVALID_VALUE,
        "workspace_errors: NULL output rejected");
  /* Multi-token sizing and checks. */
  const size_t ws1 = dcp_decode_workspace_size(&mla, 128, 256);
  check(dcp_decode_workspace_size_mtp(&mla, 1, 128, 256) == ws1, "mtp: q_len 1 sizes like the decode call");
  check(dcp_decode_workspace_size_mtp(&mla, 2, 128, 256) > ws1, "mtp: two query tokens need more workspace");
  check(dcp_decode_workspace_size_mtp(&mla, 0, 128, 256) == 0, "mtp: q_len 0 gives no workspace");
  check(dcp_decode_workspace_size_mtp(&mla, 9, 128, 256) == 0, "mtp: more than 512 MLA score rows unsupported");
  check(dcp_decode_partial_mtp(&mla, 0, f, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 0, 2, 1, 0,
                               f, 1 << 30, (float*)f, (float*)f, NULL) == DCP_ERROR_INVALID_VALUE,
        "mtp: q_len 0 rejected before launch");
#ifndef DCP_CLIENT_HOST_ONLY
  /* The allocation-free call checks its arguments before touching its scratch. */
  check(dcp_decode_partial_noalloc(&mla, f, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 2, 2, 1,
                                   0, (float*)f, (float*)f, NULL) == DCP_ERROR_INVALID_VALUE,
        "noalloc: rank >= N rejected before launch");
#endif
  /* KV append, local block table and the per-rank merge steps: argument checks. */
  check(dcp_append_kv(&mla, f, NULL, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 0, 0, 1, NULL) ==
            DCP_ERROR_INVALID_VALUE,
        "append: N = 0 rejected");
  check(dcp_append_kv(&mla, f, f, f, NULL, 10, (const int32_t*)f, 4, (const int32_t*)f, 2, 0, 2, 1, NULL) ==
            DCP_ERROR_INVALID_VALUE,
        "append: an MLA V pointer rejected");
  check(dcp_local_block_table((const int32_t*)f, 2, 8, 2, 100, 64, 0, (int32_t*)f, 4, NULL) ==
            DCP_ERROR_NOT_SUPPORTED,
        "local block table: interleave not a multiple of the page size unsupported");
  check(dcp_merge_lse((const float*)f, 0, 2, 4, (float*)f, NULL) == DCP_ERROR_INVALID_VALUE,
        "merge_lse: zero parts rejected");
  check(dcp_rescale_partial((const float*)f, (const float*)f, (const float*)f, 2, 4, 512, 7, f, NULL) ==
            DCP_ERROR_INVALID_VALUE,
        "rescale: unknown transport dtype rejected");
  check(dcp_sum_head_slice(f, DCP_DTYPE_F32, 3, 2, 4, 512, 0, (float*)f, NULL) == DCP_ERROR_INVALID_VALUE,
        "sum_head_slice: heads not divisible by the ranks rejected");
  printf("%d failures\n", failures);
  return failures != 0;
}
