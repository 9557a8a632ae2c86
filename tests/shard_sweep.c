/* Exhaustive sweep of the host shard-map entry points (dcp_shard_map, dcp_shard_locate,
 * dcp_shard_global), for tests/test_host_sanitizers.py, which builds it with
 * AddressSanitizer and UndefinedBehaviorSanitizer and compares the output with the
 * oracle's enumeration of shard ownership.
 *
 * For N = 1..8, I in {1, 2, 3, 7, 16, 64, 128, 1000} and every rank r, it writes (int64,
 * native byte order) to the file named by argv[1]: the local length of every request
 * length L = 0..LMAX; the owner and local index of every position t < LMAX; and the global
 * position of every local index j < L_r(LMAX).  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dcp.h"

#define LMAX 4096

static int write64(FILE* f, const int64_t* v, size_t n) { return fwrite(v, sizeof(int64_t), n, f) == n; }

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  FILE* f = fopen(argv[1], "wb");
  if (!f) return 2;
  static const int32_t Is[8] = {1, 2, 3, 7, 16, 64, 128, 1000};
  static int32_t lens[LMAX + 1], local[LMAX + 1], owner[LMAX];
  static int64_t out[LMAX + 1], pos[LMAX], idx[LMAX], glob[LMAX];
  for (int32_t L = 0; L <= LMAX; ++L) lens[L] = L;
  for (int32_t t = 0; t < LMAX; ++t) pos[t] = t;
  int bad = 0;
  for (int32_t N = 1; N <= 8; ++N)
    for (int k = 0; k < 8; ++k) {
      const int32_t I = Is[k];
      if (dcp_shard_locate(pos, LMAX, N, I, owner, idx) != DCP_SUCCESS) bad = 1;
      for (int32_t r = 0; r < N; ++r) {
        int64_t total = -1;
        int32_t mx = -1;
        if (dcp_shard_map(lens, LMAX + 1, N, I, r, local, &total, &mx) != DCP_SUCCESS) bad = 1;
        for (int32_t L = 0; L <= LMAX; ++L) out[L] = local[L];
        if (!write64(f, out, LMAX + 1)) bad = 1;
        for (int32_t t = 0; t < LMAX; ++t) out[t] = owner[t];
        if (!write64(f, out, LMAX) || !write64(f, idx, LMAX)) bad = 1;
        const int64_t n = local[LMAX];
        int64_t j[LMAX];
        for (int64_t i = 0; i < n; ++i) j[i] = i;
        if (dcp_shard_global(j, n, N, I, r, glob) != DCP_SUCCESS) bad = 1;
        if (!write64(f, glob, (size_t)n)) bad = 1;
      }
    }
  fclose(f);
  printf("%s\n", bad ? "errors" : "done");
  return bad;
}
