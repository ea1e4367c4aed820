/* Host-only driver for the table builder, built with sanitizers by the tests:
 * reads "n dp rank split" then n lines "E R C" from stdin, builds the table and
 * prints the info line and one line per slot. */
#include <stdio.h>
#include <stdlib.h>

#include "../../include/fp8z1.h"

int main(void) {
  int n, dp, rank, split;
  if (scanf("%d %d %d %d", &n, &dp, &rank, &split) != 4) return 2;
  fp8z1_shape* shapes = (fp8z1_shape*)calloc((size_t)(n > 0 ? n : 1), sizeof(fp8z1_shape));
  for (int i = 0; i < n; ++i) {
    long long e, r, c;
    if (scanf("%lld %lld %lld", &e, &r, &c) != 3) return 2;
    shapes[i].E = e;
    shapes[i].R = r;
    shapes[i].C = c;
  }
  fp8z1_table* t = NULL;
  int rc = fp8z1_build_table(shapes, n, dp, rank, split, &t);
  if (rc != FP8Z1_OK) {
    printf("error %d %s\n", rc, fp8z1_last_error());
    free(shapes);
    return 0;
  }
  fp8z1_table_info info;
  const fp8z1_block* ent = NULL;
  fp8z1_table_info_get(t, &info);
  fp8z1_table_entries(t, &ent);
  printf("info %lld %lld %lld %lld %lld %lld\n", (long long)info.total_blocks, (long long)info.slots_per_rank,
         (long long)info.shard_first_slot, (long long)info.shard_slots, (long long)info.valid_elems,
         (long long)info.pad_elems);
  for (long long s = 0; s < info.shard_slots; ++s)
    printf("%d %d %d %d %d %d\n", ent[s].param, ent[s].expert, ent[s].brow, ent[s].bcol, ent[s].vrows, ent[s].vcols);
  fp8z1_table_free(t);
  free(shapes);
  return 0;
}
