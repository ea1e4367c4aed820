// Host-only stand-in for fp8z1_table_free, for the sanitizer build of the table
// builder (the library's version also releases device memory; a table that never
// reached a GPU owns none).
#include "../../blockwise_fp8_zero_fold_amd/csrc/internal.h"

extern "C" void fp8z1_table_free(fp8z1_table* t) { delete t; }
