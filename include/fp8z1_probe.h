/*
 * fp8z1 streaming references: measurement aids, not part of the method.
 *
 * Each kernel moves the bytes of one of the library's kernels with the same
 * access pattern and no real arithmetic, so that a measured kernel can be
 * compared with the bandwidth the GPU sustains for that pattern as well as
 * with the published HBM peak.  Same conventions as fp8z1.h (int status,
 * asynchronous on `stream`, caller-owned device buffers, contents of the
 * written buffers are meaningless afterwards).
 */
#ifndef FP8Z1_PROBE_H
#define FP8Z1_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` (a multiple of 4096) from src to dst, 4 KB per workgroup,
 * 16-byte streaming loads and stores.  Both buffers 16-byte aligned.
 * spread = 1: workgroup b copies the b-th 4 KB tile, so the workgroups in
 * flight cover one compact range of memory; spread = S (dividing the tile
 * count): workgroup b copies tile (b % S) * (tiles / S) + b / S, so they cover
 * S far-apart ranges at once (the traffic shape of kernels whose workgroups
 * each own a large contiguous block). */
int fp8z1_probe_copy(const void* src, void* dst, int64_t bytes, int64_t spread, void* stream);

/* The update kernel's traffic over nslots 128x128 slots: per slot, read 64 KB
 * of each of g, p, m, v and write 64 KB of each of p, m, v (16-byte streaming
 * accesses) plus 16 KB of codes (plain 4-byte stores).  parts = 1: one
 * workgroup per slot, the update's own tiling; parts = 2, 4 or 8: one
 * workgroup per 1/parts of a slot, the same streams with less memory per
 * workgroup.  g, p, m, v are nslots*16384 float32, codes nslots*16384 bytes,
 * all 16-byte aligned. */
int fp8z1_probe_update_pattern(const float* g, float* p, float* m, float* v, uint8_t* codes, int64_t nslots,
                               int32_t parts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Z1_PROBE_H */
