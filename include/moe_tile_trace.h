/*
 * moe_tile_trace.h -- per-tile timeline of the packed grouped GEMMs, exported
 * only by the tile-trace build of the library (libmoe_tiletrace.so, made by
 * build.build_tile_trace(); the regular libmoe.so does not have these symbols).
 *
 * The traced library is the regular one plus timestamps: every workgroup of
 * the two packed prefill projections (moe_forward_packed on shapes that take
 * the tiled path) records, for each tile it runs, moments read from the
 * constant 100 MHz counter and from the shader clock counter.  Its results are
 * those of libmoe.so; the records only cost a few stores per tile.
 *
 * Record layout (int64): trace[proj][wg][tile][field], proj 0 = gate/up
 * projection, 1 = down projection; wg < MOE_TILE_TRACE_WGS (the workgroup
 * index), tile < MOE_TILE_TRACE_TILES (in the order the workgroup ran them;
 * later tiles are not recorded); fields:
 *   0..4   100 MHz counter at: k-loop start (after the tile's first barrier),
 *          k-loop end, after the closing barrier, after the next tile's first
 *          loads were issued, after the tile's epilogue;
 *   5..9   shader clock counter at the same moments;
 *   10     live 32-row blocks (8 where padded blocks are not skipped)
 *          + 16 * k-steps (of 32) of the tile;
 *   11     32-row blocks the tile's k-loop multiplies (the live ones, at least
 *          2; 8 where padded blocks are not skipped).
 * A record whose field 4 is 0 was not written.
 */
#ifndef MOE_TILE_TRACE_H
#define MOE_TILE_TRACE_H

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_TILE_TRACE_PROJS 2
#define MOE_TILE_TRACE_WGS 512
#define MOE_TILE_TRACE_TILES 64
#define MOE_TILE_TRACE_FIELDS 12

/* Zeroes the device trace of the current device (synchronous).  Returns 0 or a
 * HIP error code. */
int moe_tile_trace_clear(void);

/* Copies the whole trace (MOE_TILE_TRACE_PROJS * MOE_TILE_TRACE_WGS *
 * MOE_TILE_TRACE_TILES * MOE_TILE_TRACE_FIELDS int64, host memory owned by the
 * caller) after the device's work so far (synchronous).  Returns 0 or a HIP
 * error code. */
int moe_tile_trace_read(long long* host);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TILE_TRACE_H */
