/*
 * pa_probe.h — measurement probe shipped beside libpa (libpa_probe.so): the
 * HBM read rate this GPU reaches with the access pattern of the decode
 * kernels, as the practical ceiling their roofline fractions are read
 * against.  Not part of the attention path.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_probe_stream — every wavefront reads tiles_per_wave whole tiles of
 * tile_bytes (2048 or 4096) bytes from `pool`, tile
 * tile_ids[w * tiles_per_wave + i] for wavefront w (ids in [0, num_tiles);
 * others read nothing), with 16-byte lane loads of one contiguous KiB per
 * instruction and in_flight (2, 3, 4, 6 or 8) tiles in flight, as the decode
 * kernels stream K/V tiles.  nontemporal != 0 gives the loads the
 * non-temporal cache policy the decode kernels use.
 * sink[w * 64 + lane] receives the XOR of the 32-bit words the lane read
 * (it keeps the loads alive and lets a test check what was read).
 * Four wavefronts per workgroup.  Returns 0, -2 on invalid sizes, -6 when
 * the launch fails.  Asynchronous on `stream`.
 */
int pa_probe_stream(const void* pool, int64_t num_tiles, const int32_t* tile_ids,
                    int32_t num_waves, int32_t tiles_per_wave, int32_t tile_bytes,
                    int32_t in_flight, int32_t nontemporal, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
