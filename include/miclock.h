/* miclock -- engine clock probe for MI355X (gfx950), C ABI.
 *
 * Measurement tooling, not part of the attention path: it reports the shader
 * engine clock that the GPU holds while other kernels run, so that a kernel's
 * throughput can be set against the MFMA peak at the clock it actually got
 * (the dense peak is quoted at 2.4 GHz; a power-limited part runs lower under
 * sustained matrix work).
 *
 * How: each probe workgroup is one wave of which one lane works. It first
 * waits warm_ticks of the 100 MHz real-time counter (s_memrealtime), then
 * reads the shader-clock cycle counter (s_memtime) and the real-time counter
 * at the start and at the end of a window of window_ticks real-time ticks,
 * sleeping between reads (s_sleep), so it takes almost no issue slots from
 * the kernels it shares the GPU with. Cycles over real time give the clock.
 * Workgroups are dealt to the XCDs in turn (id mod 8 per XCD), so 8 or more
 * probes cover every XCD; each XCD has its own clock.
 *
 * The probe holds no LDS and a few registers: launched on a second stream
 * (default priority) just before a run of other kernels, it runs beside
 * them. The loop ends when the real-time counter has advanced by
 * warm_ticks + window_ticks, whatever else runs. */
#ifndef MICLOCK_H
#define MICLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the probe.
 *
 * out           device, uint64 [n_groups][4], written by the probe:
 *               [0] shader-clock cycles over the window, [1] real-time ticks
 *               over the window (100 MHz), [2] real-time counter at the
 *               window's start, [3] real-time counter at the probe's entry.
 *               Clock of probe i in MHz = out[i][0] / out[i][1] * 100.
 * n_groups      number of probe workgroups, 1 .. 1024
 * warm_ticks    real-time ticks to wait before the window (<= 2^32)
 * window_ticks  real-time ticks of the window, 1 .. 2^32 (about 43 s)
 * stream        hipStream_t (NULL = the null stream)
 * Returns 0 when enqueued; 1 for a NULL `out`, 2 for a size out of range
 * (nothing enqueued); 5 when the launch failed. Returns without
 * synchronising. */
int miclock_probe(uint64_t* out, int n_groups, uint64_t warm_ticks, uint64_t window_ticks,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MICLOCK_H */
