/* pa_timeline.h -- diagnostic export of libpa_decode_timeline.so.
 *
 * libpa_decode_timeline.so is the same library as libpa_decode.so (every entry
 * point of pa_decode.h, the same kernels) built with per-workgroup timestamps
 * (python split_kv_paged_pa_amd/build.py builds both).  It exists to measure
 * where the time of a decode step goes; it is not for production use: each
 * stamped workgroup writes 32 bytes, and Phase 2 takes one device-scope atomic
 * more.  libpa_decode.so does not export the function below.
 */
#ifndef PA_TIMELINE_H
#define PA_TIMELINE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the timestamp records written since the last call (at most
 * max_records; a negative max_records copies all the buffer holds, 2^18) to the
 * host buffer dst (NULL: copy nothing), then clears the records and their
 * counter.  Each record is four uint64: word 0 = kind (bits 0-3: 1 Phase 1 or
 * V1, 2 Phase 2) | XCC id << 4 | linear workgroup id << 8 | HW_ID << 32; words
 * 1-3 = start, mid point, end on the 100 MHz constant clock (10 ns ticks).
 * Returns the number of records the counter reached (records of workgroups
 * that had no work are all zero), or a negative value if a HIP call failed.
 * Synchronises the current device; call it with no kernel of this library in
 * flight on other streams. */
int pa_timeline_fetch(void *dst, int max_records);

#ifdef __cplusplus
}
#endif

#endif /* PA_TIMELINE_H */
