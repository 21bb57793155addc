/*
 * muse_attn_timeline.h -- profiling build of the decode kernels
 * (libmuse_attn_timeline.so, built by `python full_gqa_attention_amd/build.py
 * --timeline`): the library of muse_attn.h whose decode split and merge
 * kernels also record, per workgroup, the time at which each phase of their
 * work is done, read on the GPU's 100 MHz real-time clock (s_memrealtime,
 * one clock for the whole device).  The regular libmuse_attn.so does not
 * export this function.
 *
 * The stamps wait for the data each phase names; at the end a workgroup also
 * waits for its stores to complete before its last stamp.  Results are the
 * same as the regular build's (the parity tests compare them bit for bit).
 */
#ifndef MUSE_ATTN_TIMELINE_H
#define MUSE_ATTN_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

/* Workgroups recorded per launch (higher workgroup indices are not recorded)
 * and 64-bit slots per record. */
#define MUSE_TL_SPLIT_WORKGROUPS 4096
#define MUSE_TL_SPLIT_SLOTS 8
#define MUSE_TL_MERGE_WORKGROUPS 4096
#define MUSE_TL_MERGE_SLOTS 4

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the records of the most recent decode launches to host arrays:
 *   split_host[8 * b + i], workgroup b of the split kernel (decode_kernel):
 *     i = 0 start, 1 seq_len read, 2 raw Q rows arrived, 3 Q-hat shared in
 *     LDS (workgroup barrier), 4 the wave's sub-tiles done, 5 the waves'
 *     partials merged in LDS, 6 its stores complete (the split's partial, or
 *     the output when the sequence has one split), 7 sub-tiles of wave 0;
 *   merge_host[4 * b + i], workgroup b of decode_merge_kernel:
 *     i = 0 start, 1 partials, gate and seq_len arrived, 2 output stores
 *     complete, 3 live splits merged.
 * Stamps are in units of 10 ns; a record of zeros belongs to a workgroup
 * that exited early (a split past a short sequence's rows) or was not run
 * since the last clear.  Each call overwrites the records of its workgroup
 * indices, so after several launches the array holds, per index, the last
 * launch that had that workgroup.
 * split_count / merge_count: capacity of the host arrays in 64-bit values
 * (either array may be NULL); clear != 0 zeroes the device records after
 * copying.  Synchronises the device.  Returns 0 (MUSE_OK) or 7
 * (MUSE_ERR_HIP).  Host arrays, host pointers. */
int muse_decode_timeline_read(uint64_t* split_host, size_t split_count, uint64_t* merge_host,
                              size_t merge_count, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif  /* MUSE_ATTN_TIMELINE_H */
