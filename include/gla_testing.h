/*
 * gla_testing.h -- a test hook of libgla.so, separate from the operation's interface
 * in gla.h.
 *
 * The launch plan of a prefill is a function of its sizes alone: the value columns
 * per workgroup, the number of sequence segments, and the delta rule's value tile.
 * Tests call gla_testing_set_plan to force those choices, because every plan must
 * give the recurrence's result, and the sizes alone do not reach all of them.  The
 * outputs do not depend on the plan beyond rounding; the prefill tile does not change
 * them at all.
 */
#ifndef GLA_TESTING_H
#define GLA_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gla_testing_set_plan -- force launch-plan choices for every later call in the
 * process, until called again with zeros (the default: automatic choice).
 *
 *   prefill_tile      0, or the value columns per prefill workgroup (16, 32 or 64);
 *                     used for a call when it divides d_v and fits in LDS
 *   prefill_segments  0, or the number of sequence segments (>= 1; capped at the
 *                     number of chunks)
 *   delta_tile        0, or the value columns per delta-rule workgroup (16, 32 or 64);
 *                     used when at most d_v
 *
 * The settings are process-wide and are not synchronised with calls running on
 * other threads: set them only while no other thread calls the library.
 * gla_prefill_workspace_bytes follows them, so query it after setting them.
 * Returns GLA_OK, or GLA_ERR_UNSUPPORTED (-3) for a value out of range, leaving the
 * settings unchanged.
 */
int gla_testing_set_plan(int prefill_tile, int prefill_segments, int delta_tile);

#ifdef __cplusplus
}
#endif

#endif /* GLA_TESTING_H */
