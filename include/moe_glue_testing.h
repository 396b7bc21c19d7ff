/* moe_glue testing and measurement hooks -- not part of the production
 * interface in moe_glue.h.
 *
 * The library picks a route variant and an expand order per call from the
 * batch shape.  Tests force each variant in turn to check that all of them
 * give the oracle's results, and measurements force them to compare their
 * speed; production callers never call this.
 */
#ifndef MOE_GLUE_TESTING_H
#define MOE_GLUE_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Force, process-wide and until the next call, the route variant
 * (0 automatic, 1 one workgroup -- T <= 256 only, 2 two launches -- the
 * top-k, then scan and place in one launch, 3 three launches -- top-k,
 * column scan, place), the expand order of the route + expand calls above the
 * one-launch size (0 automatic, 1 token order in a launch of its own, 2 token
 * order inside the route's place launch, 3 destination order from a row list
 * the route writes, 4 destination order with placement and copy in one
 * launch), and the number of workgroups per token group of that last order
 * (0 automatic).  A forced order the shape or the route variant does not
 * allow falls back to the nearest one that applies.  Forcing any route
 * variant also makes the route + expand calls skip their one-launch form for
 * T <= 64.  Returns 0, or
 * -1 (and changes nothing) for a value out of range.  Not synchronised with
 * calls in flight on other threads. */
int moe_testing_force(int route_variant, int expand_order, int workgroups_per_group);

#ifdef __cplusplus
}
#endif
#endif /* MOE_GLUE_TESTING_H */
