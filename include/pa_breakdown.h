/*
 * pa_breakdown.h -- the breakdown library libpa_decode_breakdown.so: the
 * decode library built with PA_BREAKDOWN=1, a measuring aid beside it.  It
 * exports everything include/pa_decode.h declares, computing the same
 * results, plus the call below; libpa_decode.so does not have it.
 *
 * The flash-decoding-bench design note (rationale and implementations
 * sections) splits a decode step into the read of the KV cache by parallel
 * chunks and the merge of their partial results.  Timing the fused split
 * stopped at successive points shows what each part adds to the read:
 *
 * pa_breakdown_stop_after(stage) sets where every later fused-split launch of
 * this library stops, in every workgroup that has tiles (a workgroup that
 * writes its sequence's output directly, as a single pass, is not stopped):
 *   0  nowhere: the whole step, as the library (the default);
 *   1  after the stream of K and V rows and its arithmetic: no epilogue;
 *   2  after the waves' sums are combined into the partition's partial sums
 *      (max, sum, weighted values), which are not stored;
 *   3  after storing the partial sums: no ticket, no merge.
 * Stages 1 to 3 write no output and are for timing only.  They leave the
 * tickets as they found them, so stage 0 calls before and after them are
 * correct.  The setting is process-wide and read when a call is made.
 * Returns PA_OK or PA_ERR_VALUE (stage outside 0..3).
 */
#ifndef PA_BREAKDOWN_H
#define PA_BREAKDOWN_H

#ifdef __cplusplus
extern "C" {
#endif

int pa_breakdown_stop_after(int stage);

#ifdef __cplusplus
}
#endif

#endif /* PA_BREAKDOWN_H */
