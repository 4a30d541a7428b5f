/*
 * fd_calib.h -- choosing the unified maximum phi and the safe band from
 * observed scores (AMD MI355X, gfx950), part of the same library as
 * fd_attn.h.
 *
 * The theory page of FlashDecoding++ (section 3) sets phi beforehand from the
 * observed distribution of the scores; a row whose scores leave the band
 * [phi - a, phi + b] takes the online-softmax fallback.  A decode row stays in
 * band iff its own score range [min_t s_t, max_t s_t] fits inside the band,
 * so a set of rows fits one band of width W = a + b (phi placed anywhere)
 * iff the largest maximum minus the smallest minimum of the set is at most W.
 *
 *   fd_attn_score_stats  -- GPU pass over calibration inputs: every row's
 *                           largest and smallest score, and a histogram.
 *   fd_attn_choose_band  -- host: the narrowest band (and its phi) that keeps
 *                           all but a given fraction of the rows in band.
 *
 * Errors: FD_OK (0) or a negative FD_ERR_* code from fd_attn.h; on an error
 * nothing is enqueued and no output is written.
 */
#ifndef FD_CALIB_H
#define FD_CALIB_H

#include "fd_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Score statistics of one decode call's inputs, with the same descriptor,
 * layouts and dtypes as fd_attn_decode (include/fd_attn.h); the descriptor's
 * workspace fields are not used.  Reads q and K only.  For every row
 * (b, query head h), over the valid tokens t < seq_lens[b]:
 *
 *   s_t = scale * <q, k_t>              (fp8: k_t = k_scale[kvh] * code)
 *   row_max[b*Hq + h] = max_t s_t,  row_min[b*Hq + h] = min_t s_t
 *                                       (-inf / +inf for an empty row)
 *
 * If hist is not NULL and nbins > 0, hist[0 .. nbins+1] counts every valid
 * score: hist[0] below hist_lo, hist[1 + i] in [hist_lo + i*w, hist_lo +
 * (i+1)*w) with w = (hist_hi - hist_lo) / nbins, hist[nbins + 1] at or above
 * hist_hi.  Scores are fp32 and bins are chosen in fp32, so a score within
 * rounding of a bin edge may land in either neighbour.  Counts are uint32.
 *
 * row_max, row_min: device float[batch * num_q_heads]; hist: device
 * uint32[nbins + 2] or NULL; nbins in 0 .. 8192; hist_lo < hist_hi, both
 * finite, when a histogram is taken.  All outputs are written by the call
 * (no initialisation needed); the call enqueues two kernels on `stream` and
 * the outputs are valid once the stream has completed them.  NaN scores are
 * outside the contract (they count below hist_lo and do not move extremes).
 */
int fd_attn_score_stats(const fd_attn_desc_t *desc, const void *q, const void *k_cache,
                        const int32_t *seq_lens, const int32_t *block_table, float hist_lo,
                        float hist_hi, int32_t nbins, float *row_max, float *row_min,
                        uint32_t *hist, hipStream_t stream);

/*
 * Host function.  Given per-row extremes (host arrays of nrows floats, as
 * fd_attn_score_stats writes them; rows with row_max < row_min are empty and
 * ignored), choose the narrowest band that keeps all but
 * floor(max_flag_fraction * m) of the m non-empty rows in band:
 *
 *   W = the smallest width for which that many rows fit (exact over the
 *       given extremes), or max_width if even max_width does not suffice;
 *   a = a_share * W + pad,  b = (1 - a_share) * W + pad;
 *   phi = the centre of the widest range of phi that keeps the most rows
 *         in [phi - a_share*W, phi + (1-a_share)*W].
 *
 * pad (score units, >= 0) widens both sides so that rounding phi, a and b to
 * float, and the decode kernels' own fp32 scores, cannot flag a row the
 * choice kept (1e-3 is ample for bf16 caches).  *flagged receives how many
 * non-empty rows the returned (phi, a, b) flags, counted on the given
 * extremes.  The decode call requires a, b <= 64: keep max_width + 2*pad
 * within that.  Errors: FD_ERR_NULL, or FD_ERR_BAND for max_flag_fraction or
 * a_share outside [0, 1], max_width not positive and finite, pad negative.
 */
int fd_attn_choose_band(const float *row_max, const float *row_min, int64_t nrows,
                        double max_flag_fraction, double a_share, double max_width, double pad,
                        float *phi, float *a, float *b, int64_t *flagged);

#ifdef __cplusplus
}
#endif

#endif /* FD_CALIB_H */
