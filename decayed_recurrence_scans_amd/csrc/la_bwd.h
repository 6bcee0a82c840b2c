// la_bwd.h -- helper kernels of the linear-attention backward (the three
// gradient scans themselves run on the forward kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace drs {

// out[u][j][i] = in[u][i][j] for u < units, an R x C fp32 matrix per unit.
hipError_t transpose_units_launch(const float *in, float *out, int units, int R, int C, hipStream_t s);

// The factors of the gradient scans, one per (unit, t): the factor of the step
// visited next in the forward order, and 1 for the step the gradient scan
// visits first.  mode 1: decay[h] (unit = b*H + h); mode 2: decay[unit][t].
hipError_t shift_decay_launch(const float *decay, int mode, float *out, int units, int H, int T, int reverse,
                              hipStream_t s);

// out[u] = g_first(u) * in[u] over a D-element state per unit, where g_first is
// the factor of the first visited step (mode 1 or 2, as above).
hipError_t scale_state_launch(const float *in, const float *decay, int mode, float *out, int units, int H, int T,
                              int D, int reverse, hipStream_t s);

// c[u][t] = q.dq - k.dk over the key dimension (fp32 rows of Dk elements).
hipError_t decay_terms_launch(const float *q, const float *dq, const float *k, const float *dk, float *c,
                              long rows, int Dk, hipStream_t s);

// The same for bf16 q, k with fp32 dq, dk, which are also rounded (to nearest
// even) into the bf16 outputs dq_out, dk_out.
hipError_t decay_terms_cast_launch(const void *q, const float *dq, const void *k, const float *dk, float *c,
                                   void *dq_out, void *dk_out, long rows, int Dk, hipStream_t s);

// Per unit: A_n = sum of c over the steps visited at or after step n, plus
// <dsf, sfin> (NULL: 0); the factor gradient is A_n / g.  mode 2 writes it per
// step into ddecay [units, T]; mode 1 writes the unit's sum over t into
// partial[u], and the last workgroup to finish sets ddecay[h] = sum over b of
// partial[b*H + h] (b ascending).  done: a counter that is zero on entry and is
// left zero.  With ds0 (not NULL) it also writes ds_in = g_first * ds0 over the
// D-element state of each unit (as scale_state_launch).  One launch.
hipError_t decay_grad_launch(const float *c, const float *decay, int mode, const float *dsf, const float *sfin,
                             int D, float *ddecay, float *partial, int B, int H, int T, int reverse,
                             const float *ds0, float *ds_in, unsigned *done, hipStream_t s);

// ---- the normalised form's gradients through unnormalised fp32 scans ----------------
// bf16 -> fp32 and fp32 -> bf16 (round to nearest even), n elements, n a multiple of 8.
hipError_t cast_up_launch(const void *in, float *out, size_t n, hipStream_t s);
hipError_t cast_down_launch(const float *in, void *out, size_t n, hipStream_t s);
// rows x 16 fp32: 1 in column 0, 0 elsewhere.
hipError_t ones16_launch(float *out, size_t rows, hipStream_t s);
// Per unit, the D-vector src[u] (NULL: zeros) padded to 16 wide: as column 0 of a
// D x 16 matrix (col0) or as row 0 of a 16 x D matrix (!col0).
hipError_t pad16_launch(const float *src, float *out, int units, int D, bool col0, hipStream_t s);
// out[u] = [S[u] (D1 values, NULL: zeros) | z[u] (D2 values, element i at
// z[u * D2 * zstride + i * zstride], NULL: zeros)]: a state and its key sum as one vector
// of D1 + D2 values per unit.
hipError_t concat_state_launch(const float *S, const float *z, int zstride, float *out, int units, int D1, int D2,
                               hipStream_t s);
// out[u] = row 0 of the 16 x D matrix in[u].
hipError_t row0_launch(const float *in, float *out, int units, int D, hipStream_t s);
// From n = S^T q (rows of Dv, fp32, overwritten) and d = z^T q (column 0 of 16-wide
// rows): a = dy / d in place of n, and c = -(dy . n) / d^2 in column 0 of 16-wide
// rows (the rest 0).  dy: bf16 rows of Dv.
hipError_t norm_terms_launch(const void *dy, float *na, const float *d16, float *c16, long rows, int Dv,
                             hipStream_t s);

}  // namespace drs
