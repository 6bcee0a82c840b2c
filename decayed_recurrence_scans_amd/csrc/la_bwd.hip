// la_bwd.hip -- the small kernels around the linear-attention backward.
//
// The gradients of y_t = q_t^T S_t, S_t = g_t S_{t-1} + k_t v_t^T are again
// decayed cumulative sums (RWKV-LM discussion #189 makes the same remark for
// WKV): with G_t the gradient reaching the state leaving step t,
//   dq_t = S_t dy_t                 a forward scan of v_s k_s^T read by dy_t,
//   dk_t = G_t v_t, dv_t = G_t^T k_t  scans in the opposite order of q_s dy_s^T,
// whose factor at t is the one of the step visited next.  Those three scans run
// on the forward kernels; this file holds the glue: state transposes, the
// shifted factors, the initial-state gradient, and the factor gradient, which
// follows from dL/d(log g_t) = sum over the steps visited at or after t of
// (q . dq - k . dk), plus <dS_final, S_final>, divided by g_t.
#include "common.h"
#include "la_bwd.h"
#include "lookback.h"

namespace drs {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void transpose_units(const float *in, float *out, int units, int R, int C) {
    const size_t n = (size_t)R * C, total = n * units;
    for (size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (size_t)gridDim.x * kThreads) {
        const size_t u = g / n;
        const int e = (int)(g - u * n);
        const int j = e / R, i = e - j * R;   // output [C][R]: coalesced writes
        out[g] = in[u * n + (size_t)i * C + j];
    }
}

__device__ __forceinline__ float factor(const float *decay, int mode, int unit, int H, int T, int t) {
    return mode == 1 ? decay[unit % H] : decay[(size_t)unit * T + t];
}

__global__ __launch_bounds__(kThreads) void shift_decay(const float *decay, int mode, float *out, int units, int H,
                                                        int T, int reverse) {
    const size_t n = (size_t)units * T;
    for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (size_t)gridDim.x * kThreads) {
        const int unit = (int)(e / T), t = (int)(e - (size_t)unit * T);
        // forward order: the gradient scan runs t descending, its factor at t is g_{t+1}
        const int src = reverse ? t - 1 : t + 1;
        out[e] = (src < 0 || src >= T) ? 1.f : factor(decay, mode, unit, H, T, src);
    }
}

__global__ __launch_bounds__(kThreads) void scale_state(const float *in, const float *decay, int mode, float *out,
                                                        int units, int H, int T, int D, int reverse) {
    const size_t total = (size_t)units * D;
    for (size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (size_t)gridDim.x * kThreads) {
        const int unit = (int)(g / D);
        out[g] = factor(decay, mode, unit, H, T, reverse ? T - 1 : 0) * in[g];
    }
}

// c = q.dq - k.dk for fp32 rows: LPR lanes per row of Dk elements, 16 bytes per lane.
__global__ __launch_bounds__(kThreads) void decay_terms(const float *q, const float *dq, const float *k,
                                                        const float *dk, float *c, long rows, int Dk) {
    const int lpr = Dk / 4;                            // lanes per row (4 .. 32)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int rpw = 64 / lpr;
    const long row = ((long)blockIdx.x * (kThreads / 64) + wv) * rpw + lane / lpr;
    const int piece = lane % lpr;
    float acc = 0.f;
    if (row < rows) {
        const size_t off = (size_t)row * Dk + (size_t)piece * 4;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(q + off), da = *reinterpret_cast<const f32x4 *>(dq + off);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(k + off), db = *reinterpret_cast<const f32x4 *>(dk + off);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc = fmaf(a[r], da[r], acc);
            acc = fmaf(-b[r], db[r], acc);
        }
    }
    for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows && piece == 0) c[row] = acc;
}

// The same for bf16 inputs whose gradients dq, dk come as fp32: the terms are
// formed before any rounding, and dq, dk are rounded once into the outputs.
__global__ __launch_bounds__(kThreads) void decay_terms_cast(const uint16_t *q, const float *dq,
                                                             const uint16_t *k, const float *dk, float *c,
                                                             uint16_t *dq_out, uint16_t *dk_out, long rows, int Dk) {
    const int lpr = Dk / 8;                            // lanes per row, 8 elements each
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int rpw = 64 / lpr;
    const long row = ((long)blockIdx.x * (kThreads / 64) + wv) * rpw + lane / lpr;
    const int piece = lane % lpr;
    float acc = 0.f;
    if (row < rows) {
        const size_t off = (size_t)row * Dk + (size_t)piece * 8;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(q + off), b = *reinterpret_cast<const u32x4 *>(k + off);
        const f32x4 da0 = *reinterpret_cast<const f32x4 *>(dq + off), da1 = *reinterpret_cast<const f32x4 *>(dq + off + 4);
        const f32x4 db0 = *reinterpret_cast<const f32x4 *>(dk + off), db1 = *reinterpret_cast<const f32x4 *>(dk + off + 4);
        const float dqa[8] = {da0[0], da0[1], da0[2], da0[3], da1[0], da1[1], da1[2], da1[3]};
        const float dkb[8] = {db0[0], db0[1], db0[2], db0[3], db1[0], db1[1], db1[2], db1[3]};
        u32x4 oq, ok;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc = fmaf(bf16_lo(a[r]), dqa[2 * r], acc);
            acc = fmaf(bf16_hi(a[r]), dqa[2 * r + 1], acc);
            acc = fmaf(-bf16_lo(b[r]), dkb[2 * r], acc);
            acc = fmaf(-bf16_hi(b[r]), dkb[2 * r + 1], acc);
            oq[r] = pack_bf16x2(dqa[2 * r], dqa[2 * r + 1]);
            ok[r] = pack_bf16x2(dkb[2 * r], dkb[2 * r + 1]);
        }
        *reinterpret_cast<u32x4 *>(dq_out + off) = oq;
        *reinterpret_cast<u32x4 *>(dk_out + off) = ok;
    }
    for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows && piece == 0) c[row] = acc;
}

// One workgroup per unit: suffix sums over the visiting order, in runs of
// ceil(T / 256) consecutive steps per thread.  The kernel is latency-bound (a few
// KB per unit), so every load it needs is issued before the first is used: the
// unit's terms (held in registers for runs of up to kRunRegs steps) and the state
// planes (kPlaneRegs elements per thread at a time).
//
// Also, when ds0 is given, this unit's initial-state gradient ds_in = g_first * ds0
// (D elements), and with one factor per head the sum over the batch: each
// workgroup stores its unit's sum, and the last one to finish (counted in *done,
// zero on entry and left zero) adds them up for every head in a fixed order.
constexpr int kRunRegs = 16;
constexpr int kPlaneRegs = 16;
__global__ __launch_bounds__(kThreads) void decay_grad(const float *c, const float *decay, int mode,
                                                       const float *dsf, const float *sfin, int D, float *ddecay,
                                                       float *partial, int H, int T, int reverse,
                                                       const float *ds0, float *ds_in, unsigned *done, int B) {
    __shared__ float red[kThreads];
    __shared__ unsigned last;
    const int unit = blockIdx.x, tid = threadIdx.x;
    const int L = (T + kThreads - 1) / kThreads;
    const int n0 = tid * L, n1 = min(n0 + L, T);
    auto tof = [&](int n) { return reverse ? T - 1 - n : n; };
    const float *cu = c + (size_t)unit * T;
    const bool inreg = L <= kRunRegs;
    float cv[kRunRegs];
    if (inreg) {
#pragma unroll
        for (int j = 0; j < kRunRegs; ++j) cv[j] = n0 + j < n1 ? cu[tof(n0 + j)] : 0.f;
    }
    // <dS_final, S_final> for this unit, and the initial-state gradient
    float st = 0.f;
    const bool dot = dsf && sfin;
    const float gf = ds0 ? factor(decay, mode, unit, H, T, reverse ? T - 1 : 0) : 0.f;
    if (dot || ds0)
        for (int e0 = tid; e0 < D; e0 += kPlaneRegs * kThreads) {
            float a[kPlaneRegs], b[kPlaneRegs], x[kPlaneRegs];
#pragma unroll
            for (int j = 0; j < kPlaneRegs; ++j) {
                const int e = e0 + j * kThreads;
                const size_t i = (size_t)unit * D + (e < D ? e : 0);
                a[j] = dot ? dsf[i] : 0.f;
                b[j] = dot ? sfin[i] : 0.f;
                x[j] = ds0 ? ds0[i] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kPlaneRegs; ++j) {
                const int e = e0 + j * kThreads;
                if (e < D) {
                    st = fmaf(a[j], b[j], st);
                    if (ds0) ds_in[(size_t)unit * D + e] = gf * x[j];
                }
            }
        }
    float mine = 0.f;
    if (inreg) {
#pragma unroll
        for (int j = 0; j < kRunRegs; ++j) mine += cv[j];
    } else {
        for (int n = n0; n < n1; ++n) mine += cu[tof(n)];
    }
    // the state term's sum, then the suffix over the threads after this one
    // (Hillis-Steele on the reversed index), in one array
    red[tid] = st;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    const float sterm = red[0];
    __syncthreads();
    red[tid] = mine;
    __syncthreads();
    for (int s = 1; s < kThreads; s <<= 1) {
        const float x = tid + s < kThreads ? red[tid + s] : 0.f;
        __syncthreads();
        red[tid] += x;
        __syncthreads();
    }
    float A = red[tid] - mine + sterm;   // sum over the runs after this thread's
    float hsum = 0.f;
    auto step = [&](int n, float cn) {
        const int t = tof(n);
        A += cn;
        const float dg = A / factor(decay, mode, unit, H, T, t);
        if (mode == 2) ddecay[(size_t)unit * T + t] = dg;
        else hsum += dg;
    };
    if (inreg) {
#pragma unroll
        for (int j = kRunRegs - 1; j >= 0; --j)
            if (n0 + j < n1) step(n0 + j, cv[j]);
    } else {
        for (int n = n1 - 1; n >= n0; --n) step(n, cu[tof(n)]);
    }
    if (mode == 1) {
        __syncthreads();
        red[tid] = hsum;
        __syncthreads();
        for (int s = kThreads / 2; s > 0; s >>= 1) {
            if (tid < s) red[tid] += red[tid + s];
            __syncthreads();
        }
        if (tid == 0) {
            // device-coherent store, complete before the count (as in the look-back exchange)
            __hip_atomic_store(partial + unit, red[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_stores_complete();
            last = atomicAdd(done, 1u) == (unsigned)(B * H) - 1u ? 1u : 0u;
        }
        __syncthreads();
        if (last) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // one partial per thread (all loads in flight), then per head a sum over b in order
            for (int i0 = 0; i0 < B * H; i0 += kThreads) {
                const int i = i0 + tid;
                red[tid] = i < B * H ? __hip_atomic_load(partial + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
                __syncthreads();
                // red holds units i0 .. i0 + 255 (unit = b * H + h)
                for (int h = tid; h < H; h += kThreads) {
                    float sum = i0 == 0 ? 0.f : ddecay[h];
                    for (int u = h + ((i0 - h + H - 1) / H) * H; u < i0 + kThreads && u < B * H; u += H)
                        sum += red[u - i0];
                    ddecay[h] = sum;
                }
                __syncthreads();
            }
            if (tid == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---- the normalised form's gradients through unnormalised fp32 scans ----------------
__global__ __launch_bounds__(kThreads) void cast_up(const uint16_t *in, float *out, size_t n8) {
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (size_t)gridDim.x * kThreads) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(in + 8 * i);
        *reinterpret_cast<f32x4 *>(out + 8 * i) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
        *reinterpret_cast<f32x4 *>(out + 8 * i + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    }
}

__global__ __launch_bounds__(kThreads) void cast_down(const float *in, uint16_t *out, size_t n8) {
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (size_t)gridDim.x * kThreads) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(in + 8 * i);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(in + 8 * i + 4);
        *reinterpret_cast<u32x4 *>(out + 8 * i) =
            u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    }
}

__global__ __launch_bounds__(kThreads) void ones16(float *out, size_t n4) {   // n4 = rows * 4
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (size_t)gridDim.x * kThreads)
        *reinterpret_cast<f32x4 *>(out + 4 * i) = f32x4{(i & 3) == 0 ? 1.f : 0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(kThreads) void pad16(const float *src, float *out, int units, int D, int col0) {
    const size_t total = (size_t)units * D * 16;
    for (size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (size_t)gridDim.x * kThreads) {
        const size_t u = g / ((size_t)D * 16);
        const int e = (int)(g - u * D * 16);
        // col0: element (i, j) of a D x 16 matrix; else (j, i) of a 16 x D one
        const int i = col0 ? e / 16 : e % D, j = col0 ? e % 16 : e / D;
        out[g] = (j == 0 && src) ? src[u * D + i] : 0.f;
    }
}

__global__ __launch_bounds__(kThreads) void concat_state(const float *S, const float *z, int zstride, float *out,
                                                          int units, int D1, int D2) {
    const int D = D1 + D2;
    const size_t total = (size_t)units * D;
    for (size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (size_t)gridDim.x * kThreads) {
        const size_t u = g / D;
        const int e = (int)(g - u * D);
        if (e < D1) out[g] = S ? S[u * D1 + e] : 0.f;
        else out[g] = z ? z[(u * D2 + (e - D1)) * zstride] : 0.f;
    }
}

__global__ __launch_bounds__(kThreads) void row0(const float *in, float *out, int units, int D) {
    const size_t total = (size_t)units * D;
    for (size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (size_t)gridDim.x * kThreads) {
        const size_t u = g / D;
        out[g] = in[u * 16 * D + (g - u * D)];
    }
}

// One wave per row (grid-stride over rows); each lane takes columns lane, lane + 64.
__global__ __launch_bounds__(kThreads) void norm_terms(const uint16_t *dy, float *na, const float *d16, float *c16,
                                                       long rows, int Dv) {
    const int lane = threadIdx.x & 63;
    const long w0 = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    for (long r = w0; r < rows; r += (long)gridDim.x * (kThreads / 64)) {
        const float inv = 1.f / d16[r * 16];
        float dv[2], nv[2];
        float dyy = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = lane + 64 * j;
            dv[j] = e < Dv ? bf16_bits_to_f32(dy[r * Dv + e]) : 0.f;
            nv[j] = e < Dv ? na[r * Dv + e] : 0.f;
            dyy = fmaf(dv[j], nv[j], dyy);
        }
        for (int m = 1; m < 64; m <<= 1) dyy += __shfl_xor(dyy, m, 64);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = lane + 64 * j;
            if (e < Dv) na[r * Dv + e] = dv[j] * inv;
        }
        if (lane < 16) c16[r * 16 + lane] = lane == 0 ? -dyy * inv * inv : 0.f;
    }
}

unsigned blocks_for(size_t n) {
    size_t b = (n + kThreads - 1) / kThreads;
    return (unsigned)(b > 16384 ? 16384 : (b < 1 ? 1 : b));
}

}  // namespace

hipError_t transpose_units_launch(const float *in, float *out, int units, int R, int C, hipStream_t s) {
    hipLaunchKernelGGL(transpose_units, dim3(blocks_for((size_t)units * R * C)), dim3(kThreads), 0, s, in, out,
                       units, R, C);
    return hipGetLastError();
}

hipError_t shift_decay_launch(const float *decay, int mode, float *out, int units, int H, int T, int reverse,
                              hipStream_t s) {
    hipLaunchKernelGGL(shift_decay, dim3(blocks_for((size_t)units * T)), dim3(kThreads), 0, s, decay, mode, out,
                       units, H, T, reverse);
    return hipGetLastError();
}

hipError_t scale_state_launch(const float *in, const float *decay, int mode, float *out, int units, int H, int T,
                              int D, int reverse, hipStream_t s) {
    hipLaunchKernelGGL(scale_state, dim3(blocks_for((size_t)units * D)), dim3(kThreads), 0, s, in, decay, mode, out,
                       units, H, T, D, reverse);
    return hipGetLastError();
}

hipError_t decay_terms_launch(const float *q, const float *dq, const float *k, const float *dk, float *c,
                              long rows, int Dk, hipStream_t s) {
    const int lpr = Dk / 4;
    const long rows_per_block = (long)(kThreads / 64) * (64 / lpr);
    const unsigned grid = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(decay_terms, dim3(grid), dim3(kThreads), 0, s, q, dq, k, dk, c, rows, Dk);
    return hipGetLastError();
}

hipError_t decay_terms_cast_launch(const void *q, const float *dq, const void *k, const float *dk, float *c,
                                   void *dq_out, void *dk_out, long rows, int Dk, hipStream_t s) {
    const int lpr = Dk / 8;
    const long rows_per_block = (long)(kThreads / 64) * (64 / lpr);
    const unsigned grid = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(decay_terms_cast, dim3(grid), dim3(kThreads), 0, s, static_cast<const uint16_t *>(q), dq,
                       static_cast<const uint16_t *>(k), dk, c, static_cast<uint16_t *>(dq_out),
                       static_cast<uint16_t *>(dk_out), rows, Dk);
    return hipGetLastError();
}

hipError_t cast_up_launch(const void *in, float *out, size_t n, hipStream_t s) {
    hipLaunchKernelGGL(cast_up, dim3(blocks_for(n / 8)), dim3(kThreads), 0, s, static_cast<const uint16_t *>(in), out,
                       n / 8);
    return hipGetLastError();
}

hipError_t cast_down_launch(const float *in, void *out, size_t n, hipStream_t s) {
    hipLaunchKernelGGL(cast_down, dim3(blocks_for(n / 8)), dim3(kThreads), 0, s, in, static_cast<uint16_t *>(out),
                       n / 8);
    return hipGetLastError();
}

hipError_t ones16_launch(float *out, size_t rows, hipStream_t s) {
    hipLaunchKernelGGL(ones16, dim3(blocks_for(rows * 4)), dim3(kThreads), 0, s, out, rows * 4);
    return hipGetLastError();
}

hipError_t pad16_launch(const float *src, float *out, int units, int D, bool col0, hipStream_t s) {
    hipLaunchKernelGGL(pad16, dim3(blocks_for((size_t)units * D * 16)), dim3(kThreads), 0, s, src, out, units, D,
                       col0 ? 1 : 0);
    return hipGetLastError();
}

hipError_t concat_state_launch(const float *S, const float *z, int zstride, float *out, int units, int D1, int D2,
                               hipStream_t s) {
    hipLaunchKernelGGL(concat_state, dim3(blocks_for((size_t)units * (D1 + D2))), dim3(kThreads), 0, s, S, z, zstride,
                       out, units, D1, D2);
    return hipGetLastError();
}

hipError_t row0_launch(const float *in, float *out, int units, int D, hipStream_t s) {
    hipLaunchKernelGGL(row0, dim3(blocks_for((size_t)units * D)), dim3(kThreads), 0, s, in, out, units, D);
    return hipGetLastError();
}

hipError_t norm_terms_launch(const void *dy, float *na, const float *d16, float *c16, long rows, int Dv,
                             hipStream_t s) {
    hipLaunchKernelGGL(norm_terms, dim3(blocks_for((size_t)rows * 64)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t *>(dy), na, d16, c16, rows, Dv);
    return hipGetLastError();
}

hipError_t decay_grad_launch(const float *c, const float *decay, int mode, const float *dsf, const float *sfin,
                             int D, float *ddecay, float *partial, int B, int H, int T, int reverse,
                             const float *ds0, float *ds_in, unsigned *done, hipStream_t s) {
    hipLaunchKernelGGL(decay_grad, dim3((unsigned)(B * H)), dim3(kThreads), 0, s, c, decay, mode, dsf, sfin, D,
                       ddecay, partial, H, T, reverse, ds0, ds_in, done, B);
    return hipGetLastError();
}


}  // namespace drs
