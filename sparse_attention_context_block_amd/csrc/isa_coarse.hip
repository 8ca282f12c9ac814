// Coarse stage of pooling attention, in fp64 ([summary] 2 "Pooling
// Attention": a coarse attention map between pooled queries and pooled keys).
//
// x_ij = Q^c_i . K^c_j / sqrt(D) and S_coarse = row softmax of x.  The map
// itself is never stored: two kernels keep only what the method reads from it.
//
//   rowstats: per query block i, the row max m_i, l_i = sum_j e^{x_ij - m_i},
//             and the sharpness M_i = Var_j(S_coarse[i, j])
//             ([notes] key design 3), from l_i and q_i = sum_j e^{2(x_ij - m_i)}:
//             M_i = (N_K q_i - l_i^2) / (N_K^2 l_i^2).  In fp64 this has a
//             relative error of about 1e-11 at N_K = 800, far below any gap the
//             routing compares, and it is exactly 0 for a uniform row.
//             With alpha_ns > 0 it also stores every x_ij (fp64), which the
//             block mask of the flat query blocks ranks.
//   colsum:   per context block j, c_j = mean over source query blocks i of
//             S_coarse[i, n_src + j] ([notes] key design 1), reduced in a fixed
//             order (no atomics), so the result is deterministic.
//
// Both kernels tile x as a small fp64 GEMM: 32 query blocks x 32 key blocks
// per step, operands staged transposed in LDS, 2x2 outputs per thread.
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kT = 32;         // tile edge (rows and columns)
constexpr int kThreads = 256;  // 16 x 16 threads, 2 x 2 outputs each

// Stage rows [r0, r0 + kT) of src ([n][D] fp64) transposed into dst[D][kT];
// rows outside [0, n) are zero.
template <int D>
__device__ inline void stage_transposed(double (*dst)[kT], const double* __restrict__ src,
                                        int r0, int n) {
  constexpr int kPairs = kT * D / 2;
  for (int i = threadIdx.x; i < kPairs; i += kThreads) {
    const int r = i / (D / 2);
    const int d = (i % (D / 2)) * 2;
    double2 v = make_double2(0.0, 0.0);
    if (r0 + r < n) v = *reinterpret_cast<const double2*>(src + (int64_t)(r0 + r) * D + d);
    dst[d][r] = v.x;
    dst[d + 1][r] = v.y;
  }
}

// acc[a][b] = sum_d QT[d][2*tr + a] * KT[d][2*tc + b]
template <int D>
__device__ inline void tile_dot(const double (*QT)[kT], const double (*KT)[kT], int tr, int tc,
                                double acc[2][2]) {
  acc[0][0] = acc[0][1] = acc[1][0] = acc[1][1] = 0.0;
#pragma unroll 8
  for (int d = 0; d < D; ++d) {
    const double2 a = *reinterpret_cast<const double2*>(&QT[d][2 * tr]);
    const double2 b = *reinterpret_cast<const double2*>(&KT[d][2 * tc]);
    acc[0][0] = fma(a.x, b.x, acc[0][0]);
    acc[0][1] = fma(a.x, b.y, acc[0][1]);
    acc[1][0] = fma(a.y, b.x, acc[1][0]);
    acc[1][1] = fma(a.y, b.y, acc[1][1]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(
    const double* __restrict__ qc, const double* __restrict__ kc, int n_q, double scale,
    double* __restrict__ rowmax, double* __restrict__ rowsum, double* __restrict__ sharpness,
    double* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) double QT[D][kT];
  __shared__ __attribute__((aligned(16))) double KT[D][kT];
  const int64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * kT;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // a row's 16 threads share one wave
  const double* q = qc + bh * n_q * (int64_t)D;
  const double* k = kc + bh * n_q * (int64_t)D;

  stage_transposed<D>(QT, q, r0, n_q);
  double m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0, 0.0}, s2[2] = {0.0, 0.0};
  for (int c0 = 0; c0 < n_q; c0 += kT) {
    __syncthreads();
    stage_transposed<D>(KT, k, c0, n_q);
    __syncthreads();
    double acc[2][2];
    tile_dot<D>(QT, KT, tr, tc, acc);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (c0 + 2 * tc + b >= n_q) continue;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const double x = acc[a][b] * scale;
        if (logits && r0 + 2 * tr + a < n_q)
          logits[(bh * n_q + r0 + 2 * tr + a) * (int64_t)n_q + c0 + 2 * tc + b] = x;
        if (x > m[a]) {
          const double f = exp(m[a] - x);  // 0 when m is -inf
          l[a] *= f;
          s2[a] *= f * f;
          m[a] = x;
        }
        const double e = exp(x - m[a]);
        l[a] += e;
        s2[a] += e * e;
      }
    }
  }
  // combine the 16 column threads of each row (lanes differing in bits 0..3)
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const double mo = __shfl_xor(m[a], off);
      const double lo = __shfl_xor(l[a], off);
      const double so = __shfl_xor(s2[a], off);
      const double mn = fmax(m[a], mo);
      const double fa = (m[a] == -INFINITY) ? 0.0 : exp(m[a] - mn);
      const double fb = (mo == -INFINITY) ? 0.0 : exp(mo - mn);
      l[a] = l[a] * fa + lo * fb;
      s2[a] = s2[a] * fa * fa + so * fb * fb;
      m[a] = mn;
    }
  }
  if (tc == 0) {
    const double nk = (double)n_q;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int r = r0 + 2 * tr + a;
      if (r >= n_q) continue;
      const int64_t o = bh * n_q + r;
      rowmax[o] = m[a];
      rowsum[o] = l[a];
      const double num = nk * s2[a] - l[a] * l[a];
      sharpness[o] = num / (nk * nk * l[a] * l[a]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void colsum_kernel(
    const double* __restrict__ qc, const double* __restrict__ kc,
    const double* __restrict__ rowmax, const double* __restrict__ rowsum, int n_q, int n_src,
    int n_ctx, double scale, double* __restrict__ ctx_score) {
  __shared__ __attribute__((aligned(16))) double QT[D][kT];
  __shared__ __attribute__((aligned(16))) double KT[D][kT];
  __shared__ double mrow[kT], inv_lrow[kT];
  __shared__ double part[kThreads / 16][kT];
  const int64_t bh = blockIdx.y;
  const int c0 = blockIdx.x * kT;  // context column tile
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  const double* q = qc + bh * n_q * (int64_t)D;
  const double* k = kc + (bh * n_q + n_src) * (int64_t)D;

  stage_transposed<D>(KT, k, c0, n_ctx);
  double colacc[2] = {0.0, 0.0};
  for (int r0 = 0; r0 < n_src; r0 += kT) {
    __syncthreads();
    stage_transposed<D>(QT, q, r0, n_src);
    if (tid < kT) {
      const int r = r0 + tid;
      mrow[tid] = r < n_src ? rowmax[bh * n_q + r] : 0.0;
      inv_lrow[tid] = r < n_src ? 1.0 / rowsum[bh * n_q + r] : 0.0;
    }
    __syncthreads();
    double acc[2][2];
    tile_dot<D>(QT, KT, tr, tc, acc);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int rl = 2 * tr + a;
      if (r0 + rl >= n_src) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
        colacc[b] += exp(acc[a][b] * scale - mrow[rl]) * inv_lrow[rl];
    }
  }
  part[tr][2 * tc] = colacc[0];
  part[tr][2 * tc + 1] = colacc[1];
  __syncthreads();
  if (tid < kT) {
    const int j = c0 + tid;
    if (j < n_ctx) {
      double s = 0.0;
#pragma unroll
      for (int g = 0; g < kThreads / 16; ++g) s += part[g][tid];  // fixed order
      ctx_score[bh * n_ctx + j] = s / (double)n_src;
    }
  }
}

}  // namespace

hipError_t launch_coarse_rowstats(const double* qc, const double* kc, int BH, int n_q, int D,
                                  double* rowmax, double* rowsum, double* sharpness,
                                  double* logits, hipStream_t stream) {
  if (BH == 0 || n_q == 0) return hipSuccess;
  dim3 grid((n_q + kT - 1) / kT, BH);
  const double scale = 1.0 / sqrt((double)D);
  if (D == 128)
    hipLaunchKernelGGL(rowstats_kernel<128>, grid, dim3(kThreads), 0, stream, qc, kc, n_q, scale,
                       rowmax, rowsum, sharpness, logits);
  else
    hipLaunchKernelGGL(rowstats_kernel<64>, grid, dim3(kThreads), 0, stream, qc, kc, n_q, scale,
                       rowmax, rowsum, sharpness, logits);
  return hipGetLastError();
}

hipError_t launch_coarse_colsum(const double* qc, const double* kc, const double* rowmax,
                                const double* rowsum, int BH, int n_q, int n_src, int n_ctx,
                                int D, double* ctx_score, hipStream_t stream) {
  if (BH == 0 || n_ctx == 0 || n_src == 0) return hipSuccess;
  dim3 grid((n_ctx + kT - 1) / kT, BH);
  const double scale = 1.0 / sqrt((double)D);
  if (D == 128)
    hipLaunchKernelGGL(colsum_kernel<128>, grid, dim3(kThreads), 0, stream, qc, kc, rowmax,
                       rowsum, n_q, n_src, n_ctx, scale, ctx_score);
  else
    hipLaunchKernelGGL(colsum_kernel<64>, grid, dim3(kThreads), 0, stream, qc, kc, rowmax,
                       rowsum, n_q, n_src, n_ctx, scale, ctx_score);
  return hipGetLastError();
}

}  // namespace isa
