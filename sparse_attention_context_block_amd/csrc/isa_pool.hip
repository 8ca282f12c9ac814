// Block-mean pooling of Q, K and V: the block representatives of pooling
// attention ([summary] 2 "Pooling Attention"; [notes] key design 2 calls K^c
// and V^c the representative value of a block).  One workgroup per (block,
// head); fp64 accumulation, so the fp64 means of bf16 inputs are exact.
//
// Outputs: qc, kc [BH][n_q][D] fp64 (the coarse stage runs in fp64), and
// kc_lp, vc_lp [BH][n_q][D] in the input dtype (operands of the Taylor path).
#include "isa_internal.h"

namespace isa {
namespace {

template <typename T> struct Elt;
template <> struct Elt<bf16_bits> {
  static constexpr int kPerChunk = 8;  // 16 bytes
  __device__ static void unpack(const uint4& u, double* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (double)__uint_as_float(w[i] << 16);
      out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static bf16_bits from_double(double x) {
    return __builtin_bit_cast(bf16_bits, (__bf16)(float)x);
  }
};
template <> struct Elt<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const uint4& u, double* out) {
    out[0] = (double)__uint_as_float(u.x);
    out[1] = (double)__uint_as_float(u.y);
    out[2] = (double)__uint_as_float(u.z);
    out[3] = (double)__uint_as_float(u.w);
  }
  __device__ static float from_double(double x) { return (float)x; }
};

constexpr int kThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int N, int L_src,
    int n_src, int n_q, int block, double* __restrict__ qc, double* __restrict__ kc,
    T* __restrict__ kc_lp, T* __restrict__ vc_lp) {
  constexpr int EPC = Elt<T>::kPerChunk;
  constexpr int CH = D / EPC;          // 16-byte chunks per row
  constexpr int RP = kThreads / CH;    // rows covered per pass
  __shared__ double red[3][RP][D];

  const int blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  // block grid: source blocks from 0, context blocks from L_src, each segment
  // cut from its own start (the last block of a segment may be partial)
  int start, end;
  if (blk < n_src) {
    start = blk * block;
    end = min(start + block, L_src);
  } else {
    start = L_src + (blk - n_src) * block;
    end = min(start + block, N);
  }
  const int rows = end - start;
  const int c = tid % CH;
  const int r0 = tid / CH;

  double acc[3][EPC];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[t][e] = 0.0;

  const int64_t base = (bh * N + start) * (int64_t)D + c * EPC;
  for (int r = r0; r < rows; r += RP) {
    const int64_t off = base + (int64_t)r * D;
    const uint4 uq = *reinterpret_cast<const uint4*>(Q + off);
    const uint4 uk = *reinterpret_cast<const uint4*>(K + off);
    const uint4 uv = *reinterpret_cast<const uint4*>(V + off);
    double x[EPC];
    Elt<T>::unpack(uq, x);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[0][e] += x[e];
    Elt<T>::unpack(uk, x);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[1][e] += x[e];
    Elt<T>::unpack(uv, x);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[2][e] += x[e];
  }
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < EPC; ++e) red[t][r0][c * EPC + e] = acc[t][e];
  __syncthreads();

  const int64_t out = (bh * n_q + blk) * (int64_t)D;
  for (int idx = tid; idx < 3 * D; idx += kThreads) {
    const int t = idx / D, d = idx % D;
    double s = 0.0;
#pragma unroll
    for (int g = 0; g < RP; ++g) s += red[t][g][d];  // fixed order
    const double mean = s / (double)rows;
    if (t == 0) {
      qc[out + d] = mean;
    } else if (t == 1) {
      kc[out + d] = mean;
      kc_lp[out + d] = Elt<T>::from_double(mean);
    } else {
      vc_lp[out + d] = Elt<T>::from_double(mean);
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const void* Q, const void* K, const void* V, int BH, int N, int D_,
                        int L_src, int n_src, int n_q, int block, double* qc, double* kc,
                        void* kc_lp, void* vc_lp, hipStream_t stream) {
  (void)D_;
  dim3 grid(n_q, BH);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(Q), static_cast<const T*>(K),
                     static_cast<const T*>(V), N, L_src, n_src, n_q, block, qc, kc,
                     static_cast<T*>(kc_lp), static_cast<T*>(vc_lp));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const void* Q, const void* K, const void* V, isa_dtype_t dtype, int BH,
                       int N, int D, int L_src, int n_src, int n_q, int block, double* qc,
                       double* kc, void* kc_lp, void* vc_lp, hipStream_t stream) {
  if (BH == 0 || n_q == 0) return hipSuccess;
  if (dtype == ISA_DTYPE_BF16) {
    if (D == 128)
      return launch_typed<bf16_bits, 128>(Q, K, V, BH, N, D, L_src, n_src, n_q, block, qc, kc,
                                          kc_lp, vc_lp, stream);
    return launch_typed<bf16_bits, 64>(Q, K, V, BH, N, D, L_src, n_src, n_q, block, qc, kc,
                                       kc_lp, vc_lp, stream);
  }
  if (D == 128)
    return launch_typed<float, 128>(Q, K, V, BH, N, D, L_src, n_src, n_q, block, qc, kc, kc_lp,
                                    vc_lp, stream);
  return launch_typed<float, 64>(Q, K, V, BH, N, D, L_src, n_src, n_q, block, qc, kc, kc_lp,
                                 vc_lp, stream);
}

}  // namespace isa
