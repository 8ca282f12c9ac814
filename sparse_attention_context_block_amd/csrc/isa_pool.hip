// Block-mean pooling of Q, K and V: the block representatives of pooling
// attention ([summary] 2 "Pooling Attention"; [notes] key design 2 calls K^c
// and V^c the representative value of a block).  One workgroup per (block,
// head), or per (block, group of 8 heads) with the rotation below; fp64
// accumulation, so the fp64 means of bf16 inputs are exact.
//
// Outputs: qc, kc [BH][n_q][D] fp64 (the coarse stage runs in fp64), and
// kc_lp, vc_lp [BH][n_q][D] in the input dtype (operands of the Taylor path).
//
// With the decoupled rotary embedding ([notes] training strategy: source and
// context positions each start at 0) the kernel also rotates Q and K on the
// way: pair (2i, 2i+1) of the token at position pos turns by
// pos * base^(-2i/D) (RoFormer's rotation), computed in fp64 and rounded once,
// to nearest even, to the input dtype.  The rotated rows go to qr, kr (every
// later step reads them) and the block means are taken of the rotated,
// rounded values.
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
  // round x in place to bf16 values and pack them into a chunk
  __device__ static uint4 round_pack(double* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = bf16_bits_rne(x[2 * i]), hi = bf16_bits_rne(x[2 * i + 1]);
      x[2 * i] = (double)__uint_as_float(lo << 16);
      x[2 * i + 1] = (double)__uint_as_float(hi << 16);
      w[i] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static bf16_bits from_double(double x) { return (bf16_bits)bf16_bits_rne(x); }
};
template <> struct Elt<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const uint4& u, double* out) {
    out[0] = (double)__uint_as_float(u.x);
    out[1] = (double)__uint_as_float(u.y);
    out[2] = (double)__uint_as_float(u.z);
    out[3] = (double)__uint_as_float(u.w);
  }
  __device__ static uint4 round_pack(double* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = (float)x[i];
      x[i] = (double)f;
      w[i] = __float_as_uint(f);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ static float from_double(double x) { return (float)x; }
};

// (x, y) turned by the angle with cosine c and sine s, each product and sum
// rounded on its own (no fused multiply-add), as the textbook formula reads.
__device__ inline void rotate_pair(double& x, double& y, double c, double s) {
#pragma clang fp contract(off)
  const double xc = x * c, ys = y * s, xs = x * s, yc = y * c;
  x = xc - ys;
  y = xs + yc;
}

constexpr int kThreads = 256;
constexpr int kRopeHeads = 8;  // heads per workgroup when the kernel also rotates

// kMode: 0 no rotation; 1 rotation with the angles of a block (of at most
// kBlock rows) computed once for a group of kRopeHeads heads; 2 rotation with
// the angles computed per row and head (longer blocks).

template <typename T, int D, int kMode>
__global__ __launch_bounds__(kThreads) void pool_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int BH, int N,
    int L_src, int n_src, int n_q, int block, double* __restrict__ qc, double* __restrict__ kc,
    T* __restrict__ kc_lp, T* __restrict__ vc_lp, T* __restrict__ qr, T* __restrict__ kr,
    RopeFreq rope) {
  constexpr int EPC = Elt<T>::kPerChunk;
  constexpr int CH = D / EPC;          // 16-byte chunks per row
  constexpr int RP = kThreads / CH;    // rows covered per pass
  constexpr bool kRope = kMode != 0;
  constexpr bool kCache = kMode == 1;
  constexpr int JMAX = (kBlock + RP - 1) / RP;  // rows per thread of a block (angle cache)
  // heads per workgroup: with the angle cache, one block's angles serve this many heads
  constexpr int kHeads = kCache ? kRopeHeads : 1;
  // per-wave partial sums (the lanes of a wave are reduced with shuffles first)
  __shared__ double red[3][kThreads / 64][D];

  const int blk = blockIdx.x;
  const int64_t bh0 = (int64_t)blockIdx.y * kHeads;
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

  // rotation angles of this thread's rows (r0 + RP j) and pairs (dims
  // c EPC + 2 p, c EPC + 2 p + 1), computed once for all heads of the group
  double cs[kCache ? JMAX : 1][EPC / 2], sn[kCache ? JMAX : 1][EPC / 2];
  if constexpr (kCache) {
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      const int t = start + r0 + RP * j;
      const double pos = (double)(t < L_src ? t : t - L_src);  // positions restart at the context
#pragma unroll
      for (int pr = 0; pr < EPC / 2; ++pr)
        sincos(pos * rope.inv_freq[c * (EPC / 2) + pr], &sn[j][pr], &cs[j][pr]);
    }
  }

  for (int hh = 0; hh < kHeads; ++hh) {
    const int64_t bh = bh0 + hh;
    if (bh >= BH) break;  // uniform across the workgroup
    double acc[3][EPC];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[t][e] = 0.0;

    const int64_t base = (bh * N + start) * (int64_t)D + c * EPC;
    // rotate (if asked), store the rotated Q and K rows, and add the row's three
    // chunks to the running sums
    auto process = [&](int r, int j, const uint4& uq, const uint4& uk, const uint4& uv)
        __attribute__((always_inline)) {
      const int64_t off = base + (int64_t)r * D;
      double x[EPC], y[EPC];
      Elt<T>::unpack(uq, x);
      Elt<T>::unpack(uk, y);
      if constexpr (kRope) {
#pragma unroll
        for (int pr = 0; pr < EPC / 2; ++pr) {
          double c_, s_;
          if constexpr (kCache) {
            c_ = cs[j][pr];
            s_ = sn[j][pr];
          } else {
            const int t = start + r;
            const double pos = (double)(t < L_src ? t : t - L_src);
            sincos(pos * rope.inv_freq[c * (EPC / 2) + pr], &s_, &c_);
          }
          rotate_pair(x[2 * pr], x[2 * pr + 1], c_, s_);
          rotate_pair(y[2 * pr], y[2 * pr + 1], c_, s_);
        }
        *reinterpret_cast<uint4*>(qr + off) = Elt<T>::round_pack(x);
        *reinterpret_cast<uint4*>(kr + off) = Elt<T>::round_pack(y);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[0][e] += x[e];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[1][e] += y[e];
      Elt<T>::unpack(uv, x);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[2][e] += x[e];
    };
    // every input row is read once here: nontemporal loads (0.200 -> 0.174 ms
    // with warm caches, 0.251 -> 0.196 ms cold at the 32K shape, same box)
    auto load = [&](int r, uint4& uq, uint4& uk, uint4& uv) __attribute__((always_inline)) {
      const int64_t off = base + (int64_t)r * D;
      uq = load_nt(Q + off);
      uk = load_nt(K + off);
      uv = load_nt(V + off);
    };
    if constexpr (kCache) {
      // the launcher guarantees block <= kBlock, so JMAX passes cover a block;
      // all of this head's loads are issued before the first row is processed
      // (unconditionally: rows past a partial block's end read its last row and
      // are not processed; a conditional load makes the wait-count pass hold
      // each group of loads until the previous group has arrived)
      uint4 uq[JMAX], uk[JMAX], uv[JMAX];
#pragma unroll
      for (int j = 0; j < JMAX; ++j) load(min(r0 + RP * j, rows - 1), uq[j], uk[j], uv[j]);
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
        if (r0 + RP * j < rows) process(r0 + RP * j, j, uq[j], uk[j], uv[j]);
    } else {
      // up to four passes' loads in flight before the first row is processed
      // (rows past the end read the last row and are not processed)
      constexpr int kAhead = 4;
      for (int r = r0; r < rows; r += kAhead * RP) {
        uint4 uq[kAhead], uk[kAhead], uv[kAhead];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) load(min(r + RP * j, rows - 1), uq[j], uk[j], uv[j]);
#pragma unroll
        for (int j = 0; j < kAhead; ++j)
          if (r + RP * j < rows) process(r + RP * j, 0, uq[j], uk[j], uv[j]);
      }
    }
    // Sum the row groups: first the lanes of a wave that hold the same dims
    // (lane bits above the chunk index), then the four waves' sums in LDS.
    // Block sums of bf16 (or fp32) values in fp64 are exact, so the order of
    // the additions does not change them.
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = CH; off < 64; off <<= 1)
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[t][e] += __shfl_xor(acc[t][e], off);
    if (lane < CH) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int e = 0; e < EPC; ++e) red[t][wave][c * EPC + e] = acc[t][e];
    }
    __syncthreads();

    const int64_t out = (bh * n_q + blk) * (int64_t)D;
    for (int idx = tid; idx < 3 * D; idx += kThreads) {
      const int t = idx / D, d = idx % D;
      double s = 0.0;
#pragma unroll
      for (int g = 0; g < kThreads / 64; ++g) s += red[t][g][d];
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
    __syncthreads();  // red is reused by the next head
  }
}

// Rotation alone, for the backward with the rotary embedding: Y = X with
// every pair turned by its angle (sign = +1: the forward's rotation, the same
// arithmetic and single rounding as the pooling kernel, so Y equals the
// rotated copy the forward used bit for bit) or turned back (sign = -1: the
// gradient of the rotation, dX = R^T dY).  One thread per (token, 16-byte
// chunk), looping over the heads, so each angle's sine and cosine are computed
// once for all heads.  In place (Y == X) is allowed.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_rotate_kernel(const T* X, T* Y, int BH, int N,
                                                               int L_src, RopeFreq rope,
                                                               double sign) {
  constexpr int EPC = Elt<T>::kPerChunk;
  constexpr int CH = D / EPC;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (int64_t)N * CH) return;
  const int t = (int)(gid / CH), c = (int)(gid % CH);
  const double pos = (double)(t < L_src ? t : t - L_src);
  double cs[EPC / 2], sn[EPC / 2];
#pragma unroll
  for (int pr = 0; pr < EPC / 2; ++pr) {
    sincos(pos * rope.inv_freq[c * (EPC / 2) + pr], &sn[pr], &cs[pr]);
    sn[pr] *= sign;
  }
  for (int bh = 0; bh < BH; ++bh) {
    const int64_t off = ((int64_t)bh * N + t) * D + c * EPC;
    double x[EPC];
    Elt<T>::unpack(*reinterpret_cast<const uint4*>(X + off), x);
#pragma unroll
    for (int pr = 0; pr < EPC / 2; ++pr) rotate_pair(x[2 * pr], x[2 * pr + 1], cs[pr], sn[pr]);
    *reinterpret_cast<uint4*>(Y + off) = Elt<T>::round_pack(x);
  }
}

template <typename T, int D>
hipError_t launch_typed(const void* Q, const void* K, const void* V, int BH, int N,
                        int L_src, int n_src, int n_q, int block, double* qc, double* kc,
                        void* kc_lp, void* vc_lp, void* qr, void* kr, const RopeFreq* rope,
                        hipStream_t stream) {
  if (rope && block > kBlock) {  // the angle cache covers kBlock rows
    dim3 grid(n_q, BH);
    hipLaunchKernelGGL((pool_kernel<T, D, 2>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(Q), static_cast<const T*>(K),
                       static_cast<const T*>(V), BH, N, L_src, n_src, n_q, block, qc, kc,
                       static_cast<T*>(kc_lp), static_cast<T*>(vc_lp), static_cast<T*>(qr),
                       static_cast<T*>(kr), *rope);
  } else if (rope) {
    dim3 grid(n_q, (BH + kRopeHeads - 1) / kRopeHeads);
    hipLaunchKernelGGL((pool_kernel<T, D, 1>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(Q), static_cast<const T*>(K),
                       static_cast<const T*>(V), BH, N, L_src, n_src, n_q, block, qc, kc,
                       static_cast<T*>(kc_lp), static_cast<T*>(vc_lp), static_cast<T*>(qr),
                       static_cast<T*>(kr), *rope);
  } else {
    dim3 grid(n_q, BH);
    hipLaunchKernelGGL((pool_kernel<T, D, 0>), grid, dim3(kThreads), 0, stream,
                       static_cast<const T*>(Q), static_cast<const T*>(K),
                       static_cast<const T*>(V), BH, N, L_src, n_src, n_q, block, qc, kc,
                       static_cast<T*>(kc_lp), static_cast<T*>(vc_lp), nullptr, nullptr,
                       RopeFreq{});
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_rotate(const void* X, void* Y, isa_dtype_t dtype, int BH, int N, int D,
                              int L_src, const RopeFreq& rope, bool inverse, hipStream_t stream) {
  if (BH == 0 || N == 0) return hipSuccess;
  const double sign = inverse ? -1.0 : 1.0;
  const int64_t chunks = (int64_t)N * (D * (dtype == ISA_DTYPE_BF16 ? 2 : 4) / 16);
  const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads));
  if (dtype == ISA_DTYPE_BF16) {
    if (D == 128)
      hipLaunchKernelGGL((rope_rotate_kernel<bf16_bits, 128>), grid, dim3(kThreads), 0, stream,
                         static_cast<const bf16_bits*>(X), static_cast<bf16_bits*>(Y), BH, N,
                         L_src, rope, sign);
    else
      hipLaunchKernelGGL((rope_rotate_kernel<bf16_bits, 64>), grid, dim3(kThreads), 0, stream,
                         static_cast<const bf16_bits*>(X), static_cast<bf16_bits*>(Y), BH, N,
                         L_src, rope, sign);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((rope_rotate_kernel<float, 128>), grid, dim3(kThreads), 0, stream,
                         static_cast<const float*>(X), static_cast<float*>(Y), BH, N, L_src,
                         rope, sign);
    else
      hipLaunchKernelGGL((rope_rotate_kernel<float, 64>), grid, dim3(kThreads), 0, stream,
                         static_cast<const float*>(X), static_cast<float*>(Y), BH, N, L_src,
                         rope, sign);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const void* Q, const void* K, const void* V, isa_dtype_t dtype, int BH,
                       int N, int D, int L_src, int n_src, int n_q, int block, double* qc,
                       double* kc, void* kc_lp, void* vc_lp, void* qr, void* kr,
                       const RopeFreq* rope, hipStream_t stream) {
  if (BH == 0 || n_q == 0) return hipSuccess;
  if (rope && (!qr || !kr)) return hipErrorInvalidValue;
  if (dtype == ISA_DTYPE_BF16) {
    if (D == 128)
      return launch_typed<bf16_bits, 128>(Q, K, V, BH, N, L_src, n_src, n_q, block, qc, kc,
                                          kc_lp, vc_lp, qr, kr, rope, stream);
    return launch_typed<bf16_bits, 64>(Q, K, V, BH, N, L_src, n_src, n_q, block, qc, kc,
                                       kc_lp, vc_lp, qr, kr, rope, stream);
  }
  if (D == 128)
    return launch_typed<float, 128>(Q, K, V, BH, N, L_src, n_src, n_q, block, qc, kc, kc_lp,
                                    vc_lp, qr, kr, rope, stream);
  return launch_typed<float, 64>(Q, K, V, BH, N, L_src, n_src, n_q, block, qc, kc, kc_lp,
                                 vc_lp, qr, kr, rope, stream);
}

}  // namespace isa
