// Context Pre-Selection TopK ([notes] key design 1; [summary] 3
// "Pre-Selection") and query grouping by sharpness ([notes] key design 3;
// [summary] 3 "Grouped Computation").  One workgroup per (batch, head).
//
// TopK: keep the k context blocks with the largest c_j, ties to the smaller j.
// Routing: the n_flat query blocks with the smallest M_i (ties to the smaller
// i) take the 0-th order Taylor path; the rest are exact.
//
// Both are exact rank selections: every element's rank under the strict total
// order (key, index) is counted against all others in LDS (n <= 4096 per
// head, so O(n^2) comparisons spread over 256 threads is a few microseconds),
// and the element is kept iff its rank is below the count.  The fp64 values are
// compared through an order-preserving 64-bit integer key, so the order is
// total even for NaN and exactly k (n_flat) elements are kept.  Lists are then
// compacted in ascending index order with a fixed-order block scan.
//
// Outputs: sel [k] ascending, flat [n_flat] and sharp [n_q - n_flat]
// ascending, and the block table of K_new, kv_tab [n_src + k] =
// [0 .. n_src-1, n_src + sel...] (the gather + concat order).
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 256;

__device__ inline uint64_t order_key(double x) {
  const uint64_t u = __double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Writes the indices i < n with flag[i] != 0 to ones (ascending) and, if zeros
// is non-null, the others to zeros (ascending).  Thread t owns a contiguous
// run of the flags; the exclusive prefix of the runs' counts comes from a
// shuffle scan inside each wave plus the totals of the lower waves.
__device__ void compact(const uint8_t* flag, int n, int32_t* ones, int32_t* zeros,
                        int32_t* counts) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kThreads - 1) / kThreads;
  const int b = min(tid * per, n), e = min(b + per, n);
  int c = 0;
  for (int i = b; i < e; ++i) c += flag[i] ? 1 : 0;
  int incl = c;  // inclusive scan over the lanes of this wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) counts[wave] = incl;
  __syncthreads();
  int o1 = incl - c;
  for (int w = 0; w < wave; ++w) o1 += counts[w];
  int o0 = b - o1;  // zeros before b
  for (int i = b; i < e; ++i) {
    if (flag[i])
      ones[o1++] = i;
    else if (zeros)
      zeros[o0++] = i;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void select_route_kernel(
    const double* __restrict__ ctx_score, const double* __restrict__ sharpness, int n_src,
    int n_ctx, int n_q, int k, int n_flat, int32_t* __restrict__ sel, int32_t* __restrict__ flat,
    int32_t* __restrict__ sharp, int32_t* __restrict__ kv_tab) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);                // [n_q]
  uint8_t* flag = smem + sizeof(uint64_t) * kMaxBlocksPerHead;      // [n_q]
  int32_t* counts = reinterpret_cast<int32_t*>(flag + kMaxBlocksPerHead);  // [kThreads]
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* sel_h = sel + bh * k;
  int32_t* tab_h = kv_tab + bh * (int64_t)(n_src + k);

  // ---- TopK over c_j (descending, ties to the smaller j) ----
  for (int j = tid; j < n_ctx; j += kThreads) key[j] = order_key(ctx_score[bh * n_ctx + j]);
  __syncthreads();
  for (int j = tid; j < n_ctx; j += kThreads) {
    const uint64_t kj = key[j];
    int rank = 0;
    for (int i = 0; i < n_ctx; ++i) {
      const uint64_t ki = key[i];
      rank += (ki > kj || (ki == kj && i < j)) ? 1 : 0;
    }
    flag[j] = rank < k ? 1 : 0;
  }
  __syncthreads();
  compact(flag, n_ctx, sel_h, nullptr, counts);
  for (int t = tid; t < n_src + k; t += kThreads)
    tab_h[t] = t < n_src ? t : n_src + sel_h[t - n_src];
  __syncthreads();

  // ---- routing over M_i (ascending, ties to the smaller i) ----
  for (int i = tid; i < n_q; i += kThreads) key[i] = order_key(sharpness[bh * n_q + i]);
  __syncthreads();
  for (int i = tid; i < n_q; i += kThreads) {
    const uint64_t ki = key[i];
    int rank = 0;
    for (int j = 0; j < n_q; ++j) {
      const uint64_t kj = key[j];
      rank += (kj < ki || (kj == ki && j < i)) ? 1 : 0;
    }
    flag[i] = rank < n_flat ? 1 : 0;
  }
  __syncthreads();
  compact(flag, n_q, flat + bh * n_flat, sharp + bh * (int64_t)(n_q - n_flat), counts);
}

// Byte offset of the per-wave counts after key[n] (8 bytes each) and flag[n].
__host__ __device__ inline int ns_counts_offset(int n) { return (9 * n + 15) & ~15; }

// Block mask of one flat query block i ([notes] key design 2; the mask is
// read off the coarse map, [summary] 2 "Pooling Attention"): rank the n_kv
// blocks of K_new by x_i,kv_tab[u] (descending; the coarse probability is
// increasing in x), ties to the smaller position u, and keep the first n_ns,
// listed ascending.  One workgroup per (flat entry, head).
__global__ __launch_bounds__(kThreads) void ns_select_kernel(
    const double* __restrict__ logits, const int32_t* __restrict__ flat,
    const int32_t* __restrict__ kv_tab, int n_q, int n_flat, int n_kv, int n_ns,
    int32_t* __restrict__ ns) {
  // LDS sized by n_kv at launch (a few KB), so many workgroups share a CU
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);                     // [n_kv]
  uint8_t* flag = smem + sizeof(uint64_t) * n_kv;                        // [n_kv]
  int32_t* counts = reinterpret_cast<int32_t*>(smem + ns_counts_offset(n_kv));  // [waves]
  const int f = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int i = flat[bh * n_flat + f];
  const double* row = logits + (bh * n_q + i) * (int64_t)n_q;
  const int32_t* tab = kv_tab + bh * n_kv;
  for (int u = tid; u < n_kv; u += kThreads) key[u] = order_key(row[tab[u]]);
  __syncthreads();
  for (int u = tid; u < n_kv; u += kThreads) {
    const uint64_t ku = key[u];
    int rank = 0;
    for (int v = 0; v < n_kv; ++v) {
      const uint64_t kv = key[v];
      rank += (kv > ku || (kv == ku && v < u)) ? 1 : 0;
    }
    flag[u] = rank < n_ns ? 1 : 0;
  }
  __syncthreads();
  compact(flag, n_kv, ns + (bh * n_flat + f) * (int64_t)n_ns, nullptr, counts);
}

}  // namespace

hipError_t launch_ns_select(const double* logits, const int32_t* flat, const int32_t* kv_tab,
                            int BH, int n_q, int n_flat, int n_kv, int n_ns, int32_t* ns,
                            hipStream_t stream) {
  if (BH == 0 || n_flat == 0 || n_ns == 0) return hipSuccess;
  if (n_kv < 1 || n_kv > kMaxBlocksPerHead || n_ns > n_kv) return hipErrorInvalidValue;
  const size_t lds = ns_counts_offset(n_kv) + sizeof(int32_t) * (kThreads / 64);
  hipLaunchKernelGGL(ns_select_kernel, dim3(n_flat, BH), dim3(kThreads), lds, stream, logits,
                     flat, kv_tab, n_q, n_flat, n_kv, n_ns, ns);
  return hipGetLastError();
}

hipError_t launch_select_route(const double* ctx_score, const double* sharpness, int BH,
                               int n_src, int n_ctx, int n_q, int k, int n_flat, int32_t* sel,
                               int32_t* flat, int32_t* sharp, int32_t* kv_tab,
                               hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  const size_t lds = sizeof(uint64_t) * kMaxBlocksPerHead + kMaxBlocksPerHead +
                     sizeof(int32_t) * kThreads;
  hipLaunchKernelGGL(select_route_kernel, dim3(BH), dim3(kThreads), lds, stream, ctx_score,
                     sharpness, n_src, n_ctx, n_q, k, n_flat, sel, flat, sharp, kv_tab);
  return hipGetLastError();
}

}  // namespace isa
