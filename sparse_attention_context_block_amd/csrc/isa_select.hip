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
// head, so O(n^2) comparisons spread over 1024 threads; an element's count is
// split over several adjacent lanes while there are fewer elements than
// threads, and their integer parts are summed), and the element is kept iff its
// rank is below the count.  The fp64 values are
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
constexpr int kSelThreads = 1024;  // select_route_kernel
typedef double f64x2_t __attribute__((ext_vector_type(2)));

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
  const int per = (n + kSelThreads - 1) / kSelThreads;
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

// flag[j] = 1 iff fewer than `keep` of the n keys precede key j in the strict
// total order `before(key_i, i, key_j, j)`.  Element j's count is taken by P
// adjacent lanes (P a power of two that divides the wave, all lanes of a
// workgroup take the same number of rounds), lane `part` counting the keys
// part, part + P, ...; a butterfly over the P lanes adds the parts.
template <typename Before>
__device__ void rank_flags(const uint64_t* key, int n, int keep, uint8_t* flag, Before before) {
  int P = 1;
  while (P < 64 && P * 2 * n <= kSelThreads) P *= 2;
  const int tid = threadIdx.x;
  for (int base = 0; base < n * P; base += kSelThreads) {
    const int x = base + tid, j = x / P, part = x % P;
    int rank = 0;
    if (j < n) {
      const uint64_t kj = key[j];
      int i = part;
      for (; i + 7 * P < n; i += 8 * P) {  // eight LDS reads in flight
        uint64_t kk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kk[u] = key[i + u * P];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += before(kk[u], i + u * P, kj, j) ? 1 : 0;
      }
      for (; i < n; i += P) rank += before(key[i], i, kj, j) ? 1 : 0;
    }
    for (int off = 1; off < P; off <<= 1) rank += __shfl_xor(rank, off, 64);
    if (j < n && part == 0) flag[j] = rank < keep ? 1 : 0;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_route_kernel(
    const double* __restrict__ ctx_score, const double* __restrict__ sharpness, int n_src,
    int n_ctx, int n_q, int k, int n_flat, int32_t* __restrict__ sel, int32_t* __restrict__ flat,
    int32_t* __restrict__ sharp, int32_t* __restrict__ kv_tab) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);                // [n_q]
  uint8_t* flag = smem + sizeof(uint64_t) * kMaxBlocksPerHead;      // [n_q]
  int32_t* counts = reinterpret_cast<int32_t*>(flag + kMaxBlocksPerHead);  // [waves]
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* sel_h = sel + bh * k;
  int32_t* tab_h = kv_tab + bh * (int64_t)(n_src + k);

  // ---- TopK over c_j (descending, ties to the smaller j) ----
  for (int j = tid; j < n_ctx; j += kSelThreads) key[j] = order_key(ctx_score[bh * n_ctx + j]);
  __syncthreads();
  rank_flags(key, n_ctx, k, flag, [](uint64_t ki, int i, uint64_t kj, int j) {
    return ki > kj || (ki == kj && i < j);
  });
  __syncthreads();
  compact(flag, n_ctx, sel_h, nullptr, counts);
  for (int t = tid; t < n_src + k; t += kSelThreads)
    tab_h[t] = t < n_src ? t : n_src + sel_h[t - n_src];
  __syncthreads();

  // ---- routing over M_i (ascending, ties to the smaller i) ----
  for (int i = tid; i < n_q; i += kSelThreads) key[i] = order_key(sharpness[bh * n_q + i]);
  __syncthreads();
  rank_flags(key, n_q, n_flat, flag, [](uint64_t kj, int j, uint64_t ki, int i) {
    return kj < ki || (kj == ki && j < i);
  });
  __syncthreads();
  compact(flag, n_q, flat + bh * n_flat, sharp + bh * (int64_t)(n_q - n_flat), counts);
}

// Block mask of the flat query blocks ([notes] key design 2; the mask is read
// off the coarse map, [summary] 2 "Pooling Attention"): for flat block i, rank
// the n_kv blocks of K_new by the coarse logit x_i,kv_tab[u] = Q^c_i .
// K^c_kv_tab[u] / sqrt(D) (descending; the coarse probability is increasing in
// x), ties to the smaller position u, and keep the first n_ns, listed
// ascending.  One workgroup per (G consecutive flat entries, head): G = 4
// while the keys of the G rows fit 64 KB of LDS with the rest, else 1.
//
// The logits are computed here, in fp64 from the pooled rows, for the n_kv
// blocks each row ranks only (no [N_Q, N_Q] logit matrix is stored).  16 lanes
// share a pooled key row: each sums D / 16 consecutive dims with fused
// multiply-adds for every flat row of the workgroup, then a fixed-order
// butterfly over the 16 lanes.  The sum runs in another order than the coarse
// map's MFMA tiles, so a logit may differ from the one behind the statistics
// in its last bits; only near-ties can rank differently.
//
// Selection: each wave takes one of the workgroup's rows, with no workgroup
// barrier.  A radix select over the 64-bit order keys finds the n_ns-th
// largest key K* exactly, 8 bits per pass from the top (a wave-private 256-bin
// histogram of the keys that still match the digits found so far; the wave
// then locates the bin that holds the wanted rank).  Kept: every key above K*,
// and of the keys equal to K* the ones with the smallest positions, as many
// as are still wanted.  The kept positions are then listed ascending with a
// wave prefix scan.

// LDS layout for G rows: keys [G][n] (8 bytes each), block table [n], per-wave
// histograms [4][256].
__host__ __device__ inline int ns_tab_offset(int G, int n) { return 8 * G * n; }
__host__ __device__ inline int ns_hist_offset(int G, int n) {
  return (ns_tab_offset(G, n) + 4 * n + 15) & ~15;
}
__host__ __device__ inline int ns_lds_bytes(int G, int n) {
  return ns_hist_offset(G, n) + 4 * 256 * (kThreads / 64);
}

// Orders the wave's LDS accesses: its lanes' LDS operations execute in order,
// and the fence keeps the compiler from moving one lane's reads above another
// lane's writes.
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// One wave: the n_ns largest of key[0..n) (ties to the smaller position),
// written ascending to out[0..n_ns).
__device__ void wave_top(const uint64_t* key, int n, int n_ns, int32_t* hist, int32_t* out) {
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0, mask = 0;
  int want = n_ns;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0;
    wave_fence();
    for (int u = lane; u < n; u += 64) {
      const uint64_t k = key[u];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    wave_fence();
    // lane l owns bins 4 l .. 4 l + 3 (higher lanes: larger digits)
    const int b0 = hist[4 * lane], b1 = hist[4 * lane + 1], b2 = hist[4 * lane + 2],
              b3 = hist[4 * lane + 3];
    const int own = b0 + b1 + b2 + b3;
    int above = own;  // keys in the bins of lanes l .. 63
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_down(above, off);
      if (lane + off < 64) above += y;
    }
    const int higher = above - own;
    // exactly one lane holds the wanted rank: higher < want <= above
    int d = 0, acc = 0;
    const bool mine = higher < want && want <= above;
    if (mine) {
      acc = higher;
      d = 4 * lane + 3;
      const int bins[4] = {b0, b1, b2, b3};
      for (int j = 3; j >= 0; --j) {
        if (acc + bins[j] >= want) {
          d = 4 * lane + j;
          break;
        }
        acc += bins[j];
      }
    }
    const uint64_t who = __builtin_amdgcn_ballot_w64(mine);
    const int src = __builtin_ctzll(who);
    d = __shfl(d, src);
    acc = __shfl(acc, src);
    want -= acc;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)255 << shift;
    wave_fence();
  }
  // prefix is K*; `want` keys equal to it are kept, the smallest positions first
  const int per = (n + 63) / 64;
  const int b = min(lane * per, n), e = min(b + per, n);
  int c = 0, eq = 0;
  for (int u = b; u < e; ++u) {
    const uint64_t k = key[u];
    c += k > prefix ? 1 : 0;
    eq += k == prefix ? 1 : 0;
  }
  // exclusive prefixes of the equal keys and of the kept keys over the lanes
  int eq_incl = eq;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(eq_incl, off);
    if (lane >= off) eq_incl += y;
  }
  int eq_before = eq_incl - eq;
  const int kept = c + max(0, min(eq, want - eq_before));
  int kept_incl = kept;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(kept_incl, off);
    if (lane >= off) kept_incl += y;
  }
  int o = kept_incl - kept;
  for (int u = b; u < e; ++u) {
    const uint64_t k = key[u];
    bool keep = k > prefix;
    if (k == prefix) keep = eq_before++ < want;
    if (keep) out[o++] = u;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void ns_select_kernel(
    const double* __restrict__ qc, const double* __restrict__ kc, double scale,
    const int32_t* __restrict__ flat, const int32_t* __restrict__ kv_tab, int n_q, int n_flat,
    int n_kv, int n_ns, int32_t* __restrict__ ns) {
  static_assert(G <= kThreads / 64, "one wave per row");
  constexpr int kPer = D / 16;  // dims per lane
  constexpr int kRows = 4;      // key rows per group in flight
  constexpr int kGroups = kThreads / 16;
  // LDS sized by n_kv at launch (a few KB at common lengths)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);                           // [G][n_kv]
  int32_t* tab_s = reinterpret_cast<int32_t*>(smem + ns_tab_offset(G, n_kv));  // [n_kv]
  int32_t* hist = reinterpret_cast<int32_t*>(smem + ns_hist_offset(G, n_kv));  // [waves][256]
  const int f0 = blockIdx.x * G;
  const int rows = min(G, n_flat - f0);
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int sub = tid & 15;  // lane within the 16-lane group of one key row
  const int grp = tid >> 4;
  const double* kh = kc + bh * n_q * (int64_t)D;
  for (int u = tid; u < n_kv; u += kThreads) tab_s[u] = kv_tab[bh * n_kv + u];
  // this lane's dims of the workgroup's flat rows (a missing row repeats the
  // first; its keys are never ranked)
  double qv[G][kPer];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int i = flat[bh * n_flat + f0 + (g < rows ? g : 0)];
    const f64x2_t* qrow = reinterpret_cast<const f64x2_t*>(qc + (bh * n_q + i) * (int64_t)D);
#pragma unroll
    for (int c = 0; c < kPer / 2; ++c) {
      const f64x2_t t = qrow[sub * (kPer / 2) + c];
      qv[g][2 * c] = t[0];
      qv[g][2 * c + 1] = t[1];
    }
  }
  __syncthreads();
  // kRows key rows per group in flight (the loads are cache hits whose
  // latency, not their bytes, bounds this loop)
  for (int u0 = grp; u0 < n_kv; u0 += kRows * kGroups) {
    f64x2_t kv[kRows][kPer / 2];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int u = min(u0 + r * kGroups, n_kv - 1);  // (a clamped row is not stored)
      const f64x2_t* krow = reinterpret_cast<const f64x2_t*>(kh + tab_s[u] * (int64_t)D);
#pragma unroll
      for (int c = 0; c < kPer / 2; ++c) kv[r][c] = krow[sub * (kPer / 2) + c];
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int u = u0 + r * kGroups;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < kPer / 2; ++c) {
          acc = fma(qv[g][2 * c], kv[r][c][0], acc);
          acc = fma(qv[g][2 * c + 1], kv[r][c][1], acc);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
        if (sub == 0 && u < n_kv) key[g * n_kv + u] = order_key(acc * scale);
      }
    }
  }
  __syncthreads();
  if (wave < rows)
    wave_top(key + wave * n_kv, n_kv, n_ns, hist + 256 * wave,
             ns + (bh * n_flat + f0 + wave) * (int64_t)n_ns);
}

}  // namespace

hipError_t launch_ns_select(const double* qc, const double* kc, const int32_t* flat,
                            const int32_t* kv_tab, int BH, int n_q, int D, int n_flat, int n_kv,
                            int n_ns, int32_t* ns, hipStream_t stream) {
  if (BH == 0 || n_flat == 0 || n_ns == 0) return hipSuccess;
  if (n_kv < 1 || n_kv > kMaxBlocksPerHead || n_ns > n_kv || (D != 64 && D != 128))
    return hipErrorInvalidValue;
  const double scale = 1.0 / sqrt((double)D);
  const bool four = ns_lds_bytes(4, n_kv) <= 65536;
  const int G = four ? 4 : 1;
  const size_t lds = ns_lds_bytes(G, n_kv);
  const dim3 grid((n_flat + G - 1) / G, BH);
  if (D == 128 && four)
    hipLaunchKernelGGL((ns_select_kernel<128, 4>), grid, dim3(kThreads), lds, stream, qc, kc,
                       scale, flat, kv_tab, n_q, n_flat, n_kv, n_ns, ns);
  else if (D == 128)
    hipLaunchKernelGGL((ns_select_kernel<128, 1>), grid, dim3(kThreads), lds, stream, qc, kc,
                       scale, flat, kv_tab, n_q, n_flat, n_kv, n_ns, ns);
  else if (four)
    hipLaunchKernelGGL((ns_select_kernel<64, 4>), grid, dim3(kThreads), lds, stream, qc, kc,
                       scale, flat, kv_tab, n_q, n_flat, n_kv, n_ns, ns);
  else
    hipLaunchKernelGGL((ns_select_kernel<64, 1>), grid, dim3(kThreads), lds, stream, qc, kc,
                       scale, flat, kv_tab, n_q, n_flat, n_kv, n_ns, ns);
  return hipGetLastError();
}

hipError_t launch_select_route(const double* ctx_score, const double* sharpness, int BH,
                               int n_src, int n_ctx, int n_q, int k, int n_flat, int32_t* sel,
                               int32_t* flat, int32_t* sharp, int32_t* kv_tab,
                               hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  const size_t lds = sizeof(uint64_t) * kMaxBlocksPerHead + kMaxBlocksPerHead +
                     sizeof(int32_t) * (kSelThreads / 64);
  hipLaunchKernelGGL(select_route_kernel, dim3(BH), dim3(kSelThreads), lds, stream, ctx_score,
                     sharpness, n_src, n_ctx, n_q, k, n_flat, sel, flat, sharp, kv_tab);
  return hipGetLastError();
}

}  // namespace isa
