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
//             S_coarse[i, n_src + j] ([notes] key design 1).
//
// Both kernels form x in 16 x 16 tiles with v_mfma_f64_16x16x4_f64.  A lane
// (q, g) (q = lane % 16, g = lane / 16) holds dims (D/4) g .. (D/4) g + D/4 - 1
// of one row of each operand, so step s of a tile multiplies dims (D/4) g + s
// of row q of A and column q of B, and the D/4 steps together sum all D dims.
// The lane then holds x[g + 4 r][q] in register r of the tile (this fp64 MFMA
// spreads the output rows over the lane groups first, unlike the 32-bit ones,
// whose register r of lane group g holds row 4 g + r).  Each wave copies its
// operand tiles (16 contiguous rows) into a private LDS buffer with coalesced
// loads and reads its runs from there.  A workgroup's four waves split the
// tiles of one 16-row (rowstats) or 16-column (colsum) strip four ways; their
// partial results are combined in a fixed order (no atomics), so every result
// is deterministic.
#include "isa_internal.h"

namespace isa {
namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));
// native vector (not HIP's double2 class) so staged values stay in registers
typedef double f64x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // four waves
constexpr int kTile = 16;

// A wave's private LDS copy of one 16-row operand tile ([n][D] fp64 rows
// row0 .. row0 + 15; rows past n - 1 read row n - 1, and the results they feed
// are never used).  The tile's rows are contiguous in memory, so each global
// load instruction reads 1 KB in one piece (lane l: bytes 16 l .. 16 l + 15 of
// its row); rows sit 16 bytes apart more than their length in LDS, which makes
// every ds_read_b128 of read_part below free of bank conflicts for D = 128.
template <int D>
struct WaveTile {
  static constexpr int kRowBytes = D * 8 + 16;
  static constexpr int kBytes = kTile * kRowBytes;
  static constexpr int kLanesPerRow = D * 8 / 16;         // 64 or 32
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // 1 or 2
  static constexpr int kLoads = kTile / kRowsPerLoad;
};

template <int D>
__device__ __forceinline__ void tile_load(f64x2_t (&st)[WaveTile<D>::kLoads],
                                          const double* __restrict__ base, int row0, int n,
                                          int lane) {
  using W = WaveTile<D>;
#pragma unroll
  for (int i = 0; i < W::kLoads; ++i) {
    const int row = min(row0 + i * W::kRowsPerLoad + lane / W::kLanesPerRow, n - 1);
    st[i] = *reinterpret_cast<const f64x2_t*>(base + (int64_t)row * D +
                                              2 * (lane % W::kLanesPerRow));
  }
}

template <int D>
__device__ __forceinline__ void tile_store(const f64x2_t (&st)[WaveTile<D>::kLoads],
                                           unsigned char* lds, int lane) {
  using W = WaveTile<D>;
#pragma unroll
  for (int i = 0; i < W::kLoads; ++i)
    *reinterpret_cast<f64x2_t*>(lds + (i * W::kRowsPerLoad + lane / W::kLanesPerRow) *
                                          W::kRowBytes +
                                16 * (lane % W::kLanesPerRow)) = st[i];
}

// The tile is written and read by the lanes of one wave only, whose LDS
// accesses execute in order; the fence keeps the compiler from moving the
// reads of one lane's operand above the writes of the other lanes.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// Lane (q, g)'s operand from a staged tile: row q, dims (D/4) g .. + D/4 - 1.
template <int D>
__device__ __forceinline__ void read_part(double (&v)[D / 4], const unsigned char* lds, int q,
                                          int g) {
  const unsigned char* p = lds + q * WaveTile<D>::kRowBytes + (D / 4) * 8 * g;
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const f64x2_t t = *reinterpret_cast<const f64x2_t*>(p + 16 * i);
    v[2 * i] = t[0];
    v[2 * i + 1] = t[1];
  }
}

// x[g + 4 r][q] = sum_d A[g + 4 r][d] B[q][d] for the lane (q, g)
template <int D>
__device__ inline f64x4_t tile_dot(const double (&a)[D / 4], const double (&b)[D / 4]) {
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < D / 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// Online (m, sum e^{x-m}, sum e^{2(x-m)}) of one row.  m is a reference
// point, not necessarily the row max: it is raised only when a logit exceeds
// it by more than kLazy (e^16 keeps every term and sum far inside fp64), so
// most tiles need one exponential per logit.  The stored pair (m, l) is
// consistent for any m, and M_i = (N q - l^2) / (N^2 l^2) is a ratio in
// which the factor e^{-m} cancels.
constexpr double kLazy = 16.0;

struct RowStat {
  double m, l, s2;
};

__device__ inline void stat_raise(RowStat& st, double x) {
  if (x > st.m) {
    const double f = exp(st.m - x);  // 0 when m is -inf
    st.l *= f;
    st.s2 *= f * f;
    st.m = x;
  }
}

__device__ inline void stat_accumulate(RowStat& st, double x) {
  const double e = exp(x - st.m);
  st.l += e;
  st.s2 += e * e;
}

__device__ inline RowStat stat_merge(const RowStat& a, const RowStat& b) {
  const double mn = fmax(a.m, b.m);
  const double fa = (a.m == -INFINITY) ? 0.0 : exp(a.m - mn);
  const double fb = (b.m == -INFINITY) ? 0.0 : exp(b.m - mn);
  return {mn, a.l * fa + b.l * fb, a.s2 * fa * fa + b.s2 * fb * fb};
}

// One workgroup = 16 query blocks (rows); wave w takes the key tiles t = w,
// w + 4, ... and keeps per-lane statistics of its rows g, g + 4, g + 8, g + 12.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void rowstats_kernel(
    const double* __restrict__ qc, const double* __restrict__ kc, int n_q, double scale,
    double* __restrict__ rowmax, double* __restrict__ rowsum, double* __restrict__ sharpness) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[4][WaveTile<D>::kBytes];
  __shared__ RowStat part[4][kTile];
  const int64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const double* qh = qc + bh * n_q * (int64_t)D;
  const double* kh = kc + bh * n_q * (int64_t)D;
  unsigned char* my = tiles[wave];
  const int n_tiles = (n_q + kTile - 1) / kTile;
  const int last = n_tiles - 1;

  f64x2_t stg[WaveTile<D>::kLoads];
  double a[D / 4];
  tile_load<D>(stg, qh, r0, n_q, lane);
  tile_store<D>(stg, my, lane);
  wave_lds_fence();
  read_part<D>(a, my, q, g);
  wave_lds_fence();
  tile_load<D>(stg, kh, min(wave, last) * kTile, n_q, lane);

  RowStat st[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) st[r] = {-INFINITY, 0.0, 0.0};
  for (int t = wave; t < n_tiles; t += 4) {
    tile_store<D>(stg, my, lane);
    wave_lds_fence();
    // the next tile's loads overlap this tile's MFMAs and exponentials (the
    // tile index is clamped; nothing reads the last load)
    tile_load<D>(stg, kh, min(t + 4, last) * kTile, n_q, lane);
    double b[D / 4];
    read_part<D>(b, my, q, g);
    wave_lds_fence();
    const f64x4_t x = tile_dot<D>(a, b);
    const int col = t * kTile + q;
    const bool col_ok = col < n_q;
    double xs[4];
    bool raise = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xs[r] = x[r] * scale;
      raise |= col_ok && xs[r] > st[r].m + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // uniform branch, rare after the first tile
      if (col_ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) stat_raise(st[r], xs[r]);
      }
    }
    if (col_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        stat_accumulate(st[r], xs[r]);
      }
    }
  }
  // merge the 16 column lanes of each row (lanes differing in bits 0..3)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const RowStat o = {__shfl_xor(st[r].m, off), __shfl_xor(st[r].l, off),
                         __shfl_xor(st[r].s2, off)};
      st[r] = stat_merge(st[r], o);
    }
  }
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][g + 4 * r] = st[r];
  }
  __syncthreads();
  if (threadIdx.x < kTile) {
    const int row = r0 + threadIdx.x;
    if (row < n_q) {
      RowStat s = part[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) s = stat_merge(s, part[w][threadIdx.x]);  // fixed order
      const double nk = (double)n_q;
      const int64_t o = bh * n_q + row;
      rowmax[o] = s.m;
      rowsum[o] = s.l;
      sharpness[o] = (nk * s.s2 - s.l * s.l) / (nk * nk * s.l * s.l);
    }
  }
}

// One workgroup = 16 context blocks (columns); wave w takes the source row
// tiles t = w, w + 4, ...; lane (q, g) sums the probabilities of its rows
// g, g + 4, g + 8, g + 12 into column q.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void colsum_kernel(
    const double* __restrict__ qc, const double* __restrict__ kc,
    const double* __restrict__ rowmax, const double* __restrict__ rowsum, int n_q, int n_src,
    int n_ctx, double scale, double* __restrict__ ctx_score) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[4][WaveTile<D>::kBytes];
  __shared__ double part[4][kTile];
  const int64_t bh = blockIdx.y;
  const int c0 = blockIdx.x * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const double* qh = qc + bh * n_q * (int64_t)D;
  const double* kh = kc + (bh * n_q + n_src) * (int64_t)D;
  const double* mh = rowmax + bh * n_q;
  const double* lh = rowsum + bh * n_q;
  unsigned char* my = tiles[wave];
  const int n_tiles = (n_src + kTile - 1) / kTile;
  const int last = n_tiles - 1;

  f64x2_t stg[WaveTile<D>::kLoads];
  double bcol[D / 4];
  tile_load<D>(stg, kh, c0, n_ctx, lane);
  tile_store<D>(stg, my, lane);
  wave_lds_fence();
  read_part<D>(bcol, my, q, g);
  wave_lds_fence();
  // row statistics of the lane's rows travel with their tile
  auto row_stats = [&](int t, double (&m)[4], double (&il)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(t * kTile + g + 4 * r, n_src - 1);
      m[r] = mh[row];
      il[r] = 1.0 / lh[row];
    }
  };
  double m[4], l[4];
  tile_load<D>(stg, qh, min(wave, last) * kTile, n_src, lane);
  row_stats(min(wave, last), m, l);

  double colacc = 0.0;
  for (int t = wave; t < n_tiles; t += 4) {
    tile_store<D>(stg, my, lane);
    wave_lds_fence();
    const double mc[4] = {m[0], m[1], m[2], m[3]}, ilc[4] = {l[0], l[1], l[2], l[3]};
    tile_load<D>(stg, qh, min(t + 4, last) * kTile, n_src, lane);
    row_stats(min(t + 4, last), m, l);
    double a[D / 4];
    read_part<D>(a, my, q, g);
    wave_lds_fence();
    const f64x4_t x = tile_dot<D>(a, bcol);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = t * kTile + g + 4 * r;
      if (row < n_src) colacc += exp(x[r] * scale - mc[r]) * ilc[r];
    }
  }
  // column q: the four lane groups in order, then the four waves in order
  colacc += __shfl_xor(colacc, 16);
  colacc += __shfl_xor(colacc, 32);
  if (g == 0) part[wave][q] = colacc;
  __syncthreads();
  if (threadIdx.x < kTile) {
    const int j = c0 + threadIdx.x;
    if (j < n_ctx) {
      const double s = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                       part[3][threadIdx.x];
      ctx_score[bh * n_ctx + j] = s / (double)n_src;
    }
  }
}

}  // namespace

hipError_t launch_coarse_rowstats(const double* qc, const double* kc, int BH, int n_q, int D,
                                  double* rowmax, double* rowsum, double* sharpness,
                                  hipStream_t stream) {
  if (BH == 0 || n_q == 0) return hipSuccess;
  dim3 grid((n_q + kTile - 1) / kTile, BH);
  const double scale = 1.0 / sqrt((double)D);
  if (D == 128)
    hipLaunchKernelGGL(rowstats_kernel<128>, grid, dim3(kThreads), 0, stream, qc, kc, n_q, scale,
                       rowmax, rowsum, sharpness);
  else
    hipLaunchKernelGGL(rowstats_kernel<64>, grid, dim3(kThreads), 0, stream, qc, kc, n_q, scale,
                       rowmax, rowsum, sharpness);
  return hipGetLastError();
}

hipError_t launch_coarse_colsum(const double* qc, const double* kc, const double* rowmax,
                                const double* rowsum, int BH, int n_q, int n_src, int n_ctx,
                                int D, double* ctx_score, hipStream_t stream) {
  if (BH == 0 || n_ctx == 0 || n_src == 0) return hipSuccess;
  dim3 grid((n_ctx + kTile - 1) / kTile, BH);
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
