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
// whose register r of lane group g holds row 4 g + r).  The operands
// come straight from global memory as contiguous runs of D/4 doubles; nothing
// is staged in LDS.  A workgroup's four waves split the tiles of one 16-row
// (rowstats) or 16-column (colsum) strip four ways; their partial results are
// combined in a fixed order (no atomics), so every result is deterministic.
#include "isa_internal.h"

namespace isa {
namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves
constexpr int kTile = 16;

// One lane's part of a 16-row operand tile: row `row` of base ([n][D], n >= 1),
// dims (D/4) g .. + D/4 - 1.  Rows past the end read row n - 1: the results
// they feed are never used.  The load is unconditional, so the wait for one
// operand buffer never includes the other buffer's loads.
template <int D>
__device__ inline void load_part(double (&v)[D / 4], const double* __restrict__ base, int row,
                                 int n, int g) {
  const double2* p =
      reinterpret_cast<const double2*>(base + (int64_t)min(row, n - 1) * D + (D / 4) * g);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const double2 t = p[i];
    v[2 * i] = t.x;
    v[2 * i + 1] = t.y;
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

// Online (max, sum e^{x-m}, sum e^{2(x-m)}) of one row.
struct RowStat {
  double m, l, s2;
};

__device__ inline void stat_add(RowStat& st, double x) {
  if (x > st.m) {
    const double f = exp(st.m - x);  // 0 when m is -inf
    st.l *= f;
    st.s2 *= f * f;
    st.m = x;
  }
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
    double* __restrict__ rowmax, double* __restrict__ rowsum, double* __restrict__ sharpness,
    double* __restrict__ logits) {
  __shared__ RowStat part[4][kTile];
  const int64_t bh = blockIdx.y;
  const int r0 = blockIdx.x * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const double* qh = qc + bh * n_q * (int64_t)D;
  const double* kh = kc + bh * n_q * (int64_t)D;

  double a[D / 4];
  load_part<D>(a, qh, r0 + q, n_q, g);
  RowStat st[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) st[r] = {-INFINITY, 0.0, 0.0};

  const int n_tiles = (n_q + kTile - 1) / kTile;
  auto consume = [&](const f64x4_t& x, int t) __attribute__((always_inline)) {
    const int col = t * kTile + q;
    if (col >= n_q) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double xs = x[r] * scale;
      const int row = r0 + g + 4 * r;
      if (logits && row < n_q) logits[(bh * n_q + row) * (int64_t)n_q + col] = xs;
      stat_add(st[r], xs);
    }
  };
  // the next tile's loads are issued as soon as the MFMAs have read the
  // operand and overlap the exponentials of this tile; the second wave on the
  // SIMD covers the rest of their latency (tile indices past the last tile are
  // clamped, and nothing reads the last load)
  double b[D / 4];
  const int last = n_tiles - 1;
  load_part<D>(b, kh, min(wave, last) * kTile + q, n_q, g);
  for (int t = wave; t < n_tiles; t += 4) {
    const f64x4_t x = tile_dot<D>(a, b);
    load_part<D>(b, kh, min(t + 4, last) * kTile + q, n_q, g);
    consume(x, t);
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
  __shared__ double part[4][kTile];
  const int64_t bh = blockIdx.y;
  const int c0 = blockIdx.x * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const double* qh = qc + bh * n_q * (int64_t)D;
  const double* kh = kc + (bh * n_q + n_src) * (int64_t)D;
  const double* mh = rowmax + bh * n_q;
  const double* lh = rowsum + bh * n_q;

  double bcol[D / 4];
  load_part<D>(bcol, kh, c0 + q, n_ctx, g);
  double colacc = 0.0;
  const int n_tiles = (n_src + kTile - 1) / kTile;
  auto consume = [&](const f64x4_t& x, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = t * kTile + g + 4 * r;
      if (row < n_src) colacc += exp(x[r] * scale - mh[row]) / lh[row];
    }
  };
  double a[D / 4];
  const int last = n_tiles - 1;
  load_part<D>(a, qh, min(wave, last) * kTile + q, n_src, g);
  for (int t = wave; t < n_tiles; t += 4) {
    const f64x4_t x = tile_dot<D>(a, bcol);
    load_part<D>(a, qh, min(t + 4, last) * kTile + q, n_src, g);
    consume(x, t);
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
                                  double* logits, hipStream_t stream) {
  if (BH == 0 || n_q == 0) return hipSuccess;
  dim3 grid((n_q + kTile - 1) / kTile, BH);
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
