// fp32 online-softmax attention on the vector ALUs: the FP32 variant of the
// exact path, the 0-th order Taylor path and the dense baseline ([notes] key
// design 2), taking the same AttnParams block tables as the bf16 MFMA kernel.
// It serves small fp32 problems; it is not tuned for throughput.
//
// Workgroup = one 64-row query block; 4 threads per query row, each owning a
// quarter of D.  Keys stream through LDS in 32-row tiles.
#include "isa_debug.h"
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int DP = D / 4;  // dims per thread
  __shared__ __attribute__((aligned(16))) float Ks[kTile][D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile][D];
  const int64_t bh = blockIdx.y;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int row = tid >> 2, part = tid & 3;
  // query row: row 31 & row of slice 2e + row / 32 of the query list; rows past
  // a partial block's end read the slice's first row and are not stored
  const int32_t* qlist = p.q_tab ? p.q_tab + bh * p.q_tab_stride : nullptr;
  const Slice qs = list_slice(p.grid, qlist, p.n_q_slices, p.half_shift, 2 * e + (row >> 5));
  const bool q_ok = (row & 31) < qs.cnt;
  const int64_t qrow = (int64_t)qs.start + (q_ok ? (row & 31) : 0);
  const float* Qh = static_cast<const float*>(p.q) + bh * p.q_head_stride;
  const float* Kh = static_cast<const float*>(p.k) + bh * p.kv_head_stride;
  const float* Vh = static_cast<const float*>(p.v) + bh * p.kv_head_stride;
  const int32_t* tab = p.kv_tab ? p.kv_tab + bh * p.kv_tab_stride : nullptr;
  // Block table: virtual key row r is row r & 31 of slice r / 32 of the block
  // list; rows past a slice's valid rows are skipped.  Row table (pooled rows):
  // the partial blocks' rows (the source tail at K_new position n_src - 1, the
  // context tail last if kept) carry the weight (tokens / len).
  const bool row_table = p.kv_row_table != 0;
  const int kv_slices = p.kv_rows / 32;
  const int src_tail = p.grid.src_tail(), ctx_tail = p.grid.ctx_tail();
  const int pu0 = (row_table && src_tail) ? p.grid.n_src - 1 : -1;
  const int pu1 = (row_table && ctx_tail && tab[p.kv_rows - 1] == p.grid.n_blocks() - 1)
                      ? p.kv_rows - 1 : -1;
  const float lw0 = src_tail ? logf((float)src_tail / p.grid.len) : 0.0f;
  const float lw1 = ctx_tail ? logf((float)ctx_tail / p.grid.len) : 0.0f;

  float q[DP], o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    q[i] = Qh[qrow * D + part * DP + i];
    o[i] = 0.0f;
  }
  // natural-log domain, scale = ln 2 * scale_log2 = 1/sqrt(D)
  const float scale = p.scale_log2 * 0.69314718055994531f;
  float m = -INFINITY, l = 0.0f;
  for (int t0 = 0; t0 < p.kv_rows; t0 += kTile) {
    const int n = min(kTile, p.kv_rows - t0);
    __syncthreads();
    for (int i = tid; i < kTile * (D / 4); i += kThreads) {
      const int r = i / (D / 4), c = (i % (D / 4)) * 4;
      const int rr = min(t0 + r, p.kv_rows - 1);
      int64_t src;
      if (!row_table) {
        const Slice sl = list_slice(p.grid, tab, kv_slices, p.half_shift, rr >> 5);
        src = (int64_t)sl.start + min(rr & 31, max(sl.cnt - 1, 0));
      } else {
        src = tab ? tab[rr] : rr;
      }
      *reinterpret_cast<float4*>(&Ks[r][c]) = *reinterpret_cast<const float4*>(Kh + src * D + c);
      *reinterpret_cast<float4*>(&Vs[r][c]) = *reinterpret_cast<const float4*>(Vh + src * D + c);
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const int rr = t0 + j;
      float wbias = 0.0f;
      if (!row_table) {
        if ((rr & 31) >= list_slice(p.grid, tab, kv_slices, p.half_shift, rr >> 5).cnt)
          continue;  // past a partial block's end, or an empty slice
      } else {
        wbias = (rr == pu0) ? lw0 : ((rr == pu1) ? lw1 : 0.0f);
      }
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < DP; ++i) s = fmaf(q[i], Ks[j][part * DP + i], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s = s * scale + wbias;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float pj = expf(s - m_new);
      l = l * alpha + pj;
#pragma unroll
      for (int i = 0; i < DP; ++i) o[i] = fmaf(pj, Vs[j][part * DP + i], o[i] * alpha);
      m = m_new;
    }
  }
  if (!q_ok) return;
  const float inv = 1.0f / l;
  float* Oh = static_cast<float*>(p.o) + bh * p.q_head_stride;
#pragma unroll
  for (int i = 0; i < DP; ++i) Oh[qrow * D + part * DP + i] = o[i] * inv;
  if (p.lse && part == 0) p.lse[bh * p.lse_head_stride + qrow] = m + logf(l) + p.lse_offset;
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, isa_dtype_t dtype, hipStream_t stream) {
  if (dtype == ISA_DTYPE_BF16) {
    // block tables (exact path, dense): the one-wave-per-SIMD kernel where it
    // applies, else the ping-pong kernel; row tables: the 4-wave kernel
    const uint32_t dbg = debug_flags();
    if (p.kv_row_table || (dbg & kDebug4WaveExact)) return launch_attention_bf16(p, stream);
    if (!(dbg & kDebugPingPongExact) && attention_w64_supported(p))
      return launch_attention_w64(p, stream);
    return launch_attention_pp(p, stream);
  }
  if (p.BH == 0 || p.n_q_entries == 0) return hipSuccess;
  dim3 grid(p.n_q_entries, p.BH);
  if (p.D == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace isa
