// Flat query blocks with a block mask: the 0-th order Taylor path of ISA in
// which the top blocks of each query block's coarse row are computed token by
// token ([notes] key design 2: per (query block, key block) pair, mask 1 takes
// the exact online-softmax update, mask 0 the representative update with K^c_j,
// V^c_j and weight b; [summary] 4: alpha_ns, the no-sparsity ratio).  Both
// kinds of terms share one online softmax per row:
//   l = sum_t e^{s_t - m} + sum_j b e^{s^c_j - m},  O = (...) / l.
// The weight b is carried as -log2(b) on the exact tokens (exp2 domain) and
// +ln(b) on the LSE, so the representative terms need no scaling.
//
// One workgroup = 2 waves = one flat query block (64 rows, 32 per wave); the
// key tiles of a block are its own, so workgroups do not share them.  Tiles:
//   t < n_ns:   the 64 tokens of K_new block ns[t] (rows of K, V);
//   t >= n_ns:  64 representative rows u = 64 (t - n_ns) + r of K_new
//               (rows of the pooled K^c, V^c), masked past n_kv and for the
//               blocks already taken exactly (an LDS bitmap).
// The MFMA layout, the transposed V staging and the lazy rescale are those of
// the other bf16 attention kernels (S^T = K Q^T, O^T += V^T P^T with
// v_mfma_f32_32x32x16_bf16, one query per lane column).
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 128;
constexpr int kBN = 64;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct FlatSmem {
  static constexpr int kKStride = D * 2 + 16;
  static constexpr int kVStride = kBN * 2 + 16;
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kMaskOff = 2 * kStage;
  static constexpr int kTotal = kMaskOff + kMaxBlocksPerHead / 8;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_flat_bf16_kernel(FlatParams p) {
  using S = FlatSmem<D>;
  constexpr int KC = D / 8;                 // 16-byte chunks per row
  constexpr int KCH = kBN * KC / kThreads;  // K chunks per thread (4 or 8)
  constexpr int VCH = KC / 8;               // V d-chunk rounds per thread (1 or 2)
  constexpr int NKK = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kTotal];
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem + S::kMaskOff);

  const int64_t bh = blockIdx.y;
  const int f = blockIdx.x;  // flat entry
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_kv = p.n_kv;
  const int n_ns = p.n_ns;
  const int32_t* tab = p.kv_tab + bh * n_kv;
  const int32_t* ns = p.ns + (bh * p.n_flat + f) * n_ns;

  // ---- bitmap of the K_new positions computed exactly ----
  for (int w = tid; w < (n_kv + 31) / 32; w += kThreads) mask[w] = 0u;
  __syncthreads();
  for (int t = tid; t < n_ns; t += kThreads) atomicOr(&mask[ns[t] >> 5], 1u << (ns[t] & 31));

  // ---- this wave's 32 query rows ----
  const int qblk = p.flat[bh * p.n_flat + f];
  // the tail rows of a partial query block read its first row and are not stored
  const int qr = wave * 32 + l32;
  const bool q_ok = qr < p.grid.rows(qblk);
  const int64_t qrow = (int64_t)p.grid.start(qblk) + (q_ok ? qr : 0);
  const bf16_bits* Qh = static_cast<const bf16_bits*>(p.q) + bh * p.q_head_stride;
  bf16x8_t qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 16 * kk + 8 * hi);

  const bf16_bits* Kh = static_cast<const bf16_bits*>(p.k) + bh * p.kv_head_stride;
  const bf16_bits* Vh = static_cast<const bf16_bits*>(p.v) + bh * p.kv_head_stride;
  const bf16_bits* Kch = static_cast<const bf16_bits*>(p.kc) + bh * p.kc_head_stride;
  const bf16_bits* Vch = static_cast<const bf16_bits*>(p.vc) + bh * p.kc_head_stride;
  const int n_rep_tiles = (n_kv + kBN - 1) / kBN;
  const int n_tiles = n_ns + n_rep_tiles;

  // source row r of tile t (exact tiles: rows of K/V; representative tiles:
  // rows of K^c/V^c, past-the-end rows clamped to a valid row and masked later)
  auto src_row = [&](int t, int r) -> int64_t {
    if (t < n_ns) {
      const int blk = tab[ns[t]];  // a partial block repeats its last row
      return (int64_t)p.grid.start(blk) + min(r, p.grid.rows(blk) - 1);
    }
    return tab[min((t - n_ns) * kBN + r, n_kv - 1)];
  };
  // Partial blocks (the tail of each segment) sit at K_new positions n_src - 1
  // and, if the context tail is kept, n_kv - 1: taken exactly, their missing
  // tokens are masked; as representatives they carry the weight (tokens / b).
  const int src_tail = p.grid.src_tail();
  const int ctx_tail = p.grid.ctx_tail();
  const int pu0 = src_tail ? p.grid.n_src - 1 : -1;
  const int pu1 = (ctx_tail && tab[n_kv - 1] == p.grid.n_blocks() - 1) ? n_kv - 1 : -1;
  const float w0 = src_tail ? log2f((float)src_tail / kBN) / p.scale_log2 : 0.0f;
  const float w1 = ctx_tail ? log2f((float)ctx_tail / kBN) / p.scale_log2 : 0.0f;

  u32x4 kst[KCH];
  u32x4 vst[4 * VCH];
  // V^T staging: key group vg = tid % 16 (4 keys), d chunk vd = tid / 16 + 8 c
  const int vg = tid % (kBN / 4);
  const int vd0 = tid / (kBN / 4);
  const int vq = vg & 3;
  const int vpos = (vg >> 2) * 16 + (((vq & 1) << 1) | (vq >> 1)) * 4;

  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const bool exact = t < n_ns;
    const bf16_bits* kb = exact ? Kh : Kch;
    const bf16_bits* vb = exact ? Vh : Vch;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      kst[i] = *reinterpret_cast<const u32x4*>(kb + src_row(t, c / KC) * D + (c % KC) * 8);
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vst[4 * c + r] = *reinterpret_cast<const u32x4*>(
            vb + src_row(t, 4 * vg + r) * D + (vd0 + 8 * c) * 8);
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    unsigned char* ks = smem + buf * S::kStage;
    unsigned char* vs = ks + S::kKBytes;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(ks + (c / KC) * S::kKStride + (c % KC) * 16) = kst[i];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      unsigned char* vrow = vs + ((vd0 + 8 * c) * 8) * S::kVStride + vpos * 2;
      const u32x4 a = vst[4 * c], b = vst[4 * c + 1], d2 = vst[4 * c + 2], d3 = vst[4 * c + 3];
      // word w of a key's 8 dims holds dims 2w (low half) and 2w+1 (high half)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint2*>(vrow + (2 * w) * S::kVStride) =
            make_uint2(pack2(a[w], b[w], false), pack2(d2[w], d3[w], false));
        *reinterpret_cast<uint2*>(vrow + (2 * w + 1) * S::kVStride) =
            make_uint2(pack2(a[w], b[w], true), pack2(d2[w], d3[w], true));
      }
    }
  };

  f32x16_t oacc[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[j][r] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float sl2 = p.scale_log2;
  const float exact_bias2 = p.exact_bias_log2;  // -log2(b)
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  load_tile(0);
  store_tile(0);
  __syncthreads();  // also publishes the bitmap

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const unsigned char* ks = smem + buf * S::kStage;
    const unsigned char* vs = ks + S::kKBytes;
    const bool exact = t < n_ns;

    f32x16_t sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[s][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            ks + (32 * s + l32) * S::kKStride + (16 * kk + 8 * hi) * 2);
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[s], 0, 0, 0);
      }
    }
    // representative tiles: mask rows past n_kv and blocks taken exactly, and
    // weight a partial block's row; exact tiles: mask a partial block's tail
    if (!exact) {
      const int u0 = (t - n_ns) * kBN;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int u = u0 + 32 * s + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (u == pu0) sacc[s][r] += w0;
          if (u == pu1) sacc[s][r] += w1;
          if (u >= n_kv || ((mask[u >> 5] >> (u & 31)) & 1u)) sacc[s][r] = -INFINITY;
        }
    } else {
      const int pos = ns[t];
      const int vt = (pos == pu0) ? src_tail : ((pos == pu1) ? ctx_tail : kBN);
      if (vt < kBN) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * s + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= vt) sacc[s][r] = -INFINITY;
          }
      }
    }
    const float bias2 = exact ? exact_bias2 : 0.0f;

    float tmax = sacc[0][0];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[s][r]);
    {
      const uint32_t u = __float_as_uint(tmax);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float tmax_s = fmaf(tmax, sl2, bias2);  // -inf for a fully masked tile
    if (__builtin_amdgcn_ballot_w64(tmax_s > m_run + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_run, tmax_s);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][r] *= alpha;
      m_run = m_new;
    }
    const float off = bias2 - m_run;
    bf16x8_t pk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e2 = 0; e2 < 8; e2 += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e2], sl2, off));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e2 + 1], sl2, off));
        bf16x2_t pr;
        pr[0] = (__bf16)p0;
        pr[1] = (__bf16)p1;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
        pk[c][e2] = pr[0];
        pk[c][e2 + 1] = pr[1];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            vs + (32 * j + l32) * S::kVStride + (16 * c + 8 * hi) * 2);
        oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[c], oacc[j], 0, 0, 0);
      }
    }
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, bf16 round-to-nearest-even, LSE (+ ln b) ----
  {
    const uint32_t u = __float_as_uint(l_run);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = 1.0f / l_run;
  bf16_bits* Oh = static_cast<bf16_bits*>(p.o) + bh * p.q_head_stride + qrow * D;
#pragma unroll
  for (int j = 0; j < ND && q_ok; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x2_t a, b;
      a[0] = (__bf16)(oacc[j][4 * g + 0] * inv);
      a[1] = (__bf16)(oacc[j][4 * g + 1] * inv);
      b[0] = (__bf16)(oacc[j][4 * g + 2] * inv);
      b[1] = (__bf16)(oacc[j][4 * g + 3] * inv);
      uint2 w;
      w.x = __builtin_bit_cast(uint32_t, a);
      w.y = __builtin_bit_cast(uint32_t, b);
      *reinterpret_cast<uint2*>(Oh + 32 * j + 8 * g + 4 * hi) = w;
    }
  }
  if (p.lse && hi == 0 && q_ok) {
    p.lse[bh * p.lse_head_stride + qrow] =
        (m_run + __log2f(l_run)) * 0.69314718055994531f + p.lse_offset;
  }
}

// fp32 VALU variant (small fp32 problems): one workgroup per flat query block,
// 4 threads per row; the key sequence is the same as above, natural-log domain.
constexpr int kF32Threads = 256;
constexpr int kF32Tile = 32;

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_flat_f32_kernel(FlatParams p) {
  constexpr int DP = D / 4;
  __shared__ __attribute__((aligned(16))) float Ks[kF32Tile][D];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Tile][D];
  __shared__ uint32_t mask[kMaxBlocksPerHead / 32];
  const int64_t bh = blockIdx.y;
  const int f = blockIdx.x;
  const int tid = threadIdx.x;
  const int row = tid >> 2, part = tid & 3;
  const int n_kv = p.n_kv, n_ns = p.n_ns;
  const int32_t* tab = p.kv_tab + bh * n_kv;
  const int32_t* ns = p.ns + (bh * p.n_flat + f) * n_ns;
  for (int w = tid; w < (n_kv + 31) / 32; w += kF32Threads) mask[w] = 0u;
  __syncthreads();
  for (int t = tid; t < n_ns; t += kF32Threads) atomicOr(&mask[ns[t] >> 5], 1u << (ns[t] & 31));

  const int qblk = p.flat[bh * p.n_flat + f];
  const bool q_ok = row < p.grid.rows(qblk);
  const int64_t qrow = (int64_t)p.grid.start(qblk) + (q_ok ? row : 0);
  const float* Qh = static_cast<const float*>(p.q) + bh * p.q_head_stride;
  const float* Kh = static_cast<const float*>(p.k) + bh * p.kv_head_stride;
  const float* Vh = static_cast<const float*>(p.v) + bh * p.kv_head_stride;
  const float* Kch = static_cast<const float*>(p.kc) + bh * p.kc_head_stride;
  const float* Vch = static_cast<const float*>(p.vc) + bh * p.kc_head_stride;
  float q[DP], o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    q[i] = Qh[qrow * D + part * DP + i];
    o[i] = 0.0f;
  }
  const float scale = p.scale_log2 * 0.69314718055994531f;     // 1 / sqrt(D)
  const float bias = p.exact_bias_log2 * 0.69314718055994531f;  // -ln(b)
  const int src_tail = p.grid.src_tail(), ctx_tail = p.grid.ctx_tail();
  const int pu0 = src_tail ? p.grid.n_src - 1 : -1;
  const int pu1 = (ctx_tail && tab[n_kv - 1] == p.grid.n_blocks() - 1) ? n_kv - 1 : -1;
  const float lw0 = src_tail ? logf((float)src_tail / kBlock) : 0.0f;
  const float lw1 = ctx_tail ? logf((float)ctx_tail / kBlock) : 0.0f;
  const int n_exact_rows = n_ns * kBlock;
  const int n_rows = n_exact_rows + n_kv;
  float m = -INFINITY, l = 0.0f;
  for (int t0 = 0; t0 < n_rows; t0 += kF32Tile) {
    const int n = min(kF32Tile, n_rows - t0);
    __syncthreads();
    for (int i = tid; i < kF32Tile * (D / 4); i += kF32Threads) {
      const int r = i / (D / 4), c = (i % (D / 4)) * 4;
      const int rr = min(t0 + r, n_rows - 1);
      const bool ex = rr < n_exact_rows;
      int64_t src;
      if (ex) {
        const int blk = tab[ns[rr / kBlock]];
        src = (int64_t)p.grid.start(blk) + min(rr % kBlock, p.grid.rows(blk) - 1);
      } else {
        src = tab[rr - n_exact_rows];
      }
      const float* kb = ex ? Kh : Kch;
      const float* vb = ex ? Vh : Vch;
      *reinterpret_cast<float4*>(&Ks[r][c]) = *reinterpret_cast<const float4*>(kb + src * D + c);
      *reinterpret_cast<float4*>(&Vs[r][c]) = *reinterpret_cast<const float4*>(vb + src * D + c);
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const int rr = t0 + j;
      const bool ex = rr < n_exact_rows;
      float wbias = 0.0f;
      if (!ex) {
        const int u = rr - n_exact_rows;
        if ((mask[u >> 5] >> (u & 31)) & 1u) continue;  // taken exactly
        wbias = (u == pu0) ? lw0 : ((u == pu1) ? lw1 : 0.0f);
      } else {
        const int pos = ns[rr / kBlock];
        const int vt = (pos == pu0) ? src_tail : ((pos == pu1) ? ctx_tail : kBlock);
        if (rr % kBlock >= vt) continue;  // past a partial block's tail
      }
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < DP; ++i) s = fmaf(q[i], Ks[j][part * DP + i], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s = s * scale + (ex ? bias : wbias);
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

hipError_t launch_attention_flat(const FlatParams& p, isa_dtype_t dtype, hipStream_t stream) {
  if (p.BH == 0 || p.n_flat == 0) return hipSuccess;
  if (p.n_kv < 1 || p.n_kv > kMaxBlocksPerHead || p.n_ns < 0 || p.n_ns > p.n_kv)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.n_flat, (unsigned)p.BH);
  if (dtype == ISA_DTYPE_BF16) {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_flat_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_flat_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_flat_f32_kernel<128>, grid, dim3(kF32Threads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_flat_f32_kernel<64>, grid, dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace isa
