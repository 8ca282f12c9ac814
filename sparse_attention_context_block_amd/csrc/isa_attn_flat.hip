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
// One workgroup = 4 waves = one flat query block (64 rows, 16 per wave); the
// key tiles of a block are its own, so workgroups do not share them and the
// kernel is bound by the latency of its tile loads.  It is therefore built to
// keep many tiles in flight: v_mfma_f32_16x16x32_bf16 on 16 query rows per
// wave keeps a wave under 128 VGPRs, and one K and one V buffer (the next
// tile waits in registers) keep a workgroup at 36 KB of LDS, so four
// workgroups share a CU.  Tiles:
//   t < n_ns:   the 64 tokens of K_new block ns[t] (rows of K, V);
//   t >= n_ns:  64 representative rows u = 64 (t - n_ns) + r of K_new
//               (rows of the pooled K^c, V^c), masked past n_kv and for the
//               blocks already taken exactly (an LDS bitmap).
// Layout (lane l, q = l % 16, g = l / 16): S^T = K Q^T in 16x16 subtiles, lane
// holding keys 16 st + 4 g + i of query q; P^T enters O^T += V^T P^T as the B
// operand with 32-key chunks whose eight slots of group g are keys
// 32 c + 4 g + (0..3) and 32 c + 16 + 4 g + (0..3) -- exactly the registers
// the S^T accumulators leave in the lane, so P needs no shuffle.  V stays
// row-major in LDS (a plain copy) and the matching V^T operand comes from two
// transposing reads (ds_read_b64_tr_b16) per chunk.
#include "isa_debug.h"
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D>
struct FlatSmem {
  // Row strides measured on gfx950: 16 lanes reading one 16-byte chunk of 16
  // consecutive rows (the K operand) run conflict-free at 2 D + 32 bytes and
  // at half rate at 2 D + 16; the transposing V reads run at the same rate
  // for both.
  static constexpr int kKStride = D * 2 + 32;
  static constexpr int kVStride = D * 2 + 32;
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kVBytes = kBN * kVStride;
  static constexpr int kMaskOff = kKBytes + kVBytes;
  static constexpr int kTotal = kMaskOff + kMaxBlocksPerHead / 8;
};

// Tables up to this many entries (the exact tiles' block ids, then the row
// table of the representative tiles) are copied into LDS once per workgroup:
// a tile's row lookups then cost an LDS read instead of dependent scalar or
// vector loads from global memory, each waited on at once.  896 ints fill the
// LDS left over with four workgroups per CU.
constexpr int kLdsTab = 896;

template <int D, bool kTabInLds>
__global__ __launch_bounds__(kThreads, 4) void attn_flat_bf16_kernel(FlatParams p) {
  using S = FlatSmem<D>;
  constexpr int KC = D / 8;                 // 16-byte chunks per row
  constexpr int NCH = kBN * KC / kThreads;  // chunks per thread of a K (or V) tile: 2 or 4
  constexpr int NKK = D / 32;               // k-steps of the S MFMA
  constexpr int ND = D / 16;                // 16-dim subtiles of O
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kTotal];
  unsigned char* const ks_lds = smem;
  unsigned char* const vs_lds = smem + S::kKBytes;
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem + S::kMaskOff);
  __shared__ int32_t tabs[kTabInLds ? kLdsTab : 1];

  // XCD-aware: consecutive flat entries of a head run on one XCD, so the K/V
  // blocks they share stay in that XCD's L2
  const int total = p.n_flat * p.BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= total) return;  // whole workgroup, before any barrier
  const int64_t bh = lid / p.n_flat;
  const int f = lid % p.n_flat;  // flat entry
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane & 15;
  const int g = lane >> 4;
  const int n_kv = p.n_kv;
  const int n_ns = p.n_ns;
  const int32_t* tab = p.kv_tab + bh * n_kv;
  const int32_t* ns = p.ns + (bh * p.n_flat + f) * n_ns;
  // Loop-invariant scalars pinned in scalar registers (left alone, the compiler
  // reloads them from the kernel arguments inside the tile loop).
  BlockGrid gr;
  gr.L_src = __builtin_amdgcn_readfirstlane(p.grid.L_src);
  gr.n_src = __builtin_amdgcn_readfirstlane(p.grid.n_src);
  gr.N = __builtin_amdgcn_readfirstlane(p.grid.N);
  gr.len = __builtin_amdgcn_readfirstlane(p.grid.len);
  asm("" : "+s"(gr.L_src), "+s"(gr.n_src), "+s"(gr.N), "+s"(gr.len));
  if constexpr (kTabInLds) {
    // exact tile t: block tab[ns[t]] at tabs[t]; representative row u: tab[u]
    // at tabs[n_ns + u]
    for (int i = tid; i < n_ns + n_kv; i += kThreads) tabs[i] = i < n_ns ? tab[ns[i]] : tab[i - n_ns];
  }

  // ---- bitmap of the K_new positions computed exactly ----
  for (int w = tid; w < (n_kv + 31) / 32; w += kThreads) mask[w] = 0u;
  __syncthreads();
  for (int t = tid; t < n_ns; t += kThreads) atomicOr(&mask[ns[t] >> 5], 1u << (ns[t] & 31));

  // ---- this wave's 16 query rows; lane (q, g) holds dims 32 kk + 8 g .. + 7 ----
  const int qblk = p.flat[bh * p.n_flat + f];
  // the tail rows of a partial query block read its first row and are not stored
  const int qr = wave * 16 + q;
  const bool q_ok = qr < gr.rows(qblk);
  const int64_t qrow = (int64_t)gr.start(qblk) + (q_ok ? qr : 0);
  const bf16_bits* Qh = static_cast<const bf16_bits*>(p.q) + bh * p.q_head_stride;
  bf16x8_t qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 32 * kk + 8 * g);

  const bf16_bits* Kh = static_cast<const bf16_bits*>(p.k) + bh * p.kv_head_stride;
  const bf16_bits* Vh = static_cast<const bf16_bits*>(p.v) + bh * p.kv_head_stride;
  const bf16_bits* Kch = static_cast<const bf16_bits*>(p.kc) + bh * p.kc_head_stride;
  const bf16_bits* Vch = static_cast<const bf16_bits*>(p.vc) + bh * p.kc_head_stride;
  const int n_rep_tiles = (n_kv + kBN - 1) / kBN;
  const int n_tiles = n_ns + n_rep_tiles;

  // source row r of tile t (exact tiles: rows of K/V; representative tiles:
  // rows of K^c/V^c, past-the-end rows clamped to a valid row and masked later)
  auto exact_blk = [&](int t) -> int {
    return __builtin_amdgcn_readfirstlane(kTabInLds ? tabs[t] : tab[ns[t]]);
  };
  // source row r of representative tile t (rows past n_kv read a valid row
  // and are masked)
  auto rep_row = [&](int t, int r) -> int {
    const int u = min((t - n_ns) * kBN + r, n_kv - 1);
    return kTabInLds ? tabs[n_ns + u] : tab[u];
  };
  // Partial blocks (the tail of each segment) sit at K_new positions n_src - 1
  // and, if the context tail is kept, n_kv - 1: taken exactly, their missing
  // tokens are masked; as representatives they carry the weight (tokens / b).
  const int src_tail = gr.src_tail();
  const int ctx_tail = gr.ctx_tail();
  const int pu0 = src_tail ? gr.n_src - 1 : -1;
  const int pu1 = (ctx_tail && tab[n_kv - 1] == gr.n_blocks() - 1) ? n_kv - 1 : -1;
  float sl2 = p.scale_log2;
  float exact_bias2 = p.exact_bias_log2;  // -log2(b)
  asm("" : "+s"(sl2), "+s"(exact_bias2));
  const float w0 = src_tail ? log2f((float)src_tail / kBN) / sl2 : 0.0f;
  const float w1 = ctx_tail ? log2f((float)ctx_tail / kBN) / sl2 : 0.0f;

  // staging: chunk c = tid + 256 i is row c / KC, 16-byte column c % KC (KC
  // consecutive threads read one row); K and V are both plain row-major copies
  u32x4 st[NCH];
  // blk: the block of exact tile t (read once per tile by the caller)
  auto load_rows = [&](int t, int blk, const bf16_bits* full, const bf16_bits* pooled)
      __attribute__((always_inline)) {
    if (t < n_ns) {  // a partial block repeats its last row
      const int64_t st0 = gr.start(blk);
      const int last = gr.rows(blk) - 1;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + kThreads * i;
        st[i] = *reinterpret_cast<const u32x4*>(full + (st0 + min(c / KC, last)) * D + (c % KC) * 8);
      }
    } else {
      int rows[NCH];  // pooled row ids (< n_q)
#pragma unroll
      for (int i = 0; i < NCH; ++i) rows[i] = rep_row(t, (tid + kThreads * i) / KC);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + kThreads * i;
        st[i] = *reinterpret_cast<const u32x4*>(pooled + (int64_t)rows[i] * D + (c % KC) * 8);
      }
    }
  };
  auto store_rows = [&](unsigned char* dst, int stride) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(dst + (c / KC) * stride + (c % KC) * 16) = st[i];
    }
  };

  f32x4_t oacc[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[j][i] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;  // this lane's share of the row sum (reduced at the end)

  // One K and one V buffer: K(t+1) is loaded while S(t) runs and stored once
  // every wave is past S(t); V(t+1) is loaded while O += V(t) P(t) runs and
  // stored once every wave is past it.  Each store is published by the next
  // barrier, before the first read of that buffer.
  int blk_cur = n_ns > 0 ? exact_blk(0) : 0;  // block of exact tile t
  load_rows(0, blk_cur, Kh, Kch);
  store_rows(ks_lds, S::kKStride);
  load_rows(0, blk_cur, Vh, Vch);
  store_rows(vs_lds, S::kVStride);
  __syncthreads();  // also publishes the bitmap

  for (int t = 0; t < n_tiles; ++t) {
    const bool more = t + 1 < n_tiles;
    const bool exact = t < n_ns;
    const int blk_nxt = t + 1 < n_ns ? exact_blk(t + 1) : 0;  // block of exact tile t + 1
    if (more) load_rows(t + 1, blk_nxt, Kh, Kch);

    // S^T subtile s: keys 16 s + 4 g + i of query q
    f32x4_t sacc[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[s4][i] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            ks_lds + (16 * s4 + q) * S::kKStride + (32 * kk + 8 * g) * 2);
        sacc[s4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[kk], sacc[s4], 0, 0, 0);
      }
    }
    // representative tiles: mask rows past n_kv and blocks taken exactly, and
    // weight a partial block's row; exact tiles: mask a partial block's tail
    if (!exact) {
      const int u0 = (t - n_ns) * kBN;
      // bits of keys u0 .. u0 + 63 of the bitmap (u0 is a multiple of 64)
      const int w0i = u0 >> 5;
      const uint32_t mlo = mask[w0i];
      const uint32_t mhi = w0i + 1 < kMaxBlocksPerHead / 32 ? mask[w0i + 1] : 0u;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = u0 + 16 * s4 + 4 * g + i;
          if (u == pu0) sacc[s4][i] += w0;
          if (u == pu1) sacc[s4][i] += w1;
          const int k = 16 * s4 + 4 * g + i;  // key within the tile
          if (u >= n_kv || (((k < 32 ? mlo : mhi) >> (k & 31)) & 1u)) sacc[s4][i] = -INFINITY;
        }
    } else {
      // valid tokens of the block (only the segment tails are partial)
      const int vt = gr.rows(blk_cur);
      if (vt < kBN) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * s4 + 4 * g + i >= vt) sacc[s4][i] = -INFINITY;
      }
    }
    const float bias2 = exact ? exact_bias2 : 0.0f;

    // row max over the tile: 16 values here, then across the four lane groups
    float tmax = sacc[0][0];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sacc[s4][i]);
    {
      // each swap returns {own, partner} in an order that depends on the lane's
      // row of 16 (or half of 32), so take both
      uint32_t u = __float_as_uint(tmax);
      const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      tmax = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      u = __float_as_uint(tmax);
      const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      tmax = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    }
    const float tmax_s = fmaf(tmax, sl2, bias2);  // -inf for a fully masked tile
    if (__builtin_amdgcn_ballot_w64(tmax_s > m_run + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_run, tmax_s);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[j][i] *= alpha;
      m_run = m_new;
    }
    const float off = bias2 - m_run;
    // P^T operand of chunk c: slots 0-3 = subtile 2c, slots 4-7 = subtile 2c + 1
    bf16x8_t pk[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * c + h][i], sl2, off));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * c + h][i + 1], sl2, off));
          bf16x2_t pr;
          pr[0] = (__bf16)p0;
          pr[1] = (__bf16)p1;
          // the row sum adds the fp32 exponentials (a packed bf16 dot product
          // would issue on the matrix pipe and wait for the MFMAs)
          l_run = (l_run + p0) + p1;
          pk[c][4 * h + i] = pr[0];
          pk[c][4 * h + i + 1] = pr[1];
        }
      }
    }
    __syncthreads();  // every wave is past S(t): K may be overwritten
    if (more) {
      store_rows(ks_lds, S::kKStride);
      load_rows(t + 1, blk_nxt, Vh, Vch);
    }
    // O^T subtile j (dims 16 j + 4 g + i of query q) += V^T P^T; the V^T operand
    // of chunk c is two transposing reads: keys 32 c + 4 g + (0..3) and
    // 32 c + 16 + 4 g + (0..3) at dims 16 j .. 16 j + 15 (lane q of a group
    // addresses key row q / 4, dims 4 (q % 4) .. + 3 of its four-key group)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        const unsigned char* base =
            vs_lds + (32 * c + 4 * g + (q >> 2)) * S::kVStride + (16 * j + 4 * (q & 3)) * 2;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)base);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(base + 16 * S::kVStride));
        const v8i16 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, both);
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[c], oacc[j], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is past O += V(t) P(t); K(t+1) is visible
    if (more) store_rows(vs_lds, S::kVStride);
    blk_cur = blk_nxt;
  }

  // ---- epilogue: O / l, bf16 round-to-nearest-even, LSE (+ ln b) ----
  {
    uint32_t u = __float_as_uint(l_run);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    l_run = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);  // own + partner
    u = __float_as_uint(l_run);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_run = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  }
  const float inv = 1.0f / l_run;
  bf16_bits* Oh = static_cast<bf16_bits*>(p.o) + bh * p.q_head_stride + qrow * D;
#pragma unroll
  for (int j = 0; j < ND && q_ok; ++j) {
    bf16x2_t a, b;
    a[0] = (__bf16)(oacc[j][0] * inv);
    a[1] = (__bf16)(oacc[j][1] * inv);
    b[0] = (__bf16)(oacc[j][2] * inv);
    b[1] = (__bf16)(oacc[j][3] * inv);
    uint2 w;
    w.x = __builtin_bit_cast(uint32_t, a);
    w.y = __builtin_bit_cast(uint32_t, b);
    *reinterpret_cast<uint2*>(Oh + 16 * j + 4 * g) = w;
  }
  if (p.lse && g == 0 && q_ok) {
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
    const int64_t total = (int64_t)p.n_flat * p.BH;
    const dim3 grid1((unsigned)(((total + 7) / 8) * 8));
    const bool lds_tab = p.n_ns + p.n_kv <= kLdsTab && !(debug_flags() & kDebugGlobalTables);
    if (p.D == 128) {
      if (lds_tab)
        hipLaunchKernelGGL((attn_flat_bf16_kernel<128, true>), grid1, dim3(kThreads), 0, stream, p);
      else
        hipLaunchKernelGGL((attn_flat_bf16_kernel<128, false>), grid1, dim3(kThreads), 0, stream, p);
    } else {
      if (lds_tab)
        hipLaunchKernelGGL((attn_flat_bf16_kernel<64, true>), grid1, dim3(kThreads), 0, stream, p);
      else
        hipLaunchKernelGGL((attn_flat_bf16_kernel<64, false>), grid1, dim3(kThreads), 0, stream, p);
    }
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_flat_f32_kernel<128>, grid, dim3(kF32Threads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_flat_f32_kernel<64>, grid, dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace isa
