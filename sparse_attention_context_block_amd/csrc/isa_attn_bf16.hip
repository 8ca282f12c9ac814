// bf16 MFMA online-softmax attention for gfx950: the exact path of ISA, its
// 0-th order Taylor path and the dense baseline ([notes] key design 2 gives
// both update rules: the exact branch accumulates l += rowsum(exp(S)),
// O += exp(S) V; the representative branch uses K^c_j, V^c_j in place of the
// whole block with l and O scaled by the block length; both end with O / l).
//
// The two paths differ only in where their keys come from, which the
// AttnParams block table expresses:
//   exact:  keys = rows of K_new, read through the block table
//           (source blocks, then the selected context blocks): the gather +
//           concat of Context Pre-Selection is fused into the tile loads;
//   Taylor: keys = the pooled K^c_j, V^c_j of the same blocks (one table
//           entry per row); every block of a full-block grid has the same
//           weight b, which cancels in O / l and adds ln b to the LSE.
//
// Work decomposition (CDNA4, wave64):
//   workgroup = 4 waves = 128 query rows (two 64-row query blocks of a
//   worklist); each wave owns 32 query rows.  Keys stream in 64-row tiles
//   through double-buffered LDS (K row-major, V transposed).
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on the M axis): every lane
//   then holds 16 scores of ONE query per 32-key subtile, so the row max and
//   row sum need one permlane32 swap instead of a 32-lane reduction.
//   O^T += V^T P^T, again 32x32x16 MFMA: the P^T operand is built in
//   registers straight from the S^T accumulators; the key order inside each
//   16-key chunk this implies is undone by the order V^T is written to LDS.
//   Softmax in the exp2 domain; the running max is only raised when a tile
//   exceeds it by more than 2^8, so the O rescale is skipped for almost
//   every tile (exact: the same max is used in numerator and denominator).
//   Query blocks of a head are mapped to one XCD so its keys stay in that
//   XCD's L2.
#include "isa_debug.h"
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;          // keys per tile
// Row tables up to this length are copied into LDS once per workgroup, so a
// tile's row lookups cost an LDS read instead of a global round trip ahead of
// its data loads (8 KB: two workgroups per CU still fit).
constexpr int kTabLds = 2048;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D>
struct Smem {
  static constexpr int kKStride = D * 2 + 16;    // bytes per K row (padded)
  static constexpr int kVStride = kBN * 2 + 16;  // bytes per V^T row (padded)
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
};

// kSrc: 0 = block table, 1 = row table read from global memory, 2 = row
// table copied into LDS (at most kTabLds rows)
template <int D, int kSrc>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(AttnParams p) {
  constexpr bool kRowTable = kSrc != 0;
  using S = Smem<D>;
  constexpr int KC = D / 8;      // 16-byte chunks per K row
  constexpr int KCH = kBN * KC / kThreads;  // K chunks per thread per tile (2 or 4)
  static_assert(KCH == 2 || KCH == 4, "D must be 64 or 128");
  constexpr int NKK = D / 16;    // k-steps of the S MFMA
  constexpr int ND = D / 32;     // d subtiles of O
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kTotal];
  __shared__ int32_t tab_s[kSrc == 2 ? kTabLds : 1];

  // ---- XCD-aware mapping of workgroups to (head, query tile) ----
  const int wg_per_head = (p.n_q_entries + 1) / 2;
  const int total = wg_per_head * p.BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= total) return;
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- this wave's 32 query rows ----
  // (slice 2e + (wave & 1) of the query list; rows past a partial block's end
  // read the slice's first row and are not stored)
  const int e = qt * 2 + (wave >> 1);
  const bool wave_valid = e < p.n_q_entries;
  const int32_t* qlist = p.q_tab ? p.q_tab + bh * p.q_tab_stride : nullptr;
  const Slice qs = list_slice(p.grid, qlist, wave_valid ? p.n_q_slices : 0, p.half_shift,
                              2 * e + (wave & 1));
  const bool q_ok = l32 < qs.cnt;
  const int64_t qrow = (int64_t)qs.start + (q_ok ? l32 : 0);
  const bf16_bits* Qh = static_cast<const bf16_bits*>(p.q) + bh * p.q_head_stride;
  bf16x8_t qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 16 * kk + 8 * hi);

  // ---- key source rows ----
  const bf16_bits* Kh = static_cast<const bf16_bits*>(p.k) + bh * p.kv_head_stride;
  const bf16_bits* Vh = static_cast<const bf16_bits*>(p.v) + bh * p.kv_head_stride;
  const int32_t* tab = p.kv_tab ? p.kv_tab + bh * p.kv_tab_stride : nullptr;
  // Block table: tile t is the slices 2t and 2t + 1 of the block list (keys
  // past a slice's valid rows are masked).  Row table (the Taylor path): every
  // key row is looked up.
  const bool row_table = kRowTable;  // launcher: kv_row_table set
  const int kv_slices = p.kv_rows / 32;
  const int n_tiles = (p.kv_rows + kBN - 1) / kBN;
  auto slice_of = [&](int eta) -> Slice {
    return list_slice(p.grid, tab, kv_slices, p.half_shift, eta);
  };
  Slice sl_a{0, 0}, sl_b{0, 0};  // slices of the tile being loaded (block table)
  auto src_row = [&](int t, int r) -> int64_t {
    if (!row_table) {  // rows past a slice's valid rows repeat its last one
      const Slice& sl = (r & 32) ? sl_b : sl_a;
      return (int64_t)sl.start + min(r & 31, max(sl.cnt - 1, 0));
    }
    const int u = min(t * kBN + r, p.kv_rows - 1);  // rows past the end: valid, then masked
    return kSrc == 2 ? tab_s[u] : tab[u];
  };
  // Row table (pooled rows): the partial blocks' rows (the source tail at K_new
  // position n_src - 1, the context tail last if kept) carry the weight
  // (tokens / len) as a logit offset.
  const int src_tail = p.grid.src_tail();
  const int ctx_tail = p.grid.ctx_tail();
  const int pt0 = (row_table && src_tail) ? p.grid.n_src - 1 : -1;
  const int pt1 = (row_table && ctx_tail && tab[p.kv_rows - 1] == p.grid.n_blocks() - 1)
                      ? p.kv_rows - 1 : -1;
  const float w0 = src_tail ? log2f((float)src_tail / p.grid.len) / p.scale_log2 : 0.0f;
  const float w1 = ctx_tail ? log2f((float)ctx_tail / p.grid.len) / p.scale_log2 : 0.0f;

  // staging registers for the next tile (named, so they stay in VGPRs)
  uint4 k0, k1, k2, k3;  // K chunks c = tid + 256 i (i < KCH <= 4)
  uint4 v0, v1, v2, v3;
  // K: chunk c = tid + 256 i -> row c / KC, column chunk c % KC
  // V: thread -> key group vg = tid % 16 (4 keys), d chunk vd = tid / 16 (8 dims).
  // The key group varies fastest so that the 16 lanes of an LDS write phase
  // land on 16 different 8-byte bank pairs of one V^T row band (rows 8 apart
  // share banks, positions inside a row do not).
  const int vg = tid % (kBN / 4);
  const int vd = tid / (kBN / 4);
  const bool v_active = vd < KC;
  // keys 4vg..4vg+3 sit in 16-key chunk vg/4 at quad q = vg%4; inside a chunk
  // the PV operand wants quad order (0, 2, 1, 3): position quad = swap of q's bits
  const int vq = vg & 3;
  const int vpos = (vg >> 2) * 16 + (((vq & 1) << 1) | (vq >> 1)) * 4;

  auto load_tile = [&](int t) {
    if (!row_table) {
      sl_a = slice_of(2 * t);
      sl_b = slice_of(2 * t + 1);
    }
#define ISA_K_LOAD(I, R)                                                                \
  {                                                                                     \
    const int c = tid + kThreads * I;                                                   \
    R = *reinterpret_cast<const uint4*>(Kh + src_row(t, c / KC) * D + (c % KC) * 8);    \
  }
    ISA_K_LOAD(0, k0)
    ISA_K_LOAD(1, k1)
    if constexpr (KCH > 2) {
      ISA_K_LOAD(2, k2)
      ISA_K_LOAD(3, k3)
    }
#undef ISA_K_LOAD
    if (v_active) {
      const bf16_bits* vb = Vh + vd * 8;
      v0 = *reinterpret_cast<const uint4*>(vb + src_row(t, 4 * vg + 0) * D);
      v1 = *reinterpret_cast<const uint4*>(vb + src_row(t, 4 * vg + 1) * D);
      v2 = *reinterpret_cast<const uint4*>(vb + src_row(t, 4 * vg + 2) * D);
      v3 = *reinterpret_cast<const uint4*>(vb + src_row(t, 4 * vg + 3) * D);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* ks = smem + buf * S::kStage;
    unsigned char* vs = ks + S::kKBytes;
#define ISA_K_STORE(I, R)                                                                \
  {                                                                                      \
    const int c = tid + kThreads * I;                                                    \
    *reinterpret_cast<uint4*>(ks + (c / KC) * S::kKStride + (c % KC) * 16) = R;          \
  }
    ISA_K_STORE(0, k0)
    ISA_K_STORE(1, k1)
    if constexpr (KCH > 2) {
      ISA_K_STORE(2, k2)
      ISA_K_STORE(3, k3)
    }
#undef ISA_K_STORE
    if (v_active) {
      unsigned char* vrow = vs + (vd * 8) * S::kVStride + vpos * 2;
      // word w of a key's 8 dims holds dims 2w (low half) and 2w+1 (high half)
#define ISA_VT_STORE(W, F)                                                              \
  *reinterpret_cast<uint2*>(vrow + (2 * W) * S::kVStride) =                            \
      make_uint2(pack2(v0.F, v1.F, false), pack2(v2.F, v3.F, false));                  \
  *reinterpret_cast<uint2*>(vrow + (2 * W + 1) * S::kVStride) =                        \
      make_uint2(pack2(v0.F, v1.F, true), pack2(v2.F, v3.F, true));
      ISA_VT_STORE(0, x)
      ISA_VT_STORE(1, y)
      ISA_VT_STORE(2, z)
      ISA_VT_STORE(3, w)
#undef ISA_VT_STORE
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

  if constexpr (kSrc == 2) {
    for (int i = tid; i < p.kv_rows; i += kThreads) tab_s[i] = tab[i];
    __syncthreads();
  }
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const unsigned char* ks = smem + buf * S::kStage;
    const unsigned char* vs = ks + S::kKBytes;

    // S^T (64 keys x 32 queries) = K_tile Q^T
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

    // mask keys past the end (only a row-table tile can be partial)
    const int valid = p.kv_rows - t * kBN;
    if (kRowTable && valid < kBN) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * s + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= valid) sacc[s][r] = -INFINITY;
        }
    }
    if (kRowTable) {
      // weight of a partial block's pooled row
      const int u0 = pt0 - t * kBN, u1 = pt1 - t * kBN;
      if ((pt0 >= 0 && u0 >= 0 && u0 < kBN) || (pt1 >= 0 && u1 >= 0 && u1 < kBN)) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * s + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key == u0) sacc[s][r] += w0;
            if (key == u1) sacc[s][r] += w1;
          }
      }
    } else {
      const Slice ta = slice_of(2 * t), tb = slice_of(2 * t + 1);
      if (ta.cnt < 32 || tb.cnt < 32) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * hi + (r & 3);  // within slice s
            if (key >= (s ? tb.cnt : ta.cnt)) sacc[s][r] = -INFINITY;
          }
      }
    }

    // online softmax (exp2 domain); lane and lane^32 hold the same query
    float tmax = sacc[0][0];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[s][r]);
    {
      // the swap returns {own, partner} in an order that depends on the half
      // of the wave, so take both
      const uint32_t u = __float_as_uint(tmax);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float tmax_s = tmax * sl2;
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

    bf16x8_t pk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e2 = 0; e2 < 8; e2 += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e2], sl2, -m_run));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e2 + 1], sl2, -m_run));
        bf16x2_t pr;
        pr[0] = (__bf16)p0;
        pr[1] = (__bf16)p1;
        // the row sum adds the fp32 exponentials (a packed bf16 dot product
        // would issue on the matrix pipe and wait for the MFMAs)
        l_run = (l_run + p0) + p1;
        pk[c][e2] = pr[0];
        pk[c][e2 + 1] = pr[1];
      }
    }

    // O^T (D x 32 queries) += V^T P^T
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

  // ---- epilogue: O / l, bf16 round-to-nearest-even, LSE ----
  {
    const uint32_t u = __float_as_uint(l_run);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // own + partner
  }
  if (!wave_valid) return;
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

}  // namespace

hipError_t launch_attention_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.BH == 0 || p.n_q_entries == 0) return hipSuccess;
  const int wg_per_head = (p.n_q_entries + 1) / 2;
  const int64_t total = (int64_t)wg_per_head * p.BH;
  const dim3 grid((unsigned)(((total + 7) / 8) * 8));
  const bool row_table = p.kv_row_table != 0;
  if (!row_table && p.kv_rows % 32 != 0) return hipErrorInvalidValue;
  const bool lds_tab = p.kv_rows <= kTabLds && !(debug_flags() & kDebugGlobalTables);
  const int src = !row_table ? 0 : (lds_tab ? 2 : 1);
#define ISA_BF16_LAUNCH(DD, SRC) \
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, SRC>), grid, dim3(kThreads), 0, stream, p)
  if (p.D == 128) {
    if (src == 2) ISA_BF16_LAUNCH(128, 2);
    else if (src == 1) ISA_BF16_LAUNCH(128, 1);
    else ISA_BF16_LAUNCH(128, 0);
  } else {
    if (src == 2) ISA_BF16_LAUNCH(64, 2);
    else if (src == 1) ISA_BF16_LAUNCH(64, 1);
    else ISA_BF16_LAUNCH(64, 0);
  }
#undef ISA_BF16_LAUNCH
  return hipGetLastError();
}

}  // namespace isa
