// Ping-pong variant of the bf16 MFMA online-softmax attention for gfx950,
// used for the exact path of ISA (keys of K_new through the block table) and
// the dense baseline ([notes] key design 2: the exact branch accumulates
// l += rowsum(exp(S)), O += exp(S) V, and ends with O / l).
//
// One workgroup = 8 waves = 256 query rows (four 64-row query blocks of a
// worklist); each wave owns 32 rows with the same MFMA layout as the 4-wave
// kernel (S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, one
// permlane32 swap per row reduction).  The 8 waves form two groups, A (waves
// 0-3) and B (waves 4-7), one wave of each per SIMD.  Per key tile a wave has
// a VALU phase (softmax of S(t), packing P(t), staging the next tile into
// LDS) and an MFMA phase (O += V(t) P(t), then S(t+1) = K(t+1) Q^T).  The
// groups run half a tile apart and switch phases at workgroup barriers, so
// while one group's waves issue MFMAs the other group's waves on the same
// SIMDs do their softmax:
//
//   phase:   0        1        2        3       ...  2t+1     2t+2
//   A:     S(0)     soft(0)  PV(0)S(1) soft(1)  ...  soft(t)  PV(t)S(t+1)
//   B:     stV(0)   S(0)     soft(0)  PV(0)S(1) ...  PV(t-1)S(t)  soft(t)
//
// Group A stages the K tiles (row-major), group B the V tiles (transposed), each
// during its own VALU phase.  K(t+1) is written in A's phase 2t+1 into the
// buffer that held K(t-1), last read in B's phase 2t-1; V(t+1) is written in
// B's phase 2t+2 into the buffer of V(t-1), last read in B's phase 2t+1; each
// is first read one phase after it is written.  Both groups execute 2n+2
// barriers for n key tiles.
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 512;
constexpr int kGroup = 256;  // threads per group
constexpr int kBN = 64;      // keys per tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// Workgroup barrier between phases.
__device__ __forceinline__ void phase_barrier() { __syncthreads(); }

template <int D>
struct Lds {
  static constexpr int kKStride = D * 2 + 16;    // bytes per K row (padded)
  static constexpr int kVStride = kBN * 2 + 16;  // bytes per V^T row (padded)
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kTotal = 2 * kKBytes + 2 * kVBytes;
};

template <int D, int kShift>  // kShift: log2 of the 32-row slices per block
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_pp_kernel(AttnParams p) {
  using S = Lds<D>;
  constexpr int KC = D / 8;                  // 16-byte chunks per row
  constexpr int KCH = kBN * KC / kGroup;     // K chunks per group-A thread (2 or 4)
  static_assert(KCH == 2 || KCH == 4, "D must be 64 or 128");
  constexpr int NKK = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kTotal];

  // ---- XCD-aware mapping of workgroups to (head, query tile) ----
  const int wg_per_head = (p.n_q_entries + 3) / 4;
  const int total = wg_per_head * p.BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  // whole workgroup, before any barrier (the barrier counts below assume >= 1 tile)
  if (lid >= total || p.kv_rows < 32) return;
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const bool gA = wave < 4;
  const int gtid = tid & (kGroup - 1);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- this wave's 32 query rows ----
  // (slice 2e + (wave & 1) of the query list; rows past a partial block's end
  // read the slice's first row and are not stored)
  const int e = qt * 4 + (wave >> 1);
  const bool wave_valid = e < p.n_q_entries;
  const int32_t* qlist = p.q_tab ? p.q_tab + bh * p.q_tab_stride : nullptr;
  const Slice qs = list_slice(p.grid, qlist, wave_valid ? p.n_q_slices : 0, kShift,
                              2 * e + (wave & 1));
  const bool q_ok = l32 < qs.cnt;
  const int64_t qrow = (int64_t)qs.start + (q_ok ? l32 : 0);
  const bf16_bits* Qh = static_cast<const bf16_bits*>(p.q) + bh * p.q_head_stride;
  bf16x8_t qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 16 * kk + 8 * hi);

  // ---- key tiles: tile u is the slices 2u and 2u + 1 of the block table ----
  const bf16_bits* Kh = static_cast<const bf16_bits*>(p.k) + bh * p.kv_head_stride;
  const bf16_bits* Vh = static_cast<const bf16_bits*>(p.v) + bh * p.kv_head_stride;
  const int32_t* tab = p.kv_tab ? p.kv_tab + bh * p.kv_tab_stride : nullptr;
  const int kv_slices = p.kv_rows / 32;
  const int n_tiles = (kv_slices + 1) / 2;
  const int last = n_tiles - 1;
  // The block grid stays in scalar registers (left alone, the compiler reloads
  // its fields from the kernel arguments on every tile, each load waited on at
  // once).
  BlockGrid g;
  g.L_src = __builtin_amdgcn_readfirstlane(p.grid.L_src);
  g.n_src = __builtin_amdgcn_readfirstlane(p.grid.n_src);
  g.N = __builtin_amdgcn_readfirstlane(p.grid.N);
  g.len = __builtin_amdgcn_readfirstlane(p.grid.len);
  asm("" : "+s"(g.L_src), "+s"(g.n_src), "+s"(g.N), "+s"(g.len));
  // The two slices of tile u (keys past a slice's valid rows, of partial blocks
  // or past an odd slice count, are masked), as the block ids read from the
  // table (TileIds) and as their rows (TileSrc).  Ids are read one iteration
  // before they are decoded, so no tile waits on a table read.
  struct TileSrc {
    Slice a, b;
  };
  struct TileIds {
    int a, b;
  };
  auto tile_ids = [&](int u) -> TileIds {
    if constexpr (kShift == 0) {  // one block per slice
      const int ea = 2 * u, eb = min(2 * u + 1, kv_slices - 1);
      return {tab ? tab[ea] : ea, tab ? tab[eb] : eb};
    } else {  // both slices in block u >> (kShift - 1)
      const int e = u >> (kShift - 1);
      const int blk = tab ? tab[e] : e;
      return {blk, blk};
    }
  };
  auto decode = [&](TileIds id, int u) -> TileSrc {
    TileSrc ts;
    if constexpr (kShift == 0) {
      ts.a = Slice{g.start(id.a), min(g.rows(id.a), 32)};
      ts.b = 2 * u + 1 < kv_slices ? Slice{g.start(id.b), min(g.rows(id.b), 32)} : Slice{0, 0};
    } else {
      const int sub = (u & ((1 << (kShift - 1)) - 1)) * 2;
      const int st = g.start(id.a), rows = g.rows(id.a);
      const int ca = min(max(rows - 32 * sub, 0), 32);
      const int cb = min(max(rows - 32 * (sub + 1), 0), 32);
      ts.a = Slice{ca > 0 ? st + 32 * sub : st, ca};
      ts.b = Slice{cb > 0 ? st + 32 * (sub + 1) : st, cb};
    }
    ts.a.start = __builtin_amdgcn_readfirstlane(ts.a.start);
    ts.a.cnt = __builtin_amdgcn_readfirstlane(ts.a.cnt);
    ts.b.start = __builtin_amdgcn_readfirstlane(ts.b.start);
    ts.b.cnt = __builtin_amdgcn_readfirstlane(ts.b.cnt);
    return ts;
  };
  auto tile_src = [&](int u) -> TileSrc { return decode(tile_ids(u), u); };

  // group A stages K: chunk c = gtid + 256 i -> row c / KC, column chunk c % KC
  uint4 k0, k1, k2, k3;
  // group B stages V^T: key group vg = gtid % 16 (4 keys), d chunk vd = gtid / 16
  uint4 v0, v1, v2, v3;
  const int vg = gtid % (kBN / 4);
  const int vd = gtid / (kBN / 4);
  const bool v_active = !gA && vd < KC;
  const int vq = vg & 3;
  const int vpos = (vg >> 2) * 16 + (((vq & 1) << 1) | (vq >> 1)) * 4;
  auto k_lds = [&](int b) { return smem + b * S::kKBytes; };
  auto v_lds = [&](int b) { return smem + 2 * S::kKBytes + b * S::kVBytes; };

  auto load_k = [&](const TileSrc& ts) __attribute__((always_inline)) {
    // rows past a slice's valid rows repeat its last one (they are masked)
    const bf16_bits* base_a = Kh + (int64_t)ts.a.start * D;
    const bf16_bits* base_b = Kh + (int64_t)ts.b.start * D;
    const int last_a = max(ts.a.cnt - 1, 0), last_b = max(ts.b.cnt - 1, 0);
    // chunk c = gtid + 256 I is row c / KC: slice ((256 / KC) I) / 32 of the tile
#define ISA_K_LOAD(I, R)                                                                \
  {                                                                                     \
    const int c = gtid + kGroup * I;                                                    \
    constexpr bool kSecond = ((kGroup / KC) * I) / 32 != 0;                             \
    const int row = min((c / KC) & 31, kSecond ? last_b : last_a);                      \
    R = *reinterpret_cast<const uint4*>((kSecond ? base_b : base_a) + row * D + (c % KC) * 8); \
  }
    ISA_K_LOAD(0, k0)
    ISA_K_LOAD(1, k1)
    if constexpr (KCH > 2) {
      ISA_K_LOAD(2, k2)
      ISA_K_LOAD(3, k3)
    }
#undef ISA_K_LOAD
  };
  auto store_k = [&](int b) __attribute__((always_inline)) {
    unsigned char* ks = k_lds(b);
#define ISA_K_STORE(I, R)                                                               \
  {                                                                                     \
    const int c = gtid + kGroup * I;                                                    \
    *reinterpret_cast<uint4*>(ks + (c / KC) * S::kKStride + (c % KC) * 16) = R;         \
  }
    ISA_K_STORE(0, k0)
    ISA_K_STORE(1, k1)
    if constexpr (KCH > 2) {
      ISA_K_STORE(2, k2)
      ISA_K_STORE(3, k3)
    }
#undef ISA_K_STORE
  };
  auto load_v = [&](const TileSrc& ts) __attribute__((always_inline)) {
    if (v_active) {
      // keys 4 vg .. 4 vg + 3 lie in slice vg / 8 of the tile
      const bool second = vg >= 8;
      const bf16_bits* vb = Vh + (int64_t)(second ? ts.b.start : ts.a.start) * D + vd * 8;
      const int last = max((second ? ts.b.cnt : ts.a.cnt) - 1, 0);
      const int r0 = 4 * (vg & 7);
      v0 = *reinterpret_cast<const uint4*>(vb + min(r0 + 0, last) * D);
      v1 = *reinterpret_cast<const uint4*>(vb + min(r0 + 1, last) * D);
      v2 = *reinterpret_cast<const uint4*>(vb + min(r0 + 2, last) * D);
      v3 = *reinterpret_cast<const uint4*>(vb + min(r0 + 3, last) * D);
    }
  };
  auto store_v = [&](int b) __attribute__((always_inline)) {
    if (v_active) {
      unsigned char* vrow = v_lds(b) + (vd * 8) * S::kVStride + vpos * 2;
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
  f32x16_t sacc[2];
  bf16x8_t pk[4];

  // S^T (64 keys x 32 queries) = K_tile Q^T
  auto qk = [&](const unsigned char* ks) __attribute__((always_inline)) {
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
  };
  // online softmax of sacc (exp2 domain) into the packed P^T operands
  auto softmax = [&](const TileSrc& ts) __attribute__((always_inline)) {
    {
      if (ts.a.cnt < 32 || ts.b.cnt < 32) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * hi + (r & 3);  // within slice s
            if (key >= (s ? ts.b.cnt : ts.a.cnt)) sacc[s][r] = -INFINITY;
          }
      }
    }
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
  };
  // O^T (D x 32 queries) += V^T P^T
  auto pv = [&](const unsigned char* vs) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            vs + (32 * j + l32) * S::kVStride + (16 * c + 8 * hi) * 2);
        oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[c], oacc[j], 0, 0, 0);
      }
    }
  };

  // ---- prologue (phase -1 and phase 0; B also phase 1) ----
  // tiles t, t + 1, t + 2 of the loop below, and the ids of tile t + 3
  TileSrc cur = tile_src(0), n1 = tile_src(min(1, last)), n2 = tile_src(min(2, last));
  TileIds id3 = tile_ids(min(3, last));
  if (gA) {
    load_k(cur);
    store_k(0);
  } else {
    load_v(cur);
  }
  phase_barrier();                                 // barrier 1
  if (gA) {                                        // phase 0: A computes S(0)
    qk(k_lds(0));
    if (n_tiles > 1) load_k(n1);
  } else {                                         // phase 0: B stores V(0)
    store_v(0);
    if (n_tiles > 1) load_v(n1);
  }
  phase_barrier();                                 // barrier 2
  if (!gA) {                                       // phase 1: B computes S(0)
    qk(k_lds(0));
    phase_barrier();                               // barrier 3 (A: end of its soft(0))
  }

  // ---- main loop: VALU phase, barrier, MFMA phase, barrier ----
  for (int t = 0; t < n_tiles; ++t) {
    // tile t + 3 from the ids read one iteration ago; read those of tile t + 4
    const TileSrc n3 = decode(id3, min(t + 3, last));
    id3 = tile_ids(min(t + 4, last));
    softmax(cur);
    if (t + 1 < n_tiles) {
      if (gA) {
        store_k((t + 1) & 1);
        if (t + 2 < n_tiles) load_k(n2);
      } else {
        store_v((t + 1) & 1);
        if (t + 2 < n_tiles) load_v(n2);
      }
    }
    cur = n1;
    n1 = n2;
    n2 = n3;
    // keep the exps of the softmax in this VALU phase: without the fences the
    // scheduler moves them past the barrier into the MFMA phase
    __builtin_amdgcn_sched_barrier(0);
    phase_barrier();
    __builtin_amdgcn_sched_barrier(0);
    pv(v_lds(t & 1));
    if (t + 1 < n_tiles) qk(k_lds((t + 1) & 1));
    // A: 2 barriers per tile; B skips the one after its last MFMA phase
    if (gA || t + 1 < n_tiles) phase_barrier();
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

hipError_t launch_attention_pp(const AttnParams& p, hipStream_t stream) {
  if (p.BH == 0 || p.n_q_entries == 0) return hipSuccess;
  if (p.kv_rows < 32 || p.kv_rows % 32 != 0 || p.kv_row_table) return hipErrorInvalidValue;
  if (p.half_shift < 0 || p.half_shift > 2) return hipErrorInvalidValue;
  const int wg_per_head = (p.n_q_entries + 3) / 4;
  const int64_t total = (int64_t)wg_per_head * p.BH;
  const dim3 grid((unsigned)(((total + 7) / 8) * 8));
#define ISA_PP_LAUNCH(DD, SH) \
  hipLaunchKernelGGL((attn_fwd_pp_kernel<DD, SH>), grid, dim3(kThreads), 0, stream, p)
  if (p.D == 128) {
    if (p.half_shift == 1) ISA_PP_LAUNCH(128, 1);
    else if (p.half_shift == 0) ISA_PP_LAUNCH(128, 0);
    else ISA_PP_LAUNCH(128, 2);
  } else {
    if (p.half_shift == 1) ISA_PP_LAUNCH(64, 1);
    else if (p.half_shift == 0) ISA_PP_LAUNCH(64, 0);
    else ISA_PP_LAUNCH(64, 2);
  }
#undef ISA_PP_LAUNCH
  return hipGetLastError();
}

}  // namespace isa
