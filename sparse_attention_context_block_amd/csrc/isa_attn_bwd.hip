// Backward of ISA with the forward's decisions held fixed: the trainable path
// of the pages ([notes] overall framework: the whole forward and backward are
// written as trainable kernels; highlights: the backward makes the sparse
// attention trainable end to end).  The pages print no gradient formulas; the
// decisions (TopK, routing) are constants, so the gradient flows through
//   exact rows:  P = softmax(q K_new^T / sqrt(D)), O = P V_new;
//   flat rows:   pi_j = w_j e^{q.K^c_j / sqrt(D)} / l, O = sum_j pi_j V^c_j,
//                with K^c_j, V^c_j the means of block j, so every token t of
//                block j receives dK^c_j / w_j and dV^c_j / w_j;
// and context rows whose block was not kept receive zero.
//
// Kernels (bf16 operands, fp32 accumulation, v_mfma_f32_32x32x16_bf16):
//   bwd_delta:   delta_r = dO_r . O_r.
//   bwd_prep:    block table of K_new from sel, keep flags, and the bf16 means
//                of the kept K/V blocks (the same values the forward used).
//   attn_bwd_dq: per 32 query rows (a wave), over the key tiles:
//                S^T = K Q^T, P^T = exp(S^T - lse), dP^T = V dO^T,
//                dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
//   attn_bwd_dkdv: per 32 keys (a wave), over the query blocks:
//                S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
//                Row-table mode (Taylor): keys are the pooled rows; writes
//                fp32 dK^c, dV^c.  Block-table mode (exact): writes dK, dV
//                rows of the kept blocks, adding dK^c / w and dV^c / w.
//   bwd_zero_unselected: zero dK, dV rows of context blocks not kept.
// Every operand whose contraction index is the key (or query) axis is staged
// transposed in LDS with the same in-chunk quad order (0, 2, 1, 3) the MFMA
// accumulator layout gives the packed P / dS operands (see the forward kernel).
#include <math.h>
#include <string.h>

#include "isa_internal.h"

namespace isa {

struct BwdParams {
  const bf16_bits* q;
  const bf16_bits* k;       // key source rows (K, or pooled K^c for row-table mode)
  const bf16_bits* v;       // value source rows (V, or pooled V^c)
  const bf16_bits* dout;
  const float* lse;         // forward LSE [BH][N]
  const float* delta;       // [BH][N]
  const int32_t* q_tab;     // [BH][q_tab_stride] 64-row query blocks
  int64_t q_tab_stride;
  int32_t n_q_entries;
  const int32_t* kv_tab;    // [BH][kv_tab_stride]
  int64_t kv_tab_stride;
  int32_t kv_rows;          // rows of the virtual K_new
  int64_t q_head_stride;    // elements between heads of Q, dO, dQ
  int64_t kv_head_stride;   // elements between heads of the key source
  int64_t lse_head_stride;  // N
  int32_t BH;
  float scale_log2;         // log2(e) / sqrt(D)
  float inv_sqrt_d;         // 1 / sqrt(D)
  float lse_offset;         // ln w (row-table mode), 0 (exact)
  // outputs
  bf16_bits* dq;            // [BH][N][D]
  float* dkc;               // row-table mode: [BH][kv_rows][D]
  float* dvc;
  bf16_bits* dk;            // block-table mode: [BH][N][D]
  bf16_bits* dv;
  const float* dkc_in;      // block-table mode: Taylor dK^c, dV^c to broadcast (or null)
  const float* dvc_in;
  int64_t dkc_head_stride;  // kv_rows of the Taylor buffers * D
  float inv_w;              // 1 / block weight
};

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;
// native vector (not HIP's uint4 struct) so staging registers never leave VGPRs
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// LDS tile of 64 rows x D bf16, row-major with a 16-byte row pad.
template <int D>
struct RM {
  static constexpr int kStride = D * 2 + 16;
  static constexpr int kBytes = kBN * kStride;
};
// LDS tile of D rows x 64 (transposed), quad-permuted positions, 16-byte pad.
template <int D>
struct TR {
  static constexpr int kStride = kBN * 2 + 16;
  static constexpr int kBytes = D * kStride;
};

// 16-byte chunk swizzle of the transposed tile: chunk c of row r sits at
// chunk c ^ tr_swz(r).  With the 16-byte row pad it keeps both the staging
// stores (one row per 8 dims, 16 threads a row group) and the MFMA operand
// reads (32 consecutive rows, one chunk) spread over all LDS banks.
__device__ __forceinline__ int tr_swz(int row) {
  const int x = (row >> 4) & 7;
  return x ^ ((x & 1) << 2);
}

// Byte offsets of the operand reads from a transposed tile: lane (l32, hi)
// reads chunk 2 C + hi of row 32 j + l32.  With b = bit 4 of the row, the
// swizzled chunk is (hi ^ b) + 2 ((C ^ j) & 1) + 4 (((C ^ j) >> 1) ^ b), so two
// per-lane bases and compile-time offsets cover every (j, C).
template <int D>
struct TrReader {
  int base0, base1;
  __device__ __forceinline__ void init(int l32, int hi) {
    const int b = (l32 >> 4) & 1;
    const int common = l32 * TR<D>::kStride + 16 * (hi ^ b);
    base0 = common + 64 * b;
    base1 = common + 64 * (1 - b);
  }
  __device__ __forceinline__ int off(int j, int C) const {
    const int k = C ^ j;
    return ((k >> 1) ? base1 : base0) + 32 * j * TR<D>::kStride + 32 * (k & 1);
  }
};

// Staging of one 64-row tile (rows given by row_of(r)) into registers and then
// into LDS: row-major only, or row-major and transposed from the same loads.
template <int D>
struct TileStager {
  static constexpr int KC = D / 8;                     // 16-byte chunks per row
  static constexpr int KCH = kBN * KC / kThreads;      // row-major chunks per thread
  u32x4 r0, r1, r2, r3;  // row-major only: chunk c = tid + 256 i
  u32x4 t0, t1, t2, t3;  // both layouts: rows 4 tg + i at chunk td
  bool t_active;
  int rm_off, tr_off;    // this thread's store offsets in the two layouts
  int tg, td;

  __device__ __forceinline__ void init(int tid) {
    // KC consecutive threads read one row (coalesced); the row groups of four
    // consecutive thread rows go in the order (0, 2, 1, 3), so each 32-lane
    // half of a transposed store fills whole 16-byte chunks
    td = tid % KC;
    const int q = tid / KC;
    tg = (q & ~3) | (((q & 1) << 1) | ((q >> 1) & 1));
    t_active = q < kBN / 4;
    // position of row 4 tg in the transposed layout (quad order (0, 2, 1, 3))
    const int tq = tg & 3;
    const int tpos = (tg >> 2) * 16 + (((tq & 1) << 1) | (tq >> 1)) * 4;
    rm_off = 4 * tg * RM<D>::kStride + td * 16;
    tr_off = td * 8 * TR<D>::kStride + 16 * ((tpos >> 3) ^ tr_swz(td * 8)) + (tpos & 7) * 2;
  }
  template <bool kTR, typename RowOf>
  __device__ __forceinline__ void load(const bf16_bits* base, int tid, RowOf row_of) {
    if constexpr (!kTR) {
#define ISA_LD(I, R)                                                                    \
  {                                                                                     \
    const int c = tid + kThreads * I;                                                   \
    R = *reinterpret_cast<const u32x4*>(base + row_of(c / KC) * D + (c % KC) * 8);      \
  }
      ISA_LD(0, r0)
      ISA_LD(1, r1)
      if constexpr (KCH > 2) {
        ISA_LD(2, r2)
        ISA_LD(3, r3)
      }
#undef ISA_LD
    } else {
      if (t_active) {
        const bf16_bits* b = base + td * 8;
        t0 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 0) * D);
        t1 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 1) * D);
        t2 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 2) * D);
        t3 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 3) * D);
      }
    }
  }
  template <bool kTR>
  __device__ __forceinline__ void store(unsigned char* rm, unsigned char* tr, int tid) {
    if constexpr (!kTR) {
#define ISA_ST(I, R)                                                                   \
  {                                                                                    \
    const int c = tid + kThreads * I;                                                  \
    *reinterpret_cast<u32x4*>(rm + (c / KC) * RM<D>::kStride + (c % KC) * 16) = R;     \
  }
      ISA_ST(0, r0)
      ISA_ST(1, r1)
      if constexpr (KCH > 2) {
        ISA_ST(2, r2)
        ISA_ST(3, r3)
      }
#undef ISA_ST
    } else {
      if (t_active) {
        unsigned char* r = rm + rm_off;
        *reinterpret_cast<u32x4*>(r) = t0;
        *reinterpret_cast<u32x4*>(r + RM<D>::kStride) = t1;
        *reinterpret_cast<u32x4*>(r + 2 * RM<D>::kStride) = t2;
        *reinterpret_cast<u32x4*>(r + 3 * RM<D>::kStride) = t3;
        // dims 8 td .. 8 td + 7 share one swizzle (rows 16 apart differ)
        unsigned char* row = tr + tr_off;
#define ISA_TS(W, F)                                                                    \
  *reinterpret_cast<uint2*>(row + (2 * W) * TR<D>::kStride) =                          \
      make_uint2(pack2(t0.F, t1.F, false), pack2(t2.F, t3.F, false));                  \
  *reinterpret_cast<uint2*>(row + (2 * W + 1) * TR<D>::kStride) =                      \
      make_uint2(pack2(t0.F, t1.F, true), pack2(t2.F, t3.F, true));
        ISA_TS(0, x)
        ISA_TS(1, y)
        ISA_TS(2, z)
        ISA_TS(3, w)
#undef ISA_TS
      }
    }
  }
};

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.0f;
  return z;
}

__device__ inline int64_t xcd_lid(int n_per_head, int BH, bool* valid) {
  const int total = n_per_head * BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  *valid = lid < total;
  return lid;
}

// --------------------------------------------------------------------------
// dQ: one wave = 32 query rows; a workgroup = two 64-row query blocks.
// --------------------------------------------------------------------------
template <int D, bool kRowTable>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int NKK = D / 16;
  constexpr int ND = D / 32;
  constexpr int kStage = RM<D>::kBytes * 2 + TR<D>::kBytes;  // K rm, V rm, K tr
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int wg_per_head = (p.n_q_entries + 1) / 2;
  bool ok;
  const int64_t lid = xcd_lid(wg_per_head, p.BH, &ok);
  if (!ok) return;
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int e = qt * 2 + (wave >> 1);
  const bool wave_valid = e < p.n_q_entries;
  const int qblk = wave_valid ? p.q_tab[bh * p.q_tab_stride + e] : 0;
  const int64_t qrow = (int64_t)qblk * kBlock + (wave & 1) * 32 + l32;
  const bf16_bits* Qh = p.q + bh * p.q_head_stride;
  const bf16_bits* dOh = p.dout + bh * p.q_head_stride;
  bf16x8_t qreg[NKK], oreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 16 * kk + 8 * hi);
    oreg[kk] = *reinterpret_cast<const bf16x8_t*>(dOh + qrow * D + 16 * kk + 8 * hi);
  }
  // An empty register dependency retires these loads here (one vmcnt wait).
  // Otherwise the wait pass cannot prove them done inside the loop and waits
  // for the next tile's prefetch loads before every MFMA that reads them.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm("" : "+v"(qreg[kk]), "+v"(oreg[kk]));
  const float lse2 = (p.lse[bh * p.lse_head_stride + qrow] - p.lse_offset) * 1.4426950408889634f;
  const float dlt = p.delta[bh * p.lse_head_stride + qrow];

  const bf16_bits* Kh = p.k + bh * p.kv_head_stride;
  const bf16_bits* Vh = p.v + bh * p.kv_head_stride;
  const int32_t* tab = p.kv_tab + bh * p.kv_tab_stride;
  const int n_tiles = (p.kv_rows + kBN - 1) / kBN;

  TileStager<D> ks, vs;
  ks.init(tid);
  vs.init(tid);
  TrReader<D> trr;
  trr.init(l32, hi);
  auto load = [&](int t) __attribute__((always_inline)) {
    if constexpr (kRowTable) {
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return tab[min(t * kBN + r, p.kv_rows - 1)]; };
      ks.template load<true>(Kh, tid, row_of);
      vs.template load<false>(Vh, tid, row_of);
    } else {
      const int64_t r0 = (int64_t)tab[t] * kBN;
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
      ks.template load<true>(Kh, tid, row_of);
      vs.template load<false>(Vh, tid, row_of);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    ks.template store<true>(b, b + 2 * RM<D>::kBytes, tid);
    vs.template store<false>(b + RM<D>::kBytes, nullptr, tid);
  };

  f32x16_t dq[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) dq[j] = zero16();
  const float sl2 = p.scale_log2;

  load(0);
  store(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load(t + 1);
    const unsigned char* krm = smem + buf * kStage;
    const unsigned char* vrm = krm + RM<D>::kBytes;
    const unsigned char* ktr = krm + 2 * RM<D>::kBytes;

    // four independent accumulator chains (s, dp of both key halves), so no
    // MFMA waits on the one before it
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = zero16();
      dp[h] = zero16();
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = (32 * h + l32) * RM<D>::kStride + (16 * kk + 8 * hi) * 2;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krm + off);
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[h], 0, 0, 0);
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(vrm + off);
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, oreg[kk], dp[h], 0, 0, 0);
      }
    }
    // mask keys past the end (only a row-table tile can be partial): P = 0
    const int valid = p.kv_rows - t * kBN;
    if (kRowTable && valid < kBN) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * h + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= valid) s[h][r] = -INFINITY;
        }
    }
    // dS^T = P^T (dP^T - delta), packed as the B operand of dQ^T += K^T dS^T:
    // chunk C takes registers 8 (C & 1) .. + 7 of subtile C >> 1
    bf16x8_t ds0, ds1, ds2, ds3;
#define ISA_DS(V, C)                                                                    \
  _Pragma("unroll") for (int e2 = 0; e2 < 8; ++e2) {                                    \
    const int r = 8 * ((C) & 1) + e2;                                                   \
    const float pr = __builtin_amdgcn_exp2f(fmaf(s[(C) >> 1][r], sl2, -lse2));          \
    V[e2] = (__bf16)(pr * (dp[(C) >> 1][r] - dlt));                                     \
  }
    ISA_DS(ds0, 0)
    ISA_DS(ds1, 1)
    ISA_DS(ds2, 2)
    ISA_DS(ds3, 3)
#undef ISA_DS
#define ISA_DQ(V, C)                                                                    \
  _Pragma("unroll") for (int j = 0; j < ND; ++j) {                                      \
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ktr + trr.off(j, C));         \
    dq[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, V, dq[j], 0, 0, 0);              \
  }
    ISA_DQ(ds0, 0)
    ISA_DQ(ds1, 1)
    ISA_DQ(ds2, 2)
    ISA_DQ(ds3, 3)
#undef ISA_DQ
    if (t + 1 < n_tiles) store(buf ^ 1);
    __syncthreads();
  }
  if (!wave_valid) return;
  bf16_bits* dQh = p.dq + bh * p.q_head_stride + qrow * D;
  const float sc = p.inv_sqrt_d;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x2_t a, b;
      a[0] = (__bf16)(dq[j][4 * g + 0] * sc);
      a[1] = (__bf16)(dq[j][4 * g + 1] * sc);
      b[0] = (__bf16)(dq[j][4 * g + 2] * sc);
      b[1] = (__bf16)(dq[j][4 * g + 3] * sc);
      *reinterpret_cast<uint2*>(dQh + 32 * j + 8 * g + 4 * hi) =
          make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
    }
  }
}

// --------------------------------------------------------------------------
// dK, dV: one wave = 32 keys; a workgroup = 128 keys (two 64-row blocks).
// --------------------------------------------------------------------------
template <int D, bool kRowTable>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NKK = D / 16;
  constexpr int ND = D / 32;
  // Q rm, dO rm, Q tr, dO tr, lse2[64], delta[64]
  constexpr int kStage = 2 * RM<D>::kBytes + 2 * TR<D>::kBytes + 2 * kBN * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int kv_wgs = (p.kv_rows + 127) / 128;
  bool ok;
  const int64_t lid = xcd_lid(kv_wgs, p.BH, &ok);
  if (!ok) return;
  const int64_t bh = lid / kv_wgs;
  const int kt = lid % kv_wgs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // this wave's 32 keys (virtual rows of K_new)
  const int vrow = kt * 128 + wave * 32 + l32;
  const bool key_valid = vrow < p.kv_rows;
  const int32_t* tab = p.kv_tab + bh * p.kv_tab_stride;
  const int vr = min(vrow, p.kv_rows - 1);
  const int64_t krow = kRowTable ? (int64_t)tab[vr] : (int64_t)tab[vr >> 6] * kBN + (vr & 63);
  const bf16_bits* Kh = p.k + bh * p.kv_head_stride;
  const bf16_bits* Vh = p.v + bh * p.kv_head_stride;
  bf16x8_t kreg[NKK], vreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kreg[kk] = *reinterpret_cast<const bf16x8_t*>(Kh + krow * D + 16 * kk + 8 * hi);
    vreg[kk] = *reinterpret_cast<const bf16x8_t*>(Vh + krow * D + 16 * kk + 8 * hi);
  }
  // retire these loads here (see the dQ kernel)
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm("" : "+v"(kreg[kk]), "+v"(vreg[kk]));

  const bf16_bits* Qh = p.q + bh * p.q_head_stride;
  const bf16_bits* dOh = p.dout + bh * p.q_head_stride;
  const float* lseh = p.lse + bh * p.lse_head_stride;
  const float* dlth = p.delta + bh * p.lse_head_stride;
  const int32_t* qtab = p.q_tab + bh * p.q_tab_stride;
  TileStager<D> qs, os;
  qs.init(tid);
  os.init(tid);
  TrReader<D> trr;
  trr.init(l32, hi);
  float st_lse = 0.0f;  // thread tid < 64: lse2 of query row tid; 64..127: delta
  auto load = [&](int e) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)qtab[e] * kBlock;
    auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
    qs.template load<true>(Qh, tid, row_of);
    os.template load<true>(dOh, tid, row_of);
    if (tid < kBN)
      st_lse = (lseh[r0 + tid] - p.lse_offset) * 1.4426950408889634f;
    else if (tid < 2 * kBN)
      st_lse = dlth[r0 + tid - kBN];
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    qs.template store<true>(b, b + 2 * RM<D>::kBytes, tid);
    os.template store<true>(b + RM<D>::kBytes, b + 2 * RM<D>::kBytes + TR<D>::kBytes, tid);
    if (tid < 2 * kBN)
      reinterpret_cast<float*>(b + 2 * RM<D>::kBytes + 2 * TR<D>::kBytes)[tid] = st_lse;
  };

  f32x16_t dk[ND], dv[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    dk[j] = zero16();
    dv[j] = zero16();
  }
  const float sl2 = p.scale_log2;
  const int n_q = p.n_q_entries;
  if (n_q > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int e = 0; e < n_q; ++e) {
    const int buf = e & 1;
    if (e + 1 < n_q) load(e + 1);
    const unsigned char* qrm = smem + buf * kStage;
    const unsigned char* orm = qrm + RM<D>::kBytes;
    const unsigned char* qtr = qrm + 2 * RM<D>::kBytes;
    const unsigned char* otr = qtr + TR<D>::kBytes;
    const float* lse_s = reinterpret_cast<const float*>(otr + TR<D>::kBytes);
    const float* dlt_s = lse_s + kBN;

    // S (64 queries x 32 keys) = Q K^T and dP = dO V^T; lane = key, regs = queries
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = zero16();
      dp[h] = zero16();
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // four independent accumulator chains
        const int off = (32 * h + l32) * RM<D>::kStride + (16 * kk + 8 * hi) * 2;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(qrm + off);
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kreg[kk], s[h], 0, 0, 0);
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(orm + off);
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, vreg[kk], dp[h], 0, 0, 0);
      }
    }
    // P and dS = P (dP - delta), packed as the B operands of the query
    // contractions; chunk C takes registers 8 (C & 1) .. + 7 of subtile C >> 1,
    // whose queries are 32 h + 8 (r >> 2) + 4 hi + (r & 3)
    bf16x8_t pk0, pk1, pk2, pk3, dk0, dk1, dk2, dk3;
#define ISA_PDS(PV, DV, C)                                                              \
  _Pragma("unroll") for (int g2 = 0; g2 < 2; ++g2) {                                    \
    const int h = (C) >> 1;                                                             \
    const int rb = 8 * ((C) & 1) + 4 * g2;                                              \
    const int q0 = 32 * h + 8 * (rb >> 2) + 4 * hi;                                     \
    const float4 l4 = *reinterpret_cast<const float4*>(lse_s + q0);                     \
    const float4 d4 = *reinterpret_cast<const float4*>(dlt_s + q0);                     \
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[h][rb + 0], sl2, -l4.x));            \
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[h][rb + 1], sl2, -l4.y));            \
    const float p2 = __builtin_amdgcn_exp2f(fmaf(s[h][rb + 2], sl2, -l4.z));            \
    const float p3 = __builtin_amdgcn_exp2f(fmaf(s[h][rb + 3], sl2, -l4.w));            \
    PV[4 * g2 + 0] = (__bf16)p0;                                                        \
    PV[4 * g2 + 1] = (__bf16)p1;                                                        \
    PV[4 * g2 + 2] = (__bf16)p2;                                                        \
    PV[4 * g2 + 3] = (__bf16)p3;                                                        \
    DV[4 * g2 + 0] = (__bf16)(p0 * (dp[h][rb + 0] - d4.x));                             \
    DV[4 * g2 + 1] = (__bf16)(p1 * (dp[h][rb + 1] - d4.y));                             \
    DV[4 * g2 + 2] = (__bf16)(p2 * (dp[h][rb + 2] - d4.z));                             \
    DV[4 * g2 + 3] = (__bf16)(p3 * (dp[h][rb + 3] - d4.w));                             \
  }
    ISA_PDS(pk0, dk0, 0)
    ISA_PDS(pk1, dk1, 1)
    ISA_PDS(pk2, dk2, 2)
    ISA_PDS(pk3, dk3, 3)
#undef ISA_PDS
    // dV^T += dO^T P, dK^T += Q^T dS (contraction over the 64 queries)
#define ISA_KV(PV, DV, C)                                                               \
  _Pragma("unroll") for (int j = 0; j < ND; ++j) {                                      \
    const int off = trr.off(j, C);                                                      \
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(otr + off);                   \
    dv[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, PV, dv[j], 0, 0, 0);             \
    const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(qtr + off);                   \
    dk[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, DV, dk[j], 0, 0, 0);             \
  }
    ISA_KV(pk0, dk0, 0)
    ISA_KV(pk1, dk1, 1)
    ISA_KV(pk2, dk2, 2)
    ISA_KV(pk3, dk3, 3)
#undef ISA_KV
    if (e + 1 < n_q) store(buf ^ 1);
    __syncthreads();
  }
  if (!key_valid) return;

  // lane = key; accumulator register r of subtile j holds dim 32 j + 8 (r >> 2) + 4 hi + (r & 3)
  const float sc = p.inv_sqrt_d;
  if constexpr (kRowTable) {
    float* dkc = p.dkc + bh * p.dkc_head_stride + (int64_t)vrow * D;
    float* dvc = p.dvc + bh * p.dkc_head_stride + (int64_t)vrow * D;
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * j + 8 * g + 4 * hi;
        *reinterpret_cast<float4*>(dkc + d0) =
            make_float4(dk[j][4 * g] * sc, dk[j][4 * g + 1] * sc, dk[j][4 * g + 2] * sc,
                        dk[j][4 * g + 3] * sc);
        *reinterpret_cast<float4*>(dvc + d0) =
            make_float4(dv[j][4 * g], dv[j][4 * g + 1], dv[j][4 * g + 2], dv[j][4 * g + 3]);
      }
  } else {
    // the Taylor path's pooled gradient of this key's block, spread over its tokens
    const int blk = vrow >> 6;
    const float* tk = p.dkc_in ? p.dkc_in + bh * p.dkc_head_stride + (int64_t)blk * D : nullptr;
    const float* tv = p.dvc_in ? p.dvc_in + bh * p.dkc_head_stride + (int64_t)blk * D : nullptr;
    bf16_bits* dKh = p.dk + bh * p.q_head_stride + krow * D;
    bf16_bits* dVh = p.dv + bh * p.q_head_stride + krow * D;
    const float iw = p.inv_w;
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * j + 8 * g + 4 * hi;
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = dk[j][4 * g + i] * sc;
          b[i] = dv[j][4 * g + i];
        }
        if (tk) {
          const float4 x = *reinterpret_cast<const float4*>(tk + d0);
          const float4 y = *reinterpret_cast<const float4*>(tv + d0);
          a[0] += x.x * iw; a[1] += x.y * iw; a[2] += x.z * iw; a[3] += x.w * iw;
          b[0] += y.x * iw; b[1] += y.y * iw; b[2] += y.z * iw; b[3] += y.w * iw;
        }
        bf16x2_t a0, a1, b0, b1;
        a0[0] = (__bf16)a[0]; a0[1] = (__bf16)a[1]; a1[0] = (__bf16)a[2]; a1[1] = (__bf16)a[3];
        b0[0] = (__bf16)b[0]; b0[1] = (__bf16)b[1]; b1[0] = (__bf16)b[2]; b1[1] = (__bf16)b[3];
        *reinterpret_cast<uint2*>(dKh + d0) =
            make_uint2(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1));
        *reinterpret_cast<uint2*>(dVh + d0) =
            make_uint2(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1));
      }
  }
}

// delta_r = dO_r . O_r over D (one thread per row, fp32)
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16_bits* __restrict__ O,
                                                             const bf16_bits* __restrict__ dO,
                                                             int64_t rows,
                                                             float* __restrict__ delta) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= rows) return;
  const uint4* o = reinterpret_cast<const uint4*>(O + r * D);
  const uint4* g = reinterpret_cast<const uint4*>(dO + r * D);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const uint4 a = o[i], b = g[i];
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(wa[k] << 16), __uint_as_float(wb[k] << 16), acc);
      acc = fmaf(__uint_as_float(wa[k] & 0xffff0000u), __uint_as_float(wb[k] & 0xffff0000u), acc);
    }
  }
  delta[r] = acc;
}

// Per (kept block t, head): block table entry and the bf16 means of the block's
// K and V rows (fp64 sums, rounded as the forward's pooling rounds them).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    const bf16_bits* __restrict__ K, const bf16_bits* __restrict__ V,
    const int32_t* __restrict__ sel, int N, int n_src, int k, int32_t* __restrict__ kv_tab,
    int32_t* __restrict__ iota, bf16_bits* __restrict__ kc, bf16_bits* __restrict__ vc) {
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int n_kv = n_src + k;
  const int blk = t < n_src ? t : n_src + sel[bh * k + (t - n_src)];
  if (threadIdx.x == 0) {
    kv_tab[bh * n_kv + t] = blk;
    if (bh == 0) iota[t] = t;  // identity row table of the compact pooled rows
  }
  __shared__ double red[2][kThreads / D * 2][D];
  const int tid = threadIdx.x;
  const int d = tid % D;
  const int g = tid / D;           // row group
  constexpr int G = kThreads / D;  // row groups
  const bf16_bits* kb = K + (bh * N + (int64_t)blk * kBlock) * D;
  const bf16_bits* vb = V + (bh * N + (int64_t)blk * kBlock) * D;
  double sk = 0.0, sv = 0.0;
  for (int r = g; r < kBlock; r += G) {
    sk += (double)__uint_as_float((uint32_t)kb[r * D + d] << 16);
    sv += (double)__uint_as_float((uint32_t)vb[r * D + d] << 16);
  }
  red[0][g][d] = sk;
  red[1][g][d] = sv;
  __syncthreads();
  if (tid < D) {
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      a += red[0][i][tid];
      b += red[1][i][tid];
    }
    const int64_t o = (bh * n_kv + t) * (int64_t)D + tid;
    kc[o] = (bf16_bits)bf16_bits_rne(a * (1.0 / kBlock));  // as the forward's pooling rounds
    vc[o] = (bf16_bits)bf16_bits_rne(b * (1.0 / kBlock));
  }
}

// dK, dV rows of context blocks that were not kept are zero.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_zero_unselected_kernel(
    const int32_t* __restrict__ sel, int N, int L_src, int k, bf16_bits* __restrict__ dK,
    bf16_bits* __restrict__ dV) {
  const int j = blockIdx.x;  // context block
  const int64_t bh = blockIdx.y;
  for (int i = 0; i < k; ++i)
    if (sel[bh * k + i] == j) return;  // kept: written by the exact kernel
  uint4* a = reinterpret_cast<uint4*>(dK + (bh * N + L_src + (int64_t)j * kBlock) * D);
  uint4* b = reinterpret_cast<uint4*>(dV + (bh * N + L_src + (int64_t)j * kBlock) * D);
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int i = threadIdx.x; i < kBlock * D / 8; i += kThreads) {
    a[i] = z;
    b[i] = z;
  }
}

template <typename Kern>
hipError_t launch_xcd(Kern kern, int per_head, int BH, const BwdParams& p, hipStream_t s) {
  const int64_t total = (int64_t)per_head * BH;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)(((total + 7) / 8) * 8)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Backward launch sequence (see the top of this file).
hipError_t launch_backward(const BwdLaunch& L, hipStream_t s) {
  const int BH = L.BH, D = L.D;
  const int64_t rows = (int64_t)BH * L.N;
  hipError_t e;
#define ISA_CHECK(x) \
  if ((e = (x)) != hipSuccess) return e;
  if (rows > 0) {
    if (D == 128)
      hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                         dim3(kThreads), 0, s, L.O, L.dO, rows, L.delta);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                         dim3(kThreads), 0, s, L.O, L.dO, rows, L.delta);
    ISA_CHECK(hipGetLastError());
  }
  const int n_kv = L.n_src + L.k;
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(n_kv, BH), dim3(kThreads), 0, s, L.K, L.V,
                       L.sel, L.N, L.n_src, L.k, L.kv_tab, L.iota, L.kc, L.vc);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(n_kv, BH), dim3(kThreads), 0, s, L.K, L.V, L.sel,
                       L.N, L.n_src, L.k, L.kv_tab, L.iota, L.kc, L.vc);
  ISA_CHECK(hipGetLastError());

  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = L.Q;
  p.dout = L.dO;
  p.lse = L.lse;
  p.delta = L.delta;
  p.kv_tab = L.kv_tab;
  p.kv_tab_stride = n_kv;
  p.q_head_stride = (int64_t)L.N * D;
  p.lse_head_stride = L.N;
  p.BH = BH;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  p.inv_sqrt_d = (float)(1.0 / sqrt((double)D));
  p.dq = L.dQ;
  p.dk = L.dK;
  p.dv = L.dV;
  p.dkc_head_stride = (int64_t)n_kv * D;

  // Taylor path (flat query blocks against the pooled kept blocks)
  BwdParams pt = p;
  pt.k = L.kc;
  pt.v = L.vc;
  pt.kv_rows = n_kv;
  pt.kv_head_stride = (int64_t)n_kv * D;
  pt.lse_offset = (float)log((double)kBlock);
  pt.q_tab = L.flat;
  pt.q_tab_stride = L.n_flat;
  pt.n_q_entries = L.n_flat;
  // keys = pooled rows t of this head's compact K^c_new: an identity row table
  pt.kv_tab = L.iota;
  pt.kv_tab_stride = 0;
  pt.dkc = L.dkc;
  pt.dvc = L.dvc;
  if (L.n_flat > 0) {
    if (D == 128) {
      ISA_CHECK(launch_xcd(attn_bwd_dkdv_kernel<128, true>, (n_kv + 127) / 128, BH, pt, s));
      ISA_CHECK(launch_xcd(attn_bwd_dq_kernel<128, true>, (L.n_flat + 1) / 2, BH, pt, s));
    } else {
      ISA_CHECK(launch_xcd(attn_bwd_dkdv_kernel<64, true>, (n_kv + 127) / 128, BH, pt, s));
      ISA_CHECK(launch_xcd(attn_bwd_dq_kernel<64, true>, (L.n_flat + 1) / 2, BH, pt, s));
    }
  }

  // exact path (sharp query blocks against K_new through the block table)
  BwdParams pe = p;
  pe.k = L.K;
  pe.v = L.V;
  pe.kv_rows = n_kv * kBlock;
  pe.kv_head_stride = (int64_t)L.N * D;
  pe.lse_offset = 0.0f;
  pe.q_tab = L.sharp;
  pe.q_tab_stride = L.n_sharp;
  pe.n_q_entries = L.n_sharp;
  pe.dkc_in = L.n_flat > 0 ? L.dkc : nullptr;
  pe.dvc_in = L.n_flat > 0 ? L.dvc : nullptr;
  pe.inv_w = 1.0f / (float)kBlock;
  if (D == 128) {
    ISA_CHECK(launch_xcd(attn_bwd_dkdv_kernel<128, false>, (n_kv * kBlock + 127) / 128, BH, pe, s));
    if (L.n_sharp > 0)
      ISA_CHECK(launch_xcd(attn_bwd_dq_kernel<128, false>, (L.n_sharp + 1) / 2, BH, pe, s));
  } else {
    ISA_CHECK(launch_xcd(attn_bwd_dkdv_kernel<64, false>, (n_kv * kBlock + 127) / 128, BH, pe, s));
    if (L.n_sharp > 0)
      ISA_CHECK(launch_xcd(attn_bwd_dq_kernel<64, false>, (L.n_sharp + 1) / 2, BH, pe, s));
  }
  if (L.n_ctx > 0) {
    if (D == 128)
      hipLaunchKernelGGL(bwd_zero_unselected_kernel<128>, dim3(L.n_ctx, BH), dim3(kThreads), 0, s,
                         L.sel, L.N, L.L_src, L.k, L.dK, L.dV);
    else
      hipLaunchKernelGGL(bwd_zero_unselected_kernel<64>, dim3(L.n_ctx, BH), dim3(kThreads), 0, s,
                         L.sel, L.N, L.L_src, L.k, L.dK, L.dV);
    ISA_CHECK(hipGetLastError());
  }
#undef ISA_CHECK
  return hipSuccess;
}

}  // namespace isa
