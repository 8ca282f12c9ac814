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
// Kernels (bf16 operands, fp32 accumulation, v_mfma_f32_16x16x32_bf16):
//   bwd_delta:   delta_r = dO_r . O_r.
//   bwd_prep:    block table of K_new from sel, keep flags, and the bf16 means
//                of the kept K/V blocks (the same values the forward used).
//   attn_bwd_dq16: per 16 query rows (a wave), over the key tiles:
//                S^T = K Q^T, P^T = exp(S^T - lse), dP^T = V dO^T,
//                dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
//   attn_bwd_dkdv16: per 16 keys (a wave), over the query blocks:
//                S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
//                Row-table mode (Taylor): keys are the pooled rows; writes
//                fp32 dK^c, dV^c.  Block-table mode (exact): writes dK, dV
//                rows of the kept blocks, adding dK^c / w and dV^c / w.
//   bwd_zero_unselected: zero dK, dV rows of context blocks not kept.
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

__device__ inline int64_t xcd_lid(int n_per_head, int BH, bool* valid) {
  const int total = n_per_head * BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  *valid = lid < total;
  return lid;
}

// --------------------------------------------------------------------------
// 16x16 variants (v_mfma_f32_16x16x32_bf16, 8 waves, 16 rows per wave).
// Every product is arranged so that the S / dP accumulators a lane holds are
// exactly the B-operand slots of the next product (lane l, q = l % 16,
// g = l / 16 holds rows 4 g + i of each 16-row subtile; the 32-wide contraction
// chunk c takes slots 8 g + (0..3) = rows 32 c + 4 g + (0..3) and
// 8 g + (4..7) = rows 32 c + 16 + 4 g + (0..3)).  Operands whose contraction
// runs over a tile's rows come from a transposed copy of the tile whose 64
// positions follow that slot order, so every operand is one ds_read_b128.
// A wave fits in 256 VGPRs: two waves share each SIMD.
//
// LDS layouts, chosen by measuring each access pattern alone on gfx950
// (time and SQ_LDS_BANK_CONFLICT): 16-lane groups reading one 16-byte chunk
// of 16 consecutive rows run conflict-free with a row stride of 288 or 160
// bytes and at half rate with 272 or 144; transposing ds_read_b64_tr_b16
// reads move a third of the bytes per cycle of a b128 read, which is why the
// copies are staged transposed:
//   row-major tile:  64 rows, stride 2 D + 32 bytes;
//   transposed tile: D rows (dims) x 64 positions, stride 160 bytes, the
//                    16-byte chunk index XORed with (row >> 4) & 7.  Without
//                    it the staging writes (one row per 8 dims) collide 16-fold;
//                    an XOR that also varies inside a 16-row group (row >> 3)
//                    doubles the cost of the operand reads.
// --------------------------------------------------------------------------
constexpr int kT16 = 512;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <int D>
struct RS {
  static constexpr int kStride = D * 2 + 32;
  static constexpr int kBytes = kBN * kStride;
  __device__ static __forceinline__ int off(int row, int byte) { return row * kStride + byte; }
};
struct TS {
  static constexpr int kStride = kBN * 2 + 32;
  template <int D>
  static constexpr int bytes() { return D * kStride; }
  __device__ static __forceinline__ int off(int row, int byte) {
    return row * kStride + (((byte >> 4) ^ ((row >> 4) & 7)) << 4) + (byte & 15);
  }
};

// Position of tile row r in the transposed tile (the slot order above): rows
// 32 c + 4 g + j sit at 32 c + 8 g + j, rows 32 c + 16 + 4 g + j at
// 32 c + 8 g + 4 + j.
__device__ __forceinline__ int slot_pos(int r) {
  const int c = r >> 5, x = r & 31;
  return 32 * c + 8 * ((x & 15) >> 2) + 4 * (x >> 4) + (x & 3);
}

// Stages one 64-row tile (rows row_of(r)) of a [.., D] bf16 array with 256
// threads: thread (td = t % KC, tg = t / KC) loads rows 4 tg .. 4 tg + 3 at
// 16-byte column td (KC threads read one row: coalesced) and writes them to
// the row-major tile and, if tr is not null, to the transposed tile.
template <int D>
struct Stager16 {
  static constexpr int KC = D / 8;
  u32x4 t0, t1, t2, t3;
  int td, tg;
  bool active;
  __device__ __forceinline__ void init(int t) {
    td = t % KC;
    tg = t / KC;
    active = tg < kBN / 4;
  }
  template <typename RowOf>
  __device__ __forceinline__ void load(const bf16_bits* base, RowOf row_of) {
    if (!active) return;
    const bf16_bits* b = base + td * 8;
    t0 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 0) * D);
    t1 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 1) * D);
    t2 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 2) * D);
    t3 = *reinterpret_cast<const u32x4*>(b + row_of(4 * tg + 3) * D);
  }
  __device__ __forceinline__ void store(unsigned char* rm, unsigned char* tr) {
    if (!active) return;
    unsigned char* r = rm + RS<D>::off(4 * tg, td * 16);
    *reinterpret_cast<u32x4*>(r) = t0;
    *reinterpret_cast<u32x4*>(r + RS<D>::kStride) = t1;
    *reinterpret_cast<u32x4*>(r + 2 * RS<D>::kStride) = t2;
    *reinterpret_cast<u32x4*>(r + 3 * RS<D>::kStride) = t3;
    if (tr) {
      // dims 8 td + e: four rows' values of one dim are 8 consecutive bytes
      const int byte = 2 * slot_pos(4 * tg);
#define ISA_TS16(W, F)                                                                  \
  *reinterpret_cast<uint2*>(tr + TS::off(8 * td + 2 * W, byte)) =                      \
      make_uint2(pack2(t0.F, t1.F, false), pack2(t2.F, t3.F, false));                  \
  *reinterpret_cast<uint2*>(tr + TS::off(8 * td + 2 * W + 1, byte)) =                  \
      make_uint2(pack2(t0.F, t1.F, true), pack2(t2.F, t3.F, true));
      ISA_TS16(0, x)
      ISA_TS16(1, y)
      ISA_TS16(2, z)
      ISA_TS16(3, w)
#undef ISA_TS16
    }
  }
};

// The 16x32 operand of a transposed tile: lane (q, g) reads dims row0 + q,
// slots 8 g .. 8 g + 7 of contraction chunk c.
__device__ __forceinline__ bf16x8_t ts_operand(const unsigned char* tr, int row0, int c, int q,
                                               int g) {
  return *reinterpret_cast<const bf16x8_t*>(tr + TS::off(row0 + q, (32 * c + 8 * g) * 2));
}

__device__ __forceinline__ bf16x8_t pack_slots(const f32x4_t& a, const f32x4_t& b) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (__bf16)a[i];
    v[4 + i] = (__bf16)b[i];
  }
  return v;
}

// dK, dV: a wave owns 16 keys (lane q: key q), a workgroup 128 keys; over the
// query blocks: S = Q K^T and dP = dO V^T (queries x keys), P, dS = P (dP -
// delta), dV^T += dO^T P and dK^T += Q^T dS (dims x keys).
template <int D, bool kRowTable>
__global__ __launch_bounds__(kT16) void attn_bwd_dkdv16_kernel(BwdParams p) {
  constexpr int NKK = D / 32;
  constexpr int ND = D / 16;
  // Q, dO row-major; Q, dO transposed; lse2[64], delta[64]
  constexpr int kStage = 2 * RS<D>::kBytes + 2 * TS::bytes<D>() + 2 * kBN * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int kv_wgs = (p.kv_rows + 127) / 128;
  bool ok;
  const int64_t lid = xcd_lid(kv_wgs, p.BH, &ok);
  if (!ok) return;
  const int64_t bh = lid / kv_wgs;
  const int kt = lid % kv_wgs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 15, g = lane >> 4;

  // this wave's 16 keys (virtual rows of K_new); lane (q, g) holds dims
  // 32 kk + 8 g .. + 7 of key q
  const int vrow = kt * 128 + wave * 16 + q;
  const bool key_valid = vrow < p.kv_rows;
  const int32_t* tab = p.kv_tab + bh * p.kv_tab_stride;
  const int vr = min(vrow, p.kv_rows - 1);
  const int64_t krow = kRowTable ? (int64_t)tab[vr] : (int64_t)tab[vr >> 6] * kBN + (vr & 63);
  const bf16_bits* Kh = p.k + bh * p.kv_head_stride;
  const bf16_bits* Vh = p.v + bh * p.kv_head_stride;
  bf16x8_t kreg[NKK], vreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kreg[kk] = *reinterpret_cast<const bf16x8_t*>(Kh + krow * D + 32 * kk + 8 * g);
    vreg[kk] = *reinterpret_cast<const bf16x8_t*>(Vh + krow * D + 32 * kk + 8 * g);
  }
  // retire these loads here (see the dQ kernel)
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm("" : "+v"(kreg[kk]), "+v"(vreg[kk]));

  const bf16_bits* Qh = p.q + bh * p.q_head_stride;
  const bf16_bits* dOh = p.dout + bh * p.q_head_stride;
  const float* lseh = p.lse + bh * p.lse_head_stride;
  const float* dlth = p.delta + bh * p.lse_head_stride;
  const int32_t* qtab = p.q_tab + bh * p.q_tab_stride;
  // threads 0-255 stage Q, 256-511 stage dO (both layouts)
  const int half = tid >> 8;
  Stager16<D> st;
  st.init(tid & 255);
  float st_lse = 0.0f;  // thread tid < 64: lse2 of query row tid; 64..127: delta
  auto load = [&](int e) __attribute__((always_inline)) {
    const int64_t r0 = (int64_t)qtab[e] * kBlock;
    auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
    st.load(half ? dOh : Qh, row_of);
    if (tid < kBN)
      st_lse = (lseh[r0 + tid] - p.lse_offset) * 1.4426950408889634f;
    else if (tid < 2 * kBN)
      st_lse = dlth[r0 + tid - kBN];
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    st.store(b + half * RS<D>::kBytes, b + 2 * RS<D>::kBytes + half * TS::bytes<D>());
    if (tid < 2 * kBN)
      reinterpret_cast<float*>(b + 2 * RS<D>::kBytes + 2 * TS::bytes<D>())[tid] = st_lse;
  };

  f32x4_t dk[ND], dv[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dk[j][i] = 0.0f;
      dv[j][i] = 0.0f;
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
    const unsigned char* qt = smem + buf * kStage;
    const unsigned char* ot = qt + RS<D>::kBytes;
    const unsigned char* qtr = ot + RS<D>::kBytes;
    const unsigned char* otr = qtr + TS::bytes<D>();
    const float* lse_s = reinterpret_cast<const float*>(otr + TS::bytes<D>());
    const float* dlt_s = lse_s + kBN;

    // S and dP subtile n: queries 16 n + 4 g + i, key q
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[n][i] = 0.0f;
        dp[n][i] = 0.0f;
      }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {  // eight independent accumulator chains
        const int off = RS<D>::off(16 * n + q, (32 * kk + 8 * g) * 2);
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(qt + off);
        s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kreg[kk], s[n], 0, 0, 0);
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(ot + off);
        dp[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, vreg[kk], dp[n], 0, 0, 0);
      }
    }
    // P and dS; the query chunk c of the B operands takes subtiles 2c, 2c + 1
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float4 l4 = *reinterpret_cast<const float4*>(lse_s + 16 * n + 4 * g);
      const float4 d4 = *reinterpret_cast<const float4*>(dlt_s + 16 * n + 4 * g);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[n][i], sl2, -lv[i]));
        s[n][i] = pr;
        dp[n][i] = pr * (dp[n][i] - dv4[i]);
      }
    }
    const bf16x8_t pk0 = pack_slots(s[0], s[1]), pk1 = pack_slots(s[2], s[3]);
    const bf16x8_t ds0 = pack_slots(dp[0], dp[1]), ds1 = pack_slots(dp[2], dp[3]);
    // dV^T += dO^T P, dK^T += Q^T dS: dims 16 j + 4 g + i of key q
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const bf16x8_t a0 = ts_operand(otr, 16 * j, 0, q, g);
      dv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, pk0, dv[j], 0, 0, 0);
      const bf16x8_t b0 = ts_operand(qtr, 16 * j, 0, q, g);
      dk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, ds0, dk[j], 0, 0, 0);
      const bf16x8_t a1 = ts_operand(otr, 16 * j, 1, q, g);
      dv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, pk1, dv[j], 0, 0, 0);
      const bf16x8_t b1 = ts_operand(qtr, 16 * j, 1, q, g);
      dk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, ds1, dk[j], 0, 0, 0);
    }
    if (e + 1 < n_q) store(buf ^ 1);
    __syncthreads();
  }
  if (!key_valid) return;

  // lane (q, g): key q, dims 16 j + 4 g .. + 3
  const float sc = p.inv_sqrt_d;
  if constexpr (kRowTable) {
    float* dkc = p.dkc + bh * p.dkc_head_stride + (int64_t)vrow * D;
    float* dvc = p.dvc + bh * p.dkc_head_stride + (int64_t)vrow * D;
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int d0 = 16 * j + 4 * g;
      *reinterpret_cast<float4*>(dkc + d0) =
          make_float4(dk[j][0] * sc, dk[j][1] * sc, dk[j][2] * sc, dk[j][3] * sc);
      *reinterpret_cast<float4*>(dvc + d0) = make_float4(dv[j][0], dv[j][1], dv[j][2], dv[j][3]);
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
    for (int j = 0; j < ND; ++j) {
      const int d0 = 16 * j + 4 * g;
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = dk[j][i] * sc;
        b[i] = dv[j][i];
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

// dQ: a wave owns 16 query rows (lane q: query q), a workgroup two 64-row
// query blocks; over the key tiles: S^T = K Q^T and dP^T = V dO^T (keys x
// queries), P^T, dS^T, dQ^T += K^T dS^T (dims x queries).
template <int D, bool kRowTable>
__global__ __launch_bounds__(kT16) void attn_bwd_dq16_kernel(BwdParams p) {
  constexpr int NKK = D / 32;
  constexpr int ND = D / 16;
  constexpr int kStage = 2 * RS<D>::kBytes + TS::bytes<D>();  // K, V row-major; K transposed
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

  const int wg_per_head = (p.n_q_entries + 1) / 2;
  bool ok;
  const int64_t lid = xcd_lid(wg_per_head, p.BH, &ok);
  if (!ok) return;
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 15, g = lane >> 4;

  const int e = qt * 2 + (wave >> 2);
  const bool wave_valid = e < p.n_q_entries;
  const int qblk = wave_valid ? p.q_tab[bh * p.q_tab_stride + e] : 0;
  const int64_t qrow = (int64_t)qblk * kBlock + (wave & 3) * 16 + q;
  const bf16_bits* Qh = p.q + bh * p.q_head_stride;
  const bf16_bits* dOh = p.dout + bh * p.q_head_stride;
  bf16x8_t qreg[NKK], oreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qreg[kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow * D + 32 * kk + 8 * g);
    oreg[kk] = *reinterpret_cast<const bf16x8_t*>(dOh + qrow * D + 32 * kk + 8 * g);
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

  // threads 0-255 stage K (both layouts), 256-511 stage V (row-major)
  const int half = tid >> 8;
  Stager16<D> st;
  st.init(tid & 255);
  const bf16_bits* src = half ? Vh : Kh;
  auto load = [&](int t) __attribute__((always_inline)) {
    if constexpr (kRowTable) {
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t {
        return tab[min(t * kBN + r, p.kv_rows - 1)];
      };
      st.load(src, row_of);
    } else {
      const int64_t r0 = (int64_t)tab[t] * kBN;
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
      st.load(src, row_of);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    st.store(b + half * RS<D>::kBytes, half ? nullptr : b + 2 * RS<D>::kBytes);
  };

  f32x4_t dq[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) dq[j][i] = 0.0f;
  const float sl2 = p.scale_log2;

  load(0);
  store(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load(t + 1);
    const unsigned char* kt = smem + buf * kStage;
    const unsigned char* vt = kt + RS<D>::kBytes;
    const unsigned char* ktr = vt + RS<D>::kBytes;

    // S^T and dP^T subtile n: keys 16 n + 4 g + i, query q
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[n][i] = 0.0f;
        dp[n][i] = 0.0f;
      }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int off = RS<D>::off(16 * n + q, (32 * kk + 8 * g) * 2);
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt + off);
        s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[kk], s[n], 0, 0, 0);
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(vt + off);
        dp[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, oreg[kk], dp[n], 0, 0, 0);
      }
    }
    // keys past the end (only a row-table tile can be partial): P = 0
    const int valid = p.kv_rows - t * kBN;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[n][i], sl2, -lse2));
        const bool live = !kRowTable || 16 * n + 4 * g + i < valid;
        dp[n][i] = live ? pr * (dp[n][i] - dlt) : 0.0f;
      }
    const bf16x8_t ds0 = pack_slots(dp[0], dp[1]), ds1 = pack_slots(dp[2], dp[3]);
    // dQ^T += K^T dS^T: dims 16 j + 4 g + i of query q
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const bf16x8_t a0 = ts_operand(ktr, 16 * j, 0, q, g);
      dq[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ds0, dq[j], 0, 0, 0);
      const bf16x8_t a1 = ts_operand(ktr, 16 * j, 1, q, g);
      dq[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ds1, dq[j], 0, 0, 0);
    }
    if (t + 1 < n_tiles) store(buf ^ 1);
    __syncthreads();
  }
  if (!wave_valid) return;
  bf16_bits* dQh = p.dq + bh * p.q_head_stride + qrow * D;
  const float sc = p.inv_sqrt_d;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    bf16x2_t a, b;
    a[0] = (__bf16)(dq[j][0] * sc);
    a[1] = (__bf16)(dq[j][1] * sc);
    b[0] = (__bf16)(dq[j][2] * sc);
    b[1] = (__bf16)(dq[j][3] * sc);
    *reinterpret_cast<uint2*>(dQh + 16 * j + 4 * g) =
        make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
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
hipError_t launch_xcd(Kern kern, int per_head, int BH, const BwdParams& p, hipStream_t s,
                      int threads = kThreads) {
  const int64_t total = (int64_t)per_head * BH;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)(((total + 7) / 8) * 8)), dim3(threads), 0, s, p);
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
      ISA_CHECK(launch_xcd(attn_bwd_dkdv16_kernel<128, true>, (n_kv + 127) / 128, BH, pt, s, kT16));
      ISA_CHECK(launch_xcd(attn_bwd_dq16_kernel<128, true>, (L.n_flat + 1) / 2, BH, pt, s, kT16));
    } else {
      ISA_CHECK(launch_xcd(attn_bwd_dkdv16_kernel<64, true>, (n_kv + 127) / 128, BH, pt, s, kT16));
      ISA_CHECK(launch_xcd(attn_bwd_dq16_kernel<64, true>, (L.n_flat + 1) / 2, BH, pt, s, kT16));
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
    ISA_CHECK(launch_xcd(attn_bwd_dkdv16_kernel<128, false>, (n_kv * kBlock + 127) / 128, BH, pe, s, kT16));
    if (L.n_sharp > 0)
      ISA_CHECK(launch_xcd(attn_bwd_dq16_kernel<128, false>, (L.n_sharp + 1) / 2, BH, pe, s, kT16));
  } else {
    ISA_CHECK(launch_xcd(attn_bwd_dkdv16_kernel<64, false>, (n_kv * kBlock + 127) / 128, BH, pe, s, kT16));
    if (L.n_sharp > 0)
      ISA_CHECK(launch_xcd(attn_bwd_dq16_kernel<64, false>, (L.n_sharp + 1) / 2, BH, pe, s, kT16));
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
