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
  // block mask inside flat rows (n_ns > 0), tables from bwd_ns_tables_kernel and
  // bwd_ns_keylists_kernel
  const uint32_t* ns_mask;  // [BH][n_flat][ns_words]: bit u set if K_new block u is exact
  int32_t ns_words;         // for flat entry f
  int32_t n_flat;
  const int32_t* tok_list;  // [BH][n_pairs][tok_cap]: flat entries 2c, 2c + 1, the union of
  const int32_t* tok_cnt;   // their exact blocks, ascending, as u * 4 + (bit j: entry 2c + j)
  int32_t tok_cap;          // 2 n_ns
  const bf16_bits* k_tok;   // token rows of the exact blocks (K, V) and the original
  const bf16_bits* v_tok;   // block of each K_new position ([BH][n_kv])
  const int32_t* kvb_tab;
  int32_t n_kv;
  int64_t tok_head_stride;  // N * D
  const int32_t* fq_off;    // [BH][n_kwg + 1] offsets into fq_list per 128-key group of
  const int32_t* fq_list;   // K_new: flat query blocks (q * 4 + bit j: key block 2 p + j)
  int64_t fq_cap;           // n_flat * n_ns entries per head
  // general blocks (partial blocks, b != 64): a 64-row tile is two 32-row
  // slices of a block list (list_slice); the entries and key rows count tiles
  BlockGrid grid;
  int32_t shift;            // log2(b / 32)
  int32_t q_slices;         // slices of the query list (its blocks << shift)
  int32_t kv_slices;        // slices of K_new (n_kv << shift)
};

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;

// A 64-row tile as two 32-row slices (start, valid rows); rows past a
// slice's count read its last valid row (or its start when it is empty, which
// list_slice keeps inside the head) and count as invalid.
struct TileRows {
  int32_t s0, c0, s1, c1;
  __device__ __forceinline__ int64_t row(int r) const {
    const int i = r & 31, c = r < 32 ? c0 : c1;
    return (int64_t)(r < 32 ? s0 : s1) + (i < c ? i : (c > 0 ? c - 1 : 0));
  }
  __device__ __forceinline__ bool valid(int r) const { return (r & 31) < (r < 32 ? c0 : c1); }
};
__device__ __forceinline__ TileRows tile_rows(const BlockGrid& g, const int32_t* list,
                                              int n_slices, int shift, int tile) {
  const Slice a = list_slice(g, list, n_slices, shift, 2 * tile);
  const Slice b = list_slice(g, list, n_slices, shift, 2 * tile + 1);
  return TileRows{a.start, a.cnt, b.start, b.cnt};
}
// the one tile of block blk at b = 64
__device__ __forceinline__ TileRows block_tile64(const BlockGrid& g, int blk) {
  return tile_rows(g, nullptr, 0x7fffffff, 1, blk);
}
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
constexpr int kPipe = 2;  // LDS operand reads run this many product steps ahead
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

// A scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Runs NS steps whose operands come from LDS: step s reads its operands
// (rd(s)) P steps before its products run (mm(s)), into a ring of P + 1
// register slots the callers index with s % (P + 1).  Fenced, so the
// compiler neither sinks the reads next to their use (one LDS latency per
// product, the order it picks under register pressure) nor hoists them all.
template <int NS, int P, typename Rd, typename Mm>
__device__ __forceinline__ void pipelined(Rd rd, Mm mm) {
#pragma unroll
  for (int st = 0; st < P; ++st) rd(st);
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if (st + P < NS) rd(st + P);
    fence();
    mm(st);
    fence();
  }
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
// kMask (block mask inside flat rows): in block-table mode the query blocks
// are the sharp ones followed by this group's list of flat blocks that take
// its keys token by token, each with a bit per 64-key half (a half whose bit
// is clear skips the block: its P is 0); in row-table mode a flat block's
// exact blocks are masked out of its pooled keys (P = 0).
// kGen (partial blocks, b != 64): query entries and block-table keys are
// 64-row tiles of two 32-row slices; rows past a slice's count are invalid
// (a query row gets P = 0 through an infinite LSE, a key is not written), and
// a pooled key's weight w_j enters as log2(w_j / b) in its exponent.
template <int D, bool kRowTable, bool kMask = false, bool kGen = false>
__global__ __launch_bounds__(kT16) void attn_bwd_dkdv16_kernel(BwdParams p) {
  constexpr int NKK = D / 32;
  constexpr int ND = D / 16;
  // Q, dO row-major; Q, dO transposed; lse2[64], delta[64]; (mask: 4 flag words)
  constexpr int kFlags = 2 * RS<D>::kBytes + 2 * TS::bytes<D>() + 2 * kBN * 4;
  constexpr int kStage = kFlags + (kMask ? 16 : 0);
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
  bool key_valid = vrow < p.kv_rows;
  const int32_t* tab = p.kv_tab + bh * p.kv_tab_stride;
  const int vr = min(vrow, p.kv_rows - 1);
  int64_t krow;
  float wbias = 0.0f;  // kGen, row-table: log2(w_j / b) of this pooled key
  if constexpr (kRowTable) {
    krow = tab[vr];
    if constexpr (kGen)
      wbias = log2f((float)p.grid.rows(p.kvb_tab[bh * p.n_kv + vr]) / (float)p.grid.len);
  } else if constexpr (kGen) {
    const TileRows tr = tile_rows(p.grid, tab, p.kv_slices, p.shift, vr >> 6);
    krow = tr.row(vr & 63);
    key_valid = key_valid && tr.valid(vr & 63);
  } else {
    krow = (int64_t)tab[vr >> 6] * kBN + (vr & 63);
  }
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
  int n_q = p.n_q_entries;
  const int32_t* fql = nullptr;
  if constexpr (kMask && !kRowTable) {
    const int32_t* off = p.fq_off + bh * (kv_wgs + 1) + kt;
    fql = p.fq_list + bh * p.fq_cap + off[0];
    n_q += off[1] - off[0];
  }
  const uint32_t* nsm = nullptr;
  if constexpr (kMask && kRowTable) nsm = p.ns_mask + bh * p.n_flat * p.ns_words;
  // threads 0-255 stage Q, 256-511 stage dO (both layouts).  Two register
  // stages alternate, so a query block's loads are issued two iterations
  // before its LDS copy is written (the LDS holds two blocks: no room for a
  // third).
  const int half = tid >> 8;
  struct Stage {
    Stager16<D> st;
    float lse;       // thread tid < 64: lse of query row tid; 64..127: delta (as loaded)
    uint32_t fl[4];  // mask (uniform): the block's half bits, or the four words of
                     // the pooled-key mask that cover this group's 128 keys
    bool qv;         // kGen: query row tid & 63 is inside its slice
  };
  Stage sa, sb;
  sa.st.init(tid & 255);
  sb.st.init(tid & 255);
  sa.lse = sb.lse = 0.0f;
  sa.qv = sb.qv = true;
  auto load = [&](Stage& x, int e) __attribute__((always_inline)) {
    if constexpr (kMask && kRowTable) {  // words 4 kt .. 4 kt + 3
      const uint32_t* row = nsm + (int64_t)e * p.ns_words;
#pragma unroll
      for (int j = 0; j < 4; ++j) x.fl[j] = row[min(kt * 4 + j, p.ns_words - 1)];
    }
    if constexpr (kGen) {
      TileRows tr;
      if constexpr (kMask && !kRowTable) {
        if (e < p.n_q_entries) {
          tr = tile_rows(p.grid, qtab, p.q_slices, p.shift, e);
          x.fl[0] = 3u;
        } else {
          const int ent = fql[e - p.n_q_entries];
          tr = block_tile64(p.grid, ent >> 2);
          x.fl[0] = (uint32_t)(ent & 3);
        }
      } else {
        tr = tile_rows(p.grid, qtab, p.q_slices, p.shift, e);
      }
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return tr.row(r); };
      x.st.load(half ? dOh : Qh, row_of);
      x.lse = (tid & kBN ? dlth : lseh)[tr.row(tid & (kBN - 1))];
      x.qv = tr.valid(tid & (kBN - 1));
      return;
    }
    int64_t r0;
    if constexpr (kMask && !kRowTable) {
      const int ent = e < p.n_q_entries ? qtab[e] * 4 + 3 : fql[e - p.n_q_entries];
      r0 = (int64_t)(ent >> 2) * kBlock;
      x.fl[0] = (uint32_t)(ent & 3);
    } else {
      r0 = (int64_t)qtab[e] * kBlock;
    }
    auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
    x.st.load(half ? dOh : Qh, row_of);
    // Every thread issues one more load (threads past 127 discard theirs), and
    // the value is converted only when stored: the same loads in every
    // iteration, with no arithmetic on them here, let the wait before each
    // store count exactly the newer stage's loads as still in flight.
    x.lse = (tid & kBN ? dlth : lseh)[r0 + (tid & (kBN - 1))];
  };
  auto store = [&](Stage& x, int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    x.st.store(b + half * RS<D>::kBytes, b + 2 * RS<D>::kBytes + half * TS::bytes<D>());
    if (tid < 2 * kBN) {
      float l = tid < kBN ? (x.lse - p.lse_offset) * 1.4426950408889634f : x.lse;
      if constexpr (kGen)  // a row outside its slice: P = 2^-inf = 0
        if (tid < kBN && !x.qv) l = INFINITY;
      reinterpret_cast<float*>(b + 2 * RS<D>::kBytes + 2 * TS::bytes<D>())[tid] = l;
    }
    if constexpr (kMask)
      if (tid < 4)
        reinterpret_cast<uint32_t*>(b + kFlags)[tid] =
            tid == 0 ? x.fl[0] : tid == 1 ? x.fl[1] : tid == 2 ? x.fl[2] : x.fl[3];
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
  if (n_q > 0) {
    load(sa, 0);
    store(sa, 0);
    load(sa, min(1, n_q - 1));
    load(sb, min(2, n_q - 1));
  }
  __syncthreads();
  // iteration e computes with query block e (LDS buffer e & 1), then writes
  // block e + 1 from stage x into the other buffer and reloads x with e + 3
  auto iteration = [&](int e, Stage& x) __attribute__((always_inline)) {
    const int buf = e & 1;
    const unsigned char* qt = smem + buf * kStage;
    const unsigned char* ot = qt + RS<D>::kBytes;
    const unsigned char* qtr = ot + RS<D>::kBytes;
    const unsigned char* otr = qtr + TS::bytes<D>();
    const float* lse_s = reinterpret_cast<const float*>(otr + TS::bytes<D>());
    const float* dlt_s = lse_s + kBN;
    // mask: a half of the group not in this block's list skips it; a pooled
    // key that is exact for this flat block has P = 2^-inf = 0 (and dS = 0)
    bool active = true;
    float bias = wbias;
    if constexpr (kMask && !kRowTable)
      active = (__builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(qt + kFlags)) >>
                (wave >> 2)) & 1;
    if constexpr (kMask && kRowTable)
      bias = ((*reinterpret_cast<const uint32_t*>(qt + kFlags + 4 * (wave >> 1)) >>
               ((wave & 1) * 16 + q)) & 1) ? -INFINITY : wbias;
    if (active) {
      // S and dP subtile n: queries 16 n + 4 g + i, key q
      f32x4_t s[4], dp[4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[n][i] = 0.0f;
          dp[n][i] = 0.0f;
        }
      // step st = 4 kk + n: the Q and dO operands of subtile n, chunk kk
      constexpr int P = kPipe;
      bf16x8_t ra[P + 1], rb[P + 1];
      pipelined<4 * NKK, P>(
          [&](int st) __attribute__((always_inline)) {
            const int off = RS<D>::off(16 * (st & 3) + q, (32 * (st >> 2) + 8 * g) * 2);
            ra[st % (P + 1)] = *reinterpret_cast<const bf16x8_t*>(qt + off);
            rb[st % (P + 1)] = *reinterpret_cast<const bf16x8_t*>(ot + off);
          },
          [&](int st) __attribute__((always_inline)) {
            const int n = st & 3, kk = st >> 2;
            s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[st % (P + 1)], kreg[kk], s[n], 0,
                                                            0, 0);
            dp[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[st % (P + 1)], vreg[kk], dp[n],
                                                             0, 0, 0);
          });
      // step st = 2 j + c of the dV, dK products: the dO^T and Q^T operands of
      // dims 16 j .. + 15, query chunk c; the first reads overlap the softmax
      auto rd_t = [&](int st) __attribute__((always_inline)) {
        ra[st % (P + 1)] = ts_operand(otr, 16 * (st >> 1), st & 1, q, g);
        rb[st % (P + 1)] = ts_operand(qtr, 16 * (st >> 1), st & 1, q, g);
      };
#pragma unroll
      for (int st = 0; st < P; ++st) rd_t(st);
      // P and dS; the query chunk c of the B operands takes subtiles 2c, 2c + 1
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + 16 * n + 4 * g);
        const float4 d4 = *reinterpret_cast<const float4*>(dlt_s + 16 * n + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = fmaf(s[n][i], sl2, -lv[i]);
          if constexpr ((kMask || kGen) && kRowTable) x += bias;
          const float pr = __builtin_amdgcn_exp2f(x);
          s[n][i] = pr;
          dp[n][i] = pr * (dp[n][i] - dv4[i]);
        }
      }
      const bf16x8_t pk[2] = {pack_slots(s[0], s[1]), pack_slots(s[2], s[3])};
      const bf16x8_t ds[2] = {pack_slots(dp[0], dp[1]), pack_slots(dp[2], dp[3])};
      // dV^T += dO^T P, dK^T += Q^T dS: dims 16 j + 4 g + i of key q
#pragma unroll
      for (int st = 0; st < 2 * ND; ++st) {
        if (st + P < 2 * ND) rd_t(st + P);
        fence();
        const int j = st >> 1, c = st & 1;
        dv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[st % (P + 1)], pk[c], dv[j], 0, 0, 0);
        dk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[st % (P + 1)], ds[c], dk[j], 0, 0, 0);
        fence();
      }
    }
    if (e + 1 < n_q) store(x, buf ^ 1);
    load(x, min(e + 3, n_q - 1));  // (past the end: a block loaded again, unused)
    __syncthreads();
  };
  int e = 0;
  for (; e + 1 < n_q; e += 2) {
    iteration(e, sa);
    iteration(e + 1, sb);
  }
  if (e < n_q) iteration(e, sa);
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
    int blk = vrow >> 6;  // K_new position of the key's block
    float iw = p.inv_w;
    if constexpr (kGen) {
      blk = (2 * (vrow >> 6) + ((vrow & 63) >> 5)) >> p.shift;
      iw = 1.0f / (float)p.grid.rows(tab[blk]);
    }
    const float* tk = p.dkc_in ? p.dkc_in + bh * p.dkc_head_stride + (int64_t)blk * D : nullptr;
    const float* tv = p.dvc_in ? p.dvc_in + bh * p.dkc_head_stride + (int64_t)blk * D : nullptr;
    bf16_bits* dKh = p.dk + bh * p.q_head_stride + krow * D;
    bf16_bits* dVh = p.dv + bh * p.q_head_stride + krow * D;
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
// kMask (flat rows under the block mask, row-table mode): a flat block's
// exact blocks are masked out of the pooled key tiles (P = 0), and after
// them come the token tiles of the union of the two blocks' exact blocks,
// each with a bit per block (a block whose bit is clear skips the tile).
// Token terms have weight 1, so their P uses the LSE without the ln w offset.
// kGen (partial blocks, b != 64): query entries and block-table key tiles are
// 64-row tiles of two 32-row slices; a query row outside its slice is not
// written, a key outside its slice has P = 0, and a pooled key's weight w_j
// enters as log2(w_j / b) in its exponent.
template <int D, bool kRowTable, bool kMask = false, bool kGen = false>
__global__ __launch_bounds__(kT16) void attn_bwd_dq16_kernel(BwdParams p) {
  static_assert(!kMask || kRowTable, "the mask applies to the flat rows' pooled keys");
  constexpr int NKK = D / 32;
  constexpr int ND = D / 16;
  // K, V row-major; K transposed; (mask or general blocks: the tile's flag word)
  constexpr bool kFlagWord = kMask || (kGen && !kRowTable);
  constexpr int kFlags = 2 * RS<D>::kBytes + TS::bytes<D>();
  constexpr int kStage = kFlags + (kFlagWord ? 16 : 0);
  constexpr int kMaxWords = kMaxBlocksPerHead / 32;
  constexpr bool kWeights = kGen && kRowTable;  // per pooled key log2(w_j / b)
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];
  __shared__ uint32_t nsm_s[kMask ? 2 * kMaxWords : 1];  // the two blocks' mask rows
  __shared__ __attribute__((aligned(16))) float lw_s[kWeights ? kMaxBlocksPerHead + kBN : 1];

  const int wg_per_head = (p.n_q_entries + 1) / 2;
  bool ok;
  const int64_t lid = xcd_lid(wg_per_head, p.BH, &ok);
  if (!ok) return;
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 15, g = lane >> 4;
  const int e = qt * 2 + (wave >> 2);
  bool wave_valid = e < p.n_q_entries;
  int64_t qrow;
  if constexpr (kGen) {  // entry e: tile e of the query list
    const TileRows tr = tile_rows(p.grid, p.q_tab + bh * p.q_tab_stride, p.q_slices, p.shift, e);
    qrow = tr.row((wave & 3) * 16 + q);
    wave_valid = wave_valid && tr.valid((wave & 3) * 16 + q);  // (per lane)
  } else {
    const int qblk = wave_valid ? p.q_tab[bh * p.q_tab_stride + e] : 0;
    qrow = (int64_t)qblk * kBlock + (wave & 3) * 16 + q;
  }
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
  const float lse_raw = p.lse[bh * p.lse_head_stride + qrow];
  const float lse2 = (lse_raw - p.lse_offset) * 1.4426950408889634f;
  const float lse2_tok = lse_raw * 1.4426950408889634f;  // token tiles (mask)
  const float dlt = p.delta[bh * p.lse_head_stride + qrow];

  const bf16_bits* Kh = p.k + bh * p.kv_head_stride;
  const bf16_bits* Vh = p.v + bh * p.kv_head_stride;
  const int32_t* tab = p.kv_tab + bh * p.kv_tab_stride;
  const int n_rep = (p.kv_rows + kBN - 1) / kBN;  // tiles of the key source
  int n_tiles = n_rep;
  const int32_t* tl = nullptr;
  const int32_t* kvb = nullptr;
  const bf16_bits *Kt = nullptr, *Vt = nullptr;
  if constexpr (kMask) {
    const int64_t pair = bh * wg_per_head + qt;
    tl = p.tok_list + pair * p.tok_cap;
    n_tiles += p.tok_cnt[pair];
    kvb = p.kvb_tab + bh * p.n_kv;
    Kt = p.k_tok + bh * p.tok_head_stride;
    Vt = p.v_tok + bh * p.tok_head_stride;
    for (int i = tid; i < 2 * p.ns_words; i += kT16) {
      const int j = i / p.ns_words, w = i - j * p.ns_words, f = qt * 2 + j;
      nsm_s[j * kMaxWords + w] =
          f < p.n_q_entries ? p.ns_mask[(bh * p.n_flat + f) * p.ns_words + w] : 0u;
    }
  }
  if constexpr (kWeights) {
    const int32_t* kvb_h = p.kvb_tab + bh * p.n_kv;
    const float inv_len = 1.0f / (float)p.grid.len;
    for (int u = tid; u < n_rep * kBN; u += kT16)
      lw_s[u] = u < p.n_kv ? log2f((float)p.grid.rows(kvb_h[u]) * inv_len) : 0.0f;
  }

  // threads 0-255 stage K (both layouts), 256-511 stage V (row-major).  Two
  // register stages alternate, so a key tile's loads are issued two
  // iterations before its LDS copy is written.
  const int half = tid >> 8;
  struct Stage {
    Stager16<D> st;
    uint32_t fl;  // bits 0-1: a token tile's block bits (mask); 8-15, 16-23: the
                  // valid rows of the tile's two slices (general blocks)
  };
  Stage sa, sb;
  sa.st.init(tid & 255);
  sb.st.init(tid & 255);
  sa.fl = sb.fl = 0u;
  const bf16_bits* src = half ? Vh : Kh;
  auto load = [&](Stage& x, int t) __attribute__((always_inline)) {
    if constexpr (kMask) {
      if (t >= n_rep) {  // token tile of K_new block ent >> 2
        const int ent = tl[t - n_rep];
        if constexpr (kGen) {
          const TileRows tr = block_tile64(p.grid, kvb[ent >> 2]);
          x.fl = (uint32_t)(ent & 3) | ((uint32_t)tr.c0 << 8) | ((uint32_t)tr.c1 << 16);
          auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return tr.row(r); };
          x.st.load(half ? Vt : Kt, row_of);
        } else {
          const int64_t r0 = (int64_t)kvb[ent >> 2] * kBlock;
          x.fl = (uint32_t)(ent & 3);
          auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
          x.st.load(half ? Vt : Kt, row_of);
        }
        return;
      }
    }
    if constexpr (kGen && !kRowTable) {  // tile t of K_new
      const TileRows tr = tile_rows(p.grid, tab, p.kv_slices, p.shift, t);
      x.fl = ((uint32_t)tr.c0 << 8) | ((uint32_t)tr.c1 << 16);
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return tr.row(r); };
      x.st.load(src, row_of);
      return;
    }
    if constexpr (kRowTable) {
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t {
        return tab[min(t * kBN + r, p.kv_rows - 1)];
      };
      x.st.load(src, row_of);
    } else {
      const int64_t r0 = (int64_t)tab[t] * kBN;
      auto row_of = [&](int r) __attribute__((always_inline)) -> int64_t { return r0 + r; };
      x.st.load(src, row_of);
    }
  };
  auto store = [&](Stage& x, int buf) __attribute__((always_inline)) {
    unsigned char* b = smem + buf * kStage;
    x.st.store(b + half * RS<D>::kBytes, half ? nullptr : b + 2 * RS<D>::kBytes);
    if constexpr (kFlagWord)
      if (tid == 0) *reinterpret_cast<uint32_t*>(b + kFlags) = x.fl;
  };

  f32x4_t dq[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) dq[j][i] = 0.0f;
  const float sl2 = p.scale_log2;

  load(sa, 0);
  store(sa, 0);
  // the same loads in every iteration (a tile past the end is the last one
  // loaded again, unused), so the wait before each store counts exactly the
  // newer stage's loads as still in flight
  load(sa, min(1, n_tiles - 1));
  load(sb, min(2, n_tiles - 1));
  __syncthreads();
  // iteration t computes with key tile t (LDS buffer t & 1), then writes tile
  // t + 1 from stage x into the other buffer and reloads x with tile t + 3
  auto iteration = [&](int t, Stage& x) __attribute__((always_inline)) {
    const int buf = t & 1;
    const unsigned char* kt = smem + buf * kStage;
    const unsigned char* vt = kt + RS<D>::kBytes;
    const unsigned char* ktr = vt + RS<D>::kBytes;
    // mask: a token tile not among this block's exact blocks is skipped; a
    // pooled key that is one of them has P = 0
    bool active = true, tok = false;
    uint64_t km = 0;
    uint32_t fw = 0;  // the tile's flag word
    if constexpr (kFlagWord)
      fw = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(kt + kFlags));
    if constexpr (kMask) {
      tok = t >= n_rep;
      if (tok) {
        active = (fw >> (wave >> 2)) & 1;
      } else {
        const uint32_t* m = nsm_s + (wave >> 2) * kMaxWords;
        km = (uint64_t)m[min(2 * t, p.ns_words - 1)] |
             ((uint64_t)m[min(2 * t + 1, p.ns_words - 1)] << 32);
      }
    }
    if (active) {
      // S^T and dP^T subtile n: keys 16 n + 4 g + i, query q
      f32x4_t s[4], dp[4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[n][i] = 0.0f;
          dp[n][i] = 0.0f;
        }
      // step st = 4 kk + n: the K and V operands of subtile n, chunk kk
      constexpr int P = kPipe;
      bf16x8_t ra[P + 1], rb[P + 1];
      pipelined<4 * NKK, P>(
          [&](int st) __attribute__((always_inline)) {
            const int off = RS<D>::off(16 * (st & 3) + q, (32 * (st >> 2) + 8 * g) * 2);
            ra[st % (P + 1)] = *reinterpret_cast<const bf16x8_t*>(kt + off);
            rb[st % (P + 1)] = *reinterpret_cast<const bf16x8_t*>(vt + off);
          },
          [&](int st) __attribute__((always_inline)) {
            const int n = st & 3, kk = st >> 2;
            s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[st % (P + 1)], qreg[kk], s[n], 0,
                                                            0, 0);
            dp[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb[st % (P + 1)], oreg[kk], dp[n],
                                                             0, 0, 0);
          });
      // step st = 2 j + c of the dQ products (K^T operand of dims 16 j .. + 15,
      // key chunk c), read 2 P steps ahead; the first reads overlap the softmax
      constexpr int P2 = 2 * kPipe;
      bf16x8_t rt[P2 + 1];
      auto rd_t = [&](int st) __attribute__((always_inline)) {
        rt[st % (P2 + 1)] = ts_operand(ktr, 16 * (st >> 1), st & 1, q, g);
      };
#pragma unroll
      for (int st = 0; st < P2; ++st) rd_t(st);
      // keys past the end (only a row-table tile can be partial, or, with
      // general blocks, any tile past its slices' counts): P = 0
      const int valid = tok ? kBN : p.kv_rows - t * kBN;
      const float l2 = tok ? lse2_tok : lse2;
      const bool by_slices = kGen && (!kRowTable || tok);
      const int c0 = (fw >> 8) & 0xff, c1 = (fw >> 16) & 0xff;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float4 wb = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if constexpr (kWeights)
          if (!tok) wb = *reinterpret_cast<const float4*>(lw_s + t * kBN + 16 * n + 4 * g);
        const float wbi[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * n + 4 * g + i;
          float x = fmaf(s[n][i], sl2, -l2);
          if constexpr (kWeights) x += wbi[i];
          const float pr = __builtin_amdgcn_exp2f(x);
          bool live;
          if constexpr (kGen)
            live = by_slices ? (key < 32 ? key < c0 : key - 32 < c1) : key < valid;
          else
            live = !kRowTable || key < valid;
          live = live && !((km >> key) & 1);
          dp[n][i] = live ? pr * (dp[n][i] - dlt) : 0.0f;
        }
      }
      const bf16x8_t ds[2] = {pack_slots(dp[0], dp[1]), pack_slots(dp[2], dp[3])};
      // dQ^T += K^T dS^T: dims 16 j + 4 g + i of query q
#pragma unroll
      for (int st = 0; st < 2 * ND; ++st) {
        if (st + P2 < 2 * ND) rd_t(st + P2);
        fence();
        dq[st >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rt[st % (P2 + 1)], ds[st & 1],
                                                              dq[st >> 1], 0, 0, 0);
        fence();
      }
    }
    if (t + 1 < n_tiles) store(x, buf ^ 1);
    load(x, min(t + 3, n_tiles - 1));
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    iteration(t, sa);
    iteration(t + 1, sb);
  }
  if (t < n_tiles) iteration(t, sa);
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

// delta_r = dO_r . O_r over D, fp32: D / 8 consecutive lanes per row, each
// with one 16-byte load of O and of dO (a wave reads whole rows, so every load
// instruction covers contiguous memory); the lanes' partial sums are combined
// by a butterfly in a fixed order.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16_bits* __restrict__ O,
                                                             const bf16_bits* __restrict__ dO,
                                                             int64_t rows,
                                                             float* __restrict__ delta) {
  constexpr int kLanes = D / 8;  // 16 or 8 lanes per row
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t r = i / kLanes;
  float acc = 0.0f;
  if (r < rows) {
    const uint4 a = load_nt(reinterpret_cast<const uint4*>(O) + i);
    const uint4 b = load_nt(reinterpret_cast<const uint4*>(dO) + i);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(wa[k] << 16), __uint_as_float(wb[k] << 16), acc);
      acc = fmaf(__uint_as_float(wa[k] & 0xffff0000u), __uint_as_float(wb[k] & 0xffff0000u), acc);
    }
  }
  // (every lane of the wave takes part: rows never straddle a wave)
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (r < rows && (threadIdx.x & (kLanes - 1)) == 0) delta[r] = acc;
}

// Per (kept block t, head): block table entry and the bf16 means of the block's
// K and V rows (fp64 sums divided by the block's length, rounded as the
// forward's pooling rounds them).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    const bf16_bits* __restrict__ K, const bf16_bits* __restrict__ V,
    const int32_t* __restrict__ sel, BlockGrid grid, int k, int32_t* __restrict__ kv_tab,
    int32_t* __restrict__ iota, bf16_bits* __restrict__ kc, bf16_bits* __restrict__ vc) {
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int n_src = grid.n_src, n_kv = n_src + k;
  const int blk = t < n_src ? t : n_src + sel[bh * k + (t - n_src)];
  if (threadIdx.x == 0) {
    kv_tab[bh * n_kv + t] = blk;
    if (bh == 0) iota[t] = t;  // identity row table of the compact pooled rows
  }
  // D / 8 lanes per row, each summing one 16-byte chunk (8 dims) of every
  // G-th row; the G row groups are then added in a fixed order.  (A sum of at
  // most 128 bf16 values, 8 significant bits each, is exact in fp64 unless
  // they span more than 2^38 in magnitude, so the order does not change it.)
  constexpr int C = D / 8;         // 16-byte chunks per row
  constexpr int G = kThreads / C;  // row groups
  __shared__ double red[2][G][D];
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int g = tid / C;
  const int rows = grid.rows(blk);
  const bf16_bits* kb = K + (bh * grid.N + grid.start(blk)) * D + 8 * c;
  const bf16_bits* vb = V + (bh * grid.N + grid.start(blk)) * D + 8 * c;
  double sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.0;
  for (int r = g; r < rows; r += G) {
    const uint4 a = load_nt(kb + (int64_t)r * D), b = load_nt(vb + (int64_t)r * D);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sk[2 * w] += (double)__uint_as_float(wa[w] << 16);
      sk[2 * w + 1] += (double)__uint_as_float(wa[w] & 0xffff0000u);
      sv[2 * w] += (double)__uint_as_float(wb[w] << 16);
      sv[2 * w + 1] += (double)__uint_as_float(wb[w] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][g][8 * c + e] = sk[e];
    red[1][g][8 * c + e] = sv[e];
  }
  __syncthreads();
  if (tid < D) {
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      a += red[0][i][tid];
      b += red[1][i][tid];
    }
    const int64_t o = (bh * n_kv + t) * (int64_t)D + tid;
    kc[o] = (bf16_bits)bf16_bits_rne(a / (double)rows);  // as the forward's pooling rounds
    vc[o] = (bf16_bits)bf16_bits_rne(b / (double)rows);
  }
}

// dK, dV rows of context blocks that were not kept are zero.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_zero_unselected_kernel(
    const int32_t* __restrict__ sel, BlockGrid grid, int k, bf16_bits* __restrict__ dK,
    bf16_bits* __restrict__ dV) {
  const int j = blockIdx.x;  // context block
  const int64_t bh = blockIdx.y;
  for (int i = 0; i < k; ++i)
    if (sel[bh * k + i] == j) return;  // kept: written by the exact kernel
  const int blk = grid.n_src + j;
  uint4* a = reinterpret_cast<uint4*>(dK + (bh * grid.N + grid.start(blk)) * D);
  uint4* b = reinterpret_cast<uint4*>(dV + (bh * grid.N + grid.start(blk)) * D);
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int i = threadIdx.x; i < grid.rows(blk) * D / 8; i += kThreads) {
    a[i] = z;
    b[i] = z;
  }
}

// Block-mask tables of the backward, per (pair c of flat entries, head): the
// mask rows of entries 2c and 2c + 1 (bit u: K_new block u is exact for the
// entry) and the ascending union of their exact blocks as u * 4 + bits (bit j:
// exact for entry 2c + j).  Positions outside [0, n_kv) are ignored.
__global__ __launch_bounds__(kThreads) void bwd_ns_tables_kernel(
    const int32_t* __restrict__ ns, int n_flat, int n_ns, int n_kv, int words,
    uint32_t* __restrict__ mask, int32_t* __restrict__ tok_list, int32_t* __restrict__ tok_cnt) {
  constexpr int kMaxWords = kMaxBlocksPerHead / 32;
  __shared__ uint32_t m[2][kMaxWords];
  __shared__ int pre[kMaxWords + 1];
  const int c = blockIdx.x, n_pairs = gridDim.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kMaxWords; i += kThreads) m[i / kMaxWords][i % kMaxWords] = 0u;
  __syncthreads();
  for (int i = tid; i < 2 * n_ns; i += kThreads) {
    const int j = i / n_ns, f = 2 * c + j;
    if (f < n_flat) {
      const int u = ns[(bh * n_flat + f) * n_ns + (i - j * n_ns)];
      if ((unsigned)u < (unsigned)n_kv) atomicOr(&m[j][u >> 5], 1u << (u & 31));
    }
  }
  __syncthreads();
  for (int i = tid; i < 2 * words; i += kThreads) {
    const int j = i / words, w = i - j * words, f = 2 * c + j;
    if (f < n_flat) mask[(bh * n_flat + f) * words + w] = m[j][w];
  }
  if (tid < words) pre[tid + 1] = __popc(m[0][tid] | m[1][tid]);
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  if (tid == 0)
    for (int w = 1; w <= words; ++w) pre[w] += pre[w - 1];
  __syncthreads();
  const int64_t pair = bh * n_pairs + c;
  if (tid < words) {
    const uint32_t a = m[0][tid], b = m[1][tid];
    uint32_t bits = a | b;
    int32_t* out = tok_list + pair * (2 * (int64_t)n_ns);
    int pos = pre[tid];
    while (bits) {
      const int k = __ffs(bits) - 1;
      out[pos++] = (tid * 32 + k) * 4 + (int)((a >> k) & 1u) + 2 * (int)((b >> k) & 1u);
      bits &= bits - 1;
    }
  }
  if (tid == 0) tok_cnt[pair] = pre[words];
}

// Per head: for every group p of 128 keys of K_new (blocks 2p and 2p + 1), the
// flat entries whose mask row has either block, ascending, as flat[f] * 4 +
// bits (bit j: block 2p + j), in CSR form (off[p] .. off[p + 1]).  One thread
// per group scans the mask rows twice (count, then fill): deterministic.
constexpr int kListThreads = 1024;
__global__ __launch_bounds__(kListThreads) void bwd_ns_keylists_kernel(
    const uint32_t* __restrict__ mask, const int32_t* __restrict__ flat, int n_flat, int words,
    int n_kwg, int64_t cap, int32_t* __restrict__ off, int32_t* __restrict__ list) {
  __shared__ int cnt[kMaxBlocksPerHead / 2 + 1];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t* mh = mask + bh * n_flat * words;
  for (int p = tid; p < n_kwg; p += kListThreads) {
    const int w = p >> 4, sh = (2 * p) & 31;
    int c = 0;
    for (int f = 0; f < n_flat; ++f) c += ((mh[(int64_t)f * words + w] >> sh) & 3u) != 0u;
    cnt[p + 1] = c;
  }
  if (tid == 0) cnt[0] = 0;
  __syncthreads();
  if (tid == 0)
    for (int p = 1; p <= n_kwg; ++p) cnt[p] += cnt[p - 1];
  __syncthreads();
  int32_t* oh = off + bh * (n_kwg + 1);
  int32_t* lh = list + bh * cap;
  const int32_t* fh = flat + bh * n_flat;
  for (int p = tid; p <= n_kwg; p += kListThreads) oh[p] = cnt[p];
  for (int p = tid; p < n_kwg; p += kListThreads) {
    const int w = p >> 4, sh = (2 * p) & 31;
    int pos = cnt[p];
    for (int f = 0; f < n_flat; ++f) {
      const uint32_t b = (mh[(int64_t)f * words + w] >> sh) & 3u;
      if (b) lh[pos++] = fh[f] * 4 + (int)b;
    }
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

// The attention kernels of one head dimension: Taylor dK^c/dV^c and flat-row
// dQ, then exact dK/dV and sharp-row dQ, each in the variant the plan needs.
template <int D, bool kGen>
hipError_t launch_paths(const BwdParams& pt, const BwdParams& pe, bool masked, int n_flat_tiles,
                        int n_sharp_tiles, int n_kv, int key_tiles, int BH, hipStream_t s) {
  hipError_t e;
  if (n_flat_tiles > 0) {
    const int kg = (n_kv + 127) / 128, qg = (n_flat_tiles + 1) / 2;
    e = masked ? launch_xcd(attn_bwd_dkdv16_kernel<D, true, true, kGen>, kg, BH, pt, s, kT16)
               : launch_xcd(attn_bwd_dkdv16_kernel<D, true, false, kGen>, kg, BH, pt, s, kT16);
    if (e != hipSuccess) return e;
    e = masked ? launch_xcd(attn_bwd_dq16_kernel<D, true, true, kGen>, qg, BH, pt, s, kT16)
               : launch_xcd(attn_bwd_dq16_kernel<D, true, false, kGen>, qg, BH, pt, s, kT16);
    if (e != hipSuccess) return e;
  }
  const int eg = (key_tiles * kBN + 127) / 128, sg = (n_sharp_tiles + 1) / 2;
  e = masked ? launch_xcd(attn_bwd_dkdv16_kernel<D, false, true, kGen>, eg, BH, pe, s, kT16)
             : launch_xcd(attn_bwd_dkdv16_kernel<D, false, false, kGen>, eg, BH, pe, s, kT16);
  if (e != hipSuccess) return e;
  if (n_sharp_tiles > 0)
    return launch_xcd(attn_bwd_dq16_kernel<D, false, false, kGen>, sg, BH, pe, s, kT16);
  return hipSuccess;
}

// Backward launch sequence (see the top of this file).
hipError_t launch_backward(const BwdLaunch& L, hipStream_t s) {
  const int BH = L.BH, D = L.D;
  const int64_t rows = (int64_t)BH * L.N;
  hipError_t e;
#define ISA_CHECK(x) \
  if ((e = (x)) != hipSuccess) return e;
  if (rows > 0) {
    const int64_t threads = rows * (D / 8);
    const dim3 dgrid((unsigned)((threads + kThreads - 1) / kThreads));
    if (D == 128)
      hipLaunchKernelGGL(bwd_delta_kernel<128>, dgrid, dim3(kThreads), 0, s, L.O, L.dO, rows,
                         L.delta);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<64>, dgrid, dim3(kThreads), 0, s, L.O, L.dO, rows,
                         L.delta);
    ISA_CHECK(hipGetLastError());
  }
  BlockGrid grid;
  grid.L_src = L.L_src;
  grid.n_src = L.n_src;
  grid.N = L.N;
  grid.len = L.block;
  const int n_kv = L.n_src + L.k;
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(n_kv, BH), dim3(kThreads), 0, s, L.K, L.V,
                       L.sel, grid, L.k, L.kv_tab, L.iota, L.kc, L.vc);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(n_kv, BH), dim3(kThreads), 0, s, L.K, L.V, L.sel,
                       grid, L.k, L.kv_tab, L.iota, L.kc, L.vc);
  ISA_CHECK(hipGetLastError());

  // General blocks (a partial block, or b != 64): 64-row tiles of 32-row
  // slices; otherwise a tile is a block.
  const bool gen = L.block != kBlock || (L.L_src % kBlock) != 0 || ((L.N - L.L_src) % kBlock) != 0;
  const int shift = L.block == 32 ? 0 : L.block == 64 ? 1 : 2;
  auto tiles = [&](int n_blocks) { return ((n_blocks << shift) + 1) / 2; };
  const int key_tiles = gen ? tiles(n_kv) : n_kv;
  const int flat_tiles = gen ? tiles(L.n_flat) : L.n_flat;
  const int sharp_tiles = gen ? tiles(L.n_sharp) : L.n_sharp;

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
  p.grid = grid;
  p.shift = shift;
  p.kv_slices = n_kv << shift;
  p.kvb_tab = L.kv_tab;
  p.n_kv = n_kv;

  // block mask inside flat rows: tables of the exact blocks per flat block
  const bool masked = L.n_ns > 0 && L.n_flat > 0;
  const int words = (n_kv + 31) / 32;
  const int n_pairs = (L.n_flat + 1) / 2;
  const int n_kwg = (n_kv + 1) / 2;  // 128-key groups of the exact dK/dV kernel
  if (masked) {
    hipLaunchKernelGGL(bwd_ns_tables_kernel, dim3(n_pairs, BH), dim3(kThreads), 0, s, L.ns,
                       L.n_flat, L.n_ns, n_kv, words, L.ns_mask, L.tok_list, L.tok_cnt);
    ISA_CHECK(hipGetLastError());
    hipLaunchKernelGGL(bwd_ns_keylists_kernel, dim3(BH), dim3(kListThreads), 0, s, L.ns_mask,
                       L.flat, L.n_flat, words, n_kwg, (int64_t)L.n_flat * L.n_ns, L.fq_off,
                       L.fq_list);
    ISA_CHECK(hipGetLastError());
    p.ns_mask = L.ns_mask;
    p.ns_words = words;
    p.n_flat = L.n_flat;
    p.tok_list = L.tok_list;
    p.tok_cnt = L.tok_cnt;
    p.tok_cap = 2 * L.n_ns;
    p.k_tok = L.K;
    p.v_tok = L.V;
    p.tok_head_stride = (int64_t)L.N * D;
    p.fq_off = L.fq_off;
    p.fq_list = L.fq_list;
    p.fq_cap = (int64_t)L.n_flat * L.n_ns;
  }

  // Taylor path (flat query blocks against the pooled kept blocks; with the
  // mask, also the token tiles of their exact blocks in the dQ kernel)
  BwdParams pt = p;
  pt.k = L.kc;
  pt.v = L.vc;
  pt.kv_rows = n_kv;
  pt.kv_head_stride = (int64_t)n_kv * D;
  pt.lse_offset = (float)log((double)L.block);
  pt.q_tab = L.flat;
  pt.q_tab_stride = L.n_flat;
  pt.n_q_entries = flat_tiles;
  pt.q_slices = L.n_flat << shift;
  // keys = pooled rows t of this head's compact K^c_new: an identity row table
  pt.kv_tab = L.iota;
  pt.kv_tab_stride = 0;
  pt.dkc = L.dkc;
  pt.dvc = L.dvc;

  // exact path (sharp query blocks against K_new through the block table;
  // with the mask, then the flat blocks that take these keys token by token)
  BwdParams pe = p;
  pe.k = L.K;
  pe.v = L.V;
  pe.kv_rows = key_tiles * kBN;
  pe.kv_head_stride = (int64_t)L.N * D;
  pe.lse_offset = 0.0f;
  pe.q_tab = L.sharp;
  pe.q_tab_stride = L.n_sharp;
  pe.n_q_entries = sharp_tiles;
  pe.q_slices = L.n_sharp << shift;
  pe.dkc_in = L.n_flat > 0 ? L.dkc : nullptr;
  pe.dvc_in = L.n_flat > 0 ? L.dvc : nullptr;
  pe.inv_w = 1.0f / (float)L.block;

  auto paths = D == 128 ? (gen ? launch_paths<128, true> : launch_paths<128, false>)
                        : (gen ? launch_paths<64, true> : launch_paths<64, false>);
  ISA_CHECK(paths(pt, pe, masked, flat_tiles, sharp_tiles, n_kv, key_tiles, BH, s));
  if (L.n_ctx > 0) {
    if (D == 128)
      hipLaunchKernelGGL(bwd_zero_unselected_kernel<128>, dim3(L.n_ctx, BH), dim3(kThreads), 0, s,
                         L.sel, grid, L.k, L.dK, L.dV);
    else
      hipLaunchKernelGGL(bwd_zero_unselected_kernel<64>, dim3(L.n_ctx, BH), dim3(kThreads), 0, s,
                         L.sel, grid, L.k, L.dK, L.dV);
    ISA_CHECK(hipGetLastError());
  }
#undef ISA_CHECK
  return hipSuccess;
}

}  // namespace isa
