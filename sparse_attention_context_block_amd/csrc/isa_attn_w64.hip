// One-wave-per-SIMD bf16 MFMA online-softmax attention for gfx950 at head
// dimension 128: the exact path of ISA (keys of K_new read in place through the
// block table, the fused gather + concat of [notes] key design 1) and the
// dense baseline.  [notes] key design 2, exact branch: per key tile,
// l += rowsum(exp(S)), O += exp(S) V; at the end O / l.
//
// One workgroup = 4 waves = 256 query rows (four 64-row query tiles of a
// worklist); each wave owns 64 rows as two 32-row halves.  Products, with
// v_mfma_f32_32x32x16_bf16 throughout:
//   S^T (64 keys x 32 queries of half h) = K_tile Q_h^T   (keys on the M axis:
//       a lane holds 16 scores of one query per 32-key subtile, so the row max
//       and row sum need one permlane32 swap);
//   O_h^T (128 dims x 32 queries) += V^T P_h^T           (P^T packed straight
//       from the S^T accumulators).
// Each K or V^T operand fragment read from LDS feeds the MFMAs of both halves,
// so a wave moves half the LDS bytes per flop of a 32-row wave.  O stays in
// AGPRs (the PV products are written as inline asm on AGPR accumulators), so
// the softmax has the VGPR file to itself.
//
// Key tiles (64 consecutive token rows of one block) are copied HBM/L2 -> LDS
// with direct-to-LDS loads (global_load_lds_dwordx4: no VGPR staging, no VALU)
// into rings of 3 K and 5 V tiles: tile t + 3 is requested at the start of
// iteration t and must have landed at the end of iteration t + 1.  K rows are padded to
// 272 bytes (the K operand reads, 32 rows of one 16-byte chunk per half-wave,
// are conflict-free), V rows to 320 bytes (each transposing read,
// ds_read_b64_tr_b16, covers 8 rows x 64 bytes, conflict-free at this stride);
// a pad slot receives a duplicate of its row's last chunk.
//
// Software pipeline of one wave over key tile t: 64 MFMA slots of one product
// each, O += V(t-1) P(t-1) in slots 0-31 and S(t+1) = K(t+1) Q^T in slots
// 32-63, with the softmax of tile t issued between the products, one
// exponential per slot.  S is double-buffered (the scores of tiles t and t+1
// live in two register sets), so the exponentials of a tile run on while the
// next tile's products fill the other set.  A single wave issues in order, so
// the schedule is written out slot by slot (the table above the loop) and
// fenced, which keeps the compiler from regrouping it.  Each iteration ends at
// a barrier: tile t+2 has landed, and every wave is done with V(t-1) and
// K(t+1), whose ring slots the next iteration's loads reuse.
//
// Softmax reference: a wave issues one instruction at a time and a product
// hides only about half of its own 32 cycles of other work, so the per-tile
// row maxima of the online softmax (32 max3 and a cross-lane decision per
// tile) are not taken.  Each tile is exponentiated against a running
// reference, first the row maxima of tile 0; its row sums, complete before
// any product reads the tile's weights, show whether that was safe.  A sum
// above 2^8 raises the reference by its next power of two (O and l rescaled
// exactly; the tile's own sum is taken over the bf16 weights the products
// use).  A sum above 2^64 or not finite means the weights may have
// overflowed: the workgroup writes a NaN mark into its first output, and a
// second launch of this kernel recomputes the marked workgroups from the exact
// row maxima (every other workgroup of that launch reads its mark and exits).
//
// The products are inline asm, whose latency the compiler does not know: every
// read of their results is placed a product or an explicit wait after them, no
// accumulator may be dead while its product is in flight (the compiler would
// give its registers away), and paths join only after a wait.
#include <type_traits>

#include "isa_internal.h"

namespace isa {
namespace {

// f(integral_constant<int, I>) for I = B .. E - 1, each call with a constant I
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kThreads = 256;
constexpr int kD = 128;
constexpr int kBN = 64;                       // keys per tile
constexpr int kKStride = 272;                 // bytes per K row in LDS
constexpr int kVStride = 320;                 // bytes per V row in LDS
constexpr int kKTile = kBN * kKStride;        // 17408
constexpr int kVTile = kBN * kVStride;        // 20480
constexpr int kNK = 3, kNV = 5;               // ring slots
constexpr int kVBase = kNK * kKTile;          // V ring after the K ring
constexpr int kLds = kVBase + kNV * kVTile;   // 154624 bytes
constexpr int kKSlots = kBN * (kKStride / 16);  // 1088 16-byte slots per K tile
// A tile's row sum against the current reference above kRebase raises the
// reference; above kOverflow (or not finite) its exponentials may have
// overflowed and the workgroup is marked.
constexpr float kRebase = 256.0f;
constexpr float kOverflow = 18446744073709551616.0f;  // 2^64
static_assert(kKSlots <= 17 * 64 && kBN * (kVStride / 16) == 20 * 64, "DMA split");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u4;

// 16 bytes per lane from sbase + voff into LDS at m0 + 16 * lane, with
// m0 = lds + LdsOff written in the same statement (one wait state between the
// write of m0 and the load that reads it).  The load counts in vmcnt only; the
// caller waits on it before the barrier that publishes the tile.
template <uint32_t LdsOff>
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds), "n"(LdsOff)
               : "memory", "m0", "scc");
}

// O^T (32 dims x 32 queries) += V^T fragment x P^T fragment, accumulator in AGPRs.
// The products are volatile statements, so they keep their program order
// with the other volatile statements below (the anchors and the hazard waits).
__device__ __forceinline__ void mfma_pv(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// S^T (32 keys x 32 queries) = K fragment x Q^T fragment (first: C = 0, else
// accumulate).  Its first reader is a phase later.
// The Q^T operand is held in AGPRs (it is only ever an MFMA operand), which
// leaves the VGPRs to S, P and the softmax.
__device__ __forceinline__ void mfma_qk(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b,
                                        bool first) {
  if (first)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}

// The compiler does not see the latency of the products above (they are inline
// asm), so every VALU access to their results first waits 24 cycles here: a
// 32x32x16 product writes its result at most 16 passes after issue.  The
// accumulators are operands, so no access can be moved across the wait.
__device__ __forceinline__ void wait_o(f32x16_t (&o)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]),
                 "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
}
__device__ __forceinline__ void wait_s(f32x16_t (&s)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}
// the same for key subtile k of both halves only
__device__ __forceinline__ void wait_s(f32x16_t (&s)[2][2], int k) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0][k]), "+v"(s[1][k]));
}
// a use of S that keeps its registers reserved up to this point
__device__ __forceinline__ void keep_s(const f32x16_t (&s)[2][2]) {
  asm volatile("" ::"v"(s[0][0]), "v"(s[0][1]), "v"(s[1][0]), "v"(s[1][1]));
}
// VALU writes of the Q^T operands (AGPRs) before the first product reads them.
__device__ __forceinline__ void wait_q(bf16x8_t (&q)[2][8]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+a"(q[0][0]), "+a"(q[0][1]), "+a"(q[0][2]), "+a"(q[0][3]), "+a"(q[0][4]),
                 "+a"(q[0][5]), "+a"(q[0][6]), "+a"(q[0][7]), "+a"(q[1][0]), "+a"(q[1][1]),
                 "+a"(q[1][2]), "+a"(q[1][3]), "+a"(q[1][4]), "+a"(q[1][5]), "+a"(q[1][6]),
                 "+a"(q[1][7]));
}
// Keeps a step's softmax work before the next step's products: the value must
// be computed here (without this, the compiler sinks the exponentials of a
// phase past its products, to where their results are first used).
__device__ __forceinline__ void anchor(float x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// max of two finite scores or -inf: a plain v_max_f32 (fmaxf would first
// canonicalize each operand that does not come from arithmetic, here the
// outputs of a lane swap, with two more instructions)
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// kShift: log2 of the 32-row slices per block, 1 (b = 64) or 2 (b = 128).
// kPartial: some key tiles may hold fewer than 64 valid rows (plans whose
// source or context length is not a multiple of b); without it every tile is
// whole, and the loop carries no masking or clamping code.
// kFixup: the second launch, which recomputes (from the exact row maxima) the
// workgroups whose exponentials the first one found overflowed; the others
// exit at once.
template <int kShift, bool kPartial, bool kFixup>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_w64_kernel(AttnParams p) {
  static_assert(kShift == 1 || kShift == 2, "a key tile is 64 rows of one block");
  constexpr int D = kD;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLds];

  // ---- XCD-aware mapping of workgroups to (head, query tile) ----
  const int wg_per_head = (p.n_q_entries + 3) / 4;
  const int total = wg_per_head * p.BH;
  const int per_xcd = (total + 7) / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= total || p.kv_rows < kBN) return;  // whole workgroup, before any barrier
  const int64_t bh = lid / wg_per_head;
  const int qt = lid % wg_per_head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- this wave's 64 query rows: half h is slice 2e + h of the query list
  // (rows past a partial block's end read the slice's first row, not stored) ----
  const int e = qt * 4 + wave;
  const bool wave_valid = e < p.n_q_entries;
  const int32_t* qlist = p.q_tab ? p.q_tab + bh * p.q_tab_stride : nullptr;
  if constexpr (kFixup) {
    // the first launch's mark: dim 0 of row 0 of wave 0's first half; not NaN:
    // the whole workgroup exits before loading anything else
    const Slice q0 = list_slice(p.grid, qlist, p.n_q_slices, kShift, 2 * (qt * 4));
    const bf16_bits mark =
        *(static_cast<const bf16_bits*>(p.o) + bh * p.q_head_stride + (int64_t)q0.start * D);
    if (!((mark & 0x7f80u) == 0x7f80u && (mark & 0x7fu) != 0)) return;
  }
  const bf16_bits* Qh = static_cast<const bf16_bits*>(p.q) + bh * p.q_head_stride;
  bool q_ok[2];
  int64_t qrow[2];
  bf16x8_t qreg[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const Slice qs = list_slice(p.grid, qlist, wave_valid ? p.n_q_slices : 0, kShift, 2 * e + h);
    q_ok[h] = l32 < qs.cnt;
    qrow[h] = (int64_t)qs.start + (q_ok[h] ? l32 : 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qreg[h][kk] = *reinterpret_cast<const bf16x8_t*>(Qh + qrow[h] * D + 16 * kk + 8 * hi);
  }
  wait_q(qreg);

  // ---- key tiles: tile u = rows 64 * (u mod 2^(kShift-1)) .. + 63 of block
  // tab[u >> (kShift-1)] (fewer at a partial block; an empty tile is masked) ----
  const char* Kh = reinterpret_cast<const char*>(static_cast<const bf16_bits*>(p.k) +
                                                 bh * p.kv_head_stride);
  const char* Vh = reinterpret_cast<const char*>(static_cast<const bf16_bits*>(p.v) +
                                                 bh * p.kv_head_stride);
  const int32_t* tab = p.kv_tab ? p.kv_tab + bh * p.kv_tab_stride : nullptr;
  const int n_tiles = p.kv_rows / kBN;
  BlockGrid g;
  g.L_src = __builtin_amdgcn_readfirstlane(p.grid.L_src);
  g.n_src = __builtin_amdgcn_readfirstlane(p.grid.n_src);
  g.N = __builtin_amdgcn_readfirstlane(p.grid.N);
  g.len = __builtin_amdgcn_readfirstlane(p.grid.len);
  asm("" : "+s"(g.L_src), "+s"(g.n_src), "+s"(g.N), "+s"(g.len));
  struct Tile {
    int start, cnt;
  };
  // block id of tile u (u clamped to the last tile): a scalar load, issued an
  // iteration or more before its use so no wait on it stalls the LDS reads
  auto tile_id = [&](int u) -> int {
    const int eb = min(u, n_tiles - 1) >> (kShift - 1);
    return tab ? tab[eb] : eb;
  };
  auto tile_of = [&](int blk, int u) -> Tile {
    const int sub = (u & ((1 << (kShift - 1)) - 1)) * kBN;
    const int st = g.start(blk);
    const int rows = g.rows(blk) - sub;
    Tile tl = rows > 0 ? Tile{st + sub, rows < kBN ? rows : kBN} : Tile{st, 0};
    tl.start = __builtin_amdgcn_readfirstlane(tl.start);
    tl.cnt = __builtin_amdgcn_readfirstlane(tl.cnt);
    return tl;
  };

  // ---- direct-to-LDS copy of one tile (this wave's share) ----
  // slot s = 64 (4 i + wave) + lane of the padded tile: K row s / 17, V row s / 20;
  // a pad slot loads its row's chunk 15 (harmless).  voff = row * 256 + chunk * 16.
  uint32_t voff_k[5], voff_v[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int s = 64 * (4 * i + wave) + lane;
    const int rk = s / 17, ck = min(s % 17, 15);
    voff_k[i] = (uint32_t)(min(rk, kBN - 1) * 256 + ck * 16);
    const int rv = s / 20, cv = min(s % 20, 15);
    voff_v[i] = (uint32_t)(rv * 256 + cv * 16);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
  // Tile u (block id blk) into ring slots u mod 3 (K) and u mod 5 (V); tiles
  // past the end copy the last tile again into their (unused) slots, so every
  // iteration issues the same number of loads and the wait counts stay exact.
  // dma_plan resolves the tile on the scalar unit; dma_issue(d, i) issues load
  // i of this wave's share: i = 0-3 K rows, 4-8 V rows, 9 the last K rows
  // (wave 0 only).  The loop issues one load per slot, so the wave's in-order
  // issue never stalls behind a burst of address work.
  struct Dma {
    const char* kb;
    const char* vb;
    uint32_t km0, vm0, last;
    bool full;
  };
  auto dma_plan = [&](int blk, int u) -> Dma {
    const Tile tl = tile_of(blk, min(u, n_tiles - 1));
    Dma d;
    d.kb = Kh + (int64_t)tl.start * (D * 2);
    d.vb = Vh + (int64_t)tl.start * (D * 2);
    d.km0 = lds0 + (u % kNK) * kKTile + 1024 * wave;
    d.vm0 = lds0 + kVBase + (u % kNV) * kVTile + 1024 * wave;
    d.full = !kPartial || tl.cnt == kBN;
    d.last = (uint32_t)max(tl.cnt - 1, 0);
    return d;
  };
  auto dma_issue = [&](const Dma& d, auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    // rows past the tile's valid rows repeat its last one (they are masked)
    auto clamp = [&](uint32_t vo) { return min(vo >> 8, d.last) * 256u + (vo & 255u); };
    constexpr bool k = i < 4 || i == 9;
    constexpr int ii = i < 4 ? i : (i == 9 ? 4 : i - 4);
    const uint32_t vo = k ? voff_k[ii] : voff_v[ii];
    if (i == 9 && wave != 0) return;
    if (d.full)
      dma16<4096 * ii>(k ? d.kb : d.vb, vo, k ? d.km0 : d.vm0);
    else
      dma16<4096 * ii>(k ? d.kb : d.vb, clamp(vo), k ? d.km0 : d.vm0);
  };
  auto dma_tile = [&](int blk, int u) __attribute__((always_inline)) {
    const Dma d = dma_plan(blk, u);
    static_for<0, 10>([&](auto i_c) __attribute__((always_inline)) { dma_issue(d, i_c); });
  };
  // Loads per tile: 9 per wave (10 for wave 0).  vmcnt <= 9 leaves the most
  // recent tile in flight and completes every earlier one (wave 0 also waits
  // for one load of the most recent tile).
#define ISA_WAIT_ALL_BUT_LAST_TILE() asm volatile("s_waitcnt vmcnt(9)" ::: "memory")
#define ISA_BARRIER() asm volatile("s_barrier" ::: "memory")

  // ---- per-lane LDS addresses of the operand fragments ----
  // K fragment f = (s, kk) = (f >> 3, f & 7): row 32 s + l32, dims 16 kk + 8 hi .. + 7
  const uint32_t k_lane = lds0 + (uint32_t)(l32 * kKStride + hi * 16);
  // V^T fragment f = (c, j) = (f >> 2, f & 3): two transposing reads of rows
  // 16 c + 8 r + 4 (G >> 1) + (q >> 2) (r = 0, 1), dims 32 j + 16 (G & 1) + 4 (q & 3)
  // .. + 3, lane = 16 G + q; together they hold keys 16 c + 8 (e >> 2) + 4 hi + (e & 3)
  // of dim 32 j + l32 in slot e, the order of the P^T operand below
  const int G = lane >> 4, q = lane & 15;
  const uint32_t v_lane = lds0 + (uint32_t)((4 * (G >> 1) + (q >> 2)) * kVStride +
                                            32 * (G & 1) + 8 * (q & 3));
  // (kaddr, vaddr: absolute LDS byte addresses of the lane's fragment 0 in a
  // slot; every fragment is that address plus a constant, which the reads take
  // as their immediate offset)
  auto k_frag = [&](uint32_t kaddr, int f) -> bf16x8_t {
    return *(const lds_bf16x8*)(uintptr_t)(kaddr + (f >> 3) * (32 * kKStride) + 32 * (f & 7));
  };
  auto v_frag = [&](uint32_t vaddr, int f) -> bf16x8_t {
    const uint32_t b = vaddr + (f >> 2) * (16 * kVStride) + 64 * (f & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)b);
    const v4i16 hh =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(b + 8 * kVStride));
    const v4i16 both[2] = {lo, hh};
    return __builtin_bit_cast(bf16x8_t, both);
  };
  // per-iteration fragment base: one VGPR add, hidden from the optimizer so it
  // neither hoists per-fragment addresses into registers nor splits the sum
  auto lane_addr = [&](uint32_t lane_off, uint32_t slot_off) -> uint32_t {
    uint32_t a = lane_off + slot_off;
    asm volatile("" : "+v"(a));
    return a;
  };

  // ---- state ----
  f32x16_t oacc[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[h][j][r] = 0.0f;
  // S^T of two consecutive tiles: [tile parity][half][key subtile]
  f32x16_t sacc[2][2][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[b][h][s][r] = 0.0f;
  bf16x8_t pk[2][4];  // [half][16-key chunk]: P^T operands (zero before tile 0)
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) pk[h][c][e2] = (__bf16)0.0f;
  // Reference of O and l per half (scaled log2 units) and its negative, which
  // the exponentials add.  A tile is exponentiated against the current
  // reference, not against its own row max, and the row sums of its
  // exponentials, complete before any product reads them, show whether that
  // was safe: a sum above kRebase (or not finite) sends the tile down the rare
  // path, which takes its exact row maxima, raises the reference, redoes its
  // exponentials and rescales O and l.
  float m_run[2], mneg[2];
  float l_run[2] = {0.0f, 0.0f};
  float l_tile[2] = {0.0f, 0.0f};  // this lane's part of the current tile's row sums
  // a rebase at the end of tile t: O (which then still takes P(t) against the
  // old reference) is rescaled after P(t)'s products, in slot 31 of the next
  // iteration or at the end of the tail
  float alpha[2] = {1.0f, 1.0f};
  bool up[2] = {false, false};
  bool dirty = false;  // a tile's row sum was not finite or above kOverflow
  float m_init[2] = {0.0f, 0.0f};  // fix-up launch: the exact row maxima
  __shared__ int vote[4];          // the waves' marks
  // exponentials waiting for their pair's pack: element j at j & 7
  float pe[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float sl2 = p.scale_log2;
  asm("" : "+s"(sl2));

  // Element j (0-63) of a tile's P: pair p = j >> 1 of chunk c = p >> 3, half
  // (p >> 2) & 1, slot 2 (p & 3) + (j & 1) of the P^T operand, which is key
  // 16 c + 8 (e2 >> 2) + 4 hi + (e2 & 3) of the half's query: register
  // 8 (c & 1) + e2 of S^T subtile c >> 1.
  auto elem = [&](int par, int j) __attribute__((always_inline)) {
    const int pr = j >> 1, c = pr >> 3, h = (pr >> 2) & 1, e2 = 2 * (pr & 3) + (j & 1);
    pe[j & 7] =
        __builtin_amdgcn_exp2f(fmaf(sacc[par][h][c >> 1][8 * (c & 1) + e2], sl2, mneg[h]));
    anchor(pe[j & 7]);
  };
  // Pair p into P^T (bf16, round to nearest even) and into the tile's row sum,
  // which adds the fp32 exponentials: v_dot2c_f32_bf16 on the packed pair
  // issues on the matrix pipe and would wait for the product in flight.
  // Pairs 0 and 4 are the first of their half in a tile.
  auto pack = [&](int pr) __attribute__((always_inline)) {
    const int c = pr >> 3, h = (pr >> 2) & 1, e2 = 2 * (pr & 3);
    const float a0 = pe[(2 * pr) & 7], a1 = pe[(2 * pr + 1) & 7];
    pk[h][c][e2] = (__bf16)a0;
    pk[h][c][e2 + 1] = (__bf16)a1;
    // (the packed pair is used only by the next tile's products: without the
    // anchor the compiler sinks the conversion out of its slot, to the start
    // of the next iteration, where no product is in flight to hide it)
    anchor(__uint_as_float(__builtin_bit_cast(u32x4, pk[h][c])[pr & 3]));
    if (pr == 0 || pr == 4)
      l_tile[h] = a0 + a1;
    else
      l_tile[h] = (l_tile[h] + a0) + a1;
    anchor(l_tile[h]);
  };
  // slot of the pack of pair p: chunk 0's pairs wait for slot 8 (P(t-1) chunk 0
  // is read in slots 0-7), the others follow their elements by one slot
  auto pack_slot = [](int pr) constexpr -> int {
    return pr < 4 ? 8 + pr : (pr < 7 ? 2 * pr + 4 - (pr - 4) : 2 * pr + 2);
  };
  // keys >= cnt of subtile s get -inf (partial tiles only)
  auto mask_subtile = [&](int par, int s, int cnt) __attribute__((always_inline)) {
    if (kPartial && cnt < kBN) {
      wait_s(sacc[par], s);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * s + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= cnt) sacc[par][h][s][r] = -INFINITY;
        }
    }
  };
  // the row maxima of S^T set par (both subtiles; the partner lane holds the
  // other 32 keys of the row), in scaled log2 units
  auto row_max = [&](int par, float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t = sacc[par][h][0][0];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int r = 0; r < 16; ++r) t = fmaxf(t, sacc[par][h][s2][r]);
      const uint32_t u = __float_as_uint(t);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mx[h] = max2(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
    }
  };
  // Tile t fully exponentiated and packed: fold its row sums into l.  Rare: a
  // sum above kRebase.  Then the reference rises by the next power of two of
  // the sum (so P(t) against the new one is at most 1), l is rescaled here and O
  // after P(t)'s products (slot 31 of the next iteration, or the tail).  A sum
  // above kOverflow (or not finite) means P(t) may hold infinities: the
  // workgroup is marked for the fix-up launch.
  auto check_tile = [&]() __attribute__((always_inline)) {
    const bool any =
        __builtin_amdgcn_ballot_w64(!(max2(l_tile[0], l_tile[1]) <= kRebase)) != 0;
    fence();
    if (any) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t u = __float_as_uint(l_tile[h]);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const float L = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // the row's sum
        const bool big = !(L <= kRebase);
        dirty = dirty || !(L <= kOverflow);
        // A rebased row's sum is taken again over the packed bf16 weights the
        // products use, so that numerator and denominator hold the same
        // weights: its largest weight, which dominates the row, is not 1 here.
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) part += (float)pk[h][c][e2];
        const float lt = big ? part : l_tile[h];
        const uint32_t w = __float_as_uint(lt);
        const auto sw2 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
        const float L2 = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
        const float k = big ? ceilf(__builtin_amdgcn_logf(L2)) : 0.0f;
        alpha[h] = __builtin_amdgcn_exp2f(-k);  // a power of two: exact
        m_run[h] += k;
        mneg[h] = -m_run[h];
        up[h] = __builtin_amdgcn_ballot_w64(big) != 0;
        l_run[h] = (l_run[h] + lt) * alpha[h];
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        l_run[h] += l_tile[h];
        up[h] = false;
      }
    }
    fence();
  };
  // O *= alpha after a rebase (rare), once the products that read O are done
  auto rescale_o = [&]() __attribute__((always_inline)) {
    fence();
    if (up[0] || up[1]) {
      wait_o(oacc);  // the accumulating products finish before O is read
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[h][j][r] *= alpha[h];
      wait_o(oacc);  // and the writes land before the next product reads O
    }
  };

  // block ids of the tiles the loop requests next (t + 3) and masks (t + 1),
  // and the valid rows of the current tile
  int id_t1 = 0, id_t2 = 0, id_t3 = 0, cnt_cur = 0;

  // ---- the tile loop: 64 MFMA slots per tile, one product each ----
  //   slots  0-31  O += V(t-1) P(t-1): slot i is fragment i >> 1, half i & 1
  //   slots 32-63  S(t+1) = K(t+1) Q^T: slot 32 + i is fragment i >> 1, half i & 1
  //                (into the other S set: S(t) stays until its exponentials end)
  // VALU work placed after the products (packs before exponentials), spread so
  // that each slot's work fits the 32 cycles of its product (in-order issue
  // makes a second product wait for the first; work that does not fit delays
  // the next product):
  //   every slot    one exponential of tile t: element = slot (subtile 0, keys
  //                 0-31, in slots 0-31; its products ended in the previous
  //                 iteration's slot 47; subtile 1 from slot 32)
  //   packs         pair p (elements 2p, 2p + 1) of tile t: chunk 0 (pairs 0-7)
  //                 in slots 8-16, after P(t-1) chunk 0 was last read (slot 7);
  //                 pair p >= 7 in slot 2p + 2 (chunk c from slot 16c + 2, after
  //                 P(t-1) chunk c was last read in slot 8c + 7); pair 31 after
  //                 slot 63
  //   after slot 63  tile t's row sums checked and folded into l (rare: rebase)
  //   odd slots 21-39  loads of tile t + 3, one per slot (into the ring slots
  //                 of K(t) and V(t-2), which no wave reads after the last barrier)
  // Fragment reads run three fragments (six slots) ahead of their products.
  auto iteration = [&](int t, auto par_c) __attribute__((always_inline)) {
    constexpr int P = decltype(par_c)::value;  // parity of tile t
    constexpr int Q = P ^ 1;                   // of tiles t - 1 and t + 1
    // tile t + 3 is requested in odd slots 21-39 (its block id was read at the
    // end of the last iteration)
    const Dma dma = dma_plan(id_t3, t + 3);
    const int cnt_next = tile_of(id_t1, min(t + 1, n_tiles - 1)).cnt;
    const uint32_t vprev = lane_addr(v_lane, kVBase + ((t + kNV - 1) % kNV) * kVTile);
    const uint32_t knext = lane_addr(k_lane, ((t + 1) % kNK) * kKTile);
    bf16x8_t vf[16], kf[16];
    vf[0] = v_frag(vprev, 0);
    vf[1] = v_frag(vprev, 1);
    vf[2] = v_frag(vprev, 2);
    fence();
    static_for<0, 64>([&](auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      // ---- fragment reads, three fragments ahead ----
      if constexpr (slot < 32 && (slot & 1) == 0 && (slot >> 1) + 3 < 16)
        vf[(slot >> 1) + 3] = v_frag(vprev, (slot >> 1) + 3);
      if constexpr (slot >= 26 && slot < 58 && (slot & 1) == 0)
        kf[(slot - 26) >> 1] = k_frag(knext, (slot - 26) >> 1);
      // ---- the product ----
      if constexpr (slot < 32) {
        constexpr int f = slot >> 1, h = slot & 1;
        mfma_pv(oacc[h][f & 3], vf[f], pk[h][f >> 2]);
      } else {
        constexpr int f = (slot - 32) >> 1, h = slot & 1;
        mfma_qk(sacc[Q][h][f >> 3], kf[f], qreg[h][f & 7], (f & 7) == 0);
      }
      // ---- VALU work of this slot ----
      if constexpr (slot == 32) mask_subtile(P, 1, cnt_cur);  // (partial tiles)
      static_for<0, 31>([&](auto pr_c) __attribute__((always_inline)) {
        constexpr int pr = decltype(pr_c)::value;
        if constexpr (pack_slot(pr) == slot) pack(pr);
      });
      elem(P, slot);
      if constexpr (slot == 31) rescale_o();  // (rare) after P(t-1)'s products
      if constexpr (slot == 48) mask_subtile(Q, 0, cnt_next);
      if constexpr (slot >= 21 && slot < 40 && (slot & 1) == 1)
        dma_issue(dma, std::integral_constant<int, ((slot - 21) >> 1)>{});
      fence();
    });
    pack(31);
    check_tile();
    cnt_cur = cnt_next;
    id_t1 = id_t2;
    id_t2 = id_t3;

    // Tile t + 2 has landed (this wave's loads), and after the barrier every
    // wave's: the next iteration reads K(t+2) and V(t); the loads it issues
    // overwrite the slots of K(t) and V(t-2), which every wave has finished.
    // The block id of tile t + 4 is read here with a scalar load waited on in
    // the same statement: the wave waits at the barrier anyway, and no LDS read
    // is in flight.  (A plain C++ load after the DMA statements, which clobber
    // memory, would become a vector load whose wait drains every tile load.)
    if (tab) {
      const int32_t* idp = tab + (min(t + 4, n_tiles - 1) >> (kShift - 1));
      asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier"
                   : "=s"(id_t3)
                   : "s"(idp)
                   : "memory");
    } else {
      id_t3 = min(t + 4, n_tiles - 1) >> (kShift - 1);
      asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
    }
  };
  // ---- last tile: O += V(n-1) P(n-1) ----
  // Ends with every product written: the caller's paths join after it, and a
  // register copy the compiler places at a join would otherwise read an
  // accumulator before its product (inline asm, of unknown latency) wrote it.
  auto tail = [&]() __attribute__((always_inline)) {
    // The paths into the tail may keep O in other registers; the copies the
    // compiler then places at the join must land before the first product
    // reads O (inline asm: the compiler inserts no wait states for it).
    wait_o(oacc);
    const uint32_t vlast = lane_addr(v_lane, kVBase + ((n_tiles - 1) % kNV) * kVTile);
    bf16x8_t vf[16];
    vf[0] = v_frag(vlast, 0);
    vf[1] = v_frag(vlast, 1);
    vf[2] = v_frag(vlast, 2);
    static_for<0, 32>([&](auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      if constexpr ((slot & 1) == 0 && (slot >> 1) + 3 < 16)
        vf[(slot >> 1) + 3] = v_frag(vlast, (slot >> 1) + 3);
      constexpr int f = slot >> 1, h = slot & 1;
      mfma_pv(oacc[h][f & 3], vf[f], pk[h][f >> 2]);
      fence();
    });
    rescale_o();  // (rare) a rebase at the end of the last tile
    // drain the loads issued for tiles past the end before the workgroup exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    wait_o(oacc);
    // The last iteration's S products (of the tile after the last) are never
    // read; without a use the compiler would hand their registers to other
    // values while those products are still in flight and would overwrite them.
    keep_s(sacc[0]);
    keep_s(sacc[1]);
  };
  // The exact row maxima over every key tile (K only, one tile at a time): the
  // fix-up launch's reference for a workgroup the first launch marked.
  auto exact_maxima = [&]() {
    float tm[2] = {-INFINITY, -INFINITY};
    for (int u = 0; u < n_tiles; ++u) {
      const int blk = tile_id(u);
      const Dma d = dma_plan(blk, u);
      dma_issue(d, std::integral_constant<int, 0>{});
      dma_issue(d, std::integral_constant<int, 1>{});
      dma_issue(d, std::integral_constant<int, 2>{});
      dma_issue(d, std::integral_constant<int, 3>{});
      dma_issue(d, std::integral_constant<int, 9>{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const uint32_t kk0 = lane_addr(k_lane, (u % kNK) * kKTile);
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const bf16x8_t kfr = k_frag(kk0, f);
#pragma unroll
        for (int h = 0; h < 2; ++h) mfma_qk(sacc[0][h][f >> 3], kfr, qreg[h][f & 7], (f & 7) == 0);
      }
      wait_s(sacc[0]);
      const int cnt = tile_of(blk, u).cnt;
      mask_subtile(0, 0, cnt);
      mask_subtile(0, 1, cnt);
      float mx[2];
      row_max(0, mx);
      tm[0] = max2(tm[0], mx[0]);
      tm[1] = max2(tm[1], mx[1]);
      __syncthreads();  // every wave is done with the slot before it is reused
    }
    m_init[0] = tm[0];
    m_init[1] = tm[1];
  };

  // The first launch takes tile 0's row maxima as the first reference; the
  // fix-up launch, for the workgroups the first one marked, the exact row
  // maxima over every tile, so that no tile can exceed its reference.
  if constexpr (kFixup) exact_maxima();
  // ---- prologue: tiles 0-2 requested, 0 and 1 landed; S(0) and the first
  // reference (tile 0's exact row maxima) ----
  // The first iteration's O += V(-1) P(-1) reads V slot kNV - 1 with P = 0:
  // zero that slot so the product is exactly 0.
  {
    lds_u4* z = (lds_u4*)(uintptr_t)(lds0 + kVBase + (kNV - 1) * kVTile);
#pragma unroll
    for (int i = 0; i < kVTile / 16 / kThreads; ++i) z[tid + kThreads * i] = u32x4{0u, 0u, 0u, 0u};
  }
  id_t3 = tile_id(3);
  id_t1 = tile_id(1);
  id_t2 = tile_id(2);
  dma_tile(tile_id(0), 0);
  dma_tile(id_t1, 1);
  dma_tile(id_t2, 2);
  ISA_WAIT_ALL_BUT_LAST_TILE();
  __syncthreads();  // (also publishes the zeroed slot)
  cnt_cur = tile_of(tile_id(0), 0).cnt;
  {
    bf16x8_t kf[16];
    const uint32_t k0 = lane_addr(k_lane, 0);
    kf[0] = k_frag(k0, 0);
    kf[1] = k_frag(k0, 1);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      if (f + 2 < 16) kf[f + 2] = k_frag(k0, f + 2);
#pragma unroll
      for (int h = 0; h < 2; ++h) mfma_qk(sacc[0][h][f >> 3], kf[f], qreg[h][f & 7], (f & 7) == 0);
    }
    wait_s(sacc[0]);  // S(0) is read next by VALU
    mask_subtile(0, 0, cnt_cur);
    mask_subtile(0, 1, cnt_cur);
    float mx[2];
    row_max(0, mx);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m_run[h] = kFixup ? m_init[h] : mx[h];
      mneg[h] = -m_run[h];
    }
  }

  // Two iterations per trip (tile parity 0, then 1): the two copies of the
  // body alternate between the two S sets.
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    iteration(t, std::integral_constant<int, 0>{});
    iteration(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < n_tiles) iteration(t, std::integral_constant<int, 0>{});
  tail();

  // the waves' marks: a marked workgroup is redone by the fix-up launch
  bool redo = false;
  if constexpr (!kFixup) {
    if (lane == 0) vote[wave] = dirty ? 1 : 0;
    __syncthreads();
    redo = (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
  }

  // ---- epilogue: O / l, bf16 round-to-nearest-even, LSE ----
  if (!wave_valid) return;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = __float_as_uint(l_run[h]);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // own + partner
    const float inv = 1.0f / l;
    if (!q_ok[h]) continue;
    bf16_bits* Oh = static_cast<bf16_bits*>(p.o) + bh * p.q_head_stride + qrow[h] * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        bf16x2_t a, b;
        a[0] = (__bf16)(oacc[h][j][4 * gg + 0] * inv);
        a[1] = (__bf16)(oacc[h][j][4 * gg + 1] * inv);
        b[0] = (__bf16)(oacc[h][j][4 * gg + 2] * inv);
        b[1] = (__bf16)(oacc[h][j][4 * gg + 3] * inv);
        uint2 w;
        w.x = __builtin_bit_cast(uint32_t, a);
        w.y = __builtin_bit_cast(uint32_t, b);
        *reinterpret_cast<uint2*>(Oh + 32 * j + 8 * gg + 4 * hi) = w;
      }
    }
    if (p.lse && hi == 0) {
      p.lse[bh * p.lse_head_stride + qrow[h]] =
          (m_run[h] + __log2f(l)) * 0.69314718055994531f + p.lse_offset;
    }
  }
  // a marked workgroup: a NaN in dim 0 of its first row (wave 0, half 0, row 0,
  // always valid), which the fix-up launch reads
  if (!kFixup && redo && wave == 0 && lane == 0)
    *(static_cast<bf16_bits*>(p.o) + bh * p.q_head_stride + qrow[0] * D) = (bf16_bits)0x7fc0u;
#undef ISA_WAIT_ALL_BUT_LAST_TILE
#undef ISA_BARRIER
}

}  // namespace

bool attention_w64_supported(const AttnParams& p) {
  return p.D == kD && !p.kv_row_table && (p.half_shift == 1 || p.half_shift == 2) &&
         p.kv_rows >= kBN && p.kv_rows % kBN == 0;
}

hipError_t launch_attention_w64(const AttnParams& p, hipStream_t stream) {
  if (p.BH == 0 || p.n_q_entries == 0) return hipSuccess;
  if (!attention_w64_supported(p)) return hipErrorInvalidValue;
  const int wg_per_head = (p.n_q_entries + 3) / 4;
  const int64_t total = (int64_t)wg_per_head * p.BH;
  const dim3 grid((unsigned)(((total + 7) / 8) * 8));
  // whole tiles only when both segments are whole numbers of blocks
  const bool partial = p.grid.src_tail() != 0 || p.grid.ctx_tail() != 0;
  // then the fix-up launch (a workgroup reads one value and exits unless the
  // first launch marked it)
#define ISA_W64_LAUNCH(S, PART)                                                            \
  hipLaunchKernelGGL((attn_fwd_w64_kernel<S, PART, false>), grid, dim3(kThreads), 0, stream, p); \
  hipLaunchKernelGGL((attn_fwd_w64_kernel<S, PART, true>), grid, dim3(kThreads), 0, stream, p);
  if (p.half_shift == 1) {
    if (partial) {
      ISA_W64_LAUNCH(1, true)
    } else {
      ISA_W64_LAUNCH(1, false)
    }
  } else {
    if (partial) {
      ISA_W64_LAUNCH(2, true)
    } else {
      ISA_W64_LAUNCH(2, false)
    }
  }
#undef ISA_W64_LAUNCH
  return hipGetLastError();
}

}  // namespace isa
