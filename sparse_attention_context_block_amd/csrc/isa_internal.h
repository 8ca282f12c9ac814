// Internal declarations shared by the ISA kernels and the C-ABI host layer.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "isa.h"

namespace isa {

typedef uint16_t bf16_bits;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// Two bf16 from two words: the low halves (high = false) or the high halves
// (high = true) of lo_word and hi_word, lo_word's in the low half of the
// result.  One byte permute (v_perm_b32).
__device__ __forceinline__ uint32_t pack2(uint32_t lo_word, uint32_t hi_word, bool high) {
  return __builtin_amdgcn_perm(hi_word, lo_word, high ? 0x07060302u : 0x05040100u);
}

// fp64 -> bf16 bits, round to nearest even, in one rounding: truncate to fp32
// and keep the lost part as a sticky bit (round to odd, exact for any later
// rounding to 22 or fewer significant bits), then round the fp32 to bf16.
__device__ __forceinline__ uint32_t bf16_bits_rne(double x) {
  const float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 16 bytes at p with the nontemporal hint, for inputs a kernel reads once:
// they stream through the caches instead of displacing what is reused (a plain
// 1 GB read measured 6.3 against 5.1 TB/s when part of it was cache-resident).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v x = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// Height of the attention kernels' key and query tiles, and the block length
// of the kernels that are built for one (the block-mask kernel, the backward).
constexpr int kBlock = 64;

// Block grid of a [source | context] sequence ([notes] key design 1 counts
// ceil(L_ctx / b) context blocks): the source and the context are each cut
// into len-token blocks from their own start, so the last block of each
// segment may be partial.  Block b starts at len * b (b < n_src) or at
// L_src + len * (b - n_src) and holds min(len, segment end - start) tokens.
// A sequence without context (L_src = N) is a plain grid.
struct BlockGrid {
  int32_t L_src;  // tokens of the source segment
  int32_t n_src;  // its blocks, ceil(L_src / len)
  int32_t N;      // all tokens
  int32_t len;    // block length b
  __host__ __device__ __forceinline__ int start(int b) const {
    return b < n_src ? b * len : L_src + (b - n_src) * len;
  }
  __host__ __device__ __forceinline__ int rows(int b) const {
    const int end = b < n_src ? L_src : N;
    const int n = end - start(b);
    return n < len ? n : len;
  }
  __host__ __device__ __forceinline__ int n_blocks() const {
    return n_src + (N - L_src + len - 1) / len;
  }
  // tokens of the partial last block of each segment (0: the segment is whole)
  __host__ __device__ __forceinline__ int src_tail() const { return L_src % len; }
  __host__ __device__ __forceinline__ int ctx_tail() const { return (N - L_src) % len; }
};

// A 32-row slice of a block list.  With 2^shift slices per block (len =
// 32 << shift), slice eta of the list is rows 32 sub .. 32 sub + 31 of block
// list[eta >> shift] (list NULL: block eta >> shift), sub = eta mod 2^shift;
// only the rows inside the block count.  A slice past the list's n_slices, or
// past the end of a partial block, is empty (cnt 0) and starts at a valid row
// of the head.  The attention kernels' 64-row tiles are slices 2u and 2u + 1.
struct Slice {
  int32_t start;  // first token row
  int32_t cnt;    // valid rows, 0..32
};
__device__ __forceinline__ Slice list_slice(const BlockGrid& g, const int32_t* list,
                                            int n_slices, int shift, int eta) {
  if (eta >= n_slices) return Slice{0, 0};
  const int e = eta >> shift, sub = eta & ((1 << shift) - 1);
  const int blk = list ? list[e] : e;
  const int st = g.start(blk);
  const int cnt = g.rows(blk) - 32 * sub;
  if (cnt <= 0) return Slice{st, 0};
  return Slice{st + 32 * sub, cnt < 32 ? cnt : 32};
}

// The two slices 2u and 2u + 1 (key tile u) of a block list with 2^kShift
// slices per block, made wave-uniform (scalar registers) for the tile loops.
// With kShift >= 1 both lie in one block, list[u >> (kShift - 1)].
template <int kShift>
__device__ __forceinline__ void tile_slices(const BlockGrid& g, const int32_t* list,
                                            int n_slices, int u, Slice& a, Slice& b) {
  if constexpr (kShift == 0) {
    a = list_slice(g, list, n_slices, 0, 2 * u);
    b = list_slice(g, list, n_slices, 0, 2 * u + 1);
  } else {
    const int e = u >> (kShift - 1);
    const int sub = (u & ((1 << (kShift - 1)) - 1)) * 2;
    const int blk = list ? list[e] : e;
    const int st = g.start(blk), rows = g.rows(blk);
    const int ca = min(max(rows - 32 * sub, 0), 32);
    const int cb = min(max(rows - 32 * (sub + 1), 0), 32);
    a = Slice{ca > 0 ? st + 32 * sub : st, ca};
    b = Slice{cb > 0 ? st + 32 * (sub + 1) : st, cb};
  }
  a.start = __builtin_amdgcn_readfirstlane(a.start);
  a.cnt = __builtin_amdgcn_readfirstlane(a.cnt);
  b.start = __builtin_amdgcn_readfirstlane(b.start);
  b.cnt = __builtin_amdgcn_readfirstlane(b.cnt);
}

// ---------------------------------------------------------------------------
// Attention launch description shared by the exact path, the 0-th order
// Taylor path and the dense baseline.  Blocks have grid.len = 32 << half_shift
// tokens.  Query rows: the 32-row slices of the blocks listed in q_tab (NULL:
// block e is block e), n_q_slices of them; 64-row query tile e is slices 2e
// and 2e + 1.  Keys: with a block table (kv_row_table = 0) the slices of the
// blocks listed in kv_tab (NULL: identity), kv_rows / 32 of them, key tile u
// being slices 2u and 2u + 1 and empty rows masked; with a row table
// (kv_row_table = 1) key r is row kv_tab[r] of the K/V arrays (pooled block
// rows of the Taylor path), kv_rows keys.
// ---------------------------------------------------------------------------
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                // may be null
  const int32_t* q_tab;      // [BH][q_tab_stride] or null
  int64_t q_tab_stride;
  int32_t n_q_entries;       // 64-row query tiles per head, ceil(n_q_slices / 2)
  int32_t n_q_slices;        // 32-row query slices per head
  const int32_t* kv_tab;     // [BH][kv_tab_stride] or null
  int64_t kv_tab_stride;
  int32_t kv_rows;           // keys per head: 32 per slice (block table) or one per row
  int32_t kv_row_table;      // 1: kv_tab names rows; 0: kv_tab names blocks
  int32_t half_shift;        // log2(grid.len / 32)
  int64_t q_head_stride;     // elements between heads of Q and O
  int64_t kv_head_stride;    // elements between heads of the K/V arrays
  int64_t lse_head_stride;   // floats between heads of lse
  int32_t BH;
  int32_t D;
  float scale_log2;          // log2(e) / sqrt(D)
  float lse_offset;          // added to every lse (ln of a uniform block weight)
  // token layout of the blocks.  With a row table the keys are pooled block
  // rows: a partial block's row (K_new position n_src - 1 for the source
  // tail, the last position for a kept context tail) enters with the extra
  // weight log of (its tokens / len).
  BlockGrid grid;
};

hipError_t launch_attention(const AttnParams& p, isa_dtype_t dtype, hipStream_t stream);

// bf16 kernels: the 4-wave kernel (any key source; used for row tables), the
// one-wave-per-SIMD kernel (block tables at D = 128 with 64- or 128-token
// blocks: exact path, dense) and the 8-wave ping-pong kernel (the other block
// tables: D = 64, 32-token blocks).
hipError_t launch_attention_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attention_pp(const AttnParams& p, hipStream_t stream);
bool attention_w64_supported(const AttnParams& p);
hipError_t launch_attention_w64(const AttnParams& p, hipStream_t stream);

// Flat query blocks with a block mask (alpha_ns > 0): per flat block, the
// K_new blocks listed in ns token by token, every other block of K_new through
// its pooled row.
struct FlatParams {
  const void* q;            // token rows [BH][N][D]
  const void* k;
  const void* v;
  const void* kc;           // pooled rows [BH][n_q][D], same dtype
  const void* vc;
  void* o;
  float* lse;
  const int32_t* flat;      // [BH][n_flat] flat query blocks
  const int32_t* kv_tab;    // [BH][n_kv] block ids of K_new
  const int32_t* ns;        // [BH][n_flat][n_ns] K_new positions computed exactly
  int32_t n_flat, n_kv, n_ns;
  int64_t q_head_stride;    // N * D (Q, O)
  int64_t kv_head_stride;   // N * D (K, V)
  int64_t kc_head_stride;   // n_q * D (K^c, V^c)
  int64_t lse_head_stride;  // N
  int32_t BH, D;
  float scale_log2;         // log2(e) / sqrt(D)
  float exact_bias_log2;    // -log2(b): exact tokens weigh 1 against b per block
  float lse_offset;         // ln(b)
  BlockGrid grid;           // token layout of the blocks (partial segment tails)
};
hipError_t launch_attention_flat(const FlatParams& p, isa_dtype_t dtype, hipStream_t stream);
hipError_t launch_ns_select(const double* qc, const double* kc, const int32_t* flat,
                            const int32_t* kv_tab, int BH, int n_q, int D, int n_flat, int n_kv,
                            int n_ns, int32_t* ns, hipStream_t stream);

// Frequencies of the rotary embedding, base^(-2i/D) for the D/2 pairs
// (computed on the host, passed by value).
struct RopeFreq {
  double inv_freq[64];
};

// Block means of Q, K, V; with rope (non-null) Q and K are first rotated and
// the rotated rows written to qr, kr.
hipError_t launch_pool(const void* Q, const void* K, const void* V, isa_dtype_t dtype,
                       int BH, int N, int D, int L_src, int n_src, int n_q, int block,
                       double* qc, double* kc, void* kc_lp, void* vc_lp, void* qr, void* kr,
                       const RopeFreq* rope, hipStream_t stream);

// Every pair of X turned by its rotary angle (inverse: turned back), rounded
// once to the storage type, into Y (may be X).  The forward direction equals
// the pooling kernel's rotation bit for bit.
hipError_t launch_rope_rotate(const void* X, void* Y, isa_dtype_t dtype, int BH, int N, int D,
                              int L_src, const RopeFreq& rope, bool inverse, hipStream_t stream);

hipError_t launch_coarse_rowstats(const double* qc, const double* kc, int BH, int n_q, int D,
                                  double* rowmax, double* rowsum, double* sharpness,
                                  hipStream_t stream);

hipError_t launch_coarse_colsum(const double* qc, const double* kc, const double* rowmax,
                                const double* rowsum, int BH, int n_q, int n_src, int n_ctx,
                                int D, double* ctx_score, hipStream_t stream);

hipError_t launch_select_route(const double* ctx_score, const double* sharpness, int BH,
                               int n_src, int n_ctx, int n_q, int k, int n_flat,
                               int32_t* sel, int32_t* flat, int32_t* sharp, int32_t* kv_tab,
                               hipStream_t stream);

hipError_t launch_gather(const void* K, const void* V, const int32_t* sel, isa_dtype_t dtype,
                         int BH, int N, int D, int n_src, int k, int block,
                         void* K_new, void* V_new, hipStream_t stream);

// Backward launch description (bf16 only).  Workspace pointers: delta
// [BH*N] f32, kv_tab [BH*(n_src+k)] i32, iota [n_src+k] i32, kc/vc
// [BH*(n_src+k)*D] bf16 (means of the kept blocks), dkc/dvc same shape f32.
struct BwdLaunch {
  int BH, D, N, L_src, n_src, n_ctx, k, n_flat, n_sharp;
  int block;  // b (32, 64 or 128); partial blocks allowed
  const bf16_bits *Q, *K, *V, *O, *dO;
  const float* lse;
  const int32_t *sel, *flat, *sharp;
  bf16_bits *dQ, *dK, *dV;
  float* delta;
  int32_t *kv_tab, *iota;
  bf16_bits *kc, *vc;
  float *dkc, *dvc;
  // block mask inside flat rows (n_ns > 0 and n_flat > 0)
  int n_ns;
  const int32_t* ns;        // [BH][n_flat][n_ns] exact K_new blocks per flat block
  uint32_t* ns_mask;        // [BH][n_flat][ceil(n_kv / 32)]
  int32_t *tok_list, *tok_cnt;  // [BH][ceil(n_flat / 2)][2 n_ns], [BH][ceil(n_flat / 2)]
  int32_t *fq_off, *fq_list;    // [BH][ceil(n_kv / 2) + 1], [BH][n_flat n_ns]
};

hipError_t launch_backward(const BwdLaunch& L, hipStream_t stream);

// Largest number of query blocks the selection kernel handles per head.
constexpr int kMaxBlocksPerHead = 4096;

}  // namespace isa
