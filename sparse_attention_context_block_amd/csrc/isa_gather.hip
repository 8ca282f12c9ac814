// Gather + concat of Context Pre-Selection, materialised ([notes] key design
// 1; [summary] 3 "Pre-Selection": the kept context blocks are gathered and
// concatenated after the source into K_new, V_new).
//
// K_new[t * b + r] = K[src(t) * b + r] with src(t) = t for the n_src source
// blocks and n_src + sel[t - n_src] for the kept context blocks.  One
// workgroup copies one 64-row block of K and of V with 16-byte loads and
// stores (fully coalesced: a block is one contiguous region of b * D
// elements in both layouts).
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint4* __restrict__ K, const uint4* __restrict__ V, const int32_t* __restrict__ sel,
    int n_src, int k, int64_t head_chunks, int64_t head_chunks_new, int block_chunks,
    uint4* __restrict__ K_new, uint4* __restrict__ V_new) {
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int src = t < n_src ? t : n_src + sel[bh * k + (t - n_src)];
  const uint4* ks = K + bh * head_chunks + (int64_t)src * block_chunks;
  const uint4* vs = V + bh * head_chunks + (int64_t)src * block_chunks;
  uint4* kd = K_new + bh * head_chunks_new + (int64_t)t * block_chunks;
  uint4* vd = V_new + bh * head_chunks_new + (int64_t)t * block_chunks;
  for (int i = threadIdx.x; i < block_chunks; i += kThreads) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace

hipError_t launch_gather(const void* K, const void* V, const int32_t* sel, isa_dtype_t dtype,
                         int BH, int N, int D, int n_src, int k, int block, void* K_new,
                         void* V_new, hipStream_t stream) {
  const int n_kv = n_src + k;
  if (BH == 0 || n_kv == 0) return hipSuccess;
  const int elt = dtype == ISA_DTYPE_BF16 ? 2 : 4;
  const int64_t row_chunks = (int64_t)D * elt / 16;
  const int block_chunks = (int)(row_chunks * block);
  const int64_t head_chunks = (int64_t)N * row_chunks;
  const int64_t head_chunks_new = (int64_t)n_kv * block * row_chunks;
  hipLaunchKernelGGL(gather_kernel, dim3(n_kv, BH), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(K), static_cast<const uint4*>(V), sel, n_src, k,
                     head_chunks, head_chunks_new, block_chunks, static_cast<uint4*>(K_new),
                     static_cast<uint4*>(V_new));
  return hipGetLastError();
}

}  // namespace isa
