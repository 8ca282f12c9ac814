// C-ABI host layer: plan validation, workspace layout and the launch
// sequence of the ISA forward ([notes] overall framework: pooling attention,
// Context Pre-Selection, grouping by query sharpness, the exact and the 0-th
// order Taylor paths, merge).  Host code only (plus the device array that
// serves as isa_forward_noalloc's workspace); every step of the path runs in
// the device kernels of the other files.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <atomic>
#include <new>
#include <string.h>

#include "isa_debug.h"
#include "isa_internal.h"
#include "isa_testing.h"

namespace isa {
std::atomic<uint32_t> g_debug_flags{0};
uint32_t debug_flags() { return g_debug_flags.load(std::memory_order_relaxed); }
}  // namespace isa

using namespace isa;

struct WorkspaceLayout {
  size_t qc, kc, kc_lp, vc_lp, rowmax, rowsum, sharpness, ctx_score, sel, flat, sharp, kv_tab;
  size_t ns;          // only with n_ns > 0 and n_flat > 0
  size_t qr, kr;      // only with the rotary embedding: rotated Q, K
  size_t total;
};

struct isa_plan_s {
  isa_plan_desc_t d;
  isa_plan_info_t info;
  WorkspaceLayout ws;
  int64_t N;
  int32_t BH;
  BlockGrid grid;   // token layout of the blocks
  int32_t half_shift;  // log2(block / 32): the attention kernels' 32-row slices per block
  bool aligned;     // L_src and L_ctx are multiples of the block length
  bool rope;        // decoupled rotary embedding of Q and K
  RopeFreq freq;    // its pair frequencies base^(-2i/D)
};

namespace {

thread_local int g_last_hip_error = 0;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

isa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return ISA_OK;
  g_last_hip_error = (int)e;
  return ISA_ERR_HIP;
}

// Failure injection (isa_testing_fail_launch): launches to let through before
// the failing one, and the error it reports (0: disarmed).
std::atomic<int32_t> g_fail_skip{0};
std::atomic<int32_t> g_fail_error{0};

// hipSuccess to go ahead with the next launch, or the injected error (the
// launch is then not issued and the hook disarms).
hipError_t injected_failure() {
  if (g_fail_error.load(std::memory_order_relaxed) == 0) return hipSuccess;
  if (g_fail_skip.load(std::memory_order_relaxed) > 0) {
    g_fail_skip.fetch_sub(1, std::memory_order_relaxed);
    return hipSuccess;
  }
  return (hipError_t)g_fail_error.exchange(0, std::memory_order_relaxed);
}

#define ISA_LAUNCH(expr)                                     \
  do {                                                       \
    hipError_t e_ = injected_failure();                      \
    if (e_ == hipSuccess) e_ = (expr);                       \
    isa_status_t s_ = hip_status(e_);                        \
    if (s_ != ISA_OK) return s_;                             \
  } while (0)

bool log_enabled() {
  const char* v = getenv("ISA_LOG");
  return v && *v && strcmp(v, "0") != 0;
}

size_t elt_size(isa_dtype_t t) { return t == ISA_DTYPE_BF16 ? 2 : 4; }

// Context blocks kept: ceil(alpha_s * n_ctx); query blocks sent to the Taylor
// path: floor(alpha_f * n_q).  The 1e-6 guard keeps a product that is an
// integer up to double rounding on that integer.
int64_t select_count(double alpha_s, int64_t n_ctx) {
  int64_t k = (int64_t)ceil(alpha_s * (double)n_ctx - 1e-6);
  return k < 0 ? 0 : (k > n_ctx ? n_ctx : k);
}
int64_t flat_count(double alpha_f, int64_t n_q) {
  int64_t n = (int64_t)floor(alpha_f * (double)n_q + 1e-6);
  return n < 0 ? 0 : (n > n_q ? n_q : n);
}
// K_new blocks computed exactly per flat query block: ceil(alpha_ns * n_kv).
int64_t ns_count(double alpha_ns, int64_t n_kv) {
  int64_t n = (int64_t)ceil(alpha_ns * (double)n_kv - 1e-6);
  return n < 0 ? 0 : (n > n_kv ? n_kv : n);
}

bool ratio_ok(double a) { return a >= 0.0 && a <= 1.0; }  // false for NaN

}  // namespace

extern "C" {

const char* isa_status_string(isa_status_t s) {
  switch (s) {
    case ISA_OK: return "ISA_OK";
    case ISA_ERR_INVALID_ARG: return "ISA_ERR_INVALID_ARG: invalid argument";
    case ISA_ERR_UNSUPPORTED: return "ISA_ERR_UNSUPPORTED: valid but not supported by this build";
    case ISA_ERR_WORKSPACE: return "ISA_ERR_WORKSPACE: workspace missing or too small";
    case ISA_ERR_HIP: return "ISA_ERR_HIP: a HIP call failed";
  }
  return "ISA_ERR_UNKNOWN: unknown status";
}

int isa_last_hip_error(void) { return g_last_hip_error; }

isa_status_t isa_debug_set_flags(uint32_t flags) {
  static_assert(isa::kDebugGlobalTables == ISA_DEBUG_GLOBAL_TABLES &&
                    isa::kDebug4WaveExact == ISA_DEBUG_4WAVE_EXACT &&
                    isa::kDebugPingPongExact == ISA_DEBUG_PINGPONG_EXACT,
                "debug flag bits");
  if (flags & ~isa::kDebugAll) return ISA_ERR_INVALID_ARG;
  if ((flags & isa::kDebug4WaveExact) && (flags & isa::kDebugPingPongExact))
    return ISA_ERR_INVALID_ARG;
  isa::g_debug_flags.store(flags, std::memory_order_relaxed);
  return ISA_OK;
}

isa_status_t isa_testing_fail_launch(int32_t skip, int32_t hip_error) {
  if (skip < 0 || hip_error < 0) return ISA_ERR_INVALID_ARG;
  g_fail_error.store(0, std::memory_order_relaxed);
  g_fail_skip.store(skip, std::memory_order_relaxed);
  g_fail_error.store(hip_error, std::memory_order_relaxed);
  return ISA_OK;
}

isa_status_t isa_plan_create(isa_plan_t* out, const isa_plan_desc_t* desc) {
  if (!out || !desc) return ISA_ERR_INVALID_ARG;
  *out = nullptr;
  const isa_plan_desc_t d = *desc;
  if (d.B < 0 || d.H < 0 || d.D < 1 || d.block < 1 || d.L_src < 1 || d.L_ctx < 0)
    return ISA_ERR_INVALID_ARG;
  if (!ratio_ok(d.alpha_s) || !ratio_ok(d.alpha_f) || !ratio_ok(d.alpha_ns))
    return ISA_ERR_INVALID_ARG;
  if (!(d.rope_base >= 0.0) || isinf(d.rope_base)) return ISA_ERR_INVALID_ARG;
  if (d.dtype != ISA_DTYPE_BF16 && d.dtype != ISA_DTYPE_FP32) return ISA_ERR_INVALID_ARG;
  if ((int64_t)d.L_src + d.L_ctx > INT32_MAX / 2) return ISA_ERR_UNSUPPORTED;
  if ((d.block != 32 && d.block != 64 && d.block != 128) || (d.D != 64 && d.D != 128))
    return ISA_ERR_UNSUPPORTED;
  const int64_t BH = (int64_t)d.B * d.H;
  if (BH > 65535) return ISA_ERR_UNSUPPORTED;

  isa_plan_s* p = new (std::nothrow) isa_plan_s;
  if (!p) return ISA_ERR_INVALID_ARG;
  memset(p, 0, sizeof(*p));
  p->d = d;
  p->BH = (int32_t)BH;
  p->N = (int64_t)d.L_src + d.L_ctx;
  p->aligned = d.L_src % d.block == 0 && d.L_ctx % d.block == 0;
  p->half_shift = d.block == 32 ? 0 : (d.block == 64 ? 1 : 2);
  p->rope = d.rope_base > 0.0;
  // pair i of D/2 turns by pos * base^(-2i/D) (the exponent as -2 i / D in double)
  for (int i = 0; p->rope && i < d.D / 2; ++i)
    p->freq.inv_freq[i] = pow(d.rope_base, -2.0 * i / d.D);
  isa_plan_info_t& in = p->info;
  in.n_src_blocks = (d.L_src + d.block - 1) / d.block;
  in.n_ctx_blocks = (d.L_ctx + d.block - 1) / d.block;
  in.n_q_blocks = in.n_src_blocks + in.n_ctx_blocks;
  if (in.n_q_blocks > kMaxBlocksPerHead) {
    delete p;
    return ISA_ERR_UNSUPPORTED;
  }
  in.k = select_count(d.alpha_s, in.n_ctx_blocks);
  in.n_kv_blocks = in.n_src_blocks + in.k;
  in.l_new = (int64_t)d.L_src + in.k * d.block;
  in.n_flat = flat_count(d.alpha_f, in.n_q_blocks);
  in.n_sharp = in.n_q_blocks - in.n_flat;
  in.n_ns = ns_count(d.alpha_ns, in.n_kv_blocks);
  // the block-mask kernel is built for 64-token blocks
  if (in.n_ns > 0 && in.n_flat > 0 && d.block != kBlock) {
    delete p;
    return ISA_ERR_UNSUPPORTED;
  }
  p->grid.L_src = d.L_src;
  p->grid.n_src = (int32_t)in.n_src_blocks;
  p->grid.N = (int32_t)p->N;
  p->grid.len = d.block;

  WorkspaceLayout& w = p->ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t pooled = (size_t)BH * in.n_q_blocks * d.D;
  w.qc = take(pooled * sizeof(double));
  w.kc = take(pooled * sizeof(double));
  w.kc_lp = take(pooled * elt_size(d.dtype));
  w.vc_lp = take(pooled * elt_size(d.dtype));
  w.rowmax = take((size_t)BH * in.n_q_blocks * sizeof(double));
  w.rowsum = take((size_t)BH * in.n_q_blocks * sizeof(double));
  w.sharpness = take((size_t)BH * in.n_q_blocks * sizeof(double));
  w.ctx_score = take((size_t)BH * in.n_ctx_blocks * sizeof(double));
  w.sel = take((size_t)BH * in.k * sizeof(int32_t));
  w.flat = take((size_t)BH * in.n_flat * sizeof(int32_t));
  w.sharp = take((size_t)BH * in.n_sharp * sizeof(int32_t));
  w.kv_tab = take((size_t)BH * in.n_kv_blocks * sizeof(int32_t));
  const bool masked = in.n_ns > 0 && in.n_flat > 0;
  w.ns = masked ? take((size_t)BH * in.n_flat * in.n_ns * sizeof(int32_t)) : 0;
  const size_t tokens = (size_t)BH * p->N * d.D * elt_size(d.dtype);
  w.qr = p->rope ? take(tokens) : 0;
  w.kr = p->rope ? take(tokens) : 0;
  w.total = off;
  in.workspace_bytes = off;
  if (log_enabled())
    fprintf(stderr,
            "[isa] plan B=%d H=%d L_src=%d L_ctx=%d D=%d b=%d alpha_s=%g alpha_f=%g "
            "alpha_ns=%g %s rope_base=%g: n_src=%lld n_ctx=%lld k=%lld N_K'=%lld L_new=%lld "
            "n_flat=%lld n_sharp=%lld n_ns=%lld workspace=%zu bytes\n",
            d.B, d.H, d.L_src, d.L_ctx, d.D, d.block, d.alpha_s, d.alpha_f, d.alpha_ns,
            d.dtype == ISA_DTYPE_BF16 ? "bf16" : "fp32", d.rope_base,
            (long long)in.n_src_blocks, (long long)in.n_ctx_blocks, (long long)in.k,
            (long long)in.n_kv_blocks, (long long)in.l_new, (long long)in.n_flat,
            (long long)in.n_sharp, (long long)in.n_ns, in.workspace_bytes);
  *out = p;
  return ISA_OK;
}

isa_status_t isa_plan_get_info(isa_plan_t plan, isa_plan_info_t* info) {
  if (!plan || !info) return ISA_ERR_INVALID_ARG;
  *info = plan->info;
  return ISA_OK;
}

isa_status_t isa_plan_destroy(isa_plan_t plan) {
  delete plan;
  return ISA_OK;
}

}  // extern "C"

namespace {

isa_status_t record(void* const* events, int i, hipStream_t s) {
  if (!events) return ISA_OK;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), s));
}

isa_status_t forward_impl(isa_plan_t plan, const void* Q, const void* K, const void* V, void* O,
                          float* lse, const isa_aux_t* aux, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events) {
  if (!plan) return ISA_ERR_INVALID_ARG;
  if (plan->BH == 0) return ISA_OK;
  if (!Q || !K || !V || !O) return ISA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ISA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < plan->ws.total || !aligned16(workspace))
    return ISA_ERR_WORKSPACE;
  const isa_plan_desc_t& d = plan->d;
  const isa_plan_info_t& in = plan->info;
  const WorkspaceLayout& L = plan->ws;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  double* qc = reinterpret_cast<double*>(w + L.qc);
  double* kc = reinterpret_cast<double*>(w + L.kc);
  void* kc_lp = w + L.kc_lp;
  void* vc_lp = w + L.vc_lp;
  double* rowmax = reinterpret_cast<double*>(w + L.rowmax);
  double* rowsum = reinterpret_cast<double*>(w + L.rowsum);
  double* sharpness = (aux && aux->sharpness) ? aux->sharpness
                                              : reinterpret_cast<double*>(w + L.sharpness);
  double* ctx_score = (aux && aux->ctx_score) ? aux->ctx_score
                                              : reinterpret_cast<double*>(w + L.ctx_score);
  int32_t* sel = (aux && aux->sel) ? aux->sel : reinterpret_cast<int32_t*>(w + L.sel);
  int32_t* flat = (aux && aux->flat) ? aux->flat : reinterpret_cast<int32_t*>(w + L.flat);
  int32_t* sharp = (aux && aux->sharp) ? aux->sharp : reinterpret_cast<int32_t*>(w + L.sharp);
  int32_t* kv_tab = reinterpret_cast<int32_t*>(w + L.kv_tab);
  const bool masked = in.n_ns > 0 && in.n_flat > 0;
  int32_t* ns = !masked ? nullptr
                        : (aux && aux->ns) ? aux->ns : reinterpret_cast<int32_t*>(w + L.ns);
  const int BH = plan->BH, D = d.D, N = (int)plan->N;
  const int n_q = (int)in.n_q_blocks, n_src = (int)in.n_src_blocks, n_ctx = (int)in.n_ctx_blocks;

  isa_status_t st;
#define ISA_STAGE(i)                                   \
  do {                                                 \
    if ((st = record(events, (i), s)) != ISA_OK) return st; \
  } while (0)
  ISA_STAGE(0);
  // 0. with the decoupled rotary embedding, the pooling kernel rotates Q and K
  //    into the workspace and every later step reads the rotated copies
  void* qr = plan->rope ? w + L.qr : nullptr;
  void* kr = plan->rope ? w + L.kr : nullptr;
  // 1. pooling attention: block means, then the coarse map's row statistics
  //    and sharpness, and the context column means (all fp64)
  ISA_LAUNCH(launch_pool(Q, K, V, d.dtype, BH, N, D, d.L_src, n_src, n_q, d.block, qc, kc,
                         kc_lp, vc_lp, qr, kr, plan->rope ? &plan->freq : nullptr, s));
  if (plan->rope) {
    Q = qr;
    K = kr;
  }
  ISA_STAGE(1);
  ISA_LAUNCH(launch_coarse_rowstats(qc, kc, BH, n_q, D, rowmax, rowsum, sharpness, s));
  ISA_STAGE(2);
  ISA_LAUNCH(launch_coarse_colsum(qc, kc, rowmax, rowsum, BH, n_q, n_src, n_ctx, D, ctx_score,
                                  s));
  ISA_STAGE(3);
  // 2-3. TopK of the context blocks (block table of K_new) and routing
  ISA_LAUNCH(launch_select_route(ctx_score, sharpness, BH, n_src, n_ctx, n_q, (int)in.k,
                                 (int)in.n_flat, sel, flat, sharp, kv_tab, s));
  //    block mask of the flat query blocks: their top n_ns blocks of K_new
  if (masked)
    ISA_LAUNCH(launch_ns_select(qc, kc, flat, kv_tab, BH, n_q, D, (int)in.n_flat,
                                (int)in.n_kv_blocks, (int)in.n_ns, ns, s));
  ISA_STAGE(4);

  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  // 4a. exact path: sharp query blocks over the rows of K_new
  AttnParams pe;
  memset(&pe, 0, sizeof(pe));
  pe.q = Q;
  pe.k = K;
  pe.v = V;
  pe.o = O;
  pe.lse = lse;
  // (both lists are read in 32-row slices, 2^half_shift per block)
  const int hs = plan->half_shift;
  pe.q_tab = sharp;
  pe.q_tab_stride = in.n_sharp;
  pe.n_q_slices = (int)in.n_sharp << hs;
  pe.n_q_entries = (pe.n_q_slices + 1) / 2;
  pe.kv_tab = kv_tab;
  pe.kv_tab_stride = in.n_kv_blocks;
  pe.kv_rows = 32 * ((int)in.n_kv_blocks << hs);
  pe.kv_row_table = 0;
  pe.half_shift = hs;
  pe.q_head_stride = plan->N * D;
  pe.kv_head_stride = plan->N * D;
  pe.lse_head_stride = plan->N;
  pe.BH = BH;
  pe.D = D;
  pe.scale_log2 = scale_log2;
  pe.lse_offset = 0.0f;
  pe.grid = plan->grid;
  ISA_LAUNCH(launch_attention(pe, d.dtype, s));
  ISA_STAGE(5);

  // 4b. 0-th order Taylor path: flat query blocks over the block means of the
  //     K_new blocks; every block holds b tokens, weight b.  With the block
  //     mask, each flat block's n_ns blocks enter token by token instead.
  if (masked) {
    FlatParams pf;
    memset(&pf, 0, sizeof(pf));
    pf.q = Q;
    pf.k = K;
    pf.v = V;
    pf.kc = kc_lp;
    pf.vc = vc_lp;
    pf.o = O;
    pf.lse = lse;
    pf.flat = flat;
    pf.kv_tab = kv_tab;
    pf.ns = ns;
    pf.n_flat = (int)in.n_flat;
    pf.n_kv = (int)in.n_kv_blocks;
    pf.n_ns = (int)in.n_ns;
    pf.q_head_stride = plan->N * D;
    pf.kv_head_stride = plan->N * D;
    pf.kc_head_stride = (int64_t)n_q * D;
    pf.lse_head_stride = plan->N;
    pf.BH = BH;
    pf.D = D;
    pf.scale_log2 = scale_log2;
    pf.exact_bias_log2 = (float)(-log2((double)d.block));
    pf.lse_offset = (float)log((double)d.block);
    pf.grid = plan->grid;
    ISA_LAUNCH(launch_attention_flat(pf, d.dtype, s));
    ISA_STAGE(6);
    return ISA_OK;
  }
  AttnParams pt = pe;
  pt.k = kc_lp;
  pt.v = vc_lp;
  pt.q_tab = flat;
  pt.q_tab_stride = in.n_flat;
  pt.n_q_slices = (int)in.n_flat << hs;
  pt.n_q_entries = (pt.n_q_slices + 1) / 2;
  pt.kv_rows = (int)in.n_kv_blocks;
  pt.kv_row_table = 1;
  pt.kv_head_stride = (int64_t)n_q * D;
  pt.lse_offset = (float)log((double)d.block);
  ISA_LAUNCH(launch_attention(pt, d.dtype, s));
  ISA_STAGE(6);
#undef ISA_STAGE
  return ISA_OK;
}

// ---- the workspace of isa_forward_noalloc ----
// One copy per device: a device variable of this code object, reserved when
// the code object is loaded on a device.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current, and
// only that address is ever handed to a kernel.
constexpr size_t kStaticWorkspaceBytes = ISA_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The array's address on the device of `stream` (the current device for the
// NULL stream).  Concurrent first calls resolve the same address.
isa_status_t static_workspace(hipStream_t stream, void** out) {
  int cur = -1;
  isa_status_t st = hip_status(hipGetDevice(&cur));
  if (st != ISA_OK) return st;
  int dev = cur;
  if (stream && (st = hip_status(hipStreamGetDevice(stream, &dev))) != ISA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return ISA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (dev != cur && (st = hip_status(hipSetDevice(dev))) != ISA_OK) return st;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (dev != cur) {
      const isa_status_t back = hip_status(hipSetDevice(cur));
      if (st == ISA_OK) st = back;
    }
    if (st != ISA_OK) return st;
    if (!p) return ISA_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ISA_OK;
}

}  // namespace

extern "C" {

isa_status_t isa_forward(isa_plan_t plan, const void* Q, const void* K, const void* V, void* O,
                         float* lse, const isa_aux_t* aux, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return forward_impl(plan, Q, K, V, O, lse, aux, workspace, workspace_bytes, stream, nullptr);
}

isa_status_t isa_forward_profiled(isa_plan_t plan, const void* Q, const void* K, const void* V,
                                  void* O, float* lse, const isa_aux_t* aux, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return ISA_ERR_INVALID_ARG;
  return forward_impl(plan, Q, K, V, O, lse, aux, workspace, workspace_bytes, stream, events);
}

isa_status_t isa_forward_noalloc(isa_plan_t plan, const void* Q, const void* K, const void* V,
                                 void* O, float* lse, const isa_aux_t* aux, void* stream) {
  if (!plan) return ISA_ERR_INVALID_ARG;
  if (plan->ws.total > kStaticWorkspaceBytes) return ISA_ERR_WORKSPACE;
  if (plan->BH == 0) return ISA_OK;
  void* ws = nullptr;
  const isa_status_t st = static_workspace(static_cast<hipStream_t>(stream), &ws);
  if (st != ISA_OK) return st;
  return forward_impl(plan, Q, K, V, O, lse, aux, ws, kStaticWorkspaceBytes, stream, nullptr);
}

isa_status_t isa_gather(isa_plan_t plan, const void* K, const void* V, const int32_t* sel,
                        void* K_new, void* V_new, void* stream) {
  if (!plan) return ISA_ERR_INVALID_ARG;
  if (plan->BH == 0) return ISA_OK;
  if (!K || !V || !K_new || !V_new || (!sel && plan->info.k > 0)) return ISA_ERR_INVALID_ARG;
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_new) || !aligned16(V_new))
    return ISA_ERR_INVALID_ARG;
  if (!plan->aligned) return ISA_ERR_UNSUPPORTED;  // K_new's length would depend on sel
  const isa_plan_desc_t& d = plan->d;
  ISA_LAUNCH(launch_gather(K, V, sel, d.dtype, plan->BH, (int)plan->N, d.D,
                           (int)plan->info.n_src_blocks, (int)plan->info.k, d.block, K_new, V_new,
                           static_cast<hipStream_t>(stream)));
  return ISA_OK;
}

isa_status_t isa_dense_forward(int32_t B, int32_t H, int32_t N, int32_t D, isa_dtype_t dtype,
                               const void* Q, const void* K, const void* V, void* O, float* lse,
                               void* stream) {
  if (B < 0 || H < 0 || N < 0 || D < 1) return ISA_ERR_INVALID_ARG;
  if (dtype != ISA_DTYPE_BF16 && dtype != ISA_DTYPE_FP32) return ISA_ERR_INVALID_ARG;
  if ((int64_t)B * H == 0 || N == 0) return ISA_OK;
  if (!Q || !K || !V || !O) return ISA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ISA_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || N % kBlock != 0 || (int64_t)B * H > 65535)
    return ISA_ERR_UNSUPPORTED;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = lse;
  p.n_q_entries = N / kBlock;
  p.n_q_slices = N / 32;
  p.kv_rows = N;
  p.kv_row_table = 0;
  p.half_shift = 1;
  p.q_head_stride = (int64_t)N * D;
  p.kv_head_stride = (int64_t)N * D;
  p.lse_head_stride = N;
  p.BH = B * H;
  p.D = D;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  p.grid.L_src = N;  // no context: a plain grid of whole 64-token blocks
  p.grid.n_src = N / kBlock;
  p.grid.N = N;
  p.grid.len = kBlock;
  ISA_LAUNCH(launch_attention(p, dtype, static_cast<hipStream_t>(stream)));
  return ISA_OK;
}

}  // extern "C"

namespace {

struct BwdLayout {
  size_t delta, kv_tab, iota, kc, vc, dkc, dvc;
  size_t qr, kr;  // rotary embedding only: the rotated Q and K
  // block mask only: exact-block tables of the flat blocks
  size_t ns_mask, tok_list, tok_cnt, fq_off, fq_list;
  size_t total;
};

BwdLayout bwd_layout(const isa_plan_s* p) {
  BwdLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t BH = (size_t)p->BH, n_kv = (size_t)p->info.n_kv_blocks, D = (size_t)p->d.D;
  w.delta = take(BH * (size_t)p->N * sizeof(float));
  w.kv_tab = take(BH * n_kv * sizeof(int32_t));
  w.iota = take(n_kv * sizeof(int32_t));
  w.kc = take(BH * n_kv * D * 2);
  w.vc = take(BH * n_kv * D * 2);
  w.dkc = take(BH * n_kv * D * sizeof(float));
  w.dvc = take(BH * n_kv * D * sizeof(float));
  const size_t tokens = BH * (size_t)p->N * D * elt_size(p->d.dtype);
  w.qr = p->rope ? take(tokens) : 0;
  w.kr = p->rope ? take(tokens) : 0;
  const size_t n_flat = (size_t)p->info.n_flat, n_ns = (size_t)p->info.n_ns;
  const bool masked = n_ns > 0 && n_flat > 0;
  const size_t words = (n_kv + 31) / 32, pairs = (n_flat + 1) / 2, kwg = (n_kv + 1) / 2;
  w.ns_mask = masked ? take(BH * n_flat * words * sizeof(uint32_t)) : 0;
  w.tok_list = masked ? take(BH * pairs * 2 * n_ns * sizeof(int32_t)) : 0;
  w.tok_cnt = masked ? take(BH * pairs * sizeof(int32_t)) : 0;
  w.fq_off = masked ? take(BH * (kwg + 1) * sizeof(int32_t)) : 0;
  w.fq_list = masked ? take(BH * n_flat * n_ns * sizeof(int32_t)) : 0;
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

size_t isa_backward_workspace_bytes(isa_plan_t plan) {
  if (!plan) return 0;
  return bwd_layout(plan).total;
}

isa_status_t isa_backward(isa_plan_t plan, const void* Q, const void* K, const void* V,
                          const void* O, const void* dO, const float* lse, const isa_aux_t* aux,
                          void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!plan) return ISA_ERR_INVALID_ARG;
  if (plan->BH == 0) return ISA_OK;
  const isa_plan_info_t& in = plan->info;
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !aux) return ISA_ERR_INVALID_ARG;
  const bool masked = in.n_ns > 0 && in.n_flat > 0;
  if ((in.k > 0 && !aux->sel) || (in.n_flat > 0 && !aux->flat) || (in.n_sharp > 0 && !aux->sharp) ||
      (masked && !aux->ns))
    return ISA_ERR_INVALID_ARG;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
  for (const void* q : ptrs)
    if (!aligned16(q)) return ISA_ERR_INVALID_ARG;
  if (plan->d.dtype != ISA_DTYPE_BF16) return ISA_ERR_UNSUPPORTED;
  const BwdLayout W = bwd_layout(plan);
  if (!workspace || workspace_bytes < W.total || !aligned16(workspace)) return ISA_ERR_WORKSPACE;
  char* w = static_cast<char*>(workspace);
  BwdLaunch L;
  L.BH = plan->BH;
  L.D = plan->d.D;
  L.N = (int)plan->N;
  L.L_src = plan->d.L_src;
  L.block = plan->d.block;
  L.n_src = (int)in.n_src_blocks;
  L.n_ctx = (int)in.n_ctx_blocks;
  L.k = (int)in.k;
  L.n_flat = (int)in.n_flat;
  L.n_sharp = (int)in.n_sharp;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int N = (int)plan->N, D = plan->d.D;
  if (plan->rope) {
    // the forward saw the rotated Q and K: rotate them again (bit-identical to
    // the forward's copies), differentiate at them, and turn dQ, dK back below
    ISA_LAUNCH(launch_rope_rotate(Q, w + W.qr, plan->d.dtype, plan->BH, N, D, plan->d.L_src,
                                  plan->freq, false, s));
    ISA_LAUNCH(launch_rope_rotate(K, w + W.kr, plan->d.dtype, plan->BH, N, D, plan->d.L_src,
                                  plan->freq, false, s));
    Q = w + W.qr;
    K = w + W.kr;
  }
  L.Q = static_cast<const bf16_bits*>(Q);
  L.K = static_cast<const bf16_bits*>(K);
  L.V = static_cast<const bf16_bits*>(V);
  L.O = static_cast<const bf16_bits*>(O);
  L.dO = static_cast<const bf16_bits*>(dO);
  L.lse = lse;
  L.sel = aux->sel;
  L.flat = aux->flat;
  L.sharp = aux->sharp;
  L.dQ = static_cast<bf16_bits*>(dQ);
  L.dK = static_cast<bf16_bits*>(dK);
  L.dV = static_cast<bf16_bits*>(dV);
  L.delta = reinterpret_cast<float*>(w + W.delta);
  L.kv_tab = reinterpret_cast<int32_t*>(w + W.kv_tab);
  L.iota = reinterpret_cast<int32_t*>(w + W.iota);
  L.kc = reinterpret_cast<bf16_bits*>(w + W.kc);
  L.vc = reinterpret_cast<bf16_bits*>(w + W.vc);
  L.dkc = reinterpret_cast<float*>(w + W.dkc);
  L.dvc = reinterpret_cast<float*>(w + W.dvc);
  L.n_ns = masked ? (int)in.n_ns : 0;
  L.ns = masked ? aux->ns : nullptr;
  L.ns_mask = masked ? reinterpret_cast<uint32_t*>(w + W.ns_mask) : nullptr;
  L.tok_list = masked ? reinterpret_cast<int32_t*>(w + W.tok_list) : nullptr;
  L.tok_cnt = masked ? reinterpret_cast<int32_t*>(w + W.tok_cnt) : nullptr;
  L.fq_off = masked ? reinterpret_cast<int32_t*>(w + W.fq_off) : nullptr;
  L.fq_list = masked ? reinterpret_cast<int32_t*>(w + W.fq_list) : nullptr;
  ISA_LAUNCH(launch_backward(L, s));
  if (plan->rope) {
    // dQ = R^T dQ', dK = R^T dK' (each pair turned back by its angle)
    ISA_LAUNCH(launch_rope_rotate(dQ, dQ, plan->d.dtype, plan->BH, N, D, plan->d.L_src,
                                  plan->freq, true, s));
    ISA_LAUNCH(launch_rope_rotate(dK, dK, plan->d.dtype, plan->BH, N, D, plan->d.L_src,
                                  plan->freq, true, s));
  }
  return ISA_OK;
}

}  // extern "C"
