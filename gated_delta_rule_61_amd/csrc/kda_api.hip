// kda_api.hip -- the C ABI (include/kda.h): argument validation, workspace
// layout and launch order.  No allocation, no synchronisation; all work goes
// on the caller's stream.
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.hpp"

// Device scratch of kda_chunk_fwd_noalloc: the segmented schedule's workspace
// in a file-scope array instead of caller memory.  Every GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` only
// names the symbol; its device address is taken per device below.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  g_last_hip = (int)e;
  return KDA_ERR_HIP;
}

// KDA_SYNC_DEBUG set and not "0" (read on every call): an entry point waits
// for its stream after its launches and reports a failure of its kernels
// there, as KDA_ERR_HIP, instead of leaving it to a later call.
bool sync_debug() {
  const char* e = getenv("KDA_SYNC_DEBUG");
  return e && e[0] && e[0] != '0';
}
int finish(hipError_t e, void* stream) {
  if (e == hipSuccess && sync_debug()) {
    e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  return hip_status(e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }

// head sizes the chunked kernels are built for
int check_chunk_dims(int B, int T, int H, int dk, int dv, int dt) {
  if (!valid_dtype(dt)) return KDA_ERR_DTYPE;
  if (B < 0 || T < 0 || H < 0) return KDA_ERR_SHAPE;
  if (dt == KDA_BF16 && !((dk == 128 && dv == 128) || (dk == 64 && dv == 64))) return KDA_ERR_SHAPE;
  if (dt == KDA_F32 && !((dk == 128 && dv == 128) || (dk == 64 && dv == 64))) return KDA_ERR_SHAPE;
  // 32-bit byte offsets inside one chunk of one tensor, 64-bit elsewhere
  if ((int64_t)H * dk * 64 * 4 > INT32_MAX || (int64_t)H * dv * 64 * 4 > INT32_MAX) return KDA_ERR_SHAPE;
  return KDA_OK;
}

// fp32 at d = 128: the two-launch fp32-operand path (a workspace is required)
bool f32_wide(int dk, int dt) { return dt == KDA_F32 && dk == 128; }
// bf16 at d = 64: the same path when the caller passes its workspace (the
// one-launch kernel's bf16 operands otherwise)
bool f32_ops_d64(int dk, int dt, int flags) { return dt == KDA_BF16 && dk == 64 && flags == 0; }

// The staged schedule and its single steps: as check_chunk_dims, except fp32
// at d = 128, whose operand tiles the staged kernels cannot hold.
int check_staged_dims(int B, int T, int H, int dk, int dv, int dt) {
  const int st = check_chunk_dims(B, T, H, dk, dv, dt);
  if (st) return st;
  return f32_wide(dk, dt) ? KDA_ERR_SHAPE : KDA_OK;
}

int check_step_dims(int N, int H, int dk, int dv, int dt) {
  if (!valid_dtype(dt)) return KDA_ERR_DTYPE;
  if (N < 0 || H < 0) return KDA_ERR_SHAPE;
  // one 256-thread workgroup per sequence and head, in one launch dimension
  // of at most 2^32 - 1 work-items
  if ((int64_t)N * H > KDA_STEP_MAX_HEADS) return KDA_ERR_SHAPE;
  if (!((dk == 128 && dv == 128) || (dk == 64 && dv == 64))) return KDA_ERR_SHAPE;
  return KDA_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StagedWs {
  size_t b, W, U, Delta, S, total;
};

StagedWs staged_layout(int B, int T, int H, int dk, int dv) {
  const size_t tok = (size_t)B * (size_t)T * (size_t)H;
  const size_t nch = ((size_t)T + 63) / 64;
  StagedWs w;
  size_t off = 0;
  w.b = off; off += round256(tok * dk * 4);
  w.W = off; off += round256(tok * dk * 4);
  w.U = off; off += round256(tok * dv * 4);
  w.Delta = off; off += round256(tok * dv * 4);
  w.S = off; off += round256((size_t)B * H * nch * dk * dv * 4);
  w.total = off;
  return w;
}

int env_nsplit() {
  const char* e = getenv("KDA_FUSED_NSPLIT");
  if (!e) return 0;
  const int v = atoi(e);
  return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 0;
}

// KDA_FUSED_PIPELINE=0 selects the non-pipelined fused schedule everywhere
// (kept for comparison and for checking one schedule against the other).
int env_pipeline() {
  const char* e = getenv("KDA_FUSED_PIPELINE");
  return (e && e[0] == '0') ? 0 : 1;
}

// Compute units of the current device (0 when there is none).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// Segments per sequence of the segmented prefill schedule for these sizes
// (0: one pass).  It applies where the pipelined kernel does; the count comes
// from the launch cost model, or from KDA_SEGMENTS (0 or 1: off; n >= 3:
// about n segments of equal length).
int segment_count(int B, int T, int H, int dk, int dv, int dtype, bool variant = false) {
  if (dtype != KDA_BF16 || dk != 128 || dv != 128) return 0;
  if (!variant && (env_nsplit() > 1 || !env_pipeline())) return 0;
  if ((int64_t)B * H <= 0 || T <= 0) return 0;
  const char* e = getenv("KDA_SEGMENTS");
  if (e) {
    const int want = atoi(e);
    if (want < 3) return 0;
    const int N = (T + 63) / 64;
    const int L = (N + want - 1) / want, P = (N + L - 1) / L;
    return P >= 3 ? P : 0;
  }
  return kda::prefill_segments(B * H, T, device_cus());
}

#define KDA_REQUIRE(cond, code) \
  do {                          \
    if (!(cond)) return (code); \
  } while (0)

// q, k, v, g, o are read/written as 16-byte vectors; beta, and g with a
// scalar gate, only need the alignment of their element type.  Without the
// delta rule beta is not read.
int check_tokens(const void* q, const void* k, const void* v, const void* g, const void* beta, const void* o,
                 int dtype, int flags = 0) {
  const bool need_beta = (flags & KDA_NO_DELTA) == 0;
  KDA_REQUIRE(q && k && v && g && o && (beta || !need_beta), KDA_ERR_NULL);
  const uintptr_t esz = dtype == KDA_BF16 ? 2u : 4u;
  const bool g_ok = (flags & KDA_GATE_SCALAR) ? reinterpret_cast<uintptr_t>(g) % esz == 0 : aligned16(g);
  KDA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && g_ok && aligned16(o) &&
              (!need_beta || (reinterpret_cast<uintptr_t>(beta) % esz) == 0), KDA_ERR_ALIGN);
  return KDA_OK;
}

bool valid_flags(int flags) { return (flags & ~(KDA_GATE_SCALAR | KDA_NO_DELTA)) == 0; }

// Per-device address of `scratch`, looked up once per device with that device
// current (hipGetSymbolAddress; no allocation).  nullptr and the HIP error on
// failure.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(hipStream_t stream, void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// sizes and dtype for which the prefill variants exist (the pipelined kernel)
bool variant_dims(int dk, int dv, int dt) { return dt == KDA_BF16 && dk == 128 && dv == 128; }

// The backward's flags: a variant, and KDA_STATES_SAVED on the chunked path.
bool valid_bwd_flags(int flags, int d_k, int d_v, int dtype) {
  if (!valid_flags(flags & ~KDA_STATES_SAVED)) return false;
  return !(flags & KDA_STATES_SAVED) || variant_dims(d_k, d_v, dtype);
}

}  // namespace

extern "C" {

int kda_version(void) { return 10000; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "unsupported or negative size (supported: d_k = d_v in {64,128}; the staged schedule: 64 for fp32)";
    case KDA_ERR_DTYPE: return "unsupported dtype";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return hipGetErrorString((hipError_t)g_last_hip);
    case KDA_ERR_ARG: return "invalid argument";
    case KDA_ERR_SCRATCH: return "these sizes need more device scratch than kda_chunk_fwd_noalloc holds "
                                 "(KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
    default: return "unknown status";
  }
}

int kda_last_hip_error(void) { return g_last_hip; }

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype) {
  if (check_chunk_dims(B, T, H, d_k, d_v, dtype) != KDA_OK) return 0;
  if (f32_wide(d_k, dtype) || f32_ops_d64(d_k, dtype, 0))
    return (int64_t)B * H * T == 0 ? 0 : kda::prefill_f32_workspace(B * H, T, d_k);
  return kda::prefill_segment_workspace(B * H, segment_count(B, T, H, d_k, d_v, dtype));
}

size_t kda_chunk_fwd_ex_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype, int flags) {
  if (flags == 0) return kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, dtype);
  if (!valid_flags(flags) || !variant_dims(d_k, d_v, dtype) || check_chunk_dims(B, T, H, d_k, d_v, dtype))
    return 0;
  return kda::prefill_segment_workspace(B * H, segment_count(B, T, H, d_k, d_v, dtype, true));
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return kda_chunk_fwd_ex(q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, dtype, 0, workspace,
                          workspace_bytes, stream);
}

int kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v, int dtype,
                     int flags, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_chunk_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_flags(flags) && (flags == 0 || variant_dims(d_k, d_v, dtype)), KDA_ERR_ARG);
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype, flags);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  if (f32_wide(d_k, dtype)) {
    // fp32 at d = 128: chunk quantities through the workspace, then the state pass
    kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, 0, 0, 0};
    if (T > 0) {
      KDA_REQUIRE(workspace && workspace_bytes >= kda::prefill_f32_workspace(B * H, T, d_k), KDA_ERR_WORKSPACE);
      KDA_REQUIRE(aligned16(workspace), KDA_ERR_ALIGN);
      a.ws = static_cast<float*>(workspace);
    }
    return finish(kda::launch_prefill_f32(a, (hipStream_t)stream), stream);
  }
  if (f32_ops_d64(d_k, dtype, flags) && T > 0 && workspace && aligned16(workspace) &&
      workspace_bytes >= kda::prefill_f32_workspace(B * H, T, d_k)) {
    // bf16 at d = 64 with its workspace: fp32 operands
    kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, 1, 0, 0};
    a.ws = static_cast<float*>(workspace);
    return finish(kda::launch_prefill_f32(a, (hipStream_t)stream), stream);
  }
  // (the variants run on the pipelined kernel whatever the schedule overrides say)
  kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, dtype == KDA_BF16,
                     flags ? 0 : env_nsplit(), flags ? 1 : env_pipeline()};
  a.variant = flags;
  // segmented schedule when the caller passes the workspace it needs
  const int nseg = segment_count(B, T, H, d_k, d_v, dtype, flags != 0);
  if (nseg >= 3 && workspace && aligned16(workspace) &&
      workspace_bytes >= kda::prefill_segment_workspace(B * H, nseg)) {
    a.nseg = nseg;
    a.seg_len = kda::prefill_segment_len(T, nseg);
    a.ws = static_cast<float*>(workspace);
  }
  return finish(kda::launch_fused(a, (hipStream_t)stream), stream);
}

int kda_chunk_fwd_save(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v, int dtype,
                       int flags, void* bwd_workspace, size_t bwd_workspace_bytes, void* stream) {
  int st = check_chunk_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_flags(flags) && variant_dims(d_k, d_v, dtype), KDA_ERR_ARG);
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype, flags);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  const size_t need = kda_chunk_bwd_ex_workspace_size(B, T, H, d_k, d_v, dtype, flags);
  KDA_REQUIRE(need == 0 || (bwd_workspace && bwd_workspace_bytes >= need), KDA_ERR_WORKSPACE);
  KDA_REQUIRE(aligned16(bwd_workspace), KDA_ERR_ALIGN);
  // the pipelined kernel, one pass, storing each chunk's entry state where
  // the backward's state pass would (the workspace's first region)
  kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, 1, 0, 1};
  a.variant = flags;
  a.states = T > 0 ? bwd_workspace : nullptr;
  return finish(kda::launch_fused(a, (hipStream_t)stream), stream);
}

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v, int dtype,
                          void* stream) {
  int st = check_chunk_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  const size_t need = kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, dtype);
  KDA_REQUIRE(need <= (size_t)KDA_NOALLOC_SCRATCH_BYTES, KDA_ERR_SCRATCH);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return kda_chunk_fwd(q, k, v, g, beta, S0, o, S_T, B, T, H, d_k, d_v, dtype, ws, need, stream);
}

int kda_varlen_schedule(const int32_t* cu_seqlens, int N, int T_total, int32_t* seq_order, void* stream) {
  KDA_REQUIRE(N >= 0 && T_total >= 0, KDA_ERR_SHAPE);
  KDA_REQUIRE(N <= kda::kMaxScheduleSeqs, KDA_ERR_SHAPE);
  if (N == 0) return KDA_OK;
  KDA_REQUIRE(cu_seqlens && seq_order, KDA_ERR_NULL);
  KDA_REQUIRE((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) == 0 && (reinterpret_cast<uintptr_t>(seq_order) & 3u) == 0,
              KDA_ERR_ALIGN);
  return finish(kda::launch_varlen_schedule(cu_seqlens, N, T_total, seq_order, (hipStream_t)stream), stream);
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* S0, void* o, float* S_T, const int32_t* cu_seqlens,
                         const int32_t* seq_order, int N, int T_total, int H, int d_k, int d_v, int dtype,
                         int flags, void* stream) {
  return kda_chunk_fwd_varlen_ws(q, k, v, g, beta, S0, o, S_T, cu_seqlens, seq_order, N, T_total, H, d_k, d_v,
                                 dtype, flags, nullptr, 0, stream);
}

size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v, int dtype, int flags) {
  if (check_chunk_dims(N, T_total, H, d_k, d_v, dtype) || !valid_flags(flags) || !variant_dims(d_k, d_v, dtype))
    return 0;
  if ((int64_t)N * H == 0) return 0;
  return kda::varlen_segments(N, T_total, H, device_cus()).bytes;
}

int kda_chunk_fwd_varlen_ws(const void* q, const void* k, const void* v, const void* g, const void* beta,
                            const float* S0, void* o, float* S_T, const int32_t* cu_seqlens,
                            const int32_t* seq_order, int N, int T_total, int H, int d_k, int d_v, int dtype,
                            int flags, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_chunk_dims(N, T_total, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_flags(flags) && variant_dims(d_k, d_v, dtype), KDA_ERR_ARG);
  if ((int64_t)N * H == 0) return KDA_OK;
  KDA_REQUIRE(cu_seqlens != nullptr, KDA_ERR_NULL);
  KDA_REQUIRE((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) == 0 && (reinterpret_cast<uintptr_t>(seq_order) & 3u) == 0,
              KDA_ERR_ALIGN);
  if (T_total > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype, flags);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, N, T_total, H, d_k, d_v, 1, 0, 1};
  a.variant = flags;
  a.cu_seqlens = cu_seqlens;
  a.seq_order = seq_order;
  // segmented schedule when the caller passes the workspace it needs
  const kda::VarlenSeg vs = kda::varlen_segments(N, T_total, H, device_cus());
  if (vs.L > 0 && workspace && aligned16(workspace) && workspace_bytes >= vs.bytes) {
    a.plan = static_cast<int*>(workspace);
    a.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + vs.plan_bytes);
    a.seg_len = vs.L;
    a.plan_j1 = vs.j1;
    a.plan_j3 = vs.j3;
    a.plan_ns = vs.ns;
  }
  return finish(kda::launch_fused(a, (hipStream_t)stream), stream);
}

int kda_chunk_fwd_varlen_save(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const float* S0, void* o, float* S_T, const int32_t* cu_seqlens,
                              const int32_t* seq_order, int N, int T_total, int H, int d_k, int d_v, int dtype,
                              int flags, void* bwd_workspace, size_t bwd_workspace_bytes, void* stream) {
  int st = check_chunk_dims(N, T_total, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_flags(flags) && variant_dims(d_k, d_v, dtype), KDA_ERR_ARG);
  if ((int64_t)N * H == 0) return KDA_OK;
  KDA_REQUIRE(cu_seqlens != nullptr, KDA_ERR_NULL);
  KDA_REQUIRE((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) == 0 && (reinterpret_cast<uintptr_t>(seq_order) & 3u) == 0,
              KDA_ERR_ALIGN);
  if (T_total > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype, flags);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  const size_t need = kda_chunk_bwd_varlen_workspace_size(N, T_total, H, d_k, d_v, dtype, flags);
  KDA_REQUIRE(need == 0 || (bwd_workspace && bwd_workspace_bytes >= need), KDA_ERR_WORKSPACE);
  KDA_REQUIRE(aligned16(bwd_workspace), KDA_ERR_ALIGN);
  // one pass, each chunk's entry state into the backward's slot layout
  kda::PrefillArgs a{q, k, v, g, beta, S0, o, S_T, N, T_total, H, d_k, d_v, 1, 0, 1};
  a.variant = flags;
  a.cu_seqlens = cu_seqlens;
  a.seq_order = seq_order;
  a.states = T_total > 0 ? bwd_workspace : nullptr;
  return finish(kda::launch_fused(a, (hipStream_t)stream), stream);
}

size_t kda_chunk_bwd_ex_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype, int flags) {
  if (!valid_bwd_flags(flags, d_k, d_v, dtype)) return 0;
  if (check_chunk_dims(B, T, H, d_k, d_v, dtype) != KDA_OK) return 0;
  if (!variant_dims(d_k, d_v, dtype)) return kda::backward_tok_workspace(B, T, H, d_k);
  size_t n = kda::backward_workspace(B * H, T);
  // scalar gate: the broadcast gate (bf16) and the per-channel dg (fp32), [B,T,H,d_k] each
  if (flags & KDA_GATE_SCALAR) n += (size_t)B * T * H * d_k * (2 + 4);
  return n;
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype) {
  return kda_chunk_bwd_ex_workspace_size(B, T, H, d_k, d_v, dtype, 0);
}

int kda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, const float* S0,
                     const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                     float* dS0, int B, int T, int H, int d_k, int d_v, int dtype, int flags, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_chunk_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_bwd_flags(flags, d_k, d_v, dtype), KDA_ERR_ARG);
  const bool sg = (flags & KDA_GATE_SCALAR) != 0, nd = (flags & KDA_NO_DELTA) != 0;
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    st = check_tokens(q, k, v, g, beta, dO, dtype, flags);
    if (st) return st;
    KDA_REQUIRE(dq && dk && dv && dg && (dbeta || nd), KDA_ERR_NULL);
    KDA_REQUIRE(aligned16(dq) && aligned16(dk) && aligned16(dv) && (sg || aligned16(dg)) &&
                (reinterpret_cast<uintptr_t>(dg) & 1u) == 0 && (reinterpret_cast<uintptr_t>(dbeta) & 1u) == 0,
                KDA_ERR_ALIGN);
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(dS_T) && aligned16(dS0), KDA_ERR_ALIGN);
  const size_t need = kda_chunk_bwd_ex_workspace_size(B, T, H, d_k, d_v, dtype, flags);
  KDA_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), KDA_ERR_WORKSPACE);
  KDA_REQUIRE(aligned16(workspace), KDA_ERR_ALIGN);
  if (!variant_dims(d_k, d_v, dtype)) {
    // fp32, or d = 64: the token recurrence's reverse mode
    kda::BackwardArgs a{q, k, v, g, nd ? nullptr : beta, S0, dO, dS_T, dq, dk, dv, dg, nd ? nullptr : dbeta, dS0,
                        B, T, H, nullptr, nullptr, nullptr, nullptr, flags, nullptr, 0};
    return finish(kda::launch_backward_tok(a, d_k, dtype == KDA_BF16, workspace, (hipStream_t)stream), stream);
  }
  // workspace: chunk states, chunk-end adjoints (bf16 d_k x d_v each), the
  // per-chunk operand blocks; then (scalar gate) the broadcast gate and the
  // per-channel dg
  char* ws = static_cast<char*>(workspace);
  const size_t nst = (size_t)B * H * (size_t)((T + 63) / 64) * d_k * d_v * 2;
  const size_t base = kda::backward_workspace(B * H, T);
  const int64_t rows = (int64_t)B * T * H;
  void* gfull = ws + base;
  float* dg32 = reinterpret_cast<float*>(ws + base + (size_t)rows * d_k * 2);
  kda::BackwardArgs a{q, k, v, sg ? gfull : g, nd ? nullptr : beta, S0, dO, dS_T, dq, dk, dv, dg,
                      nd ? nullptr : dbeta, dS0, B, T, H, workspace, ws + nst, ws + 2 * nst,
                      sg ? dg32 : nullptr, nd ? kda::kVarNoDelta : 0, nullptr, 0,
                      (flags & KDA_STATES_SAVED) ? 1 : 0};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (sg && T > 0 && (e = kda::launch_gate_expand(g, gfull, rows, s)) != hipSuccess) return hip_status(e);
  if ((e = kda::launch_backward(a, s)) != hipSuccess) return hip_status(e);
  if (sg && T > 0) return finish(kda::launch_gate_reduce(dg32, dg, rows, s), stream);
  return finish(hipSuccess, stream);
}

size_t kda_chunk_bwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v, int dtype, int flags) {
  if (!valid_bwd_flags(flags, d_k, d_v, dtype)) return 0;
  if (check_chunk_dims(N, T_total, H, d_k, d_v, dtype) != KDA_OK || !variant_dims(d_k, d_v, dtype)) return 0;
  if ((int64_t)N * H == 0 || T_total == 0) return 0;
  size_t n = kda::backward_varlen_workspace(N, T_total, H);
  if (flags & KDA_GATE_SCALAR) n += (size_t)T_total * H * d_k * (2 + 4);
  return n;
}

int kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dg,
                         void* dbeta, float* dS0, const int32_t* cu_seqlens, int N, int T_total, int H, int d_k,
                         int d_v, int dtype, int flags, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_chunk_dims(N, T_total, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_bwd_flags(flags, d_k, d_v, dtype) && variant_dims(d_k, d_v, dtype), KDA_ERR_ARG);
  const bool sg = (flags & KDA_GATE_SCALAR) != 0, nd = (flags & KDA_NO_DELTA) != 0;
  if ((int64_t)N * H == 0) return KDA_OK;
  KDA_REQUIRE(cu_seqlens != nullptr, KDA_ERR_NULL);
  KDA_REQUIRE((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) == 0, KDA_ERR_ALIGN);
  if (T_total > 0) {
    st = check_tokens(q, k, v, g, beta, dO, dtype, flags);
    if (st) return st;
    KDA_REQUIRE(dq && dk && dv && dg && (dbeta || nd), KDA_ERR_NULL);
    KDA_REQUIRE(aligned16(dq) && aligned16(dk) && aligned16(dv) && (sg || aligned16(dg)) &&
                (reinterpret_cast<uintptr_t>(dg) & 1u) == 0 && (reinterpret_cast<uintptr_t>(dbeta) & 1u) == 0,
                KDA_ERR_ALIGN);
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(dS_T) && aligned16(dS0), KDA_ERR_ALIGN);
  const size_t need = kda_chunk_bwd_varlen_workspace_size(N, T_total, H, d_k, d_v, dtype, flags);
  KDA_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), KDA_ERR_WORKSPACE);
  KDA_REQUIRE(aligned16(workspace), KDA_ERR_ALIGN);
  // workspace: chunk states, chunk-end adjoints, operand blocks (nslots x H
  // blocks each); then (scalar gate) the broadcast gate and the per-channel dg
  char* ws = static_cast<char*>(workspace);
  const int nslots = kda::backward_varlen_slots(N, T_total);
  const size_t nst = (size_t)nslots * H * d_k * d_v * 2;
  const size_t base = kda::backward_varlen_workspace(N, T_total, H);
  const int64_t rows = (int64_t)T_total * H;
  void* gfull = ws + base;
  float* dg32 = reinterpret_cast<float*>(ws + base + (size_t)rows * d_k * 2);
  kda::BackwardArgs a{q, k, v, sg ? gfull : g, nd ? nullptr : beta, S0, dO, dS_T, dq, dk, dv, dg,
                      nd ? nullptr : dbeta, dS0, N, T_total, H, workspace, ws + nst, ws + 2 * nst,
                      sg ? dg32 : nullptr, nd ? kda::kVarNoDelta : 0, cu_seqlens, nslots,
                      (flags & KDA_STATES_SAVED) ? 1 : 0};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (sg && T_total > 0 && (e = kda::launch_gate_expand(g, gfull, rows, s)) != hipSuccess) return hip_status(e);
  if ((e = kda::launch_backward(a, s)) != hipSuccess) return hip_status(e);
  if (sg && T_total > 0) return finish(kda::launch_gate_reduce(dg32, dg, rows, s), stream);
  return finish(hipSuccess, stream);
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta, const float* S0,
                  const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                  float* dS0, int B, int T, int H, int d_k, int d_v, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return kda_chunk_bwd_ex(q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, B, T, H, d_k, d_v, dtype, 0,
                          workspace, workspace_bytes, stream);
}

size_t kda_chunk_fwd_staged_workspace_size(int B, int T, int H, int d_k, int d_v, int dtype) {
  if (check_staged_dims(B, T, H, d_k, d_v, dtype)) return 0;
  return staged_layout(B, T, H, d_k, d_v).total;
}

int kda_chunk_fwd_staged(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v,
                         int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_staged_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    st = check_tokens(q, k, v, g, beta, o, dtype);
    if (st) return st;
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  const StagedWs w = staged_layout(B, T, H, d_k, d_v);
  KDA_REQUIRE(workspace != nullptr && workspace_bytes >= w.total, KDA_ERR_WORKSPACE);
  KDA_REQUIRE(aligned16(workspace), KDA_ERR_ALIGN);
  char* ws = static_cast<char*>(workspace);
  kda::StageArgs a{q, k, v, g, beta, S0, o, S_T,
                   reinterpret_cast<float*>(ws + w.b), reinterpret_cast<float*>(ws + w.W),
                   reinterpret_cast<float*>(ws + w.U), reinterpret_cast<float*>(ws + w.Delta),
                   reinterpret_cast<float*>(ws + w.S), B, T, H, d_k, d_v, dtype == KDA_BF16};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kda::launch_stage_cumsum(a, s);
  if (e == hipSuccess) e = kda::launch_stage_ut(a, s);
  if (e == hipSuccess) e = kda::launch_stage_state(a, s);
  if (e == hipSuccess) e = kda::launch_stage_output(a, s);
  return finish(e, stream);
}

int kda_stage_cumsum(const void* g, float* b, int B, int T, int H, int d_k, int dtype, void* stream) {
  int st = check_staged_dims(B, T, H, d_k, d_k, dtype);
  if (st) return st;
  if ((int64_t)B * H * T == 0) return KDA_OK;
  KDA_REQUIRE(g && b, KDA_ERR_NULL);
  KDA_REQUIRE(aligned16(g) && aligned16(b), KDA_ERR_ALIGN);
  kda::StageArgs a{};
  a.g = g; a.b = b; a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_k; a.bf16 = dtype == KDA_BF16;
  return finish(kda::launch_stage_cumsum(a, (hipStream_t)stream), stream);
}

int kda_stage_ut(const void* k, const void* v, const void* beta, const float* b, float* W, float* U, int B,
                 int T, int H, int d_k, int d_v, int dtype, void* stream) {
  int st = check_staged_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  if ((int64_t)B * H * T == 0) return KDA_OK;
  KDA_REQUIRE(k && v && beta && b && W && U, KDA_ERR_NULL);
  KDA_REQUIRE(aligned16(k) && aligned16(v) && aligned16(b) && aligned16(W) && aligned16(U), KDA_ERR_ALIGN);
  kda::StageArgs a{};
  a.k = k; a.v = v; a.beta = beta; a.b = const_cast<float*>(b); a.W = W; a.U = U;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.bf16 = dtype == KDA_BF16;
  return finish(kda::launch_stage_ut(a, (hipStream_t)stream), stream);
}

int kda_stage_state(const void* k, const float* b, const float* W, const float* U, const float* S0, float* Delta,
                    float* S_chunks, float* S_T, int B, int T, int H, int d_k, int d_v, int dtype, void* stream) {
  int st = check_staged_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  if ((int64_t)B * H == 0) return KDA_OK;
  if (T > 0) {
    KDA_REQUIRE(k && b && W && U && Delta && S_chunks, KDA_ERR_NULL);
    KDA_REQUIRE(aligned16(k) && aligned16(b) && aligned16(W) && aligned16(U) && aligned16(Delta) &&
                aligned16(S_chunks), KDA_ERR_ALIGN);
  }
  KDA_REQUIRE(aligned16(S0) && aligned16(S_T), KDA_ERR_ALIGN);
  kda::StageArgs a{};
  a.k = k; a.b = const_cast<float*>(b); a.W = const_cast<float*>(W); a.U = const_cast<float*>(U);
  a.S0 = S0; a.Delta = Delta; a.S_chunks = S_chunks; a.S_T = S_T;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.bf16 = dtype == KDA_BF16;
  return finish(kda::launch_stage_state(a, (hipStream_t)stream), stream);
}

int kda_stage_output(const void* q, const void* k, const float* b, const float* Delta, const float* S_chunks,
                     void* o, int B, int T, int H, int d_k, int d_v, int dtype, void* stream) {
  int st = check_staged_dims(B, T, H, d_k, d_v, dtype);
  if (st) return st;
  if ((int64_t)B * H * T == 0) return KDA_OK;
  KDA_REQUIRE(q && k && b && Delta && S_chunks && o, KDA_ERR_NULL);
  KDA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(b) && aligned16(Delta) && aligned16(S_chunks) &&
              aligned16(o), KDA_ERR_ALIGN);
  kda::StageArgs a{};
  a.q = q; a.k = k; a.b = const_cast<float*>(b); a.Delta = const_cast<float*>(Delta);
  a.S_chunks = const_cast<float*>(S_chunks); a.o = o;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.bf16 = dtype == KDA_BF16;
  return finish(kda::launch_stage_output(a, (hipStream_t)stream), stream);
}

int kda_recurrent_step(const void* q, const void* k, const void* v, const void* g, const void* beta, float* S,
                       void* o, int N, int H, int d_k, int d_v, int dtype, void* stream) {
  return kda_recurrent_step_ex(q, k, v, g, beta, S, o, N, H, d_k, d_v, dtype, 0, stream);
}

int kda_recurrent_step_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, float* S,
                          void* o, int N, int H, int d_k, int d_v, int dtype, int flags, void* stream) {
  int st = check_step_dims(N, H, d_k, d_v, dtype);
  if (st) return st;
  KDA_REQUIRE(valid_flags(flags), KDA_ERR_ARG);
  if ((int64_t)N * H == 0) return KDA_OK;
  st = check_tokens(q, k, v, g, beta, o, dtype, flags);
  if (st) return st;
  KDA_REQUIRE(S != nullptr, KDA_ERR_NULL);
  KDA_REQUIRE(aligned16(S), KDA_ERR_ALIGN);
  kda::DecodeArgs a{q, k, v, g, beta, S, o, N, H, d_k, d_v, dtype == KDA_BF16};
  a.variant = flags;
  return finish(kda::launch_decode(a, (hipStream_t)stream), stream);
}

}  // extern "C"
