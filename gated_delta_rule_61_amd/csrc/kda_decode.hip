// kda_decode.hip -- one-token recurrent decode step (HBM-streaming).
//
// Per sequence/head the step reads the d_k x d_v fp32 state once and writes it
// once ("Demystifying Hybrid LLM Architectures: Linear Attention, Residuals,
// and Latent MoE" §2.1: constant per-step cost; §2.3: retrieve, erase/write,
// read).  With D = Diag(exp g):
//     S' = D S,  r = S'^T k,  delta = beta (v - r),  S_new = S' + k delta^T,
//     o  = S_new^T q = S'^T q + delta (k . q)
// so r and S'^T q are two column reductions over the same registers and the
// state never makes a second trip through HBM.
//
// Mapping: one 256-thread workgroup per (sequence, head).  Thread t owns
// columns [4*(t % CG), +4) (one 16-byte load per row) and rows
// t / CG + RG*i, so each wavefront reads whole 512-byte state rows: fully
// coalesced 16-byte loads/stores.  Column partial sums meet in LDS.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// Variants (V): a scalar gate reads one g per sequence and head and decays
// every row by it; without the delta rule delta = v (nothing is retrieved or
// erased, beta is not read), so only S'^T q is reduced.
template <typename T, int DK, int DV, int V>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr bool SG = (V & kVarScalarGate) != 0, ND = (V & kVarNoDelta) != 0;
  constexpr int NT = 256;
  constexpr int CG = DV / 4;        // float4 column groups
  constexpr int RG = NT / CG;       // row groups
  constexpr int RPT = DK / RG;      // rows per thread
  static_assert(RG * CG == NT && RPT * RG == DK, "decode tiling");

  const int64_t head = blockIdx.x;  // n * H + h
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  float* S = a.S + head * (int64_t)(DK * DV);

  // 1. stream this thread's slice of the state (all loads in flight at once)
  floatx4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (int64_t)(rg + RG * i) * DV + 4 * cg));

  __shared__ float sk[DK], sq[DK], sa[DK], sv[DV];
  __shared__ float red_r[RG][DV], red_s[RG][DV];
  __shared__ float sdelta[DV];
  __shared__ float skq;

  const T* qh = reinterpret_cast<const T*>(a.q) + head * DK;
  const T* kh = reinterpret_cast<const T*>(a.k) + head * DK;
  const T* gh = reinterpret_cast<const T*>(a.g) + head * (SG ? 1 : DK);
  const T* vh = reinterpret_cast<const T*>(a.v) + head * DV;
  const float beta = ND ? 1.f : to_f32(reinterpret_cast<const T*>(a.beta)[head]);
  if (tid < DK) {
    sk[tid] = to_f32(kh[tid]);
    sq[tid] = to_f32(qh[tid]);
    sa[tid] = fast_exp(to_f32(gh[SG ? 0 : tid]));
  }
  if (tid < DV) sv[tid] = to_f32(vh[tid]);
  __syncthreads();

  // k . q by the first wavefront
  if (tid < kWave) {
    float p = 0.f;
    for (int c = tid; c < DK; c += kWave) p += sk[c] * sq[c];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) p += __shfl_xor(p, off);
    if (tid == 0) skq = p;
  }

  // 2. decay rows, then partial column sums of S'^T k and S'^T q
  floatx4 r = {0.f, 0.f, 0.f, 0.f}, sqv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    s[i] *= sa[row];
    if constexpr (!ND) r += sk[row] * s[i];
    sqv += sq[row] * s[i];
  }
  if constexpr (!ND) *reinterpret_cast<floatx4*>(&red_r[rg][4 * cg]) = r;
  *reinterpret_cast<floatx4*>(&red_s[rg][4 * cg]) = sqv;
  __syncthreads();

  // 3. per column: delta_j and o_j
  if (tid < DV) {
    float rr = 0.f, ss = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      if constexpr (!ND) rr += red_r[j][tid];
      ss += red_s[j][tid];
    }
    const float d = ND ? sv[tid] : beta * (sv[tid] - rr);
    sdelta[tid] = d;
    T* oh = reinterpret_cast<T*>(a.o) + head * DV;
    oh[tid] = from_f32<T>(ss + d * skq);
  }
  __syncthreads();

  // 4. rank-one write and store back in place
  const floatx4 d4 = *reinterpret_cast<const floatx4*>(&sdelta[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    floatx4 out = s[i] + sk[row] * d4;
    __builtin_nontemporal_store(out, reinterpret_cast<floatx4*>(S + (int64_t)row * DV + 4 * cg));
  }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int64_t nh = (int64_t)a.N * a.H;
  if (nh == 0) return hipSuccess;
  const dim3 grid((unsigned)nh), block(256);
  switch (a.variant) {
    case 0: hipLaunchKernelGGL((decode_kernel<T, DK, DV, 0>), grid, block, 0, s, a); break;
    case kVarScalarGate: hipLaunchKernelGGL((decode_kernel<T, DK, DV, kVarScalarGate>), grid, block, 0, s, a); break;
    case kVarNoDelta: hipLaunchKernelGGL((decode_kernel<T, DK, DV, kVarNoDelta>), grid, block, 0, s, a); break;
    case kVarScalarGate | kVarNoDelta:
      hipLaunchKernelGGL((decode_kernel<T, DK, DV, kVarScalarGate | kVarNoDelta>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.bf16) {
    if (a.dk == 128 && a.dv == 128) return launch_decode_t<bf16, 128, 128>(a, s);
    if (a.dk == 64 && a.dv == 64) return launch_decode_t<bf16, 64, 64>(a, s);
  } else {
    if (a.dk == 128 && a.dv == 128) return launch_decode_t<float, 128, 128>(a, s);
    if (a.dk == 64 && a.dv == 64) return launch_decode_t<float, 64, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
