// kda_backward_tok.hip -- gradient of the chunked forward for the sizes the
// chunked backward (kda_backward.hip, bf16 at d = 128) does not cover: fp32
// inputs at d = 64 or 128, bf16 inputs at d = 64, every variant.
//
// The forward is a function of its inputs alone, whatever the chunking
// ("Hybrid Linear Attention Architecture: Making LLM Training and Inference
// More Efficient" §IV: the chunked and the token form compute the same
// states), so its gradient is the reverse-mode derivative of the token
// recurrence ("...More Efficient" §3.3 for the KDA update and its scalar-gate
// and decay-only variants; read-out after the update, "Kimi Linear ..."
// §2.3).  Per token, with a = exp(g_t) per key channel (one value with a
// scalar gate), Sb = Diag(a) S_{t-1}, u = Sb^T k, r = v - u (r = v without
// the delta rule), S_t = Sb + beta k r^T (k v^T without it), o = S_t^T q:
//   G  = dS_t + q do^T           w_j = sum_c k_c G[c][j]
//   dq = S_t do                  dv  = beta w   (w without the delta rule)
//   dbeta = r . w                dk  = beta G r - beta Sb w   (G v)
//   dSb = G - beta k w^T  (G)    da_c = sum_j dSb[c][j] S_{t-1}[c][j]
//   dg = a da (summed over the channels with a scalar gate)
//   dS_{t-1} = Diag(a) dSb
// Launches:
//   tok_ckpt_kernel   the forward, storing the state at every chunk start;
//   tok_bwd_kernel    per (sequence x head, 16 value columns), the chunks in
//                     reverse: the chunk's token states recomputed from its
//                     checkpoint into a scratch block, then the reverse steps;
//                     dv and dS0 complete, dq, dk, dg, dbeta as partial sums
//                     over the column slices;
//   tok_reduce_kernel the slices' partial sums into dq, dk, dg, dbeta.
// A parity-grade path: every step is fp32 vector arithmetic, one token at a
// time; the chunked kernels are the fast ones.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace tokb {

constexpr int C = 64;      // tokens per checkpoint interval
constexpr int NT = 256;    // threads (4 wavefronts)
constexpr int CW = 16;     // value columns per workgroup

// Thread (j, rg): column j = tid % 16 of the workgroup's slice, rows
// rg + 16 i (rg = tid / 16, i < DK / 16).  The 16 consecutive lanes of a
// row group share their rows (row sums by lane shuffles); the column sums
// combine the four lanes of a wavefront that share j, then the four
// wavefronts in LDS.
template <int DK>
struct Tile {
  static constexpr int R = DK / 16;   // rows per thread
};

__device__ __forceinline__ float row_sum16(float x) {
  // sum over the caller's group of 16 lanes, in every lane of it (butterfly)
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

// sum over the 64 rows groups sharing column j: the four lanes j, j+16,
// j+32, j+48 of each wavefront, then the four wavefronts through red[4][16]
// (two barriers; the caller alternates between two buffers so that no barrier
// is needed before the next write)
__device__ __forceinline__ float col_sum(float x, float* red, int tid) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  const int lane = tid & 63, w = tid >> 6;
  if (lane < CW) red[w * CW + lane] = x;
  __syncthreads();
  const int j = tid & (CW - 1);
  return (red[j] + red[CW + j]) + (red[2 * CW + j] + red[3 * CW + j]);
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

// LDS of the backward kernel (floats): k, q, a of the chunk [C][DK]; v, dO,
// r of the slice [C][CW]; beta [C]; two column-sum buffers [4][CW].
template <int DK>
struct Lds {
  static constexpr int K = 0, Q = K + C * DK, A = Q + C * DK, V = A + C * DK, DO = V + C * CW, RR = DO + C * CW,
                       BETA = RR + C * CW, RED = BETA + C, END = RED + 2 * 4 * CW;
  static constexpr int BYTES = END * 4;
};

// Inputs of chunk n (tokens t0 .. t0 + nv - 1) into LDS: k, q and a = exp(g)
// for every channel, v and dO for the slice's columns, beta (1 without the
// delta rule).
template <typename T, int DK, int V>
__device__ __forceinline__ void stage_chunk(const BackwardArgs& a, float* sm, int bb, int h, int t0, int nv,
                                            int col0, int tid) {
  typedef Lds<DK> L;
  const int H = a.H;
  for (int e = tid; e < C * DK; e += NT) {
    const int t = e / DK, c = e % DK;
    float kv = 0.f, qv = 0.f, av = 1.f;
    if (t < nv) {
      const int64_t row = ((int64_t)bb * a.T + t0 + t) * H + h;
      kv = ld<T>(a.k, row * DK + c);
      qv = ld<T>(a.q, row * DK + c);
      av = __expf(ld<T>(a.g, (V & kVarScalarGate) ? row : row * DK + c));
    }
    sm[L::K + e] = kv;
    sm[L::Q + e] = qv;
    sm[L::A + e] = av;
  }
  for (int e = tid; e < C * CW; e += NT) {
    const int t = e / CW, j = e % CW;
    float vv = 0.f, dov = 0.f;
    if (t < nv) {
      const int64_t row = ((int64_t)bb * a.T + t0 + t) * H + h;
      vv = ld<T>(a.v, row * DK + col0 + j);
      dov = ld<T>(a.dO, row * DK + col0 + j);
    }
    sm[L::V + e] = vv;
    sm[L::DO + e] = dov;
  }
  if (tid < C) {
    float bt = 1.f;
    if ((V & kVarNoDelta) == 0)
      bt = tid < nv ? ld<T>(a.beta, ((int64_t)bb * a.T + t0 + tid) * H + h) : 0.f;
    sm[L::BETA + tid] = bt;
  }
}

// One forward token step on the thread's rows (S in, S out): returns r_j
// (the residual column value v_j - u_j, or v_j without the delta rule).
template <int DK, int V>
__device__ __forceinline__ float fwd_step(float (&S)[Tile<DK>::R], const float* sm, float* red, int t, int rg,
                                          int j, int tid) {
  typedef Lds<DK> L;
  constexpr int R = Tile<DK>::R;
  const float* kt = sm + L::K + t * DK;
  const float* at = sm + L::A + t * DK;
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = rg + 16 * i;
    S[i] *= at[c];
    p += kt[c] * S[i];
  }
  const float vj = sm[L::V + t * CW + j];
  float r;
  if constexpr ((V & kVarNoDelta) != 0) {
    r = vj;
  } else {
    r = vj - col_sum(p, red, tid);
  }
  const float bk = sm[L::BETA + t];
#pragma unroll
  for (int i = 0; i < R; ++i) S[i] += bk * kt[rg + 16 * i] * r;
  return r;
}

// ---------------------------------------------------------------------------
// Forward with checkpoints: the state at the start of every chunk into
// ckpt[head][n][DK][DV] (the slice's columns).  grid = B*H*(DV/16).
// ---------------------------------------------------------------------------
template <typename T, int DK, int V>
__global__ __launch_bounds__(NT) void tok_ckpt_kernel(BackwardArgs a, float* ckpt) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  typedef Lds<DK> L;
  constexpr int R = Tile<DK>::R, NS = DK / CW;
  const int head = blockIdx.x / NS, col0 = (blockIdx.x % NS) * CW;
  const int bb = head / a.H, h = head % a.H;
  const int tid = threadIdx.x, j = tid & (CW - 1), rg = tid >> 4;
  const int nch = (a.T + C - 1) / C;
  float S[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    S[i] = a.S0 ? a.S0[((int64_t)head * DK + rg + 16 * i) * DK + col0 + j] : 0.f;
  for (int n = 0; n < nch; ++n) {
    float* ck = ckpt + ((int64_t)head * nch + n) * DK * DK;
#pragma unroll
    for (int i = 0; i < R; ++i) ck[(rg + 16 * i) * DK + col0 + j] = S[i];
    const int t0 = n * C, nv = min(C, a.T - t0);
    __syncthreads();   // the previous chunk is done with LDS
    stage_chunk<T, DK, V>(a, sm, bb, h, t0, nv, col0, tid);
    __syncthreads();
    for (int t = 0; t < nv; ++t) fwd_step<DK, V>(S, sm, sm + L::RED + (t & 1) * 4 * CW, t, rg, j, tid);
  }
}

// ---------------------------------------------------------------------------
// Reverse pass.  grid = B*H*(DV/16).  Scratch per workgroup: the C token
// states S_{t-1} of the current chunk, [C][NT][R] (each thread's values
// contiguous).  Partial sums: part + split * rows * (3 DK + 1): dq, dk, dg
// ([rows][DK] each) and dbeta ([rows]).
// ---------------------------------------------------------------------------
template <typename T, int DK, int V>
__global__ __launch_bounds__(NT) void tok_bwd_kernel(BackwardArgs a, const float* ckpt, float* scratch,
                                                     float* part) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  typedef Lds<DK> L;
  constexpr int R = Tile<DK>::R, NS = DK / CW;
  constexpr bool ND = (V & kVarNoDelta) != 0;
  constexpr bool SG = (V & kVarScalarGate) != 0;
  const int head = blockIdx.x / NS, split = blockIdx.x % NS, col0 = split * CW;
  const int bb = head / a.H, h = head % a.H;
  const int tid = threadIdx.x, j = tid & (CW - 1), rg = tid >> 4;
  const int nch = (a.T + C - 1) / C;
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  float* pq = part + (int64_t)split * rows * (3 * DK + 1);
  float* pk = pq + rows * DK;
  float* pg = pk + rows * DK;
  float* pb = pg + rows * DK;
  float* scr = scratch + (int64_t)blockIdx.x * C * NT * R;
  float dS[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    dS[i] = a.dS_T ? a.dS_T[((int64_t)head * DK + rg + 16 * i) * DK + col0 + j] : 0.f;
  for (int n = nch - 1; n >= 0; --n) {
    const int t0 = n * C, nv = min(C, a.T - t0);
    const float* ck = ckpt + ((int64_t)head * nch + n) * DK * DK;
    float S[R];
#pragma unroll
    for (int i = 0; i < R; ++i) S[i] = ck[(rg + 16 * i) * DK + col0 + j];
    __syncthreads();   // the previous chunk is done with LDS
    stage_chunk<T, DK, V>(a, sm, bb, h, t0, nv, col0, tid);
    __syncthreads();
    // forward over the chunk: S_{t-1} to the scratch block, r_j to LDS
    for (int t = 0; t < nv; ++t) {
#pragma unroll
      for (int i = 0; i < R; ++i) scr[((int64_t)t * NT + tid) * R + i] = S[i];
      const float r = fwd_step<DK, V>(S, sm, sm + L::RED + (t & 1) * 4 * CW, t, rg, j, tid);
      if (rg == 0) sm[L::RR + t * CW + j] = r;
    }
    __syncthreads();
    // reverse over the chunk
    for (int t = nv - 1; t >= 0; --t) {
      const int64_t row = ((int64_t)bb * a.T + t0 + t) * a.H + h;
      const float* kt = sm + L::K + t * DK;
      const float* qt = sm + L::Q + t * DK;
      const float* at = sm + L::A + t * DK;
      const float bk = sm[L::BETA + t];
      const float r = sm[L::RR + t * CW + j];
      const float doj = sm[L::DO + t * CW + j];
      float Sp[R], Sb[R], G[R];
      float wp = 0.f;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = rg + 16 * i;
        Sp[i] = scr[((int64_t)t * NT + tid) * R + i];
        Sb[i] = at[c] * Sp[i];
        G[i] = dS[i] + qt[c] * doj;
        wp += kt[c] * G[i];
      }
      const float w = col_sum(wp, sm + L::RED + (t & 1) * 4 * CW, tid);
      // dv (complete for the slice's columns) and dbeta (partial)
      if (rg == 0) {
        T* dv = static_cast<T*>(a.dv);
        dv[row * DK + col0 + j] = from_f32<T>(ND ? w : bk * w);
      }
      if constexpr (!ND) {
        const float db = row_sum16(r * w);
        if (tid == 0) pb[row] = db;
      }
      // per-row sums over the slice's columns: dq, dk, da
      float dSb[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = rg + 16 * i;
        const float St = Sb[i] + bk * kt[c] * r;
        float xk;
        if constexpr (ND) {
          dSb[i] = G[i];
          xk = G[i] * r;   // r = v without the delta rule
        } else {
          dSb[i] = G[i] - bk * kt[c] * w;
          xk = bk * (G[i] * r - Sb[i] * w);
        }
        const float xq = row_sum16(St * doj);
        const float xkk = row_sum16(xk);
        const float xa = row_sum16(dSb[i] * Sp[i]);
        if (j == 0) {
          pq[row * DK + c] = xq;
          pk[row * DK + c] = xkk;
          pg[row * DK + c] = at[c] * xa;
        }
        dS[i] = at[c] * dSb[i];
      }
    }
  }
  if (a.dS0) {
#pragma unroll
    for (int i = 0; i < R; ++i) a.dS0[((int64_t)head * DK + rg + 16 * i) * DK + col0 + j] = dS[i];
  }
  (void)SG;
}

// ---------------------------------------------------------------------------
// Sum of the slices' partial sums into dq, dk, dg (dtype T; a scalar gate's
// dg summed over the channels too) and dbeta.  grid over rows.
// ---------------------------------------------------------------------------
template <typename T, int DK, int V>
__global__ __launch_bounds__(NT) void tok_reduce_kernel(BackwardArgs a, const float* part) {
  constexpr int NS = DK / CW;
  constexpr bool ND = (V & kVarNoDelta) != 0;
  constexpr bool SG = (V & kVarScalarGate) != 0;
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  const int64_t stride = rows * (3 * DK + 1);
  const int64_t row = blockIdx.x * (int64_t)(NT / DK) + threadIdx.x / DK;
  const int c = threadIdx.x % DK;
  const bool live = row < rows;   // (no early return: the scalar gate's sum has a barrier)
  float q = 0.f, k = 0.f, g = 0.f, b = 0.f;
  if (live) {
    for (int s = 0; s < NS; ++s) {
      const float* p = part + s * stride;
      q += p[row * DK + c];
      k += p[rows * DK + row * DK + c];
      g += p[2 * rows * DK + row * DK + c];
      if (!ND && c == 0) b += p[3 * rows * DK + row];
    }
    static_cast<T*>(a.dq)[row * DK + c] = from_f32<T>(q);
    static_cast<T*>(a.dk)[row * DK + c] = from_f32<T>(k);
    if (!ND && c == 0) static_cast<T*>(a.dbeta)[row] = from_f32<T>(b);
  }
  if constexpr (SG) {
    // channel sum of g within this row: the DK threads of the row are
    // consecutive, so reduce through LDS
    __shared__ float red[NT];
    red[threadIdx.x] = g;
    __syncthreads();
    if (live && c == 0) {
      float s = 0.f;
      for (int e = 0; e < DK; ++e) s += red[threadIdx.x + e];
      static_cast<T*>(a.dg)[row] = from_f32<T>(s);
    }
  } else {
    if (live) static_cast<T*>(a.dg)[row * DK + c] = from_f32<T>(g);
  }
}

template <typename T, int DK, int V>
hipError_t launch_t(const BackwardArgs& a, char* ws, hipStream_t s) {
  constexpr int NS = DK / CW;
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t nch = (a.T + C - 1) / C;
  const int64_t rows = BH * a.T;
  float* ckpt = reinterpret_cast<float*>(ws);
  float* scratch = ckpt + BH * nch * DK * DK;
  float* part = scratch + BH * NS * C * NT * Tile<DK>::R;
  if (BH * NS > INT32_MAX || (rows * DK + NT - 1) / NT > INT32_MAX) return hipErrorInvalidValue;
  const int bytes = Lds<DK>::BYTES;
  hipError_t e;
  auto ck = tok_ckpt_kernel<T, DK, V>;
  auto bw = tok_bwd_kernel<T, DK, V>;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(ck), hipFuncAttributeMaxDynamicSharedMemorySize,
                               bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(bw), hipFuncAttributeMaxDynamicSharedMemorySize,
                               bytes)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(ck, dim3((unsigned)(BH * NS)), dim3(NT), bytes, s, a, ckpt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bw, dim3((unsigned)(BH * NS)), dim3(NT), bytes, s, a, ckpt, scratch, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rows > 0) {
    hipLaunchKernelGGL((tok_reduce_kernel<T, DK, V>), dim3((unsigned)((rows * DK + NT - 1) / NT)), dim3(NT), 0, s,
                       a, part);
  }
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_v(const BackwardArgs& a, char* ws, hipStream_t s) {
  switch (a.variant) {
    case 0: return launch_t<T, DK, 0>(a, ws, s);
    case kVarScalarGate: return launch_t<T, DK, kVarScalarGate>(a, ws, s);
    case kVarNoDelta: return launch_t<T, DK, kVarNoDelta>(a, ws, s);
    case kVarScalarGate | kVarNoDelta: return launch_t<T, DK, kVarScalarGate | kVarNoDelta>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tokb

size_t backward_tok_workspace(int B, int T, int H, int d) {
  const int64_t BH = (int64_t)B * H, nch = (T + tokb::C - 1) / tokb::C, rows = BH * T;
  const int64_t NS = d / tokb::CW;
  const int64_t floats = BH * nch * d * d + BH * NS * tokb::C * tokb::NT * (d / 16) + NS * rows * (3 * d + 1);
  return (size_t)floats * sizeof(float);
}

hipError_t launch_backward_tok(const BackwardArgs& a, int d, bool bf16in, void* ws, hipStream_t s) {
  if ((int64_t)a.B * a.H == 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  if (bf16in) {
    if (d == 64) return tokb::launch_v<bf16, 64>(a, w, s);
  } else {
    if (d == 64) return tokb::launch_v<float, 64>(a, w, s);
    if (d == 128) return tokb::launch_v<float, 128>(a, w, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
