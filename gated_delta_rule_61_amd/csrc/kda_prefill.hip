// kda_prefill.hip -- chunkwise-parallel KDA forward on gfx950.
//
// The chunked form ("Hybrid Linear Attention Architecture: Making LLM
// Training and Inference More Efficient" §IV; "Linear Attention Architecture
// Deep Dive: From State Updates to Efficient Chunked Computation" §5), with a
// chunk of C = 64 tokens, positions r inside the chunk, and the in-chunk
// cumulative log-gate b_r = sum_{m<=r} g_m:
//   Kg = exp(b)*K,  Kd = exp(-b)*K,  Qg = exp(b)*Q,  Kb = exp(b_C - b)*K
//   L  = StrictTril(Diag(beta) Kg Kd^T),  A = (I + L)^-1
//   W  = A Diag(beta) Kg,  U = A Diag(beta) V
//   Delta = U - W S,   O = Qg S + Tril(Qg Kd^T) Delta,
//   S <- Diag(exp b_C) S + Kb^T Delta
//
// Kernels in this file
//   fused_fwd_kernel      production schedule: one workgroup per (sequence,
//                         head, column split of the state) walks the chunks in
//                         order; every intermediate lives in LDS/registers, so
//                         HBM sees q,k,v,g,beta once and o once.
//   stage_*_kernel        the staged schedule (cumsum, UT transform, state
//                         passing, output) with fp32 intermediates in HBM,
//                         built from the same device blocks; used to check each
//                         step on its own.
//
// Workgroup: 8 wavefronts (512 threads).  The state S of a workgroup
// (d_k x DVW fp32, DVW = d_v / NSPLIT) is held in MFMA accumulator layout in
// the registers of DVW/16 "owner" wavefronts (16 columns each) for the whole
// sequence.  A = (I + L)^-1 is applied by blocked forward substitution with
// 16x16 blocks: the four diagonal blocks are inverted by scalar forward
// substitution (one wavefront, one lane per column), the off-diagonal
// coupling runs on MFMA, column tile by column tile, in registers.
#include <algorithm>
#include <cstdlib>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int C = 64;        // chunk length
constexpr int NW = 8;        // wavefronts per workgroup
constexpr int NT = NW * kWave;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// LDS layout.  Rows of bf16/fp32 operand arrays are padded by 16 bytes so that
// the 16 rows an MFMA fragment read touches fall in different banks.
// ---------------------------------------------------------------------------
// State columns per owner wavefront: 32 (two 16-wide MFMA tiles sharing
// every A operand read) when the workgroup has at least 32 columns.
template <int DVW> struct StateTiles {
  static constexpr int NTILE = DVW >= 32 ? 2 : 1;
  static constexpr int OWN = DVW / (16 * NTILE);        // owner wavefronts
};

template <typename T, int DK, int DVW>
struct Layout {
  static constexpr int PE = 16 / (int)sizeof(T);
  static constexpr int LDK = DK + PE;     // [C][DK] arrays
  static constexpr int LDC = C + PE;      // [*][C] arrays
  static constexpr int LDV = DVW + PE;    // [C][DVW] value tile
  static constexpr int LDG = DK + 4;      // fp32 gate rows
  static constexpr int LDD = 16 + PE;     // diagonal-inverse blocks
  static constexpr int LDL = 20;          // fp32 diagonal blocks of L (16-byte rows)
  static constexpr int NSEG = NT / DK;    // cumsum row segments
  static constexpr int SZ_CK = C * LDK * (int)sizeof(T);
  static constexpr int O_KT = 0;
  static constexpr int O_KH = O_KT + SZ_CK;            // later reused for -W
  static constexpr int O_QT = O_KH + SZ_CK;
  static constexpr int O_KBT = O_QT + SZ_CK;
  static constexpr int O_V = O_KBT + DK * LDC * (int)sizeof(T);    // Kb^T, swizzled
  static constexpr int O_G = O_V + C * LDV * (int)sizeof(T);
  static constexpr int SZ_GATE = C * LDG * 4;
  static constexpr int SZ_LP = 2 * C * LDC * (int)sizeof(T) + 4 * 16 * LDL * 4 + 4 * 16 * LDD * (int)sizeof(T);
  static constexpr int SZ_G = SZ_GATE > SZ_LP ? SZ_GATE : SZ_LP;
  // inside the gate region, once the gates are consumed:
  static constexpr int O_LN = O_G;                                   // -L (off-diagonal blocks)
  static constexpr int O_P = O_LN + C * LDC * (int)sizeof(T);        // Tril(Qg Kd^T)
  static constexpr int O_LD = O_P + C * LDC * (int)sizeof(T);        // fp32 diagonal blocks of L
  static constexpr int O_DB = O_LD + 4 * 16 * LDL * 4;                // (I + L_ii)^-1
  static constexpr int O_TOT = O_G + SZ_G;
  static constexpr int O_BETA = O_TOT + NSEG * DK * 4;
  static constexpr int O_GAM = O_BETA + C * 4;
  static constexpr int O_BC = O_GAM + DK * 4;
  // per owner wavefront: its 64 x (16*NTILE) output block, rows padded by 8 bytes
  static constexpr int LDS_O = 16 * StateTiles<DVW>::NTILE + 8 / (int)sizeof(T);
  static constexpr int O_QK = O_BC + DK * 4;                          // q_t . k_t per row
  static constexpr int O_STG = O_QK + C * 4;
  static constexpr int BYTES = O_STG + StateTiles<DVW>::OWN * C * LDS_O * (int)sizeof(T);
};

template <typename T, int DK, int DVW>
struct Smem {
  typedef Layout<T, DK, DVW> Lay;
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  TL* Kt; TL* Kh; TL* Wn; TL* Qt; TF* KbT; T* V;
  float* G; TF* Ln; TF* P; float* Ld; TF* Db;
  float* tot; float* beta; float* gam; float* bC; float* qk;
  T* stg;
  // `opaque` is an offset the compiler cannot see through (zero at run time):
  // rebuilding the view with it every chunk keeps LDS address arithmetic
  // inside the chunk loop instead of pinning one register per address.
  __device__ explicit Smem(unsigned char* base0, uint32_t opaque = 0) { set(base0 + opaque); }
  // Barrier, then re-derive every LDS pointer from an opaque zero offset, so
  // that address arithmetic of the next phase stays in that phase.
  __device__ __forceinline__ void sync_rebase(unsigned char* base0) {
    __syncthreads();
    uint32_t opq = 0;
    asm volatile("" : "+s"(opq));
    set(base0 + opq);
  }
  __device__ __forceinline__ void set(unsigned char* base) {
    Kt = reinterpret_cast<TL*>(base + Lay::O_KT);
    Kh = reinterpret_cast<TL*>(base + Lay::O_KH);
    Wn = Kh;
    Qt = reinterpret_cast<TL*>(base + Lay::O_QT);
    KbT = reinterpret_cast<TF*>(base + Lay::O_KBT);
    V = reinterpret_cast<T*>(base + Lay::O_V);
    G = reinterpret_cast<float*>(base + Lay::O_G);
    Ln = reinterpret_cast<TF*>(base + Lay::O_LN);
    P = reinterpret_cast<TF*>(base + Lay::O_P);
    Ld = reinterpret_cast<float*>(base + Lay::O_LD);
    Db = reinterpret_cast<TF*>(base + Lay::O_DB);
    tot = reinterpret_cast<float*>(base + Lay::O_TOT);
    beta = reinterpret_cast<float*>(base + Lay::O_BETA);
    gam = reinterpret_cast<float*>(base + Lay::O_GAM);
    bC = reinterpret_cast<float*>(base + Lay::O_BC);
    qk = reinterpret_cast<float*>(base + Lay::O_QK);
    stg = reinterpret_cast<T*>(base + Lay::O_STG);
  }
};

// Kb^T is stored [d_k][C + pad] (row stride LDC); token t of channel c sits at
// column t ^ kb_swz(c).  The XOR moves whole 4-token groups, so MFMA operand
// reads (4 consecutive tokens) stay contiguous, while the transposed 2-byte
// writes of one wavefront (16 channel groups x 4 tokens) and the operand reads
// (16 channels x 2 token groups) each land in distinct LDS banks.  It depends
// on c only through c / 8, so a thread writing 8 consecutive channels computes
// it once.
__device__ __forceinline__ int kb_swz(int c) { return 4 * ((c >> 3) & 15); }

// ---------------------------------------------------------------------------
// Global -> register staging of one chunk of one head.
// A 16-byte vector index idx covers row idx / VPR, elements (idx % VPR) * VN.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct RowVecs {
  static constexpr int VN = VecTraits<T>::N;
  static constexpr int VPR = D / VN;                     // vectors per row
  static constexpr int TOTAL = C * VPR;
  static constexpr int PER = (TOTAL + NT - 1) / NT;      // per thread
};

struct TokIdx {   // addressing of [B,T,H,D] token-major tensors
  int64_t row0;   // (b*T + t0) * H + h  (token index of chunk row 0)
  int64_t rstride;// H
};

// Raw buffer resource over `bytes` bytes from `base`: loads past the end read
// zero and stores past the end are dropped, which handles a partial last
// chunk without branches and keeps 64-bit addresses in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Bytes covered by rows [0, nv) of a chunk whose rows are `rstride` elements
// apart and `width` elements wide.
__device__ __forceinline__ uint32_t chunk_bytes(int nv, int rstride, int width, int esize) {
  return nv > 0 ? (uint32_t)(((nv - 1) * rstride + width) * esize) : 0u;
}

// 16-byte vectors of one chunk (rows of D elements, `rstride` elements apart)
// into registers through a buffer resource.
template <typename T, int D>
__device__ __forceinline__ void buf_load_rows(Vec16* r, __amdgpu_buffer_rsrc_t rs, int rstride, int tid) {
  typedef RowVecs<T, D> RV;
#pragma unroll
  for (int i = 0; i < RV::PER; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / RV::VPR, cv = idx % RV::VPR;
    const uint32_t off = idx < RV::TOTAL ? (uint32_t)(row * rstride * (int)sizeof(T) + cv * 16) : 0x80000000u;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    r[i].w[0] = x[0]; r[i].w[1] = x[1]; r[i].w[2] = x[2]; r[i].w[3] = x[3];
  }
}

template <typename T>
__device__ __forceinline__ float buf_load_scalar(__amdgpu_buffer_rsrc_t rs, uint32_t off);
template <>
__device__ __forceinline__ float buf_load_scalar<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const unsigned short u = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
  return __uint_as_float(((uint32_t)u) << 16);
}
template <>
__device__ __forceinline__ float buf_load_scalar<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

template <typename T>
__device__ __forceinline__ void buf_store_scalar(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v);
template <>
__device__ __forceinline__ void buf_store_scalar<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  const bf16 b = static_cast<bf16>(v);
  __builtin_amdgcn_raw_buffer_store_b16(*reinterpret_cast<const unsigned short*>(&b), rs, off, 0, 0);
}
template <>
__device__ __forceinline__ void buf_store_scalar<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
}

template <typename T, int D>
__device__ __forceinline__ void load_rows(Vec16* r, const T* base, int ld_elems,
                                          int col_off, const TokIdx& ti, int nvalid, int tid) {
  typedef RowVecs<T, D> RV;
#pragma unroll
  for (int i = 0; i < RV::PER; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / RV::VPR, cv = idx % RV::VPR;
    Vec16 z; z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0u;
    r[i] = z;
    if (idx < RV::TOTAL && row < nvalid)
      r[i] = ldg16(base + (ti.row0 + (int64_t)row * ti.rstride) * ld_elems + col_off + cv * RV::VN);
  }
}

template <typename T, int DK, int DV, int DVW>
struct ChunkRegs {
  Vec16 q[RowVecs<T, DK>::PER];
  Vec16 k[RowVecs<T, DK>::PER];
  Vec16 g[RowVecs<T, DK>::PER];
  Vec16 v[RowVecs<T, DVW>::PER];
  uint32_t beta_bits;   // raw bits: converting at load time would wait for the whole prefetch
};

template <typename T> __device__ __forceinline__ float bits_to_f32(uint32_t u);
template <> __device__ __forceinline__ float bits_to_f32<bf16>(uint32_t u) { return __uint_as_float(u << 16); }
template <> __device__ __forceinline__ float bits_to_f32<float>(uint32_t u) { return __uint_as_float(u); }

// ---------------------------------------------------------------------------
// Device blocks of the chunk computation.
// ---------------------------------------------------------------------------

// g (registers) -> G (fp32 LDS); beta -> LDS.
// Column order of the fp32 gate rows in LDS.  With d_k = 128 and 8 channels
// per thread, channel c = 8a + 4b + r is stored at 64b + 4a + r: the first
// halves of all 16 channel groups of a row are contiguous, then the second
// halves, so each 16-byte access of the 16 lanes of a row hits 64 distinct
// banks.  Other shapes keep the natural order.
template <int DK, int VN> struct GateCols {
  static constexpr bool PERM = (DK == 128 && VN == 8);
  static __device__ __forceinline__ int pos(int c) {
    return PERM ? (((c >> 2) & 1) * 64 + (c >> 3) * 4 + (c & 3)) : c;
  }
  static __device__ __forceinline__ int chan(int j) {   // inverse of pos
    return PERM ? (((j & 63) >> 2) * 8 + (j >> 6) * 4 + (j & 3)) : j;
  }
};

// The 8 (or 4) gates of one thread's vector: two (one) 16-byte LDS accesses.
template <int DK, int VN>
__device__ __forceinline__ void gate_store(float* row, int c0, const float* f) {
  if constexpr (GateCols<DK, VN>::PERM) {
    const int a = c0 >> 3;
    *reinterpret_cast<floatx4*>(row + 4 * a) = floatx4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<floatx4*>(row + 64 + 4 * a) = floatx4{f[4], f[5], f[6], f[7]};
  } else {
#pragma unroll
    for (int e = 0; e < VN; ++e) row[c0 + e] = f[e];
  }
}
template <int DK, int VN>
__device__ __forceinline__ void gate_load(const float* row, int c0, float* f) {
  if constexpr (GateCols<DK, VN>::PERM) {
    const int a = c0 >> 3;
    const floatx4 lo = *reinterpret_cast<const floatx4*>(row + 4 * a);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(row + 64 + 4 * a);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  } else {
#pragma unroll
    for (int e = 0; e < VN; ++e) f[e] = row[c0 + e];
  }
}

// 2^x by the hardware instruction (results below the fp32 normal range
// flush towards zero, which is below every tolerance here).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// g (registers) -> G (fp32 LDS, multiplied by `scale`); beta -> LDS.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void stage_gates(Smem<T, DK, DVW>& sm, const Vec16* g,
                                            float beta, int tid, float scale) {
  typedef RowVecs<T, DK> RV;
  typedef Layout<T, DK, DVW> Lay;
#pragma unroll
  for (int i = 0; i < RV::PER; ++i) {
    const int idx = tid + NT * i;
    if (idx < RV::TOTAL) {
      const int row = idx / RV::VPR, c0 = (idx % RV::VPR) * RV::VN;
      float f[RV::VN];
      vec_to_f32<T>(g[i], f);
#pragma unroll
      for (int e = 0; e < RV::VN; ++e) f[e] *= scale;
      gate_store<DK, RV::VN>(&sm.G[row * Lay::LDG], c0, f);
    }
  }
  if (tid < C) sm.beta[tid] = beta;
}

// In-chunk inclusive cumulative sum of G over rows (in place), then
// bC = b at the last row and gam = exp(bC).  Contains one barrier; the caller
// must barrier before reading the result.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void chunk_cumsum(Smem<T, DK, DVW>& sm, int tid) {
  typedef Layout<T, DK, DVW> Lay;
  constexpr int NSEG = Lay::NSEG;
  constexpr int RPS = C / NSEG;
  const int c = tid % DK, seg = tid / DK;
  float v[RPS];
#pragma unroll
  for (int r = 0; r < RPS; ++r) v[r] = sm.G[(seg * RPS + r) * Lay::LDG + c];
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < RPS; ++r) {
    run += v[r];
    v[r] = run;
  }
  sm.tot[seg * DK + c] = run;
  __syncthreads();
  float off = 0.f;
  for (int s = 0; s < seg; ++s) off += sm.tot[s * DK + c];
#pragma unroll
  for (int r = 0; r < RPS; ++r) sm.G[(seg * RPS + r) * Lay::LDG + c] = v[r] + off;
  if (seg == NSEG - 1) {
    // this thread scanned physical column c; record its channel's totals
    const int ch = GateCols<DK, VecTraits<T>::N>::chan(c);
    const float bl = run + off;
    sm.bC[ch] = bl;
    sm.gam[ch] = hw_exp2(bl);
  }
}

// Elementwise gate application from the registers of this thread:
//   Kt = exp(b) k, Kh = exp(-b) k, Qt = exp(b) q, KbT^T = exp(bC - b) k, V = v.
template <typename T, int DK, int DVW, bool DO_KT, bool DO_KH, bool DO_QT, bool DO_KB>
__device__ __forceinline__ void apply_gates(Smem<T, DK, DVW>& sm, const Vec16* kq, const Vec16* qq, int tid) {
  typedef RowVecs<T, DK> RV;
  typedef Layout<T, DK, DVW> Lay;
#pragma unroll
  for (int i = 0; i < RV::PER; ++i) {
    const int idx = tid + NT * i;
    if (idx < RV::TOTAL) {
      const int row = idx / RV::VPR, c0 = (idx % RV::VPR) * RV::VN;
      float kf[RV::VN], qf[RV::VN];
      vec_to_f32<T>(kq[i], kf);
      if (DO_QT) vec_to_f32<T>(qq[i], qf);
      typedef typename Operands<T>::TL TL;
      typedef typename Operands<T>::TF TF;
      TL kt[RV::VN], kh[RV::VN], qt[RV::VN];
      float bv[RV::VN];
      gate_load<DK, RV::VN>(&sm.G[row * Lay::LDG], c0, bv);
#pragma unroll
      for (int e = 0; e < RV::VN; ++e) {
        // G holds log2-scaled cumulative gates: exp(b) = exp2(G)
        const float ep = hw_exp2(bv[e]);
        const float em = hw_exp2(-bv[e]);
        kt[e] = from_f32<TL>(kf[e] * ep);
        kh[e] = from_f32<TL>(kf[e] * em);
        if (DO_QT) qt[e] = from_f32<TL>(qf[e] * ep);
        if (DO_KB) sm.KbT[(c0 + e) * Lay::LDC + (row ^ kb_swz(c0))] = from_f32<TF>(kf[e] * (sm.gam[c0 + e] * em));
      }
      if (DO_KT) *reinterpret_cast<Vec16*>(&sm.Kt[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(kt);
      if (DO_KH) *reinterpret_cast<Vec16*>(&sm.Kh[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(kh);
      if (DO_QT) *reinterpret_cast<Vec16*>(&sm.Qt[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(qt);
    }
    if (DO_QT) {
      // the diagonal of P is q_t . k_t (the gates cancel): summed in fp32 from
      // the inputs over the VPR threads that hold one row
      float d = 0.f;
      if (idx < RV::TOTAL) {
        float kf[RV::VN], qf[RV::VN];
        vec_to_f32<T>(kq[i], kf);
        vec_to_f32<T>(qq[i], qf);
#pragma unroll
        for (int e = 0; e < RV::VN; ++e) d += qf[e] * kf[e];
      }
#pragma unroll
      for (int off = RV::VPR / 2; off > 0; off >>= 1) d += __shfl_xor(d, off);
      if (idx < RV::TOTAL && idx % RV::VPR == 0) sm.qk[idx / RV::VPR] = d;
    }
  }
}

template <typename T, int DK, int DVW>
__device__ __forceinline__ void stage_values(Smem<T, DK, DVW>& sm, const Vec16* v, int tid) {
  typedef RowVecs<T, DVW> RV;
  typedef Layout<T, DK, DVW> Lay;
#pragma unroll
  for (int i = 0; i < RV::PER; ++i) {
    const int idx = tid + NT * i;
    if (idx < RV::TOTAL) {
      const int row = idx / RV::VPR, c0 = (idx % RV::VPR) * RV::VN;
      *reinterpret_cast<Vec16*>(&sm.V[row * Lay::LDV + c0]) = v[i];
    }
  }
}

// Tiles (I, J) of L = StrictTril(Diag(beta) Kt Kh^T) or of P = Tril(Qt Kh^T),
// NTL at a time so that their operand reads and MFMAs overlap.  L's diagonal
// blocks go to Ld (fp32) for the inverse, its off-diagonal blocks to Ln as -L;
// P goes to P (both in the TF type).  P's blocks (0,1) and (2,3) above the
// diagonal are written as zeros because 32-wide reduction slabs read them.
template <typename T, int DK, int DVW, int NTL>
__device__ __forceinline__ void lp_tiles(Smem<T, DK, DVW>& sm, const bool (&isL)[NTL], const int (&I)[NTL],
                                         const int (&J)[NTL], int lane) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
  floatx4 acc[NTL];
#pragma unroll
  for (int t = 0; t < NTL; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) {
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      if (I[t] >= J[t]) {
        const TL* A = isL[t] ? sm.Kt : sm.Qt;
        const typename M::F32 af = M::lds32(A + (16 * I[t] + l16) * Lay::LDK + 32 * ks + 4 * g4);
        const typename M::F32 bf = M::lds32(sm.Kh + (16 * J[t] + l16) * Lay::LDK + 32 * ks + 4 * g4);
        acc[t] = M::mma32(af, bf, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int il = 4 * g4 + j;             // row inside the block
      const int i = 16 * I[t] + il, jc = 16 * J[t] + l16;
      float val = acc[t][j];
      if (isL[t]) {
        val *= sm.beta[i];
        if (I[t] == J[t]) {
          if (il <= l16) val = 0.f;
          sm.Ld[(I[t] * 16 + il) * Lay::LDL + l16] = val;
        } else {
          sm.Ln[i * Lay::LDC + jc] = from_f32<TF>(-val);
        }
      } else {
        if ((I[t] == J[t] && il < l16) || I[t] < J[t]) val = 0.f;
        if (I[t] == J[t] && il == l16) val = sm.qk[i];
        sm.P[i * Lay::LDC + jc] = from_f32<TF>(val);
      }
    }
  }
}

template <typename T, int DK, int DVW>
__device__ __forceinline__ void lp_tile(Smem<T, DK, DVW>& sm, bool isL, int I, int J, int lane) {
  const bool l[1] = {isL};
  const int i[1] = {I}, j[1] = {J};
  lp_tiles<T, DK, DVW, 1>(sm, l, i, j, lane);
}

// (I + L_bb)^-1 of one diagonal 16x16 block by forward substitution: lane c
// (mod 16) solves (I + L_bb) x = e_c for column c of the inverse.  Rows of
// L_bb are read as 16-byte vectors; a scheduling fence every four rows bounds
// how many are held in registers at once.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void diag_inverse_block(Smem<T, DK, DVW>& sm, int blk, int lane) {
  typedef Layout<T, DK, DVW> Lay;
  const int c = lane & 15;
  const float* Lb = sm.Ld + blk * 16 * Lay::LDL;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float row[16];
#pragma unroll
    for (int m4 = 0; m4 < (r + 3) / 4; ++m4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(Lb + r * Lay::LDL + 4 * m4);
      row[4 * m4 + 0] = v[0]; row[4 * m4 + 1] = v[1]; row[4 * m4 + 2] = v[2]; row[4 * m4 + 3] = v[3];
    }
    float sacc = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < r; ++m) sacc -= row[m] * x[m];
    x[r] = sacc;
    if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.Db[(blk * 16 + r) * Lay::LDD + c] = from_f32<typename Operands<T>::TF>(x[r]);
  }
}

// The intra-chunk matrices of one chunk, without a barrier between the L
// diagonal blocks and their inverses: wavefronts 0-3 each compute one diagonal
// block of L and invert it; the other wavefronts compute the off-diagonal L
// blocks and the P blocks meanwhile.  With DO_L false all wavefronts share P.
template <typename T, int DK, int DVW, bool DO_L, bool DO_P>
__device__ __forceinline__ void intra_chunk_matrices(Smem<T, DK, DVW>& sm, int wave, int lane) {
  // off-diagonal L blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2) and P blocks
  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3) (0,1) (2,3)
  constexpr int NL = DO_L ? 6 : 0;
  constexpr int NP = DO_P ? 12 : 0;
  constexpr int FIRST = DO_L ? 4 : 0;
  if (DO_L && wave < 4) {
    lp_tile<T, DK, DVW>(sm, true, wave, wave, lane);
    diag_inverse_block<T, DK, DVW>(sm, wave, lane);   // same wavefront: LDS order suffices
    return;
  }
  // tile t < NL: off-diagonal L, else P; handled two at a time
  constexpr int STEP = NW - FIRST;
  auto decode = [](int t, bool& isL, int& I, int& J) {
    isL = t < NL;
    const int u = isL ? t : t - NL;
    I = isL ? (int)((0x333221ull >> (4 * u)) & 15u) : (int)((0x203333222110ull >> (4 * u)) & 15u);
    J = isL ? (int)((0x210100ull >> (4 * u)) & 15u) : (int)((0x313210210100ull >> (4 * u)) & 15u);
  };
  for (int t = wave - FIRST; t < NL + NP; t += 2 * STEP) {
    if (t + STEP < NL + NP) {
      bool l[2]; int I[2], J[2];
      decode(t, l[0], I[0], J[0]);
      decode(t + STEP, l[1], I[1], J[1]);
      lp_tiles<T, DK, DVW, 2>(sm, l, I, J, lane);
    } else {
      bool l[1]; int I[1], J[1];
      decode(t, l[0], I[0], J[0]);
      lp_tiles<T, DK, DVW, 1>(sm, l, I, J, lane);
    }
  }
}

// Blocked forward substitution for NT 16-column tiles at once:
//   X_I = D_I (beta * Src_I - sum_{M<I} L_IM X_M),  I = 0..3,
// Src rows from LDS (ld = row stride, col[t] = first column of tile t).  The
// tiles' dependency chains are independent, so their MFMAs interleave.  X stays
// in registers (C layout, fp32).
template <typename T, int DK, int DVW, typename TS, int NTL>
__device__ __forceinline__ void fwd_subst_tiles(Smem<T, DK, DVW>& sm, const TS* src, int ld, const int (&col)[NTL],
                                                floatx4 (&X)[NTL][4], int lane) {
  typedef Mma<typename Operands<T>::TF> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    floatx4 acc[NTL];
    const floatx4 bt = *reinterpret_cast<const floatx4*>(&sm.beta[16 * I + 4 * g4]);
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t][j] = bt[j] * to_f32(src[(16 * I + 4 * g4 + j) * ld + col[t] + l16]);
#pragma unroll
    for (int Mb = 0; Mb < I; ++Mb) {
      const typename M::F16 af = M::lds16(sm.Ln + (16 * I + l16) * Lay::LDC + 16 * Mb + 4 * g4);
#pragma unroll
      for (int t = 0; t < NTL; ++t) acc[t] = M::mma16(af, M::frag16(X[t][Mb]), acc[t]);
    }
    const typename M::F16 df = M::lds16(sm.Db + (16 * I + l16) * Lay::LDD + 4 * g4);
#pragma unroll
    for (int t = 0; t < NTL; ++t) X[t][I] = M::mma16(df, M::frag16(acc[t]), zero);
  }
}

// One tile (the staged kernels).
template <typename T, int DK, int DVW, typename TS>
__device__ __forceinline__ void fwd_subst_tile(Smem<T, DK, DVW>& sm, const TS* src, int ld, int col0,
                                               floatx4 (&X)[4], int lane) {
  const int col[1] = {col0};
  fwd_subst_tiles<T, DK, DVW, TS, 1>(sm, src, ld, col, *reinterpret_cast<floatx4(*)[1][4]>(&X), lane);
}

// Store -W of a 16-column tile into Wn (row-major [C][DK]).
template <typename T, int DK, int DVW>
__device__ __forceinline__ void store_negw(Smem<T, DK, DVW>& sm, const floatx4 (&X)[4], int col0, int lane) {
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sm.Wn[(16 * I + 4 * g4 + j) * Lay::LDK + col0 + l16] = from_f32<typename Operands<T>::TL>(-X[I][j]);
}

// ---- products against the state, for NTILE 16-column tiles per wavefront.
// S[nt][rt]: rows 16rt.. of the state (key channels), C layout.

// Dx[nt][I] += A1[rows 16I..] @ S[nt]   and, if A2, O[nt][I] += A2[rows 16I..] @ S[nt]
// (A1 = -W gives Delta = U - W S; A2 = Qt gives the read-out of the chunk-entry
// state).  Each A fragment is read once and used for every tile.
template <typename TL, int DK, int NTILE, bool WITH_O>
__device__ __forceinline__ void rows_times_state(const TL* A1, const TL* A2, int lda,
                                                 const floatx4 (&S)[NTILE][DK / 16],
                                                 floatx4 (&Dx)[NTILE][4], floatx4 (&O)[NTILE][4], int lane) {
  typedef Mma<TL> M;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) {
    typename M::F32 sf[NTILE];
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) sf[nt] = M::frag32(S[nt][2 * ks], S[nt][2 * ks + 1]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const typename M::F32 a1 = M::lds32(A1 + (16 * I + l16) * lda + 32 * ks + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) Dx[nt][I] = M::mma32(a1, sf[nt], Dx[nt][I]);
      if (WITH_O) {
        const typename M::F32 a2 = M::lds32(A2 + (16 * I + l16) * lda + 32 * ks + 4 * g4);
#pragma unroll
        for (int nt = 0; nt < NTILE; ++nt) O[nt][I] = M::mma32(a2, sf[nt], O[nt][I]);
      }
    }
  }
}

// O[nt][I] += P[rows 16I..] @ Delta[nt]  (P lower triangular: slab 1 only for I >= 2)
template <typename T, int DK, int DVW, int NTILE>
__device__ __forceinline__ void intra_output(Smem<T, DK, DVW>& sm,
                                             const typename Mma<typename Operands<T>::TF>::F32 (&Df)[NTILE][2],
                                             floatx4 (&O)[NTILE][4], int lane) {
  typedef Mma<typename Operands<T>::TF> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const typename M::F32 a0 = M::lds32(sm.P + (16 * I + l16) * Lay::LDC + 4 * g4);
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) O[nt][I] = M::mma32(a0, Df[nt][0], O[nt][I]);
    if (I >= 2) {
      const typename M::F32 a1 = M::lds32(sm.P + (16 * I + l16) * Lay::LDC + 32 + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) O[nt][I] = M::mma32(a1, Df[nt][1], O[nt][I]);
    }
  }
}

// S <- Diag(gam) S + Kb^T @ Delta, Kb^T read through its swizzle.
template <typename T, int DK, int DVW, int NTILE>
__device__ __forceinline__ void state_update(Smem<T, DK, DVW>& sm,
                                             const typename Mma<typename Operands<T>::TF>::F32 (&Df)[NTILE][2],
                                             floatx4 (&S)[NTILE][DK / 16], int lane) {
  typedef typename Operands<T>::TF TF;
  typedef Mma<TF> M;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt) {
    const floatx4 gm = *reinterpret_cast<const floatx4*>(&sm.gam[16 * rt + 4 * g4]);
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) S[nt][rt] *= gm;
    const int c = 16 * rt + l16;
    const int sw = kb_swz(c);
    const TF* row = sm.KbT + c * Layout<T, DK, DVW>::LDC;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t0 = 32 * h + 4 * g4;      // tokens t0..t0+3 and t0+16..t0+19
      const typename M::F16 lo = M::lds16(row + (t0 ^ sw));
      const typename M::F16 hi = M::lds16(row + ((t0 + 16) ^ sw));
      const typename M::F32 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) S[nt][rt] = M::mma32(a, Df[nt][h], S[nt][rt]);
    }
  }
}

// Write an owner wavefront's 64 x (16*NTILE) output block to o: C layout ->
// its private LDS staging rows -> 16-byte buffer stores (rows past the end of
// the sequence fall outside the buffer range and are dropped).
template <typename T, int DK, int DVW, int NTILE>
__device__ __forceinline__ void store_output(Smem<T, DK, DVW>& sm, const floatx4 (&O)[NTILE][4], int owner_idx,
                                             __amdgpu_buffer_rsrc_t ro, int row_elems, int col, int lane) {
  typedef Layout<T, DK, DVW> Lay;
  constexpr int W = 16 * NTILE;
  constexpr int LD = Lay::LDS_O;
  T* st = sm.stg + owner_idx * C * LD;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int j = 0; j < 4; ++j) st[(16 * I + 4 * g4 + j) * LD + 16 * nt + l16] = from_f32<T>(O[nt][I][j]);
  // 8-byte reads (rows are 8-byte aligned), paired into 16-byte stores
  constexpr int E8 = 8 / (int)sizeof(T);          // elements per 8 bytes
  constexpr int VPR = W / (2 * E8);              // 16-byte vectors per row
  constexpr int PER = C * VPR / kWave;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = lane + kWave * i;
    const int row = idx / VPR, cv = idx % VPR;
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x2 a = *reinterpret_cast<const u32x2*>(st + row * LD + cv * 2 * E8);
    const u32x2 b = *reinterpret_cast<const u32x2*>(st + row * LD + cv * 2 * E8 + E8);
    const u32x4 v = {a[0], a[1], b[0], b[1]};
    __builtin_amdgcn_raw_buffer_store_b128(v, ro, (uint32_t)((row * row_elems + col + cv * 2 * E8) * (int)sizeof(T)), 0, 0);
  }
}

// C-layout tile rows of a [B,T,H,D] tensor: lane's 4 rows of column col.
template <typename T>
__device__ __forceinline__ void store_tile_rows(T* base, int D, const TokIdx& ti, int rowblk, int col,
                                                const floatx4& v, int nvalid, int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * rowblk + 4 * g4 + j;
    if (row < nvalid) base[(ti.row0 + (int64_t)row * ti.rstride) * D + col] = from_f32<T>(v[j]);
  }
}

template <typename T>
__device__ __forceinline__ floatx4 load_tile_rows_f32(const float* base, int D, const TokIdx& ti, int rowblk,
                                                      int col, int nvalid, int lane) {
  const int g4 = lane >> 4;
  floatx4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * rowblk + 4 * g4 + j;
    r[j] = row < nvalid ? base[(ti.row0 + (int64_t)row * ti.rstride) * D + col] : 0.f;
  }
  return r;
}

// state tile io: S[(head*DK + row) * DV + col], tile nt at columns col + 16 nt
template <int DK, int DV, int NTILE>
__device__ __forceinline__ void load_state(floatx4 (&S)[NTILE][DK / 16], const float* S0, int64_t head, int col,
                                           int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S[nt][rt][j] = S0 ? S0[(head * DK + 16 * rt + 4 * g4 + j) * DV + col + 16 * nt] : 0.f;
}

template <int DK, int DV, int NTILE>
__device__ __forceinline__ void store_state(const floatx4 (&S)[NTILE][DK / 16], float* out, int64_t head, int col,
                                            int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[(head * DK + 16 * rt + 4 * g4 + j) * DV + col + 16 * nt] = S[nt][rt][j];
}

// Workgroup -> (head, split): the NSPLIT workgroups of one head get block ids
// congruent modulo 8, so they are dispatched to the same XCD and share its L2
// for the chunk inputs they all read.
template <int NSPLIT>
__device__ __forceinline__ void block_to_head(int bid, int& head, int& split) {
  const int x = bid & 7, y = bid >> 3;
  split = y % NSPLIT;
  head = (y / NSPLIT) * 8 + x;
}

// Issue the global loads of chunk n into registers (zero past the end).
template <typename T, int DK, int DV, int DVW>
__device__ __forceinline__ void fetch_chunk(ChunkRegs<T, DK, DV, DVW>& rg, const PrefillArgs& a, int bb, int h,
                                            int n, int col0, int tid) {
  const int t0 = n * C;
  const int nv = min(C, a.T - t0);
  const int64_t tok0 = ((int64_t)bb * a.T + t0) * a.H + h;
  const int es = (int)sizeof(T);
  const uint32_t kb = chunk_bytes(nv, a.H * DK, DK, es);
  buf_load_rows<T, DK>(rg.q, make_rsrc(reinterpret_cast<const T*>(a.q) + tok0 * DK, kb), a.H * DK, tid);
  buf_load_rows<T, DK>(rg.k, make_rsrc(reinterpret_cast<const T*>(a.k) + tok0 * DK, kb), a.H * DK, tid);
  buf_load_rows<T, DK>(rg.g, make_rsrc(reinterpret_cast<const T*>(a.g) + tok0 * DK, kb), a.H * DK, tid);
  buf_load_rows<T, DVW>(rg.v, make_rsrc(reinterpret_cast<const T*>(a.v) + tok0 * DV + col0,
                                        chunk_bytes(nv, a.H * DV, DVW, es)), a.H * DV, tid);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<const T*>(a.beta) + tok0, chunk_bytes(nv, a.H, 1, es));
  const uint32_t boff = tid < C ? (uint32_t)(tid * a.H * es) : 0x80000000u;
  if constexpr (sizeof(T) == 2)
    rg.beta_bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, boff, 0, 0);
  else
    rg.beta_bits = __builtin_amdgcn_raw_buffer_load_b32(rb, boff, 0, 0);
}


// ---------------------------------------------------------------------------
// Fused forward.
// ---------------------------------------------------------------------------
// One 16x16 tile with compile-time block indices (straight-line code, so the
// operand reads and MFMAs of consecutive tiles overlap).  IS_L: L tile (I > J
// to Ln as -L, I == J to Ld in fp32); else P tile (I < J written as zeros).
template <typename T, int DK, int DVW, bool IS_L, int I, int J>
__device__ __forceinline__ void lp_tile_ct(Smem<T, DK, DVW>& sm, int lane) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (I >= J) {
    const TL* A = IS_L ? sm.Kt : sm.Qt;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const typename M::F32 af = M::lds32(A + (16 * I + l16) * Lay::LDK + 32 * ks + 4 * g4);
      const typename M::F32 bf = M::lds32(sm.Kh + (16 * J + l16) * Lay::LDK + 32 * ks + 4 * g4);
      acc = M::mma32(af, bf, acc);
    }
  }
  if constexpr (IS_L) {
    const floatx4 bt = *reinterpret_cast<const floatx4*>(&sm.beta[16 * I + 4 * g4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int il = 4 * g4 + j;
      float val = acc[j] * bt[j];
      if constexpr (I == J) {
        sm.Ld[(I * 16 + il) * Lay::LDL + l16] = (il > l16) ? val : 0.f;
      } else {
        sm.Ln[(16 * I + il) * Lay::LDC + 16 * J + l16] = from_f32<TF>(-val);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int il = 4 * g4 + j;
      float val = acc[j];
      if constexpr (I == J) val = (il > l16) ? val : (il == l16 ? sm.qk[16 * I + il] : 0.f);
      if constexpr (I < J) val = 0.f;
      sm.P[(16 * I + il) * Lay::LDC + 16 * J + l16] = from_f32<TF>(val);
    }
  }
}

// The off-diagonal L blocks and the P blocks, split over four "tile"
// wavefronts (tw = 0..3) with the same MFMA count each.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void lp_tile_schedule(Smem<T, DK, DVW>& sm, int tw, int lane) {
  switch (tw) {
    case 0:
      lp_tile_ct<T, DK, DVW, true, 1, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, true, 2, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 0, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 1, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 0, 1>(sm, lane);
      break;
    case 1:
      lp_tile_ct<T, DK, DVW, true, 2, 1>(sm, lane);
      lp_tile_ct<T, DK, DVW, true, 3, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 1, 1>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 2, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 2, 3>(sm, lane);
      break;
    case 2:
      lp_tile_ct<T, DK, DVW, true, 3, 1>(sm, lane);
      lp_tile_ct<T, DK, DVW, true, 3, 2>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 2, 1>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 2, 2>(sm, lane);
      break;
    default:
      lp_tile_ct<T, DK, DVW, false, 3, 0>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 3, 1>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 3, 2>(sm, lane);
      lp_tile_ct<T, DK, DVW, false, 3, 3>(sm, lane);
      break;
  }
}

// Diagonal block b of L and its inverse (I + L_bb)^-1 by forward
// substitution, lane c (mod 16) solving for column c.  The whole block is read
// into registers first, so the substitution chain waits on LDS only once.
template <typename T, int DK, int DVW, int B>
__device__ __forceinline__ void diag_block_inverse_ct(Smem<T, DK, DVW>& sm, int lane) {
  typedef Layout<T, DK, DVW> Lay;
  lp_tile_ct<T, DK, DVW, true, B, B>(sm, lane);      // same wavefront: LDS order suffices
  const int c = lane & 15;
  const float* Lb = sm.Ld + B * 16 * Lay::LDL;
  float Lr[16][16];
#pragma unroll
  for (int r = 1; r < 16; ++r)
#pragma unroll
    for (int m4 = 0; m4 < (r + 3) / 4; ++m4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(Lb + r * Lay::LDL + 4 * m4);
      Lr[r][4 * m4 + 0] = v[0]; Lr[r][4 * m4 + 1] = v[1]; Lr[r][4 * m4 + 2] = v[2]; Lr[r][4 * m4 + 3] = v[3];
    }
  // keep every read above this point: one wait for all of them instead of one
  // per row group
  __builtin_amdgcn_sched_barrier(0);
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float sacc = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < r; ++m) sacc -= Lr[r][m] * x[m];
    x[r] = sacc;
  }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.Db[(B * 16 + r) * Lay::LDD + c] = from_f32<typename Operands<T>::TF>(x[r]);
  }
}

template <typename T, int DK, int DVW>
__device__ __forceinline__ void diag_block_inverse(Smem<T, DK, DVW>& sm, int b, int lane) {
  switch (b) {
    case 0: diag_block_inverse_ct<T, DK, DVW, 0>(sm, lane); break;
    case 1: diag_block_inverse_ct<T, DK, DVW, 1>(sm, lane); break;
    case 2: diag_block_inverse_ct<T, DK, DVW, 2>(sm, lane); break;
    default: diag_block_inverse_ct<T, DK, DVW, 3>(sm, lane); break;
  }
}

// Re-derive the thread / lane ids from an opaque copy: per-lane index
// arithmetic is then recomputed in each phase (a few VALU ops) instead of
// being hoisted out of the chunk loop and held in registers for its length.
#define KDA_FRESH_LANE()                           \
  do {                                             \
    int t_ = threadIdx.x;                          \
    asm volatile("" : "+v"(t_));                   \
    tid = t_;                                      \
    lane = t_ & 63;                                \
  } while (0)

// The gate phase of one chunk, shared by both wavefront roles: log2-scaled
// in-chunk cumulative sum, the gated operands, and the next chunk's loads.
// Three barriers; leaves the LDS view rebased after the last one.
template <typename T, int DK, int DV, int DVW>
__device__ __forceinline__ void gate_phase(Smem<T, DK, DVW>& sm, unsigned char* smem_raw, ChunkRegs<T, DK, DV, DVW>& rg,
                                           const PrefillArgs& a, int bb, int h, int n, int nchunks, int col0,
                                           int& tid, int& lane) {
  sm.sync_rebase(smem_raw);              // previous chunk is done with LDS
  KDA_FRESH_LANE();
  stage_gates<T, DK, DVW>(sm, rg.g, bits_to_f32<T>(rg.beta_bits), tid, kLog2e);
  __syncthreads();
  chunk_cumsum<T, DK, DVW>(sm, tid);
  sm.sync_rebase(smem_raw);
  KDA_FRESH_LANE();
  apply_gates<T, DK, DVW, true, true, true, true>(sm, rg.k, rg.q, tid);
  stage_values<T, DK, DVW>(sm, rg.v, tid);
  // Next chunk's loads overlap this chunk's math.  Issued unconditionally:
  // past the last chunk the buffer range is empty and they return zeros.  (A
  // branch here would make the loaded registers merge with the old ones and
  // force a wait for the loads right away.)
  fetch_chunk<T, DK, DV, DVW>(rg, a, bb, h, n + 1, col0, tid);
  sm.sync_rebase(smem_raw);
  KDA_FRESH_LANE();
}

// ---------------------------------------------------------------------------
// Fused forward.  The workgroup's wavefronts take two roles, each running its
// own copy of the chunk loop with the same barrier sequence (seven per chunk):
//   owners (waves 0..OWN-1): hold 16*NTILE state columns in registers; take
//     tile-schedule slots of L / P and read the entry state (O = Qt S), solve
//     their U tiles, then Delta, O += P Delta, the output and the S update.
//   workers (the rest): waves OWN..OWN+3 each invert one diagonal block of L,
//     the others take the remaining tile-schedule slots; all solve W tiles.
// Separate loops keep the state registers and the workers' temporaries apart,
// so the prefetched next chunk never has to leave its registers early.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV, int NSPLIT>
__global__ __launch_bounds__(NT) void fused_fwd_kernel(PrefillArgs a) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TF> MF;
  constexpr int DVW = DV / NSPLIT;
  constexpr int NTILE = StateTiles<DVW>::NTILE;
  constexpr int OWN = StateTiles<DVW>::OWN;
  typedef Layout<T, DK, DVW> Lay;
  static_assert(OWN >= 1 && OWN <= 4, "column split");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];

  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int head, split;
  block_to_head<NSPLIT>(blockIdx.x, head, split);
  if (head >= a.B * a.H) return;
  const int bb = head / a.H, h = head % a.H;
  const int col0 = split * DVW;
  const int nchunks = (a.T + C - 1) / C;
  ChunkRegs<T, DK, DV, DVW> rg;
  if (nchunks > 0) fetch_chunk<T, DK, DV, DVW>(rg, a, bb, h, 0, col0, tid);
  Smem<T, DK, DVW> sm(smem_raw);

  if (wave < OWN) {
    // ------------------------------------------------------------ owners
    const int wcol = col0 + 16 * NTILE * wave;   // first state column
    floatx4 S[NTILE][DK / 16];
    load_state<DK, DV, NTILE>(S, a.S0, head, wcol + (lane & 15), lane);
    for (int n = 0; n < nchunks; ++n) {
      const int t0 = n * C;
      const int nv = min(C, a.T - t0);
      gate_phase<T, DK, DV, DVW>(sm, smem_raw, rg, a, bb, h, n, nchunks, col0, tid, lane);

      // this owner's share of the L / P blocks, and the read-out of the
      // chunk-entry state O = Qt S (needs only the gated queries)
      lp_tile_schedule<T, DK, DVW>(sm, wave, lane);
      floatx4 O[NTILE][4];
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I) O[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
      rows_times_state<TL, DK, NTILE, false>(sm.Qt, sm.Qt, Lay::LDK, S, O, O, lane);
      sm.sync_rebase(smem_raw);
      KDA_FRESH_LANE();

      // this owner's U tiles, kept in registers
      floatx4 Ux[NTILE][4];
      int ucol[NTILE];
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) ucol[nt] = 16 * (NTILE * wave + nt);
      fwd_subst_tiles<T, DK, DVW, T, NTILE>(sm, sm.V, Lay::LDV, ucol, Ux, lane);
      sm.sync_rebase(smem_raw);
      KDA_FRESH_LANE();

      // Delta = U - W S (Ux holds U), the intra-chunk term O += P Delta, and
      // the state update
      rows_times_state<TL, DK, NTILE, false>(sm.Wn, sm.Wn, Lay::LDK, S, Ux, Ux, lane);
      typename MF::F32 Df[NTILE][2];
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) {
        Df[nt][0] = MF::frag32(Ux[nt][0], Ux[nt][1]);
        Df[nt][1] = MF::frag32(Ux[nt][2], Ux[nt][3]);
      }
      intra_output<T, DK, DVW, NTILE>(sm, Df, O, lane);
      const int64_t tok0 = ((int64_t)bb * a.T + t0) * a.H + h;
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc(reinterpret_cast<T*>(a.o) + tok0 * DV, chunk_bytes(nv, a.H * DV, DV, (int)sizeof(T)));
      store_output<T, DK, DVW, NTILE>(sm, O, wave, ro, a.H * DV, wcol, lane);
      state_update<T, DK, DVW, NTILE>(sm, Df, S, lane);
    }
    if (a.S_T) store_state<DK, DV, NTILE>(S, a.S_T, head, wcol + (lane & 15), lane);
  } else {
    // ------------------------------------------------------------ workers
    constexpr int NNO = NW - OWN;
    for (int n = 0; n < nchunks; ++n) {
      gate_phase<T, DK, DV, DVW>(sm, smem_raw, rg, a, bb, h, n, nchunks, col0, tid, lane);

      // waves OWN..OWN+3 invert the diagonal blocks of L; the rest take the
      // tile schedule slots the owners leave
      if (wave < OWN + 4) diag_block_inverse<T, DK, DVW>(sm, wave - OWN, lane);
      else lp_tile_schedule<T, DK, DVW>(sm, wave - 4, lane);
      sm.sync_rebase(smem_raw);
      KDA_FRESH_LANE();

      // W tiles i = wave - OWN + k (NW - OWN), two at a time, to LDS as -W
      for (int i = wave - OWN; i < DK / 16; i += 2 * NNO) {
        if (i + NNO < DK / 16) {
          const int wc[2] = {16 * i, 16 * (i + NNO)};
          floatx4 Wx[2][4];
          fwd_subst_tiles<T, DK, DVW, TL, 2>(sm, sm.Kt, Lay::LDK, wc, Wx, lane);
          store_negw<T, DK, DVW>(sm, Wx[0], wc[0], lane);
          store_negw<T, DK, DVW>(sm, Wx[1], wc[1], lane);
        } else {
          floatx4 Wx[4];
          fwd_subst_tile<T, DK, DVW>(sm, sm.Kt, Lay::LDK, 16 * i, Wx, lane);
          store_negw<T, DK, DVW>(sm, Wx, 16 * i, lane);
        }
      }
      sm.sync_rebase(smem_raw);
      KDA_FRESH_LANE();
      // (the owners' Delta / output / state update runs here)
    }
  }
}

// ---------------------------------------------------------------------------
// Staged schedule.
// ---------------------------------------------------------------------------

// b = in-chunk cumsum of g (fp32 out).  grid (chunks, B*H)
template <typename T, int DK>
__global__ __launch_bounds__(NT) void stage_cumsum_kernel(StageArgs a) {
  typedef Layout<T, DK, 16> Lay;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem<T, DK, 16> sm(smem_raw);
  const int tid = threadIdx.x;
  const int n = blockIdx.x, head = blockIdx.y;
  const int bb = head / a.H, h = head % a.H;
  const int t0 = n * C, nv = min(C, a.T - t0);
  TokIdx ti;
  ti.row0 = ((int64_t)bb * a.T + t0) * a.H + h;
  ti.rstride = a.H;
  Vec16 gr[RowVecs<T, DK>::PER];
  load_rows<T, DK>(gr, reinterpret_cast<const T*>(a.g), DK, 0, ti, nv, tid);
  stage_gates<T, DK, 16>(sm, gr, 0.f, tid, 1.0f);   // natural-log units: b is an output
  __syncthreads();
  chunk_cumsum<T, DK, 16>(sm, tid);
  __syncthreads();
  for (int idx = tid; idx < C * DK; idx += NT) {
    const int row = idx / DK, c = idx % DK;
    if (row < nv)
      a.b[(ti.row0 + (int64_t)row * ti.rstride) * DK + c] = sm.G[row * Lay::LDG + GateCols<DK, VecTraits<T>::N>::pos(c)];
  }
}

// load fp32 b rows into G, and bC/gam from the last valid row
template <typename T, int DK, int DVW>
__device__ __forceinline__ void load_b(Smem<T, DK, DVW>& sm, const float* b, const TokIdx& ti, int nv, int tid) {
  typedef Layout<T, DK, DVW> Lay;
  for (int idx = tid; idx < C * DK; idx += NT) {
    const int row = idx / DK, c = idx % DK;
    // rows past the end repeat the last valid row (zero gate beyond T)
    const int rr = row < nv ? row : nv - 1;
    sm.G[row * Lay::LDG + GateCols<DK, VecTraits<T>::N>::pos(c)] =
        kLog2e * b[(ti.row0 + (int64_t)rr * ti.rstride) * DK + c];
  }
  if (tid < DK) {
    const float bl = kLog2e * b[(ti.row0 + (int64_t)(nv - 1) * ti.rstride) * DK + tid];
    sm.bC[tid] = bl;
    sm.gam[tid] = hw_exp2(bl);
  }
}

// W, U per chunk.  grid (chunks, B*H)
template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void stage_ut_kernel(StageArgs a) {
  typedef Layout<T, DK, DV> Lay;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem<T, DK, DV> sm(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x, head = blockIdx.y;
  const int bb = head / a.H, h = head % a.H;
  const int t0 = n * C, nv = min(C, a.T - t0);
  TokIdx ti;
  ti.row0 = ((int64_t)bb * a.T + t0) * a.H + h;
  ti.rstride = a.H;
  Vec16 kr[RowVecs<T, DK>::PER];
  Vec16 vr[RowVecs<T, DV>::PER];
  load_rows<T, DK>(kr, reinterpret_cast<const T*>(a.k), DK, 0, ti, nv, tid);
  load_rows<T, DV>(vr, reinterpret_cast<const T*>(a.v), DV, 0, ti, nv, tid);
  const float beta = (tid < nv) ? to_f32(reinterpret_cast<const T*>(a.beta)[ti.row0 + (int64_t)tid * ti.rstride]) : 0.f;
  load_b<T, DK, DV>(sm, a.b, ti, nv, tid);
  if (tid < C) sm.beta[tid] = beta;
  __syncthreads();
  apply_gates<T, DK, DV, true, true, false, false>(sm, kr, kr, tid);
  stage_values<T, DK, DV>(sm, vr, tid);
  __syncthreads();
  intra_chunk_matrices<T, DK, DV, true, false>(sm, wave, lane);
  __syncthreads();
  const int l16 = lane & 15;
  for (int t = wave; t < DK / 16 + DV / 16; t += NW) {
    floatx4 X[4];
    if (t < DK / 16) {
      fwd_subst_tile<T, DK, DV>(sm, sm.Kt, Lay::LDK, 16 * t, X, lane);
#pragma unroll
      for (int I = 0; I < 4; ++I) store_tile_rows<float>(a.W, DK, ti, I, 16 * t + l16, X[I], nv, lane);
    } else {
      const int vc = 16 * (t - DK / 16);
      fwd_subst_tile<T, DK, DV>(sm, sm.V, Lay::LDV, vc, X, lane);
#pragma unroll
      for (int I = 0; I < 4; ++I) store_tile_rows<float>(a.U, DV, ti, I, vc + l16, X[I], nv, lane);
    }
  }
}

// Sequential state pass.  grid (B*H*NSPLIT) with the fused kernel's mapping.
template <typename T, int DK, int DV, int NSPLIT>
__global__ __launch_bounds__(NT) void stage_state_kernel(StageArgs a) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> ML;
  typedef Mma<TF> MF;
  constexpr int DVW = DV / NSPLIT;
  constexpr int OWN = DVW / 16;
  typedef Layout<T, DK, DVW> Lay;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem<T, DK, DVW> sm(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int head, split;
  block_to_head<NSPLIT>(blockIdx.x, head, split);
  if (head >= a.B * a.H) return;
  const int bb = head / a.H, h = head % a.H;
  const bool owner = wave < OWN;
  const int wcol = split * DVW + 16 * wave;
  const int l16 = lane & 15;
  const int nchunks = (a.T + C - 1) / C;

  floatx4 S[1][DK / 16];
  if (owner) load_state<DK, DV, 1>(S, a.S0, head, wcol + l16, lane);
  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * C, nv = min(C, a.T - t0);
    TokIdx ti;
    ti.row0 = ((int64_t)bb * a.T + t0) * a.H + h;
    ti.rstride = a.H;
    Vec16 kr[RowVecs<T, DK>::PER];
    load_rows<T, DK>(kr, reinterpret_cast<const T*>(a.k), DK, 0, ti, nv, tid);
    __syncthreads();
    load_b<T, DK, DVW>(sm, a.b, ti, nv, tid);
    for (int idx = tid; idx < C * DK; idx += NT) {
      const int row = idx / DK, c = idx % DK;
      const float w = row < nv ? a.W[(ti.row0 + (int64_t)row * ti.rstride) * DK + c] : 0.f;
      sm.Wn[row * Lay::LDK + c] = from_f32<TL>(-w);
    }
    __syncthreads();
    apply_gates<T, DK, DVW, false, false, false, true>(sm, kr, kr, tid);
    __syncthreads();
    if (owner) {
      const int64_t nstates = (int64_t)nchunks;
      float* Sc = a.S_chunks + ((int64_t)head * nstates + n) * DK * DV;
#pragma unroll
      for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sc[(int64_t)(16 * rt + 4 * (lane >> 4) + j) * DV + wcol + l16] = S[0][rt][j];
      floatx4 Dx[1][4], unused[1][4];
#pragma unroll
      for (int I = 0; I < 4; ++I) Dx[0][I] = load_tile_rows_f32<T>(a.U, DV, ti, I, wcol + l16, nv, lane);
      rows_times_state<TL, DK, 1, false>(sm.Wn, sm.Wn, Lay::LDK, S, Dx, unused, lane);
#pragma unroll
      for (int I = 0; I < 4; ++I) store_tile_rows<float>(a.Delta, DV, ti, I, wcol + l16, Dx[0][I], nv, lane);
      typename MF::F32 Df[1][2];
      Df[0][0] = MF::frag32(Dx[0][0], Dx[0][1]);
      Df[0][1] = MF::frag32(Dx[0][2], Dx[0][3]);
      state_update<T, DK, DVW, 1>(sm, Df, S, lane);
    }
  }
  if (owner && a.S_T) store_state<DK, DV, 1>(S, a.S_T, head, wcol + l16, lane);
}

// O = Qt S_[n] + Tril(Qt Kh^T) Delta.  grid (chunks, B*H)
template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void stage_output_kernel(StageArgs a) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> ML;
  typedef Mma<TF> MF;
  typedef Layout<T, DK, DV> Lay;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem<T, DK, DV> sm(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x, head = blockIdx.y;
  const int bb = head / a.H, h = head % a.H;
  const int t0 = n * C, nv = min(C, a.T - t0);
  const int nchunks = (a.T + C - 1) / C;
  const int l16 = lane & 15;
  TokIdx ti;
  ti.row0 = ((int64_t)bb * a.T + t0) * a.H + h;
  ti.rstride = a.H;
  Vec16 kr[RowVecs<T, DK>::PER], qr[RowVecs<T, DK>::PER];
  load_rows<T, DK>(kr, reinterpret_cast<const T*>(a.k), DK, 0, ti, nv, tid);
  load_rows<T, DK>(qr, reinterpret_cast<const T*>(a.q), DK, 0, ti, nv, tid);
  load_b<T, DK, DV>(sm, a.b, ti, nv, tid);
  __syncthreads();
  apply_gates<T, DK, DV, false, true, true, false>(sm, kr, qr, tid);
  __syncthreads();
  intra_chunk_matrices<T, DK, DV, false, true>(sm, wave, lane);
  __syncthreads();
  for (int ct = wave; ct < DV / 16; ct += NW) {
    const int col = 16 * ct + l16;
    floatx4 S[1][DK / 16];
    const float* Sc = a.S_chunks + ((int64_t)head * nchunks + n) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[0][rt][j] = Sc[(int64_t)(16 * rt + 4 * (lane >> 4) + j) * DV + col];
    floatx4 O[1][4], unused[1][4];
#pragma unroll
    for (int I = 0; I < 4; ++I) O[0][I] = floatx4{0.f, 0.f, 0.f, 0.f};
    rows_times_state<TL, DK, 1, false>(sm.Qt, sm.Qt, Lay::LDK, S, O, unused, lane);
    floatx4 Dx[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) Dx[I] = load_tile_rows_f32<T>(a.Delta, DV, ti, I, col, nv, lane);
    typename MF::F32 Df[1][2];
    Df[0][0] = MF::frag32(Dx[0], Dx[1]);
    Df[0][1] = MF::frag32(Dx[2], Dx[3]);
    intra_output<T, DK, DV, 1>(sm, Df, O, lane);
#pragma unroll
    for (int I = 0; I < 4; ++I) store_tile_rows<T>(reinterpret_cast<T*>(a.o), DV, ti, I, col, O[0][I], nv, lane);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined forward for bf16 inputs with d_k = d_v = 128.
//
// Only the readout O = Qt S + P Delta and the update of S depend on the state;
// everything else of a chunk (gates, gated operands, L, (I+L)^-1, W, U, P) does
// not.  The workgroup therefore runs two chunks at once: while the four owner
// wavefronts (state columns 32o..32o+31 in registers) finish chunk n, the four
// worker wavefronts prepare chunk n+1.  One "slot" has four phases separated
// by workgroup barriers:
//   1   owners: Delta = U - W S, O += P Delta, store O, S update      (chunk n)
//       workers: in-chunk cumsum of the gates, Kt Kh Qt Kt^T          (n+1)
//   2a  owners: P tiles;  worker 0: diagonal L blocks and their inverses;
//       workers 1-3: off-diagonal L blocks;  all workers: Kb^T, V^T    (n+1)
//   2b  owners: O = Qt S (entry state of n+1);  worker 0: the off-diagonal
//       blocks of A' = (I+L)^-1 Diag(beta)                             (n+1)
//   3   workers: W = A' Kt;  owners: U = A' V                          (n+1)
// The inverse is formed explicitly (blocked, 16x16 diagonal blocks solved by
// substitution in fp32, couplings on MFMA), so that W and U are plain
// products.  Worker wavefront w owns gate channels 32w..32w+31 of every token:
// its lanes hold 4 consecutive tokens x 8 channels, the in-chunk prefix sum
// runs in registers (DPP row shifts across the 16 token groups), and the
// transposed operands are written 4 tokens at a time.
// ---------------------------------------------------------------------------
// Internal template flags of fused_pipe_kernel, beside the variant bits: the
// state-mode instantiation (chunk-entry states out, no outputs), so that the
// forward proper carries none of its code; and the instantiation of the
// segmented schedule's first pass, the only one that holds the two-state
// owners (whose registers would otherwise size every other launch too).
constexpr int kPipeStates = 4;
constexpr int kPipeDual = 8;
// and the third pass's instantiation, whose entry states come from the
// workspace in the owners' fragment order (sfrag_index)
constexpr int kPipeSegIn = 16;

namespace pipe {

constexpr int DK = 128, DV = 128;
constexpr int LDK = DK + 16;     // bf16 [C][DK] rows (16-byte chunks swizzled, see rmo)
constexpr int LDT = C + 16;      // fp16 [D][C] rows (transposed operands), [C][C] rows
constexpr int LDB = 24;          // fp16 16x16 solver blocks
constexpr int LDL = 20;          // fp32 16x16 diagonal blocks of L (transposed)
constexpr int SZ_RM = C * LDK * 2;
constexpr int SZ_TR = DK * LDT * 2;
constexpr int SZ_CC = C * LDT * 2;
constexpr int O_KT = 0;
constexpr int O_KH = O_KT + SZ_RM;
constexpr int O_QT = O_KH + SZ_RM;
constexpr int O_WN = O_QT + SZ_RM;       // -W; scratch of the solver wavefront in phase 2
constexpr int O_KTT = O_WN + SZ_RM;
constexpr int O_KBT = O_KTT + SZ_TR;
constexpr int O_VT = O_KBT + SZ_TR;      // V^T
constexpr int O_P = O_VT + SZ_TR;
constexpr int O_A = O_P + SZ_CC;
constexpr int O_BETA = O_A + SZ_CC;
constexpr int O_GAM = O_BETA + C * 4;    // two chunk parities
constexpr int O_QK = O_GAM + 2 * DK * 4;  // q_t . k_t partial sums, per worker
constexpr int NQK = 16;                   // q.k partial sums per token (worker lane groups)
// Operand reference of each chunk: the integer log2 exponent rho_c per key
// channel that the gated operands are taken relative to (three buffers, by
// chunk index mod 3), and per worker two flag bits (two chunk parities):
// bit 0 its channels' referenced operands fit fp16, bit 1 a reference moved.
constexpr int O_RHO = O_QK + NQK * C * 4;  // int [3][DK]
constexpr int O_FLG = O_RHO + 3 * DK * 4;  // int [2][4]
constexpr int BYTES = O_FLG + 2 * 4 * 4;
// solver scratch inside the -W region
constexpr int S_LDT = 0;                           // fp32 [4][16][LDL]: L_II^T
constexpr int S_LN = S_LDT + 4 * 16 * LDL * 4;     // fp16 [6][16][LDB]: -L_IJ, I > J
constexpr int S_D = S_LN + 6 * 16 * LDB * 2;       // fp16 [4][16][LDB]: D_I = (I + L_II)^-1
constexpr int S_DT = S_D + 4 * 16 * LDB * 2;       // fp16 [4][16][LDB]: D_I^T
constexpr int S_END = S_DT + 4 * 16 * LDB * 2;
static_assert(S_END <= SZ_RM, "solver scratch");
static_assert(BYTES <= 160 * 1024, "LDS");

struct Ptr {
  bf16 *Kt, *Kh, *Qt, *Wn;
  f16 *KtT, *KbT, *VT, *P, *A;
  float *beta, *gam, *qk;
  float* rho;
  int* flg;
  float* LdT; f16 *Ln, *D, *Dt;
  __device__ __forceinline__ void set(unsigned char* b) {
    Kt = reinterpret_cast<bf16*>(b + O_KT);
    Kh = reinterpret_cast<bf16*>(b + O_KH);
    Qt = reinterpret_cast<bf16*>(b + O_QT);
    Wn = reinterpret_cast<bf16*>(b + O_WN);
    KtT = reinterpret_cast<f16*>(b + O_KTT);
    KbT = reinterpret_cast<f16*>(b + O_KBT);
    VT = reinterpret_cast<f16*>(b + O_VT);
    P = reinterpret_cast<f16*>(b + O_P);
    A = reinterpret_cast<f16*>(b + O_A);
    beta = reinterpret_cast<float*>(b + O_BETA);
    gam = reinterpret_cast<float*>(b + O_GAM);
    qk = reinterpret_cast<float*>(b + O_QK);
    rho = reinterpret_cast<float*>(b + O_RHO);
    flg = reinterpret_cast<int*>(b + O_FLG);
    LdT = reinterpret_cast<float*>(b + O_WN + S_LDT);
    Ln = reinterpret_cast<f16*>(b + O_WN + S_LN);
    D = reinterpret_cast<f16*>(b + O_WN + S_D);
    Dt = reinterpret_cast<f16*>(b + O_WN + S_DT);
  }
  // barrier, then rebuild the pointers from an offset the compiler cannot see
  // through, so that each phase computes its own LDS addresses
  __device__ __forceinline__ void sync(unsigned char* b) {
    __syncthreads();
    uint32_t opq = 0;
    asm volatile("" : "+s"(opq));
    set(b + opq);
  }
};

typedef Mma<bf16> MB;
typedef Mma<f16> MH;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Reduction-index order in LDS.  A product with one operand from registers in
// C layout (the state S, or Delta) reads, for lane group g, the indices
// {4g..4g+3, 16+4g..16+4g+3} of each 32-index slab.  The arrays read against
// such operands (Kt Kh Qt -W along the key channels, Kb^T and P along the
// tokens) store index k of a slab at position slot32(k), which makes that set
// the 16 contiguous bytes at 8g: one ds_read_b128 per fragment instead of two
// 8-byte reads.  Products of two such arrays read both the same way and pair
// the same indices.
__device__ __forceinline__ int slot32(int k) {
  return (k & ~31) + 8 * ((k & 15) >> 2) + 4 * ((k >> 4) & 1) + (k & 3);
}

// Element offset of element e of token row t in the row-major bf16 arrays
// (Kt, Kh, Qt, -W): rows of 144 elements, and the 16-byte chunks of row t
// permuted by XOR with (t / 4) mod 8.  With this pitch and swizzle the MFMA
// fragment reads (16 rows x one chunk per lane group) are free of LDS bank
// conflicts, and the workers' 8-byte stores of rows 4m + i are at most
// 2-way (measured with the LDS bank-conflict counter: natural rows of 136
// elements gave 2-way conflicts on every fragment read and 8-way on the
// stores).  [D][C] fp16 rows of 80 elements likewise make their fragment
// reads conflict-free.
__device__ __forceinline__ int rmo(int t, int e) { return t * LDK + (e ^ ((t << 1) & 56)); }
// The same offsets split into a per-lane part and a compile-time part, so
// that each access is one immediate offset from a lane base:
//  * MFMA fragment of rows 16I + l16, 32-element slab ks, lane group g4:
//    rmo(16I + l16, 32ks + 8g4) = frag_lane + frag_off(I, ks);
//  * stores of rows 16I + l16 at element 32s + 8g4 + e (e < 8): likewise with
//    slab s and + e.
__device__ __forceinline__ int frag_lane(int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  return l16 * LDK + ((8 * g4) ^ ((2 * l16) & 24));
}
__device__ __forceinline__ constexpr int frag_off(int I, int ks) { return 16 * I * LDK + 32 * (ks ^ (I & 1)); }

// Value column, relative to the owner's first, of column i of the owner's
// state tile nt.  An owner's two 16-column MFMA tiles interleave in groups of
// four, so that the four output columns a lane holds in each tile (4g..4g+3)
// are the 8 adjacent columns 8g..8g+7: one 16-byte store per token.
__device__ __forceinline__ int vcol(int nt, int i) { return 8 * (i >> 2) + 4 * nt + (i & 3); }

// State tiles of an owner in that column order, from / to one head's fp32
// [d_k][d_v] matrix (S0 NULL: zeros; ident: the identity).
__device__ __forceinline__ void load_state_v(floatx4 (&S)[2][DK / 16], const float* S0, bool ident, int col0,
                                             int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * g4 + j, col = col0 + vcol(nt, l16);
        S[nt][rt][j] = S0 ? S0[row * DV + col] : (ident && row == col ? 1.f : 0.f);
      }
}
__device__ __forceinline__ void store_state_v(const floatx4 (&S)[2][DK / 16], float* out, int col0, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[(16 * rt + 4 * g4 + j) * DV + col0 + vcol(nt, l16)] = S[nt][rt][j];
}

// The same tiles in fp32 in the owners' fragment order, for the segmented
// schedule's workspace (entry states and offsets N): owner o = col0 / 32, tile
// (nt, rt) is the 256-float block 8 (2 o + nt) + rt, inside which lane (g, i)
// holds elements 4 (16 g + i) .. + 3 = rows 16 rt + 4 g .. + 3 of value
// column col0 + vcol(nt, i): one 16-byte access per lane and tile, a whole
// 1 KB block per wave access.
__device__ __forceinline__ int sfrag_index(int r, int c) {
  const int cl = c & 31, nt = (cl >> 2) & 1, i = 4 * (cl >> 3) + (cl & 3);
  return ((8 * (2 * (c >> 5) + nt) + (r >> 4)) * 64 + 16 * ((r >> 2) & 3) + i) * 4 + (r & 3);
}
__device__ __forceinline__ void load_state_f(floatx4 (&S)[2][DK / 16], const float* src, int col0, int lane) {
  const floatx4* s4 = reinterpret_cast<const floatx4*>(src);
  const int o = col0 >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt) S[nt][rt] = s4[(8 * (2 * o + nt) + rt) * 64 + lane];
}
__device__ __forceinline__ void store_state_f(const floatx4 (&S)[2][DK / 16], float* out, int col0, int lane) {
  floatx4* o4 = reinterpret_cast<floatx4*>(out);
  const int o = col0 >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt) o4[(8 * (2 * o + nt) + rt) * 64 + lane] = S[nt][rt];
}

// The same tiles as bf16 in the owners' fragment order: owner o = col0 / 32,
// tile (nt, rt) is the 256-element block 8 (2 o + nt) + rt, inside which
// lane (g, i) holds elements 16 i + 4 g .. + 3, i.e. rows 16 rt + 4 g .. + 3
// of value column col0 + vcol(nt, i).  Each wave store writes one whole
// block (512 contiguous bytes), and the 16 key rows 16 rt .. + 15 of one
// value column are 32 contiguous bytes.
// (S is referenced, Diag(2^rho) S: each row is divided by 2^rho first.)
__device__ __forceinline__ void store_state_t(const floatx4 (&S)[2][DK / 16], const float* rho, bf16* out, int col0,
                                              int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int o = col0 >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt) {
      const floatx4 e = *reinterpret_cast<const floatx4*>(rho + 16 * rt + 4 * g4);
      bf16x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = (bf16)__builtin_amdgcn_ldexpf(S[nt][rt][j], -(int)e[j]);
      *reinterpret_cast<bf16x4*>(out + (8 * (2 * o + nt) + rt) * 256 + 16 * l16 + 4 * g4) = x;
    }
}

// Workspace matrix (fp32, d_k x d_v) of the segmented schedule: for sequence /
// head `head` and segment s, kind 0 = entry state, 1 = transition M, 2 = offset N
// (entry states and N in the owners' fp32 fragment order, sfrag_index; M as
// split bf16 parts in the combine's operand order, mfrag_index).
__device__ __forceinline__ float* seg_mat(float* ws, int64_t head, int nseg, int s, int kind) {
  return ws + ((head * nseg + s) * 3 + kind) * (int64_t)(DK * DV);
}

// Transition M of the segmented schedule for the combine kernel's products
// (v_mfma_f32_16x16x32_bf16 on a 16-row tile, M split into a bf16 high part
// and the bf16 rounding of the rest): element (r, c), part h (0 high, 1
// low) sits in the A-operand vector (16 bytes) of lane 16 ((c / 8) % 4) +
// r % 16 for row tile r / 16, 32-index slab c / 32 and part h, at position
// c % 8; a lane of the combine reads each of its operands as one vector.
__device__ __forceinline__ int mfrag_index(int r, int c, int h) {
  return ((((r >> 4) * 4 + (c >> 5)) * 2 + h) * 64 + 16 * ((c >> 3) & 3) + (r & 15)) * 8 + (c & 7);
}
// Owner o's columns 32o .. 32o+31 of M are exactly slab o of that order, so
// each owner writes its slab alone: its 128 x 32 block goes row-major into
// its own LDS area `stage` (128 rows of 36 floats), and each lane reads back
// the eight columns of one row that form one of its vectors, splits them and
// stores the high and the low vector (16 bytes each, a whole 1 KB block per
// wave store).  The area is read only by the wave that wrote it, after its
// writes (LDS operations of one wavefront complete in order).
constexpr int kMStageRow = 36;
__device__ __forceinline__ void store_state_mfrag(const floatx4 (&S)[2][DK / 16], float* out, int col0, int lane,
                                                  float* stage) {
  const int g4 = lane >> 4, l16 = lane & 15, o = col0 >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) stage[(16 * rt + 4 * g4 + j) * kMStageRow + vcol(nt, l16)] = S[nt][rt][j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  bf16x8* o16 = reinterpret_cast<bf16x8*>(out);
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt) {
    const float* src = stage + (16 * rt + l16) * kMStageRow + 8 * g4;
    const floatx4 x0 = *reinterpret_cast<const floatx4*>(src), x1 = *reinterpret_cast<const floatx4*>(src + 4);
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? x0[e] : x1[e - 4];
      hi[e] = (bf16)x;
      lo[e] = (bf16)(x - (float)hi[e]);
    }
    o16[((rt * 4 + o) * 2 + 0) * 64 + lane] = hi;
    o16[((rt * 4 + o) * 2 + 1) * 64 + lane] = lo;
  }
}

// Keeps a batch of LDS reads ahead of the products that use them (otherwise
// the scheduler sinks each read next to its product to save registers, and
// every product then waits for a full LDS round trip).
#define KDA_READS_FIRST() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void unpack8(const Vec16& v, float* f) {
#pragma unroll
  for (int k = 0; k < 4; ++k) { f[2 * k] = bf_lo(v.w[k]); f[2 * k + 1] = bf_hi(v.w[k]); }
}
// x + (value of the lane K places lower in the same 16-lane row, 0 if none)
template <int K>
__device__ __forceinline__ float add_row_shr(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + K, 0xF, 0xF, true));
}
// lane 15 of the caller's 16-lane row (ds_swizzle bit mode: and 0x10, or 0x0f)
__device__ __forceinline__ float row_last(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F0));
}

// Chunk inputs of one worker wavefront: rows 4m..4m+3 (m = lane % 16) and
// channels 32w + 8(lane / 16) .. +8.  (Owner o loads the value columns
// 32o.. of v in the same lane layout.)
struct WRegs {
  Vec16 q[4], k[4], g[4];
  uint32_t gs[4];      // scalar-gate variant: the gates of tokens 4m..4m+3 (bf16 bits)
  uint32_t beta_bits;
};

__device__ __forceinline__ uint32_t wlane_off(int H, int w, int lane) {
  return (uint32_t)((4 * (lane & 15) * H * DK + 32 * w + 8 * (lane >> 4)) * 2);
}

__device__ __forceinline__ Vec16 ld16(__amdgpu_buffer_rsrc_t rs, uint32_t vo, int so) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, 0);
  Vec16 v;
  v.w[0] = x[0]; v.w[1] = x[1]; v.w[2] = x[2]; v.w[3] = x[3];
  return v;
}

// Buffer resources and offsets of one chunk's q, k, g, beta for a worker.
// Scalar gate: g is [B, T, H] and the lane reads the gates of its tokens
// 4m..4m+3 (go, then gr bytes apart).  No delta rule: beta is not read.
template <int V>
struct QkgSrc {
  __amdgpu_buffer_rsrc_t q, k, g, b;
  uint32_t vo, boff, go;
  int rs, gr;
  __device__ __forceinline__ QkgSrc(const PrefillArgs& a, int bb, int h, int n, int w, int lane) {
    const int t0 = n * C, nv = min(C, a.T - t0);
    const int64_t tok0 = ((int64_t)bb * a.T + t0) * a.H + h;
    const uint32_t bytes = chunk_bytes(nv, a.H * DK, DK, 2);
    q = make_rsrc(reinterpret_cast<const bf16*>(a.q) + tok0 * DK, bytes);
    k = make_rsrc(reinterpret_cast<const bf16*>(a.k) + tok0 * DK, bytes);
    vo = wlane_off(a.H, w, lane);
    rs = a.H * DK * 2;
    if constexpr ((V & kVarScalarGate) != 0) {
      g = make_rsrc(reinterpret_cast<const bf16*>(a.g) + tok0, chunk_bytes(nv, a.H, 1, 2));
      go = (uint32_t)(4 * (lane & 15) * a.H * 2);
      gr = a.H * 2;
    } else {
      g = make_rsrc(reinterpret_cast<const bf16*>(a.g) + tok0 * DK, bytes);
      go = vo;
      gr = rs;
    }
    if constexpr ((V & kVarNoDelta) == 0) {
      b = make_rsrc(reinterpret_cast<const bf16*>(a.beta) + tok0, chunk_bytes(nv, a.H, 1, 2));
      boff = (uint32_t)(lane * a.H * 2);
    }
  }
  // this chunk's gates (of the variant's layout) into r
  __device__ __forceinline__ void load_g(WRegs& r) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr ((V & kVarScalarGate) != 0)
        r.gs[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(g, go, i * gr, 0);
      else
        r.g[i] = ld16(g, go, i * gr);
    }
  }
};

template <int V>
__device__ __forceinline__ void fetch_qkg(WRegs& r, const PrefillArgs& a, int bb, int h, int n, int w, int lane) {
  const QkgSrc<V> src(a, bb, h, n, w, lane);
  src.load_g(r);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = ld16(src.k, src.vo, i * src.rs);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.q[i] = ld16(src.q, src.vo, i * src.rs);
  if constexpr ((V & kVarNoDelta) == 0)
    r.beta_bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src.b, src.boff, 0, 0);
}

__device__ __forceinline__ void fetch_v(Vec16 (&v)[4], const PrefillArgs& a, int bb, int h, int n, int w, int lane) {
  const int t0 = n * C, nv = min(C, a.T - t0);
  const int64_t tok0 = ((int64_t)bb * a.T + t0) * a.H + h;
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(reinterpret_cast<const bf16*>(a.v) + tok0 * DV, chunk_bytes(nv, a.H * DV, DV, 2));
  const uint32_t vo = wlane_off(a.H, w, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, i * a.H * DV * 2, 0);
    v[i].w[0] = x[0]; v[i].w[1] = x[1]; v[i].w[2] = x[2]; v[i].w[3] = x[3];
  }
}

// In-chunk prefix sums of a worker's gate channels, log2-scaled (b[i][e]:
// token 4m + i, channel e of the lane's eight), and the chunk decay
// gm[e] = 2^b_C.  Computed one slot ahead of their use, in phase 2b where the
// workers are otherwise idle.
struct Gates {
  float b[4][8];
  float gm[8];
  float bc[8];   // b_C of each channel (unreferenced)
  float dev;     // largest distance of a referenced range from 0 (lane's channels)
};

// lane 0 of the caller's 16-lane row (ds_swizzle bit mode: and 0x10)
__device__ __forceinline__ float row_first(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x010));
}

// Operand precision of a chunk.  The products Qg Kd^T (P), Kg Kd^T (L) and
// Qg S only need the gate ratios 2^(b_t - b_j) (and, for Qg S, the state
// scaled by rows), so they use Qg' = q 2^(b - rho), Kg' = k 2^(b - rho),
// Kd' = k 2^(rho - b) and S' = Diag(2^rho) S for a per-channel reference
// exponent rho.  While every referenced exponent b - rho of a chunk lies
// within +-kRefBits, fp16 carries these operands with 3 more mantissa bits
// than bf16 at the same MFMA rate (the rounding of these gated operands is
// what dominates the output error with bf16 operands); a chunk beyond that
// (a channel decaying by more than 2 kRefBits bits inside one chunk, or a
// positive log-gate) keeps bf16 operands, for which any reference fits.
// The reference of a channel is sticky: it moves (to the middle of the
// chunk's range) only when a chunk leaves +-kRefBits around it, so the
// owners, which hold S' = Diag(2^rho) S instead of S, rarely rescale.
constexpr float kRefBits = 8.f;

// Combined flags of the four workers for the chunk of parity par: bit 0 all
// of them fit fp16, bit 1 a reference moved.  Wave-uniform.
__device__ __forceinline__ int chunk_flags(const Ptr& p, int par) {
  typedef int intx4 __attribute__((ext_vector_type(4)));
  const intx4 f = *reinterpret_cast<const intx4*>(p.flg + par * 4);
  const int all = f[0] & f[1] & f[2] & f[3], any = f[0] | f[1] | f[2] | f[3];
  return __builtin_amdgcn_readfirstlane((all & 1) | (any & 2));
}

// Largest value of a non-negative x over the wavefront (DPP row maxima, then
// the four row results), wave-uniform.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true)));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Prefix sums of the gates in r.g, log2-scaled and taken relative to the
// reference rho of each of the lane's channels; r.g is then reloaded with the
// gates of the chunk that nx addresses (the next scan's input).  With g <= 0
// the sums fall from b_1 <= 0 to b_C, so the referenced ones lie in
// [b_C - rho, -rho]; gt.bc keeps b_C and gt.dev the largest distance of that
// range from 0 over the lane's channels (ref_commit acts on it).  With a
// scalar gate the one sum per token is formed once and copied to all eight
// channels (whose references then stay equal).
template <int V>
__device__ __forceinline__ void worker_scan(WRegs& r, Gates& gt, const float (&rho)[8], const QkgSrc<V>& nx) {
  constexpr int NE = (V & kVarScalarGate) != 0 ? 1 : 8;   // distinct channels
  float x[4][NE];
  if constexpr (NE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i][0] = bf_lo(r.gs[i]) * kLog2e;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unpack8(r.g[i], x[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] *= kLog2e;
    }
  }
  nx.load_g(r);
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < NE; ++e) x[i][e] += x[i - 1][e];
  float dev = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const float tot = x[3][e];
    float s = add_row_shr<1>(tot);
    s = add_row_shr<2>(s);
    s = add_row_shr<4>(s);
    s = add_row_shr<8>(s);
    const float off = s - tot - rho[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) gt.b[i][e] = x[i][e] + off;
    const float bC = row_last(s);
    gt.gm[e] = exp2_hw(bC);
    gt.bc[e] = bC;
    dev = fmaxf(dev, fmaxf(-rho[e], rho[e] - bC));
  }
  gt.dev = dev;
  if constexpr (NE == 1) {
#pragma unroll
    for (int e = 1; e < 8; ++e) {
#pragma unroll
      for (int i = 0; i < 4; ++i) gt.b[i][e] = gt.b[i][0];
      gt.gm[e] = gt.gm[0];
      gt.bc[e] = gt.bc[0];
    }
  }
}

// Commits the reference of the chunk scanned into gt (once per chunk, off the
// scan's critical path): (rarely) a channel whose referenced range leaves
// +-kRefBits moves its reference to rint(b_C / 2), the middle of the chunk's
// range, shifting rho and the sums in place; then the worker's flag bits for
// the chunk (parity par: bit 0 its channels fit fp16, bit 1 a reference
// moved) and its references (buffer buf) go to LDS.  Wave-uniform branches.
__device__ __forceinline__ void ref_commit(const Ptr& p, Gates& gt, float (&rho)[8], int w, int lane, int par,
                                           int buf) {
  int flags = 1;
  if (__builtin_amdgcn_ballot_w64(gt.dev > kRefBits) != 0) {
    bool moved = false, over = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dv = fmaxf(-rho[e], rho[e] - gt.bc[e]);
      const float d = dv > kRefBits ? __builtin_rintf(0.5f * gt.bc[e]) - rho[e] : 0.f;
      rho[e] += d;
#pragma unroll
      for (int i = 0; i < 4; ++i) gt.b[i][e] -= d;
      moved |= d != 0.f;
      over |= fmaxf(-rho[e], rho[e] - gt.bc[e]) > kRefBits;
    }
    flags = (__builtin_amdgcn_ballot_w64(over) == 0 ? 1 : 0) | (__builtin_amdgcn_ballot_w64(moved) != 0 ? 2 : 0);
  }
  if (lane == 0) p.flg[par * 4 + w] = flags;
  if ((lane & 15) == 0) {
    const int c0 = 32 * w + 8 * (lane >> 4);
    *reinterpret_cast<floatx4*>(p.rho + buf * DK + c0) = floatx4{rho[0], rho[1], rho[2], rho[3]};
    *reinterpret_cast<floatx4*>(p.rho + buf * DK + c0 + 4) = floatx4{rho[4], rho[5], rho[6], rho[7]};
  }
}

// A chunk that keeps bf16 operands drops its reference (rho = 0: the plain
// gated operands, as every bf16 product and the fp16 Kg^T, Kb^T of such a
// chunk need): the sums go back to b, and if a reference of this worker was
// nonzero its flag word for the chunk (parity par) gets the "moved" bit, so
// that the owners move their state back.  Called once the four workers'
// operand choice for the chunk is known.
__device__ __forceinline__ void worker_unref(const Ptr& p, Gates& gt, float (&rho)[8], int w, int lane, int par) {
  bool nz = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    nz |= rho[e] != 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) gt.b[i][e] += rho[e];
    rho[e] = 0.f;
  }
  if (__builtin_amdgcn_ballot_w64(nz) != 0 && lane == 0) p.flg[par * 4 + w] |= 2;
}

// The lane's channel references to LDS (buffer buf) for the owners.
__device__ __forceinline__ void worker_rho(const Ptr& p, const float (&rho)[8], int w, int lane, int buf) {
  if ((lane & 15) == 0) {
    const int c0 = 32 * w + 8 * (lane >> 4);
    *reinterpret_cast<floatx4*>(p.rho + buf * DK + c0) = floatx4{rho[0], rho[1], rho[2], rho[3]};
    *reinterpret_cast<floatx4*>(p.rho + buf * DK + c0 + 4) = floatx4{rho[4], rho[5], rho[6], rho[7]};
  }
}

// Phase 1 of a worker: from the referenced prefix sums b' = b - rho,
// Kt = 2^b' k, Kh = 2^-b' k, Qt = 2^b' q (row-major; fp16 or bf16 as the
// chunk's operand choice f16m says), the chunk decay gam = 2^b_C of its
// channels and the q.k partial sums; Kt^T and Kb' = gam Kh = 2^rho Kb stay in
// registers as fp16 (kt_t[e], kb[e] = tokens 4m..4m+3 of channel e) and are
// stored transposed in phase 2a.  (Against the owners' referenced state
// S' = Diag(2^rho) S these referenced operands give the same products as the
// plain ones: W' S' = W S with W' = A' Kt, and Kb'^T Delta = Diag(2^rho)
// Kb^T Delta.)
//
// Phase 1 is the workers' critical phase: the next-but-one chunk's k and q
// are loaded elsewhere (k at the end of phase 2a, q in phase 2b), into the
// registers this phase has consumed.  Issued here, row by row, the same loads
// made the kernel 7 % slower.
//
// Without the delta rule Kt (row-major and transposed) has no reader and is
// not formed.
template <int V>
__device__ __forceinline__ void worker_apply(const Ptr& p, const WRegs& r, const Gates& gt, int w, int lane, int par,
                                             bool f16m, f16x4 (&kb)[8], f16x4 (&kt_t)[8]) {
  constexpr bool ND = (V & kVarNoDelta) != 0;
  const int j = lane >> 4, m = lane & 15;
  const int c0 = 32 * w + 8 * j;
  if (m == 0) {
    *reinterpret_cast<floatx4*>(p.gam + par * DK + c0) = floatx4{gt.gm[0], gt.gm[1], gt.gm[2], gt.gm[3]};
    *reinterpret_cast<floatx4*>(p.gam + par * DK + c0 + 4) = floatx4{gt.gm[4], gt.gm[5], gt.gm[6], gt.gm[7]};
  }
  // rows 4m + i: rmo(4m + i, e) = 4m LDK + i LDK + (e ^ ((m & 7) << 3)) for i < 4
  const int wb0 = 4 * m * LDK + (slot32(c0) ^ ((m & 7) << 3));
  const int wb1 = 4 * m * LDK + (slot32(c0 + 4) ^ ((m & 7) << 3));
  float qk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float kf[8], qf[8];
    unpack8(r.k[i], kf);
    unpack8(r.q[i], qf);
    // q_t . k_t over the lane's 8 channels, straight from the bf16 pairs
    float d = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, r.q[i].w[u]), __builtin_bit_cast(bf16x2, r.k[i].w[u]),
                                          d, false);
    qk[i] = d;
    float kt[8], kh[8], qt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // (a scalar gate: the same factors for every channel)
      const int es = (V & kVarScalarGate) ? 0 : e;
      const float ep = exp2_hw(gt.b[i][es]);
      const float em = exp2_hw(-gt.b[i][es]);
      kt[e] = kf[e] * ep;
      kh[e] = kf[e] * em;
      qt[e] = qf[e] * ep;
      if constexpr (!ND) kt_t[e][i] = (f16)kt[e];
      kb[e][i] = (f16)(kh[e] * gt.gm[es]);
    }
    // channels c0..c0+3 and c0+4..c0+7 sit apart in the slab order
    const int r0 = wb0 + i * LDK, r1 = wb1 + i * LDK;
    if (f16m) {
      f16* Kt = reinterpret_cast<f16*>(p.Kt);
      f16* Kh = reinterpret_cast<f16*>(p.Kh);
      f16* Qt = reinterpret_cast<f16*>(p.Qt);
      if constexpr (!ND) {
        *reinterpret_cast<f16x4*>(Kt + r0) = f16x4{(f16)kt[0], (f16)kt[1], (f16)kt[2], (f16)kt[3]};
        *reinterpret_cast<f16x4*>(Kt + r1) = f16x4{(f16)kt[4], (f16)kt[5], (f16)kt[6], (f16)kt[7]};
      }
      *reinterpret_cast<f16x4*>(Kh + r0) = f16x4{(f16)kh[0], (f16)kh[1], (f16)kh[2], (f16)kh[3]};
      *reinterpret_cast<f16x4*>(Kh + r1) = f16x4{(f16)kh[4], (f16)kh[5], (f16)kh[6], (f16)kh[7]};
      *reinterpret_cast<f16x4*>(Qt + r0) = f16x4{(f16)qt[0], (f16)qt[1], (f16)qt[2], (f16)qt[3]};
      *reinterpret_cast<f16x4*>(Qt + r1) = f16x4{(f16)qt[4], (f16)qt[5], (f16)qt[6], (f16)qt[7]};
    } else {
      if constexpr (!ND) {
        *reinterpret_cast<bf16x4*>(p.Kt + r0) = bf16x4{(bf16)kt[0], (bf16)kt[1], (bf16)kt[2], (bf16)kt[3]};
        *reinterpret_cast<bf16x4*>(p.Kt + r1) = bf16x4{(bf16)kt[4], (bf16)kt[5], (bf16)kt[6], (bf16)kt[7]};
      }
      *reinterpret_cast<bf16x4*>(p.Kh + r0) = bf16x4{(bf16)kh[0], (bf16)kh[1], (bf16)kh[2], (bf16)kh[3]};
      *reinterpret_cast<bf16x4*>(p.Kh + r1) = bf16x4{(bf16)kh[4], (bf16)kh[5], (bf16)kh[6], (bf16)kh[7]};
      *reinterpret_cast<bf16x4*>(p.Qt + r0) = bf16x4{(bf16)qt[0], (bf16)qt[1], (bf16)qt[2], (bf16)qt[3]};
      *reinterpret_cast<bf16x4*>(p.Qt + r1) = bf16x4{(bf16)qt[4], (bf16)qt[5], (bf16)qt[6], (bf16)qt[7]};
    }
  }
  // the diagonal of P is q_t . k_t (the gates cancel): summed in fp32 from
  // the inputs instead of from the separately rounded gated operands; each
  // lane group leaves its 8-channel partial sums, which the P tiles add up
  *reinterpret_cast<floatx4*>(p.qk + (4 * w + j) * C + 4 * m) = floatx4{qk[0], qk[1], qk[2], qk[3]};
}

// Phase 2a of a worker: Kt^T and Kb^T from registers (4 tokens per store).
// (Kt^T only with the delta rule.)
template <int V>
__device__ __forceinline__ void worker_kbt(const Ptr& p, const f16x4 (&kb)[8], const f16x4 (&kt_t)[8], int w,
                                           int lane) {
  const int j = lane >> 4, m = lane & 15;
  const int c0 = 32 * w + 8 * j;
  if constexpr ((V & kVarNoDelta) == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<f16x4*>(p.KtT + (c0 + e) * LDT + 4 * m) = kt_t[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<f16x4*>(p.KbT + (c0 + e) * LDT + slot32(4 * m)) = kb[e];
}

// Phase 1 of owner o (for the next chunk): V^T rows 32o .. 32o + 31 (its own
// value columns) from registers, 4 tokens per 8-byte store.
__device__ __forceinline__ void owner_vt(const Ptr& p, const Vec16 (&v)[4], int o, int lane) {
  const int j = lane >> 4, m = lane & 15;
  const int c0 = 32 * o + 8 * j;
  f16x4 vt[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vf[8];
    unpack8(v[i], vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[e][i] = (f16)vf[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<f16x4*>(p.VT + (c0 + e) * LDT + 4 * m) = vt[e];
}

// Products whose two operands both come from LDS use 16-byte fragments: lane
// group g supplies indices 8g..8g+7 of each 32-index slab (one ds_read_b128
// per fragment).  Every fragment of a group of tiles is read before the first
// product, so the reads overlap each other instead of each waiting in turn.
//
// Transposed tiles: A and B fragments have the same lane layout (lane (g, i)
// holds the slab indices of row / column i), so passing them to the MFMA in
// swapped order yields the transposed product (A B)^T in C layout, where a
// lane holds four consecutive columns of one row.  Tiles that are stored to a
// row-major array are computed this way and written 8 bytes per lane: 2-byte
// LDS writes cost several times more than wide ones.
__device__ __forceinline__ MB::F32 ldc_b(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ MH::F32 ldc_h(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }

// A 16-byte operand fragment of the row-major gated arrays (Kt, Kh, Qt),
// which hold fp16 or bf16 values as the chunk's operand choice says.
template <typename TT>
__device__ __forceinline__ typename Mma<TT>::F32 ldc_g(const bf16* p) {
  return *reinterpret_cast<const typename Mma<TT>::F32*>(p);
}

// NTL 16x16 tiles X_t = A[rows 16 I_t ..] Kh[rows 16 J_t ..]^T of row-major
// [C][DK] arrays of TT (C layout).
// (A_t = Qt where useQ[t], else Kt)
template <typename TT, int NTL, bool SWAP>
__device__ __forceinline__ void kh_tiles(const Ptr& p, const bool (&useQ)[NTL], const int (&I)[NTL],
                                         const int (&J)[NTL], floatx4 (&acc)[NTL], int lane) {
  typedef Mma<TT> MT;
  const bf16* Kh = p.Kh;
  const int fl = frag_lane(lane);
  typename MT::F32 af[NTL][DK / 32], bf[NTL][DK / 32];
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      af[t][ks] = ldc_g<TT>((useQ[t] ? p.Qt : p.Kt) + fl + frag_off(I[t], ks));
      bf[t][ks] = ldc_g<TT>(Kh + fl + frag_off(J[t], ks));
    }
  KDA_READS_FIRST();
#pragma unroll
  for (int t = 0; t < NTL; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
    for (int t = 0; t < NTL; ++t)
      acc[t] = SWAP ? MT::mma32(bf[t][ks], af[t][ks], acc[t]) : MT::mma32(af[t][ks], bf[t][ks], acc[t]);
}

__device__ __forceinline__ int ln_block(int I, int J) { return I * (I - 1) / 2 + J; }

// One tile (I, J) of P = Tril(Qt Kh^T) (isP) or of L = Diag(beta) Kt Kh^T,
// stored as -L, both fp16, from its transposed accumulator (lane: row l16,
// columns 4g..4g+3).
__device__ __forceinline__ void lp_store(const Ptr& p, bool isP, int I, int J, floatx4 acc, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  f16x4 v;
  if (isP) {
    float dg = 0.f;
    if (I == J) {
      const int row = 16 * I + l16;
      float sp[NQK];
#pragma unroll
      for (int u = 0; u < NQK; ++u) sp[u] = p.qk[u * C + row];
#pragma unroll
      for (int st = 1; st < NQK; st *= 2)
#pragma unroll
        for (int u = 0; u + st < NQK; u += 2 * st) sp[u] += sp[u + st];
      dg = sp[0];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float x = (I > J || l16 >= 4 * g4 + jj) ? acc[jj] : 0.f;
      if (I == J && l16 == 4 * g4 + jj) x = dg;
      v[jj] = (f16)x;
    }
    *reinterpret_cast<f16x4*>(p.P + (16 * I + l16) * LDT + slot32(16 * J + 4 * g4)) = v;
  } else {
    const float bt = -p.beta[16 * I + l16];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) v[jj] = (f16)(acc[jj] * bt);
    *reinterpret_cast<f16x4*>(p.Ln + ln_block(I, J) * 16 * LDB + l16 * LDB + 4 * g4) = v;
  }
}

// Workers in phase 2a: blocks (I_t, J_t) of P = Tril(Qt Kh^T) (isP[t]) and
// off-diagonal blocks of L = Diag(beta) Kt Kh^T, stored as -L, all fp16.
template <typename TT, int NTL>
__device__ __forceinline__ void lp_block_tiles(const Ptr& p, const bool (&isP)[NTL], const int (&I)[NTL],
                                            const int (&J)[NTL], int lane) {
  floatx4 acc[NTL];
  kh_tiles<TT, NTL, true>(p, isP, I, J, acc, lane);     // lane: row l16, columns 4g..4g+3
#pragma unroll
  for (int t = 0; t < NTL; ++t) lp_store(p, isP[t], I[t], J[t], acc[t], lane);
}

// The tiles of P (isP) or L in row blocks I0, I0 + 1 and column blocks J0,
// J0 + 1 that are needed (all four below the diagonal; with I0 == J0 the
// three of the lower triangle), from one read of those two row blocks of Qt
// (or Kt) and of Kh: 16 fragments for three or four tiles instead of eight
// per tile.
template <typename TT, bool DIAG>
__device__ __forceinline__ void lp_block22(const Ptr& p, bool isP, int I0, int J0, int lane) {
  typedef Mma<TT> MT;
  const int fl = frag_lane(lane);
  const bf16* A = isP ? p.Qt : p.Kt;
  typename MT::F32 af[2][DK / 32], bf[2][DK / 32];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      af[x][ks] = ldc_g<TT>(A + fl + frag_off(I0 + x, ks));
      bf[x][ks] = ldc_g<TT>(p.Kh + fl + frag_off(J0 + x, ks));
    }
  KDA_READS_FIRST();
  floatx4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        if (!DIAG || y <= x) acc[x][y] = MT::mma32(bf[y][ks], af[x][ks], acc[x][y]);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
      if (!DIAG || y <= x) lp_store(p, isP, I0 + x, J0 + y, acc[x][y], lane);
}

// fp32 16 x 16 x 16 products on the fp16 matrix cores: each operand split as
// hi + lo with hi = fp16(x), lo = fp16(x - hi), and the product formed from
// the three terms above 2^-22 relative (lo lo dropped).  Three fp16 MFMAs cost
// about a fifth of the four fp32 ones they replace; operands must lie inside
// the fp16 range.
struct Split16 { f16x4 hi, lo; };
__device__ __forceinline__ Split16 split16(const floatx4& x) {
  Split16 r;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    r.hi[jj] = (f16)x[jj];
    r.lo[jj] = (f16)(x[jj] - (float)r.hi[jj]);
  }
  return r;
}
__device__ __forceinline__ floatx4 mma16_split(const Split16& a, const Split16& b, floatx4 c) {
  c = MH::mma16(a.lo, b.hi, c);
  c = MH::mma16(a.hi, b.lo, c);
  return MH::mma16(a.hi, b.hi, c);
}

// Owner I in phase 2a: diagonal block I of L and D_I = (I + L_II)^-1 in fp32.
// With N = -L_II (strictly lower, N^16 = 0), D_I = (I + N)(I + N^2)(I + N^4)
// (I + N^8): three squarings and three products (split fp16 products, fp32
// accumulation) instead of a 15-step substitution.  For unit keys |N| <= 1
// and every factor lies far inside the fp16 range, where D_I is stored.  Every factor is kept in accumulator layout together
// with its transpose: the accumulator tile of X^T is exactly the A-operand
// fragment of X (lane (g, i): X[i][4g..4g+3]), and the tile of X is the
// B-operand fragment, so X Y needs tiles of X^T and Y, and (X Y)^T = Y^T X^T
// tiles of Y and X^T.  D_I and D_I^T come out in accumulator layout: D_I^T's
// tile is D_I by rows.  Writes D_I, D_I^T and block (I, I) of A' = D_I Diag(beta),
// 8 bytes per lane.
template <typename TT>
__device__ __forceinline__ void solver_block(const Ptr& p, int I, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  typedef Mma<TT> MT;
  floatx4 n, nt;   // N and N^T tiles
  {
    const int fl = frag_lane(lane);
    typename MT::F32 af[DK / 32], bf[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      af[ks] = ldc_g<TT>(p.Kt + fl + frag_off(I, ks));
      bf[ks] = ldc_g<TT>(p.Kh + fl + frag_off(I, ks));
    }
    KDA_READS_FIRST();
    floatx4 x = {0.f, 0.f, 0.f, 0.f}, xt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      x = MT::mma32(af[ks], bf[ks], x);     // lane: (Kt Kh^T)[4g + jj][l16]
      xt = MT::mma32(bf[ks], af[ks], xt);   // lane: (Kt Kh^T)[l16][4g + jj]
    }
    const floatx4 bt = *reinterpret_cast<const floatx4*>(p.beta + 16 * I + 4 * g4);
    const float bl = p.beta[16 * I + l16];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      n[jj] = (4 * g4 + jj > l16) ? -x[jj] * bt[jj] : 0.f;
      nt[jj] = (l16 > 4 * g4 + jj) ? -xt[jj] * bl : 0.f;
    }
  }
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  floatx4 eye;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) eye[jj] = (4 * g4 + jj == l16) ? 1.f : 0.f;
  // powers
  const Split16 sn = split16(n), snt = split16(nt);
  const Split16 sn2 = split16(mma16_split(snt, sn, z)), sn2t = split16(mma16_split(sn, snt, z));
  const Split16 sn4 = split16(mma16_split(sn2t, sn2, z)), sn4t = split16(mma16_split(sn2, sn2t, z));
  const Split16 sn8 = split16(mma16_split(sn4t, sn4, z));
  // D = D1 (I + N^2)(I + N^4)(I + N^8), D1 = I + N; D_k+1 = D_k + D_k M, D_k+1^T = D_k^T + M^T D_k^T
  floatx4 d = eye + n, dt = eye + nt;
  {
    const Split16 sdt = split16(dt);
    const floatx4 e = mma16_split(sdt, sn2, d), et = mma16_split(sn2, sdt, dt);
    d = e;
    dt = et;
  }
  {
    const Split16 sdt = split16(dt);
    const floatx4 e = mma16_split(sdt, sn4, d), et = mma16_split(sn4, sdt, dt);
    d = e;
    dt = et;
  }
  {
    const Split16 sdt = split16(dt);
    const floatx4 e = mma16_split(sdt, sn8, d), et = mma16_split(sn8, sdt, dt);
    d = e;
    dt = et;
  }
  // d: lane (g, c) = D[4g + jj][c] -> D^T row c; dt: lane (g, c) = D[c][4g + jj] -> D row c
  const int c = l16;
  const floatx4 bt = *reinterpret_cast<const floatx4*>(p.beta + 16 * I + 4 * g4);
  f16x4 dcol, drow, arow;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    dcol[jj] = (f16)d[jj];
    drow[jj] = (f16)dt[jj];
    arow[jj] = (f16)(dt[jj] * bt[jj]);
  }
  *reinterpret_cast<f16x4*>(p.Dt + (I * 16 + c) * LDB + 4 * g4) = dcol;
  *reinterpret_cast<f16x4*>(p.D + (I * 16 + c) * LDB + 4 * g4) = drow;
  // row 16I + c of A', columns 16I + 4g .. 16I + 4g + 3
  *reinterpret_cast<f16x4*>(p.A + (16 * I + c) * LDT + 16 * I + 4 * g4) = arow;
}

// Phase 2b, one worker per block column J = 0, 1, 2: the off-diagonal blocks
// of A = (I + L)^-1 below D_J,
//   A_IJ = D_I Y_IJ,  Y_IJ = (-L_IJ) D_J + sum_{J < K < I} (-L_IK) A_KJ,
// top to bottom with the blocks of the column kept in registers (accumulator
// tiles serve directly as B operands); A'_IJ = A_IJ Diag(beta_J).
template <int J>
__device__ __forceinline__ void solver_offdiag_col(const Ptr& p, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  auto Lf = [&](int I, int K) { return MH::lds16(p.Ln + ln_block(I, K) * 16 * LDB + l16 * LDB + 4 * g4); };
  auto Df = [&](int I) { return MH::lds16(p.D + (I * 16 + l16) * LDB + 4 * g4); };
  MH::F16 lf[4][4], df[4];
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    df[I] = Df(I);
#pragma unroll
    for (int K = J; K < I; ++K) lf[I][K] = Lf(I, K);
  }
  const MH::F16 dtj = MH::lds16(p.Dt + (J * 16 + l16) * LDB + 4 * g4);
  const floatx4 bj = *reinterpret_cast<const floatx4*>(p.beta + 16 * J + 4 * g4);
  KDA_READS_FIRST();
  MH::F16 af[4];
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    floatx4 y = MH::mma16(lf[I][J], dtj, z);
#pragma unroll
    for (int K = J + 1; K < I; ++K) y = MH::mma16(lf[I][K], af[K], y);
    const MH::F16 yf = MH::frag16(y);
    if (I < 3) af[I] = MH::frag16(MH::mma16(df[I], yf, z));
    // A'_IJ from the transposed product: lane holds row l16, columns 4g..4g+3
    const floatx4 at = MH::mma16(yf, df[I], z);
    f16x4 v;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) v[jj] = (f16)(at[jj] * bj[jj]);
    *reinterpret_cast<f16x4*>(p.A + (16 * I + l16) * LDT + 16 * J + 4 * g4) = v;
  }
}

// Phase 3, workers: W^T tile rows 32w.. of W = A' Kt (fp16 products from Kt^T
// and A'), stored as -W into the row-major bf16 array.  A' is lower
// triangular, so token blocks 0 and 1 need only the first 32-token slab.
// (Kt^T holds the referenced k 2^(b - rho): this is W' = W Diag(2^-rho), the
// matrix the owners' referenced state needs.)
__device__ __forceinline__ void worker_w(const Ptr& p, int w, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const int fl = frag_lane(lane);
  MH::F32 ka[2][2], ab[4][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) ka[ct][sl] = ldc_h(p.KtT + (32 * w + 16 * ct + l16) * LDT + 32 * sl + 8 * g4);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int sl = 0; sl < (tb >= 2 ? 2 : 1); ++sl) ab[tb][sl] = ldc_h(p.A + (16 * tb + l16) * LDT + 32 * sl + 8 * g4);
  KDA_READS_FIRST();
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      floatx4 acc = MH::mma32(ka[ct][0], ab[tb][0], floatx4{0.f, 0.f, 0.f, 0.f});
      if (tb >= 2) acc = MH::mma32(ka[ct][1], ab[tb][1], acc);
      bf16x4 o;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[jj] = (bf16)(-acc[jj]);
      // = rmo(16 tb + l16, slot32(32 w + 16 ct + 4 g4))
      *reinterpret_cast<bf16x4*>(p.Wn + fl + 16 * tb * LDK + 32 * (w ^ (tb & 1)) + 4 * ct) = o;
    }
}

// Phase 3, owners: U = A' V for columns col0 .. col0 + 31 (C layout).
template <int NTL>
__device__ __forceinline__ void owner_u(const Ptr& p, int col0, floatx4 (&U)[NTL][4], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  MH::F32 vb[NTL][2], aa[4][2];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) vb[nt][sl] = ldc_h(p.VT + (col0 + vcol(nt, l16)) * LDT + 32 * sl + 8 * g4);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int sl = 0; sl < (tb >= 2 ? 2 : 1); ++sl) aa[tb][sl] = ldc_h(p.A + (16 * tb + l16) * LDT + 32 * sl + 8 * g4);
  KDA_READS_FIRST();
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
      U[nt][tb] = MH::mma32(aa[tb][0], vb[nt][0], floatx4{0.f, 0.f, 0.f, 0.f});
      if (tb >= 2) U[nt][tb] = MH::mma32(aa[tb][1], vb[nt][1], U[nt][tb]);
    }
}

// Phase 3, owners, without the delta rule: U = V for columns col0 ..
// col0 + 31 in the layout of owner_u (the values are the pseudo-values when
// nothing is erased), read from V^T.
__device__ __forceinline__ void owner_v_rows(const Ptr& p, int col0, floatx4 (&U)[2][4], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const f16x4 x = *reinterpret_cast<const f16x4*>(p.VT + (col0 + vcol(nt, l16)) * LDT + 16 * tb + 4 * g4);
      U[nt][tb] = floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
}

// Dx[nt][I] += A[rows 16I..] @ S[nt] (A row-major bf16 in LDS, S in registers),
// every A fragment read before the products.  With SWAP the tiles are held
// transposed (lane: token l16, state columns 4g..4g+3).
template <bool SWAP, int NTL>
__device__ __forceinline__ void rows_times_state_b(const bf16* A, const floatx4 (&S)[NTL][DK / 16],
                                                   floatx4 (&Dx)[NTL][4], int lane) {
  const int fl = frag_lane(lane);
  // two halves of the reduction, each half's fragments read ahead of its
  // products (the second half's reads overlap the first half's MFMAs)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    MB::F32 af[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int I = 0; I < 4; ++I) af[k2][I] = ldc_b(A + fl + frag_off(I, 2 * hf + k2));
    KDA_READS_FIRST();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ks = 2 * hf + k2;
      MB::F32 sf[NTL];
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) sf[nt] = MB::frag32(S[nt][2 * ks], S[nt][2 * ks + 1]);
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
          Dx[nt][I] = SWAP ? MB::mma32(sf[nt], af[k2][I], Dx[nt][I]) : MB::mma32(af[k2][I], sf[nt], Dx[nt][I]);
    }
  }
}

// Phase 2b, owners, for a chunk with fp16 operands: Dx[nt][I] += Qt'[rows
// 16I..] @ S', the tiles held transposed as rows_times_state_b<true> holds
// them, with Qt' (fp16, LDS) and the owner's referenced state S' as fp16
// fragments; with SCALE, S' enters as S' 2^-kx (the caller puts 2^kx back on
// Dx), for a state beyond the fp16 range.
template <bool SCALE>
__device__ __forceinline__ void qt_times_state_h(const bf16* Qt, int kx, const floatx4 (&S)[2][DK / 16],
                                                 floatx4 (&Dx)[2][4], int lane) {
  const int fl = frag_lane(lane);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    MH::F32 af[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int I = 0; I < 4; ++I) af[k2][I] = ldc_g<f16>(Qt + fl + frag_off(I, 2 * hf + k2));
    KDA_READS_FIRST();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ks = 2 * hf + k2;
      MH::F32 sf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if constexpr (SCALE) {
          floatx4 lo, hi;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            lo[jj] = __builtin_amdgcn_ldexpf(S[nt][2 * ks][jj], -kx);
            hi[jj] = __builtin_amdgcn_ldexpf(S[nt][2 * ks + 1][jj], -kx);
          }
          sf[nt] = MH::frag32(lo, hi);
        } else {
          sf[nt] = MH::frag32(S[nt][2 * ks], S[nt][2 * ks + 1]);
        }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) Dx[nt][I] = MH::mma32(sf[nt], af[k2][I], Dx[nt][I]);
    }
  }
}

// Whether every lane's 32 values of Dx are finite (wave-uniform).  A sum is
// enough: an Inf or NaN among them makes it non-finite, and the rare finite
// values whose sum overflows only send the caller down its exact path.
__device__ __forceinline__ bool tiles_finite(const floatx4 (&Dx)[2][4]) {
  float s = 0.f;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int I = 0; I < 4; ++I) s += (Dx[nt][I][0] + Dx[nt][I][1]) + (Dx[nt][I][2] + Dx[nt][I][3]);
  return __builtin_amdgcn_ballot_w64(!__builtin_isfinite(s)) == 0;
}

// Scale exponent kx >= 0 that keeps an owner's referenced state below 2^15
// in magnitude.  Wave-uniform.
__device__ __forceinline__ int state_f16_shift(const floatx4 (&S)[2][DK / 16]) {
  // a tree of three-input maxima over the lane's 64 values
  float m[16];
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      m[2 * rt + h] = fmaxf(fmaxf(fabsf(S[0][rt][2 * h]), fabsf(S[0][rt][2 * h + 1])),
                            fmaxf(fabsf(S[1][rt][2 * h]), fabsf(S[1][rt][2 * h + 1])));
#pragma unroll
  for (int st = 8; st > 0; st >>= 1)
#pragma unroll
    for (int i = 0; i < st; ++i) m[i] = fmaxf(m[i], m[i + st]);
  // |S'| < 2^ex; S' 2^-kx < 2^15
  const int ex = __builtin_amdgcn_frexp_expf(wave_max_nonneg(m[0]));
  return max(0, ex - 15);
}

// Rows of an owner's state tiles times 2^e_row, e_row = rho_a[row] -
// rho_b[row] (moving the state's reference; sign -1 with rho_b NULL divides
// by 2^rho_a, i.e. back to the plain state).
__device__ __forceinline__ void state_rescale(floatx4 (&S)[2][DK / 16], const float* rho_a, const float* rho_b,
                                              int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt) {
    floatx4 e = *reinterpret_cast<const floatx4*>(rho_a + 16 * rt + 4 * g4);
    if (rho_b) e -= *reinterpret_cast<const floatx4*>(rho_b + 16 * rt + 4 * g4);
    else e = -e;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) S[nt][rt][jj] = __builtin_amdgcn_ldexpf(S[nt][rt][jj], (int)e[jj]);
  }
}

// Phase 1, owners: O += P Delta, S <- Diag(gam) S + Kb^T Delta.
template <int NTL>
__device__ __forceinline__ void owner_intra(const Ptr& p, const MH::F32 (&Df)[NTL][2], floatx4 (&O)[NTL][4], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  MH::F32 pa[4][2];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int sl = 0; sl < (I >= 2 ? 2 : 1); ++sl) pa[I][sl] = ldc_h(p.P + (16 * I + l16) * LDT + 32 * sl + 8 * g4);
  KDA_READS_FIRST();
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
      O[nt][I] = MH::mma32(Df[nt][0], pa[I][0], O[nt][I]);
      if (I >= 2) O[nt][I] = MH::mma32(Df[nt][1], pa[I][1], O[nt][I]);
    }
}

template <int NTL>
__device__ __forceinline__ void owner_state(const Ptr& p, const MH::F32 (&Df)[NTL][2], floatx4 (&S)[NTL][DK / 16],
                                            int par, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    MH::F32 ka[DK / 32][2];
#pragma unroll
    for (int r2 = 0; r2 < DK / 32; ++r2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ka[r2][h] = ldc_h(p.KbT + (16 * (hf * DK / 32 + r2) + l16) * LDT + 32 * h + 8 * g4);
    KDA_READS_FIRST();
#pragma unroll
    for (int r2 = 0; r2 < DK / 32; ++r2) {
      const int rt = hf * DK / 32 + r2;
      const floatx4 gm = *reinterpret_cast<const floatx4*>(p.gam + par * DK + 16 * rt + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        S[nt][rt] *= gm;
        S[nt][rt] = MH::mma32(ka[r2][0], Df[nt][0], S[nt][rt]);
        S[nt][rt] = MH::mma32(ka[r2][1], Df[nt][1], S[nt][rt]);
      }
    }
  }
}

// The two products above for two states of the same chunk (the offset and
// the transition of a segment, run together): each operand fragment read
// from LDS once for both, one 32-index slab at a time (two states leave
// fewer registers for reads ahead).
__device__ __forceinline__ void rows_times_state2_b(const bf16* A, const floatx4 (&S)[2][DK / 16],
                                                    const floatx4 (&S2)[2][DK / 16], floatx4 (&Dx)[2][4],
                                                    floatx4 (&Dx2)[2][4], int lane) {
  const int fl = frag_lane(lane);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    MB::F32 af[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) af[I] = ldc_b(A + fl + frag_off(I, ks));
    KDA_READS_FIRST();
    MB::F32 sf[2], sf2[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      sf[nt] = MB::frag32(S[nt][2 * ks], S[nt][2 * ks + 1]);
      sf2[nt] = MB::frag32(S2[nt][2 * ks], S2[nt][2 * ks + 1]);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        Dx[nt][I] = MB::mma32(af[I], sf[nt], Dx[nt][I]);
        Dx2[nt][I] = MB::mma32(af[I], sf2[nt], Dx2[nt][I]);
      }
  }
}

__device__ __forceinline__ void owner_state2(const Ptr& p, const MH::F32 (&Df)[2][2], const MH::F32 (&Df2)[2][2],
                                             floatx4 (&S)[2][DK / 16], floatx4 (&S2)[2][DK / 16], int par,
                                             int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    MH::F32 ka[DK / 32][2];
#pragma unroll
    for (int r2 = 0; r2 < DK / 32; ++r2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ka[r2][h] = ldc_h(p.KbT + (16 * (hf * DK / 32 + r2) + l16) * LDT + 32 * h + 8 * g4);
    KDA_READS_FIRST();
#pragma unroll
    for (int r2 = 0; r2 < DK / 32; ++r2) {
      const int rt = hf * DK / 32 + r2;
      const floatx4 gm = *reinterpret_cast<const floatx4*>(p.gam + par * DK + 16 * rt + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        S[nt][rt] *= gm;
        S[nt][rt] = MH::mma32(ka[r2][0], Df[nt][0], S[nt][rt]);
        S[nt][rt] = MH::mma32(ka[r2][1], Df[nt][1], S[nt][rt]);
        S2[nt][rt] *= gm;
        S2[nt][rt] = MH::mma32(ka[r2][0], Df2[nt][0], S2[nt][rt]);
        S2[nt][rt] = MH::mma32(ka[r2][1], Df2[nt][1], S2[nt][rt]);
      }
    }
  }
}

// Phase 1, owners: the output tile straight to memory.  O is held transposed
// (lane: token 16I + l16, tile columns 4g..4g+3 of both tiles), which in the
// owner's column order are the 8 adjacent value columns col0 + 8g .. + 7.
__device__ __forceinline__ void owner_store(const floatx4 (&O)[2][4], __amdgpu_buffer_rsrc_t ro, int row_elems,
                                            int col0, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    bf16x8 v;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v[jj] = (bf16)O[0][I][jj];
      v[4 + jj] = (bf16)O[1][I][jj];
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                           (uint32_t)(((16 * I + l16) * row_elems + col0 + 8 * g4) * 2), 0, 0);
  }
}

}  // namespace pipe

namespace pipe {
// Phase 2a tile schedules of the workers, per operand type.
// No delta rule: the ten P blocks, three / three / two / two per worker.
template <typename TT>
__device__ __forceinline__ void nd_p_tiles(const Ptr& p, int w, int lane) {
  switch (w) {
    case 0: { const bool q[3] = {1, 1, 1}; const int I[3] = {0, 3, 3}, J[3] = {0, 0, 3};
              lp_block_tiles<TT, 3>(p, q, I, J, lane); break; }
    case 1: { const bool q[3] = {1, 1, 1}; const int I[3] = {1, 1, 3}, J[3] = {0, 1, 1};
              lp_block_tiles<TT, 3>(p, q, I, J, lane); break; }
    case 2: { const bool q[2] = {1, 1}; const int I[2] = {2, 2}, J[2] = {0, 1};
              lp_block_tiles<TT, 2>(p, q, I, J, lane); break; }
    default: { const bool q[2] = {1, 1}; const int I[2] = {2, 3}, J[2] = {2, 2};
               lp_block_tiles<TT, 2>(p, q, I, J, lane); break; }
  }
}
// State only: the six off-diagonal L blocks.
template <typename TT>
__device__ __forceinline__ void state_l_tiles(const Ptr& p, int w, int lane) {
  switch (w) {
    case 0: { const bool q[2] = {0, 0}; const int I[2] = {1, 2}, J[2] = {0, 1};
              lp_block_tiles<TT, 2>(p, q, I, J, lane); break; }
    case 1: { const bool q[2] = {0, 0}; const int I[2] = {2, 3}, J[2] = {0, 2};
              lp_block_tiles<TT, 2>(p, q, I, J, lane); break; }
    case 2: { const bool q[1] = {0}; const int I[1] = {3}, J[1] = {0};
              lp_block_tiles<TT, 1>(p, q, I, J, lane); break; }
    default: { const bool q[1] = {0}; const int I[1] = {3}, J[1] = {1};
               lp_block_tiles<TT, 1>(p, q, I, J, lane); break; }
  }
}
// With outputs: P in three groups sharing operand rows (blocks 2-3 x 0-1;
// the lower triangles of 0-1 x 0-1 and of 2-3 x 2-3), and the L blocks
// (2-3) x (0-1); the owners form L(1,0), L(3,2) and the diagonal blocks.
template <typename TT>
__device__ __forceinline__ void pl_tiles(const Ptr& p, int w, int lane) {
  switch (w) {
    case 0: lp_block22<TT, false>(p, true, 2, 0, lane); break;
    case 1: lp_block22<TT, true>(p, true, 0, 0, lane); break;
    case 2: lp_block22<TT, true>(p, true, 2, 2, lane); break;
    default: lp_block22<TT, false>(p, false, 2, 0, lane); break;
  }
}
}  // namespace pipe

// Device plan of the segmented schedule for packed sequences (written by
// varlen_plan_kernel; N sequences, tables of j1 / j3 entries):
//   count[0], count[1]  jobs of pass 1 and pass 3; count[2] segmented sequences
//   nsegs[N]   segments of each sequence (P < 3: run whole in pass 1)
//   mapbase[N] first map slot of a segmented sequence (slots of H x 3 maps)
//   segseq[N]  the segmented sequences, in order
//   table1[j1], table3[j3]  jobs (sequence, index inside the sequence)
struct VarlenPlan {
  const int* count; const int* nsegs; const int* mapbase; const int* segseq;
  const int2* table1; const int2* table3;
  __device__ VarlenPlan(const int* p, int N, int j1, int j3) {
    count = p;
    nsegs = p + 4;
    mapbase = nsegs + N;
    segseq = mapbase + N;
    table1 = reinterpret_cast<const int2*>(p + varlen_plan_table_offset(N));
    table3 = table1 + j1;
    (void)j3;
  }
};

// V: variant flags (kVarScalarGate, kVarNoDelta).  Without the delta rule
// A' = I and W = 0: the pseudo-values are the values, so the L blocks, the
// solver, W and the W S product drop out and only P, Kh, Qt, Kb remain.
template <int V>
__global__ __launch_bounds__(NT) void fused_pipe_kernel(PrefillArgs a) {
  using namespace pipe;
  constexpr bool ND = (V & kVarNoDelta) != 0;
  constexpr bool ST = (V & kPipeStates) != 0;
  constexpr bool DU = (V & kPipeDual) != 0;
  constexpr bool SI = (V & kPipeSegIn) != 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work of this workgroup: chunks c0 .. c0 + nchunks - 1 of one sequence and
  // head, entry state from s0p (NULL: zeros, or the identity if ident), final
  // state to sTp (NULL: dropped), outputs formed and stored if outp (else only
  // the state runs: no P, no Qg S), values used unless vzero.
  // One pass: the whole sequence.  Segmented (nseg segments of seg_len
  // chunks): pass 1 runs segment 0 (its final state is segment 1's entry
  // state) and, state only, for each segment s = 1 .. nseg-2 in one
  // workgroup the offset N_s (from zero) and the transition M_s (from the
  // identity, values zero) of S_end = M_s S_start + N_s; pass 3 runs segments
  // 1 .. nseg-1 from their entry states, which the combine kernel has formed
  // in between.
  int head, c0 = 0, nchunks = (a.T + C - 1) / C;
  const float* s0p = nullptr;
  float* sTp = nullptr;
  bool sTf = false;   // sTp is a workspace entry state (fragment order)
  bool ident = false, outp = true, vzero = false;
  // a middle segment of the segmented schedule: its offset N_s (state from
  // zero, into sTp) and its transition M_s (state from the identity with the
  // values zeroed, into smp) in one run, state only
  bool dual = false;
  float* smp = nullptr;
  // packed sequences, segmented: this workgroup's segment (-1: the whole
  // sequence) and the sequence's first map slot
  int vsg = -1, vmap0 = 0;
  if (a.pass == 0) {
    int split;
    block_to_head<1>(blockIdx.x, head, split);
    if (head >= a.B * a.H) return;
    if (a.cu_seqlens && a.seq_order) {
      // packed sequences in the given order (longest first balances the
      // tail); entries clamped into range
      const int sq = min(max(a.seq_order[head / a.H], 0), a.B - 1);
      head = sq * a.H + head % a.H;
    }
    if (a.S0) s0p = a.S0 + (int64_t)head * DK * DV;
    if (a.S_T) sTp = a.S_T + (int64_t)head * DK * DV;
    if (ST) outp = a.o != nullptr;   // chunk-entry states, with or without the outputs
  } else if (a.plan) {
    // packed sequences, segmented (the plan kernel's job tables): pass 1 runs
    // whole short sequences and, for the long ones, segment 0, the offsets
    // N_s and the transitions M_s; pass 3 runs segments 1 .. P-1
    const VarlenPlan vp(a.plan, a.B, a.plan_j1, a.plan_j3);
    const int job = blockIdx.x / a.H, hh = blockIdx.x % a.H;
    if (job >= (a.pass == 1 ? vp.count[0] : vp.count[1])) return;
    const int2 jb = (a.pass == 1 ? vp.table1 : vp.table3)[job];
    const int sq = jb.x, k = jb.y, P = vp.nsegs[sq];
    head = sq * a.H + hh;
    vmap0 = vp.mapbase[sq];
    const float* S0h = a.S0 ? a.S0 + (int64_t)head * DK * DV : nullptr;
    float* STh = a.S_T ? a.S_T + (int64_t)head * DK * DV : nullptr;
    auto vmap = [&](int sgi, int kind) {
      return a.ws + (((int64_t)(vmap0 + sgi) * a.H + hh) * 3 + kind) * (int64_t)(DK * DV);
    };
    if (a.pass == 1) {
      if (P < 3) {
        s0p = S0h;
        sTp = STh;
      } else if (k == 0) {
        vsg = 0;
        s0p = S0h;
        sTp = vmap(1, 0);
        sTf = true;
      } else {
        vsg = k;
        outp = false;
        dual = true;
        sTp = vmap(k, 2);
        smp = vmap(k, 1);
      }
    } else {
      vsg = k + 1;
      s0p = vmap(vsg, 0);
      if (vsg == P - 1) sTp = STh;
    }
  } else {
    const int njobs = a.nseg - 1;
    head = blockIdx.x / njobs;
    const int job = blockIdx.x % njobs;
    if (head >= a.B * a.H) return;
    int sg;
    if (a.pass == 1) {
      sg = job;
      if (job == 0) {
        if (a.S0) s0p = a.S0 + (int64_t)head * DK * DV;
        sTp = seg_mat(a.ws, head, a.nseg, 1, 0);
        sTf = true;
      } else {
        outp = false;
        dual = true;
        sTp = seg_mat(a.ws, head, a.nseg, sg, 2);
        smp = seg_mat(a.ws, head, a.nseg, sg, 1);
      }
    } else {
      sg = job + 1;
      s0p = seg_mat(a.ws, head, a.nseg, sg, 0);
      if (sg == a.nseg - 1 && a.S_T) sTp = a.S_T + (int64_t)head * DK * DV;
    }
    c0 = sg * a.seg_len;
    nchunks = min(a.seg_len, nchunks - c0);
  }
  int bb = head / a.H;
  const int h = head % a.H;
  // chunk-entry states: chunk n of this sequence is block st0 + n * stn
  // (packed sequences: slot floor(cu[b] / C) + b + n, head-minor)
  int64_t st0 = (int64_t)head * ((a.T + C - 1) / C), stn = 1;
  if (a.cu_seqlens) {
    // packed sequences: sequence bb is tokens [cu[bb], cu[bb+1]) of the
    // [T, H, d] tensors, clamped to them; from here on it is addressed as a
    // batch of one sequence
    const int e0 = min(max(a.cu_seqlens[bb], 0), a.T);
    const int e1 = min(max(a.cu_seqlens[bb + 1], e0), a.T);
    const int64_t r0 = (int64_t)e0 * a.H;   // first row of the sequence
    st0 = (int64_t)(e0 / C + bb) * a.H + h;
    stn = a.H;
    a.q = reinterpret_cast<const bf16*>(a.q) + r0 * DK;
    a.k = reinterpret_cast<const bf16*>(a.k) + r0 * DK;
    a.g = reinterpret_cast<const bf16*>(a.g) + r0 * ((V & kVarScalarGate) ? 1 : DK);
    a.v = reinterpret_cast<const bf16*>(a.v) + r0 * DV;
    a.o = reinterpret_cast<bf16*>(a.o) + r0 * DV;
    if constexpr ((V & kVarNoDelta) == 0) a.beta = reinterpret_cast<const bf16*>(a.beta) + r0;
    a.T = e1 - e0;
    bb = 0;
    nchunks = (a.T + C - 1) / C;
    if (vsg >= 0) {
      c0 = vsg * a.seg_len;
      nchunks = min(a.seg_len, nchunks - c0);
    }
  }
  Ptr p;
  p.set(smem_raw);
  // blocks (0,1) and (2,3) of P and A' above the diagonal are read by the
  // 32-token reduction slabs and never written otherwise (in P they are spread
  // over rows 0-15 and 32-47 by the slab order: clear those rows whole, the
  // written blocks are rewritten every chunk)
  for (int idx = tid; idx < 2 * 16 * 16; idx += NT) {
    const int blk = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
    const int row = 32 * blk + r, col = 32 * blk + 16 + c;
    p.A[row * LDT + col] = (f16)0.f;
  }
  for (int idx = tid; idx < 2 * 16 * 64; idx += NT) {
    const int blk = idx >> 10, r = (idx >> 6) & 15, c = idx & 63;
    p.P[(32 * blk + r) * LDT + c] = (f16)0.f;
  }
  // the reference before the first chunk (buffer of chunk -1) is 0
  if (tid < DK) p.rho[2 * DK + tid] = 0.f;

  if (!ST && DU && dual && wave < 4) {
    // ---------------------------------------------------- owners, two states
    // N (from zero, with the values) and M (from the identity, values zero):
    // the same chunk operands, so the workers' half of the work is shared;
    // the owners' products read each operand fragment once for both states.
    // The phases and barriers are those of a state-only run.
    const int o = wave;
    const int col0 = 32 * o;
    floatx4 S[2][DK / 16], SM[2][DK / 16];
    load_state_v(S, nullptr, false, col0, lane);
    load_state_v(SM, nullptr, true, col0, lane);
    floatx4 U[2][4];
    Vec16 vr[4];
    if (nchunks > 0) fetch_v(vr, a, bb, h, c0, o, lane);
    __syncthreads();   // the workers' operand choice of the first chunk
    for (int n = -1; n < nchunks; ++n) {
      const bool nxt = n + 1 < nchunks;
      p.sync(smem_raw);
      // phase 1: V^T of chunk n+1 first (its registers are free during the
      // products), then chunk n for both states (Delta_M = -W S_M)
      if (nxt) owner_vt(p, vr, o, lane);
      if (n >= 0) {
        floatx4 UM[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int I = 0; I < 4; ++I) UM[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!ND) rows_times_state2_b(p.Wn, S, SM, U, UM, lane);
        MH::F32 Df[2][2], DfM[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          Df[nt][0] = MH::frag32(U[nt][0], U[nt][1]);
          Df[nt][1] = MH::frag32(U[nt][2], U[nt][3]);
          DfM[nt][0] = MH::frag32(UM[nt][0], UM[nt][1]);
          DfM[nt][1] = MH::frag32(UM[nt][2], UM[nt][3]);
        }
        owner_state2(p, Df, DfM, S, SM, n & 1, lane);
      }
      fetch_v(vr, a, bb, h, c0 + n + 2, o, lane);
      p.sync(smem_raw);
      // phase 2a: diagonal block o of L and its inverse (chunk n+1)
      const bool f16m = (chunk_flags(p, (n + 1) & 1) & 1) != 0;
      if (!ND && nxt) {
        if (f16m)
          solver_block<f16>(p, o, lane);
        else
          solver_block<bf16>(p, o, lane);
      }
      p.sync(smem_raw);
      // phase 2b: both states move to the reference of chunk n+1 where it changed
      const int fl = nxt ? chunk_flags(p, (n + 1) & 1) : 0;
      if (fl & 2) {
        state_rescale(S, p.rho + ((n + 1) % 3) * DK, p.rho + ((n + 3) % 3) * DK, lane);
        state_rescale(SM, p.rho + ((n + 1) % 3) * DK, p.rho + ((n + 3) % 3) * DK, lane);
      }
      p.sync(smem_raw);
      // phase 3: U of chunk n+1
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I) U[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (nxt) {
        if constexpr (ND)
          owner_v_rows(p, col0, U, lane);
        else
          owner_u(p, col0, U, lane);
      }
    }
    // back from the last chunk's reference
    state_rescale(S, p.rho + ((nchunks + 2) % 3) * DK, nullptr, lane);
    store_state_f(S, sTp, col0, lane);
    state_rescale(SM, p.rho + ((nchunks + 2) % 3) * DK, nullptr, lane);
    // (after the loop the workers touch only rho and the flags: the four
    // row-major operand areas are free, one per owner)
    static_assert(DK * kMStageRow * 4 <= SZ_RM && O_KH == O_KT + SZ_RM && O_QT == O_KH + SZ_RM &&
                      O_WN == O_QT + SZ_RM && O_WN + SZ_RM <= O_RHO, "map staging areas");
    store_state_mfrag(SM, smp, col0, lane, reinterpret_cast<float*>(smem_raw + O_KT + o * SZ_RM));
  } else if (wave < 4) {
    // ---------------------------------------------------------------- owners
    const int o = wave;
    const int col0 = 32 * o;
    floatx4 S[2][DK / 16];
    // (the third pass's entry states come from the workspace, always)
    if constexpr (SI)
      load_state_f(S, s0p, col0, lane);
    else
      load_state_v(S, s0p, ident, col0, lane);
    floatx4 O[2][4], U[2][4];
    Vec16 vr[4];
    if (nchunks > 0) fetch_v(vr, a, bb, h, c0, o, lane);
    __syncthreads();   // the workers' operand choice of the first chunk
    // S holds the state referenced to the current chunk, Diag(2^rho) S; the
    // reference before the first chunk is 0
    for (int n = -1; n < nchunks; ++n) {
      const bool nxt = n + 1 < nchunks;
      p.sync(smem_raw);
      // phase 1: finish chunk n
      if (n >= 0) {
        if constexpr (!ND) rows_times_state_b<false>(p.Wn, S, U, lane);
        MH::F32 Df[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          Df[nt][0] = MH::frag32(U[nt][0], U[nt][1]);
          Df[nt][1] = MH::frag32(U[nt][2], U[nt][3]);
        }
        if (outp) {
          owner_intra(p, Df, O, lane);
          const int t0 = (c0 + n) * C, nv = min(C, a.T - t0);
          const int64_t tok0 = ((int64_t)bb * a.T + t0) * a.H + h;
          const __amdgpu_buffer_rsrc_t ro =
              make_rsrc(reinterpret_cast<bf16*>(a.o) + tok0 * DV, chunk_bytes(nv, a.H * DV, DV, 2));
          owner_store(O, ro, a.H * DV, col0, lane);
        }
        if constexpr (ST)
          store_state_t(S, p.rho + ((n + 3) % 3) * DK,
                        reinterpret_cast<bf16*>(a.states) + (st0 + (int64_t)(c0 + n) * stn) * DK * DV, col0, lane);
        owner_state(p, Df, S, n & 1, lane);
      }
      // V^T of chunk n+1 (U is formed in phase 3)
      if (nxt && !vzero) owner_vt(p, vr, o, lane);
      // values of chunk n+2 into the registers just consumed: unconditional
      // (zeros past the end), so that no branch merges them with old values
      fetch_v(vr, a, bb, h, c0 + n + 2, o, lane);
      p.sync(smem_raw);
      // phase 2a: diagonal block o of L and its inverse (chunk n+1)
      const bool f16m = (chunk_flags(p, (n + 1) & 1) & 1) != 0;
      if (!ND && nxt) {
        if (f16m)
          solver_block<f16>(p, o, lane);
        else
          solver_block<bf16>(p, o, lane);
      }
      // with outputs the workers form the P blocks and the L blocks (2-3) x
      // (0-1); owners 0 and 1 form L(1,0) and L(3,2)
      if (!ND && nxt && outp && o < 2) {
        const bool q[1] = {false};
        const int I1[1] = {o == 0 ? 1 : 3}, J1[1] = {o == 0 ? 0 : 2};
        if (f16m)
          lp_block_tiles<f16, 1>(p, q, I1, J1, lane);
        else
          lp_block_tiles<bf16, 1>(p, q, I1, J1, lane);
      }
      p.sync(smem_raw);
      // phase 2b: entry-state readout of chunk n+1
      // O and U are (re)defined on every path, so their previous values are
      // not kept alive through the other phases
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I) O[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int fl = nxt ? chunk_flags(p, (n + 1) & 1) : 0;
      // the state moves to the reference of chunk n+1 where it changed
      if (fl & 2) {
        state_rescale(S, p.rho + ((n + 1) % 3) * DK, p.rho + ((n + 3) % 3) * DK, lane);
      }
      if (nxt && outp) {
        if (fl & 1) {
          // the state as fp16 as it is; an entry beyond the fp16 range turns
          // into Inf there and makes the product non-finite: then (rarely)
          // again with the state scaled into range
          qt_times_state_h<false>(p.Qt, 0, S, O, lane);
          if (!tiles_finite(O)) {
            const int kx = state_f16_shift(S);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
              for (int I = 0; I < 4; ++I) O[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
            qt_times_state_h<true>(p.Qt, kx, S, O, lane);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
              for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) O[nt][I][jj] = __builtin_amdgcn_ldexpf(O[nt][I][jj], kx);
          }
        } else {
          rows_times_state_b<true>(p.Qt, S, O, lane);
        }
      }
      p.sync(smem_raw);
      // phase 3: U of chunk n+1
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I) U[nt][I] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (nxt && !vzero) {
        if constexpr (ND)
          owner_v_rows(p, col0, U, lane);
        else
          owner_u(p, col0, U, lane);
      }
    }
    if (sTp) {
      // back from the last chunk's reference
      state_rescale(S, p.rho + ((nchunks + 2) % 3) * DK, nullptr, lane);
      if (sTf)
        store_state_f(S, sTp, col0, lane);
      else
        store_state_v(S, sTp, col0, lane);
    }
  } else {
    // --------------------------------------------------------------- workers
    const int w = wave - 4;
    WRegs r;
    Gates gt;
    float rho[8];   // reference exponents of the lane's channels
#pragma unroll
    for (int e = 0; e < 8; ++e) rho[e] = 0.f;
    fetch_qkg<V>(r, a, bb, h, c0, w, lane);   // zeros when the sequence is empty
    worker_scan<V>(r, gt, rho, QkgSrc<V>(a, bb, h, c0 + 1, w, lane));
    ref_commit(p, gt, rho, w, lane, 0, 0);
    __syncthreads();
    // operand choice of the chunk being prepared
    bool f16m = (chunk_flags(p, 0) & 1) != 0;
    if (!f16m) {
      worker_unref(p, gt, rho, w, lane, 0);
      worker_rho(p, rho, w, lane, 0);
    }
    for (int n = -1; n < nchunks; ++n) {
      const bool nxt = n + 1 < nchunks;
      f16x4 kb[8], kt_t[8];
      p.sync(smem_raw);
      if (n >= 0) {
        // the operand choice of chunk n+1 (its flags were committed in the
        // previous slot's phase 3); a bf16 chunk drops its reference
        f16m = (chunk_flags(p, (n + 1) & 1) & 1) != 0;
        if (!f16m) {
          worker_unref(p, gt, rho, w, lane, (n + 1) & 1);
          worker_rho(p, rho, w, lane, (n + 1) % 3);
        }
      }
      // phase 1: gated operands of chunk n+1.  Runs on every slot (past the
      // last chunk on zeros, into arrays nobody reads again), so the loads of
      // the other phases are never under a branch: loaded registers merging
      // with old ones at a join would make the merge wait for them.
      {
        const QkgSrc<V> nx(a, bb, h, c0 + n + 2, w, lane);
        if constexpr (!ND) {
          if (w == 0) p.beta[lane] = __uint_as_float(r.beta_bits << 16);
          r.beta_bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(nx.b, nx.boff, 0, 0);
        }
        worker_apply<V>(p, r, gt, w, lane, (n + 1) & 1, f16m, kb, kt_t);
      }
      p.sync(smem_raw);
      // phase 2a: Kt^T, Kb^T; the ten P blocks and two off-diagonal blocks of
      // L, three each (the owners form the other four L blocks; state-only
      // runs: the six L blocks alone; no delta rule: the P blocks alone)
      if (ND && nxt && outp) {
        worker_kbt<V>(p, kb, kt_t, w, lane);
        if (f16m)
          nd_p_tiles<f16>(p, w, lane);
        else
          nd_p_tiles<bf16>(p, w, lane);
      } else if (ND && nxt) {
        worker_kbt<V>(p, kb, kt_t, w, lane);
      } else if (nxt && !outp) {
        worker_kbt<V>(p, kb, kt_t, w, lane);
        if (f16m)
          state_l_tiles<f16>(p, w, lane);
        else
          state_l_tiles<bf16>(p, w, lane);
      } else if (nxt) {
        // P in three groups sharing operand rows (blocks 2-3 x 0-1; the
        // lower triangles of 0-1 x 0-1 and of 2-3 x 2-3), and the L blocks
        // (2-3) x (0-1); the owners form L(1,0), L(3,2) and the diagonal blocks
        worker_kbt<V>(p, kb, kt_t, w, lane);
        if (f16m)
          pl_tiles<f16>(p, w, lane);
        else
          pl_tiles<bf16>(p, w, lane);
      }
      // k of chunk n+2 into the registers phase 1 consumed
      {
        const QkgSrc<V> nk(a, bb, h, c0 + n + 2, w, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.k[i] = ld16(nk.k, nk.vo, i * nk.rs);
      }
      p.sync(smem_raw);
      // phase 2b: workers 1-3: the off-diagonal blocks of A' in block columns
      // 0-2; all: gate prefix sums of chunk n+2 and the gate loads of chunk
      // n+3 (on every slot)
      if (!ND && nxt) {
        if (w == 1)
          solver_offdiag_col<0>(p, lane);
        else if (w == 2)
          solver_offdiag_col<1>(p, lane);
        else if (w == 3)
          solver_offdiag_col<2>(p, lane);
      }
      worker_scan<V>(r, gt, rho, QkgSrc<V>(a, bb, h, c0 + n + 3, w, lane));
      // q of chunk n+2
      {
        const QkgSrc<V> nk(a, bb, h, c0 + n + 2, w, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.q[i] = ld16(nk.q, nk.vo, i * nk.rs);
      }
      p.sync(smem_raw);
      // phase 3: W; the references and operand flags of chunk n+2
      if (!ND && nxt) worker_w(p, w, lane);
      ref_commit(p, gt, rho, w, lane, n & 1, (n + 2) % 3);
    }
  }
}

// ---------------------------------------------------------------------------
// Segmented schedule, between the two passes: the entry state of each
// segment, S_{s+1} = M_s S_s + N_s for s = 1 .. nseg-2 (S_1 is segment 0's
// final state).  The columns of the state never mix, so each sequence and
// head is split into NSC workgroups of 16 columns; wavefront w forms rows
// 32w .. 32w+31 of the slice.  Each fp32 product runs as three bf16 MFMAs
// (v_mfma_f32_16x16x32_bf16) on split operands, x = hi + lo with hi the bf16
// rounding of x and lo that of x - hi: hi hi + hi lo + lo hi, relative error
// about 2^-16 (the dropped lo lo term and the rounding of lo), against 2^-8
// for the bf16 operands of the state update the maps stand for.  M_s comes
// from the workspace already split, in the A-operand order (mfrag_index),
// straight into registers two steps ahead; the slice of S_s alternates
// between two LDS buffers, split and stored column by column, so that each
// B operand of a lane is one 16-byte read.
// ---------------------------------------------------------------------------
namespace segc {
constexpr int NTC = 256;
constexpr int NSC = 8;               // column slices per sequence and head
constexpr int CW = 128 / NSC;        // columns per slice
constexpr int LDS_T = 136;           // bf16 per slice column (its 128 rows, padded)
constexpr int PART = CW * LDS_T;     // bf16 of one part (high or low) of a buffer
constexpr int BYTES = 2 * 2 * PART * 2;
}  // namespace segc

__global__ __launch_bounds__(segc::NTC) void seg_combine_kernel(PrefillArgs a) {
  using namespace segc;
  constexpr int D = 128;
  typedef Mma<bf16> CM;
  typedef CM::F32 Frag;   // bf16x8
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* T0 = reinterpret_cast<bf16*>(smem_raw);   // buffer 0: high part, then low part
  bf16* T1 = T0 + 2 * PART;
  const int col0 = (blockIdx.x % NSC) * CW;
  int nseg = a.nseg;
  // maps of segment s of this sequence and head: batched sequences keep them
  // per head (nseg x 3); packed ones from their plan's first slot (H x 3 per slot)
  int64_t mbase, mslot;
  if (a.plan) {
    const VarlenPlan vp(a.plan, a.B, a.plan_j1, a.plan_j3);
    const int i = blockIdx.x / (NSC * a.H), hh = (blockIdx.x / NSC) % a.H;
    if (i >= vp.count[2]) return;
    const int sq = vp.segseq[i];
    nseg = vp.nsegs[sq];
    mbase = (int64_t)vp.mapbase[sq] * a.H + hh;
    mslot = a.H;
  } else {
    const int head = blockIdx.x / NSC;
    if (head >= a.B * a.H) return;
    mbase = (int64_t)head * a.nseg;
    mslot = 1;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  auto mat = [&](int s, int kind) { return a.ws + ((mbase + s * mslot) * 3 + kind) * (D * D); };
  // the lane's A operands of M_s: tile u (rows 32 wave + 16 u ..), slab kk, part h
  auto load_m = [&](int s, Frag (&m)[2][4][2]) {
    const Frag* src = reinterpret_cast<const Frag*>(mat(s, 1));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) m[u][kk][h] = src[(((2 * wave + u) * 4 + kk) * 2 + h) * 64 + lane];
  };
  // N_s of the lane's eight entries (the accumulator's start)
  // (entry states and N in the owners' fragment order: the lane's four rows
  // of a tile, 4 g4 .. + 3, are one vector)
  auto sfrag = [&](int u) { return pipe::sfrag_index(32 * wave + 16 * u + 4 * g4, col0 + l16); };
  auto load_n = [&](int s, floatx4 (&nr)[2]) {
    const float* Nm = mat(s, 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) nr[u] = *reinterpret_cast<const floatx4*>(Nm + sfrag(u));
  };
  auto split = [](float x, bf16& hi, bf16& lo) {
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
  };
  // three register sets of the maps: step s uses set (s - 1) % 3 and loads
  // the maps of step s + 2 into set (s + 1) % 3
  Frag mA[2][4][2], mB[2][4][2], mC[2][4][2];
  floatx4 nA[2], nB[2], nC[2];
  // S_1 (the slice's 128 x 16 entries, two 16-byte pieces per thread) and
  // the first two steps' maps, all in flight together
  // (piece v = tid + 256 u: rows 4 (v / 16) .. + 3 of slice column v % 16)
  static_assert(D * CW / 4 == 2 * NTC, "two pieces of the slice per thread");
  floatx4 sv[2];
  {
    const float* src = mat(1, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = tid + u * NTC;
      sv[u] = *reinterpret_cast<const floatx4*>(src + pipe::sfrag_index(4 * (v >> 4), col0 + (v & 15)));
    }
  }
  if (nseg > 2) {
    load_m(1, mA);
    load_n(1, nA);
    load_m(min(2, nseg - 2), mB);
    load_n(min(2, nseg - 2), nB);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = tid + u * NTC, r0 = 4 * (v >> 4), c = v & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) split(sv[u][j], T0[c * LDS_T + r0 + j], T0[PART + c * LDS_T + r0 + j]);
  }
  __syncthreads();
  // Step s: S_{s+1} = M_s S_s + N_s, from buffer (s - 1) % 2 into the other.
  // The maps of step s + 2 are loaded during the products (loads complete in
  // order; the last steps reload maps already held, so that no load is under
  // a branch).  One barrier per step: the buffer a step writes was last read
  // a step earlier.
  auto step = [&](const Frag (&mc)[2][4][2], const floatx4 (&nc)[2], Frag (&mf)[2][4][2], floatx4 (&nf)[2],
                  int sg) {
    const bf16* Tc = (sg & 1) ? T0 : T1;
    bf16* Tn = (sg & 1) ? T1 : T0;
    const int nx = min(sg + 2, nseg - 2);
    floatx4 acc[2] = {nc[0], nc[1]};
    load_m(nx, mf);
    load_n(nx, nf);
    // B operands: rows 32 kk + 8 g4 .. + 7 of slice column l16, both parts
    Frag bh[4], bl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bh[kk] = *reinterpret_cast<const Frag*>(Tc + l16 * LDS_T + 32 * kk + 8 * g4);
      bl[kk] = *reinterpret_cast<const Frag*>(Tc + PART + l16 * LDS_T + 32 * kk + 8 * g4);
    }
    // the small terms first
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        acc[u] = CM::mma32(mc[u][kk][1], bh[kk], acc[u]);
        acc[u] = CM::mma32(mc[u][kk][0], bl[kk], acc[u]);
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u] = CM::mma32(mc[u][kk][0], bh[kk], acc[u]);
    float* dst = mat(sg + 1, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<floatx4*>(dst + sfrag(u)) = acc[u];
      bf16x4 hi, lo;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16 h_, l_;
        split(acc[u][jj], h_, l_);
        hi[jj] = h_;
        lo[jj] = l_;
      }
      const int r0 = 32 * wave + 16 * u + 4 * g4;
      *reinterpret_cast<bf16x4*>(Tn + l16 * LDS_T + r0) = hi;
      *reinterpret_cast<bf16x4*>(Tn + PART + l16 * LDS_T + r0) = lo;
    }
    __syncthreads();
  };
  int sg = 1;
  for (; sg + 3 < nseg; sg += 3) {
    step(mA, nA, mC, nC, sg);
    step(mB, nB, mA, nA, sg + 1);
    step(mC, nC, mB, nB, sg + 2);
  }
  if (sg + 1 < nseg) step(mA, nA, mC, nC, sg);
  if (sg + 2 < nseg) step(mB, nB, mA, nA, sg + 1);
}

// ---------------------------------------------------------------------------
// Plan of the segmented schedule for packed sequences (one workgroup, one
// thread per sequence or start position, N <= kPlanThreads).  Sequence b
// (clamped as the prefill clamps it) has nc_b chunks and P_b = ceil(nc_b / L)
// segments; it is segmented if P_b >= 3.  Pass 1 runs the unsegmented
// sequences whole (in the start order `order`, longest first if it is the
// order kda_varlen_schedule writes) and then, per segmented sequence,
// segment 0 and the P_b - 2 runs that form the state maps of its middle
// segments (two maps each); pass 3 runs segments 1 .. P_b-1.
// Layout as VarlenPlan reads it.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int block_excl_scan(int x, int* buf, int& total) {
  const int tid = threadIdx.x;
  buf[tid] = x;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int y = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += y;
    __syncthreads();
  }
  total = buf[kPlanThreads - 1];
  const int r = buf[tid] - x;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(const int* cu, const int* order, int N, int T,
                                                                   int L, int* plan, int j1max, int j3max) {
  __shared__ int buf[kPlanThreads];
  __shared__ int nsg[kPlanThreads];
  const int tid = threadIdx.x;
  int* nsegs = plan + 4;
  int* mapbase = nsegs + N;
  int* segseq = mapbase + N;
  int2* table1 = reinterpret_cast<int2*>(plan + varlen_plan_table_offset(N));
  int2* table3 = table1 + j1max;
  // segments of sequence tid
  int P = 0;
  if (tid < N) {
    const int e0 = min(max(cu[tid], 0), T);
    const int e1 = min(max(cu[tid + 1], e0), T);
    const int nc = (e1 - e0 + C - 1) / C;
    P = (nc + L - 1) / L;
    nsegs[tid] = P;
  }
  nsg[tid] = P;
  __syncthreads();
  const bool seg = P >= 3;
  // unsegmented sequences by start position
  const int b_i = tid < N ? (order ? min(max(order[tid], 0), N - 1) : tid) : 0;
  const bool whole_i = tid < N && nsg[b_i] < 3;
  int U, S1, S3, SL, NS;
  const int u_off = block_excl_scan(whole_i ? 1 : 0, buf, U);
  const int s1_off = block_excl_scan(seg ? P - 1 : 0, buf, S1);
  const int s3_off = block_excl_scan(seg ? P - 1 : 0, buf, S3);
  const int sl_off = block_excl_scan(seg ? P : 0, buf, SL);
  const int ns_off = block_excl_scan(seg ? 1 : 0, buf, NS);
  if (whole_i && u_off < j1max) table1[u_off] = make_int2(b_i, 0);
  if (tid < N) {
    mapbase[tid] = seg ? sl_off : -1;
    if (seg) {
      segseq[ns_off] = tid;
      for (int k = 0; k < P - 1; ++k)
        if (U + s1_off + k < j1max) table1[U + s1_off + k] = make_int2(tid, k);
      for (int k = 0; k < P - 1; ++k)
        if (s3_off + k < j3max) table3[s3_off + k] = make_int2(tid, k);
    }
  }
  if (tid == 0) {
    plan[0] = min(U + S1, j1max);
    plan[1] = min(S3, j3max);
    plan[2] = NS;
    plan[3] = SL;
  }
}

VarlenSeg varlen_segments(int N, int T_total, int H, int cus) {
  VarlenSeg v{};
  if (N <= 0 || N > kPlanThreads || H <= 0 || T_total <= 0) return v;
  const int64_t nct = ((int64_t)T_total + C - 1) / C;   // chunks of the longest possible sequence
  const int64_t ncs = nct + N;                           // bound on the chunks of all sequences
  int64_t L;
  const char* e = getenv("KDA_SEGMENTS");
  if (e) {
    // about n segments for a sequence holding all the tokens (tests)
    const int want = atoi(e);
    if (want < 3) return v;
    L = (nct + want - 1) / want;
  } else {
    // segments of about one CU's share of the work, so that a sequence
    // holding all the tokens runs each pass in one round of workgroups
    // ((P - 1) H <= CUs); worth it only when one sequence can be three of them
    if (cus <= 0) return v;
    L = std::max<int64_t>(16, (ncs * H + cus + H - 1) / (cus + H));
  }
  if (L < 1 || nct < 2 * L + 1) return v;
  const int64_t ns = std::min<int64_t>(N, nct / (2 * L + 1));   // segmented sequences have > 2L chunks
  const int64_t slots = ncs / L + ns;                              // sum of their segment counts
  const int64_t j1 = N + slots, j3 = slots;
  if (j1 * H > INT32_MAX || ns * H * segc::NSC > INT32_MAX) return v;
  v.L = (int)L;
  v.j1 = (int)j1;
  v.j3 = (int)j3;
  v.ns = (int)ns;
  v.slots = (int)slots;
  v.plan_bytes = ((size_t)(varlen_plan_table_offset(N) + 2 * (j1 + j3)) * sizeof(int) + 255) / 256 * 256;
  v.bytes = v.plan_bytes + (size_t)slots * H * 3 * 128 * 128 * sizeof(float);
  return v;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <typename K>
static hipError_t set_smem(K kern, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

static inline int grid_heads(int BH, int nsplit) { return ((BH + 7) / 8) * 8 * nsplit; }

template <typename T, int DK, int DV, int NSPLIT>
static hipError_t launch_fused_t(const PrefillArgs& a, hipStream_t s) {
  constexpr int DVW = DV / NSPLIT;
  const int bytes = Layout<T, DK, DVW>::BYTES;
  auto kern = fused_fwd_kernel<T, DK, DV, NSPLIT>;
  hipError_t e = set_smem(kern, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid_heads(a.B * a.H, NSPLIT)), dim3(NT), bytes, s, a);
  return hipGetLastError();
}

int fused_default_nsplit(int BH, int dv) {
  // enough workgroups to cover the 256 compute units, each doing >= 16 columns
  int ns = 1;
  const int maxs = dv / 16;
  while (ns < maxs && (int64_t)BH * ns < 256) ns *= 2;
  return ns;
}

template <typename T, int DK, int DV>
static hipError_t launch_fused_d(const PrefillArgs& a, hipStream_t s) {
  const int ns = a.nsplit > 0 ? a.nsplit : fused_default_nsplit(a.B * a.H, DV);
  switch (ns) {
    case 1: return launch_fused_t<T, DK, DV, 1>(a, s);
    case 2: return launch_fused_t<T, DK, DV, 2>(a, s);
    case 4: return launch_fused_t<T, DK, DV, 4>(a, s);
    case 8: if (DV >= 128) return launch_fused_t<T, DK, DV, (DV >= 128 ? 8 : 4)>(a, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// The segmented schedule: pass 1 (segment 0 and the maps of the middle
// segments, with the two-state owners), the combine, pass 3.
template <int V>
static hipError_t launch_pipe_seg(const PrefillArgs& a, hipStream_t s) {
  const int bytes = pipe::BYTES;
  auto fused_pipe_pass1 = ::kda::fused_pipe_kernel<V | kPipeDual>;
  auto fused_pipe_pass3 = ::kda::fused_pipe_kernel<V | kPipeSegIn>;
  hipError_t e = set_smem(fused_pipe_pass1, bytes);
  if (e != hipSuccess) return e;
  if ((e = set_smem(fused_pipe_pass3, bytes)) != hipSuccess) return e;
  const int BH = a.B * a.H;
  if (a.plan) {
    // packed sequences, segmented: the plan, whole short sequences with
    // segment 0 and the maps of the long ones, entry states, then segments
    // 1 .. P-1 (grids at the plan's bounds; surplus workgroups exit)
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a.cu_seqlens, a.seq_order, a.B, a.T,
                       a.seg_len, a.plan, a.plan_j1, a.plan_j3);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    PrefillArgs a1 = a, a3 = a;
    a1.pass = 1;
    a3.pass = 3;
    hipLaunchKernelGGL(fused_pipe_pass1, dim3(a.plan_j1 * a.H), dim3(NT), bytes, s, a1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.plan_ns > 0 && a.plan_j3 > 0) {
      if ((e = set_smem(seg_combine_kernel, segc::BYTES)) != hipSuccess) return e;
      hipLaunchKernelGGL(seg_combine_kernel, dim3(a.plan_ns * a.H * segc::NSC), dim3(segc::NTC), segc::BYTES, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(fused_pipe_pass3, dim3(a.plan_j3 * a.H), dim3(NT), bytes, s, a3);
    }
    return hipGetLastError();
  }
  // segment 0 and the maps of the middle segments, entry states, then
  // segments 1 .. nseg-1
  PrefillArgs a1 = a, a3 = a;
  a1.pass = 1;
  a3.pass = 3;
  hipLaunchKernelGGL(fused_pipe_pass1, dim3(BH * (a.nseg - 1)), dim3(NT), bytes, s, a1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = set_smem(seg_combine_kernel, segc::BYTES)) != hipSuccess) return e;
  hipLaunchKernelGGL(seg_combine_kernel, dim3(BH * segc::NSC), dim3(segc::NTC), segc::BYTES, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(fused_pipe_pass3, dim3(BH * (a.nseg - 1)), dim3(NT), bytes, s, a3);
  return hipGetLastError();
}

template <int V>
static hipError_t launch_pipe_v(const PrefillArgs& a, hipStream_t s) {
  const int bytes = pipe::BYTES;
  auto fused_pipe_kernel = ::kda::fused_pipe_kernel<V>;
  hipError_t e = set_smem(fused_pipe_kernel, bytes);
  if (e != hipSuccess) return e;
  const int BH = a.B * a.H;
  if (a.plan || a.nseg >= 3) {
    if constexpr ((V & kPipeStates) == 0) return launch_pipe_seg<V>(a, s);
    return hipErrorInvalidValue;
  }
  PrefillArgs a0 = a;
  a0.pass = 0;
  hipLaunchKernelGGL(fused_pipe_kernel, dim3(grid_heads(BH, 1)), dim3(NT), bytes, s, a0);
  return hipGetLastError();
}

static hipError_t launch_pipe(const PrefillArgs& a, hipStream_t s) {
  // chunk-entry states (for the backward): KDA or no delta rule, one pass
  if (a.states) {
    if (a.nseg >= 3) return hipErrorInvalidValue;
    switch (a.variant) {
      case 0: return launch_pipe_v<kPipeStates>(a, s);
      case kVarNoDelta: return launch_pipe_v<kPipeStates | kVarNoDelta>(a, s);
      case kVarScalarGate: return launch_pipe_v<kPipeStates | kVarScalarGate>(a, s);
      case kVarScalarGate | kVarNoDelta: return launch_pipe_v<kPipeStates | kVarScalarGate | kVarNoDelta>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.variant) {
    case 0: return launch_pipe_v<0>(a, s);
    case kVarScalarGate: return launch_pipe_v<kVarScalarGate>(a, s);
    case kVarNoDelta: return launch_pipe_v<kVarNoDelta>(a, s);
    case kVarScalarGate | kVarNoDelta: return launch_pipe_v<kVarScalarGate | kVarNoDelta>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Segments per sequence for the segmented schedule, from a cost model in
// units of one chunk step of one workgroup: one pass takes N steps; nseg
// segments of L chunks take (1 + 0.9 (rounds of pass 1 - 1) + rounds of
// pass 3) (L + 2) (pass 1's first round holds the full runs of segment 0,
// its other rounds only two-state runs at about 0.9 of a full step; 2:
// pipeline fill and state traffic per workgroup) plus about a quarter of a
// step per combine step, where a round is one workgroup per compute unit.  0 if one pass is
// cheaper.
int prefill_segments(int BH, int T, int cus) {
  const int N = (T + C - 1) / C;
  if (BH <= 0 || cus <= 0 || N < 12) return 0;
  double best = N + 2.0;
  int best_p = 0;
  for (int P = 3; P <= 64; ++P) {
    const int L = (N + P - 1) / P, Pe = (N + L - 1) / L;
    if (Pe != P) continue;   // only counts that split into equal-length segments (bar the last)
    const int r1 = (BH * (P - 1) + cus - 1) / cus, r3 = r1;
    const double cost = (1.0 + 0.9 * (r1 - 1) + r3) * (L + 2.0) + 0.25 * (P - 2);
    if (cost < best) { best = cost; best_p = P; }
  }
  return best_p;
}

int prefill_segment_len(int T, int nseg) {
  const int N = (T + C - 1) / C;
  return nseg > 0 ? (N + nseg - 1) / nseg : N;
}

size_t prefill_segment_workspace(int BH, int nseg) {
  return nseg >= 3 ? (size_t)BH * nseg * 3 * 128 * 128 * sizeof(float) : 0;
}

// ---------------------------------------------------------------------------
// Processing order of packed sequences: indices sorted by decreasing chunk
// count (ties by index), so the longest sequences start first and the short
// ones fill in behind them.  One workgroup; a bitonic sort of 64-bit keys
// (inverted chunk count, index) in LDS.  Lengths are clamped exactly as the
// prefill kernel clamps them.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(const int* cu, int N, int T, int P,
                                                                        int* order) {
  extern __shared__ unsigned long long keys[];
  const int tid = threadIdx.x;
  for (int i = tid; i < P; i += kSchedThreads) {
    unsigned long long key = ~0ull;
    if (i < N) {
      const int e0 = min(max(cu[i], 0), T);
      const int e1 = min(max(cu[i + 1], e0), T);
      const unsigned nch = (unsigned)((e1 - e0 + C - 1) / C);
      key = ((unsigned long long)(0xFFFFFFFFu - nch) << 32) | (unsigned)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kSchedThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = keys[i], y = keys[ixj];
          if ((x > y) == ((i & k) == 0)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < N; i += kSchedThreads) order[i] = (int)(keys[i] & 0xFFFFFFFFu);
}

hipError_t launch_varlen_schedule(const int* cu_seqlens, int N, int T, int* order, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (N > kMaxScheduleSeqs) return hipErrorInvalidValue;
  int P = 1;
  while (P < N) P <<= 1;
  const int bytes = P * 8;
  hipError_t e = set_smem(varlen_schedule_kernel, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), bytes, s, cu_seqlens, N, T, P, order);
  return hipGetLastError();
}

hipError_t launch_fused(const PrefillArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  // the variants and packed sequences exist in the pipelined kernel only
  if (a.variant != 0 || a.cu_seqlens) {
    if (!(a.bf16 && a.dk == 128 && a.dv == 128) || (a.cu_seqlens && a.nseg >= 3)) return hipErrorInvalidValue;
    return launch_pipe(a, s);
  }
  if (a.bf16) {
    if (a.dk == 128 && a.dv == 128) {
      // the pipelined kernel without a column split is the faster one at every
      // measured head count (B1 H16 T4096: 0.33 ms against 0.45 ms for the best
      // split; B1 H32 T131072: 10.3 ms against 14.0 ms); an explicit split or
      // a disabled pipeline selects the serial kernel
      if (a.nsplit <= 1 && a.pipeline) return launch_pipe(a, s);
      return launch_fused_d<bf16, 128, 128>(a, s);
    }
    if (a.dk == 64 && a.dv == 64) return launch_fused_d<bf16, 64, 64>(a, s);
  } else {
    if (a.dk == 64 && a.dv == 64) return launch_fused_d<float, 64, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK>
static hipError_t launch_cumsum_t(const StageArgs& a, hipStream_t s) {
  const int bytes = Layout<T, DK, 16>::BYTES;
  auto kern = stage_cumsum_kernel<T, DK>;
  hipError_t e = set_smem(kern, bytes);
  if (e != hipSuccess) return e;
  const int nch = (a.T + C - 1) / C;
  hipLaunchKernelGGL(kern, dim3(nch, a.B * a.H), dim3(NT), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t launch_ut_t(const StageArgs& a, hipStream_t s) {
  const int bytes = Layout<T, DK, DV>::BYTES;
  auto kern = stage_ut_kernel<T, DK, DV>;
  hipError_t e = set_smem(kern, bytes);
  if (e != hipSuccess) return e;
  const int nch = (a.T + C - 1) / C;
  hipLaunchKernelGGL(kern, dim3(nch, a.B * a.H), dim3(NT), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int DK, int DV, int NSPLIT>
static hipError_t launch_state_t(const StageArgs& a, hipStream_t s) {
  constexpr int DVW = DV / NSPLIT;
  const int bytes = Layout<T, DK, DVW>::BYTES;
  auto kern = stage_state_kernel<T, DK, DV, NSPLIT>;
  hipError_t e = set_smem(kern, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid_heads(a.B * a.H, NSPLIT)), dim3(NT), bytes, s, a);
  return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t launch_output_t(const StageArgs& a, hipStream_t s) {
  const int bytes = Layout<T, DK, DV>::BYTES;
  auto kern = stage_output_kernel<T, DK, DV>;
  hipError_t e = set_smem(kern, bytes);
  if (e != hipSuccess) return e;
  const int nch = (a.T + C - 1) / C;
  hipLaunchKernelGGL(kern, dim3(nch, a.B * a.H), dim3(NT), bytes, s, a);
  return hipGetLastError();
}

#define KDA_DISPATCH(FN, ...)                                                   \
  do {                                                                          \
    if (a.bf16) {                                                               \
      if (a.dk == 128 && a.dv == 128) return FN<bf16, 128, 128 __VA_ARGS__>(a, s); \
      if (a.dk == 64 && a.dv == 64) return FN<bf16, 64, 64 __VA_ARGS__>(a, s);  \
    } else {                                                                    \
      if (a.dk == 64 && a.dv == 64) return FN<float, 64, 64 __VA_ARGS__>(a, s); \
    }                                                                           \
    return hipErrorInvalidValue;                                                \
  } while (0)

hipError_t launch_stage_cumsum(const StageArgs& a, hipStream_t s) {
  if (a.B * a.H == 0 || a.T == 0) return hipSuccess;
  if (a.bf16) {
    if (a.dk == 128) return launch_cumsum_t<bf16, 128>(a, s);
    if (a.dk == 64) return launch_cumsum_t<bf16, 64>(a, s);
  } else {
    if (a.dk == 64) return launch_cumsum_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stage_ut(const StageArgs& a, hipStream_t s) {
  if (a.B * a.H == 0 || a.T == 0) return hipSuccess;
  KDA_DISPATCH(launch_ut_t);
}

hipError_t launch_stage_state(const StageArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  KDA_DISPATCH(launch_state_t, , 1);
}

hipError_t launch_stage_output(const StageArgs& a, hipStream_t s) {
  if (a.B * a.H == 0 || a.T == 0) return hipSuccess;
  KDA_DISPATCH(launch_output_t);
}

}  // namespace kda
