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
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int C = 64;        // chunk length
constexpr int NW = 8;        // wavefronts per workgroup
constexpr int NT = NW * kWave;

// ---------------------------------------------------------------------------
// LDS layout.  Rows of bf16/fp32 operand arrays are padded by 16 bytes so that
// the 16 rows an MFMA fragment read touches fall in different banks.
// ---------------------------------------------------------------------------
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
  static constexpr int O_V = O_KBT + DK * LDC * (int)sizeof(T);
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
  static constexpr int BYTES = O_BC + DK * 4;
};

template <typename T, int DK, int DVW>
struct Smem {
  typedef Layout<T, DK, DVW> Lay;
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  TL* Kt; TL* Kh; TL* Wn; TL* Qt; TF* KbT; T* V;
  float* G; TF* Ln; TF* P; float* Ld; TF* Db;
  float* tot; float* beta; float* gam; float* bC;
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
  }
};

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
  float beta;
};

// ---------------------------------------------------------------------------
// Device blocks of the chunk computation.
// ---------------------------------------------------------------------------

// g (registers) -> G (fp32 LDS); beta -> LDS.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void stage_gates(Smem<T, DK, DVW>& sm, const Vec16* g,
                                            float beta, int tid) {
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
      for (int e = 0; e < RV::VN; ++e) sm.G[row * Lay::LDG + c0 + e] = f[e];
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
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < RPS; ++r) {
    float* p = &sm.G[(seg * RPS + r) * Lay::LDG + c];
    run += *p;
    *p = run;
  }
  sm.tot[seg * DK + c] = run;
  __syncthreads();
  float off = 0.f;
  for (int s = 0; s < seg; ++s) off += sm.tot[s * DK + c];
#pragma unroll
  for (int r = 0; r < RPS; ++r) sm.G[(seg * RPS + r) * Lay::LDG + c] += off;
  if (seg == NSEG - 1) {
    const float bl = run + off;
    sm.bC[c] = bl;
    sm.gam[c] = fast_exp(bl);
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
#pragma unroll
      for (int e = 0; e < RV::VN; ++e) {
        const float b = sm.G[row * Lay::LDG + c0 + e];
        const float ep = fast_exp(b);
        const float em = fast_exp(-b);
        kt[e] = from_f32<TL>(kf[e] * ep);
        kh[e] = from_f32<TL>(kf[e] * em);
        if (DO_QT) qt[e] = from_f32<TL>(qf[e] * ep);
        if (DO_KB) sm.KbT[(c0 + e) * Lay::LDC + row] = from_f32<TF>(kf[e] * fast_exp(sm.bC[c0 + e] - b));
      }
      if (DO_KT) *reinterpret_cast<Vec16*>(&sm.Kt[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(kt);
      if (DO_KH) *reinterpret_cast<Vec16*>(&sm.Kh[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(kh);
      if (DO_QT) *reinterpret_cast<Vec16*>(&sm.Qt[row * Lay::LDK + c0]) = *reinterpret_cast<Vec16*>(qt);
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

// Lower-triangular 16x16 block list of a 64x64 matrix; for P the blocks (0,1)
// and (2,3) are included (as zeros) because 32-wide reduction slabs read them.
__device__ __forceinline__ void blk_ij(int t, int& I, int& J) {
  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3) (0,1) (2,3),
  // packed 4 bits per entry (no indexed private arrays)
  I = (int)((0x203333222110ull >> (4 * t)) & 15u);
  J = (int)((0x313210210100ull >> (4 * t)) & 15u);
}

// L = StrictTril(Diag(beta) Kt Kh^T) (fp32 diagonal blocks, -L off-diagonal
// in T) and/or P = Tril(Qt Kh^T) (T), distributed over the wavefronts.
template <typename T, int DK, int DVW, bool DO_L, bool DO_P>
__device__ __forceinline__ void lp_tiles(Smem<T, DK, DVW>& sm, int wave, int lane) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
  constexpr int NL = DO_L ? 10 : 0;
  constexpr int NP = DO_P ? 12 : 0;
  for (int tile = wave; tile < NL + NP; tile += NW) {
    const bool isL = tile < NL;
    int I, J;
    blk_ij(isL ? tile : tile - NL, I, J);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (I >= J) {
      const TL* A = isL ? sm.Kt : sm.Qt;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const typename M::F32 af = M::lds32(A + (16 * I + l16) * Lay::LDK + 32 * ks + 4 * g4);
        const typename M::F32 bf = M::lds32(sm.Kh + (16 * J + l16) * Lay::LDK + 32 * ks + 4 * g4);
        acc = M::mma32(af, bf, acc);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int il = 4 * g4 + j;             // row inside the block
      const int i = 16 * I + il, jc = 16 * J + l16;
      float val = acc[j];
      if (isL) {
        val *= sm.beta[i];
        if (I == J) {
          if (il <= l16) val = 0.f;
          sm.Ld[(I * 16 + il) * Lay::LDL + l16] = val;
        } else {
          sm.Ln[i * Lay::LDC + jc] = from_f32<TF>(-val);
        }
      } else {
        if (I == J && il < l16) val = 0.f;
        if (I < J) val = 0.f;
        sm.P[i * Lay::LDC + jc] = from_f32<TF>(val);
      }
    }
  }
}

// (I + L_ii)^-1 for the four diagonal 16x16 blocks, by forward substitution:
// lane = 16 * block + column; column c of the inverse solves (I + L_ii) x = e_c.
// Rows of L_ii are read as 16-byte vectors; a scheduling fence every four
// rows bounds how many of them are held in registers at once.
template <typename T, int DK, int DVW>
__device__ __forceinline__ void diag_inverse(Smem<T, DK, DVW>& sm, int lane) {
  typedef Layout<T, DK, DVW> Lay;
  const int blk = lane >> 4, c = lane & 15;
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
    float s = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < r; ++m) s -= row[m] * x[m];
    x[r] = s;
    if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) sm.Db[(blk * 16 + r) * Lay::LDD + c] = from_f32<typename Operands<T>::TF>(x[r]);
}

// Blocked forward substitution for one 16-column tile:
//   X_I = D_I (beta * Src_I - sum_{M<I} L_IM X_M),  I = 0..3,
// Src rows from LDS (ld = row stride, col0 = first column).  X stays in
// registers (C layout, fp32).
template <typename T, int DK, int DVW, typename TS>
__device__ __forceinline__ void fwd_subst_tile(Smem<T, DK, DVW>& sm, const TS* src, int ld, int col0,
                                               floatx4 (&X)[4], int lane) {
  typedef Mma<typename Operands<T>::TF> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    floatx4 acc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * I + 4 * g4 + j;
      acc[j] = sm.beta[row] * to_f32(src[row * ld + col0 + l16]);
    }
#pragma unroll
    for (int Mb = 0; Mb < I; ++Mb) {
      const typename M::F16 af = M::lds16(sm.Ln + (16 * I + l16) * Lay::LDC + 16 * Mb + 4 * g4);
      acc = M::mma16(af, M::frag16(X[Mb]), acc);
    }
    const typename M::F16 df = M::lds16(sm.Db + (16 * I + l16) * Lay::LDD + 4 * g4);
    X[I] = M::mma16(df, M::frag16(acc), zero);
  }
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

// State as reduction operand: fragments of 32 state rows (key channels).
template <typename TO, int DK>
__device__ __forceinline__ void state_frags(const floatx4 (&S)[DK / 16], typename Mma<TO>::F32 (&Sf)[DK / 32]) {
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) Sf[ks] = Mma<TO>::frag32(S[2 * ks], S[2 * ks + 1]);
}

// acc[I] (+)= A[rows 16I..] @ S  for the four 16-token row blocks, A in LDS [C][LDK].
template <typename T, int DK>
__device__ __forceinline__ void rows_times_state(const T* A, int lda, const typename Mma<T>::F32 (&Sf)[DK / 32],
                                                 floatx4 (&acc)[4], int lane) {
  typedef Mma<T> M;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      acc[I] = M::mma32(M::lds32(A + (16 * I + l16) * lda + 32 * ks + 4 * g4), Sf[ks], acc[I]);
}

// O[I] += P[rows 16I..] @ Delta  (P lower triangular: slab 1 only for I >= 2)
template <typename T, int DK, int DVW>
__device__ __forceinline__ void intra_output(Smem<T, DK, DVW>& sm,
                                             const typename Mma<typename Operands<T>::TF>::F32 (&Df)[2],
                                             floatx4 (&O)[4], int lane) {
  typedef Mma<typename Operands<T>::TF> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    O[I] = M::mma32(M::lds32(sm.P + (16 * I + l16) * Lay::LDC + 4 * g4), Df[0], O[I]);
    if (I >= 2) O[I] = M::mma32(M::lds32(sm.P + (16 * I + l16) * Lay::LDC + 32 + 4 * g4), Df[1], O[I]);
  }
}

// S <- Diag(gam) S + KbT @ Delta
template <typename T, int DK, int DVW>
__device__ __forceinline__ void state_update(Smem<T, DK, DVW>& sm,
                                             const typename Mma<typename Operands<T>::TF>::F32 (&Df)[2],
                                             floatx4 (&S)[DK / 16], int lane) {
  typedef Mma<typename Operands<T>::TF> M;
  typedef Layout<T, DK, DVW> Lay;
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) S[rt][j] *= sm.gam[16 * rt + 4 * g4 + j];
    S[rt] = M::mma32(M::lds32(sm.KbT + (16 * rt + l16) * Lay::LDC + 4 * g4), Df[0], S[rt]);
    S[rt] = M::mma32(M::lds32(sm.KbT + (16 * rt + l16) * Lay::LDC + 32 + 4 * g4), Df[1], S[rt]);
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

// state tile io: S[(head*DK + row) * DV + col]
template <int DK, int DV>
__device__ __forceinline__ void load_state(floatx4 (&S)[DK / 16], const float* S0, int64_t head, int col, int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[rt][j] = S0 ? S0[(head * DK + 16 * rt + 4 * g4 + j) * DV + col] : 0.f;
}

template <int DK, int DV>
__device__ __forceinline__ void store_state(const floatx4 (&S)[DK / 16], float* out, int64_t head, int col, int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[(head * DK + 16 * rt + 4 * g4 + j) * DV + col] = S[rt][j];
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
  rg.beta = buf_load_scalar<T>(rb, tid < C ? (uint32_t)(tid * a.H * es) : 0x80000000u);
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

// ---------------------------------------------------------------------------
// Fused forward.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV, int NSPLIT>
__global__ __launch_bounds__(NT) void fused_fwd_kernel(PrefillArgs a) {
  typedef typename Operands<T>::TL TL;
  typedef typename Operands<T>::TF TF;
  typedef Mma<TL> ML;
  typedef Mma<TF> MF;
  constexpr int DVW = DV / NSPLIT;
  constexpr int OWN = DVW / 16;
  typedef Layout<T, DK, DVW> Lay;
  static_assert(OWN >= 1 && OWN <= NW, "column split");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];

  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int head, split;
  block_to_head<NSPLIT>(blockIdx.x, head, split);
  if (head >= a.B * a.H) return;
  const int bb = head / a.H, h = head % a.H;
  const int col0 = split * DVW;
  const bool owner = wave < OWN;
  const int wcol = col0 + 16 * wave;


  floatx4 S[DK / 16];
  if (owner) load_state<DK, DV>(S, a.S0, head, wcol + (lane & 15), lane);

  const int nchunks = (a.T + C - 1) / C;
  ChunkRegs<T, DK, DV, DVW> rg;
  if (nchunks > 0) fetch_chunk<T, DK, DV, DVW>(rg, a, bb, h, 0, col0, tid);
  Smem<T, DK, DVW> sm(smem_raw);

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * C;
    const int nv = min(C, a.T - t0);
    TokIdx ti;
    ti.row0 = ((int64_t)bb * a.T + t0) * a.H + h;
    ti.rstride = a.H;

    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();              // previous chunk is done with LDS
    stage_gates<T, DK, DVW>(sm, rg.g, rg.beta, tid);
    __syncthreads();
    chunk_cumsum<T, DK, DVW>(sm, tid);
    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();
    apply_gates<T, DK, DVW, true, true, true, true>(sm, rg.k, rg.q, tid);
    stage_values<T, DK, DVW>(sm, rg.v, tid);
    if (n + 1 < nchunks) fetch_chunk<T, DK, DV, DVW>(rg, a, bb, h, n + 1, col0, tid);  // overlaps this chunk's math
    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();

    // L and P products
    lp_tiles<T, DK, DVW, true, true>(sm, wave, lane);
    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();
    if (wave == 0) diag_inverse<T, DK, DVW>(sm, lane);
    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();

    // forward substitution: U tile of each owner in its registers, W to LDS
    floatx4 Ux[4];
    for (int t = wave; t < OWN + DK / 16; t += NW) {
      if (t < OWN) {
        fwd_subst_tile<T, DK, DVW>(sm, sm.V, Lay::LDV, 16 * t, Ux, lane);
      } else {
        floatx4 Wx[4];
        const int wc = 16 * (t - OWN);
        fwd_subst_tile<T, DK, DVW>(sm, sm.Kt, Lay::LDK, wc, Wx, lane);
        store_negw<T, DK, DVW>(sm, Wx, wc, lane);
      }
    }
    sm.sync_rebase(smem_raw);
    KDA_FRESH_LANE();

    if (owner) {
      typename ML::F32 Sf[DK / 32];
      state_frags<TL, DK>(S, Sf);
      // read-out of the chunk-entry state, O = Qt S, and Delta = U - W S
      floatx4 O[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) O[I] = floatx4{0.f, 0.f, 0.f, 0.f};
      rows_times_state<TL, DK>(sm.Qt, Lay::LDK, Sf, O, lane);
      rows_times_state<TL, DK>(sm.Wn, Lay::LDK, Sf, Ux, lane);
      typename MF::F32 Df[2];
      Df[0] = MF::frag32(Ux[0], Ux[1]);
      Df[1] = MF::frag32(Ux[2], Ux[3]);
      intra_output<T, DK, DVW>(sm, Df, O, lane);
      {
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(reinterpret_cast<T*>(a.o) + ti.row0 * DV, chunk_bytes(nv, a.H * DV, DV, (int)sizeof(T)));
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            buf_store_scalar<T>(ro, (uint32_t)(((16 * I + 4 * (lane >> 4) + j) * a.H * DV + wcol + (lane & 15)) * (int)sizeof(T)), O[I][j]);
      }
      state_update<T, DK, DVW>(sm, Df, S, lane);
    }
  }
  if (owner && a.S_T) store_state<DK, DV>(S, a.S_T, head, wcol + (lane & 15), lane);
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
  stage_gates<T, DK, 16>(sm, gr, 0.f, tid);
  __syncthreads();
  chunk_cumsum<T, DK, 16>(sm, tid);
  __syncthreads();
  for (int idx = tid; idx < C * DK; idx += NT) {
    const int row = idx / DK, c = idx % DK;
    if (row < nv) a.b[(ti.row0 + (int64_t)row * ti.rstride) * DK + c] = sm.G[row * Lay::LDG + c];
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
    sm.G[row * Lay::LDG + c] = b[(ti.row0 + (int64_t)rr * ti.rstride) * DK + c];
  }
  if (tid < DK) {
    const float bl = b[(ti.row0 + (int64_t)(nv - 1) * ti.rstride) * DK + tid];
    sm.bC[tid] = bl;
    sm.gam[tid] = fast_exp(bl);
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
  lp_tiles<T, DK, DV, true, false>(sm, wave, lane);
  __syncthreads();
  if (wave == 0) diag_inverse<T, DK, DV>(sm, lane);
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

  floatx4 S[DK / 16];
  if (owner) load_state<DK, DV>(S, a.S0, head, wcol + l16, lane);
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
        for (int j = 0; j < 4; ++j) Sc[(int64_t)(16 * rt + 4 * (lane >> 4) + j) * DV + wcol + l16] = S[rt][j];
      typename ML::F32 Sf[DK / 32];
      state_frags<TL, DK>(S, Sf);
      floatx4 Dx[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) Dx[I] = load_tile_rows_f32<T>(a.U, DV, ti, I, wcol + l16, nv, lane);
      rows_times_state<TL, DK>(sm.Wn, Lay::LDK, Sf, Dx, lane);
#pragma unroll
      for (int I = 0; I < 4; ++I) store_tile_rows<float>(a.Delta, DV, ti, I, wcol + l16, Dx[I], nv, lane);
      typename MF::F32 Df[2];
      Df[0] = MF::frag32(Dx[0], Dx[1]);
      Df[1] = MF::frag32(Dx[2], Dx[3]);
      state_update<T, DK, DVW>(sm, Df, S, lane);
    }
  }
  if (owner && a.S_T) store_state<DK, DV>(S, a.S_T, head, wcol + l16, lane);
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
  lp_tiles<T, DK, DV, false, true>(sm, wave, lane);
  __syncthreads();
  for (int ct = wave; ct < DV / 16; ct += NW) {
    const int col = 16 * ct + l16;
    floatx4 S[DK / 16];
    const float* Sc = a.S_chunks + ((int64_t)head * nchunks + n) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[rt][j] = Sc[(int64_t)(16 * rt + 4 * (lane >> 4) + j) * DV + col];
    typename ML::F32 Sf[DK / 32];
    state_frags<TL, DK>(S, Sf);
    floatx4 O[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) O[I] = floatx4{0.f, 0.f, 0.f, 0.f};
    rows_times_state<TL, DK>(sm.Qt, Lay::LDK, Sf, O, lane);
    floatx4 Dx[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) Dx[I] = load_tile_rows_f32<T>(a.Delta, DV, ti, I, col, nv, lane);
    typename MF::F32 Df[2];
    Df[0] = MF::frag32(Dx[0], Dx[1]);
    Df[1] = MF::frag32(Dx[2], Dx[3]);
    intra_output<T, DK, DV>(sm, Df, O, lane);
#pragma unroll
    for (int I = 0; I < 4; ++I) store_tile_rows<T>(reinterpret_cast<T*>(a.o), DV, ti, I, col, O[I], nv, lane);
  }
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

hipError_t launch_fused(const PrefillArgs& a, hipStream_t s) {
  if (a.B * a.H == 0) return hipSuccess;
  if (a.bf16) {
    if (a.dk == 128 && a.dv == 128) return launch_fused_d<bf16, 128, 128>(a, s);
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
