// kda_backward.hip -- backward of the chunked KDA forward (bf16, d_k = d_v = 128).
//
// The gradient of the forward with respect to q, k, v, g, beta and S0, given
// the adjoints of o and S_T.  The pages give the forward only ("Hybrid Linear
// Attention Architecture: Making LLM Training and Inference More Efficient"
// §3.3 for the rule, §IV for the chunked form and its training purpose); the
// backward here is the reverse-mode derivative of that chunked form, chunk by
// chunk.  Per chunk, with the forward's notation (b the in-chunk cumulative
// log-gate, Kg = e^b k, Kd = e^-b k, Qg = e^b q, gamma = e^{b_C}, L =
// StrictTril(Diag(beta) Kg Kd^T), A = (I + L)^-1, A' = A Diag(beta), entry
// state S, chunk-end adjoint dS):
//
//   Delta  = A' (V - Kg S)                        (= U - W S)
//   dDelta = P^T dO + Kd (gamma . dS)             (P = Tril(Qg Kd^T), exact diagonal q.k)
//   dS_prev = gamma . dS + Qg^T dO - Kg^T (A'^T dDelta)
//   M = Tril(dO Delta^T)        dQg = dO S^T + M Kd      dKd = M^T Qg + dG^T Kg
//   dKb~ = Delta (gamma . dS)^T (= gamma . dKb)      dW = -dDelta S^T
//   dV = A'^T dDelta            dKg = Diag(beta) (A^T dW + dL Kd)
//   dA = (dDelta V^T + dW Kg^T) Diag(beta)     dL = -StrictTril(A^T dA A^T)   dG = Diag(beta) dL
//   dbeta = rowsum((A^T dDelta) . V) + rowsum((A^T dW) . Kg) + rowsum(Kg . (dL Kd))
//   db = Kg.dKg - Kd.(dKd + dKb~) + Qg.dQg, plus at the chunk end
//        sum_t Kd.dKb~ + gamma . rowsum(dS . S);   dg = reverse in-chunk cumsum of db
//   dq = e^b dQg + M_tt k_t,   dk = e^b dKg + e^-b (dKd + dKb~) + M_tt q_t
// (M's diagonal and P's diagonal carry no gate factors and are kept exact).
//
// Four launches:
//   1. the pipelined forward kernel in state mode (its own instantiation):
//      the entry state S_[n] of every chunk, bf16, in the forward owners'
//      fragment order;
//   2. bwd_prep_kernel, per (chunk, sequence, head): A = (I + L)^-1 and P^T
//      (bf16 64 x 64 each), the gated operands Kg, Kd, Qg (bf16 64 x 128),
//      gamma and beta, into a per-chunk operand block;
//   3. bwd_chain_kernel, per (sequence, head): the adjoint recursion over the
//      chunks in reverse (dS fp32 in registers, eight value-column tiles per
//      wave), storing each chunk-end adjoint (bf16, 16 x 16 tiles) and dS0;
//   4. bwd_grad_kernel, per (chunk, sequence, head): all gradients of the
//      chunk from its entry state, its chunk-end adjoint and its operand block.
// Packed sequences use the same launches: chunk n of sequence b sits in slot
// floor(cu[b] / 64) + b + n of the per-chunk arrays (head-minor).
// Matrix products: v_mfma_f32_16x16x32_bf16 on bf16 operands from LDS (16-byte
// fragments, or pairs of transpose reads), fp32 accumulation; the
// unit-triangular inverse in fp32.
#include <stdint.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace bwd {

constexpr int C = 64, D = 128, NT = 512;
constexpr int P128 = 136;   // bf16 rows of 128 (8-byte fragment reads conflict-free)
constexpr int P64 = 72;     // bf16 rows of 64
constexpr int PF = 68;      // fp32 rows of 64
constexpr int PB = 132;     // fp32 rows of 128
typedef Mma<bf16> MB;
typedef Mma<float> MF;

// ---------------------------------------------------------------- fragments
// Operand fragment of a 16-index slab (lane group g: indices k..k+3 with
// k = slab + 4g; lane i: row m0 + i), read either from a row-major array whose
// rows are the fragment rows (indices contiguous, one 8-byte read) or from one
// whose rows are the indices, with one LDS transpose read
// (ds_read_b64_tr_b16).  That instruction works on each 16-lane group alone:
// lane i receives, for r = 0..3, element i % 4 of the four 16-bit elements at
// the address of lane 4r + i / 4.  So lane j addresses row k + j / 4, columns
// m0 + 4 (j % 4) .. + 3, and lane i receives p[k + r][m0 + i] (m0 a multiple
// of 4 and ld a multiple of 4: 8-byte aligned addresses).
__device__ __forceinline__ bf16x4 fr_row(const bf16* p, int ld, int row, int k) {
  return *reinterpret_cast<const bf16x4*>(p + row * ld + k);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 fr_tr(const bf16* p, int ld, int m0, int k, int lane) {
  const int j = lane & 15;
  const bf16* a = p + (k + (j >> 2)) * ld + m0 + 4 * (j & 3);
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
  return __builtin_bit_cast(bf16x4, x);
}
// The same for a 32-index slab and v_mfma_f32_16x16x32_bf16 (lane group g:
// indices k..k+7 with k = slab + 8g): one 16-byte read, or two transpose
// reads (indices k..k+3, k+4..k+7).
__device__ __forceinline__ bf16x8 fr_row8(const bf16* p, int ld, int row, int k) {
  return *reinterpret_cast<const bf16x8*>(p + row * ld + k);
}
__device__ __forceinline__ bf16x8 fr_tr8(const bf16* p, int ld, int m0, int k, int lane) {
  const bf16x4 lo = fr_tr(p, ld, m0, k, lane), hi = fr_tr(p, ld, m0, k + 4, lane);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Out tile (m0.., n0..) += sum_{k < K} X[m][k] Z[n][k]; XR / ZR: X / Z stored
// with k contiguous (else stored transposed, k = row).  C layout result:
// lane (g, i) holds Out[m0 + 4g + r][n0 + i].
template <bool XR, bool ZR, bool SWAP = false>
__device__ __forceinline__ floatx4 mm(const bf16* X, int ldx, const bf16* Z, int ldz, int m0, int n0, int K,
                                      floatx4 acc, int lane) {
  const int g = lane >> 4, i = lane & 15;
  for (int k = 0; k < K; k += 32) {
    const bf16x8 a = XR ? fr_row8(X, ldx, m0 + i, k + 8 * g) : fr_tr8(X, ldx, m0, k + 8 * g, lane);
    const bf16x8 b = ZR ? fr_row8(Z, ldz, n0 + i, k + 8 * g) : fr_tr8(Z, ldz, n0, k + 8 * g, lane);
    acc = SWAP ? MB::mma32(b, a, acc) : MB::mma32(a, b, acc);
  }
  return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }
// x if keep, else zeros (word by word)
__device__ __forceinline__ Vec16 keep_or_zero(const Vec16& x, bool keep) {
  Vec16 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r.w[w] = keep ? x.w[w] : 0u;
  return r;
}

// NTL tiles (m0[t].., n0..) of the same product shape sharing their Z
// columns: each Z fragment is read once per 16-index step for all of them.
// SWAP: the tiles are formed transposed (operands swapped), so lane (g, i)
// holds Out[m0 + i][n0 + 4g + r]: four adjacent columns of one row.
template <bool XR, bool ZR, int NTL, bool SWAP = false>
__device__ __forceinline__ void mm_zs(const bf16* X, int ldx, const int (&m0)[NTL], const bf16* Z, int ldz, int n0,
                                      int K, floatx4 (&acc)[NTL], int lane) {
  const int g = lane >> 4, i = lane & 15;
  for (int k = 0; k < K; k += 32) {
    const bf16x8 b = ZR ? fr_row8(Z, ldz, n0 + i, k + 8 * g) : fr_tr8(Z, ldz, n0, k + 8 * g, lane);
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const bf16x8 a = XR ? fr_row8(X, ldx, m0[t] + i, k + 8 * g) : fr_tr8(X, ldx, m0[t], k + 8 * g, lane);
      acc[t] = SWAP ? MB::mma32(b, a, acc[t]) : MB::mma32(a, b, acc[t]);
    }
  }
}

// C-layout tile -> row-major dst[m][n] (2-byte stores)
__device__ __forceinline__ void st_rm(bf16* dst, int ld, int m0, int n0, floatx4 v, int lane) {
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(m0 + 4 * g + r) * ld + n0 + i] = (bf16)v[r];
}
// Transposed-layout tile (lane: row m0 + i, columns n0 + 4g ..) -> row-major
// dst[m][n] (8-byte stores)
__device__ __forceinline__ void st_rm8(bf16* dst, int ld, int m0, int n0, floatx4 v, int lane) {
  const int g = lane >> 4, i = lane & 15;
  bf16x4 x;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (bf16)v[r];
  *reinterpret_cast<bf16x4*>(dst + (m0 + i) * ld + n0 + 4 * g) = x;
}
// C-layout tile -> transposed row-major dst[n][m] (8-byte stores)
__device__ __forceinline__ void st_tr(bf16* dst, int ld, int m0, int n0, floatx4 v, int lane) {
  const int g = lane >> 4, i = lane & 15;
  bf16x4 x;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (bf16)v[r];
  *reinterpret_cast<bf16x4*>(dst + (n0 + i) * ld + m0 + 4 * g) = x;
}

// Sum over the 16 lanes of the caller's 16-lane row (lanes i = 0..15, same g),
// in every lane of the row: a butterfly of DPP row rotations (row_ror by 8,
// 4, 2, 1), VALU only.
template <int K>
__device__ __forceinline__ float add_row_ror(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + K, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x = add_row_ror<8>(x);
  x = add_row_ror<4>(x);
  x = add_row_ror<2>(x);
  return add_row_ror<1>(x);
}

// ---------------------------------------------------------------- chunk basics
struct Chunk {
  int64_t row0;   // token index (b*T + t0)*H + h of the chunk's first token
  int nv;         // valid rows
  int rstride;    // elements between rows of a [.., H, 128] tensor (= H*128)
};

// Shared LDS of the chunk basics (offsets in bytes from the kernel's base).
struct Basics {
  bf16 *Kg, *Kd, *Qg;   // [64][P128]
  bf16 *A;              // [64][P64] (I + L)^-1, unscaled; upper part zero
  bf16 *PT;             // [64][P64] P^T (P = Tril(Qg Kd^T), diagonal q.k)
  float *beta, *gam, *qk;   // [64], [128], [64]
};

// Inclusive prefix sums down the 64 rows of the 128 columns of bs (fp32
// [64][PB]), in place: thread (column c, row group of 16) sums its rows in
// registers, the four group totals meet in `tot` (4 x 128 floats of scratch
// after the array).  gam (if not NULL) receives exp of each column's total.
// REV: suffix sums (from the last row up) instead.
template <bool REV>
__device__ void scan_cols(float* bs, float* gam, int tid) {
  float* tot = bs + C * PB;
  const int c = tid & 127, rg = tid >> 7;
  // row of step r of my group
  auto row = [&](int r) { return REV ? C - 1 - (16 * rg + r) : 16 * rg + r; };
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = bs[row(r) * PB + c];
#pragma unroll
  for (int r = 1; r < 16; ++r) x[r] += x[r - 1];
  tot[rg * D + c] = x[15];
  __syncthreads();
  float off = 0.f;
  for (int u = 0; u < rg; ++u) off += tot[u * D + c];
#pragma unroll
  for (int r = 0; r < 16; ++r) bs[row(r) * PB + c] = x[r] + off;
  if (gam && rg == 3) gam[c] = __expf(x[15] + off);
  __syncthreads();
}

// Off-diagonal blocks of block column J (fp32 MFMA; the column's blocks in
// C layout serve as B operands).
template <int J>
__device__ __forceinline__ void solve_col(const float* Ls, float* As, int lane) {
  const int g4 = lane >> 4, i = lane & 15;
  floatx4 col[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) col[J][r] = As[(16 * J + 4 * g4 + r) * PF + 16 * J + i];
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    floatx4 t = zero4();
#pragma unroll
    for (int K = J; K < I; ++K) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(Ls + (16 * I + i) * PF + 16 * K + 4 * g4);
      t = MF::mma16(a, col[K], t);
    }
    const floatx4 d = *reinterpret_cast<const floatx4*>(As + (16 * I + i) * PF + 16 * I + 4 * g4);
    floatx4 y = MF::mma16(d, t, zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      y[r] = -y[r];
      As[(16 * I + 4 * g4 + r) * PF + 16 * J + i] = y[r];
    }
    col[I] = y;
  }
}

// A = (I + L)^-1 (fp32, in As [64][PF]) from Ls.
// Diagonal 16x16 blocks by forward substitution (one wavefront each, lane =
// column); off-diagonal blocks of block column J top to bottom,
// A_IJ = -D_I sum_{J<=K<I} L_IK A_KJ, with fp32 MFMA and the column's blocks
// kept in registers (waves 0-2, one column each).
__device__ void solve_fp32(const float* Ls, float* As, int tid) {
  const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, i = lane & 15;
  if (wave < 4) {
    const int I = wave, c = i;
    const float* Lb = Ls + 16 * I * PF + 16 * I;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r)
#pragma unroll
      for (int m = 0; m < r; ++m) x[r] -= Lb[r * PF + m] * x[m];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if (rr == 4 * g4 + r) v = x[rr];
      As[(16 * I + 4 * g4 + r) * PF + 16 * I + c] = v;
    }
  }
  // zero the strictly upper blocks
  for (int e = tid; e < C * C; e += NT) {
    const int t = e >> 6, s = e & 63;
    if ((s >> 4) > (t >> 4)) As[t * PF + s] = 0.f;
  }
  __syncthreads();
  if (wave == 0) solve_col<0>(Ls, As, lane);
  else if (wave == 1) solve_col<1>(Ls, As, lane);
  else if (wave == 2) solve_col<2>(Ls, As, lane);
  __syncthreads();
}

// ---------------------------------------------------------------- per-chunk matrices
// A = (I + L)^-1 and P^T of every chunk (bf16 [64][64] each, row-major), for
// the chain and the gradient kernels: one workgroup per (chunk, sequence,
// head), in an order that lets Qg and Kg share one buffer (P first, then G).
namespace pr {
constexpr int O_X = 0;                           // Qg, then Kg [64][P128]
constexpr int O_KD = O_X + C * P128 * 2;         // Kd
constexpr int O_BS = O_KD + C * P128 * 2;        // fp32 b (+ scan scratch); later Ls, As
constexpr int SZ_BS = (C * PB + 4 * D > 2 * C * PF ? C * PB + 4 * D : 2 * C * PF) * 4;
constexpr int O_BETA = O_BS + SZ_BS;
constexpr int O_QK = O_BETA + C * 4;
constexpr int BYTES = O_QK + C * 4;
static_assert(BYTES <= 80 * 1024, "two workgroups per compute unit");
}  // namespace pr

// Per-chunk block of the workspace (bf16 element offsets): A, P^T (64 x 64),
// the gated operands Kg, Kd, Qg (64 x 128, row-major), then fp32 gamma [128]
// and beta [64] (zero past the chunk's valid rows).
constexpr int M_A = 0, M_PT = C * C, M_KG = 2 * C * C, M_KD = M_KG + C * D, M_QG = M_KD + C * D;
constexpr int M_GAM = M_QG + C * D;
constexpr int MATS = M_GAM + 2 * (D + C);
static_assert((MATS * 2) % 16 == 0, "16-byte aligned blocks");

__device__ __forceinline__ bf16* chunk_mats(const BackwardArgs& a, int64_t idx) {
  return reinterpret_cast<bf16*>(a.mats) + idx * (int64_t)MATS;
}

// Sequence b, head h: its first row (token-major rows of H), its length, its
// chunk count, and where its chunks sit in the per-chunk arrays (states,
// adjoints, operand blocks): chunk n is block idx0 + n * istride.  A batch
// stores each (sequence, head) contiguously; packed sequences (cu_seqlens,
// entries clamped to [0, T]) put chunk n of sequence b in slot
// floor(cu[b] / C) + b + n, head-minor: the slot ranges of consecutive
// sequences are disjoint and every slot is below floor(T / C) + B.
struct SeqView {
  int64_t row0, idx0;
  int len, nch, istride;
};
__device__ __forceinline__ SeqView seq_view(const BackwardArgs& a, int b, int h) {
  SeqView v;
  if (a.cu_seqlens) {
    const int e0 = min(max(a.cu_seqlens[b], 0), a.T), e1 = min(max(a.cu_seqlens[b + 1], e0), a.T);
    v.row0 = (int64_t)e0 * a.H + h;
    v.len = e1 - e0;
    v.idx0 = (int64_t)(e0 / C + b) * a.H + h;
    v.istride = a.H;
  } else {
    v.row0 = (int64_t)b * a.T * a.H + h;
    v.len = a.T;
    v.idx0 = (int64_t)(b * a.H + h) * ((a.T + C - 1) / C);
    v.istride = 1;
  }
  v.nch = (v.len + C - 1) / C;
  return v;
}

// Block index -> (sequence, head, chunk) of the per-chunk kernels; false for
// a slot no chunk uses (packed sequences: nslots * H blocks, the sequence
// found by binary search over the slot starts floor(cu[b] / C) + b).
__device__ __forceinline__ bool chunk_of_block(const BackwardArgs& a, int blk, int& b, int& h, int& n) {
  if (!a.cu_seqlens) {
    const int N = (a.T + C - 1) / C;
    const int bh = blk / N;
    n = blk % N;
    b = bh / a.H;
    h = bh % a.H;
    return bh < a.B * a.H;
  }
  const int slot = blk / a.H;
  h = blk % a.H;
  auto start = [&](int x) { return min(max(a.cu_seqlens[x], 0), a.T) / C + x; };
  int lo = 0, hi = a.B - 1;   // largest b with start(b) <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start(mid) <= slot) lo = mid;
    else hi = mid - 1;
  }
  b = lo;
  n = slot - start(b);
  return n >= 0 && slot < a.nslots && n < seq_view(a, b, h).nch;
}

// V: variant flags (kVarNoDelta: no beta, no L or A; the A block is left
// unwritten and never read).
template <int V>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BackwardArgs a) {
  constexpr bool ND = (V & kVarNoDelta) != 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, h, n;
  if (!chunk_of_block(a, blockIdx.x, b, h, n)) return;
  const SeqView sv = seq_view(a, b, h);
  bf16* X = reinterpret_cast<bf16*>(sm + pr::O_X);
  bf16* Kd = reinterpret_cast<bf16*>(sm + pr::O_KD);
  float* bs = reinterpret_cast<float*>(sm + pr::O_BS);
  float* beta = reinterpret_cast<float*>(sm + pr::O_BETA);
  float* qkd = reinterpret_cast<float*>(sm + pr::O_QK);
  const bf16* q = reinterpret_cast<const bf16*>(a.q);
  const bf16* k = reinterpret_cast<const bf16*>(a.k);
  const bf16* g = reinterpret_cast<const bf16*>(a.g);
  const int64_t row0 = sv.row0 + (int64_t)n * C * a.H;
  const int nv = min(C, sv.len - n * C);
  bf16* Am = chunk_mats(a, sv.idx0 + (int64_t)n * sv.istride);
  bf16* PTm = Am + M_PT;

  // g, q, k of the chunk (thread: rows t = e / 16 of e = tid, tid + 512,
  // channels 8 (e % 16) .. + 8; rows past nv zero), every load issued first
  Vec16 xg[2], xq[2], xk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * NT, t = e >> 4, x0 = 8 * (e & 15);
    xg[u] = xq[u] = xk[u] = Vec16{{0u, 0u, 0u, 0u}};
    if (t < nv) {
      const int64_t off = (row0 + (int64_t)t * a.H) * D + x0;
      xg[u] = ldg16(g + off);
      xq[u] = ldg16(q + off);
      xk[u] = ldg16(k + off);
    }
  }
  if (tid < C) beta[tid] = !ND && tid < nv ? (float)reinterpret_cast<const bf16*>(a.beta)[row0 + (int64_t)tid * a.H] : 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * NT, t = e >> 4, x0 = 8 * (e & 15);
    float f[8];
    vec_to_f32<bf16>(xg[u], f);
#pragma unroll
    for (int v = 0; v < 8; ++v) bs[t * PB + x0 + v] = f[v];
  }
  __syncthreads();
  scan_cols<false>(bs, nullptr, tid);
  // Qg (into X), Kd, exact q.k
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int e = tid + uu * NT, t = e >> 4, x0 = 8 * (e & 15);
    float fq[8], fk[8];
    vec_to_f32<bf16>(xq[uu], fq);
    vec_to_f32<bf16>(xk[uu], fk);
    bf16x8 qg, kd;
    float qk = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float bb = bs[t * PB + x0 + u];
      qg[u] = (bf16)(fq[u] * __expf(bb));
      kd[u] = (bf16)(fk[u] * __expf(-bb));
      qk += fq[u] * fk[u];
    }
    *reinterpret_cast<bf16x8*>(X + t * P128 + x0) = qg;
    *reinterpret_cast<bf16x8*>(Kd + t * P128 + x0) = kd;
    *reinterpret_cast<bf16x8*>(Am + M_QG + t * D + x0) = qg;
    *reinterpret_cast<bf16x8*>(Am + M_KD + t * D + x0) = kd;
    qk = sum16(qk);
    if ((e & 15) == 0) qkd[t] = qk;
  }
  if (tid < D) reinterpret_cast<float*>(Am + M_GAM)[tid] = __expf(bs[(C - 1) * PB + tid]);
  if (tid < C) reinterpret_cast<float*>(Am + M_GAM)[D + tid] = beta[tid];
  __syncthreads();
  // P^T to memory (zero tiles where P is zero); lower tiles from Qg Kd^T
  for (int e = tid; e < C * C / 4; e += NT) {
    const int r = e >> 4, c4 = 4 * (e & 15);    // PT row r = t', columns t = c4..c4+3
    if ((r >> 4) <= (c4 >> 4)) continue;         // written below (P tile (c4/16, r/16) is lower)
    *reinterpret_cast<bf16x4*>(PTm + r * C + c4) = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
  for (int q10 = wave; q10 < 10; q10 += NT / 64) {
    int I = 0, J = 0;
    {
      int cc = 0;
      for (int x = 0; x < 4; ++x)
        for (int y = 0; y <= x; ++y) {
          if (cc == q10) { I = x; J = y; }
          ++cc;
        }
    }
    floatx4 acc = mm<true, true>(X, P128, Kd, P128, 16 * I, 16 * J, D, zero4(), lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * I + 4 * g4 + r, s2 = 16 * J + i;
      acc[r] = t > s2 ? acc[r] : (t == s2 ? qkd[t] : 0.f);
    }
    st_tr(PTm, C, 16 * I, 16 * J, acc, lane);
  }
  __syncthreads();
  // Kg (into X)
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int e = tid + uu * NT, t = e >> 4, x0 = 8 * (e & 15);
    float fk[8];
    vec_to_f32<bf16>(xk[uu], fk);
    bf16x8 kg;
#pragma unroll
    for (int u = 0; u < 8; ++u) kg[u] = (bf16)(fk[u] * __expf(bs[t * PB + x0 + u]));
    *reinterpret_cast<bf16x8*>(X + t * P128 + x0) = kg;
    *reinterpret_cast<bf16x8*>(Am + M_KG + t * D + x0) = kg;
  }
  __syncthreads();
  if constexpr (!ND) {
  // L = StrictTril(Diag(beta) Kg Kd^T) (over b: b is dead), then A
  float* Ls = bs;
  float* As = bs + C * PF;
  for (int e = tid; e < C * PF; e += NT) Ls[e] = 0.f;
  __syncthreads();
  for (int q10 = wave; q10 < 10; q10 += NT / 64) {
    int I = 0, J = 0;
    {
      int cc = 0;
      for (int x = 0; x < 4; ++x)
        for (int y = 0; y <= x; ++y) {
          if (cc == q10) { I = x; J = y; }
          ++cc;
        }
    }
    const floatx4 acc = mm<true, true>(X, P128, Kd, P128, 16 * I, 16 * J, D, zero4(), lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * I + 4 * g4 + r, s2 = 16 * J + i;
      Ls[t * PF + s2] = t > s2 ? acc[r] * beta[t] : 0.f;
    }
  }
  __syncthreads();
  solve_fp32(Ls, As, tid);
  for (int e = tid; e < C * C / 4; e += NT) {
    const int t = e >> 4, s4 = 4 * (e & 15);
    bf16x4 x;
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = (bf16)(s4 + u <= t ? As[t * PF + s4 + u] : 0.f);
    *reinterpret_cast<bf16x4*>(Am + t * C + s4) = x;
  }
  }
}

// A chunk's block of the workspace (A, P^T, Kg, Kd, Qg, gamma, beta), held in
// registers between their loads and their stores to LDS: every load of a
// thread is issued before the first store, so the loads overlap each other
// (and, in the chain, the previous chunk's products).  A, P^T take two
// 16-byte pieces per thread, Kg, Kd, Qg six, and the 192 floats of gamma and
// beta one float each (threads < 192, every thread loading one in range: a
// load under a branch, or a narrow load converted where it lands, made the
// compiler wait there for every load issued before it).  The split of the
// pieces assumes 512 threads.
struct ChunkOps {
  Vec16 m[8];
  float gb;
};
static_assert(NT == 512, "ChunkOps piece split (and the gradient kernel's staging: 64 x 64 halves, one piece per thread)");

template <int U0 = 0, int U1 = 8>
__device__ __forceinline__ void ops_issue(ChunkOps& x, const bf16* Am, int tid) {
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    const int e = tid + u * NT;
    if (u < 2) {
      const int m = e >> 9, r = (e >> 3) & 63, c8 = 8 * (e & 7);
      x.m[u] = ldg16(Am + m * C * C + r * C + c8);
    } else {
      const int f = e - 2 * C * 8, m = f >> 10, r = (f >> 4) & 63, c8 = 8 * (f & 15);
      x.m[u] = ldg16(Am + M_KG + m * C * D + r * D + c8);
    }
  }
  if (U0 == 0) x.gb = reinterpret_cast<const float*>(Am + M_GAM)[min(tid, D + C - 1)];
}

// (A, P^T and Kg, Kd, Qg adjacent in LDS, in that order)
__device__ __forceinline__ void ops_commit(const ChunkOps& x, const Basics& L, int tid) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid + u * NT;
    if (u < 2) {
      const int m = e >> 9, r = (e >> 3) & 63, c8 = 8 * (e & 7);
      *reinterpret_cast<Vec16*>(L.A + m * C * P64 + r * P64 + c8) = x.m[u];
    } else {
      const int f = e - 2 * C * 8, m = f >> 10, r = (f >> 4) & 63, c8 = 8 * (f & 15);
      *reinterpret_cast<Vec16*>(L.Kg + m * C * P128 + r * P128 + c8) = x.m[u];
    }
  }
  if (tid < D)
    L.gam[tid] = x.gb;
  else if (tid < D + C)
    L.beta[tid - D] = x.gb;
}

__device__ __forceinline__ void load_chunk(const Basics& L, const bf16* Am, int tid) {
  ChunkOps x;
  ops_issue(x, Am, tid);
  ops_commit(x, L, tid);
  __syncthreads();
}

// The chain's operands of one chunk in registers: the chunk block and dO
// (two 16-byte pieces per thread, rows past nv zero).
struct ChainOps {
  ChunkOps k;
  Vec16 o[2];
};

// In three parts, one at the start of each product phase of the chain, so
// that no phase stalls on issuing all eleven loads at once: A, P^T, gamma and
// beta; Kg, half of Kd; the rest of Kd, Qg, dO.
template <int PART>
__device__ __forceinline__ void chain_issue(ChainOps& x, const bf16* Am, const bf16* dO, const Chunk& c, int H,
                                            int tid) {
  if (PART == 0) ops_issue<0, 2>(x.k, Am, tid);
  if (PART == 1) ops_issue<2, 5>(x.k, Am, tid);
  if (PART == 2) {
    ops_issue<5, 8>(x.k, Am, tid);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * NT, t = e >> 4, c0 = 8 * (e & 15);
      x.o[u] = Vec16{{0u, 0u, 0u, 0u}};
      if (t < c.nv) x.o[u] = ldg16(dO + (c.row0 + (int64_t)t * H) * D + c0);
    }
  }
}

__device__ __forceinline__ void chain_commit(const ChainOps& x, const Basics& L, bf16* sDO, int tid) {
  ops_commit(x.k, L, tid);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * NT, t = e >> 4, c0 = 8 * (e & 15);
    *reinterpret_cast<Vec16*>(sDO + t * P128 + c0) = x.o[u];
  }
}

// ---------------------------------------------------------------- the chain
// LDS of bwd_chain_kernel (bytes).
namespace ch {
constexpr int O_KG = 0;
constexpr int O_KD = O_KG + C * P128 * 2;
constexpr int O_QG = O_KD + C * P128 * 2;
constexpr int O_A = O_QG + C * P128 * 2;
constexpr int O_PT = O_A + C * P64 * 2;
constexpr int O_DO = O_PT + C * P64 * 2;          // dO row-major [64][P128]
constexpr int O_DSG = O_DO + C * P128 * 2;        // (gamma . dS)^T [128 j][P128]
constexpr int O_DDT = O_DSG + D * P128 * 2;       // dDelta^T [128 j][P64]
constexpr int O_ET = O_DDT + D * P64 * 2;         // E^T [128 j][P64]
constexpr int O_BETA = O_ET + D * P64 * 2;
constexpr int O_GAM = O_BETA + C * 4;
constexpr int O_GAMN = O_GAM + D * 4;             // gamma of the next chunk (read before its commit)
constexpr int O_QK = O_GAMN + D * 4;
constexpr int BYTES = O_QK + C * 4;
static_assert(O_KD == O_KG + C * P128 * 2 && O_QG == O_KD + C * P128 * 2 && O_PT == O_A + C * P64 * 2,
              "load_chunk layout");
static_assert(BYTES <= 160 * 1024, "LDS");
}  // namespace ch

__device__ __forceinline__ Basics basics(unsigned char* sm, int kg, int kd, int qg, int a, int pt, int be, int ga,
                                         int qk) {
  Basics L;
  L.Kg = reinterpret_cast<bf16*>(sm + kg);
  L.Kd = reinterpret_cast<bf16*>(sm + kd);
  L.Qg = reinterpret_cast<bf16*>(sm + qg);
  L.A = reinterpret_cast<bf16*>(sm + a);
  L.PT = reinterpret_cast<bf16*>(sm + pt);
  L.beta = reinterpret_cast<float*>(sm + be);
  L.gam = reinterpret_cast<float*>(sm + ga);
  L.qk = reinterpret_cast<float*>(sm + qk);
  return L;
}

// One workgroup per (sequence, head): dS in registers (wave w: value-column
// tile w, all eight channel tiles), chunks in reverse.
// V: variant flags (kVarNoDelta: dS <- gamma . dS + Qg^T dO, no E term).
template <int V>
__global__ __launch_bounds__(NT) void bwd_chain_kernel(BackwardArgs a) {
  constexpr bool ND = (V & kVarNoDelta) != 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H, h = bh % a.H;
  const SeqView sv = seq_view(a, b, h);
  const int N = sv.nch;
  const Basics L = basics(sm, ch::O_KG, ch::O_KD, ch::O_QG, ch::O_A, ch::O_PT, ch::O_BETA, ch::O_GAM, ch::O_QK);
  bf16* sDO = reinterpret_cast<bf16*>(sm + ch::O_DO);
  bf16* sDSG = reinterpret_cast<bf16*>(sm + ch::O_DSG);
  bf16* sDDT = reinterpret_cast<bf16*>(sm + ch::O_DDT);
  bf16* sET = reinterpret_cast<bf16*>(sm + ch::O_ET);
  float* gamN = reinterpret_cast<float*>(sm + ch::O_GAMN);
  const bf16* dO = reinterpret_cast<const bf16*>(a.dO);

  const int jt = wave;   // my dS tiles: (ct, jt), ct = 0..7
  floatx4 dS[8];
  const float* dST = a.dS_T ? a.dS_T + (int64_t)bh * D * D : nullptr;
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) dS[u][r] = dST ? dST[(16 * u + 4 * g4 + r) * D + 16 * jt + i] : 0.f;

  auto chunk_of = [&](int n) {
    Chunk c;
    c.row0 = sv.row0 + (int64_t)n * C * a.H;
    c.nv = min(C, sv.len - n * C);
    c.rstride = a.H * D;
    return c;
  };
  auto blk = [&](int n) { return sv.idx0 + (int64_t)n * sv.istride; };
  // chunk-end adjoint of chunk nn (bf16, in 16 x 16 tiles: tile (j/16, c/16)
  // at position 8 (j/16) + c/16, [j%16][c%16] inside): one wave store writes
  // one whole tile, 512 contiguous bytes
  auto store_adj = [&](int nn) {
    bf16* adj = reinterpret_cast<bf16*>(a.adjoints) + blk(nn) * D * D;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      bf16x4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (bf16)dS[u][r];
      *reinterpret_cast<bf16x4*>(adj + (8 * jt + u) * 256 + 16 * i + 4 * g4) = x;
    }
  };
  // (gamma . dS)^T for the chunk whose decay gm holds
  auto stage_gds = [&](const float* gm) {
    if constexpr (!ND) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const floatx4 g4v = *reinterpret_cast<const floatx4*>(gm + 16 * u + 4 * g4);
        floatx4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = dS[u][r] * g4v[r];
        st_tr(sDSG, P128, 16 * u, 16 * jt, v, lane);
      }
    }
  };
  // Four phases per chunk: dDelta; E; the dS update with the next chunk's
  // adjoint staged; the next chunk's operands from registers to LDS.  The
  // next chunk's loads are issued in three parts (after the commit, then at
  // the start of the first two phases) and its decay goes to LDS one phase
  // before the commit, for the staging.
  ChainOps ops;
  if (N > 0) {
    chain_issue<0>(ops, chunk_mats(a, blk(N - 1)), dO, chunk_of(N - 1), a.H, tid);
    chain_issue<1>(ops, chunk_mats(a, blk(N - 1)), dO, chunk_of(N - 1), a.H, tid);
    chain_issue<2>(ops, chunk_mats(a, blk(N - 1)), dO, chunk_of(N - 1), a.H, tid);
    chain_commit(ops, L, sDO, tid);
    __syncthreads();
    store_adj(N - 1);
    stage_gds(L.gam);
    if (N > 1) chain_issue<0>(ops, chunk_mats(a, blk(N - 2)), dO, chunk_of(N - 2), a.H, tid);
    __syncthreads();
  }
  for (int n = N - 1; n >= 0; --n) {
    const bool more = n > 0;
    const Chunk cn = chunk_of(more ? n - 1 : 0);
    const bf16* Amn = chunk_mats(a, blk(more ? n - 1 : 0));
    if (more) chain_issue<1>(ops, Amn, dO, cn, a.H, tid);
    // dDelta = P^T dO + Kd (gamma . dS), stored transposed; wave w: the four
    // token tiles of value-column tile w, which share their column operands
    const int mT[4] = {0, 16, 32, 48};
    if constexpr (!ND) {
      floatx4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
      mm_zs<true, false, 4>(L.PT, P64, mT, sDO, P128, 16 * jt, C, acc, lane);
      mm_zs<true, true, 4>(L.Kd, P128, mT, sDSG, P128, 16 * jt, D, acc, lane);
#pragma unroll
      for (int x = 0; x < 4; ++x) st_tr(sDDT, P64, mT[x], 16 * jt, acc[x], lane);
    }
    __syncthreads();
    if (more) chain_issue<2>(ops, Amn, dO, cn, a.H, tid);
    // E = A'^T dDelta = Diag(beta) A^T dDelta, stored transposed
    if constexpr (!ND) {
      floatx4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
      mm_zs<false, true, 4>(L.A, P64, mT, sDDT, P64, 16 * jt, C, acc, lane);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const floatx4 bt = *reinterpret_cast<const floatx4*>(L.beta + mT[x] + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[x][r] *= bt[r];
        st_tr(sET, P64, mT[x], 16 * jt, acc[x], lane);
      }
    }
    // the next chunk's decay (its load was issued two phases ago)
    if (more && tid < D) gamN[tid] = ops.k.gb;
    __syncthreads();
    // dS <- gamma . dS + Qg^T dO - Kg^T E, in two groups of four channel tiles
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int mC[4] = {64 * hf, 64 * hf + 16, 64 * hf + 32, 64 * hf + 48};
      floatx4 p[4] = {zero4(), zero4(), zero4(), zero4()}, m[4] = {zero4(), zero4(), zero4(), zero4()};
      mm_zs<false, false, 4>(L.Qg, P128, mC, sDO, P128, 16 * jt, C, p, lane);
      if constexpr (!ND) mm_zs<false, true, 4>(L.Kg, P128, mC, sET, P64, 16 * jt, C, m, lane);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int u = 4 * hf + x;
        const floatx4 g4v = *reinterpret_cast<const floatx4*>(L.gam + 16 * u + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[u][r] = g4v[r] * dS[u][r] + p[x][r] - m[x][r];
      }
    }
    // the previous chunk's end adjoint: to memory and staged with its decay
    // ((gamma . dS)^T was last read by this chunk's dDelta)
    if (more) {
      store_adj(n - 1);
      stage_gds(gamN);
    }
    __syncthreads();
    if (more) {
      chain_commit(ops, L, sDO, tid);
      if (n > 1) chain_issue<0>(ops, chunk_mats(a, blk(n - 2)), dO, chunk_of(n - 2), a.H, tid);
      __syncthreads();
    }
  }
  if (a.dS0) {
    float* out = a.dS0 + (int64_t)bh * D * D;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(16 * u + 4 * g4 + r) * D + 16 * jt + i] = dS[u][r];
  }
}

// ---------------------------------------------------------------- gradients
namespace gr {
constexpr int O_KG = 0;
constexpr int O_KD = O_KG + C * P128 * 2;
constexpr int O_QG = O_KD + C * P128 * 2;
constexpr int O_A = O_QG + C * P128 * 2;
constexpr int O_PT = O_A + C * P64 * 2;
constexpr int O_BETA = O_PT + C * P64 * 2;
constexpr int O_GAM = O_BETA + C * 4;
constexpr int O_QK = O_GAM + D * 4;
constexpr int O_DGAM = O_QK + C * 4;          // gamma . rowsum(dS . S), [128]
constexpr int O_MD = O_DGAM + D * 4;          // diagonal of M, [64]
constexpr int O_DB = O_MD + C * 4;            // dbeta partial sums [8 waves][64]
constexpr int O_WORK = O_DB + 8 * C * 4;      // phase-dependent area
// half-loop layout inside the work area
constexpr int H_S = 0;                         // S[:, J] as [j][c]        [64][P128] bf16
constexpr int H_DSG = H_S + C * P128 * 2;      // (gamma . dS)[:, J], [j][c] [64][P128]
constexpr int H_V = H_DSG + C * P128 * 2;      // V[:, J]        [64][P64]
constexpr int H_DO = H_V + C * P64 * 2;        // dO[:, J]
constexpr int H_D = H_DO + C * P64 * 2;        // Delta[:, J]
constexpr int H_DD = H_D + C * P64 * 2;        // dDelta[:, J]
constexpr int H_XT = H_DD + C * P64 * 2;       // X = beta . (V - Kg S) [64 t][P64]; then dV[:, J]
constexpr int H_END = H_XT + C * P64 * 2;
// after the halves
constexpr int Q_DW = 0;                        // dW row-major [64][P128]
constexpr int Q_M = Q_DW + C * P128 * 2;       // M (zero diagonal) [64][P64]
constexpr int Q_DA = Q_M + C * P64 * 2;        // dA (strictly lower) [64][P64]
constexpr int Q_Z1T = Q_DA + C * P64 * 2;      // (dA A^T)^T [64][P64]
constexpr int Q_DL = Q_Z1T + C * P64 * 2;      // dL [64][P64]
constexpr int Q_DG = Q_DL + C * P64 * 2;       // Diag(beta) dL [64][P64]
constexpr int Q_END = Q_DG + C * P64 * 2;
constexpr int Z_DB = 0;                        // db fp32 [64][PB] + scan scratch (assembly)
constexpr int Z_Q = (C * PB + 4 * D) * 4;      // q, then dq, bf16 [64][P128]
constexpr int Z_K = Z_Q + C * P128 * 2;        // k, then dk
constexpr int Z_END = Z_K + C * P128 * 2;
constexpr int BYTES = O_WORK + (H_END > Q_END ? H_END : Q_END);
static_assert((C * PB + 4 * D) * 4 <= H_END, "gate scratch inside the work area");
static_assert(Q_END <= H_END, "after-halves buffers inside the work area");
static_assert(Z_END <= H_END, "assembly buffers inside the work area");
static_assert(BYTES <= 160 * 1024, "LDS");
static_assert(O_KD == O_KG + C * P128 * 2 && O_QG == O_KD + C * P128 * 2 && O_PT == O_A + C * P64 * 2,
              "load_chunk layout");
}  // namespace gr

// One workgroup per (chunk, sequence, head).  [t][c] results: wave w owns
// channels 16w .. 16w+15 (4 tiles of each); [t][j] results of a half and the
// lower [t][t'] tiles are spread over the waves.
// V: variant flags (kVarNoDelta: Delta = V, A = I, no W / L terms, no dbeta).
template <int V>
__global__ __launch_bounds__(NT) void bwd_grad_kernel(BackwardArgs a) {
  constexpr bool ND = (V & kVarNoDelta) != 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // persistent: the workgroup takes blocks blockIdx.x, + gridDim.x, ... (the
  // unused slots of packed sequences skipped) and loads the operands of its
  // next chunk during the current chunk's assembly
  const int nblk = a.cu_seqlens ? a.nslots * a.H : a.B * a.H * ((a.T + C - 1) / C);
  int b, h, n;
  int vb = blockIdx.x;
  while (vb < nblk && !chunk_of_block(a, vb, b, h, n)) vb += gridDim.x;
  if (vb >= nblk) return;
  const Basics L = basics(sm, gr::O_KG, gr::O_KD, gr::O_QG, gr::O_A, gr::O_PT, gr::O_BETA, gr::O_GAM, gr::O_QK);
  float* dgam = reinterpret_cast<float*>(sm + gr::O_DGAM);
  float* md = reinterpret_cast<float*>(sm + gr::O_MD);
  float* dbp = reinterpret_cast<float*>(sm + gr::O_DB);
  unsigned char* work = sm + gr::O_WORK;
  const bf16* q = reinterpret_cast<const bf16*>(a.q);
  const bf16* k = reinterpret_cast<const bf16*>(a.k);
  const bf16* g = reinterpret_cast<const bf16*>(a.g);
  const bf16* v = reinterpret_cast<const bf16*>(a.v);
  const bf16* dO = reinterpret_cast<const bf16*>(a.dO);
  // block index and rows of a chunk
  auto locate = [&](int b_, int h_, int n_, int64_t& bi_, Chunk& c_) {
    const SeqView sv = seq_view(a, b_, h_);
    bi_ = sv.idx0 + (int64_t)n_ * sv.istride;
    c_.row0 = sv.row0 + (int64_t)n_ * C * a.H;
    c_.nv = min(C, sv.len - n_ * C);
    c_.rstride = a.H * D;
  };
  int64_t bi;
  Chunk c;
  locate(b, h, n, bi, c);
  const int c0 = 16 * wave;     // my channel block
  auto lower_tile = [](int tq, int& I, int& J) {
    int cc = 0;
    I = J = 0;
    for (int x = 0; x < 4; ++x)
      for (int y = 0; y <= x; ++y) {
        if (cc == tq) { I = x; J = y; }
        ++cc;
      }
  };

  // lower [t][t'] tiles: tile index q = wave, wave + 8 (< 10)
  bf16* hS = reinterpret_cast<bf16*>(work + gr::H_S);
  bf16* hDSG = reinterpret_cast<bf16*>(work + gr::H_DSG);
  bf16* hV = reinterpret_cast<bf16*>(work + gr::H_V);
  bf16* hDO = reinterpret_cast<bf16*>(work + gr::H_DO);
  bf16* hD = ND ? hV : reinterpret_cast<bf16*>(work + gr::H_D);   // Delta (= V without the delta rule)
  bf16* hDD = reinterpret_cast<bf16*>(work + gr::H_DD);
  bf16* hXT = reinterpret_cast<bf16*>(work + gr::H_XT);

  // Staging of a value half: S[:, J] and gamma . dS[:, J] as [j][c] rows,
  // V[:, J] and dO[:, J] (rows past nv zero).  The half's S (blocks
  // 32 jh .. 32 jh + 31 of the owners' fragment order) and dS (tiles 32 jh ..
  // of 16 x 16) are each 16 KB contiguous: piece p = tid, tid + 512 is the
  // 16 bytes at 8 p of it, channels 8 (p % 2) .. + 8 of row p / 2 % 16 of
  // block p / 32.  The loads of half 0 are issued with the chunk's operand
  // block, those of half 1 during half 0's products.
  Vec16 xs[2], xd[2], xv, xo;
  auto half_issue = [&](int64_t bi_, const Chunk& c_, int jh, int tid) {
    const int tv = tid >> 3, xv0 = 8 * (tid & 7);   // V, dO: one piece per thread
    const bf16* Sn = reinterpret_cast<const bf16*>(a.states) + bi_ * D * D;      // fragment order
    const bf16* dSn = reinterpret_cast<const bf16*>(a.adjoints) + bi_ * D * D;   // 16 x 16 tiles
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pc = tid + u * NT;
      xs[u] = ldg16(Sn + 32 * 256 * jh + 8 * pc);
      xd[u] = ldg16(dSn + 32 * 256 * jh + 8 * pc);
    }
    // (every thread loads a row in range, rows past nv are zeroed when
    // stored: a load under a branch made the compiler wait for it at the join)
    const int tr = min(tv, c_.nv - 1);
    xv = ldg16(v + (c_.row0 + (int64_t)tr * a.H) * D + 64 * jh + xv0);
    xo = ldg16(dO + (c_.row0 + (int64_t)tr * a.H) * D + 64 * jh + xv0);
  };
  ChunkOps ops;
  ops_issue(ops, chunk_mats(a, bi), tid);
  half_issue(bi, c, 0, tid);

  for (;;) {
  // (the lane index is made opaque here so that the per-lane addresses are
  // formed inside the loop: hoisted out of it, they held enough registers
  // across the whole loop to force spills)
  int tid_o = threadIdx.x;
  asm volatile("" : "+v"(tid_o));
  const int tid = tid_o, lane = tid & 63, g4 = lane >> 4, i = lane & 15;
  const int tv = tid >> 3, xv0 = 8 * (tid & 7);   // V, dO: one piece per thread
  // per-chunk accumulators
  floatx4 aQg[4], aKd[4], aKb[4], aW[4], aKg[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) aQg[u] = aKd[u] = aKb[u] = aW[u] = aKg[u] = zero4();
  floatx4 aM[2] = {zero4(), zero4()}, aA[2] = {zero4(), zero4()};
  // gamma . rowsum(S . dS), the chunk-end term of each channel: the diagonal
  // of S (gamma . dS)^T, wave w forming its diagonal tile (channels 16w..)
  floatx4 aSD = zero4();
  // dbeta terms rowsum((A^T dDelta) . V) of the lane's rows mT[x] + 4 g4 + r,
  // summed per lane over both halves (the 16-lane sums follow the loop)
  floatx4 dvp[2] = {zero4(), zero4()};
  ops_commit(ops, L, tid);
  for (int e = tid; e < 8 * C; e += NT) dbp[e] = 0.f;
  if (tid < D) dgam[tid] = 0.f;
  __syncthreads();

#pragma unroll
  for (int jh = 0; jh < 2; ++jh) {
    const int J0 = 64 * jh;
    if (jh > 0) __syncthreads();
    {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pc = tid + u * NT, blk = pc >> 5, row = (pc >> 1) & 15, ch = 8 * (pc & 1);
        // S: block 32 jh + blk = 8 (2 o + nt) + rt, row = lane i of tile nt
        const int bs_ = 32 * jh + blk, ot = bs_ >> 3, rt = bs_ & 7;
        const int js = 32 * (ot >> 1) + 8 * (row >> 2) + 4 * (ot & 1) + (row & 3) - J0;
        *reinterpret_cast<Vec16*>(hS + js * P128 + 16 * rt + ch) = xs[u];
        // dS: tile 32 jh + blk = 8 (j / 16) + c / 16, row = j % 16
        const int bd = 32 * jh + blk, jd = 16 * (bd >> 3) + row - J0, cd = 16 * (bd & 7) + ch;
        float fd[8];
        vec_to_f32<bf16>(xd[u], fd);
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)(L.gam[cd + e] * fd[e]);
        *reinterpret_cast<bf16x8*>(hDSG + jd * P128 + cd) = y;
      }
      *reinterpret_cast<Vec16*>(hV + tv * P64 + xv0) = keep_or_zero(xv, tv < c.nv);
      *reinterpret_cast<Vec16*>(hDO + tv * P64 + xv0) = keep_or_zero(xo, tv < c.nv);
    }
    __syncthreads();
    // X = beta . (V - Kg S), stored transposed
    // (tiles (tt, jj) and (tt + 2, jj) per wave: tiles wave and wave + 8 of 16)
    const int jj = wave & 3, tA = wave >> 2;
    const int mT[2] = {16 * tA, 16 * (tA + 2)};
    if constexpr (!ND) {
      // (lane: token mT + i, value columns 16 jj + 4 g4 ..)
      floatx4 ks[2] = {zero4(), zero4()};
      mm_zs<true, true, 2, true>(L.Kg, P128, mT, hS, P128, 16 * jj, D, ks, lane);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int t = mT[x] + i;
        const bf16x4 vv = *reinterpret_cast<const bf16x4*>(hV + t * P64 + 16 * jj + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) ks[x][r] = L.beta[t] * ((float)vv[r] - ks[x][r]);
        st_rm8(hXT, P64, mT[x], 16 * jj, ks[x], lane);
      }
      __syncthreads();
    }
    // Delta = A X; dDelta = P^T dO + Kd (gamma . dS); both row-major
    {
      floatx4 dl[2] = {zero4(), zero4()}, dd[2] = {zero4(), zero4()};
      if constexpr (!ND) mm_zs<true, false, 2, true>(L.A, P64, mT, hXT, P64, 16 * jj, C, dl, lane);
      mm_zs<true, false, 2, true>(L.PT, P64, mT, hDO, P64, 16 * jj, C, dd, lane);
      mm_zs<true, true, 2, true>(L.Kd, P128, mT, hDSG, P128, 16 * jj, D, dd, lane);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if constexpr (!ND) st_rm8(hD, P64, mT[x], 16 * jj, dl[x], lane);
        st_rm8(hDD, P64, mT[x], 16 * jj, dd[x], lane);
      }
    }
    __syncthreads();
    // [t][c] products over this half's value columns
    if (jh == 0) half_issue(bi, c, 1, tid);
    // (dO S^T, Delta (g.dS)^T, dDelta S^T: the S and g.dS fragments of a step
    // serve all four row tiles; the diagonal tile of S (g.dS)^T alongside)
    for (int k = 0; k < 64; k += 32) {
      const bf16x8 fs = fr_tr8(hS, P128, c0, k + 8 * g4, lane), fd = fr_tr8(hDSG, P128, c0, k + 8 * g4, lane);
      aSD = MB::mma32(fs, fd, aSD);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        aQg[u] = MB::mma32(fr_row8(hDO, P64, 16 * u + i, k + 8 * g4), fs, aQg[u]);
        aKb[u] = MB::mma32(fr_row8(hD, P64, 16 * u + i, k + 8 * g4), fd, aKb[u]);
        if constexpr (!ND) aW[u] = MB::mma32(fr_row8(hDD, P64, 16 * u + i, k + 8 * g4), fs, aW[u]);
      }
    }
    // lower [t][t'] tiles: M += dO Delta^T, dA1 += dDelta V^T
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int tq = wave + 8 * x;
      if (tq < 10) {
        int I, J;
        lower_tile(tq, I, J);
        // (transposed tiles: lane holds row 16 I + i, columns 16 J + 4 g4 ..)
        aM[x] = mm<true, true, true>(hDO, P64, hD, P64, 16 * I, 16 * J, 64, aM[x], lane);
        if constexpr (!ND) aA[x] = mm<true, true, true>(hDD, P64, hV, P64, 16 * I, 16 * J, 64, aA[x], lane);
      }
    }
    // dV[:, J] = Diag(beta) A^T dDelta, staged row-major where X^T was (dead
    // since Delta); dbeta += rowsum((A^T dDelta) . V).  The lane's V and beta
    // of rows mT[x] + 4 g4 .. + 3 are one transpose read and one 16-byte read.
    if constexpr (!ND) {
      floatx4 xv[2] = {zero4(), zero4()};
      mm_zs<false, false, 2>(L.A, P64, mT, hDD, P64, 16 * jj, C, xv, lane);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const bf16x4 vv = fr_tr(hV, P64, 16 * jj, mT[x] + 4 * g4, lane);
        const floatx4 bt = *reinterpret_cast<const floatx4*>(L.beta + mT[x] + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dvp[x][r] += xv[x][r] * (float)vv[r];
          xv[x][r] *= bt[r];
        }
        st_rm(hXT, P64, mT[x], 16 * jj, xv[x], lane);
      }
    }
    __syncthreads();
    {
      const int t = tid >> 3, x0 = 8 * (tid & 7);
      if (t < c.nv)
        *reinterpret_cast<Vec16*>(reinterpret_cast<bf16*>(a.dv) + (c.row0 + (int64_t)t * a.H) * D + J0 + x0) =
            *reinterpret_cast<const Vec16*>((ND ? hDD : hXT) + t * P64 + x0);   // dV (= dDelta without the delta rule)
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * g4 + r == i) dgam[c0 + i] = aSD[r];
  if constexpr (!ND) {
    // (rows mT[x] + 4 g4 .. + 3 of this wave's partial-sum row; its other rows
    // are still zero, and the later terms are added by this wave alone)
    const int mT0[2] = {16 * (wave >> 2), 16 * ((wave >> 2) + 2)};
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      floatx4 sv;
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = sum16(dvp[x][r]);
      if (i == 0) *reinterpret_cast<floatx4*>(dbp + wave * C + mT0[x] + 4 * g4) = sv;
    }
  }
  // the assembly's inputs g, q, k (rows past nv zero), in flight during the
  // 64 x 64 products
  // (rows in range for every thread, zeroed past nv when stored)
  Vec16 xg[2], xq[2], xk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * NT, t = min(e >> 4, c.nv - 1), x0 = 8 * (e & 15);
    const int64_t off = (c.row0 + (int64_t)t * a.H) * D + x0;
    xg[u] = ldg16(g + off);
    xq[u] = ldg16(q + off);
    xk[u] = ldg16(k + off);
  }
  // fold dKb~ into dKd, keeping its column sums against Kd (chunk-end terms)
  float colsum = 0.f;   // sum over my rows of Kd . dKb~ for column c0 + i
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bf16x4 kd4 = fr_tr(L.Kd, P128, c0, 16 * u + 4 * g4, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      colsum += (float)kd4[r] * aKb[u][r];
      aKd[u][r] += aKb[u][r];
    }
  }
  __syncthreads();   // the half-loop buffers are dead from here

  bf16* qDW = reinterpret_cast<bf16*>(work + gr::Q_DW);
  bf16* qM = reinterpret_cast<bf16*>(work + gr::Q_M);
  bf16* qDA = reinterpret_cast<bf16*>(work + gr::Q_DA);
  bf16* qZ1T = reinterpret_cast<bf16*>(work + gr::Q_Z1T);
  bf16* qDL = reinterpret_cast<bf16*>(work + gr::Q_DL);
  bf16* qDG = reinterpret_cast<bf16*>(work + gr::Q_DG);
  // dW = -dDelta S^T (row-major); M with its diagonal moved out; zero fills
  // of the four 64 x 64 arrays whose upper blocks are never written
  {
    const Vec16 z = {{0u, 0u, 0u, 0u}};
    for (int e = tid; e < C * P64 / 8; e += NT) {
      *reinterpret_cast<Vec16*>(qM + 8 * e) = z;
      if constexpr (!ND) {
        *reinterpret_cast<Vec16*>(qDA + 8 * e) = z;
        *reinterpret_cast<Vec16*>(qDL + 8 * e) = z;
        *reinterpret_cast<Vec16*>(qDG + 8 * e) = z;
      }
    }
  }
  if constexpr (!ND) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      floatx4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = -aW[u][r];
      aW[u] = w;
      st_rm(qDW, P128, 16 * u, c0, w, lane);
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int tq = wave + 8 * x;
    if (tq < 10) {
      int I, J;
      lower_tile(tq, I, J);
      floatx4 m = aM[x];
      const int t = 16 * I + i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * J + 4 * g4 + r;
        if (t == s) md[t] = m[r];
        m[r] = t > s ? m[r] : 0.f;
      }
      st_rm8(qM, P64, 16 * I, 16 * J, m, lane);
      if constexpr (!ND) {
        // dA = (dDelta V^T + dW Kg^T) Diag(beta), strictly lower
        floatx4 da = mm<true, true, true>(qDW, P128, L.Kg, P128, 16 * I, 16 * J, D, aA[x], lane);
        const floatx4 bs4 = *reinterpret_cast<const floatx4*>(L.beta + 16 * J + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) da[r] = t > 16 * J + 4 * g4 + r ? da[r] * bs4[r] : 0.f;
        st_rm8(qDA, P64, 16 * I, 16 * J, da, lane);
      }
    }
  }
  __syncthreads();
  // Z1^T = A dA^T ( = (dA A^T)^T ), all 16 tiles
  // (tiles (I, J) and (I + 2, J) per wave: tiles wave and wave + 8 of 16)
  const int mT[2] = {16 * (wave >> 2), 16 * ((wave >> 2) + 2)};
  if constexpr (!ND) {
    floatx4 z[2] = {zero4(), zero4()};
    mm_zs<true, true, 2, true>(L.A, P64, mT, qDA, P64, 16 * (wave & 3), C, z, lane);
#pragma unroll
    for (int x = 0; x < 2; ++x) st_rm8(qZ1T, P64, mT[x], 16 * (wave & 3), z[x], lane);
  }
  // [t][c]: M Kd, M^T Qg, A^T dW
  const int mU[4] = {0, 16, 32, 48};
  mm_zs<true, false, 4>(qM, P64, mU, L.Kd, P128, c0, C, aQg, lane);
  mm_zs<false, false, 4>(qM, P64, mU, L.Qg, P128, c0, C, aKd, lane);
  if constexpr (!ND) {
    // Y = A^T dW with dW from registers (B operand of the 16-index slabs)
    bf16x4 wf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) wf[u] = MB::frag16(aW[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      floatx4 y = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) y = MB::mma16(fr_tr(L.A, P64, 16 * u, 16 * ks + 4 * g4, lane), wf[ks], y);
      // aKg holds Y + dL Kd until both are in (then Diag(beta) and the
      // dbeta term rowsum((Y + dL Kd) . Kg) follow)
#pragma unroll
      for (int r = 0; r < 4; ++r) aKg[u][r] += y[r];
    }
  }
  if constexpr (!ND) {
  __syncthreads();
  // dL = -StrictTril(A^T Z1); dG = Diag(beta) dL (upper blocks zeroed above)
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int tq = wave + 8 * x;
    if (tq < 10) {
      int I, J;
      lower_tile(tq, I, J);
      // (transposed tile: lane holds row t = 16 I + i, columns 16 J + 4 g4 ..)
      floatx4 l = mm<false, true, true>(L.A, P64, qZ1T, P64, 16 * I, 16 * J, C, zero4(), lane);
      floatx4 gg;
      const int t = 16 * I + i;
      const float bt = L.beta[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l[r] = t > 16 * J + 4 * g4 + r ? -l[r] : 0.f;
        gg[r] = l[r] * bt;
      }
      st_rm8(qDL, P64, 16 * I, 16 * J, l, lane);
      st_rm8(qDG, P64, 16 * I, 16 * J, gg, lane);
    }
  }
  __syncthreads();
  // dKg = Diag(beta) (Y + dL Kd), dbeta += rowsum(Kg . (Y + dL Kd)); dKd += dG^T Kg
  // (the lane's Kg and beta of rows 16 u + 4 g4 .. + 3: one transpose read and
  // one 16-byte read; its four partial sums go to LDS in one store)
  mm_zs<true, false, 4>(qDL, P64, mU, L.Kd, P128, c0, C, aKg, lane);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bf16x4 kg4 = fr_tr(L.Kg, P128, c0, 16 * u + 4 * g4, lane);
    const floatx4 bt = *reinterpret_cast<const floatx4*>(L.beta + 16 * u + 4 * g4);
    floatx4 sv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = sum16(aKg[u][r] * (float)kg4[r]);
      aKg[u][r] *= bt[r];
    }
    if (i == 0) *reinterpret_cast<floatx4*>(dbp + wave * C + 16 * u + 4 * g4) += sv;
  }
  mm_zs<false, false, 4>(qDG, P64, mU, L.Kg, P128, c0, C, aKd, lane);
  }
  __syncthreads();   // the work area becomes the db array

  // assembly: gate factors from b (recomputed), raw q and k staged in LDS;
  // dq and dk replace q and k there (each element read, then written, by the
  // same lane) and leave with row-wide stores
  float* bs = reinterpret_cast<float*>(work + gr::Z_DB);
  bf16* zq = reinterpret_cast<bf16*>(work + gr::Z_Q);
  bf16* zk = reinterpret_cast<bf16*>(work + gr::Z_K);
  {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * NT, t = e >> 4, x0 = 8 * (e & 15);
      const bool in = t < c.nv;
      float f[8];
      vec_to_f32<bf16>(keep_or_zero(xg[u], in), f);
#pragma unroll
      for (int uu = 0; uu < 8; ++uu) bs[t * PB + x0 + uu] = f[uu];
      *reinterpret_cast<Vec16*>(zq + t * P128 + x0) = keep_or_zero(xq[u], in);
      *reinterpret_cast<Vec16*>(zk + t * P128 + x0) = keep_or_zero(xk[u], in);
    }
  }
  // the next chunk's operand block and first value half, in flight during
  // the assembly (the last chunk loads its own again: the loads are never
  // under a branch)
  int nvb = vb + gridDim.x, nb = b, nh = h, nn = n;
  while (nvb < nblk && !chunk_of_block(a, nvb, nb, nh, nn)) nvb += gridDim.x;
  int64_t nbi = bi;
  Chunk nc = c;
  if (nvb < nblk) locate(nb, nh, nn, nbi, nc);
  ops_issue(ops, chunk_mats(a, nbi), tid);
  half_issue(nbi, nc, 0, tid);
  __syncthreads();
  scan_cols<false>(bs, nullptr, tid);
  // per element: dq, dk and db (db overwrites b in place).  The lane's four
  // q and k of rows 16u + 4 g4 .. + 3, column c0 + i, are one transpose read
  // each (the whole wavefront reads a row block before writing into it; other
  // wavefronts own other columns).
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bf16x4 q4 = fr_tr(zq, P128, c0, 16 * u + 4 * g4, lane);
    const bf16x4 k4 = fr_tr(zk, P128, c0, 16 * u + 4 * g4, lane);
    const floatx4 md4 = *reinterpret_cast<const floatx4*>(md + 16 * u + 4 * g4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * u + 4 * g4 + r, cc = c0 + i;
      const float bb = bs[t * PB + cc];
      const float ep = __expf(bb), em = __expf(-bb);
      const float qv = (float)q4[r], kv = (float)k4[r];
      const float kg = kv * ep, kd = kv * em, qg = qv * ep;
      const float dkd = aKd[u][r];
      zq[t * P128 + cc] = (bf16)(ep * aQg[u][r] + md4[r] * kv);
      zk[t * P128 + cc] = (bf16)(ep * aKg[u][r] + em * dkd + md4[r] * qv);
      bs[t * PB + cc] = kg * aKg[u][r] - kd * dkd + qg * aQg[u][r];
    }
  }
  // chunk-end terms at row 63: sum over t of Kd . dKb~ (across the 4 row
  // groups) + gamma . rowsum(dS . S)
  colsum += __shfl_xor(colsum, 16);
  colsum += __shfl_xor(colsum, 32);
  if (g4 == 0) bs[(C - 1) * PB + c0 + i] += colsum + dgam[c0 + i];
  __syncthreads();
  // dg = reverse cumulative sum of db over the chunk's rows
  scan_cols<true>(bs, nullptr, tid);
  bf16* dq = reinterpret_cast<bf16*>(a.dq);
  bf16* dk = reinterpret_cast<bf16*>(a.dk);
  bf16* dgo = reinterpret_cast<bf16*>(a.dg);
  for (int e = tid; e < C * 16; e += NT) {
    const int t = e >> 4, x0 = 8 * (e & 15);
    if (t < c.nv) {
      const int64_t off = (c.row0 + (int64_t)t * a.H) * D + x0;
      *reinterpret_cast<Vec16*>(dq + off) = *reinterpret_cast<const Vec16*>(zq + t * P128 + x0);
      *reinterpret_cast<Vec16*>(dk + off) = *reinterpret_cast<const Vec16*>(zk + t * P128 + x0);
      if (a.dg32) {
        // fp32 per-channel dg (the scalar-gate path sums it over the channels)
        *reinterpret_cast<floatx4*>(a.dg32 + off) = *reinterpret_cast<const floatx4*>(bs + t * PB + x0);
        *reinterpret_cast<floatx4*>(a.dg32 + off + 4) = *reinterpret_cast<const floatx4*>(bs + t * PB + x0 + 4);
      } else {
        bf16x8 y;
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) y[uu] = (bf16)bs[t * PB + x0 + uu];
        *reinterpret_cast<bf16x8*>(dgo + off) = y;
      }
    }
  }
  if (!ND && tid < C && tid < c.nv) {
    float s = 0.f;
    for (int w = 0; w < NT / 64; ++w) s += dbp[w * C + tid];
    reinterpret_cast<bf16*>(a.dbeta)[c.row0 + (int64_t)tid * a.H] = (bf16)s;
  }
  if (nvb >= nblk) break;
  vb = nvb;
  b = nb;
  h = nh;
  n = nn;
  bi = nbi;
  c = nc;
  __syncthreads();   // this chunk's last LDS reads are done before the next commit
  }
}

// ---------------------------------------------------------------- scalar gate
// A scalar gate g [rows] (one per token and head) is the per-channel gate with
// every channel equal, so its gradient is the channel sum of the per-channel
// gradient of the broadcast gate.  gate_expand: gfull[r][c] = g[r] (bf16,
// 16-byte stores); gate_reduce: dg[r] = sum_c dg32[r][c] (fp32 sums, one
// 16-lane row per token and head).
__global__ __launch_bounds__(256) void gate_expand_kernel(const bf16* g, bf16* gfull, int64_t rows) {
  const int64_t pieces = rows * (D / 8);
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * 256) {
    const bf16 x = g[p / (D / 8)];
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x;
    *reinterpret_cast<bf16x8*>(gfull + 8 * p) = y;
  }
}

__global__ __launch_bounds__(256) void gate_reduce_kernel(const float* dg32, bf16* dg, int64_t rows) {
  const int lane16 = threadIdx.x & 15;
  for (int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; r < rows; r += (int64_t)gridDim.x * 16) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(dg32 + r * D + 8 * lane16);
    const floatx4 b = *reinterpret_cast<const floatx4*>(dg32 + r * D + 8 * lane16 + 4);
    const float x = sum16(a[0] + a[1] + a[2] + a[3] + b[0] + b[1] + b[2] + b[3]);
    if (lane16 == 0) dg[r] = (bf16)x;
  }
}

}  // namespace bwd

hipError_t launch_gate_expand(const void* g, void* gfull, int64_t rows, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * (bwd::D / 8) + 255) / 256;
  hipLaunchKernelGGL(bwd::gate_expand_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                     reinterpret_cast<const bf16*>(g), reinterpret_cast<bf16*>(gfull), rows);
  return hipGetLastError();
}

hipError_t launch_gate_reduce(const float* dg32, void* dg, int64_t rows, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * 16 + 255) / 256;
  hipLaunchKernelGGL(bwd::gate_reduce_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                     dg32, reinterpret_cast<bf16*>(dg), rows);
  return hipGetLastError();
}

size_t backward_workspace(int BH, int T) {
  const size_t N = ((size_t)T + bwd::C - 1) / bwd::C;
  return (size_t)BH * N * (2 * bwd::D * bwd::D + bwd::MATS) * sizeof(bf16);
}

int backward_varlen_slots(int nseq, int T) { return T / bwd::C + nseq; }

size_t backward_varlen_workspace(int nseq, int T, int H) {
  return (size_t)backward_varlen_slots(nseq, T) * H * (2 * bwd::D * bwd::D + bwd::MATS) * sizeof(bf16);
}

template <typename K>
static hipError_t set_lds(K kern, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const int N = (a.T + bwd::C - 1) / bwd::C;
  // per-chunk workgroups: chunks x sequences x heads, or (packed sequences)
  // slots x heads with the unused slots returning at once
  const int nblk = a.cu_seqlens ? a.nslots * a.H : BH * N;
  hipError_t e;
  if (N > 0 && !a.states_saved) {
    // 1. chunk-entry states: the forward kernel in state mode (skipped when
    // the forward saved them)
    PrefillArgs f{};
    f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta;
    f.S0 = a.S0; f.B = a.B; f.T = a.T; f.H = a.H; f.dk = 128; f.dv = 128; f.bf16 = 1; f.pipeline = 1;
    f.states = a.states;
    f.variant = a.variant;
    f.cu_seqlens = a.cu_seqlens;
    if ((e = launch_fused(f, s)) != hipSuccess) return e;
  }
  // 2. per-chunk A and P^T
  if (N > 0) {
    auto prep = a.variant ? bwd::bwd_prep_kernel<kVarNoDelta> : bwd::bwd_prep_kernel<0>;
    if ((e = set_lds(prep, bwd::pr::BYTES)) != hipSuccess) return e;
    hipLaunchKernelGGL(prep, dim3(nblk), dim3(bwd::NT), bwd::pr::BYTES, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. adjoint recursion (also writes dS0; with T = 0 it copies dS_T)
  auto chain = a.variant ? bwd::bwd_chain_kernel<kVarNoDelta> : bwd::bwd_chain_kernel<0>;
  if ((e = set_lds(chain, bwd::ch::BYTES)) != hipSuccess) return e;
  hipLaunchKernelGGL(chain, dim3(BH), dim3(bwd::NT), bwd::ch::BYTES, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (N == 0) return hipSuccess;
  // 4. per-chunk gradients
  // (persistent: one workgroup per compute unit, which its LDS allows anyway)
  auto grad = a.variant ? bwd::bwd_grad_kernel<kVarNoDelta> : bwd::bwd_grad_kernel<0>;
  if ((e = set_lds(grad, bwd::gr::BYTES)) != hipSuccess) return e;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    cus = nblk;
  hipLaunchKernelGGL(grad, dim3(nblk < cus ? nblk : cus), dim3(bwd::NT), bwd::gr::BYTES, s, a);
  return hipGetLastError();
}

}  // namespace kda
