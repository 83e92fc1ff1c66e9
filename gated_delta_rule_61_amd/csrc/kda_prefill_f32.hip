// kda_prefill_f32.hip -- chunked KDA forward with every matrix operand in
// fp32, on gfx950: fp32 inputs at d_k = d_v = 128, and bf16 inputs at
// d_k = d_v = 64 (where fp32 operands keep short sequences inside the bf16
// tolerance; the one-launch kernel's bf16 operands do not).
//
// The one-launch prefill keeps a chunk's gated key and query tiles in LDS; in
// fp32 at d = 128 those tiles need more than a CU's 160 KB.  This path cuts
// the chunked form ("Hybrid Linear Attention Architecture: Making LLM
// Training and Inference More Efficient" §IV; "Linear Attention Architecture
// Deep Dive: From State Updates to Efficient Chunked Computation" §5) where
// the state enters:
//   f32_prep_kernel   one workgroup per (sequence x head, chunk), every chunk
//                     at once: all quantities of the chunk that do not
//                     involve the state, into a workspace block;
//   f32_state_kernel  one workgroup per (sequence x head, 32 value columns):
//                     the chunks in order, with its d x 32 slice of the
//                     state in LDS.
// With b the in-chunk prefix sums of g log2(e) per key channel (tokens past
// the end of the sequence count as g = 0), b_C their value at the chunk's
// end and r their value at its 32nd token:
//   Kt = 2^(b-r) K,  Kh = 2^(r-b) K,  Qt = 2^(b-r) Q   (Kt Kh^T = Kg Kd^T)
//   L  = StrictTril(Diag(beta) Kt Kh^T),  A = (I + L)^-1  (forward substitution)
//   W  = A Diag(beta) Kg,  U = A Diag(beta) V,  P = Tril(Qt Kh^T)
//   Qg = 2^b Q,  Kb = 2^(b_C-b) K,  gamma = 2^(b_C)
// then, chunk after chunk,
//   Delta = U - W S,  O = Qg S + P Delta,  S <- Diag(gamma) S + Kb^T Delta.
// The reference r halves the exponent range of the operands that carry
// inverse decays (Kh), so that a chunk decaying by up to e^-80 per channel
// stays inside fp32.  Every product is fp32 MFMA (v_mfma_f32_16x16x4_f32)
// with fp32 accumulation; inputs are converted to fp32 as they are read and
// the output rounded to the input type as it is stored.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace f32c {

constexpr int C = 64;          // chunk length
constexpr int NT = 256;        // threads per workgroup (4 wavefronts)
constexpr int LDC = C + 4;     // LDS rows of [C][C] tiles
constexpr int DVW = 32;        // value columns per state workgroup
constexpr int LDS_S = DVW + 4; // LDS rows of the [D][DVW] state slice and [C][DVW] values
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int LD = D + 4;          // LDS rows of [C][D] tiles (fp32)
  static constexpr int NPART = NT / D;      // token parts of the prefix sums (2 or 4)
  static constexpr int TPP = C / NPART;     // tokens per part
  static constexpr int NSPLIT = D / DVW;    // state workgroups per head
  // Workspace block of one (sequence x head, chunk), fp32, offsets in floats.
  static constexpr int64_t WS_QG = 0;                    // Qg [C][D]
  static constexpr int64_t WS_W = WS_QG + C * D;         // W  [C][D]
  static constexpr int64_t WS_KB = WS_W + C * D;         // Kb [C][D]
  static constexpr int64_t WS_U = WS_KB + C * D;         // U  [C][D]
  static constexpr int64_t WS_P = WS_U + C * D;          // P  [C][C] (zero above the diagonal)
  static constexpr int64_t WS_GM = WS_P + C * C;         // gamma [D]
  static constexpr int64_t WS_BLOCK = WS_GM + D;
  static_assert(WS_BLOCK % 4 == 0, "16-byte blocks");
  // LDS of the prep kernel (bytes): Kt, Kh, Qt tiles (Kh later holds Kg and
  // Qt the values V), L (then A in place), beta, and each part's per-channel
  // total of the prefix sums.
  static constexpr int SZ_T = C * LD * 4;
  static constexpr int P_KT = 0, P_KH = SZ_T, P_QT = 2 * SZ_T, P_L = 3 * SZ_T;
  static constexpr int P_BETA = P_L + C * LDC * 4;
  static constexpr int P_TOT = P_BETA + C * 4;
  static constexpr int PREP_BYTES = P_TOT + NPART * D * 4;
  // LDS of the state kernel: the state slice, W, Qg, Kb, P, the value slice
  // (U, then Delta in place) and gamma.
  static constexpr int S_S = 0;
  static constexpr int S_W = S_S + D * LDS_S * 4;
  static constexpr int S_QG = S_W + SZ_T;
  static constexpr int S_KB = S_QG + SZ_T;
  static constexpr int S_P = S_KB + SZ_T;
  static constexpr int S_U = S_P + C * LDC * 4;
  static constexpr int S_GM = S_U + C * LDS_S * 4;
  static constexpr int STATE_BYTES = S_GM + D * 4;
  static_assert(PREP_BYTES <= 160 * 1024 && STATE_BYTES <= 160 * 1024, "LDS");
  static_assert(NPART * D == NT && NPART * TPP == C && 32 % TPP == 0, "token parts");
};

typedef Mma<float> MF;

__device__ __forceinline__ floatx4 ld4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// Element (row, col) of a tensor [B, T, H, width] for token t0 + row of
// sequence bb, head h.
__device__ __forceinline__ int64_t tok_index(int bb, int T, int H, int h, int t, int width) {
  return (((int64_t)bb * T + t) * H + h) * width;
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

// ---------------------------------------------------------------------------
// Prep: grid = B*H*nchunks (chunk-minor), NT threads.  Thread (c, part):
// channel c = tid % D, tokens TPP part .. TPP part + TPP - 1 of the chunk.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NT) void f32_prep_kernel(PrefillArgs a) {
  typedef Geo<D> G;
  constexpr int LD = G::LD, TPP = G::TPP, NPART = G::NPART;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* Kt = reinterpret_cast<float*>(smem + G::P_KT);
  float* Kh = reinterpret_cast<float*>(smem + G::P_KH);
  float* Qt = reinterpret_cast<float*>(smem + G::P_QT);
  float* Lm = reinterpret_cast<float*>(smem + G::P_L);
  float* beta = reinterpret_cast<float*>(smem + G::P_BETA);
  float* tot = reinterpret_cast<float*>(smem + G::P_TOT);

  const int nch = (a.T + C - 1) / C;
  const int head = blockIdx.x / nch, n = blockIdx.x % nch;
  const int bb = head / a.H, h = head % a.H;
  const int t0 = n * C, nv = min(C, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & (D - 1), part = tid / D;
  float* blk = a.ws + ((int64_t)head * nch + n) * G::WS_BLOCK;
  const int64_t base = tok_index(bb, a.T, a.H, h, t0, D);   // token t0, channel 0
  const int64_t tstr = (int64_t)a.H * D;                   // token stride

  // in-chunk prefix sums: each part scans its tokens and then adds the
  // totals of the parts before it; r is the sum through token 31, b_C the
  // chunk's whole sum
  float b[TPP];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < TPP; ++i) {
    const int t = TPP * part + i;
    s += (t < nv ? ldf<T>(a.g, base + t * tstr + c) : 0.f) * kLog2e;
    b[i] = s;
  }
  tot[part * D + c] = s;
  if (tid < C) beta[tid] = tid < nv ? ldf<T>(a.beta, ((int64_t)bb * a.T + t0 + tid) * a.H + h) : 0.f;
  __syncthreads();
  float off = 0.f, r = 0.f, bC = 0.f;
#pragma unroll
  for (int pp = 0; pp < NPART; ++pp) {
    const float x = tot[pp * D + c];
    if (pp < part) off += x;
    if (pp < 32 / TPP) r += x;
    bC += x;
  }
#pragma unroll
  for (int i = 0; i < TPP; ++i) b[i] += off;

  // the gated operands: Kt, Kh, Qt to LDS; Qg, Kb to the workspace
#pragma unroll 4
  for (int i = 0; i < TPP; ++i) {
    const int t = TPP * part + i;
    const float kv = t < nv ? ldf<T>(a.k, base + t * tstr + c) : 0.f;
    const float qv = t < nv ? ldf<T>(a.q, base + t * tstr + c) : 0.f;
    const float up = exp2f(b[i] - r), dn = exp2f(r - b[i]);
    Kt[t * LD + c] = kv * up;
    Kh[t * LD + c] = kv * dn;
    Qt[t * LD + c] = qv * up;
    blk[G::WS_QG + t * D + c] = qv * exp2f(b[i]);
    blk[G::WS_KB + t * D + c] = kv * exp2f(bC - b[i]);
  }
  if (part == 0) blk[G::WS_GM + c] = exp2f(bC);
  __syncthreads();

  // L and P, 16 x 16 tiles (I, J): 16 tiles of each, 8 per wavefront; tiles
  // above the diagonal are zero (P's are stored as such, L's are not read)
  const int l16 = lane & 15, g4 = lane >> 4;
  for (int tl = wave; tl < 32; tl += 4) {
    const bool isP = tl >= 16;
    const int I = (tl & 15) >> 2, J = tl & 3;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (J <= I) {
      const float* A = (isP ? Qt : Kt) + (16 * I + l16) * LD + 4 * g4;
      const float* Bm = Kh + (16 * J + l16) * LD + 4 * g4;
#pragma unroll
      for (int sl = 0; sl < D / 16; ++sl) acc = MF::mma16(ld4(A + 16 * sl), ld4(Bm + 16 * sl), acc);
    }
    const int j = 16 * J + l16;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = 16 * I + 4 * g4 + jj;
      if (isP)
        blk[G::WS_P + i * C + j] = j <= i ? acc[jj] : 0.f;
      else if (J <= I)
        Lm[i * LDC + j] = j < i ? beta[i] * acc[jj] : 0.f;
    }
  }
  __syncthreads();

  // Kg = 2^b K over Kh, V over Qt (both are free now)
#pragma unroll 4
  for (int i = 0; i < TPP; ++i) {
    const int t = TPP * part + i;
    const float kv = t < nv ? ldf<T>(a.k, base + t * tstr + c) : 0.f;
    Kh[t * LD + c] = kv * exp2f(b[i]);
    Qt[t * LD + c] = t < nv ? ldf<T>(a.v, tok_index(bb, a.T, a.H, h, t0 + t, D) + c) : 0.f;
  }
  // A = (I + L)^-1 in place, one row after the other, one lane per column:
  // A_i = e_i - sum_{j<i} L_ij A_j (row i of L is read whole before row i of
  // A overwrites it; one wavefront, so in program order)
  if (wave == 0) {
    for (int i = 0; i < C; ++i) {
      float x = lane == i ? 1.f : 0.f;
      const float* Li = Lm + i * LDC;
      for (int j = 0; j < i; ++j) x -= Li[j] * Lm[j * LDC + lane];
      Lm[i * LDC + lane] = x;
    }
  }
  __syncthreads();

  // W = A Diag(beta) Kg and U = A Diag(beta) V: 2 (C/16) (D/16) tiles over
  // the four wavefronts; A is lower triangular, so tile row I sums token
  // slabs 0..I
  constexpr int NTW = (C / 16) * (D / 16);
  for (int tl = wave; tl < 2 * NTW; tl += 4) {
    const bool isU = tl >= NTW;
    const int I = (tl % NTW) / (D / 16), N = tl % (D / 16);
    const float* X = isU ? Qt : Kh;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int J = 0; J <= I; ++J) {
      const int t = 16 * J + 4 * g4;
      floatx4 af = ld4(Lm + (16 * I + l16) * LDC + t);
      const floatx4 bw = ld4(beta + t);
      af *= bw;
      floatx4 bf;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bf[jj] = X[(t + jj) * LD + 16 * N + l16];
      acc = MF::mma16(af, bf, acc);
    }
    float* out = blk + (isU ? G::WS_U : G::WS_W);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[(16 * I + 4 * g4 + jj) * D + 16 * N + l16] = acc[jj];
  }
}

// ---------------------------------------------------------------------------
// State pass: grid = ceil(B*H / 8) * 8 * NSPLIT, NT threads.  Wavefront w
// forms token rows 16w .. 16w+15 of Delta and O, and updates state rows
// (D/4) w .. (D/4) (w+1) - 1.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NT) void f32_state_kernel(PrefillArgs a) {
  typedef Geo<D> G;
  constexpr int LD = G::LD, NSPLIT = G::NSPLIT;
  constexpr int RW = D / 4;   // state rows per wavefront
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* S = reinterpret_cast<float*>(smem + G::S_S);
  float* Wm = reinterpret_cast<float*>(smem + G::S_W);
  float* Qg = reinterpret_cast<float*>(smem + G::S_QG);
  float* Kb = reinterpret_cast<float*>(smem + G::S_KB);
  float* Pm = reinterpret_cast<float*>(smem + G::S_P);
  float* Uv = reinterpret_cast<float*>(smem + G::S_U);
  float* gm = reinterpret_cast<float*>(smem + G::S_GM);

  // the NSPLIT slices of a head have block ids 8 apart: consecutive ids go to
  // different XCDs, so the slices of a head share one XCD's L2 for the chunk
  // blocks they all read
  const int blk = blockIdx.x;
  const int head = (blk / (8 * NSPLIT)) * 8 + blk % 8, col0 = ((blk / 8) % NSPLIT) * DVW;
  if (head >= a.B * a.H) return;
  const int bb = head / a.H, h = head % a.H;
  const int nch = (a.T + C - 1) / C;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  T* o = static_cast<T*>(a.o);

  // entry state slice: rows 0..D-1, columns col0 .. col0+31
  for (int e = tid; e < D * DVW / 4; e += NT) {
    const int row = e / (DVW / 4), c4 = 4 * (e % (DVW / 4));
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    if (a.S0) x = *reinterpret_cast<const floatx4*>(a.S0 + ((int64_t)head * D + row) * D + col0 + c4);
    *reinterpret_cast<floatx4*>(S + row * LDS_S + c4) = x;
  }

  for (int n = 0; n < nch; ++n) {
    const float* blkp = a.ws + ((int64_t)head * nch + n) * G::WS_BLOCK;
    const int t0 = n * C, nv = min(C, a.T - t0);
    // the chunk's operands to LDS
    for (int e = tid; e < C * D / 4; e += NT) {
      const int row = e / (D / 4), c4 = 4 * (e % (D / 4));
      *reinterpret_cast<floatx4*>(Wm + row * LD + c4) = ld4(blkp + G::WS_W + row * D + c4);
      *reinterpret_cast<floatx4*>(Qg + row * LD + c4) = ld4(blkp + G::WS_QG + row * D + c4);
      *reinterpret_cast<floatx4*>(Kb + row * LD + c4) = ld4(blkp + G::WS_KB + row * D + c4);
    }
    for (int e = tid; e < C * C / 4; e += NT) {
      const int row = e / (C / 4), c4 = 4 * (e % (C / 4));
      *reinterpret_cast<floatx4*>(Pm + row * LDC + c4) = ld4(blkp + G::WS_P + row * C + c4);
    }
    for (int e = tid; e < C * DVW / 4; e += NT) {
      const int row = e / (DVW / 4), c4 = 4 * (e % (DVW / 4));
      *reinterpret_cast<floatx4*>(Uv + row * LDS_S + c4) = ld4(blkp + G::WS_U + row * D + col0 + c4);
    }
    if (tid < D / 4) *reinterpret_cast<floatx4*>(gm + 4 * tid) = ld4(blkp + G::WS_GM + 4 * tid);
    __syncthreads();

    // Delta = U - W S (over U) and the inter-chunk read-out Qg S, rows 16w..
    floatx4 O[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
      const float* Wr = Wm + (16 * w + l16) * LD + 4 * g4;
      const float* Qr = Qg + (16 * w + l16) * LD + 4 * g4;
#pragma unroll
      for (int sl = 0; sl < D / 16; ++sl) {
        floatx4 sf;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sf[jj] = S[(16 * sl + 4 * g4 + jj) * LDS_S + 16 * nt + l16];
        x = MF::mma16(ld4(Wr + 16 * sl), sf, x);
        y = MF::mma16(ld4(Qr + 16 * sl), sf, y);
      }
      O[nt] = y;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float* u = Uv + (16 * w + 4 * g4 + jj) * LDS_S + 16 * nt + l16;
        *u = *u - x[jj];
      }
    }
    __syncthreads();

    // O += P Delta (P is lower triangular: token slabs 0..w), stored
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 y = O[nt];
      for (int J = 0; J <= w; ++J) {
        floatx4 df;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) df[jj] = Uv[(16 * J + 4 * g4 + jj) * LDS_S + 16 * nt + l16];
        y = MF::mma16(ld4(Pm + (16 * w + l16) * LDC + 16 * J + 4 * g4), df, y);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * w + 4 * g4 + jj;
        if (row < nv) o[tok_index(bb, a.T, a.H, h, t0 + row, D) + col0 + 16 * nt + l16] = from_f32<T>(y[jj]);
      }
    }
    // S <- Diag(gamma) S + Kb^T Delta, state rows RW w .. RW (w+1) - 1
#pragma unroll
    for (int rt = 0; rt < RW / 16; ++rt) {
      const int r0 = RW * w + 16 * rt;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        floatx4 acc;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int row = r0 + 4 * g4 + jj;
          acc[jj] = gm[row] * S[row * LDS_S + 16 * nt + l16];
        }
#pragma unroll
        for (int J = 0; J < C / 16; ++J) {
          floatx4 kf, df;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int t = 16 * J + 4 * g4 + jj;
            kf[jj] = Kb[t * LD + r0 + l16];
            df[jj] = Uv[t * LDS_S + 16 * nt + l16];
          }
          acc = MF::mma16(kf, df, acc);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[(r0 + 4 * g4 + jj) * LDS_S + 16 * nt + l16] = acc[jj];
      }
    }
    __syncthreads();
  }

  if (a.S_T) {
    for (int e = tid; e < D * DVW / 4; e += NT) {
      const int row = e / (DVW / 4), c4 = 4 * (e % (DVW / 4));
      *reinterpret_cast<floatx4*>(a.S_T + ((int64_t)head * D + row) * D + col0 + c4) =
          ld4(S + row * LDS_S + c4);
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  typedef Geo<D> G;
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t nch = (a.T + C - 1) / C;
  if (BH == 0) return hipSuccess;
  const int64_t nstate = (BH + 7) / 8 * 8 * G::NSPLIT;
  if (BH * nch > INT32_MAX || nstate > INT32_MAX) return hipErrorInvalidValue;
  hipError_t e;
  auto prep = f32_prep_kernel<T, D>;
  auto state = f32_state_kernel<T, D>;
  if (nch > 0) {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 G::PREP_BYTES)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(prep, dim3((unsigned)(BH * nch)), dim3(NT), G::PREP_BYTES, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(state), hipFuncAttributeMaxDynamicSharedMemorySize,
                               G::STATE_BYTES)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(state, dim3((unsigned)nstate), dim3(NT), G::STATE_BYTES, s, a);
  return hipGetLastError();
}

}  // namespace f32c

size_t prefill_f32_workspace(int BH, int T, int d) {
  const int64_t nch = (T + f32c::C - 1) / f32c::C;
  const int64_t block = d == 64 ? f32c::Geo<64>::WS_BLOCK : f32c::Geo<128>::WS_BLOCK;
  return (size_t)BH * nch * block * sizeof(float);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  if (!a.bf16 && a.dk == 128 && a.dv == 128) return f32c::launch_t<float, 128>(a, s);
  if (a.bf16 && a.dk == 64 && a.dv == 64) return f32c::launch_t<bf16, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
