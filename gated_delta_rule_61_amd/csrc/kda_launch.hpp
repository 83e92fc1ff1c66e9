// kda_launch.hpp -- host-side launch interface between the C-ABI layer and
// the kernel translation units.  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Variants of the recurrence, bit flags (the values of the C ABI's):
constexpr int kVarScalarGate = 1;   // g holds one log-gate per token and head ([B,T,H] / [N,H])
constexpr int kVarNoDelta = 2;      // no erase term: S_t = Diag(exp g_t) S_{t-1} + k_t v_t^T, beta unused

struct PrefillArgs {
  const void* q; const void* k; const void* v; const void* g; const void* beta;
  const float* S0; void* o; float* S_T;
  int B, T, H, dk, dv;
  int bf16;       // 1: bf16 inputs/outputs, 0: fp32
  int nsplit;     // column split of the state across workgroups (0 = auto)
  int pipeline;   // 1: software-pipelined schedule where it applies (bf16, d = 128, no split)
  // Segmented schedule of the pipelined kernel (nseg >= 3 segments of seg_len
  // chunks per sequence, see launch_pipe); nseg = 0: one pass per sequence.
  int nseg, seg_len;
  int pass;       // set by the launcher: 1 = segment 0 and the segment maps, 3 = segments 1..nseg-1
  float* ws;      // nseg_workspace_bytes() of fp32 scratch
  int variant;    // kVar* flags (nonzero: bf16, d = 128, pipelined kernel only)
  // Packed sequences (pipelined kernel, one pass): B sequences, sequence b is
  // tokens [cu_seqlens[b], cu_seqlens[b+1]) of [T, H, d] tensors; NULL: [B, T, H, d].
  const int* cu_seqlens;
  const int* seq_order;   // packed sequences: processing order (a permutation of 0..B-1), or NULL
  // Chunk-entry states (one pass; the outputs too unless o is NULL): the
  // state at the start of every chunk, bf16 in the pipelined kernel's owner
  // fragment order, one 32 KB block per chunk and head (the backward's
  // layout); NULL: normal forward.
  void* states;
  // Packed sequences, segmented: the device plan (varlen_plan_kernel) with
  // job tables of plan_j1 / plan_j3 entries, segments of seg_len chunks, the
  // segment maps in ws; NULL: no segmented schedule for packed sequences.
  int* plan;
  int plan_j1, plan_j3, plan_ns;
};

// Offset (in ints) of the job tables inside a plan for N sequences.
__host__ __device__ inline int varlen_plan_table_offset(int N) { return (4 + 3 * N + 1) & ~1; }

// Segmented schedule for packed sequences: segment length in chunks (0: one
// pass), the bounds of its job tables and map slots, and its workspace.
struct VarlenSeg {
  int L;          // chunks per segment (0: no segmented schedule)
  int j1, j3;     // job-table bounds of pass 1 and pass 3
  int ns;         // bound on the segmented sequences
  int slots;      // bound on the map slots (each H x 3 maps of d x d fp32)
  size_t plan_bytes, bytes;
};
VarlenSeg varlen_segments(int N, int T_total, int H, int cus);

struct StageArgs {
  const void* q; const void* k; const void* v; const void* g; const void* beta;
  const float* S0; void* o; float* S_T;
  float* b; float* W; float* U; float* Delta; float* S_chunks;
  int B, T, H, dk, dv, bf16;
};

struct DecodeArgs {
  const void* q; const void* k; const void* v; const void* g; const void* beta;
  float* S; void* o;
  int N, H, dk, dv, bf16;
  int variant;    // kVar* flags
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Backward of the chunked forward (bf16, d_k = d_v = 128).
struct BackwardArgs {
  const void* q; const void* k; const void* v; const void* g; const void* beta;
  const float* S0; const void* dO; const float* dS_T;
  void* dq; void* dk; void* dv; void* dg; void* dbeta; float* dS0;
  int B, T, H;
  void* states;     // bf16 [B*H][N] chunk-entry states, in the forward owners' fragment order
  void* adjoints;   // bf16 [B*H][N] adjoints of the chunk-end states, 16 x 16 tiles ([j][c] inside)
  void* mats;       // bf16 [B*H][N] per-chunk operand blocks (A, P^T, Kg, Kd, Qg, gamma, beta)
  float* dg32;      // if set: dg as fp32 [B,T,H,d_k] here instead of bf16 into dg
  int variant;      // kVar* flags: 0 or kVarNoDelta for the chunked backward, any for the token path
  // Packed sequences: B sequences, sequence b is tokens [cu_seqlens[b],
  // cu_seqlens[b+1]) of [T, H, d] tensors; the per-chunk arrays hold nslots x H
  // blocks (backward_varlen_slots).  NULL: [B, T, H, d].
  const int* cu_seqlens;
  int nslots;
  // 1: `states` already holds every chunk's entry state (written by the
  // forward with kda_chunk_fwd_save), so the state pass is skipped
  int states_saved;
};
size_t backward_workspace(int BH, int T);
// Backward for the other sizes (fp32 at d = 64 or 128, bf16 at d = 64; every
// variant): the token recurrence's reverse mode with chunk checkpoints
// (kda_backward_tok.hip).  ws holds backward_tok_workspace(B, T, H, d) bytes.
size_t backward_tok_workspace(int B, int T, int H, int d);
hipError_t launch_backward_tok(const BackwardArgs& a, int d, bool bf16in, void* ws, hipStream_t s);
int backward_varlen_slots(int nseq, int T);
size_t backward_varlen_workspace(int nseq, int T, int H);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
// scalar gate: g [rows] broadcast to bf16 [rows][128]; dg [rows] = channel sums of fp32 [rows][128]
hipError_t launch_gate_expand(const void* g, void* gfull, int64_t rows, hipStream_t s);
hipError_t launch_gate_reduce(const float* dg32, void* dg, int64_t rows, hipStream_t s);
// Order of packed sequences by decreasing chunk count (ties by index) into
// order[0..N-1]; N <= kMaxScheduleSeqs.
constexpr int kMaxScheduleSeqs = 16384;
hipError_t launch_varlen_schedule(const int* cu_seqlens, int N, int T, int* order, hipStream_t s);
hipError_t launch_fused(const PrefillArgs& a, hipStream_t s);
hipError_t launch_stage_cumsum(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_ut(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_state(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_output(const StageArgs& a, hipStream_t s);

// Chunked prefill with fp32 matrix operands, for fp32 inputs at d = 128 and
// bf16 inputs at d = 64 (two launches, see kda_prefill_f32.hip): a.ws must
// hold prefill_f32_workspace(B*H, T, d) bytes.
size_t prefill_f32_workspace(int BH, int T, int d);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);

// Default column split of the fused prefill for B*H heads on this device.
int fused_default_nsplit(int BH, int dv);

// Segments per sequence for the segmented pipelined prefill on a device with
// `cus` compute units (0: one pass), chunks per segment, and the workspace.
int prefill_segments(int BH, int T, int cus);
int prefill_segment_len(int T, int nseg);
size_t prefill_segment_workspace(int BH, int nseg);

}  // namespace kda
