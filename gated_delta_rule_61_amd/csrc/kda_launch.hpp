// kda_launch.hpp -- host-side launch interface between the C-ABI layer and
// the kernel translation units.  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
  const void* q; const void* k; const void* v; const void* g; const void* beta;
  const float* S0; void* o; float* S_T;
  int B, T, H, dk, dv;
  int bf16;       // 1: bf16 inputs/outputs, 0: fp32
  int nsplit;     // column split of the state across workgroups (0 = auto)
  int pipeline;   // 1: software-pipelined schedule where it applies (bf16, d = 128, no split)
};

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
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_fused(const PrefillArgs& a, hipStream_t s);
hipError_t launch_stage_cumsum(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_ut(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_state(const StageArgs& a, hipStream_t s);
hipError_t launch_stage_output(const StageArgs& a, hipStream_t s);

// Default column split of the fused prefill for B*H heads on this device.
int fused_default_nsplit(int BH, int dv);

}  // namespace kda
