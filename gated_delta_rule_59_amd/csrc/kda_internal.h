// Host-side launch descriptions passed from the C ABI layer (kda_api.cpp) to the kernel
// launchers. Arguments are validated before a plan is built.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodePlan {
  int N, H, dk, dv;
  bool act_bf16, out_bf16;
  const void *q, *k, *v, *g, *beta;
  float* S;
  void* o;
};

struct ChunkPlan {
  int B, T, H, dk, dv, chunk;
  const int32_t* cu_seqlens;  // device, or nullptr for a dense batch
  int n_seq;                  // B (dense) or N (packed)
  bool act_bf16, out_bf16;
  const void *q, *k, *v, *g, *beta;
  const float* S0;
  void* o;
  float* S_T;
  void* workspace;
  size_t workspace_bytes;
  float* ckpt;      // state checkpoints [ckpt_slots, H, dk, dv], or nullptr
  int ckpt_every;   // tokens between checkpoints (a multiple of chunk), 0 = none
  int ckpt_slots;
  bool pairwise_diag;  // matrix-core path: diagonal tiles pairwise (no decay bound needed)
  int segments;        // matrix-core path: walk each sequence in this many segments (>= 3), else 1
  int walk_block;      // matrix-core path: tokens per walk step, 64 (one chunk) or 128 (two
                       // chunks composed into one step)
};

hipError_t launch_decode(const DecodePlan& p, hipStream_t stream);

struct DecodeMultiPlan {
  int N, H, dk, dv, m;
  bool act_bf16, out_bf16;
  const void *q, *k, *v, *g, *beta;
  float* S;
  void* o;                // nullptr: outputs not written
  const int32_t* accept;  // nullptr: S not modified
};

hipError_t launch_decode_multi(const DecodeMultiPlan& p, hipStream_t stream);

// Generic path: fp32 arithmetic on the vector ALUs, any supported dk/dv/chunk; used for
// fp32 activations and for shapes the matrix-core path does not take.
hipError_t launch_chunk_generic(const ChunkPlan& p, hipStream_t stream);

// Matrix-core path: bf16 activations, dk = dv = 128, chunk = 64.
bool fast_path_applies(const ChunkPlan& p);
size_t fast_workspace_bytes(const ChunkPlan& p);
hipError_t launch_chunk_fast(const ChunkPlan& p, hipStream_t stream);

// Fixed device scratch of the allocation-free prefill entry point: its size, and its device
// address on the current device (looked up on the first call per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

// Device check of g in [-5, 0] and beta in [0, 1] over n_blocks workgroups (1 .. check_blocks());
// writes each workgroup's count of violations into counts[0 .. n_blocks).
int check_blocks();
hipError_t launch_check_gates(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                              bool bf16, int64_t* counts, int n_blocks, hipStream_t stream);

}  // namespace kda
