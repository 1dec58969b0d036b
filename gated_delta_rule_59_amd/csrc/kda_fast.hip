// Matrix-core chunked KDA forward (bf16 activations, dk = dv = 128, chunk = 64).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

bool fast_path_applies(const ChunkPlan&) { return false; }
size_t fast_workspace_bytes(const ChunkPlan&) { return 0; }
hipError_t launch_chunk_fast(const ChunkPlan&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
