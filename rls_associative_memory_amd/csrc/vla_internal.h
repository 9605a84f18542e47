// Internal host-side declarations shared by the C-ABI front end and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vla {

enum class Dtype : int { F32 = 0, BF16 = 1 };

struct Problem {
  int64_t streams;  // B * H
  int64_t T;
  int d;
  Dtype dtype;
  float lambda0;
  float eps;
};

// Sequential path: one workgroup per stream.  Returns hipSuccess or the launch error.
hipError_t launch_seq(const Problem &p, const void *q, const void *k, const void *v,
                      const void *u, void *out, float *S_final, float *A_final,
                      hipStream_t stream);

// Chunked path (time-segment parallel).  `ws` must hold chunk_workspace_bytes(p, C).
size_t chunk_workspace_bytes(const Problem &p, int chunk);
bool chunk_supported(const Problem &p, int chunk);
int chunk_default(const Problem &p);
hipError_t launch_chunk(const Problem &p, int chunk, const void *q, const void *k,
                        const void *v, const void *u, void *out, float *S_final,
                        float *A_final, void *ws, hipStream_t stream);

}  // namespace vla
