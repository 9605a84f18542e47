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
  bool raw_gain = false;  // gain A_t khat without the normalisation (ablation)
};

// Carried state of every stream, fp32 device tensors: the state the recurrence starts from
// (S0 [streams][d][d], A0 [streams][d][d] symmetric, n0 [streams][d]; NULL = the fixed
// start S = 0, A = I / lambda0, n = 0) and the state it ends in (NULL = not wanted).
struct StateIO {
  const float *S0 = nullptr, *A0 = nullptr, *n0 = nullptr;
  float *S_final = nullptr, *A_final = nullptr, *n_final = nullptr;
};

// Sequential path: one workgroup per stream.  Returns hipSuccess or the launch error.
hipError_t launch_seq(const Problem &p, const void *q, const void *k, const void *v,
                      const void *u, void *out, const StateIO &st, hipStream_t stream);

// Decode path (T = 1): a stream's rows spread over d / 16 workgroups.
hipError_t launch_decode(const Problem &p, const void *q, const void *k, const void *v,
                         const void *u, void *out, const StateIO &st, hipStream_t stream);

// Chunked path (time-segment parallel).  `ws` must hold chunk_workspace_bytes(p, C).
size_t chunk_workspace_bytes(const Problem &p, int chunk);
bool chunk_supported(const Problem &p, int chunk);
int chunk_default(const Problem &p);
hipError_t launch_chunk(const Problem &p, int chunk, const void *q, const void *k,
                        const void *v, const void *u, void *out, const StateIO &st, void *ws,
                        hipStream_t stream);

// Linear-attention baseline (chunked, time-segment parallel): out, S_T (S[i][j]) and n_T
// of every stream; `ws` must hold la_workspace_bytes(p).  p.lambda0 is not used.
size_t la_workspace_bytes(const Problem &p);
hipError_t launch_la(const Problem &p, const void *q, const void *k, const void *v, void *out,
                     float *S_final, float *n_final, void *ws, hipStream_t stream);

// Backward of the recurrence from the fixed start (sequential, one workgroup per stream).
struct BackwardIO {
  const void *q, *k, *v, *u, *dout;            // [streams][T][d] in the input dtype
  const float *dS_T, *dA_T, *dn_T;             // cotangents of the final state, or NULL
  float *dq, *dk, *dv, *du;                    // [streams][T][d] fp32
  float *dlambda0;                             // [streams] fp32, or NULL
};
size_t backward_workspace_bytes(const Problem &p);
hipError_t launch_backward(const Problem &p, const BackwardIO &io, void *ws, hipStream_t stream);

// While an object of this type lives, launches on the calling thread record no timing events
// (the allocation-free entry point creates no events, whatever vla_profile_enable says).
class ProfQuiet {
 public:
  ProfQuiet();
  ~ProfQuiet();
  ProfQuiet(const ProfQuiet &) = delete;
  ProfQuiet &operator=(const ProfQuiet &) = delete;

 private:
  bool prev_;
};

// Event-pair timing of one kernel launch when vla_profile_enable(1) is in effect.
class ProfScope {
 public:
  ProfScope(const char *name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope &) = delete;
  ProfScope &operator=(const ProfScope &) = delete;

 private:
  const char *name_;
  hipStream_t stream_;
  hipEvent_t ev0_ = nullptr, ev1_ = nullptr;
  bool active_ = false;
};

}  // namespace vla

// Launch a kernel, timed under `name` when profiling is enabled.
#define VLA_LAUNCH(name, kernel, grid, block, shmem, stream, ...)               \
  do {                                                                          \
    ::vla::ProfScope vla_prof_scope_(name, stream);                             \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);        \
  } while (0)
