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
// records: the workspace of the backward's chunked forward (launch_chunk_records)
size_t chunk_workspace_bytes(const Problem &p, int chunk, bool records = false);
bool chunk_supported(const Problem &p, int chunk);
int chunk_default(const Problem &p);
// With `may_split`, calls of at least 2^20 tokens on two or more streams (not under graph
// capture) run half of the streams on a library-owned second HIP stream of the device, forked
// from and joined back into `stream` with events; the result is the same either way.
hipError_t launch_chunk(const Problem &p, int chunk, const void *q, const void *k,
                        const void *v, const void *u, void *out, const StateIO &st, void *ws,
                        hipStream_t stream, bool may_split);

// The chunked path's passes up to the segment-start states (no outputs): S, A and n at the
// start of every segment [streams][P][...] and the pass's segment-map buffer
// [streams][P][2][d][d] (free for reuse once this returns), all inside `ws`.  With Md (fp64
// [streams][P][d][d], device) the segment-start A come from an fp64 inversion.
struct ChunkStates {
  float *S_seg = nullptr, *A_seg = nullptr, *n_seg = nullptr, *pib = nullptr;
  int64_t L = 0, P = 0;
};
void chunk_segments(const Problem &p, int chunk, int64_t *L, int64_t *P);
hipError_t launch_chunk_states(const Problem &p, int chunk, const void *q, const void *k,
                               const void *v, const void *u, void *ws, double *Md,
                               hipStream_t stream, ChunkStates *cs);
// The backward's token records and state checkpoints, written by the chunked forward's passes
// in place of a token-by-token replay: rec [streams][T][6d + 8] fp32, ck
// [streams][ceil(T / 64)][2][d][d] (S, A after every 64th token and each segment's last),
// n_end [streams][P][d] (n after each segment).  Also gives the segment-start states (cs).
struct BwRecords {
  float *rec = nullptr, *ck = nullptr, *n_end = nullptr;
};
hipError_t launch_chunk_records(const Problem &p, int chunk, const void *q, const void *k,
                                const void *v, const void *u, void *ws, double *Md,
                                hipStream_t stream, const BwRecords &rec, ChunkStates *cs);
// In place over each stream's P matrices [streams][P][d][d]: M_j <- M0 + sum_{j' < j} M_j' (fp64
// sums; M0 = Minit[stream], or 0 when Minit is NULL).
hipError_t launch_matrix_prefix(const Problem &p, float *M, int64_t P, const float *Minit,
                                hipStream_t stream);
// X_0 = S0[stream] (0 when NULL), X_{j+1} = X_j Pi_j + B_j with pib [streams][P][2][d][d] =
// (Pi_j, B_j), into s0 [streams][P][d][d]; when nk is not NULL also, in place over
// [streams][P][d], nk_j <- n0[stream] + sum_{j' < j} nk_j' (fp64 sums, n0 NULL = 0).
hipError_t launch_affine_prefix(const Problem &p, const float *pib, float *s0, int64_t P,
                                const float *S0, float *nk, const float *n0, hipStream_t stream);

// Linear-attention baseline (chunked, time-segment parallel): out, S_T (S[i][j]) and n_T
// of every stream; `ws` must hold la_workspace_bytes(p).  p.lambda0 is not used.
size_t la_workspace_bytes(const Problem &p);
hipError_t launch_la(const Problem &p, const void *q, const void *k, const void *v, void *out,
                     float *S_final, float *n_final, void *ws, hipStream_t stream);

// Backward of the recurrence from the fixed start (one workgroup per segment of a stream).
struct BackwardIO {
  const void *q, *k, *v, *u, *dout;            // [streams][T][d] in the input dtype
  const float *dS_T, *dA_T, *dn_T;             // cotangents of the final state, or NULL
  float *dq, *dk, *dv, *du;                    // [streams][T][d] fp32
  float *dlambda0;                             // [streams] fp32, or NULL
};
// chunk = 0: one segment per stream (token by token); else the chunked path's segments with
// that chunk length (chunk_supported must hold).
size_t backward_workspace_bytes(const Problem &p, int chunk);
hipError_t launch_backward(const Problem &p, int chunk, const BackwardIO &io, void *ws,
                           hipStream_t stream);

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
