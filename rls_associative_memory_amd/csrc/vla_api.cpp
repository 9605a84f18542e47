// C-ABI front end of the VLA forward library: argument checks, path choice, workspace,
// launches on the caller's stream.  No kernel code lives here.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <optional>
#include <vector>

#include "vla.h"
#include "vla_internal.h"

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Whether [a, a + na) and [b, b + nb) share a byte (false when either pointer is NULL).
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (a == nullptr || b == nullptr) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool d_supported(int64_t d) { return d == 32 || d == 64 || d == 96 || d == 128; }

// Shape / scalar checks shared by every entry point (no device work).
vla_status_t check_desc(const vla_desc_t *desc) {
  if (desc == nullptr) return VLA_ERROR_INVALID_VALUE;
  if (desc->B < 1 || desc->H < 1 || desc->T < 1 || desc->d < 1) return VLA_ERROR_INVALID_VALUE;
  if (desc->dtype != VLA_DTYPE_F32 && desc->dtype != VLA_DTYPE_BF16) return VLA_ERROR_INVALID_VALUE;
  if (desc->path < VLA_PATH_AUTO || desc->path > VLA_PATH_DECODE) return VLA_ERROR_INVALID_VALUE;
  if (!(desc->eps >= 0.0f) || !std::isfinite(desc->eps)) return VLA_ERROR_INVALID_VALUE;
  if (desc->chunk < 0) return VLA_ERROR_INVALID_VALUE;
  if (desc->gain != VLA_GAIN_UNIT && desc->gain != VLA_GAIN_RAW) return VLA_ERROR_INVALID_VALUE;
  // B*H*T*d must be addressable; B*H must fit a grid dimension.
  const int64_t lim = int64_t(1) << 40;
  if (desc->B > lim / desc->H) return VLA_ERROR_INVALID_VALUE;
  const int64_t bh = desc->B * desc->H;
  if (bh > (int64_t(1) << 31) - 1 || desc->T > lim / bh || desc->d > lim / (bh * desc->T))
    return VLA_ERROR_INVALID_VALUE;
  if (!d_supported(desc->d)) return VLA_ERROR_NOT_SUPPORTED;
  return VLA_SUCCESS;
}

vla::Problem make_problem(const vla_desc_t *desc, float lambda0) {
  vla::Problem p;
  p.streams = desc->B * desc->H;
  p.T = desc->T;
  p.d = static_cast<int>(desc->d);
  p.dtype = desc->dtype == VLA_DTYPE_F32 ? vla::Dtype::F32 : vla::Dtype::BF16;
  p.lambda0 = lambda0;
  p.eps = desc->eps;
  p.raw_gain = desc->gain == VLA_GAIN_RAW;
  return p;
}

// Resolve the path and chunk length; returns NOT_SUPPORTED for a forced path / chunk the
// shape cannot use.
vla_status_t resolve(const vla_desc_t *desc, const vla::Problem &p, int32_t *path, int *chunk) {
  int c = desc->chunk;
  int32_t want = desc->path;
  if (want == VLA_PATH_DECODE && p.T != 1) return VLA_ERROR_NOT_SUPPORTED;
  if (want == VLA_PATH_AUTO && p.T == 1) want = VLA_PATH_DECODE;
  if (want == VLA_PATH_AUTO && p.raw_gain) want = VLA_PATH_SEQ;  // the only multi-token path with it
  if (want == VLA_PATH_CHUNK && p.raw_gain) return VLA_ERROR_NOT_SUPPORTED;
  if (want == VLA_PATH_AUTO) {
    // Enough streams to fill the machine one workgroup each, or sequences too short to
    // amortise the segment passes: run token by token.  Otherwise split time: few streams of
    // at least 1024 tokens, or (fp32 inputs, whose segments can be as short as 64 tokens) up to
    // 256 streams of at least 256 tokens (at d = 32 both one stream of 256 tokens and 256
    // streams of 512 run faster split into segments than token by token).
    const bool few_streams = p.streams < 128;
    const bool long_seq = p.T >= 1024;
    const bool short_fp32 = p.dtype == vla::Dtype::F32 && p.streams <= 256 && p.T >= 256;
    want = (((few_streams && long_seq) || short_fp32) &&
            vla::chunk_supported(p, c ? c : vla::chunk_default(p)))
               ? VLA_PATH_CHUNK
               : VLA_PATH_SEQ;
  }
  if (want == VLA_PATH_CHUNK) {
    if (c == 0) c = vla::chunk_default(p);
    if (!vla::chunk_supported(p, c)) return VLA_ERROR_NOT_SUPPORTED;
  } else {
    c = 0;
  }
  *path = want;
  *chunk = c;
  return VLA_SUCCESS;
}

// Per-device check that the current device is gfx950, cached.
struct DeviceInfo {
  std::once_flag once;
  bool ok = false;
};
std::mutex g_dev_mu;
std::vector<DeviceInfo *> g_devs;

bool device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  DeviceInfo *info;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (static_cast<int>(g_devs.size()) <= dev) g_devs.resize(dev + 1, nullptr);
    if (g_devs[dev] == nullptr) g_devs[dev] = new DeviceInfo();
    info = g_devs[dev];
  }
  std::call_once(info->once, [&] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      info->ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  return info->ok;
}

// Library-owned workspace cache: one buffer per (device, stream), grown on demand.  Calls on
// one stream run in order, so they may share that stream's buffer; a call on another stream
// gets a buffer of its own.  Growing waits for the stream's earlier work (the only work that
// can still use the old buffer) before freeing it, which a stream under graph capture cannot
// do: such a call returns VLA_ERROR_NOT_SUPPORTED (pass a workspace instead).
struct WsCache {
  int dev = -1;
  hipStream_t stream = nullptr;
  void *ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::vector<WsCache> g_ws;

vla_status_t cached_workspace(size_t need, hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VLA_ERROR_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  WsCache *c = nullptr;
  for (WsCache &e : g_ws)
    if (e.dev == dev && e.stream == stream) c = &e;
  if (c == nullptr) {
    g_ws.push_back(WsCache{dev, stream, nullptr, 0});
    c = &g_ws.back();
  }
  if (c->bytes < need) {
    if (c->ptr != nullptr) {
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return VLA_ERROR_LAUNCH;
      if (cap != hipStreamCaptureStatusNone) return VLA_ERROR_NOT_SUPPORTED;
      if (hipStreamSynchronize(stream) != hipSuccess) return VLA_ERROR_LAUNCH;
      (void)hipFree(c->ptr);
      c->ptr = nullptr;
      c->bytes = 0;
    }
    if (hipMalloc(&c->ptr, need) != hipSuccess) {
      c->ptr = nullptr;
      return VLA_ERROR_OUT_OF_MEMORY;
    }
    c->bytes = need;
  }
  *out = c->ptr;
  return VLA_SUCCESS;
}

// Whether any output range overlaps another output or any input (inputs may alias one
// another: they are only read).  NULL pointers take part in nothing.
struct Range {
  const void *p;
  size_t n;
};
bool outputs_alias(const Range *outs, int no, const Range *ins, int ni) {
  for (int a = 0; a < no; ++a) {
    for (int b = a + 1; b < no; ++b)
      if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return true;
    for (int b = 0; b < ni; ++b)
      if (overlaps(outs[a].p, outs[a].n, ins[b].p, ins[b].n)) return true;
  }
  return false;
}

}  // namespace

extern "C" {

const char *vla_status_string(vla_status_t s) {
  switch (s) {
    case VLA_SUCCESS: return "VLA_SUCCESS";
    case VLA_ERROR_INVALID_VALUE: return "VLA_ERROR_INVALID_VALUE";
    case VLA_ERROR_NOT_SUPPORTED: return "VLA_ERROR_NOT_SUPPORTED";
    case VLA_ERROR_OUT_OF_MEMORY: return "VLA_ERROR_OUT_OF_MEMORY";
    case VLA_ERROR_LAUNCH: return "VLA_ERROR_LAUNCH";
    case VLA_ERROR_NO_DEVICE: return "VLA_ERROR_NO_DEVICE";
  }
  return "VLA_ERROR_UNKNOWN";
}

int32_t vla_version(void) { return kVersion; }

vla_status_t vla_resolve_path(const vla_desc_t *desc, int32_t *path) {
  if (path == nullptr) return VLA_ERROR_INVALID_VALUE;
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  int chunk = 0;
  return resolve(desc, make_problem(desc, 1.0f), path, &chunk);
}

vla_status_t vla_workspace_size(const vla_desc_t *desc, size_t *bytes) {
  if (bytes == nullptr) return VLA_ERROR_INVALID_VALUE;
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  const vla::Problem p = make_problem(desc, 1.0f);
  int32_t path = 0;
  int chunk = 0;
  st = resolve(desc, p, &path, &chunk);
  if (st != VLA_SUCCESS) return st;
  *bytes = path == VLA_PATH_CHUNK ? vla::chunk_workspace_bytes(p, chunk) : 0;
  return VLA_SUCCESS;
}

}  // extern "C"

namespace {

// Scratch of vla_forward_state_noalloc: one static array per device, never allocated by a
// call.  In host code `scratch` names a host-side stand-in, not device memory, so its device
// address is looked up once per device (with that device current) and only that address is
// passed to kernels.  Every allocation-free call on a device shares the array.
constexpr size_t kNoAllocScratchBytes = VLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchInfo {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void *ptr = nullptr;
};
std::mutex g_scratch_mu;
std::vector<ScratchInfo *> g_scratch;

vla_status_t scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VLA_ERROR_NO_DEVICE;
  ScratchInfo *info;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (static_cast<int>(g_scratch.size()) <= dev) g_scratch.resize(dev + 1, nullptr);
    if (g_scratch[dev] == nullptr) g_scratch[dev] = new ScratchInfo();
    info = g_scratch[dev];
  }
  std::call_once(info->once, [&] {
    void *ptr = nullptr;
    info->err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    info->ptr = info->err == hipSuccess ? ptr : nullptr;
  });
  if (info->err != hipSuccess || info->ptr == nullptr) return VLA_ERROR_LAUNCH;
  *out = info->ptr;
  return VLA_SUCCESS;
}

// vla_forward_state and vla_forward_state_noalloc.  With `noalloc` the chunked path's scratch
// is the device's static array (never an allocation), and neither timing events nor the
// events of a two-stream split of large calls are created.
vla_status_t forward_state_impl(const void *q, const void *k, const void *v, const void *u,
                                float lambda0, const float *S0, const float *A0, const float *n0,
                                void *out, float *S_final, float *A_final, float *n_final,
                                const vla_desc_t *desc, struct ihipStream_t *stream, bool noalloc) {
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  if (q == nullptr || k == nullptr || v == nullptr || u == nullptr || out == nullptr)
    return VLA_ERROR_INVALID_VALUE;
  if (A0 == nullptr && (!(lambda0 > 0.0f) || !std::isfinite(lambda0))) return VLA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(u) || !aligned16(out) ||
      !aligned16(S_final) || !aligned16(A_final) || !aligned16(n_final) || !aligned16(S0) ||
      !aligned16(A0) || !aligned16(n0))
    return VLA_ERROR_NOT_SUPPORTED;
  {  // outputs overlap neither one another nor any input (no update in place)
    const size_t bh = static_cast<size_t>(desc->B * desc->H);
    const size_t tok = bh * desc->T * desc->d * (desc->dtype == VLA_DTYPE_F32 ? 4 : 2);
    const size_t mat = bh * desc->d * desc->d * sizeof(float);
    const size_t vec = bh * desc->d * sizeof(float);
    const Range outs[4] = {{out, tok}, {S_final, mat}, {A_final, mat}, {n_final, vec}};
    const Range ins[7] = {{q, tok}, {k, tok}, {v, tok}, {u, tok}, {S0, mat}, {A0, mat}, {n0, vec}};
    if (outputs_alias(outs, 4, ins, 7)) return VLA_ERROR_INVALID_VALUE;
  }
  const vla::Problem p = make_problem(desc, A0 != nullptr ? 1.0f : lambda0);
  int32_t path = 0;
  int chunk = 0;
  st = resolve(desc, p, &path, &chunk);
  if (st != VLA_SUCCESS) return st;
  void *ws = nullptr;
  if (noalloc && desc->workspace != nullptr) return VLA_ERROR_INVALID_VALUE;
  if (path == VLA_PATH_CHUNK) {
    const size_t need = vla::chunk_workspace_bytes(p, chunk);
    if (noalloc && need > kNoAllocScratchBytes) return VLA_ERROR_NOT_SUPPORTED;
    if (desc->workspace != nullptr) {
      if (desc->workspace_bytes < need) return VLA_ERROR_INVALID_VALUE;
      if (!aligned16(desc->workspace)) return VLA_ERROR_NOT_SUPPORTED;
      ws = desc->workspace;
      const size_t bh = static_cast<size_t>(desc->B * desc->H);
      const size_t tok = bh * desc->T * desc->d * (desc->dtype == VLA_DTYPE_F32 ? 4 : 2);
      const size_t mat = bh * desc->d * desc->d * sizeof(float);
      const size_t vec = bh * desc->d * sizeof(float);
      const Range wr[1] = {{ws, need}};
      const Range all[11] = {{q, tok}, {k, tok}, {v, tok}, {u, tok}, {S0, mat}, {A0, mat}, {n0, vec},
                             {out, tok}, {S_final, mat}, {A_final, mat}, {n_final, vec}};
      if (outputs_alias(wr, 1, all, 11)) return VLA_ERROR_INVALID_VALUE;
    }
  }
  if (!device_ok()) return VLA_ERROR_NO_DEVICE;
  if (path == VLA_PATH_CHUNK && ws == nullptr) {
    st = noalloc ? scratch_address(&ws)
                 : cached_workspace(vla::chunk_workspace_bytes(p, chunk),
                                    reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != VLA_SUCCESS) return st;
  }
  vla::StateIO sio;
  sio.S0 = S0;
  sio.A0 = A0;
  sio.n0 = n0;
  sio.S_final = S_final;
  sio.A_final = A_final;
  sio.n_final = n_final;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::optional<vla::ProfQuiet> quiet;  // no timing events on the allocation-free path
  if (noalloc) quiet.emplace();
  hipError_t err;
  if (path == VLA_PATH_SEQ)
    err = vla::launch_seq(p, q, k, v, u, out, sio, s);
  else if (path == VLA_PATH_DECODE)
    err = vla::launch_decode(p, q, k, v, u, out, sio, s);
  else
    err = vla::launch_chunk(p, chunk, q, k, v, u, out, sio, ws, s, !noalloc);
  return err == hipSuccess ? VLA_SUCCESS : VLA_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

vla_status_t vla_forward_state(const void *q, const void *k, const void *v, const void *u,
                               float lambda0, const float *S0, const float *A0, const float *n0,
                               void *out, float *S_final, float *A_final, float *n_final,
                               const vla_desc_t *desc, struct ihipStream_t *stream) {
  return forward_state_impl(q, k, v, u, lambda0, S0, A0, n0, out, S_final, A_final, n_final, desc,
                            stream, false);
}

vla_status_t vla_forward_state_noalloc(const void *q, const void *k, const void *v, const void *u,
                                       float lambda0, const float *S0, const float *A0,
                                       const float *n0, void *out, float *S_final, float *A_final,
                                       float *n_final, const vla_desc_t *desc,
                                       struct ihipStream_t *stream) {
  return forward_state_impl(q, k, v, u, lambda0, S0, A0, n0, out, S_final, A_final, n_final, desc,
                            stream, true);
}

vla_status_t vla_la_workspace_size(const vla_desc_t *desc, size_t *bytes) {
  if (bytes == nullptr) return VLA_ERROR_INVALID_VALUE;
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  if (desc->path != VLA_PATH_AUTO || (desc->chunk != 0 && desc->chunk != 64) ||
      desc->gain != VLA_GAIN_UNIT)
    return VLA_ERROR_NOT_SUPPORTED;
  *bytes = vla::la_workspace_bytes(make_problem(desc, 1.0f));
  return VLA_SUCCESS;
}

vla_status_t vla_linear_attention(const void *q, const void *k, const void *v, void *out,
                                  float *S_final, float *n_final, const vla_desc_t *desc,
                                  struct ihipStream_t *stream) {
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return VLA_ERROR_INVALID_VALUE;
  if (desc->path != VLA_PATH_AUTO || (desc->chunk != 0 && desc->chunk != 64) ||
      desc->gain != VLA_GAIN_UNIT)
    return VLA_ERROR_NOT_SUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(S_final) ||
      !aligned16(n_final))
    return VLA_ERROR_NOT_SUPPORTED;
  const vla::Problem p = make_problem(desc, 1.0f);
  const size_t need = vla::la_workspace_bytes(p);
  void *ws = nullptr;
  if (desc->workspace != nullptr) {
    if (desc->workspace_bytes < need) return VLA_ERROR_INVALID_VALUE;
    if (!aligned16(desc->workspace)) return VLA_ERROR_NOT_SUPPORTED;
    ws = desc->workspace;
  }
  {  // outputs (and a caller's workspace) overlap neither one another nor any input
    const size_t bh = static_cast<size_t>(desc->B * desc->H);
    const size_t tok = bh * desc->T * desc->d * (desc->dtype == VLA_DTYPE_F32 ? 4 : 2);
    const size_t mat = bh * desc->d * desc->d * sizeof(float);
    const size_t vec = bh * desc->d * sizeof(float);
    const Range outs[4] = {{out, tok}, {S_final, mat}, {n_final, vec}, {ws, need}};
    const Range ins[3] = {{q, tok}, {k, tok}, {v, tok}};
    if (outputs_alias(outs, 4, ins, 3)) return VLA_ERROR_INVALID_VALUE;
  }
  if (!device_ok()) return VLA_ERROR_NO_DEVICE;
  if (ws == nullptr) {
    st = cached_workspace(need, reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != VLA_SUCCESS) return st;
  }
  const hipError_t err = vla::launch_la(p, q, k, v, out, S_final, n_final, ws,
                                        reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? VLA_SUCCESS : VLA_ERROR_LAUNCH;
}

// The backward's segmentation: chunk 0 = one segment per stream (VLA_PATH_SEQ), else the
// chunked path's segments (VLA_PATH_CHUNK).  AUTO splits time whenever the split gives at least
// two segments per stream, at d = 128 only up to 128 streams.  Measured on MI355X (ms per call,
// time segments against one segment per stream): fp32, d = 32, 512 tokens: 0.91 / 1.86 at 256
// streams, 2.89 / 3.81 at 1024; bf16, 4096 tokens: 33.5 / 41.9 at 1024 streams (d = 64), 72.0 /
// 80.4 (d = 96); at d = 128 (2048 tokens) 8.1 / 13.3 at 128 streams but 15.8 / 13.4 at 256 (the
// segment passes add work, which pays only while one segment per stream leaves CUs idle).  The
// split gives one segment per stream, and so the same work as SEQ, once streams x T reaches
// about 2048 segments of the shortest length.
vla_status_t resolve_backward(const vla_desc_t *desc, const vla::Problem &p, int *chunk) {
  if (desc->gain != VLA_GAIN_UNIT) return VLA_ERROR_NOT_SUPPORTED;
  int c = desc->chunk;
  switch (desc->path) {
    case VLA_PATH_SEQ:
      *chunk = 0;
      return VLA_SUCCESS;
    case VLA_PATH_CHUNK:
      if (c == 0) c = vla::chunk_default(p);
      if (!vla::chunk_supported(p, c)) return VLA_ERROR_NOT_SUPPORTED;
      *chunk = c;
      return VLA_SUCCESS;
    case VLA_PATH_AUTO: {
      if (c == 0) c = vla::chunk_default(p);
      int64_t L = 0, P = 0;
      if ((p.d <= 96 || p.streams <= 128) && vla::chunk_supported(p, c))
        vla::chunk_segments(p, c, &L, &P);
      *chunk = P >= 2 ? c : 0;
      return VLA_SUCCESS;
    }
    default:
      return VLA_ERROR_NOT_SUPPORTED;
  }
}

vla_status_t vla_backward_workspace_size(const vla_desc_t *desc, size_t *bytes) {
  if (bytes == nullptr) return VLA_ERROR_INVALID_VALUE;
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  const vla::Problem p = make_problem(desc, 1.0f);
  int chunk = 0;
  st = resolve_backward(desc, p, &chunk);
  if (st != VLA_SUCCESS) return st;
  *bytes = vla::backward_workspace_bytes(p, chunk);
  return VLA_SUCCESS;
}

vla_status_t vla_backward(const void *q, const void *k, const void *v, const void *u,
                          float lambda0, const void *d_out, const float *dS_T, const float *dA_T,
                          const float *dn_T, float *dq, float *dk, float *dv, float *du,
                          float *dlambda0, const vla_desc_t *desc, struct ihipStream_t *stream) {
  vla_status_t st = check_desc(desc);
  if (st != VLA_SUCCESS) return st;
  if (q == nullptr || k == nullptr || v == nullptr || u == nullptr || d_out == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || du == nullptr)
    return VLA_ERROR_INVALID_VALUE;
  if (!(lambda0 > 0.0f) || !std::isfinite(lambda0)) return VLA_ERROR_INVALID_VALUE;
  const vla::Problem p = make_problem(desc, lambda0);
  int chunk = 0;
  st = resolve_backward(desc, p, &chunk);
  if (st != VLA_SUCCESS) return st;
  const void *ptrs[] = {q, k, v, u, d_out, dS_T, dA_T, dn_T, dq, dk, dv, du, dlambda0};
  for (const void *x : ptrs)
    if (!aligned16(x)) return VLA_ERROR_NOT_SUPPORTED;
  const size_t need = vla::backward_workspace_bytes(p, chunk);
  void *ws = nullptr;
  if (desc->workspace != nullptr) {
    if (desc->workspace_bytes < need) return VLA_ERROR_INVALID_VALUE;
    if (!aligned16(desc->workspace)) return VLA_ERROR_NOT_SUPPORTED;
    ws = desc->workspace;
  }
  {  // gradients (and a caller's workspace) overlap neither one another nor any input
    const size_t bh = static_cast<size_t>(desc->B * desc->H);
    const size_t tok = bh * desc->T * desc->d * (desc->dtype == VLA_DTYPE_F32 ? 4 : 2);
    const size_t g32 = bh * desc->T * desc->d * sizeof(float);
    const size_t mat = bh * desc->d * desc->d * sizeof(float);
    const size_t vec = bh * desc->d * sizeof(float);
    const Range outs[6] = {{dq, g32}, {dk, g32}, {dv, g32}, {du, g32}, {dlambda0, bh * sizeof(float)},
                           {ws, need}};
    const Range ins[8] = {{q, tok}, {k, tok}, {v, tok}, {u, tok}, {d_out, tok}, {dS_T, mat}, {dA_T, mat},
                          {dn_T, vec}};
    if (outputs_alias(outs, 6, ins, 8)) return VLA_ERROR_INVALID_VALUE;
  }
  if (!device_ok()) return VLA_ERROR_NO_DEVICE;
  if (ws == nullptr) {
    st = cached_workspace(need, reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != VLA_SUCCESS) return st;
  }
  vla::BackwardIO io{q, k, v, u, d_out, dS_T, dA_T, dn_T, dq, dk, dv, du, dlambda0};
  const hipError_t err = vla::launch_backward(p, chunk, io, ws, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? VLA_SUCCESS : VLA_ERROR_LAUNCH;
}

vla_status_t vla_forward(const void *q, const void *k, const void *v, const void *u,
                         float lambda0, void *out, float *S_final, float *A_final,
                         const vla_desc_t *desc, struct ihipStream_t *stream) {
  if (!(lambda0 > 0.0f) || !std::isfinite(lambda0)) {
    const vla_status_t st = check_desc(desc);
    return st != VLA_SUCCESS ? st : VLA_ERROR_INVALID_VALUE;
  }
  return vla_forward_state(q, k, v, u, lambda0, nullptr, nullptr, nullptr, out, S_final, A_final,
                           nullptr, desc, stream);
}

}  // extern "C"
