// fno_model.cpp - the full FNO2d network on top of the spectral-conv plan and
// the per-pixel kernels: lift -> n_layers x GELU(spectral + 1x1 + bias) ->
// projection, every step in the library's HIP kernels, activations in the
// storage dtype ping-ponging through buffers the model owns.
//
// The lift is folded into the first block (both are linear in the lifted
// field): one small kernel composes the first block's spectral weights,
// 1x1 weights and bias with the lift, and the first block then runs on the
// raw feature channels, so the lifted field is never written or read. Where
// the plans allow it (fp16 / bf16 on matrix-core planes, see fno_block2d)
// every block runs as fno_block2d: the 1x1 convolution, bias and GELU are
// applied in the inverse transform's row stage, so the spectral branch's
// output is never stored either; otherwise a block is the layer followed by
// the channel-mix kernel. The forward can be replayed from a HIP graph
// captured on the model's own stream.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <vector>

#include "../../include/fno.h"
#include "common.hpp"

using namespace fno;

struct fno_model2d_s {
  int B = 0, H = 0, W = 0, in_ch = 0, ch = 0, layers = 0, m1 = 0, m2 = 0, proj = 0, out_ch = 0;
  int dtype = 0, device = 0;
  fno_plan_t plan = nullptr;   // blocks 1.. (ch -> ch)
  fno_plan_t plan0 = nullptr;  // block 0 on the features (in_ch -> ch), lift folded in
  bool fused0 = false, fused = false;  // block 0 / the other blocks run as fno_block2d
  void *mem = nullptr;
  void *act[3] = {nullptr, nullptr, nullptr};
  void *wf = nullptr, *af = nullptr, *bf = nullptr;  // block 0's folded weights
  // graph replay: the captured forward and the pointers it was captured for
  bool graph = false;
  hipStream_t cap = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<const void *> key;
};

namespace {

size_t esize(int dtype) { return dtype == FNO_F32 ? 4 : 2; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

fno_status_t status_of(hipError_t e) {
  if (e == hipSuccess) return FNO_OK;
  return e == hipErrorOutOfMemory ? FNO_ERR_OUT_OF_MEMORY : FNO_ERR_DEVICE;
}

bool valid_dtype(fno_dtype_t d) { return d == FNO_F32 || d == FNO_F16 || d == FNO_BF16; }

}  // namespace

extern "C" {

fno_status_t fno_channel_mix(const void *x, const void *A, const void *bias, const void *add, void *y, int batch,
                             int c_in, int c_out, long pixels, int act, fno_dtype_t dtype, void *stream) {
  if (!x || !A || !y || batch < 1 || c_in < 1 || c_out < 1 || pixels < 1 || (act != 0 && act != 1) ||
      !valid_dtype(dtype))
    return FNO_ERR_INVALID_ARG;
  if (batch > 65535 || c_out > 65535 * 64) return FNO_ERR_UNSUPPORTED;
  if (c_in > kMixMaxIn) return FNO_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || (add && !aligned16(add))) return FNO_ERR_INVALID_ARG;
  const size_t es = esize(dtype);
  const size_t nx = (size_t)batch * c_in * pixels * es, ny = (size_t)batch * c_out * pixels * es;
  if (overlap(x, nx, y, ny) || (add && overlap(add, ny, y, ny) && add != y)) return FNO_ERR_INVALID_ARG;
  if (add == y) return FNO_ERR_INVALID_ARG;
  hipError_t e = launch_channel_mix(x, A, bias, add, y, batch, c_in, c_out, pixels, act, (int)dtype,
                                    (hipStream_t)stream);
  if (e == hipSuccess) e = hipGetLastError();
  return status_of(e);
}

fno_status_t fno_projection(const void *x, const void *Q1, const void *q1, const void *Q2, const void *q2, void *y,
                            int batch, int c_in, int hidden, int c_out, long pixels, fno_dtype_t dtype,
                            void *stream) {
  if (!x || !Q1 || !q1 || !Q2 || !q2 || !y || batch < 1 || c_in < 1 || hidden < 1 || c_out < 1 || pixels < 1 ||
      !valid_dtype(dtype))
    return FNO_ERR_INVALID_ARG;
  if (batch > 65535 || c_in > kProjMaxIn || hidden > kProjMaxHidden || c_out > kProjMaxOut)
    return FNO_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y)) return FNO_ERR_INVALID_ARG;
  const size_t es = esize(dtype);
  if (overlap(x, (size_t)batch * c_in * pixels * es, y, (size_t)batch * c_out * pixels * es))
    return FNO_ERR_INVALID_ARG;
  hipError_t e =
      launch_projection(x, Q1, q1, Q2, q2, y, batch, c_in, hidden, c_out, pixels, (int)dtype, (hipStream_t)stream);
  if (e == hipSuccess) e = hipGetLastError();
  return status_of(e);
}

fno_status_t fno_model2d_destroy(fno_model2d_t m) {
  if (!m) return FNO_OK;
  fno_status_t st = fno_plan_destroy(m->plan);
  if (fno_plan_destroy(m->plan0) != FNO_OK) st = FNO_ERR_DEVICE;
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (prev != m->device) (void)hipSetDevice(m->device);
  if (m->exec && hipGraphExecDestroy(m->exec) != hipSuccess) st = FNO_ERR_DEVICE;
  if (m->cap && hipStreamDestroy(m->cap) != hipSuccess) st = FNO_ERR_DEVICE;
  if (m->mem && hipFree(m->mem) != hipSuccess) st = FNO_ERR_DEVICE;
  if (prev >= 0 && prev != m->device) (void)hipSetDevice(prev);
  delete m;
  return st;
}

fno_status_t fno_model2d_create(fno_model2d_t *out, int batch, int height, int width, int in_channels,
                                int channels, int n_layers, int m1, int m2, int proj_channels, int out_channels,
                                fno_dtype_t dtype, int device) {
  if (!out) return FNO_ERR_INVALID_ARG;
  *out = nullptr;
  if (batch < 1 || height < 1 || width < 1 || in_channels < 1 || channels < 1 || n_layers < 0 ||
      proj_channels < 1 || out_channels < 1 || !valid_dtype(dtype) || device < 0)
    return FNO_ERR_INVALID_ARG;
  if (in_channels > kMixMaxIn || channels > kProjMaxIn || proj_channels > kProjMaxHidden ||
      out_channels > kProjMaxOut || n_layers > 1024)
    return FNO_ERR_UNSUPPORTED;
  fno_model2d_s *m = new (std::nothrow) fno_model2d_s();
  if (!m) return FNO_ERR_OUT_OF_MEMORY;
  m->B = batch;
  m->H = height;
  m->W = width;
  m->in_ch = in_channels;
  m->ch = channels;
  m->layers = n_layers;
  m->m1 = m1;
  m->m2 = m2;
  m->proj = proj_channels;
  m->out_ch = out_channels;
  m->dtype = (int)dtype;
  m->device = device;
  const int grid[2] = {height, width}, modes[2] = {m1, m2};
  fno_status_t st = fno_plan_create(&m->plan, 2, batch, channels, channels, grid, modes, dtype, device);
  if (st == FNO_OK && n_layers > 0)
    st = fno_plan_create(&m->plan0, 2, batch, in_channels, channels, grid, modes, dtype, device);
  if (st != FNO_OK) {
    fno_model2d_destroy(m);
    return st;
  }
  // block buffers now (allocation cannot be part of a captured graph);
  // a plan the fused block does not serve keeps the two-kernel block
  if (m->plan) {
    st = fno_block2d_prepare(m->plan);
    m->fused = st == FNO_OK;
    if (st != FNO_OK && st != FNO_ERR_UNSUPPORTED) {
      fno_model2d_destroy(m);
      return st;
    }
  }
  if (m->plan0) {
    st = fno_block2d_prepare(m->plan0);
    m->fused0 = st == FNO_OK;
    if (st != FNO_OK && st != FNO_ERR_UNSUPPORTED) {
      fno_model2d_destroy(m);
      return st;
    }
  }
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (prev != device) (void)hipSetDevice(device);
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t es = esize((int)dtype);
  const size_t one = al((size_t)batch * channels * height * width * es);
  const size_t K = (size_t)2 * m1 * m2;
  const size_t nwf = al(K * in_channels * channels * 2 * es), naf = al((size_t)channels * in_channels * es),
               nbf = al((size_t)channels * es);
  // the spectral branch's output buffer only for blocks that are not fused
  const int nact = ((n_layers >= 1 && !m->fused0) || (n_layers >= 2 && !m->fused)) ? 3 : 2;
  hipError_t e = hipMalloc(&m->mem, nact * one + nwf + naf + nbf);
  if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    m->mem = nullptr;
    fno_model2d_destroy(m);
    return status_of(e);
  }
  for (int i = 0; i < nact; ++i) m->act[i] = (char *)m->mem + i * one;
  m->wf = (char *)m->mem + nact * one;
  m->af = (char *)m->wf + nwf;
  m->bf = (char *)m->af + naf;
  *out = m;
  return FNO_OK;
}

// Queue the whole forward on `stream`.
static fno_status_t enqueue_forward(fno_model2d_t m, const void *features, const void *const *params, void *out,
                                    void *stream) {
  const long P = (long)m->H * m->W;
  const fno_dtype_t dt = (fno_dtype_t)m->dtype;
  fno_status_t st = FNO_OK;
  int cur = 0, l0 = 0;
  if (m->layers > 0) {
    // block 0 on the raw features with the lift folded in: v1 lands in act[1]
    const void *const *lp = params + 2;
    hipError_t e = launch_lift_fold(params[0], params[1], lp[0], lp[1], lp[2], m->wf, m->af, m->bf,
                                    2 * m->m1 * m->m2, m->in_ch, m->ch, m->dtype, (hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
    st = status_of(e);
    if (st == FNO_OK && m->fused0) {
      st = fno_block2d(m->plan0, features, m->wf, m->af, m->bf, 1, m->act[1], stream);
    } else if (st == FNO_OK) {
      st = fno_spectral_conv2d(m->plan0, features, m->wf, m->act[2], stream);
      if (st == FNO_OK)
        st = fno_channel_mix(features, m->af, m->bf, m->act[2], m->act[1], m->B, m->in_ch, m->ch, P, 1, dt, stream);
    }
    cur = 1;
    l0 = 1;
  } else {
    st = fno_channel_mix(features, params[0], params[1], nullptr, m->act[0], m->B, m->in_ch, m->ch, P, 0, dt,
                         stream);
  }
  for (int l = l0; l < m->layers && st == FNO_OK; ++l) {
    const void *const *lp = params + 2 + 3 * l;
    const int nxt = cur == 0 ? 1 : 0;
    if (m->fused) {
      st = fno_block2d(m->plan, m->act[cur], lp[0], lp[1], lp[2], 1, m->act[nxt], stream);
    } else {
      st = fno_spectral_conv2d(m->plan, m->act[cur], lp[0], m->act[2], stream);
      if (st == FNO_OK)
        st = fno_channel_mix(m->act[cur], lp[1], lp[2], m->act[2], m->act[nxt], m->B, m->ch, m->ch, P, 1, dt, stream);
    }
    cur = nxt;
  }
  if (st == FNO_OK) {
    const void *const *pp = params + 2 + 3 * m->layers;
    st = fno_projection(m->act[cur], pp[0], pp[1], pp[2], pp[3], out, m->B, m->ch, m->proj, m->out_ch, P, dt,
                        stream);
  }
  return st;
}

// Capture the forward for these pointers into a graph on the model's stream
// (replacing an earlier capture).
static fno_status_t capture_forward(fno_model2d_t m, const void *features, const void *const *params, void *out) {
  if (!m->cap && hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking) != hipSuccess) return FNO_ERR_DEVICE;
  if (hipStreamBeginCapture(m->cap, hipStreamCaptureModeThreadLocal) != hipSuccess) return FNO_ERR_DEVICE;
  const fno_status_t st = enqueue_forward(m, features, params, out, m->cap);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(m->cap, &g);
  if (st != FNO_OK || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    return st != FNO_OK ? st : FNO_ERR_DEVICE;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (ei != hipSuccess) return FNO_ERR_DEVICE;
  if (m->exec) (void)hipGraphExecDestroy(m->exec);
  m->exec = exec;
  return FNO_OK;
}

fno_status_t fno_model2d_set_graph(fno_model2d_t m, int on) {
  if (!m || (on != 0 && on != 1)) return FNO_ERR_INVALID_ARG;
  m->graph = on != 0;
  return FNO_OK;
}

fno_status_t fno_model2d_forward(fno_model2d_t m, const void *features, const void *const *params, void *out,
                                 void *stream) {
  if (!m || !features || !params || !out) return FNO_ERR_INVALID_ARG;
  const int np = 2 + 3 * m->layers + 4;
  for (int i = 0; i < np; ++i)
    if (!params[i]) return FNO_ERR_INVALID_ARG;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return FNO_ERR_DEVICE;
  if (prev != m->device && hipSetDevice(m->device) != hipSuccess) return FNO_ERR_DEVICE;
  fno_status_t st = FNO_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) st = FNO_ERR_DEVICE;
  if (st == FNO_OK && m->graph && cs == hipStreamCaptureStatusNone) {
    std::vector<const void *> key{features, out};
    key.insert(key.end(), params, params + np);
    if (!m->exec || key != m->key) {
      st = capture_forward(m, features, params, out);
      m->key = st == FNO_OK ? key : std::vector<const void *>();
    }
    if (st == FNO_OK && hipGraphLaunch(m->exec, (hipStream_t)stream) != hipSuccess) st = FNO_ERR_DEVICE;
  } else if (st == FNO_OK) {
    st = enqueue_forward(m, features, params, out, stream);
  }
  if (prev != m->device) (void)hipSetDevice(prev);
  return st;
}

}  // extern "C"
