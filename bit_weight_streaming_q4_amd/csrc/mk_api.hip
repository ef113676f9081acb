// mk_api.hip — the C ABI of libmk (declared in include/mk.h): host-side
// argument validation, workspace carving, block packing, and the launches.
// Every entry point validates before touching the GPU; on error it enqueues
// nothing, returns a negative status and records a thread-local message.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <math.h>
#include <mutex>
#include <vector>

#include "mk.h"
#include "mk_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace

int mk::set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

// Workspace of mk_qgemv_rows_noalloc: one array per GPU, held until the
// process ends.  Host code never uses this name as an address (in host code
// it is only a stand-in for the symbol); scratch_device_ptr() returns the
// device address that hipGetSymbolAddress gives for the current device.
__device__ __attribute__((aligned(256))) uint8_t scratch[MK_NOALLOC_SCRATCH_BYTES];

namespace {

int ok() {
  g_err[0] = '\0';
  return MK_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

std::mutex g_dev_mu;
std::vector<int> g_cu;  // CU count per device (0 = not queried)

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_cu.size() <= dev) g_cu.resize(dev + 1, 0);
  if (g_cu[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 256;
    g_cu[dev] = p.multiProcessorCount;
  }
  return g_cu[dev];
}

hipStream_t S(void* s) { return (hipStream_t)s; }

std::mutex g_scratch_mu;
std::vector<void*> g_scratch;  // device address of `scratch` per device (null = not looked up)

// The current device's copy of `scratch`, looked up once per device with
// that device current.
int scratch_device_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MK_ERR_DEVICE, "no current HIP device");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MK_ERR_DEVICE, "scratch array address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MK_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MK_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_q4k(const mk_q4k* W, const char* name) {
  if (!W || !W->blocks) return fail(MK_ERR_ARG, "%s: null weight", name);
  if (W->n_out <= 0 || W->n_in <= 0) return fail(MK_ERR_SHAPE, "%s: empty matrix %d x %d", name, W->n_out, W->n_in);
  if (W->n_in % 256) return fail(MK_ERR_SHAPE, "%s: n_in = %d is not a multiple of 256", name, W->n_in);
  if (!aligned(W->blocks, 256)) return fail(MK_ERR_ALIGN, "%s: blocks not 256-B aligned", name);
  return MK_OK;
}

int check_T(int T) {
  if (T < 1 || T > MK_T_MAX) return fail(MK_ERR_RANGE, "T = %d outside 1..%d", T, MK_T_MAX);
  return MK_OK;
}

int check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(MK_ERR_ARG, "%s is null", name);
  if (!aligned(p, align)) return fail(MK_ERR_ALIGN, "%s not %zu-B aligned", name, align);
  return MK_OK;
}

// Workspace of one quantized activation record (a8 + interleaved scales).
size_t qact_bytes(int T, int K) { return align256((size_t)T * K) + align256((size_t)(K / 32) * mk::kTPadHost * 8); }

mk::QActBuf carve_qact(uint8_t*& p, int T, int K) {
  mk::QActBuf q;
  q.a8 = (int8_t*)p;
  p += align256((size_t)T * K);
  q.ssg = (float2*)p;
  p += align256((size_t)(K / 32) * mk::kTPadHost * 8);
  q.K = K;
  q.T = T;
  return q;
}

// The automatic choice follows the measured 5120 x 5120 crossover: the dot4
// launches up to kDot4MaxTAuto rows, the streaming engines above.
int pick_path(int path, int T) {
  if (path != MK_PATH_AUTO) return path;
  return T <= mk::kDot4MaxTAuto ? MK_PATH_DOT4 : MK_PATH_STEP;
}

// The FFN on the dot4 GEMV launches (fewer than kFfnStreamMinT rows): x's
// activation rows, tile counters (gate/up, then down), the gate/up partials,
// h's activation rows (written by the gate/up tile epilogues), the down
// partials.
size_t ffn_std_workspace(int T, int H, int F) {
  const int cu = device_cu_count();
  const mk::GemvPlan pg = mk::plan_gemv(T, F, H, 2, cu);
  const mk::GemvPlan pd = mk::plan_gemv(T, H, F, 1, cu);
  return qact_bytes(T, H) + align256((size_t)(pg.ntiles + pd.ntiles) * 4) + align256(pg.partial_elems * 4) +
         qact_bytes(T, F) + align256(pd.partial_elems * 4);
}

int ffn_std(const mk_q4k* gate, const mk_q4k* up, const mk_q4k* down, const float* x, int T, float* y, float* h_out,
            void* ws, void* stream) {
  const int H = gate->n_in, F = gate->n_out;
  const int cu = device_cu_count();
  const mk::GemvPlan pg = mk::plan_gemv(T, F, H, 2, cu);
  const mk::GemvPlan pd = mk::plan_gemv(T, H, F, 1, cu);
  uint8_t* wp = (uint8_t*)ws;
  const mk::QActBuf ax = carve_qact(wp, T, H);
  unsigned* tickets = (unsigned*)wp;
  wp += align256((size_t)(pg.ntiles + pd.ntiles) * 4);
  float* part_gu = (float*)wp;
  wp += align256(pg.partial_elems * 4);
  const mk::QActBuf ah = carve_qact(wp, T, F);
  float* part_d = (float*)wp;
  const int eng = MK_PATH_DOT4;
  hipStream_t st = S(stream);
  hipError_t e = mk::launch_quantize(x, T, H, ax.a8, nullptr, nullptr, ax.ssg, tickets, pg.ntiles + pd.ntiles, st);
  if (e != hipSuccess) return launch_status(e, "quantize x");
  const uint8_t* wgu[2] = {(const uint8_t*)gate->blocks, (const uint8_t*)up->blocks};
  const mk::GemvEpi eg = {tickets, mk::kEpiSiluQ8, F, h_out, ah.a8, ah.ssg};
  if ((e = mk::launch_gemv(wgu, pg, ax, eng, part_gu, eg, st)) != hipSuccess) return launch_status(e, "gate/up");
  const uint8_t* wd[2] = {(const uint8_t*)down->blocks, nullptr};
  const mk::GemvEpi ed = {tickets + pg.ntiles, mk::kEpiStore, H, y, nullptr, nullptr};
  return launch_status(mk::launch_gemv(wd, pd, ah, eng, part_d, ed, st), "down");
}

}  // namespace

extern "C" {

const char* mk_status_string(int status) {
  switch (status) {
    case MK_OK: return "ok";
    case MK_ERR_ARG: return "invalid argument";
    case MK_ERR_SHAPE: return "unsupported shape";
    case MK_ERR_ALIGN: return "misaligned pointer";
    case MK_ERR_RANGE: return "value out of range";
    case MK_ERR_WORKSPACE: return "workspace too small";
    case MK_ERR_LAUNCH: return "HIP launch failed";
    case MK_ERR_COOP: return "cooperative launch unavailable";
    case MK_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* mk_last_error(void) { return g_err; }

int mk_version(void) { return 1; }

int mk_init(int device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(MK_ERR_DEVICE, "no HIP device");
  if (device < 0 || device >= n) return fail(MK_ERR_RANGE, "device %d outside 0..%d", device, n - 1);
  if (hipSetDevice(device) != hipSuccess) return fail(MK_ERR_DEVICE, "hipSetDevice(%d) failed", device);
  device_cu_count();
  void* p;
  int r;
  if ((r = scratch_device_ptr(&p))) return r;
  return ok();
}

// ------------------------------------------------------------------ packing
size_t mk_q4k_bytes(int32_t n_out, int32_t n_in) {
  if (n_out <= 0 || n_in <= 0 || n_in % 256) return 0;
  return (size_t)((n_out + 63) / 64) * (size_t)(n_in / 256) * mk::kUnitBytesHost;
}

int mk_q4k_pack(const uint16_t* h_d, const uint16_t* h_dmin, const uint8_t* h_sc, const uint8_t* h_m,
                const uint8_t* h_q, int32_t n_out, int32_t n_in, int32_t r0, int32_t r1, void* h_blocks) {
  if (!h_d || !h_dmin || !h_sc || !h_m || !h_q || !h_blocks) return fail(MK_ERR_ARG, "pack: null pointer");
  if (n_out <= 0 || n_in <= 0 || n_in % 256) return fail(MK_ERR_SHAPE, "pack: bad shape %d x %d", n_out, n_in);
  if (r0 < 0 || r1 > n_out || r0 >= r1 || r0 % 64 || (r1 % 64 && r1 != n_out))
    return fail(MK_ERR_RANGE, "pack: row slice [%d, %d) must be tile aligned within %d", r0, r1, n_out);
  const int nsb = n_in / 256;
  const int rows = r1 - r0;
  for (size_t i = 0; i < (size_t)rows * nsb * 8; ++i)
    if (h_sc[i] > 63 || h_m[i] > 63) return fail(MK_ERR_RANGE, "pack: sc/m value above 63");
  for (size_t i = 0; i < (size_t)rows * n_in; ++i)
    if (h_q[i] > 15) return fail(MK_ERR_RANGE, "pack: code above 15");
  uint8_t* out = (uint8_t*)h_blocks;
  const int t0 = r0 / 64, t1 = (r1 + 63) / 64;
  memset(out, 0, (size_t)(t1 - t0) * nsb * mk::kUnitBytesHost);
  for (int r = r0; r < r1; ++r) {
    const int tile = r / 64 - t0, rr = r % 64;
    const size_t lr = (size_t)(r - r0);
    for (int b = 0; b < nsb; ++b) {
      uint8_t* u = out + ((size_t)tile * nsb + b) * mk::kUnitBytesHost;
      uint8_t* h = u + rr * 16;
      const uint16_t d = h_d[lr * nsb + b], dm = h_dmin[lr * nsb + b];
      h[0] = d & 0xff;
      h[1] = d >> 8;
      h[2] = dm & 0xff;
      h[3] = dm >> 8;
      const uint8_t* sc = h_sc + (lr * nsb + b) * 8;
      const uint8_t* m = h_m + (lr * nsb + b) * 8;
      for (int j = 0; j < 8; ++j) h[4 + j] = (uint8_t)(sc[j] | ((m[j] >> 4) << 6));
      for (int i = 0; i < 4; ++i) h[12 + i] = (uint8_t)((m[i] & 15) | ((m[i + 4] & 15) << 4));
      const uint8_t* q = h_q + lr * n_in + (size_t)b * 256;
      for (int j = 0; j < 8; ++j) {
        uint8_t* c = u + 1024 + j * 1024 + rr * 16;
        for (int w = 0; w < 4; ++w)
          for (int i = 0; i < 4; ++i)
            c[4 * w + i] = (uint8_t)(q[32 * j + 8 * w + i] | (q[32 * j + 8 * w + 4 + i] << 4));
      }
    }
  }
  return ok();
}

int mk_q4k_unpack(const void* h_blocks, int32_t n_out, int32_t n_in, uint16_t* h_d, uint16_t* h_dmin,
                  uint8_t* h_sc, uint8_t* h_m, uint8_t* h_q) {
  if (!h_blocks || !h_d || !h_dmin || !h_sc || !h_m || !h_q) return fail(MK_ERR_ARG, "unpack: null pointer");
  if (n_out <= 0 || n_in <= 0 || n_in % 256) return fail(MK_ERR_SHAPE, "unpack: bad shape");
  const int nsb = n_in / 256;
  const uint8_t* in = (const uint8_t*)h_blocks;
  for (int r = 0; r < n_out; ++r) {
    const int tile = r / 64, rr = r % 64;
    for (int b = 0; b < nsb; ++b) {
      const uint8_t* u = in + ((size_t)tile * nsb + b) * mk::kUnitBytesHost;
      const uint8_t* h = u + rr * 16;
      h_d[(size_t)r * nsb + b] = (uint16_t)(h[0] | (h[1] << 8));
      h_dmin[(size_t)r * nsb + b] = (uint16_t)(h[2] | (h[3] << 8));
      uint8_t* sc = h_sc + ((size_t)r * nsb + b) * 8;
      uint8_t* m = h_m + ((size_t)r * nsb + b) * 8;
      for (int j = 0; j < 8; ++j) {
        sc[j] = h[4 + j] & 63;
        const int lo = j < 4 ? (h[12 + j] & 15) : (h[12 + j - 4] >> 4);
        m[j] = (uint8_t)(lo | ((h[4 + j] >> 6) << 4));
      }
      uint8_t* q = h_q + (size_t)r * n_in + (size_t)b * 256;
      for (int j = 0; j < 8; ++j) {
        const uint8_t* c = u + 1024 + j * 1024 + rr * 16;
        for (int w = 0; w < 4; ++w)
          for (int i = 0; i < 4; ++i) {
            q[32 * j + 8 * w + i] = c[4 * w + i] & 15;
            q[32 * j + 8 * w + 4 + i] = c[4 * w + i] >> 4;
          }
      }
    }
  }
  return ok();
}

// ------------------------------------------------------------------ quantizer
int mk_quantize_rows(const float* x, int32_t T, int32_t K, int8_t* a8, float* s, int32_t* gsum, void* stream) {
  int r;
  if ((r = check_T(T))) return r;
  if (K <= 0 || K % 32) return fail(MK_ERR_SHAPE, "quantize: K = %d not a positive multiple of 32", K);
  if ((r = check_ptr(x, "x")) || (r = check_ptr(a8, "a8")) || (r = check_ptr(s, "s")) ||
      (r = check_ptr(gsum, "gsum")))
    return r;
  return launch_status(mk::launch_quantize(x, T, K, a8, s, gsum, nullptr, nullptr, 0, S(stream)), "quantize");
}

// ------------------------------------------------------------------ GEMV
// Workspace: quantized activation rows, tile counters, block partials.
size_t mk_qgemv_rows_workspace(int32_t T, int32_t n_out, int32_t n_in) {
  if (T < 1 || T > MK_T_MAX || n_out <= 0 || n_in <= 0 || n_in % 256) return 0;
  const mk::GemvPlan p = mk::plan_gemv(T, n_out, n_in, 1, device_cu_count());
  const size_t std_path = qact_bytes(T, n_in) + align256((size_t)p.ntiles * 4) + align256(p.partial_elems * 4);
  const size_t step_path = mk::engine_gemv_workspace(T, n_out, n_in, device_cu_count());
  return std_path > step_path ? std_path : step_path;
}

int mk_qgemv_rows_ex(const mk_q4k* W, const float* x, int32_t T, float* y, int32_t path, void* ws,
                     size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_q4k(W, "W")) || (r = check_T(T)) || (r = check_ptr(x, "x")) || (r = check_ptr(y, "y")))
    return r;
  if (path < MK_PATH_AUTO || path > MK_PATH_STEP) return fail(MK_ERR_ARG, "unknown path %d", path);
  const int eng = pick_path(path, T);
  if (eng == MK_PATH_STEP) {
    const size_t need = mk_qgemv_rows_workspace(T, W->n_out, W->n_in);
    if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if ((r = check_ptr(ws, "workspace", 256))) return r;
    return launch_status(mk::launch_engine_gemv((const uint8_t*)W->blocks, W->n_out, W->n_in, x, T, y, (uint8_t*)ws,
                                                 device_cu_count(), S(stream)),
                         "step-engine gemv");
  }
  if (eng == MK_PATH_DOT4 && T > mk::kDot4MaxT)
    return fail(MK_ERR_RANGE, "dot4 path supports T <= %d (T = %d)", mk::kDot4MaxT, T);
  const size_t need = mk_qgemv_rows_workspace(T, W->n_out, W->n_in);
  if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  const mk::GemvPlan p = mk::plan_gemv(T, W->n_out, W->n_in, 1, device_cu_count());
  uint8_t* wp = (uint8_t*)ws;
  const mk::QActBuf act = carve_qact(wp, T, W->n_in);
  unsigned* tickets = (unsigned*)wp;
  wp += align256((size_t)p.ntiles * 4);
  float* partial = (float*)wp;
  hipError_t e = mk::launch_quantize(x, T, W->n_in, act.a8, nullptr, nullptr, act.ssg, tickets, p.ntiles, S(stream));
  if (e != hipSuccess) return launch_status(e, "quantize");
  const uint8_t* wb[2] = {(const uint8_t*)W->blocks, nullptr};
  const mk::GemvEpi epi = {tickets, mk::kEpiStore, W->n_out, y, nullptr, nullptr};
  return launch_status(mk::launch_gemv(wb, p, act, eng, partial, epi, S(stream)), "gemv");
}

int mk_qgemv_rows(const mk_q4k* W, const float* x, int32_t T, float* y, void* ws, size_t ws_bytes, void* stream) {
  return mk_qgemv_rows_ex(W, x, T, y, MK_PATH_AUTO, ws, ws_bytes, stream);
}

int mk_qgemv_rows_noalloc(const mk_q4k* W, const float* x, int32_t T, float* y, int32_t path, void* stream) {
  int r;
  if ((r = check_q4k(W, "W")) || (r = check_T(T))) return r;
  const size_t need = mk_qgemv_rows_workspace(T, W->n_out, W->n_in);
  if (need > MK_NOALLOC_SCRATCH_BYTES)
    return fail(MK_ERR_WORKSPACE, "noalloc: a %d x %d GEMV at T = %d needs %zu bytes of workspace, above the %u-byte "
                "scratch array", W->n_out, W->n_in, T, need, (unsigned)MK_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((r = scratch_device_ptr(&ws))) return r;
  return mk_qgemv_rows_ex(W, x, T, y, path, ws, MK_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------------ FFN
// From kFfnStreamMinT rows the streaming engines (mk_step.hip; workspace:
// x's and h's records, the tickets of both stages, the gate/up and down
// partials), below them the dot4 launches (ffn_std).
size_t mk_ffn_rows_workspace(int32_t T, int32_t H, int32_t F) {
  if (T < 1 || T > MK_T_MAX || H <= 0 || F <= 0 || H % 256 || F % 256) return 0;
  return T < mk::kFfnStreamMinT ? ffn_std_workspace(T, H, F) : mk::engine_ffn_workspace(T, H, F, device_cu_count());
}

int mk_ffn_rows(const mk_q4k* gate, const mk_q4k* up, const mk_q4k* down, const float* x, int32_t T, float* y,
                float* h_out, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_q4k(gate, "gate")) || (r = check_q4k(up, "up")) || (r = check_q4k(down, "down"))) return r;
  if ((r = check_T(T)) || (r = check_ptr(x, "x")) || (r = check_ptr(y, "y"))) return r;
  if (h_out && (r = check_ptr(h_out, "h_out"))) return r;
  const int H = gate->n_in, F = gate->n_out;
  if (up->n_in != H || up->n_out != F || down->n_in != F || down->n_out != H)
    return fail(MK_ERR_SHAPE, "ffn: shapes gate %dx%d up %dx%d down %dx%d do not chain", gate->n_out, gate->n_in,
                up->n_out, up->n_in, down->n_out, down->n_in);
  if (F % 256) return fail(MK_ERR_SHAPE, "ffn: F = %d not a multiple of 256", F);
  const size_t need = mk_ffn_rows_workspace(T, H, F);
  if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  if (T < mk::kFfnStreamMinT) return ffn_std(gate, up, down, x, T, y, h_out, ws, stream);
  return launch_status(mk::launch_engine_ffn((const uint8_t*)gate->blocks, (const uint8_t*)up->blocks,
                                              (const uint8_t*)down->blocks, H, F, x, T, y, h_out, (uint8_t*)ws,
                                              device_cu_count(), S(stream)),
                       "ffn");
}

// ------------------------------------------------------------------ lm_head
size_t mk_lmhead_verify_workspace(int32_t V, int32_t H, int32_t T) {
  if (V <= 0 || H <= 0 || H % 64 || T < 1 || T > MK_T_MAX) return 0;
  return mk::lm_workspace_bytes(V, H);
}

static int check_groups(const int32_t* gs, int G, int T, std::vector<int32_t>& out) {
  if (!gs) {
    if (G != 1) return fail(MK_ERR_ARG, "h_group_start is null but G = %d", G);
    out = {0, T};
    return MK_OK;
  }
  if (G < 1 || G > MK_LM_MAX_G || G > T) return fail(MK_ERR_RANGE, "G = %d outside 1..min(T, %d)", G, MK_LM_MAX_G);
  if (gs[0] != 0 || gs[G] != T) return fail(MK_ERR_RANGE, "group starts must run from 0 to T");
  for (int g = 0; g < G; ++g)
    if (gs[g + 1] <= gs[g]) return fail(MK_ERR_RANGE, "group %d is empty", g);
  out.assign(gs, gs + G + 1);
  return MK_OK;
}

int mk_lmhead_verify(const uint16_t* W_f16, int32_t V, int32_t H, const float* hid, int32_t T,
                     const int32_t* h_group_start, int32_t G, const int32_t* drafts, int32_t* argmax,
                     int32_t* n_acc, int32_t* tokens, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_T(T))) return r;
  if (V <= 0 || H <= 0 || H % 64) return fail(MK_ERR_SHAPE, "lm_head: V = %d, H = %d (H % 64 == 0)", V, H);
  if ((r = check_ptr(W_f16, "W")) || (r = check_ptr(hid, "hid")) || (r = check_ptr(argmax, "argmax", 4)) ||
      (r = check_ptr(n_acc, "n_acc", 4)) || (r = check_ptr(tokens, "tokens", 4)))
    return r;
  std::vector<int32_t> gs;
  if ((r = check_groups(h_group_start, G, T, gs))) return r;
  if (T > G && (r = check_ptr(drafts, "drafts", 4))) return r;
  const size_t need = mk_lmhead_verify_workspace(V, H, T);
  if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  return launch_status(mk::launch_lmhead(W_f16, V, H, hid, T, gs.data(), G, drafts, argmax, n_acc, tokens, ws,
                                         device_cu_count(), S(stream)),
                       "lm_head");
}

// ------------------------------------------------------------------ sampling-mode verify
// Workspace: the lm_head stream's (ticket, fragments, block winners), the
// rows' prescale exponents, every logit [T][V], the candidates [T][32] x 2.
size_t mk_lmhead_sample_workspace(int32_t V, int32_t H, int32_t T) {
  if (V <= 0 || V > mk::kSampleMaxVocab || H <= 0 || H % 64 || T < 1 || T > MK_T_MAX) return 0;
  return mk::lm_workspace_bytes(V, H) + 256 + align256((size_t)T * V * 4) + 2 * align256((size_t)T * mk::kTopKMax * 4) +
         align256(mk::sample_part_bytes(V, T));
}

int mk_lmhead_sample(const uint16_t* W_f16, int32_t V, int32_t H, const float* hid, int32_t T,
                     const int32_t* h_group_start, int32_t G, const int32_t* drafts, int32_t top_k, float temperature,
                     const float* u_acc, const float* u_samp, int32_t* topk_idx, float* topk_logit, int32_t* n_acc,
                     int32_t* tokens, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_T(T))) return r;
  if (V <= 0 || V > mk::kSampleMaxVocab || H <= 0 || H % 64)
    return fail(MK_ERR_SHAPE, "sample: V = %d (at most %d), H = %d (H %% 64 == 0)", V, mk::kSampleMaxVocab, H);
  if (top_k < 1 || top_k > mk::kTopKMax) return fail(MK_ERR_RANGE, "sample: top_k = %d outside 1..%d", top_k, mk::kTopKMax);
  if (!(temperature > 0.0f) || !(temperature < 3.0e38f))
    return fail(MK_ERR_RANGE, "sample: temperature %g is not a positive finite value", (double)temperature);
  if ((r = check_ptr(W_f16, "W")) || (r = check_ptr(hid, "hid")) || (r = check_ptr(u_acc, "u_acc", 4)) ||
      (r = check_ptr(u_samp, "u_samp", 4)) || (r = check_ptr(n_acc, "n_acc", 4)) || (r = check_ptr(tokens, "tokens", 4)))
    return r;
  if (topk_idx && (r = check_ptr(topk_idx, "topk_idx", 4))) return r;
  if (topk_logit && (r = check_ptr(topk_logit, "topk_logit", 4))) return r;
  std::vector<int32_t> gs;
  if ((r = check_groups(h_group_start, G, T, gs))) return r;
  if (T > G && (r = check_ptr(drafts, "drafts", 4))) return r;
  const size_t need = mk_lmhead_sample_workspace(V, H, T);
  if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  uint8_t* p = (uint8_t*)ws;
  void* lm_ws = p;
  p += mk::lm_workspace_bytes(V, H);
  int* row_exp = (int*)p;
  p += 256;
  float* logits = (float*)p;
  p += align256((size_t)T * V * 4);
  int32_t* cidx = topk_idx ? topk_idx : (int32_t*)p;
  p += align256((size_t)T * mk::kTopKMax * 4);
  float* cval = topk_logit ? topk_logit : (float*)p;
  p += align256((size_t)T * mk::kTopKMax * 4);
  void* part = p;
  hipError_t e = mk::launch_lm_stream(W_f16, V, H, hid, T, gs.data(), G, drafts, nullptr, nullptr, nullptr, lm_ws,
                                      device_cu_count(), S(stream), logits, row_exp);
  if (e != hipSuccess) return launch_status(e, "sample: lm_head");
  mk::SampleArgs a = {};
  a.logits = logits;
  a.row_exp = row_exp;
  a.V = V;
  a.T = T;
  a.k = top_k;
  a.cand_idx = cidx;
  a.cand_val = cval;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  a.drafts = drafts;
  a.temperature = temperature;
  a.u_acc = u_acc;
  a.u_samp = u_samp;
  a.n_acc = n_acc;
  a.tokens = tokens;
  return launch_status(mk::launch_sample(a, part, S(stream)), "sample");
}

// ------------------------------------------------------------------ MTP draft loop
namespace {

int check_mtp(const mk_mtp* m, int32_t* H, int32_t* F) {
  int r;
  if (!m) return fail(MK_ERR_ARG, "mtp: null head");
  if ((r = check_q4k(&m->fc, "mtp fc")) || (r = check_q4k(&m->gate, "mtp gate")) ||
      (r = check_q4k(&m->up, "mtp up")) || (r = check_q4k(&m->down, "mtp down")))
    return r;
  *H = m->fc.n_out;
  *F = m->gate.n_out;
  if (*H % 256 || m->fc.n_in != 2 * *H || m->gate.n_in != *H || m->up.n_out != *F || m->up.n_in != *H ||
      m->down.n_out != *H || m->down.n_in != *F)
    return fail(MK_ERR_SHAPE, "mtp: fc must be H x 2H (H %% 256 == 0), gate/up F x H, down H x F");
  return MK_OK;
}

struct MtpLayout {
  size_t z, u, a, y, xp, prev, hid, dead, lmi, gemv, ffn, lm, total;
  size_t ws_gemv, ws_ffn, ws_lm;
};

MtpLayout mtp_layout(int H, int F, int V_draft, int T, int G) {
  MtpLayout y;
  size_t o = 0;
  auto take = [&](size_t n) { const size_t at = o; o += align256(n); return at; };
  y.z = take((size_t)T * 2 * H * 4);
  y.u = take((size_t)T * H * 4);
  y.a = take((size_t)T * H * 4);
  y.y = take((size_t)T * H * 4);
  y.xp = take((size_t)T * H * 4);
  y.prev = take((size_t)G * H * 4);
  y.hid = take((size_t)G * H * 4);
  y.dead = take((size_t)G * 4);
  y.lmi = take((size_t)2 * G * 4);
  y.ws_gemv = std::max(mk_qgemv_rows_workspace(T, H, 2 * H), mk_qgemv_rows_workspace(G, H, 2 * H));
  y.ws_ffn = std::max(mk_ffn_rows_workspace(T, H, F), mk_ffn_rows_workspace(G, H, F));
  y.ws_lm = mk::lm_workspace_bytes(V_draft, H);
  y.gemv = take(y.ws_gemv);
  y.ffn = take(y.ws_ffn);
  y.lm = take(y.ws_lm);
  y.total = o;
  return y;
}

}  // namespace

size_t mk_mtp_draft_workspace(const mk_mtp* m, int32_t V_draft, int32_t T, int32_t G) {
  int32_t H, F;
  if (check_mtp(m, &H, &F) || V_draft <= 0 || T < 1 || T > MK_T_MAX || G < 1 || G > T || G > MK_LM_MAX_G) return 0;
  return mtp_layout(H, F, V_draft, T, G).total;
}

int mk_mtp_draft(const mk_mtp* m, const uint16_t* embed_f16, int32_t V, int32_t V_draft, const float* hidden,
                 int32_t T, const int32_t* h_group_start, int32_t G, const int32_t* tokens, const int32_t* n_acc,
                 int32_t n_draft, int32_t* drafts, float* trace, void* ws, size_t ws_bytes, void* stream) {
  int r;
  int32_t H, F;
  if ((r = check_mtp(m, &H, &F)) || (r = check_T(T))) return r;
  if (V <= 0 || V_draft <= 0 || V_draft > V) return fail(MK_ERR_RANGE, "mtp: V_draft = %d outside 1..V (%d)", V_draft, V);
  if (n_draft < 1 || n_draft > MK_T_MAX) return fail(MK_ERR_RANGE, "mtp: n_draft = %d outside 1..%d", n_draft, MK_T_MAX);
  if ((r = check_ptr(embed_f16, "embed")) || (r = check_ptr(hidden, "hidden")) || (r = check_ptr(tokens, "tokens", 4)) ||
      (r = check_ptr(n_acc, "n_acc", 4)) || (r = check_ptr(drafts, "drafts", 4)))
    return r;
  if (trace && (r = check_ptr(trace, "trace"))) return r;
  std::vector<int32_t> gs;
  if ((r = check_groups(h_group_start, G, T, gs))) return r;
  const MtpLayout y = mtp_layout(H, F, V_draft, T, G);
  if (!ws || ws_bytes < y.total) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, y.total);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  uint8_t* w8 = (uint8_t*)ws;
  mk::MtpArgs a = {};
  a.embed = embed_f16;
  a.V = V;
  a.H = H;
  a.T = T;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  a.hidden = hidden;
  a.tokens = tokens;
  a.n_acc = n_acc;
  a.drafts = drafts;
  a.z = (float*)(w8 + y.z);
  a.u = (float*)(w8 + y.u);
  a.y = (float*)(w8 + y.y);
  a.xp = (float*)(w8 + y.xp);
  a.prev = (float*)(w8 + y.prev);
  a.hid = (float*)(w8 + y.hid);
  a.dead = (int32_t*)(w8 + y.dead);
  a.trace = trace;
  float* an = (float*)(w8 + y.a);
  int32_t* lm_nacc = (int32_t*)(w8 + y.lmi);
  int32_t* lm_tok = lm_nacc + G;
  std::vector<int32_t> gs1(G + 1);
  for (int g = 0; g <= G; ++g) gs1[g] = g;  // the lm_head pass: one row per group, no drafts
  hipStream_t st = S(stream);
  const int cu = device_cu_count();
  for (int pass = 0; pass < n_draft; ++pass) {
    const int rows = pass == 0 ? T : G;
    hipError_t e = mk::launch_mtp_in(a, pass, rows, st);
    if (e != hipSuccess) return launch_status(e, "mtp: input rows");
    if ((r = mk_qgemv_rows_ex(&m->fc, a.z, rows, a.u, MK_PATH_AUTO, w8 + y.gemv, y.ws_gemv, stream))) return r;
    if ((e = mk::launch_rms_rows(a.u, an, rows, H, st)) != hipSuccess) return launch_status(e, "mtp: norm");
    if ((r = mk_ffn_rows(&m->gate, &m->up, &m->down, an, rows, a.y, nullptr, w8 + y.ffn, y.ws_ffn, stream))) return r;
    const int trace_row0 = pass == 0 ? 0 : T + (pass - 1) * G;
    if ((e = mk::launch_mtp_out(a, pass, rows, trace_row0, st)) != hipSuccess) return launch_status(e, "mtp: output rows");
    if ((e = mk::launch_lmhead(embed_f16, V_draft, H, a.hid, G, gs1.data(), G, nullptr, drafts + (size_t)pass * G,
                               lm_nacc, lm_tok, w8 + y.lm, cu, st)) != hipSuccess)
      return launch_status(e, "mtp: draft lm_head");
  }
  return ok();
}

// ------------------------------------------------------------------ Gated DeltaNet
static int check_dn(const mk_deltanet* st) {
  int r;
  if (!st) return fail(MK_ERR_ARG, "deltanet: null state");
  if (st->dk != 128 || st->dv != 128) return fail(MK_ERR_SHAPE, "deltanet: dk = dv = 128 required");
  if (st->nh <= 0) return fail(MK_ERR_SHAPE, "deltanet: nh = %d", st->nh);
  if (st->T_max < 2 || st->T_max > MK_T_MAX) return fail(MK_ERR_RANGE, "deltanet: T_max = %d", st->T_max);
  if ((r = check_ptr(st->S, "S")) || (r = check_ptr(st->ring, "ring")) || (r = check_ptr(st->n_acc, "n_acc", 4)))
    return r;
  return MK_OK;
}

int mk_deltanet_step(const mk_deltanet* st, int32_t use_prev_acc, const float* q, const float* k, const float* v,
                     const float* g, const float* beta, int32_t T, float* o, void* stream) {
  int r;
  if ((r = check_dn(st))) return r;
  if (T < 1 || T > st->T_max) return fail(MK_ERR_RANGE, "deltanet: T = %d outside 1..%d", T, st->T_max);
  if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v")) || (r = check_ptr(g, "g", 4)) ||
      (r = check_ptr(beta, "beta", 4)) || (r = check_ptr(o, "o")))
    return r;
  mk::GdnArgs a;
  a.S = st->S;
  a.ring = st->ring;
  a.n_acc = st->n_acc;
  a.use_prev = use_prev_acc ? 1 : 0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.nh = st->nh;
  a.T = T;
  a.T_max = st->T_max;
  return launch_status(mk::launch_gdn_step(a, S(stream)), "deltanet step");
}

int mk_deltanet_commit(const mk_deltanet* st, void* stream) {
  int r;
  if ((r = check_dn(st))) return r;
  mk::GdnArgs a = {};
  a.S = st->S;
  a.ring = st->ring;
  a.n_acc = st->n_acc;
  a.nh = st->nh;
  a.T = 0;
  a.T_max = st->T_max;
  return launch_status(mk::launch_gdn_commit(a, S(stream)), "deltanet commit");
}

int mk_deltanet_status(const mk_deltanet* st, void* stream) {
  int r;
  if ((r = check_dn(st))) return r;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, st->n_acc + 2, sizeof(v), hipMemcpyDeviceToHost, S(stream)) != hipSuccess ||
      hipStreamSynchronize(S(stream)) != hipSuccess)
    return fail(MK_ERR_LAUNCH, "deltanet status: readback failed");
  if (!v) return ok();
  if (hipMemsetAsync(st->n_acc + 2, 0, sizeof(int32_t), S(stream)) != hipSuccess ||
      hipStreamSynchronize(S(stream)) != hipSuccess)
    return fail(MK_ERR_LAUNCH, "deltanet status: clear failed");
  return fail(MK_ERR_RANGE, "deltanet: an accept length outside 0..T_max-1 was read (nothing was replayed)");
}

// ------------------------------------------------------------------ read probe
// Measurement aid: every thread reads 16-B words of the buffer with
// nontemporal loads, grid-stride, and folds them into one word; a word that
// depends on every load is stored so that no load can be dropped.
typedef uint32_t probe_v4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_read_probe(const probe_v4* __restrict__ p, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const probe_v4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;  // practically never taken, but not removable
}

// ------------------------------------------------------------------ attention
static int check_attn(int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t cap, const int32_t* h_ctx,
                      const int32_t* h_group_start, int32_t G, std::vector<int32_t>& gs) {
  int r;
  if ((r = check_T(T))) return r;
  if (d != 128) return fail(MK_ERR_SHAPE, "attention: d = %d (128 required)", d);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return fail(MK_ERR_SHAPE, "attention: Hq = %d, Hkv = %d", Hq, Hkv);
  if (cap <= 0 || cap % 64) return fail(MK_ERR_SHAPE, "attention: cap = %d is not a positive multiple of 64", cap);
  if (cap > MK_ATTN_CAP_MAX) return fail(MK_ERR_RANGE, "attention: cap = %d > %d", cap, MK_ATTN_CAP_MAX);
  if (!h_ctx) return fail(MK_ERR_ARG, "attention: h_ctx is null");
  if (G > MK_ATTN_MAX_G) return fail(MK_ERR_RANGE, "attention: G = %d > %d", G, MK_ATTN_MAX_G);
  if ((r = check_groups(h_group_start, G, T, gs))) return r;
  const int gqa = Hq / Hkv;
  for (int g = 0; g < G; ++g) {
    const int n = gs[g + 1] - gs[g];
    if (h_ctx[g] < 0 || (long)h_ctx[g] + n > cap)
      return fail(MK_ERR_RANGE, "attention: agent %d: ctx %d + %d rows exceeds cap %d", g, h_ctx[g], n, cap);
    if (n * gqa > 64) return fail(MK_ERR_RANGE, "attention: agent %d: %d rows x %d query heads > 64", g, n, gqa);
  }
  return MK_OK;
}

size_t mk_attn_decode_workspace(int32_t T, int32_t Hq, int32_t Hkv, const int32_t* h_ctx,
                                const int32_t* h_group_start, int32_t G) {
  std::vector<int32_t> gs;
  if (check_attn(T, Hq, Hkv, 128, MK_ATTN_CAP_MAX, h_ctx, h_group_start, G, gs)) return 0;
  // the larger of the two cache formats' plans, so one size serves both
  const mk::AttnPlan p16 = mk::plan_attn(G, h_ctx, gs.data(), Hkv, device_cu_count(), false);
  const mk::AttnPlan p8 = mk::plan_attn(G, h_ctx, gs.data(), Hkv, device_cu_count(), true);
  return std::max(mk::attn_workspace_bytes(T, Hq, p16), mk::attn_workspace_bytes(T, Hq, p8));
}

static int attn_call(const float* q, const float* gate, int32_t T, int32_t Hq, const uint16_t* k_cache,
                     const uint16_t* v_cache, const int8_t* k_codes, const uint16_t* k_scales, const int8_t* v_codes,
                     const uint16_t* v_scales, int32_t Hkv, int32_t d, int32_t cap, const int32_t* h_ctx,
                     const int32_t* h_group_start, int32_t G, float* o, void* ws, size_t ws_bytes, void* stream) {
  int r;
  std::vector<int32_t> gs;
  if ((r = check_attn(T, Hq, Hkv, d, cap, h_ctx, h_group_start, G, gs))) return r;
  const bool q8 = k_codes || v_codes;
  if ((r = check_ptr(q, "q")) || (r = check_ptr(o, "o"))) return r;
  if (q8) {
    if ((r = check_ptr(k_codes, "k_codes")) || (r = check_ptr(k_scales, "k_scales")) ||
        (r = check_ptr(v_codes, "v_codes")) || (r = check_ptr(v_scales, "v_scales")))
      return r;
  } else if ((r = check_ptr(k_cache, "k_cache")) || (r = check_ptr(v_cache, "v_cache"))) {
    return r;
  }
  if (gate && !aligned(gate, 16)) return fail(MK_ERR_ALIGN, "gate not 16-B aligned");
  const mk::AttnPlan p = mk::plan_attn(G, h_ctx, gs.data(), Hkv, device_cu_count(), q8);
  const size_t need = mk::attn_workspace_bytes(T, Hq, p);
  if (!ws || ws_bytes < need) return fail(MK_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((r = check_ptr(ws, "workspace", 256))) return r;
  mk::AttnArgs a = {};
  a.q = q;
  a.gate = gate;
  a.o = o;
  a.k = k_cache;
  a.v = v_cache;
  a.k8 = k_codes;
  a.v8 = v_codes;
  a.ks = k_scales;
  a.vs = v_scales;
  a.qscale = (float)(1.4426950408889634 / sqrt(128.0));
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.gqa = Hq / Hkv;
  a.cap = cap;
  a.G = G;
  int nmax = 0;
  for (int g = 0; g < G; ++g) {
    a.ctx[g] = h_ctx[g];
    nmax = std::max(nmax, gs[g + 1] - gs[g]);
  }
  for (int g = 0; g <= G; ++g) a.gs[g] = gs[g];
  const int nb = (nmax * a.gqa + 15) / 16;
  return launch_status(mk::launch_attn(a, p, nb, q8, ws, S(stream)), "attention");
}

int mk_attn_decode(const float* q, const float* gate, int32_t T, int32_t Hq, const uint16_t* k_cache,
                   const uint16_t* v_cache, int32_t Hkv, int32_t d, int32_t cap, const int32_t* h_ctx,
                   const int32_t* h_group_start, int32_t G, float* o, void* ws, size_t ws_bytes, void* stream) {
  return attn_call(q, gate, T, Hq, k_cache, v_cache, nullptr, nullptr, nullptr, nullptr, Hkv, d, cap, h_ctx,
                   h_group_start, G, o, ws, ws_bytes, stream);
}

int mk_attn_decode_q8(const float* q, const float* gate, int32_t T, int32_t Hq, const int8_t* k_codes,
                      const uint16_t* k_scales, const int8_t* v_codes, const uint16_t* v_scales, int32_t Hkv,
                      int32_t d, int32_t cap, const int32_t* h_ctx, const int32_t* h_group_start, int32_t G,
                      float* o, void* ws, size_t ws_bytes, void* stream) {
  if (!k_codes || !v_codes) return fail(MK_ERR_ARG, "attention q8: null codes");
  return attn_call(q, gate, T, Hq, nullptr, nullptr, k_codes, k_scales, v_codes, v_scales, Hkv, d, cap, h_ctx,
                   h_group_start, G, o, ws, ws_bytes, stream);
}

int mk_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  int r;
  if ((r = check_ptr(buf, "buf")) || (r = check_ptr(sink, "sink", 4))) return r;
  if (bytes % 16) return fail(MK_ERR_SHAPE, "read probe: %zu bytes is not a multiple of 16", bytes);
  const int cu = device_cu_count();
  hipLaunchKernelGGL(k_read_probe, dim3(8 * (cu > 0 ? cu : 256)), dim3(256), 0, S(stream), (const probe_v4*)buf,
                     bytes / 16, sink);
  return launch_status(hipGetLastError(), "read probe");
}

}  // extern "C"
