// C-ABI entry points: argument validation (before any HIP call), launch
// planning, decode workspace management, and error reporting.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "fa.h"
#include "fa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() { return FA_OK; }

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Common prefill checks.  elem = bytes per element of Q/K/V/O.
int check_fwd(const void* Q, const void* K, const void* V, const void* O, const float* L, int B,
              int H, int N, int d, int causal, float scale, size_t elem, int rows_per_wg) {
  if (!Q || !K || !V || !O) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || N < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!(isfinite(scale) && scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(FA_ERR_INVALID_ARG, "Q, K, V, O must be 16-byte aligned");
  if (L && !aligned(L, 4)) return fail(FA_ERR_INVALID_ARG, "L must be 4-byte aligned");
  const int64_t q_tiles = fa::ceil_div64(N, rows_per_wg);
  if ((int64_t)B * H * q_tiles > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "grid too large");
  if ((int64_t)N * d * (int64_t)elem > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "one head of N x d elements must be under 2 GiB (N = %d)", N);
  const size_t tbytes = (size_t)B * H * N * d * elem;
  const size_t lbytes = L ? (size_t)B * H * N * sizeof(float) : 0;
  if (overlap(O, tbytes, Q, tbytes) || overlap(O, tbytes, K, tbytes) || overlap(O, tbytes, V, tbytes))
    return fail(FA_ERR_INVALID_ARG, "O overlaps an input");
  if (overlap(L, lbytes, Q, tbytes) || overlap(L, lbytes, K, tbytes) || overlap(L, lbytes, V, tbytes) ||
      overlap(L, lbytes, O, tbytes))
    return fail(FA_ERR_INVALID_ARG, "L overlaps another tensor");
  return FA_OK;
}

int check_decode(const void* q, const void* Kc, const void* Vc, const void* o, const float* lse,
                 int B, int H, const int32_t* Lkv, int cap, int d, int num_splits, float scale) {
  if (!q || !Kc || !Vc || !o || !Lkv) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (B < 1 || H < 1) return fail(FA_ERR_INVALID_ARG, "B, H must be >= 1 (got %d, %d)", B, H);
  if (B > 65535 || H > 65535) return fail(FA_ERR_INVALID_ARG, "B and H must be <= 65535");
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", d);
  if (num_splits < 0 || num_splits > 4096) return fail(FA_ERR_INVALID_ARG, "num_splits must be in [0, 4096]");
  if (cap < 0) return fail(FA_ERR_INVALID_ARG, "kv_seq_capacity must be >= 0");
  if (!(isfinite(scale) && scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(Kc, 16) || !aligned(Vc, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, Kcache, Vcache, o must be 16-byte aligned");
  if (!aligned(Lkv, 4) || (lse && !aligned(lse, 4))) return fail(FA_ERR_INVALID_ARG, "Lkv/lse_out misaligned");
  const size_t ob = (size_t)B * H * d * 2, lb = lse ? (size_t)B * H * 4 : 0;
  if (overlap(o, ob, q, ob) || overlap(o, ob, Kc, 1) || overlap(o, ob, Vc, 1) || overlap(o, ob, Lkv, (size_t)B * 4))
    return fail(FA_ERR_INVALID_ARG, "o overlaps an input");
  if (overlap(lse, lb, o, ob) || overlap(lse, lb, q, ob) || overlap(lse, lb, Lkv, (size_t)B * 4))
    return fail(FA_ERR_INVALID_ARG, "lse_out overlaps another buffer");
  return FA_OK;
}

// Backward checks.  The inputs Q, K, V, O, dO (bf16 [B, H, N, d]) and L
// (fp32 [B, H, N]) may overlap each other; the outputs dQ, dK, dV may
// overlap nothing.
int check_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
              const void* dQ, const void* dK, const void* dV, int B, int H, int N, int d, int causal,
              float scale) {
  if (!Q || !K || !V || !O || !dO || !L || !dQ || !dK || !dV) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || N < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %d not supported (64 or 128)", d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!(isfinite(scale) && scale > 0.f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  const void* t16[] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* p : t16)
    if (!aligned(p, 16)) return fail(FA_ERR_INVALID_ARG, "Q, K, V, O, dO, dQ, dK, dV must be 16-byte aligned");
  if (!aligned(L, 4)) return fail(FA_ERR_INVALID_ARG, "L must be 4-byte aligned");
  const int64_t tiles = fa::ceil_div64(N, fa::kBwdQT < fa::kBwdKV ? fa::kBwdQT : fa::kBwdKV);
  if ((int64_t)B * H * tiles > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "grid too large");
  if ((int64_t)N * d * 2 > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "one head of N x d elements must be under 2 GiB (N = %d)", N);
  const size_t tb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * sizeof(float);
  const void* outs[] = {dQ, dK, dV};
  const void* ins[] = {Q, K, V, O, dO};
  for (int i = 0; i < 3; ++i) {
    for (const void* in : ins)
      if (overlap(outs[i], tb, in, tb)) return fail(FA_ERR_INVALID_ARG, "dQ, dK, dV must not overlap an input");
    if (overlap(outs[i], tb, L, lb)) return fail(FA_ERR_INVALID_ARG, "dQ, dK, dV must not overlap L");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], tb, outs[j], tb)) return fail(FA_ERR_INVALID_ARG, "dQ, dK, dV must not overlap each other");
  }
  return FA_OK;
}

// Compute units assumed by the host-only planners (no device query).
constexpr int kPlanCUs = 256;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_bytes(int B, int H, int d, int S) {
  const size_t parts = (size_t)B * H * S;
  return align256(parts * d * sizeof(float)) + align256(parts * sizeof(float));
}

// Compute-unit count per device, queried once.
int cu_count(int* out) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    it = cache.emplace(dev, cus).first;
  }
  *out = it->second;
  return FA_OK;
}

// Automatic split count: enough split workgroups to cover every compute
// unit once, and at least 8 chunks per sequence so that unequal lengths in a
// batch still spread over the device.  Few long chunks stream better than
// many short ones, and the combine stays small.
int auto_splits(int B, int H, int cus) {
  const int64_t bh = (int64_t)B * H;
  int64_t s = fa::ceil_div64(cus, bh);
  if (s < 8) s = 8;
  if (s > 256) s = 256;
  return (int)s;
}

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

struct PagedArgs {
  const int32_t* table = nullptr;
  int max_blocks = 0, log2_bs = 0, num_blocks = 0;
};

int decode_common(const void* q, const void* Kc, const void* Vc, void* o, float* lse, int B, int H,
                  const int32_t* Lkv, int cap, int d, int S, float scale, void* ws, hipStream_t st,
                  const PagedArgs& pg = PagedArgs(), int* counters = nullptr) {
  fa::DecodeArgs a;
  a.q = q;
  a.K = Kc;
  a.V = Vc;
  a.o = o;
  a.lse_out = lse;
  a.Lkv = Lkv;
  const size_t parts = (size_t)B * H * S;
  a.part_o = static_cast<float*>(ws);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(parts * d * sizeof(float)));
  a.B = B;
  a.H = H;
  a.S = S;
  a.capacity = cap;
  a.scale = scale;
  a.table = pg.table;
  a.max_blocks = pg.max_blocks;
  a.log2_bs = pg.log2_bs;
  a.num_blocks = pg.num_blocks;
  a.counters = counters;
  hipError_t e = fa::launch_decode(a, d, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

// The library-owned decode workspace of (current device, stream), grown to
// at least `need` bytes (never while the stream is being captured).
int internal_workspace(size_t need, hipStream_t hs, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& w = g_ws[std::make_pair(dev, hs)];
  if (w.bytes < need) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(hs, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(FA_ERR_WORKSPACE, "the decode workspace must grow to %zu bytes; call once outside stream capture", need);
    if (w.ptr) {
      e = hipStreamSynchronize(hs);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      e = hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
      if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    e = hipMalloc(&w.ptr, need);
    if (e != hipSuccess) {
      w.ptr = nullptr;
      (void)hipGetLastError();
      return fail(FA_ERR_NOMEM, "hipMalloc(%zu) for the decode workspace failed", need);
    }
    w.bytes = need;
  }
  *out = w.ptr;
  return FA_OK;
}

// Scratch of the allocation-free decode (fa_decode_noalloc): the split
// partials live in this array instead of a workspace.  Every device the
// library runs on holds its own copy until the process ends; host code uses
// only the per-device address hipGetSymbolAddress returns for it (the
// array's name on the host is a stand-in, not a device address).  Calls on
// one device share its copy: calls that may overlap on a device race.  The
// split kernel writes every partial the combine reads (an empty chunk writes
// O = 0, lse = -inf), so nothing needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;  // device -> address of its scratch copy

// Address of the current device's scratch, looked up once per device (with
// that device current).  Allocates nothing.
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return e != hipSuccess ? hip_fail(e, "hipGetSymbolAddress(scratch)")
                             : fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    }
    it = g_scratch.emplace(dev, p).first;
  }
  *out = it->second;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported";
    case FA_ERR_HIP: return "HIP error";
    case FA_ERR_NOMEM: return "out of device memory";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return (1 << 16) | 0; }

// exponentials per 64 that the d = 128 bf16 forward evaluates by polynomial
static std::atomic<int> g_fwd_exp2_poly{0};

int fa_set_fwd_exp2_poly(int per64) {
  if (per64 != 0 && per64 != 4 && per64 != 8 && per64 != 16)
    return fail(FA_ERR_INVALID_ARG, "exponentials per 64 by polynomial must be 0, 4, 8 or 16 (got %d)", per64);
  g_fwd_exp2_poly.store(per64, std::memory_order_relaxed);
  return ok();
}

int fa_get_fwd_exp2_poly(void) { return g_fwd_exp2_poly.load(std::memory_order_relaxed); }

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N,
           int d, int causal, float scale, void* stream) {
  int st = check_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, 2, fa::kFwdBR);
  if (st != FA_OK) return st;
  int cus = 0;
  if ((st = cu_count(&cus)) != FA_OK) return st;
  fa::FwdArgs a{Q, K, V, O, L, B, H, N, causal, scale,
                (int)fa::fwd_grid(fa::fwd_units(B, H, N, causal), d, causal, cus),
                g_fwd_exp2_poly.load(std::memory_order_relaxed)};
  hipError_t e = fa::launch_fwd_bf16(a, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fa_fwd launch");
  return ok();
}

int fa_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* L, int B, int H,
               int N, int d, int causal, float scale, void* stream) {
  int st = check_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, 4, fa::kF32BR);
  if (st != FA_OK) return st;
  fa::FwdArgs a{Q, K, V, O, L, B, H, N, causal, scale, 0};
  hipError_t e = fa::launch_fwd_f32(a, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fa_fwd_f32 launch");
  return ok();
}

int fa_fwd_plan(int B, int H, int N, int d, int causal, fa_fwd_plan_t* out) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "null plan pointer");
  if (B < 1 || H < 1 || N < 1) return fail(FA_ERR_INVALID_ARG, "B, H, N must be >= 1");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %d not supported", d);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  const int q_tiles = (int)fa::ceil_div64(N, fa::kFwdBR);
  out->block_rows = fa::kFwdBR;
  out->block_cols = fa::kFwdBC;
  out->q_tiles = q_tiles;
  out->kv_tiles = (int)fa::ceil_div64(N, fa::kFwdBC);
  out->threads_per_workgroup = fa::fwd_threads(d, causal);
  out->lds_bytes = fa::fwd_lds_for(d, causal);
  out->work_units = fa::fwd_units(B, H, N, causal);
  out->workgroups = fa::fwd_grid(out->work_units, d, causal, kPlanCUs);
  int64_t visited = 0, masked = 0;
  for (int qt = 0; qt < q_tiles; ++qt) {
    const int n = fa::fwd_kv_tiles_for(qt, N, causal);
    visited += n;
    for (int j = 0; j < n; ++j) {
      const int kb = j * fa::kFwdBC;
      const bool ragged = kb + fa::kFwdBC > N;
      const bool diag = causal && (kb + fa::kFwdBC - 1 > qt * fa::kFwdBR);
      if (ragged || diag) ++masked;
    }
  }
  out->tiles_visited = visited * B * H;
  out->tiles_masked = masked * B * H;
  return ok();
}

int fa_decode_chunk_tokens(int kv_len, int num_splits) {
  return fa::decode_chunk_tokens(kv_len, num_splits);
}

int fa_decode_plan(int B, int H, int d, int num_splits, fa_decode_plan_t* out) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "null plan pointer");
  if (B < 1 || H < 1) return fail(FA_ERR_INVALID_ARG, "B, H must be >= 1");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %d not supported", d);
  if (num_splits < 0 || num_splits > 4096) return fail(FA_ERR_INVALID_ARG, "num_splits out of range");
  int S = num_splits;
  if (S == 0) S = auto_splits(B, H, kPlanCUs);
  out->num_splits = S;
  out->threads_per_workgroup = fa::kDecWaves * 64;
  out->split_workgroups = (int64_t)B * H * S;
  out->combine_workgroups = (int64_t)B * H;
  out->workspace_bytes = ws_bytes(B, H, d, S);
  return ok();
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || (d != 64 && d != 128) || num_splits < 0 || num_splits > 4096) return 0;
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if (cu_count(&cus) != FA_OK) return 0;
    S = auto_splits(B, H, cus);
  }
  return ws_bytes(B, H, d, S);
}

int fa_decode(const void* q, const void* Kcache, const void* Vcache, void* o, int B, int H,
              const int32_t* Lkv, int d, int num_splits, void* stream) {
  const float scale = 1.f / sqrtf((float)d);
  int st = check_decode(q, Kcache, Vcache, o, nullptr, B, H, Lkv, 0, d, num_splits, scale);
  if (st != FA_OK) return st;
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if ((st = cu_count(&cus)) != FA_OK) return st;
    S = auto_splits(B, H, cus);
  }
  const size_t need = ws_bytes(B, H, d, S);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = internal_workspace(need, hs, &ws)) != FA_OK) return st;
  return decode_common(q, Kcache, Vcache, o, nullptr, B, H, Lkv, 0, d, S, scale, ws, hs);
}

// The backward's workspace: D, then L in base 2, each B * H * N floats
// aligned to 256 bytes.
size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return 2 * align256((size_t)B * H * N * sizeof(float));
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L, void* dQ,
           void* dK, void* dV, int B, int H, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream) {
  int st = check_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, causal, scale);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(B, H, N);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  if (!workspace) {
    if (workspace_bytes != 0) return fail(FA_ERR_WORKSPACE, "null workspace with nonzero workspace_bytes");
    if ((st = internal_workspace(need, hs, &ws)) != FA_OK) return st;
  } else {
    if (!aligned(workspace, 256)) return fail(FA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes is too small (%zu needed)", workspace_bytes, need);
    const size_t tb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * sizeof(float);
    const void* tens[] = {Q, K, V, O, dO, dQ, dK, dV};
    for (const void* p : tens)
      if (overlap(workspace, need, p, tb)) return fail(FA_ERR_INVALID_ARG, "workspace overlaps a tensor");
    if (overlap(workspace, need, L, lb)) return fail(FA_ERR_INVALID_ARG, "workspace overlaps L");
  }
  float* Dws = static_cast<float*>(ws);
  float* L2ws = reinterpret_cast<float*>(static_cast<char*>(ws) + need / 2);
  fa::BwdArgs a{Q, K, V, O, dO, L, dQ, dK, dV, Dws, L2ws, B, H, N, causal, scale};
  hipError_t e = fa::launch_bwd_bf16(a, d, hs);
  if (e != hipSuccess) return hip_fail(e, "fa_bwd launch");
  return ok();
}

int fa_decode_ex(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse_out,
                 int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d, int num_splits,
                 float scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (!workspace) return fail(FA_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(FA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if ((st = cu_count(&cus)) != FA_OK) return st;
    S = auto_splits(B, H, cus);
  }
  const size_t need = ws_bytes(B, H, d, S);
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes is too small (%zu needed)", workspace_bytes, need);
  if (overlap(workspace, need, o, (size_t)B * H * d * 2) || overlap(workspace, need, q, (size_t)B * H * d * 2))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps q or o");
  return decode_common(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, S, scale,
                       workspace, static_cast<hipStream_t>(stream));
}

// The one-launch decode's workspace: a fixed region of kFusedCounters int32
// counters first (so that a workspace reused for another shape finds its
// counters where the previous call left them, at zero), then the partials.
constexpr int64_t kFusedCounters = 65536;
constexpr size_t kFusedCounterBytes = kFusedCounters * sizeof(int);

size_t fa_decode_fused_workspace_bytes(int B, int H, int d, int num_splits) {
  if ((int64_t)B * H > kFusedCounters) return 0;
  const size_t parts = fa_decode_workspace_bytes(B, H, d, num_splits);
  return parts ? kFusedCounterBytes + parts : 0;
}

int fa_decode_fused(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse_out,
                    int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d, int num_splits,
                    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (!workspace) return fail(FA_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(FA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if ((int64_t)B * H > kFusedCounters)
    return fail(FA_ERR_UNSUPPORTED, "B * H = %lld exceeds the %lld counters of the one-launch decode",
                (long long)B * H, (long long)kFusedCounters);
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if ((st = cu_count(&cus)) != FA_OK) return st;
    S = auto_splits(B, H, cus);
  }
  const size_t need = kFusedCounterBytes + ws_bytes(B, H, d, S);
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes is too small (%zu needed)", workspace_bytes, need);
  if (overlap(workspace, need, o, (size_t)B * H * d * 2) || overlap(workspace, need, q, (size_t)B * H * d * 2))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps q or o");
  if (lse_out && overlap(workspace, need, lse_out, (size_t)B * H * sizeof(float)))
    return fail(FA_ERR_INVALID_ARG, "workspace overlaps lse_out");
  int* counters = static_cast<int*>(workspace);
  return decode_common(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, S, scale,
                       static_cast<char*>(workspace) + kFusedCounterBytes, static_cast<hipStream_t>(stream),
                       PagedArgs(), counters);
}

size_t fa_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int fa_decode_noalloc(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse_out,
                      int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d, int num_splits,
                      float scale, void* stream) {
  int st = check_decode(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, num_splits, scale);
  if (st != FA_OK) return st;
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if ((st = cu_count(&cus)) != FA_OK) return st;
    S = auto_splits(B, H, cus);
  }
  const size_t need = ws_bytes(B, H, d, S);
  if (need > kNoAllocScratchBytes)
    return fail(FA_ERR_WORKSPACE,
                "fa_decode_noalloc: %d x %d x %d partials need %zu bytes, above its %zu-byte scratch "
                "(use fewer splits, or fa_decode_ex with a workspace)",
                B, H, S, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != FA_OK) return st;
  return decode_common(q, Kcache, Vcache, o, lse_out, B, H, Lkv, kv_seq_capacity, d, S, scale, ws,
                       static_cast<hipStream_t>(stream));
}

int fa_decode_paged(const void* q, const void* Kpool, const void* Vpool, void* o, float* lse_out,
                    int B, int H, const int32_t* block_table, int max_blocks, const int32_t* Lkv,
                    int num_blocks, int block_size, int d, int num_splits, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode(q, Kpool, Vpool, o, lse_out, B, H, Lkv, 0, d, num_splits, scale);
  if (st != FA_OK) return st;
  if (!block_table) return fail(FA_ERR_INVALID_ARG, "null pointer argument (block_table)");
  if (!aligned(block_table, 4)) return fail(FA_ERR_INVALID_ARG, "block_table misaligned");
  if (max_blocks < 1 || num_blocks < 1)
    return fail(FA_ERR_INVALID_ARG, "max_blocks and num_blocks must be >= 1 (got %d, %d)", max_blocks, num_blocks);
  if (block_size < fa::kPagedMinBlock || block_size > fa::kPagedMaxBlock || (block_size & (block_size - 1)))
    return fail(FA_ERR_INVALID_ARG, "block_size must be a power of two in [%d, %d] (got %d)", fa::kPagedMinBlock,
                fa::kPagedMaxBlock, block_size);
  const int64_t pool_rows = (int64_t)num_blocks * H * block_size;
  if (pool_rows > ((int64_t)1 << 40)) return fail(FA_ERR_INVALID_ARG, "pool too large");
  const size_t ob = (size_t)B * H * d * 2, tb = (size_t)B * max_blocks * 4;
  if (overlap(o, ob, block_table, tb) || (lse_out && overlap(lse_out, (size_t)B * H * 4, block_table, tb)))
    return fail(FA_ERR_INVALID_ARG, "an output overlaps block_table");
  // split count: each chunk may span at most kPagedIdsPerChunk blocks
  int64_t max_len = (int64_t)max_blocks * block_size;
  if (max_len > 0x7fffffff) max_len = 0x7fffffff;
  auto blocks_ok = [&](int S) {
    return fa::paged_blocks_per_chunk(fa::decode_chunk_tokens((int)max_len, S), block_size) <= fa::kPagedIdsPerChunk;
  };
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if ((st = cu_count(&cus)) != FA_OK) return st;
    S = auto_splits(B, H, cus);
    while (!blocks_ok(S) && S < 4096) S = S * 2 > 4096 ? 4096 : S * 2;
  }
  if (!blocks_ok(S))
    return fail(FA_ERR_UNSUPPORTED, "with %d splits a chunk may span more than %d blocks; use more splits", S,
                fa::kPagedIdsPerChunk);
  const size_t need = ws_bytes(B, H, d, S);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  if (!workspace) {
    if (workspace_bytes != 0) return fail(FA_ERR_WORKSPACE, "null workspace with nonzero workspace_bytes");
    if ((st = internal_workspace(need, hs, &ws)) != FA_OK) return st;
  } else {
    if (!aligned(workspace, 256)) return fail(FA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes is too small (%zu needed)", workspace_bytes, need);
    if (overlap(workspace, need, o, ob) || overlap(workspace, need, q, ob) || overlap(workspace, need, block_table, tb))
      return fail(FA_ERR_INVALID_ARG, "workspace overlaps another buffer");
  }
  PagedArgs pg;
  pg.table = block_table;
  pg.max_blocks = max_blocks;
  pg.log2_bs = 31 - __builtin_clz((unsigned)block_size);
  pg.num_blocks = num_blocks;
  return decode_common(q, Kpool, Vpool, o, lse_out, B, H, Lkv, 0, d, S, scale, ws, hs, pg);
}

int fa_decode_paged_splits(int B, int H, int max_blocks, int block_size, int num_splits) {
  if (B < 1 || H < 1 || max_blocks < 1 || num_splits < 0 || num_splits > 4096) return 0;
  if (block_size < fa::kPagedMinBlock || block_size > fa::kPagedMaxBlock || (block_size & (block_size - 1))) return 0;
  int64_t max_len = (int64_t)max_blocks * block_size;
  if (max_len > 0x7fffffff) max_len = 0x7fffffff;
  int S = num_splits;
  if (S == 0) {
    int cus = 0;
    if (cu_count(&cus) != FA_OK) cus = kPlanCUs;
    S = auto_splits(B, H, cus);
    while (fa::paged_blocks_per_chunk(fa::decode_chunk_tokens((int)max_len, S), block_size) > fa::kPagedIdsPerChunk &&
           S < 4096)
      S = S * 2 > 4096 ? 4096 : S * 2;
  }
  return fa::paged_blocks_per_chunk(fa::decode_chunk_tokens((int)max_len, S), block_size) <= fa::kPagedIdsPerChunk ? S : 0;
}

int fa_probe_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(FA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(FA_ERR_INVALID_ARG, "buf must be 16-byte and sink 4-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(FA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(FA_ERR_INVALID_ARG, "workgroups must be in [1, 1048576] (got %d)", workgroups);
  if (overlap(buf, bytes, sink, (size_t)workgroups * 4)) return fail(FA_ERR_INVALID_ARG, "sink overlaps buf");
  hipError_t e = fa::launch_probe_hbm_read(buf, bytes, workgroups, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "probe launch");
}

static int check_probe_mfma(int workgroups, int iters, const float* sink, const uint64_t* stamps) {
  if (!sink) return fail(FA_ERR_INVALID_ARG, "null sink");
  if (!aligned(sink, 4) || (stamps && !aligned(stamps, 8)))
    return fail(FA_ERR_INVALID_ARG, "sink must be 4-byte and stamps 8-byte aligned");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(FA_ERR_INVALID_ARG, "workgroups must be in [1, 1048576] (got %d)", workgroups);
  if (iters < 1 || iters > (1 << 24)) return fail(FA_ERR_INVALID_ARG, "iters must be in [1, 16777216] (got %d)", iters);
  if (stamps && overlap(sink, (size_t)workgroups * 256 * 4, stamps, (size_t)workgroups * 16))
    return fail(FA_ERR_INVALID_ARG, "stamps overlaps sink");
  return FA_OK;
}

int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, uint64_t* stamps, void* stream) {
  int st = check_probe_mfma(workgroups, iters, sink, stamps);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_probe_mfma_bf16(workgroups, iters, sink, stamps, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "probe launch");
}

int fa_probe_mfma_bf16_mixed(int workgroups, int iters, uint32_t seed, float* sink, uint64_t* stamps, void* stream) {
  int st = check_probe_mfma(workgroups, iters, sink, stamps);
  if (st != FA_OK) return st;
  hipError_t e =
      fa::launch_probe_mfma_bf16_mixed(workgroups, iters, seed, sink, stamps, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "probe launch");
}

int fa_release_workspace(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int status = FA_OK;
  for (auto& kv : g_ws) {
    if (!kv.second.ptr) continue;
    if ((e = hipSetDevice(kv.first.first)) == hipSuccess && (e = hipDeviceSynchronize()) == hipSuccess)
      e = hipFree(kv.second.ptr);
    if (e != hipSuccess) status = hip_fail(e, "releasing a decode workspace");
    kv.second.ptr = nullptr;
    kv.second.bytes = 0;
  }
  g_ws.clear();
  (void)hipSetDevice(prev);
  return status;
}

}  // extern "C"
