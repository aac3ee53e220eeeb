// sage_abi.cpp -- the C ABI (include/sage_attn.h): argument checks on the host,
// quantized-buffer layout, dispatch to the HIP launchers, status and error text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sage_attn.h"
#include "sage_launch.hpp"

namespace {

thread_local char g_err[512] = "";

sage_status fail(sage_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

sage_status hip_fail(hipError_t e, const char* where) {
  return fail(SAGE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Fault injection for host tests of the error paths (SAGE_FAULT_INJECT=alloc).
bool inject_alloc_failure() {
  const char* e = getenv("SAGE_FAULT_INJECT");
  return e && strcmp(e, "alloc") == 0;
}

// Checks shared by the fixed-length and the packed problem descriptors.
sage_status check_common(int d, int causal, float sm_scale, int io_dtype, int qk_fmt, int pv_fmt) {
  if (d != 64 && d != 128) return fail(SAGE_ERR_UNSUPPORTED, "head dim d=%d is not supported (64 or 128)", d);
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (io_dtype != SAGE_DT_BF16 && io_dtype != SAGE_DT_F16)
    return fail(SAGE_ERR_INVALID_ARG, "io_dtype %d is not a SAGE_DT_* value", io_dtype);
  auto known = [](int f) { return f >= SAGE_FMT_INT8 && f <= SAGE_FMT_MXFP4_QBLOCK; };
  const bool fmts_known = known(qk_fmt) && known(pv_fmt);
  if (!fmts_known) return fail(SAGE_ERR_INVALID_ARG, "qk_fmt/pv_fmt must be SAGE_FMT_* values");
  const bool int8 = qk_fmt == SAGE_FMT_INT8 || qk_fmt == SAGE_FMT_INT8_TOKEN;
  const bool mx4 = qk_fmt == SAGE_FMT_MXFP4 || qk_fmt == SAGE_FMT_MXFP4_QBLOCK;
  const bool pair_ok = (int8 && pv_fmt == SAGE_FMT_FP8) || (int8 && pv_fmt == SAGE_FMT_F16) ||
                       (mx4 && (pv_fmt == SAGE_FMT_FP8 || pv_fmt == SAGE_FMT_MXFP4 || pv_fmt == SAGE_FMT_MXFP8));
  if (!pair_ok) return fail(SAGE_ERR_UNSUPPORTED, "format pair (qk=%d, pv=%d) is not supported", qk_fmt, pv_fmt);
  return SAGE_OK;
}

// The prologue grids put query / KV instances on the second grid axis.
constexpr long long kMaxInstances = 65535;

sage_status check_problem(const sage_problem* p) {
  if (!p) return fail(SAGE_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->B < 1 || p->H < 1 || p->N < 1)
    return fail(SAGE_ERR_INVALID_ARG, "B, H and N must be >= 1 (got B=%d H=%d N=%d)", p->B, p->H, p->N);
  // (token indices inside an instance are 32-bit: N up to 2^30)
  if ((long long)p->B * p->H * ((long long)p->N + sage::kTokenPad) * p->d > (1LL << 40) ||
      (long long)p->B * p->H > kMaxInstances || p->N > (1 << 30))
    return fail(SAGE_ERR_INVALID_ARG, "problem too large");
  return check_common(p->d, p->causal, p->sm_scale, p->io_dtype, p->qk_fmt, p->pv_fmt);
}

// Packed problems: token extents per head of the quantized buffers (room for every sequence
// rounded up to 128 tokens at a 64-aligned start, see SeqGeo).
size_t packed_tokens(int total, int B) { return round_up((size_t)total, 64) + 256 * (size_t)B; }

sage_status check_varlen(const sage_varlen_problem* p) {
  if (!p) return fail(SAGE_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->B < 1 || p->H < 1 || p->H_kv < 1)
    return fail(SAGE_ERR_INVALID_ARG, "B, H and H_kv must be >= 1 (got B=%d H=%d H_kv=%d)", p->B, p->H, p->H_kv);
  if (p->H % p->H_kv != 0)
    return fail(SAGE_ERR_INVALID_ARG, "H=%d is not a multiple of H_kv=%d", p->H, p->H_kv);
  if (p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
    return fail(SAGE_ERR_INVALID_ARG, "total_q, total_k, max_seqlen_q and max_seqlen_k must be >= 0");
  if (packed_tokens(p->total_q, p->B) > (size_t)INT32_MAX || packed_tokens(p->total_k, p->B) > (size_t)INT32_MAX)
    return fail(SAGE_ERR_INVALID_ARG, "problem too large");
  const long long toks = (long long)p->H * packed_tokens(p->total_q, p->B) +
                         (long long)p->H_kv * packed_tokens(p->total_k, p->B) * 2;
  if (toks * p->d > (1LL << 40) || (long long)p->B * p->H > kMaxInstances ||
      (long long)p->B * p->H * (((long long)std::min(p->max_seqlen_q, p->total_q) + 127) / 128) > (1LL << 31) - 1)
    return fail(SAGE_ERR_INVALID_ARG, "problem too large");
  // per-block Q smoothing: a dS strip of max_seqlen_k keys per 128-query block slot
  if (p->qk_fmt == SAGE_FMT_MXFP4_QBLOCK &&
      (double)p->H * (double)sage::qblock_slots_per_head(p->total_q, p->B) *
              ((std::min(p->max_seqlen_k, p->total_k) + 127) / 128 * 128.0) * 4.0 > (double)(1LL << 40))
    return fail(SAGE_ERR_INVALID_ARG, "problem too large");
  return check_common(p->d, p->causal, p->sm_scale, p->io_dtype, p->qk_fmt, p->pv_fmt);
}

sage::Shape to_shape(const sage_problem* p) {
  sage::Shape s{};
  s.B = p->B;
  s.H = p->H;
  s.N = p->N;
  s.d = p->d;
  s.Np = (int)round_up((size_t)p->N, sage::kTokenPad);
  s.causal = p->causal;
  s.io_dtype = p->io_dtype;
  s.qk_fmt = p->qk_fmt;
  s.pv_fmt = p->pv_fmt;
  s.sm_scale = p->sm_scale;
  sage::SeqGeo& g = s.g;
  g.cu_q = g.cu_k = nullptr;
  g.B = p->B;
  g.H = g.Hkv = p->H;
  g.Nq = g.Nk = p->N;
  g.Npq = g.Npk = s.Np;
  g.nbq = g.nbk = s.Np / 64;
  return s;
}

sage::Shape to_shape(const sage_varlen_problem* p, const int* cu_q, const int* cu_k) {
  sage::Shape s{};
  s.B = p->B;
  s.H = p->H;
  s.d = p->d;
  s.causal = p->causal;
  s.io_dtype = p->io_dtype;
  s.qk_fmt = p->qk_fmt;
  s.pv_fmt = p->pv_fmt;
  s.sm_scale = p->sm_scale;
  sage::SeqGeo& g = s.g;
  g.cu_q = cu_q;
  g.cu_k = cu_k;
  g.B = p->B;
  g.H = p->H;
  g.Hkv = p->H_kv;
  g.Tq = (int)packed_tokens(p->total_q, p->B);
  g.Tk = (int)packed_tokens(p->total_k, p->B);
  g.total_q = p->total_q;
  g.total_k = p->total_k;
  // no sequence is longer than its tensor: a looser bound only sized idle grids
  g.max_q = std::min(p->max_seqlen_q, p->total_q);
  g.max_k = std::min(p->max_seqlen_k, p->total_k);
  g.nbq = (int)(round_up((size_t)g.max_q, sage::kTokenPad) / 64);
  g.nbk = (int)(round_up((size_t)g.max_k, sage::kTokenPad) / 64);
  return s;
}

// Token extents of a quantized buffer.
struct Extents {
  size_t inst_q, inst_kv;   // query / KV instances (per-instance arrays: means, FP8 V steps)
  size_t tq, tk;            // tokens over all query / KV instances (multiples of 64)
  size_t ds, corr;          // dS floats (query heads x key tokens), LSE-term floats
  size_t stats_inst;        // instances of the statistics partials (B*H)
  size_t blk_cap;           // packed sequences: entries of the (sequence, block) table; else 0
  // per-block Q smoothing: slots (a mean and a dS strip per 128-query block, qblock_slot), rows
  // of the means' fp64 copy, keys per dS strip
  size_t qb_slots, qb_rows64, qb_strip;
};

Extents extents(const sage_problem* p) {
  const size_t BH = (size_t)p->B * p->H, Np = round_up((size_t)p->N, sage::kTokenPad), nqb = Np / 128;
  return Extents{BH, BH, BH * Np, BH * Np, BH * Np, BH * (size_t)p->N, BH, 0,
                 BH * nqb, BH * (size_t)sage::qblock_padded((int)nqb), Np};
}
// (packed: the slots' fp64 rows plus 16, which the dS step's 16-slot operand reads may reach)
Extents extents(const sage_varlen_problem* p) {
  const size_t Tq = packed_tokens(p->total_q, p->B), Tk = packed_tokens(p->total_k, p->B);
  const size_t BH = (size_t)p->B * p->H;
  const size_t slots = (size_t)p->H * (size_t)sage::qblock_slots_per_head(p->total_q, p->B);
  return Extents{BH, (size_t)p->B * p->H_kv, p->H * Tq, p->H_kv * Tk, p->H * Tk, p->H * Tq, BH,
                 (size_t)sage::seq_block_capacity(p->total_q, p->total_k, p->B),
                 slots, slots + 16, round_up((size_t)std::min(p->max_seqlen_k, p->total_k), 128)};
}

void compute_layout(const Extents& E, int d_, int qk_fmt, int pv_fmt, sage_quant_layout* L) {
  const size_t d = d_;
  const bool qblk = qk_fmt == SAGE_FMT_MXFP4_QBLOCK;
  const bool mx = qk_fmt == SAGE_FMT_MXFP4 || qblk, mxv = pv_fmt == SAGE_FMT_MXFP4, mx8v = pv_fmt == SAGE_FMT_MXFP8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L->mu_k = take(E.inst_kv * d * 4);
  // per-block Q smoothing: a mean per 128-query block (then the same means in fp64, padded: the
  // dS step's operand), a dS strip per block
  L->mu_q = take(qblk ? E.qb_slots * d * 4 + E.qb_rows64 * d * 8 : E.inst_q * d * 4);
  L->q_codes = take(mx ? E.tq * d / 2 : E.tq * d);
  const bool tok = qk_fmt == SAGE_FMT_INT8_TOKEN;
  L->q_scales = take(mx ? E.tq * (d / 32) : tok ? E.tq * 4 : E.tq / 64 * 4);
  L->k_codes = take(mx ? E.tk * d / 2 : E.tk * d);
  L->k_scales = take(mx ? E.tk * (d / 32) : tok ? E.tk / 32 * 4 : E.tk / 64 * 4);
  L->v_codes = take(mxv ? E.tk * d / 2 : pv_fmt == SAGE_FMT_F16 ? E.tk * d * 2 : E.tk * d);
  L->v_scales = take(mxv || mx8v ? E.tk / 32 * d : E.inst_kv * d * 4);
  L->delta_s = take(qblk ? E.qb_slots * E.qb_strip * 4 : E.ds * 4);
  L->lse_corr = take(E.corr * 4);
  // statistics partials, then (packed sequences) the (sequence, block) table: int2 [1 + cap]
  L->stats = take(sage::kStatChunks * (E.stats_inst * d * 8 * 2 + E.stats_inst * d * 4) +
                  (E.blk_cap ? 8 * (E.blk_cap + 1) : 0));
  L->total = off;
}
void compute_layout(const sage_problem* p, sage_quant_layout* L) {
  compute_layout(extents(p), p->d, p->qk_fmt, p->pv_fmt, L);
}

sage::QuantPtrs resolve(void* buf, size_t BH, int d, const sage_quant_layout& L) {
  uint8_t* b = static_cast<uint8_t*>(buf);
  sage::QuantPtrs q;
  q.mu_k = reinterpret_cast<float*>(b + L.mu_k);
  q.mu_q = reinterpret_cast<float*>(b + L.mu_q);
  q.q_codes = b + L.q_codes;
  q.q_scales = b + L.q_scales;
  q.k_codes = b + L.k_codes;
  q.k_scales = b + L.k_scales;
  q.v_codes = b + L.v_codes;
  q.v_scales = b + L.v_scales;
  q.delta_s = reinterpret_cast<float*>(b + L.delta_s);
  q.lse_corr = reinterpret_cast<float*>(b + L.lse_corr);
  q.sums = reinterpret_cast<double*>(b + L.stats);
  q.amax_v = reinterpret_cast<uint32_t*>(b + L.stats + sage::kStatChunks * BH * d * 8 * 2);
  q.blocks = b + L.stats + sage::kStatChunks * BH * d * (8 * 2 + 4);
  return q;
}
sage::QuantPtrs resolve(void* buf, const sage_problem* p, const sage_quant_layout& L) {
  return resolve(buf, (size_t)p->B * p->H, p->d, L);
}

sage_problem make_problem(int B, int H, int N, int d, int causal, float sm, int io, int qk, int pv) {
  sage_problem p;
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.causal = causal;
  p.sm_scale = sm;
  p.io_dtype = io;
  p.qk_fmt = qk;
  p.pv_fmt = pv;
  return p;
}

sage_status check_tensors(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs) {
    if (!x) return fail(SAGE_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if (!aligned16(x)) return fail(SAGE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  return SAGE_OK;
}

// ---- scratch of the no-allocation forward (sage_attn_fwd_noalloc) ----
// One fixed array per GPU, in the library's device code, holding the quantized buffer of one
// problem.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in): hipGetSymbolAddress gives its device address, once per device with that device
// current, and that address is what the kernels receive.  Calls on one GPU share it, so
// calls that overlap on one GPU race.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device that runs `stream` (the current device
// for the null stream), looked up on the first call for that device.
sage_status scratch_for(void* stream, void** out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice((hipStream_t)stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    hipError_t r = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    }
    if (r != hipSuccess) return hip_fail(r, "hipSetDevice");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SAGE_OK;
}

// ---- SAGE_LOG=1: one line on stderr per outermost entry-point call (name, problem, status) ----
bool log_on() {
  const char* e = getenv("SAGE_LOG");
  return e && strcmp(e, "1") == 0;
}
thread_local int g_depth = 0;   // entry points calling entry points log once
struct CallScope {
  CallScope() { ++g_depth; }
  ~CallScope() { --g_depth; }
};
std::string describe(const sage_problem* p) {
  if (!p) return "problem=NULL";
  char b[160];
  snprintf(b, sizeof b, "B=%d H=%d N=%d d=%d causal=%d sm=%g io=%d qk=%d pv=%d", p->B, p->H, p->N, p->d, p->causal,
           (double)p->sm_scale, p->io_dtype, p->qk_fmt, p->pv_fmt);
  return b;
}
std::string describe(const sage_varlen_problem* p) {
  if (!p) return "problem=NULL";
  char b[200];
  snprintf(b, sizeof b, "B=%d H=%d H_kv=%d d=%d causal=%d sm=%g io=%d qk=%d pv=%d total_q=%d total_k=%d max_q=%d max_k=%d",
           p->B, p->H, p->H_kv, p->d, p->causal, (double)p->sm_scale, p->io_dtype, p->qk_fmt, p->pv_fmt, p->total_q,
           p->total_k, p->max_seqlen_q, p->max_seqlen_k);
  return b;
}
// (the problem text is formatted only when the line is printed)
template <typename Describe>
sage_status logged(const char* fn, Describe what, sage_status s) {
  if (g_depth == 1 && log_on())
    fprintf(stderr, "sage: %s(%s) -> %s%s%s\n", fn, what().c_str(), sage_status_string(s), s == SAGE_OK ? "" : ": ",
            s == SAGE_OK ? "" : g_err);
  return s;
}

// The backward behind both entry points; requant false: the quant buffer at the front of ws
// already holds the forward's quantization of these q and k.
sage_status bwd_impl(const sage_problem* p, const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     bool requant, void* stream) {
  size_t need = 0;
  sage_status s = sage_attn_bwd_ws_size(p, &need);
  if (s != SAGE_OK) return s;
  if ((s = check_tensors({q, k, v, o, dout, lse, dq, dk, dv, ws})) != SAGE_OK) return s;
  if (ws_bytes < need) return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  sage_quant_layout L;
  compute_layout(p, &L);
  hipError_t e = sage::launch_attn_bwd(to_shape(p), q, k, v, o, dout, lse, dq, dk, dv, ws, L.total,
                                       resolve(ws, p, L), requant, (hipStream_t)stream);
  return e == hipSuccess ? SAGE_OK : hip_fail(e, "backward launch");
}

}  // namespace

extern "C" {

int sage_abi_version(void) { return SAGE_ABI_VERSION; }

const char* sage_last_error(void) { return g_err; }

const char* sage_status_string(sage_status s) {
  // a C caller may pass any int; reading it as the enum type would be undefined for values
  // outside the enumerators' range, so take its bits as an int
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_INVALID_ARG: return "invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "unsupported";
    case SAGE_ERR_WORKSPACE: return "workspace too small";
    case SAGE_ERR_OUT_OF_MEMORY: return "out of device memory";
    case SAGE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

sage_status sage_quant_size(const sage_problem* p, size_t* bytes, sage_quant_layout* layout) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(p);
    if (s != SAGE_OK) return s;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
    sage_quant_layout L;
    compute_layout(p, &L);
    *bytes = L.total;
    if (layout) *layout = L;
    return SAGE_OK;
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_quantize(const void* q, const void* k, const void* v, const sage_problem* p, void* quant_buf,
                          size_t quant_bytes, void* stream) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(p);
    if (s != SAGE_OK) return s;
    if ((s = check_tensors({q, k, v, quant_buf})) != SAGE_OK) return s;
    sage_quant_layout L;
    compute_layout(p, &L);
    if (quant_bytes < L.total)
      return fail(SAGE_ERR_WORKSPACE, "quant buffer has %zu bytes, needs %zu", quant_bytes, L.total);
    hipError_t e = sage::launch_prologue(q, k, v, to_shape(p), resolve(quant_buf, p, L), (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : hip_fail(e, "quantize launch");
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_fwd_quantized(const void* quant_buf, size_t quant_bytes, const sage_problem* p, void* o,
                                    float* lse, void* stream) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(p);
    if (s != SAGE_OK) return s;
    if ((s = check_tensors({quant_buf, o})) != SAGE_OK) return s;
    if (lse && !aligned16(lse)) return fail(SAGE_ERR_INVALID_ARG, "lse must be 16-byte aligned");
    sage_quant_layout L;
    compute_layout(p, &L);
    if (quant_bytes < L.total)
      return fail(SAGE_ERR_WORKSPACE, "quant buffer has %zu bytes, needs %zu", quant_bytes, L.total);
    hipError_t e = sage::launch_attn_fwd(to_shape(p), resolve(const_cast<void*>(quant_buf), p, L), o, lse,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : hip_fail(e, "attention launch");
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_fwd_ws_size(const sage_problem* p, size_t* bytes) { return sage_quant_size(p, bytes, nullptr); }

sage_status sage_attn_fwd_ex(const sage_problem* p, const void* q, const void* k, const void* v, void* o, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(p);
    if (s != SAGE_OK) return s;
    if ((s = check_tensors({q, k, v, o, ws})) != SAGE_OK) return s;
    if (lse && !aligned16(lse)) return fail(SAGE_ERR_INVALID_ARG, "lse must be 16-byte aligned");
    sage_quant_layout L;
    compute_layout(p, &L);
    if (ws_bytes < L.total) return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    const sage::Shape sh = to_shape(p);
    const sage::QuantPtrs qp = resolve(ws, p, L);
    hipError_t e = sage::launch_prologue(q, k, v, sh, qp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    e = sage::launch_attn_fwd(sh, qp, o, lse, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : hip_fail(e, "attention launch");
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int causal,
                          float sm_scale, int qk_fmt, int pv_fmt, void* stream) {
  sage_problem p = make_problem(B, H, N, d, causal, sm_scale, SAGE_DT_BF16, qk_fmt, pv_fmt);
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(&p);
    if (s != SAGE_OK) return s;
    if ((s = check_tensors({q, k, v, o})) != SAGE_OK) return s;
    size_t bytes = 0;
    sage_quant_size(&p, &bytes, nullptr);
    void* ws = nullptr;
    if (inject_alloc_failure()) return fail(SAGE_ERR_OUT_OF_MEMORY, "injected allocation failure");
    hipError_t e = hipMallocAsync(&ws, bytes, (hipStream_t)stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(SAGE_ERR_OUT_OF_MEMORY, "hipMallocAsync(%zu): %s", bytes, hipGetErrorString(e));
    }
    s = sage_attn_fwd_ex(&p, q, k, v, o, nullptr, ws, bytes, stream);
    hipError_t f = hipFreeAsync(ws, (hipStream_t)stream);
    if (s == SAGE_OK && f != hipSuccess) return hip_fail(f, "hipFreeAsync");
    return s;
  }();
  return logged(__func__, [&] { return describe(&p); }, st_);
}

sage_status sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                                  int causal, float sm_scale, int qk_fmt, int pv_fmt, void* stream) {
  sage_problem p = make_problem(B, H, N, d, causal, sm_scale, SAGE_DT_BF16, qk_fmt, pv_fmt);
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(&p);
    if (s != SAGE_OK) return s;
    if ((s = check_tensors({q, k, v, o})) != SAGE_OK) return s;
    size_t bytes = 0;
    sage_quant_size(&p, &bytes, nullptr);
    if (bytes > kScratchBytes)
      return fail(SAGE_ERR_WORKSPACE, "the problem needs %zu bytes of scratch; the no-allocation entry holds %zu "
                  "(use sage_attn_fwd_ex with a caller workspace)", bytes, kScratchBytes);
    void* ws = nullptr;
    if ((s = scratch_for(stream, &ws)) != SAGE_OK) return s;
    return sage_attn_fwd_ex(&p, q, k, v, o, nullptr, ws, bytes, stream);
  }();
  return logged(__func__, [&] { return describe(&p); }, st_);
}

sage_status sage_attn_bwd_ws_size(const sage_problem* p, size_t* bytes) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_problem(p);
    if (s != SAGE_OK) return s;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
    if (p->qk_fmt != SAGE_FMT_INT8 || p->pv_fmt != SAGE_FMT_FP8)
      return fail(SAGE_ERR_UNSUPPORTED, "the backward supports qk_fmt=INT8, pv_fmt=FP8 only");
    sage_quant_layout L;
    compute_layout(p, &L);
    *bytes = L.total + sage::attn_bwd_ws_bytes(to_shape(p));
    return SAGE_OK;
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_bwd(const sage_problem* p, const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                          void* stream) {
  CallScope cs_;
  const sage_status st_ = bwd_impl(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, true, stream);
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_bwd_after_fwd(const sage_problem* p, const void* q, const void* k, const void* v,
                                    const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                    void* ws, size_t ws_bytes, void* stream) {
  CallScope cs_;
  const sage_status st_ = bwd_impl(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, false, stream);
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_varlen_ws_size(const sage_varlen_problem* p, size_t* bytes) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_varlen(p);
    if (s != SAGE_OK) return s;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
    sage_quant_layout L;
    compute_layout(extents(p), p->d, p->qk_fmt, p->pv_fmt, &L);
    *bytes = L.total;
    return SAGE_OK;
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

sage_status sage_attn_varlen_fwd(const sage_varlen_problem* p, const void* q, const void* k, const void* v,
                                 const int* cu_seqlens_q, const int* cu_seqlens_k, void* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  CallScope cs_;
  const sage_status st_ = [&]() -> sage_status {
    sage_status s = check_varlen(p);
    if (s != SAGE_OK) return s;
    if (!cu_seqlens_q || !cu_seqlens_k || (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
      return fail(SAGE_ERR_INVALID_ARG, "cu_seqlens_q / cu_seqlens_k must be non-NULL, 4-byte aligned");
    if (p->total_q == 0) return SAGE_OK;   // no query rows: nothing to compute
    if ((s = check_tensors({q, o, ws})) != SAGE_OK) return s;
    if (p->total_k > 0 && (s = check_tensors({k, v})) != SAGE_OK) return s;
    if (lse && !aligned16(lse)) return fail(SAGE_ERR_INVALID_ARG, "lse must be 16-byte aligned");
    sage_quant_layout L;
    compute_layout(extents(p), p->d, p->qk_fmt, p->pv_fmt, &L);
    if (ws_bytes < L.total) return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    const sage::Shape sh = to_shape(p, cu_seqlens_q, cu_seqlens_k);
    const sage::QuantPtrs qp = resolve(ws, (size_t)p->B * p->H, p->d, L);
    hipError_t e = sage::launch_prologue(q, k, v, sh, qp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    if (sh.g.nbq == 0) return SAGE_OK;     // max_seqlen_q == 0: every sequence is empty
    e = sage::launch_attn_fwd(sh, qp, o, lse, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : hip_fail(e, "attention launch");
  }();
  return logged(__func__, [&] { return describe(p); }, st_);
}

}  // extern "C"
