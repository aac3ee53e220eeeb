// sage_launch.hpp -- host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <algorithm>
#include <stdint.h>
#include <stdlib.h>

namespace sage {

// QK_INT8T: INT8 codes with a step per query token and per 32 keys (instead of per 64 tokens);
// QK_MXFP4B: MXFP4 with Q smoothed per 128-query block (dS per block and key)
enum { QK_INT8 = 1, QK_MXFP4 = 3, QK_INT8T = 6, QK_MXFP4B = 7 };
// PV_NONE: quantize Q and K only (the backward needs no V codes)
enum { PV_NONE = 0, PV_FP8 = 2, PV_MXFP4 = 3, PV_MXFP8 = 4, PV_F16 = 5 };

// Padding of the token axis in every quantized buffer (a multiple of the Q tile).
constexpr int kTokenPad = 128;
// Token chunks per head of the smoothing statistics (partial sums are kept per chunk).
constexpr int kStatChunks = 8;

// Per-block Q smoothing: the fp64 copy of the block means (the dS kernel's MFMA A operand)
// has this many rows, a whole number of 16-block groups.
inline int qblock_padded(int nb) { return (nb + 15) / 16 * 16; }

// Device pointers of one quantized buffer (offsets resolved on the host).
struct QuantPtrs {
  float* mu_k;
  float* mu_q;        // [BH, d], or [BH, Np/128, d] per 128-query block (QK_MXFP4B; then
                      // followed by the fp64 copy [BH, qblock_padded(Np/128), d])
  uint8_t* q_codes;
  void* q_scales;     // fp32 [BH, nb] (INT8), fp32 [BH, Np] (INT8T) or uint8 E8M0 [BH, Np, d/32] (MXFP4)
  uint8_t* k_codes;
  void* k_scales;
  uint8_t* v_codes;
  void* v_scales;     // fp32 [BH, d] (FP8) or uint8 E8M0 [BH, Np/32, d] (MXFP4, MXFP8)
  float* delta_s;     // [BH, Np], or [BH, Np/128, Np] per query block (QK_MXFP4B)
  float* lse_corr;
  double* sums;       // [2, kStatChunks, B*H, d]: K then Q token sums per chunk (K by KV instance)
  uint32_t* amax_v;   // [kStatChunks, B*H, d] bit patterns of max |V| per channel (by KV instance)
  void* blocks;       // packed sequences: int2 [1 + seq_block_capacity] table of (sequence, block)
};

// Token geometry of a problem.  Fixed length: B sequences of Nq query and Nk key tokens in
// [B,H,Nq,d] / [B,Hkv,Nk,d] tensors; instance (b, h) owns Npq (Npk) consecutive tokens of
// the quantized buffers from (b H + h) Npq on.  Packed (cu_q != null): sequence b is rows
// [cu[b], cu[b+1]) of [total,H,d] / [total,Hkv,d] tensors, and head h of sequence b owns
// the tokens from h T + roundup64(cu[b]) + 256 b on: room for the sequence rounded up to
// 128 tokens, found without a prefix sum over the batch.
struct SeqGeo {
  const int* cu_q;   // packed: device [B+1] query row offsets; null: fixed length
  const int* cu_k;   // packed: device [B+1] key row offsets
  int B, H, Hkv;     // H query heads; query head h reads KV head h / (H / Hkv)
  int Nq, Nk;        // fixed length: tokens per sequence
  int Npq, Npk;      // fixed length: tokens per instance in the quantized buffers
  int Tq, Tk;        // packed: tokens per head in the quantized buffers
  int total_q;       // packed: rows of q (the stride of the [H, total_q] LSE)
  int total_k;       // packed: rows of k and v
  int max_q, max_k;  // packed: the longest sequence the caller declares
  int nbq, nbk;      // 64-token blocks covering the longest query / key instance (to 128 tokens)
};

// One (sequence, head) instance of Q or of K/V.
struct Inst {
  int len;           // tokens
  size_t tok0;       // first token in the quantized buffers (a multiple of 64)
  size_t io0;        // element offset of token 0 in the I/O tensor
  int ios;           // elements from one token to the next in the I/O tensor
  size_t row0;       // packed / fixed per-token fp32 arrays (LSE correction)
  size_t lse0;       // LSE output: [B,H,Nq] fixed, [H,total_q] packed
};

// Packed sequences: the (sequence, 64-token block) pairs there can be -- each sequence b has
// 2 ceil(max(len_q, len_k) / 128) <= (len_q + len_k) / 64 + 2 of them.
inline int seq_block_capacity(long long total_q, long long total_k, long long B) {
  return (int)((total_q + total_k) / 64 + 2 * B + 1);
}
inline int seq_block_capacity(const SeqGeo& g) { return seq_block_capacity(g.total_q, g.total_k, g.B); }

// Per-block Q smoothing (QK_MXFP4B): query block qb of query instance (b, h) -- its 128
// queries from the sequence's first one, the fused kernel's query tile qb -- owns row `slot` of
// the block means and the dS strip [slot * strip, slot * strip + strip) over the KV instance's
// keys.  Fixed length: slot (b H + h) Npq / 128 + qb, strips of Npk keys.  Packed: total_q / 128
// + B + 1 slots per head, sequence b's from floor(start / 128) + b on (its ceil(len / 128)
// blocks end before sequence b + 1's first slot, since floor(s / 128) + ceil(len / 128) <=
// floor((s + len) / 128) + 1), strips of max_k rounded up to 128 keys.
__host__ __device__ inline long long qblock_slots_per_head(long long total_q, long long B) { return total_q / 128 + B + 1; }
inline size_t qblock_slots(const SeqGeo& g) {
  return g.cu_q ? (size_t)g.H * qblock_slots_per_head(g.total_q, g.B) : (size_t)g.B * g.H * (g.Npq / 128);
}
// (packed: every key length is clamped to max_k and cannot exceed total_k)
inline size_t qblock_strip(const SeqGeo& g) {
  return g.cu_q ? ((size_t)std::min(g.max_k, g.total_k) + 127) / 128 * 128 : (size_t)g.Npk;
}

#if defined(__HIPCC__)
// Packed sequence b: its first row and length, clamped so that any offsets keep every access
// inside the buffers (start in [0, total], length in [0, min(max_len, total - start)]).
__device__ __forceinline__ void packed_seq(const int* cu, int b, int total, int max_len, int& s, int& len) {
  s = min(max(cu[b], 0), total);
  const int e = min(max(cu[b + 1], s), total);
  len = min(e - s, max_len);
}
// First token of sequence b (starting at row s) in a head's packed region: a multiple of 64
// with room for the sequence rounded up to 128 before the next sequence's start.
__device__ __forceinline__ size_t packed_base(int s, int b) {
  return (size_t)((s + 63) & ~63) + 256 * (size_t)b;
}
__device__ __forceinline__ Inst q_inst(const SeqGeo& g, int b, int h, int d) {
  Inst r;
  if (g.cu_q) {
    int s;
    packed_seq(g.cu_q, b, g.total_q, g.max_q, s, r.len);
    r.tok0 = (size_t)h * g.Tq + packed_base(s, b);
    r.io0 = ((size_t)s * g.H + h) * d;
    r.ios = g.H * d;
    r.row0 = r.tok0;
    r.lse0 = (size_t)h * g.total_q + s;
  } else {
    const size_t i = (size_t)b * g.H + h;
    r.len = g.Nq;
    r.tok0 = i * g.Npq;
    r.io0 = i * g.Nq * d;
    r.ios = d;
    r.row0 = i * g.Nq;
    r.lse0 = r.row0;
  }
  return r;
}
__device__ __forceinline__ Inst k_inst(const SeqGeo& g, int b, int hk, int d) {
  Inst r;
  if (g.cu_k) {
    int s;
    packed_seq(g.cu_k, b, g.total_k, g.max_k, s, r.len);
    r.tok0 = (size_t)hk * g.Tk + packed_base(s, b);
    r.io0 = ((size_t)s * g.Hkv + hk) * d;
    r.ios = g.Hkv * d;
  } else {
    const size_t i = (size_t)b * g.Hkv + hk;
    r.len = g.Nk;
    r.tok0 = i * g.Npk;
    r.io0 = i * g.Nk * d;
    r.ios = d;
  }
  r.row0 = r.lse0 = 0;
  return r;
}
// Per-block Q smoothing: the slot of query block qb of query instance (b, h) (see
// qblock_slots_per_head); packed starts and lengths are clamped as in packed_seq, so even
// malformed offsets give slots below the head's count.
__device__ __forceinline__ size_t qblock_slot(const SeqGeo& g, int b, int h, int qb) {
  if (!g.cu_q) return ((size_t)b * g.H + h) * (g.Npq / 128) + qb;
  int s, len;
  packed_seq(g.cu_q, b, g.total_q, g.max_q, s, len);
  return (size_t)h * (size_t)qblock_slots_per_head(g.total_q, g.B) + (size_t)(s / 128 + b + qb);
}
// First key token of query head h's dS strip (MXFP4 QK: mu_q(h) . K_s per key).
__device__ __forceinline__ size_t ds_base(const SeqGeo& g, int b, int h) {
  if (!g.cu_k) return ((size_t)b * g.H + h) * g.Npk;
  int s, len;
  packed_seq(g.cu_k, b, g.total_k, g.max_k, s, len);
  return (size_t)h * g.Tk + packed_base(s, b);
}
#endif

// SAGE_DEBUG_LDS_PAD=<bytes>: extra dynamic LDS on the fused forward and backward launches, up
// to what one workgroup may hold, so that fewer workgroups share a CU.  For debugging: the
// results must not change (a difference would reveal an LDS race or a timing dependence).
template <typename Kernel>
inline size_t debug_lds_pad(Kernel kernel) {
  const char* e = getenv("SAGE_DEBUG_LDS_PAD");
  const long want = e ? strtol(e, nullptr, 10) : 0;
  if (want <= 0) return 0;
  int dev = 0, cap = 0;
  hipFuncAttributes at;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cap, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipFuncGetAttributes(&at, reinterpret_cast<const void*>(kernel)) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const size_t room = (size_t)cap > at.sharedSizeBytes ? (size_t)cap - at.sharedSizeBytes : 0;
  return std::min((size_t)want, room);
}

struct Shape {
  int B, H, N, d, Np, causal, io_dtype, qk_fmt, pv_fmt;
  float sm_scale;
  SeqGeo g;          // N / Np above are the fixed-length Nq = Nk and Npq = Npk
};

hipError_t launch_prologue(const void* q, const void* k, const void* v, const Shape& s,
                           const QuantPtrs& qp, hipStream_t stream);
hipError_t launch_attn_fwd(const Shape& s, const QuantPtrs& qp, void* o, float* lse, hipStream_t stream);

// Backward: the workspace is [forward quant buffer (qbytes) | backward extras];
// attn_bwd_ws_bytes gives the size of the extras.  requant false: the quant buffer already holds
// the forward's quantization of these q, k (the Q/K codes, steps, mu_k and LSE term are reused).
size_t attn_bwd_ws_bytes(const Shape& s);
hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                           size_t qbytes, const QuantPtrs& qp, bool requant, hipStream_t stream);

}  // namespace sage
