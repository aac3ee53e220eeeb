// prologue.hip -- the smoothing + quantization prologue (HBM-bound).
//
// Smoothing K: subtract the per-channel token mean of K before quantizing; it
// shifts every score of a query row by the same constant, so softmax is
// unchanged (SageAttention contributions, reply to reviewer wwcu W1).  Smooth
// Q for the 4-bit QK^T: Q - mean(Q), with the removed part mean(Q).K_s added
// back to every score (SageAttention2 abstract).  Per-block INT8 codes for Q
// and K (SageAttn-B, reply to reviewer xY6z W1-(2)); FP8 V (SageAttention2
// abstract); microscaling FP4 (SageAttention3 abstract) in the OCP MX layout.
//
// Two passes over the inputs:
//   stats:  per token chunk (kChunks chunks per head) exact fp64 per-channel
//           token sums of K (and Q) and max |V| per channel.  Every partial sum
//           of bf16/fp16 values at these sizes is exactly representable in fp64,
//           so the result does not depend on summation order.
//   codes:  one workgroup per 64-token block reduces the chunk partials (fixed
//           order), then writes smoothed values' block scales and codes, the
//           dS / LSE correction terms, and V transposed into tiles.
// Quotients x / step are formed as q0 = x * r, q = q0 + r * (x - step * q0) with
// r = 1 / step correctly rounded once per block: for quotients in the normal range
// this gives the correctly rounded x / step (Markstein's theorem), i.e. the same
// value as one IEEE division, at a fraction of the cost.
#include <type_traits>

#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

constexpr int kChunks = kStatChunks;

// Correctly rounded x / d (d > 0) by one correction step of the reciprocal (Markstein).  A step
// below 2^-64 (a block of subnormal or tiny inputs) has a reciprocal beyond binary32, so x and d
// are first scaled by the same power of two s = div_scale(d), exactly; r = recip_rn(d) is the
// reciprocal of the scaled step.  The correction turns x = -0 into +0, so the sign is taken
// from x (d > 0: a no-op for x != 0).
__device__ __forceinline__ float div_scale(float d) { return d < 0x1p-64f ? 0x1p64f : 1.0f; }
__device__ __forceinline__ float recip_rn(float d) { return 1.0f / (d * div_scale(d)); }
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  const float s = div_scale(d);
  const float xs = x * s, ds = d * s;
  const float q0 = xs * r;
  return copysignf(fmaf(r, fmaf(-ds, q0, xs), q0), x);
}

// 16 bytes = 8 contiguous 16-bit inputs, widened.
template <int DT>
__device__ __forceinline__ void unpack8(uint4 u, float* x) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = DT == 0 ? bf16_to_f32(w[i] & 0xffff) : f16_to_f32(w[i] & 0xffff);
    x[2 * i + 1] = DT == 0 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
  }
}
// The raw 16 bytes of row `row` of an instance at channel c0, or zeros past its end.
__device__ __forceinline__ uint4 row_raw(const uint16_t* x, const Inst& in, bool active, int row, int c0) {
  return active && row < in.len ? *reinterpret_cast<const uint4*>(x + in.io0 + (size_t)row * in.ios + c0)
                                : make_uint4(0, 0, 0, 0);
}
template <int DT>
__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = DT == 0 ? bf16_to_f32(w[i] & 0xffff) : f16_to_f32(w[i] & 0xffff);
    x[2 * i + 1] = DT == 0 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
  }
}

// Partial statistics of chunk c of one instance: tokens [c CH, (c+1) CH) with
// CH = ceil(len / kChunks).  Per-channel fp64 sums of x into out_sum[D] and, when AMAXV,
// max |v| bit patterns into out_amax[D].
template <int DT, int D, bool AMAXV>
__device__ __forceinline__ void chunk_stats(const uint16_t* __restrict__ x, const uint16_t* __restrict__ v,
                                            const Inst& in, int c, double* out_sum, uint32_t* out_amax,
                                            double (*s_x)[D], uint32_t (*s_v)[D]) {
  constexpr int C8 = D / 8, RP = 256 / C8;
  const int CH = (in.len + kChunks - 1) / kChunks;
  const int t0 = c * CH, t1 = min(in.len, t0 + CH);
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  double sx[8] = {};
  uint32_t av[8] = {};
  // four rows per thread and step, all loads issued before any is used (the 16-bit sums are
  // exact in fp64, so the order does not matter); a row past the chunk reads row t0 (valid)
  // and counts as zero
  constexpr int U = 4;
  for (int r = t0 + r0; r < t1; r += U * RP) {
    float y[U][8], z[U][8];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int rr = r + u * RP < t1 ? r + u * RP : t0;
      load8<DT>(x + in.io0 + (size_t)rr * in.ios + c0, y[u]);
      if (AMAXV) load8<DT>(v + in.io0 + (size_t)rr * in.ios + c0, z[u]);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const bool ok = r + u * RP < t1;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        sx[i] += ok ? (double)y[u][i] : 0.0;
        if (AMAXV) av[i] = max(av[i], ok ? __float_as_uint(fabsf(z[u][i])) : 0u);   // NaN-propagating
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    s_x[r0][c0 + i] = sx[i];
    if (AMAXV) s_v[r0][c0 + i] = av[i];
  }
  __syncthreads();
  if (tid < D) {
    double a = 0.0;
    uint32_t m = 0;
    for (int r = 0; r < RP; r++) {
      a += s_x[r][tid];
      if (AMAXV) m = max(m, s_v[r][tid]);
    }
    out_sum[tid] = a;
    if (AMAXV) out_amax[tid] = m;
  }
  __syncthreads();   // s_x is reused by the next call
}

// grid (kChunks, B*H), 256 threads.  Block (c, i): chunk c of KV instance i (i < B*Hkv) --
// sums of K into sums[c][i][D], max |V| (AMAXV) into amax[c][i][D] -- and, when SUMQ, of
// query instance i: sums of Q into sums[kChunks + c][i][D].
template <int DT, int D, bool SUMQ, bool AMAXV>
__global__ __launch_bounds__(256) void stats_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, SeqGeo g,
                                                    double* __restrict__ sums, uint32_t* __restrict__ amax_v) {
  constexpr int RP = 256 / (D / 8);
  const int i = blockIdx.y, c = blockIdx.x, BHm = g.B * g.H;
  __shared__ double s_x[RP][D];
  __shared__ uint32_t s_v[AMAXV ? RP : 1][D];
  if (i < g.B * g.Hkv) {
    const Inst ki = k_inst(g, i / g.Hkv, i % g.Hkv, D);
    chunk_stats<DT, D, AMAXV>(k, v, ki, c, sums + ((size_t)c * BHm + i) * D, amax_v + ((size_t)c * BHm + i) * D,
                              s_x, s_v);
  }
  if (SUMQ) {
    const Inst qi = q_inst(g, i / g.H, i % g.H, D);
    chunk_stats<DT, D, false>(q, nullptr, qi, c, sums + ((size_t)(kChunks + c) * BHm + i) * D, nullptr, s_x, s_v);
  }
}

// Reductions of the chunk partials for channel ch of instance inst (fixed order); an empty
// instance has mean 0.
__device__ __forceinline__ float chunk_mean(const double* sums, int part, int BHm, int inst, int D, int ch, int N) {
  if (N == 0) return 0.0f;
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < kChunks; c++) s += sums[((size_t)(part * kChunks + c) * BHm + inst) * D + ch];
  return (float)(s / (double)N);
}
__device__ __forceinline__ float chunk_amax(const uint32_t* amax, int BHm, int inst, int D, int ch) {
  uint32_t m = 0;
#pragma unroll
  for (int c = 0; c < kChunks; c++) m = max(m, amax[((size_t)c * BHm + inst) * D + ch]);
  return __uint_as_float(m);
}

// Block-wide max of two non-negative float bit patterns at once (NaN-propagating), 256 threads.
__device__ __forceinline__ void block_umax2(uint32_t& x, uint32_t& y, uint32_t* red) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    x = max(x, (uint32_t)__shfl_xor((int)x, o));
    y = max(y, (uint32_t)__shfl_xor((int)y, o));
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = x;
    red[4 + (threadIdx.x >> 6)] = y;
  }
  __syncthreads();
  x = max(max(red[0], red[1]), max(red[2], red[3]));
  y = max(max(red[4], red[5]), max(red[6], red[7]));
}

// clamp(rne(x / step), -127, 127), x / step correctly rounded via r = recip_rn(step).
__device__ __forceinline__ int8_t int8_code(float x, float step, float r) {
  if (step == 0.0f) return 0;
  float n = rintf(div_rn(x, step, r));
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return (int8_t)n;
}


// Fixed-length problems without grouped heads (every instance N tokens, query head bh reads
// KV instance bh): the streamlined codes kernels.

// Writes this thread's 8 fp16 V values (RNE) of token row `rl` into the [D][64] LDS transpose tile.
__device__ __forceinline__ void put_v_f16(uint16_t* s_vt, int rl, int c0, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; i++) s_vt[(c0 + i) * 64 + rl] = __builtin_bit_cast(uint16_t, (_Float16)x[i]);
}

// FP8 V of one 64-token block into its [D][64] tile of v_codes at `dst` (code = E4M3 of v over
// the channel step, zero past the instance's end), through an LDS tile of 68-byte rows.  Thread
// (c0, g) converts rows NP g .. NP g + NP - 1 at channels c0 .. c0 + 7, so a channel's NP codes
// form one 32- or 16-bit word and a wave's LDS writes spread over the banks (one byte per write,
// as the tile's natural order gives, puts 16 lanes on one bank).  Ends with a barrier and the
// tile's coalesced 16-byte stores.
constexpr int kVRow = 68;
// row8(j, x): the 8 inputs at channels c0 .. c0 + 7 of the block's token row NP g + j (zeros
// past the instance's end)
template <int D, typename RowLoad>
__device__ __forceinline__ void v_block_fp8_rows(RowLoad row8, int c0, int g, const float* dv, const float* rv,
                                                 uint8_t* s_vt, uint8_t* dst) {
  constexpr int NP = 64 / (256 / (D / 8));
  uint32_t cw[8];
#pragma unroll
  for (int i = 0; i < 8; i++) cw[i] = 0;
#pragma unroll
  for (int j = 0; j < NP; j += 2) {
    float x0[8], x1[8];
    row8(j, x0);
    row8(j + 1, x1);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float a = dv[i] == 0.0f ? 0.0f : div_rn(x0[i], dv[i], rv[i]);
      const float b = dv[i] == 0.0f ? 0.0f : div_rn(x1[i], dv[i], rv[i]);
      cw[i] = (uint32_t)(j == 0 ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)cw[i], false)
                                : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)cw[i], true));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if (NP == 4) *reinterpret_cast<uint32_t*>(s_vt + (c0 + i) * kVRow + 4 * g) = cw[i];
    else *reinterpret_cast<uint16_t*>(s_vt + (c0 + i) * kVRow + 2 * g) = (uint16_t)cw[i];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D * 4; c += 256) {
    const uint8_t* src = s_vt + (c / 4) * kVRow + 16 * (c % 4);
    const uint4 w = make_uint4(*reinterpret_cast<const uint32_t*>(src), *reinterpret_cast<const uint32_t*>(src + 4),
                               *reinterpret_cast<const uint32_t*>(src + 8), *reinterpret_cast<const uint32_t*>(src + 12));
    *reinterpret_cast<uint4*>(dst + c * 16) = w;
  }
}
// A fixed-length instance: rows t0 .. t0 + 63 of `vin`, zero past N.
template <int DT, int D>
__device__ __forceinline__ void v_block_fp8(const uint16_t* vin, int t0, int N, int c0, int g, const float* dv,
                                            const float* rv, uint8_t* s_vt, uint8_t* dst) {
  constexpr int NP = 64 / (256 / (D / 8));
  auto row8 = [&](int j, float* x) {
    const int ra = t0 + NP * g + j;
    load8<DT>(vin + (size_t)min(ra, N - 1) * D + c0, x);
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = ra < N ? x[i] : 0.0f;
  };
  v_block_fp8_rows<D>(row8, c0, g, dv, rv, s_vt, dst);
}

// INT8 Q / K codes and FP8 (PV == PV_FP8) or fp16 (PV_F16) V, or no V at all (PV_NONE: the
// backward's own quantization of Q and K).  grid (Np/64, BH), 256 threads.
template <int DT, int D, int PV, bool FINE>
__global__ __launch_bounds__(256) void quant_int8_fp8_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v, int N, int Np, int BH,
                                                             float sm, QuantPtrs qp) {
  constexpr int C8 = D / 8, RP = 256 / C8, NP = 64 / RP;
  const int bh = blockIdx.y, blk = blockIdx.x, t0 = blk * 64;
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  const size_t base = (size_t)bh * N * D;
  __shared__ float s_mu[D], s_dv[D];
  __shared__ uint32_t s_red[8];
  constexpr bool HASV = PV != PV_NONE;
  constexpr int VB = PV == PV_F16 ? 2 : 1;   // bytes per V element
  __shared__ __align__(16) uint8_t s_vt[PV == PV_FP8 ? D * kVRow : HASV ? D * 64 * VB : 16];
  if (tid < D) {
    const float mu = chunk_mean(qp.sums, 0, BH, bh, D, tid, N);
    const float dvs = HASV ? chunk_amax(qp.amax_v, BH, bh, D, tid) / 448.0f : 0.0f;
    s_mu[tid] = mu;
    s_dv[tid] = dvs;
    if (blk == 0) {
      qp.mu_k[(size_t)bh * D + tid] = mu;
      if (PV == PV_FP8) reinterpret_cast<float*>(qp.v_scales)[(size_t)bh * D + tid] = dvs;
    }
  }
  __syncthreads();
  float dv[8], rv[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    dv[i] = s_dv[c0 + i];
    rv[i] = recip_rn(dv[i]);
  }
  float xq[NP][8], xk[NP][8];
  uint32_t aq = 0, ak = 0;
  uint32_t akg[2] = {0, 0};   // FINE: |K_s| maxima of the block's two 32-token groups
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int rl = r0 + p * RP, row = t0 + rl;
    // every row loads (rows past N read row N - 1, then count as zero), so the loads of all
    // passes can be in flight together
    load8<DT>(q + base + (size_t)min(row, N - 1) * D + c0, xq[p]);
    load8<DT>(k + base + (size_t)min(row, N - 1) * D + c0, xk[p]);
    if (row < N) {
      float xv[8];
      if (PV == PV_F16) {
        load8<DT>(v + base + (size_t)row * D + c0, xv);
        put_v_f16(reinterpret_cast<uint16_t*>(s_vt), rl, c0, xv);
      }
      float cs = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        xk[p][i] = xk[p][i] - s_mu[c0 + i];
        aq = max(aq, __float_as_uint(fabsf(xq[p][i])));
        ak = max(ak, __float_as_uint(fabsf(xk[p][i])));
        if (FINE) akg[(p * RP) / 32] = max(akg[(p * RP) / 32], __float_as_uint(fabsf(xk[p][i])));
        cs += xq[p][i] * s_mu[c0 + i];
      }
      // LSE correction: sm * q_t . mu_k (reduced over the C8 threads of this row)
#pragma unroll
      for (int o = 1; o < C8; o <<= 1) cs += __shfl_xor(cs, o);
      if ((tid % C8) == 0) qp.lse_corr[(size_t)bh * N + row] = sm * cs;
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        xq[p][i] = 0.0f;
        xk[p][i] = 0.0f;
        if (PV == PV_F16) reinterpret_cast<uint16_t*>(s_vt)[(c0 + i) * 64 + rl] = 0;
      }
    }
  }
  // steps: one per 64-token block for Q and K, or (FINE) one per query token -- the row's
  // maximum over its C8 threads -- and one per 32-key group
  float dq_r[NP], rq_r[NP], dk_g[2], rk_g[2];
  if (FINE) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) a = max(a, __float_as_uint(fabsf(xq[p][i])));
#pragma unroll
      for (int o = 1; o < C8; o <<= 1) a = max(a, (uint32_t)__shfl_xor((int)a, o));
      dq_r[p] = __uint_as_float(a) / 127.0f;
      rq_r[p] = recip_rn(dq_r[p]);
    }
    block_umax2(akg[0], akg[1], s_red);
#pragma unroll
    for (int g = 0; g < 2; g++) {
      dk_g[g] = __uint_as_float(akg[g]) / 127.0f;
      rk_g[g] = recip_rn(dk_g[g]);
    }
  } else {
    block_umax2(aq, ak, s_red);
#pragma unroll
    for (int p = 0; p < NP; p++) {
      dq_r[p] = __uint_as_float(aq) / 127.0f;
      rq_r[p] = recip_rn(dq_r[p]);
    }
    dk_g[0] = dk_g[1] = __uint_as_float(ak) / 127.0f;
    rk_g[0] = rk_g[1] = recip_rn(dk_g[0]);
  }
  if (FINE) {
#pragma unroll
    for (int p = 0; p < NP; p++)
      if ((tid % C8) == 0) reinterpret_cast<float*>(qp.q_scales)[(size_t)bh * Np + t0 + r0 + p * RP] = dq_r[p];
    if (tid < 2) reinterpret_cast<float*>(qp.k_scales)[(size_t)bh * (Np / 32) + 2 * blk + tid] = dk_g[tid];
  } else if (tid == 0) {
    reinterpret_cast<float*>(qp.q_scales)[(size_t)bh * (Np / 64) + blk] = dq_r[0];
    reinterpret_cast<float*>(qp.k_scales)[(size_t)bh * (Np / 64) + blk] = dk_g[0];
  }
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int row = t0 + r0 + p * RP;
    uint32_t wq[2] = {0, 0}, wk[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      wq[i / 4] |= (uint32_t)(uint8_t)int8_code(xq[p][i], dq_r[p], rq_r[p]) << (8 * (i % 4));
      wk[i / 4] |= (uint32_t)(uint8_t)int8_code(xk[p][i], dk_g[(p * RP) / 32], rk_g[(p * RP) / 32]) << (8 * (i % 4));
    }
    const size_t off = ((size_t)bh * Np + row) * D + c0;
    *reinterpret_cast<uint2*>(qp.q_codes + off) = make_uint2(wq[0], wq[1]);
    *reinterpret_cast<uint2*>(qp.k_codes + off) = make_uint2(wk[0], wk[1]);
  }
  if (!HASV) return;
  // V tile [D][64] -> v_codes[bh][blk][D][64], coalesced 16-byte stores
  uint8_t* dst = qp.v_codes + ((size_t)bh * (Np / 64) + blk) * D * 64 * VB;
  if (PV == PV_FP8) {
    v_block_fp8<DT, D>(v + base, t0, N, c0, r0, dv, rv, s_vt, dst);
    return;
  }
  __syncthreads();
  for (int c = tid; c < D * 4 * VB; c += 256)
    *reinterpret_cast<uint4*>(dst + c * 16) = *reinterpret_cast<const uint4*>(s_vt + c * 16);
}

// MXFP4 Q_s and K_s codes (32-channel blocks), dS and LSE correction; V in FP8
// (PV == PV_FP8), MXFP4 or MXFP8 (both in 32-token blocks per channel).  grid (Np/64, BH),
// 256 threads.
template <int DT, int D, int PV, bool QB>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, int N, int Np, int BH, float sm,
                                                          QuantPtrs qp) {
  constexpr int C8 = D / 8, RP = 256 / C8, NP = 64 / RP;
  const int bh = blockIdx.y, blk = blockIdx.x, t0 = blk * 64;
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  const size_t base = (size_t)bh * N * D;
  __shared__ float s_mk[D], s_mq[D];
  __shared__ __align__(16) uint8_t s_vt[PV == PV_FP8 ? D * kVRow : 1];
  constexpr bool MXV = PV == PV_MXFP4 || PV == PV_MXFP8;
  __shared__ float s_vf[MXV ? 64 : 1][MXV ? D + 1 : 1];
  __shared__ float s_dv[PV == PV_FP8 ? D : 1];
  if (tid < D) {
    const float mk = chunk_mean(qp.sums, 0, BH, bh, D, tid, N);
    // QB: the mean of this 64-token block's 128-query block (from qblock_mean_kernel)
    const float mq = QB ? qp.mu_q[((size_t)bh * (Np / 128) + blk / 2) * D + tid] : chunk_mean(qp.sums, 1, BH, bh, D, tid, N);
    s_mk[tid] = mk;
    s_mq[tid] = mq;
    if (PV == PV_FP8) s_dv[tid] = chunk_amax(qp.amax_v, BH, bh, D, tid) / 448.0f;
    if (blk == 0) {
      qp.mu_k[(size_t)bh * D + tid] = mk;
      if (!QB) qp.mu_q[(size_t)bh * D + tid] = mq;
      if (PV == PV_FP8) reinterpret_cast<float*>(qp.v_scales)[(size_t)bh * D + tid] = s_dv[tid];
    }
  }
  __syncthreads();
  float dv[8], rv[8];
  if (PV == PV_FP8) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      dv[i] = s_dv[c0 + i];
      rv[i] = recip_rn(dv[i]);
    }
  }
  uint8_t* qe = reinterpret_cast<uint8_t*>(qp.q_scales);
  uint8_t* ke = reinterpret_cast<uint8_t*>(qp.k_scales);
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int rl = r0 + p * RP, row = t0 + rl;
    float xq[8], xk[8], xv[8];
    double ds = 0.0, cs = 0.0;
    if (row < N) {
      load8<DT>(q + base + (size_t)row * D + c0, xq);
      load8<DT>(k + base + (size_t)row * D + c0, xk);
      if (PV != PV_FP8) load8<DT>(v + base + (size_t)row * D + c0, xv);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        cs += (double)xq[i] * (double)s_mk[c0 + i];
        xq[i] = xq[i] - s_mq[c0 + i];
        xk[i] = xk[i] - s_mk[c0 + i];
        if (!QB) ds += (double)s_mq[c0 + i] * (double)xk[i];   // QB: dS comes from qblock_ds_kernel
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) xq[i] = xk[i] = xv[i] = 0.0f;
    }
    // one MX block = 32 channels = 4 neighbouring threads
    uint32_t aq = 0, ak = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      aq = max(aq, __float_as_uint(fabsf(xq[i])));
      ak = max(ak, __float_as_uint(fabsf(xk[i])));
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
      aq = max(aq, (uint32_t)__shfl_xor((int)aq, o));
      ak = max(ak, (uint32_t)__shfl_xor((int)ak, o));
    }
    const unsigned bq = mx_fp4_scale_byte(__uint_as_float(aq)), bk = mx_fp4_scale_byte(__uint_as_float(ak));
    const float sq = bq == 0 ? 1.0f : e8m0_to_float(bq), sk = bk == 0 ? 1.0f : e8m0_to_float(bk);
    const size_t off = ((size_t)bh * Np + row) * (D / 2) + c0 / 2;
    *reinterpret_cast<uint32_t*>(qp.q_codes + off) = pack_fp4x8(xq, sq);
    *reinterpret_cast<uint32_t*>(qp.k_codes + off) = pack_fp4x8(xk, sk);
    if ((c0 % 32) == 0) {
      qe[((size_t)bh * Np + row) * (D / 32) + c0 / 32] = (uint8_t)bq;
      ke[((size_t)bh * Np + row) * (D / 32) + c0 / 32] = (uint8_t)bk;
    }
#pragma unroll
    for (int o = 1; o < C8; o <<= 1) {
      ds += __shfl_xor(ds, o);
      cs += __shfl_xor(cs, o);
    }
    if ((tid % C8) == 0) {
      if (!QB) qp.delta_s[(size_t)bh * Np + row] = row < N ? (float)ds : 0.0f;
      if (row < N) qp.lse_corr[(size_t)bh * N + row] = (float)(sm * cs);
    }
    if (PV != PV_FP8) {
#pragma unroll
      for (int i = 0; i < 8; i++) s_vf[rl][c0 + i] = xv[i];
    }
  }
  if (PV == PV_FP8) {
    v_block_fp8<DT, D>(v + base, t0, N, c0, r0, dv, rv, s_vt, qp.v_codes + ((size_t)bh * (Np / 64) + blk) * D * 64);
  } else {
    __syncthreads();
    // one thread per (channel, 32-token group)
    for (int w = tid; w < D * 2; w += 256) {
      const int ch = w % D, g = w / D;
      float x[32];
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        x[i] = s_vf[32 * g + i][ch];
        a = max(a, __float_as_uint(fabsf(x[i])));
      }
      if (PV == PV_MXFP4) {
        const unsigned b = mx_fp4_scale_byte(__uint_as_float(a));
        const float sc = b == 0 ? 1.0f : e8m0_to_float(b);
        uint4 pk;
        pk.x = pack_fp4x8(x, sc);
        pk.y = pack_fp4x8(x + 8, sc);
        pk.z = pack_fp4x8(x + 16, sc);
        pk.w = pack_fp4x8(x + 24, sc);
        *reinterpret_cast<uint4*>(qp.v_codes + (((size_t)bh * (Np / 64) + blk) * D + ch) * 32 + 16 * g) = pk;
        reinterpret_cast<uint8_t*>(qp.v_scales)[((size_t)bh * (Np / 32) + 2 * blk + g) * D + ch] = (uint8_t)b;
      } else {
        // E4M3 elements: v * 2^-e is exact (b <= 246, so the factor 2^(127-b) is a normal
        // float); the floor rule can put the block max up to 512, so saturate at 448 first
        const unsigned b = mx_scale_byte<8>(__uint_as_float(a));
        const float inv = __uint_as_float((254u - b) << 23);
        float y[32];
#pragma unroll
        for (int i = 0; i < 32; i++) y[i] = fminf(fmaxf(x[i] * inv, -448.0f), 448.0f);
        uint4 pk[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
          pk[h].x = pack_fp8x4(y[16 * h], y[16 * h + 1], y[16 * h + 2], y[16 * h + 3]);
          pk[h].y = pack_fp8x4(y[16 * h + 4], y[16 * h + 5], y[16 * h + 6], y[16 * h + 7]);
          pk[h].z = pack_fp8x4(y[16 * h + 8], y[16 * h + 9], y[16 * h + 10], y[16 * h + 11]);
          pk[h].w = pack_fp8x4(y[16 * h + 12], y[16 * h + 13], y[16 * h + 14], y[16 * h + 15]);
        }
        uint4* dst = reinterpret_cast<uint4*>(qp.v_codes + (((size_t)bh * (Np / 64) + blk) * D + ch) * 64 + 32 * g);
        dst[0] = pk[0];
        dst[1] = pk[1];
        reinterpret_cast<uint8_t*>(qp.v_scales)[((size_t)bh * (Np / 32) + 2 * blk + g) * D + ch] = (uint8_t)b;
      }
    }
  }
}

// Per-block Q smoothing (MXFP4 QK): the mean of Q over each 128-query block -- the fused
// kernel's query tile -- from exact fp64 sums.  grid (Np/128, BH), 256 threads; writes
// mu_q[bh][b][D] and the same fp32 values widened to fp64, muD[bh][b][D] with NBP >= Np/128
// rows (the last block's workgroup zeroes the padding rows), the dS kernel's MFMA operand.
template <int DT, int D>
__global__ __launch_bounds__(256) void qblock_mean_kernel(const uint16_t* __restrict__ q, int N, int Np,
                                                          float* __restrict__ mu_q, double* __restrict__ muD,
                                                          int NBP) {
  constexpr int C8 = D / 8, RP = 256 / C8;
  const int bh = blockIdx.y, b = blockIdx.x, t0 = b * 128, t1 = min(N, t0 + 128), NB = Np / 128;
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  double sx[8] = {};
  for (int r = t0 + r0; r < t1; r += RP) {
    float y[8];
    load8<DT>(q + ((size_t)bh * N + r) * D + c0, y);
#pragma unroll
    for (int i = 0; i < 8; i++) sx[i] += (double)y[i];
  }
  __shared__ double s_x[RP][D];
#pragma unroll
  for (int i = 0; i < 8; i++) s_x[r0][c0 + i] = sx[i];
  __syncthreads();
  if (tid < D) {
    double a = 0.0;
    for (int r = 0; r < RP; r++) a += s_x[r][tid];
    const float m = (float)(a / (double)(t1 - t0));   // t1 > t0: Np < N + 128
    mu_q[((size_t)bh * NB + b) * D + tid] = m;
    double* md = muD + (size_t)bh * NBP * D + tid;
    md[(size_t)b * D] = (double)m;
    if (b == NB - 1)
      for (int p = NB; p < NBP; p++) md[(size_t)p * D] = 0.0;
  }
}

// Per-block Q smoothing: dS[bh][b][j] = fl32(sum_c mu_q[b][c] * Ks[j][c]) for every 128-query
// block b and key j, Ks = fl32(K - mu_k) as the codes kernel forms it, summed in fp64 in
// channel order (0 past N).  A dense fp64 contraction, so it runs on the fp64 MFMA
// (16 x 16 x 4): its result is the FMA chain c + a0 b0 + a1 b1 + a2 b2 + a3 b3 in k order
// (checked bit for bit against that chain on the GPU), so chaining it over the channels in
// order is exactly the sequential fp64 sum.  grid (Np/64, BH), 256 threads: 64 keys per
// workgroup, Ks staged in LDS; wave w takes the 16-block groups g = w, w + 4, ... against all
// 64 keys (four 16-key column tiles).  Operands: A lane l = (block 16 g + l % 16, channel
// c + l / 16) from the fp64 means muD; B lane l = (channel c + l / 16, key 16 u + l % 16).
// Result lane l, register r = (block 16 g + l / 16 + 4 r, key 16 u + l % 16).
typedef double v4d __attribute__((ext_vector_type(4)));
template <int DT, int D>
__global__ __launch_bounds__(256) void qblock_ds_kernel(const uint16_t* __restrict__ k, int N, int Np,
                                                        const float* __restrict__ mu_k,
                                                        const double* __restrict__ muD, int NBP,
                                                        float* __restrict__ delta_s) {
  constexpr int C8 = D / 8, KS = D + 4;   // row pitch: the B reads (16 rows x 4 channels) spread over the banks
  const int bh = blockIdx.y, t0 = blockIdx.x * 64, NB = Np / 128;
  __shared__ float s_ks[64 * KS];
  for (int e = threadIdx.x; e < 64 * C8; e += 256) {
    const int r = e / C8, c0 = (e % C8) * 8, row = t0 + r;
    float y[8];
    if (row < N) {
      load8<DT>(k + ((size_t)bh * N + row) * D + c0, y);
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = y[i] - mu_k[(size_t)bh * D + c0 + i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) s_ks[r * KS + c0 + i] = y[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  for (int g = w; 16 * g < NB; g += 4) {
    const double* ma = muD + ((size_t)bh * NBP + 16 * g + li) * D + lk;
    v4d acc[4];
#pragma unroll
    for (int u = 0; u < 4; u++) acc[u] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int c = 0; c < D; c += 4) {
      const double av = ma[c];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const double bv = (double)s_ks[(16 * u + li) * KS + c + lk];
        acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[u], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int key = t0 + 16 * u + li;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int blk = 16 * g + lk + 4 * r;
        if (blk < NB) delta_s[((size_t)bh * NB + blk) * Np + key] = key < N ? (float)acc[u][r] : 0.0f;
      }
    }
  }
}

// Per-block Q smoothing on packed sequences: the means of every 128-query block of every query
// instance, formed as qblock_mean_kernel forms them (the same fp64 sums in the same order), at
// the blocks' slots (qblock_slot).  grid (table capacity, H): workgroup (e, h) takes table item
// e = (b, j) for even j -- query block j / 2 of query instance (b, h) -- and returns for odd j
// and for blocks past the query sequence (the table covers the longer of its query and key
// sequences).
template <int DT, int D>
__global__ __launch_bounds__(256) void seq_qblock_mean_kernel(const uint16_t* __restrict__ q, SeqGeo g,
                                                              float* __restrict__ mu_q, double* __restrict__ muD,
                                                              const int2* __restrict__ tab) {
  constexpr int C8 = D / 8, RP = 256 / C8;
  const int e = blockIdx.x;
  if (e >= tab[0].x) return;
  const int2 it = tab[1 + e];
  if (it.y & 1) return;
  const int b = it.x, qb = it.y / 2, h = blockIdx.y;
  const Inst qi = q_inst(g, b, h, D);
  const int t0 = qb * 128, t1 = min(qi.len, t0 + 128);
  if (t0 >= t1) return;
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  double sx[8] = {};
  for (int r = t0 + r0; r < t1; r += RP) {
    float y[8];
    load8<DT>(q + qi.io0 + (size_t)r * qi.ios + c0, y);
#pragma unroll
    for (int i = 0; i < 8; i++) sx[i] += (double)y[i];
  }
  __shared__ double s_x[RP][D];
#pragma unroll
  for (int i = 0; i < 8; i++) s_x[r0][c0 + i] = sx[i];
  __syncthreads();
  if (tid < D) {
    double a = 0.0;
    for (int r = 0; r < RP; r++) a += s_x[r][tid];
    const float m = (float)(a / (double)(t1 - t0));
    const size_t slot = qblock_slot(g, b, h, qb);
    mu_q[slot * D + tid] = m;
    muD[slot * D + tid] = (double)m;
  }
}

// Per-block Q smoothing on packed sequences: dS of every block of the query heads that read KV
// head hk against keys [64 j, 64 j + 64) of KV instance (b, hk) (0 past the sequence's end),
// formed as qblock_ds_kernel forms it (the same fp64 MFMA chain over the channels in order),
// into the blocks' strips.  grid (table capacity, Hkv), item e = (b, j).  The A operand reads
// the means of 16 consecutive slots from the sequence's first; slots past its blocks (the next
// sequence's, or the 16 rows after the last head's) only feed result rows that are not stored.
template <int DT, int D>
__global__ __launch_bounds__(256) void seq_qblock_ds_kernel(const uint16_t* __restrict__ k, SeqGeo g,
                                                            const float* __restrict__ mu_k,
                                                            const double* __restrict__ muD, size_t strip,
                                                            float* __restrict__ delta_s,
                                                            const int2* __restrict__ tab) {
  constexpr int C8 = D / 8, KS = D + 4;
  const int e = blockIdx.x;
  if (e >= tab[0].x) return;
  const int2 it = tab[1 + e];
  const int b = it.x, hk = blockIdx.y, t0 = it.y * 64, grp = g.H / g.Hkv;
  const Inst ki = k_inst(g, b, hk, D);
  const int nqb = (q_inst(g, b, hk * grp, D).len + 127) / 128;
  if (t0 >= ((ki.len + 127) & ~127) || nqb == 0) return;
  __shared__ float s_ks[64 * KS];
  const float* mk = mu_k + ((size_t)b * g.Hkv + hk) * D;
  for (int x = threadIdx.x; x < 64 * C8; x += 256) {
    const int r = x / C8, c0 = (x % C8) * 8, row = t0 + r;
    float y[8];
    if (row < ki.len) {
      load8<DT>(k + ki.io0 + (size_t)row * ki.ios + c0, y);
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = y[i] - mk[c0 + i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) y[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) s_ks[r * KS + c0 + i] = y[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  for (int r = 0; r < grp; r++) {
    const size_t slot0 = qblock_slot(g, b, hk * grp + r, 0);
    for (int gq = w; 16 * gq < nqb; gq += 4) {
      const double* ma = muD + (slot0 + 16 * gq + li) * D + lk;
      v4d acc[4];
#pragma unroll
      for (int u = 0; u < 4; u++) acc[u] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
      for (int c = 0; c < D; c += 4) {
        const double av = ma[c];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const double bv = (double)s_ks[(16 * u + li) * KS + c + lk];
          acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[u], 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int key = t0 + 16 * u + li;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const int blk = 16 * gq + lk + 4 * rr;
          if (blk < nqb) delta_s[(slot0 + blk) * strip + key] = key < ki.len ? (float)acc[u][rr] : 0.0f;
        }
      }
    }
  }
}

// The instances one packed-sequence codes item serves: query head h of sequence b and, when
// h < Hkv, KV head h of the same sequence; each role is active while the item's 64-token block
// lies inside the instance rounded up to 128.
struct CodeBlock {
  Inst qi, ki, kq;   // query instance (b, h), KV instance (b, h), the KV instance query head h reads
  int bq, hq;        // sequence and head of the query instance
  int bk, hk;        // sequence and head of the KV instance
  int iq, ikv;       // their indices b H + h and b Hkv + h (statistics, means, V steps)
  bool qa, ka;
};
template <int D>
__device__ __forceinline__ CodeBlock code_block(const SeqGeo& g, int b, int h, int t0) {
  CodeBlock cb;
  cb.bq = cb.bk = b;
  cb.hq = h;
  const bool has_kv = h < g.Hkv;
  cb.hk = has_kv ? h : 0;
  cb.iq = b * g.H + h;
  cb.ikv = b * g.Hkv + cb.hk;
  cb.qi = q_inst(g, b, h, D);
  cb.ki = k_inst(g, b, cb.hk, D);
  cb.kq = k_inst(g, b, h / (g.H / g.Hkv), D);
  cb.qa = t0 < ((cb.qi.len + 127) & ~127);
  cb.ka = has_kv && t0 < ((cb.ki.len + 127) & ~127);
  return cb;
}

// The (sequence, 64-token block) pairs of a packed batch, as a table the codes kernels walk:
// tab[0].x = the count, tab[1 + e] = (b, block).  Sequence b has 2 ceil(max(len_q, len_k) /
// 128) blocks.  One workgroup: a prefix sum over the sequences (each thread a contiguous run),
// then each thread writes its runs' entries; writes stop at the capacity `cap`, so offsets
// that overlap (malformed input) cannot run past the table.
__global__ __launch_bounds__(256) void seq_blocks_kernel(SeqGeo g, int2* __restrict__ tab, int cap) {
  __shared__ int s_n[256];
  const int tid = threadIdx.x, chunk = (g.B + 255) / 256, b0 = min(g.B, tid * chunk), b1 = min(g.B, b0 + chunk);
  auto nblocks = [&](int b) {
    int s, lq, lk;
    packed_seq(g.cu_q, b, g.total_q, g.max_q, s, lq);
    packed_seq(g.cu_k, b, g.total_k, g.max_k, s, lk);
    return 2 * ((max(lq, lk) + 127) / 128);
  };
  int n = 0;
  for (int b = b0; b < b1; b++) n += nblocks(b);
  s_n[tid] = n;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive scan
    const int x = tid >= o ? s_n[tid - o] : 0;
    __syncthreads();
    s_n[tid] += x;
    __syncthreads();
  }
  int idx = s_n[tid] - n;
  for (int b = b0; b < b1; b++) {
    const int nb = nblocks(b);
    for (int j = 0; j < nb && idx < cap; j++, idx++) tab[1 + idx] = make_int2(b, j);
  }
  if (tid == 0) tab[0] = make_int2(min(s_n[255], cap), 0);
}

// Packed sequences: INT8 Q / K codes and FP8 (or fp16) V of one item (block blk of sequence b,
// query head h and, when h < Hkv, KV head h); 256 threads.
template <int DT, int D, int PV, bool FINE>
__device__ __forceinline__ void seq_int8_item(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                              const uint16_t* __restrict__ v, const SeqGeo& g, float sm,
                                              const QuantPtrs& qp, int b, int blk, int h) {
  constexpr int C8 = D / 8, RP = 256 / C8, NP = 64 / RP;
  const int t0 = blk * 64, BHm = g.B * g.H;
  const CodeBlock cb = code_block<D>(g, b, h, t0);
  if (!cb.qa && !cb.ka) return;
  const int i = cb.ikv;   // the KV instance: its statistics, mean and V steps
  const int kvq = cb.bq * g.Hkv + cb.hq / (g.H / g.Hkv);
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  __shared__ float s_mu[D], s_muq[D], s_dv[D];
  __shared__ uint32_t s_red[8];
  constexpr int VB = PV == PV_F16 ? 2 : 1;   // bytes per V element
  __shared__ __align__(16) uint8_t s_vt[PV == PV_FP8 ? D * kVRow : D * 64 * VB];
  // the KV instance query head i reads is usually instance i itself (no grouping)
  const bool own_kv = kvq == i && cb.ka;
  if (tid < D) {
    if (cb.ka) {
      const float mu = chunk_mean(qp.sums, 0, BHm, i, D, tid, cb.ki.len);
      const float dvs = chunk_amax(qp.amax_v, BHm, i, D, tid) / 448.0f;
      s_mu[tid] = mu;
      s_dv[tid] = dvs;
      if (blk == 0) {
        qp.mu_k[(size_t)i * D + tid] = mu;
        if (PV == PV_FP8) reinterpret_cast<float*>(qp.v_scales)[(size_t)i * D + tid] = dvs;
      }
    }
    if (cb.qa && !own_kv) s_muq[tid] = chunk_mean(qp.sums, 0, BHm, kvq, D, tid, cb.kq.len);
  }
  __syncthreads();
  const float* muq = own_kv ? s_mu : s_muq;
  float dv[8], rv[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    dv[i] = cb.ka ? s_dv[c0 + i] : 0.0f;
    rv[i] = recip_rn(dv[i]);
  }
  float xq[NP][8], xk[NP][8];
  uint32_t aq = 0, ak = 0;
  uint32_t akg[2] = {0, 0};   // FINE: |K_s| maxima of the block's two 32-token groups
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int rl = r0 + p * RP, row = t0 + rl;
    // the row's three loads go out together; rows past an instance's end load as zeros (no
    // effect on the maxima or the LSE term)
    const uint4 gq = row_raw(q, cb.qi, cb.qa, row, c0);
    const uint4 gk = row_raw(k, cb.ki, cb.ka, row, c0);
    const uint4 gv = PV == PV_F16 ? row_raw(v, cb.ki, cb.ka, row, c0) : make_uint4(0, 0, 0, 0);
    float cs = 0.0f;
    unpack8<DT>(gq, xq[p]);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      aq = max(aq, __float_as_uint(fabsf(xq[p][i])));
      cs += xq[p][i] * muq[c0 + i];
    }
    if (cb.ka && row < cb.ki.len) {
      float xv[8];
      unpack8<DT>(gk, xk[p]);
      if (PV == PV_F16) {
        unpack8<DT>(gv, xv);
        put_v_f16(reinterpret_cast<uint16_t*>(s_vt), rl, c0, xv);
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        xk[p][i] = xk[p][i] - s_mu[c0 + i];
        ak = max(ak, __float_as_uint(fabsf(xk[p][i])));
        if (FINE) akg[(p * RP) / 32] = max(akg[(p * RP) / 32], __float_as_uint(fabsf(xk[p][i])));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        xk[p][i] = 0.0f;
        if (PV == PV_F16) reinterpret_cast<uint16_t*>(s_vt)[(c0 + i) * 64 + rl] = 0;
      }
    }
    // LSE correction: sm * q_t . mu_k (reduced over the C8 threads of this row)
#pragma unroll
    for (int o = 1; o < C8; o <<= 1) cs += __shfl_xor(cs, o);
    if ((tid % C8) == 0 && cb.qa && row < cb.qi.len) qp.lse_corr[cb.qi.row0 + row] = sm * cs;
  }
  // steps: one per 64-token block for Q and K, or (FINE) one per query token -- the row's
  // maximum over its C8 threads -- and one per 32-key group
  float dq_r[NP], rq_r[NP], dk_g[2], rk_g[2];
  if (FINE) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) a = max(a, __float_as_uint(fabsf(xq[p][i])));
#pragma unroll
      for (int o = 1; o < C8; o <<= 1) a = max(a, (uint32_t)__shfl_xor((int)a, o));
      dq_r[p] = __uint_as_float(a) / 127.0f;
      rq_r[p] = recip_rn(dq_r[p]);
    }
    block_umax2(akg[0], akg[1], s_red);
#pragma unroll
    for (int g = 0; g < 2; g++) {
      dk_g[g] = __uint_as_float(akg[g]) / 127.0f;
      rk_g[g] = recip_rn(dk_g[g]);
    }
  } else {
    block_umax2(aq, ak, s_red);
#pragma unroll
    for (int p = 0; p < NP; p++) {
      dq_r[p] = __uint_as_float(aq) / 127.0f;
      rq_r[p] = recip_rn(dq_r[p]);
    }
    dk_g[0] = dk_g[1] = __uint_as_float(ak) / 127.0f;
    rk_g[0] = rk_g[1] = recip_rn(dk_g[0]);
  }
  if (FINE) {
#pragma unroll
    for (int p = 0; p < NP; p++)
      if ((tid % C8) == 0 && cb.qa) reinterpret_cast<float*>(qp.q_scales)[cb.qi.tok0 + t0 + r0 + p * RP] = dq_r[p];
    if (tid < 2 && cb.ka) reinterpret_cast<float*>(qp.k_scales)[cb.ki.tok0 / 32 + 2 * blk + tid] = dk_g[tid];
  } else if (tid == 0) {
    if (cb.qa) reinterpret_cast<float*>(qp.q_scales)[cb.qi.tok0 / 64 + blk] = dq_r[0];
    if (cb.ka) reinterpret_cast<float*>(qp.k_scales)[cb.ki.tok0 / 64 + blk] = dk_g[0];
  }
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int row = t0 + r0 + p * RP;
    uint32_t wq[2] = {0, 0}, wk[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      wq[i / 4] |= (uint32_t)(uint8_t)int8_code(xq[p][i], dq_r[p], rq_r[p]) << (8 * (i % 4));
      wk[i / 4] |= (uint32_t)(uint8_t)int8_code(xk[p][i], dk_g[(p * RP) / 32], rk_g[(p * RP) / 32]) << (8 * (i % 4));
    }
    if (cb.qa) *reinterpret_cast<uint2*>(qp.q_codes + (cb.qi.tok0 + row) * D + c0) = make_uint2(wq[0], wq[1]);
    if (cb.ka) *reinterpret_cast<uint2*>(qp.k_codes + (cb.ki.tok0 + row) * D + c0) = make_uint2(wk[0], wk[1]);
  }
  if (cb.ka) {
    // V tile [D][64] -> the instance's tile blk of v_codes [..][D][64], coalesced 16-byte stores
    uint8_t* dst = qp.v_codes + (cb.ki.tok0 / 64 + blk) * D * 64 * VB;
    if (PV == PV_FP8) {
      auto row8 = [&](int jr, float* x) { unpack8<DT>(row_raw(v, cb.ki, true, t0 + NP * r0 + jr, c0), x); };
      v_block_fp8_rows<D>(row8, c0, r0, dv, rv, s_vt, dst);
      return;
    }
    __syncthreads();
    for (int c = tid; c < D * 4 * VB; c += 256)
      *reinterpret_cast<uint4*>(dst + c * 16) = *reinterpret_cast<const uint4*>(s_vt + c * 16);
  }
}
// grid (table capacity, H): workgroup (e, h) takes the table's item e for query head h.
template <int DT, int D, int PV, bool FINE>
__global__ __launch_bounds__(256) void quant_int8_fp8_seq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v, SeqGeo g, float sm,
                                                             QuantPtrs qp) {
  const int2* tab = reinterpret_cast<const int2*>(qp.blocks);
  const int n = tab[0].x;
  const int e = blockIdx.x;
  if (e >= n) return;
  const int2 it = tab[1 + e];
  seq_int8_item<DT, D, PV, FINE>(q, k, v, g, sm, qp, it.x, it.y, blockIdx.y);
}

// Packed sequences or grouped KV heads: MXFP4 Q_s and K_s codes (32-channel blocks), dS and
// LSE correction; V in FP8 (PV == PV_FP8), MXFP4 or MXFP8 (both in 32-token blocks per
// channel).  grid (blocks of the longest instance, B*H), 256 threads.  dS = mu_q . K_s is written for each query head that
// reads KV instance i (one without grouped heads, in the row loop; H / Hkv of them after it).
template <int DT, int D, int PV, bool QB>
__device__ __forceinline__ void seq_mxfp4_item(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                               const uint16_t* __restrict__ v, const SeqGeo& g, float sm,
                                               const QuantPtrs& qp, int b, int blk, int h) {
  constexpr int C8 = D / 8, RP = 256 / C8, NP = 64 / RP;
  constexpr bool MXV = PV == PV_MXFP4 || PV == PV_MXFP8;
  const int t0 = blk * 64, BHm = g.B * g.H;
  const CodeBlock cb = code_block<D>(g, b, h, t0);
  if (!cb.qa && !cb.ka) return;
  const int i = cb.ikv, iq = cb.iq;   // KV instance (statistics, means, V steps), query instance
  const int grp = g.H / g.Hkv;
  const int kvq = cb.bq * g.Hkv + cb.hq / grp;
  const bool own_kv = kvq == i && cb.ka;   // query head h reads KV head h (no grouping)
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  __shared__ float s_mk[D], s_mkq[D], s_mq[D];
  __shared__ __align__(16) uint8_t s_vt[PV == PV_FP8 ? D * kVRow : 1];
  __shared__ float s_vf[MXV ? 64 : 1][MXV ? D + 1 : 1];
  __shared__ float s_dv[PV == PV_FP8 ? D : 1];
  if (tid < D) {
    if (cb.ka) {
      const float mk = chunk_mean(qp.sums, 0, BHm, i, D, tid, cb.ki.len);
      s_mk[tid] = mk;
      if (PV == PV_FP8) s_dv[tid] = chunk_amax(qp.amax_v, BHm, i, D, tid) / 448.0f;
      if (blk == 0) {
        qp.mu_k[(size_t)i * D + tid] = mk;
        if (PV == PV_FP8) reinterpret_cast<float*>(qp.v_scales)[(size_t)i * D + tid] = s_dv[tid];
      }
    }
    // mu_q of the query instance: its own smoothing, and (grp == 1) the dS of the KV instance,
    // which that query head reads -- needed whenever either role is active.  QB: the mean of
    // this block's 128-query block (seq_qblock_mean_kernel), and dS comes from
    // seq_qblock_ds_kernel
    if (QB) {
      s_mq[tid] = cb.qa ? qp.mu_q[qblock_slot(g, b, h, blk / 2) * D + tid] : 0.0f;
    } else {
      const float mq = chunk_mean(qp.sums, 1, BHm, iq, D, tid, cb.qi.len);
      s_mq[tid] = mq;
      if (cb.qa && blk == 0) qp.mu_q[(size_t)iq * D + tid] = mq;
    }
    if (cb.qa && !own_kv) s_mkq[tid] = chunk_mean(qp.sums, 0, BHm, kvq, D, tid, cb.kq.len);
  }
  __syncthreads();
  const float* mkq = own_kv ? s_mk : s_mkq;
  float dv[8], rv[8];
  if (PV == PV_FP8) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      dv[i] = cb.ka ? s_dv[c0 + i] : 0.0f;
      rv[i] = recip_rn(dv[i]);
    }
  }
  uint8_t* qe = reinterpret_cast<uint8_t*>(qp.q_scales);
  uint8_t* ke = reinterpret_cast<uint8_t*>(qp.k_scales);
  const size_t ds_own = ds_base(g, cb.bk, cb.hk * grp);   // grp == 1: query head (bk, hk)
  float xk[NP][8];
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int rl = r0 + p * RP, row = t0 + rl;
    const bool qv = cb.qa && row < cb.qi.len, kv = cb.ka && row < cb.ki.len;
    // the row's three loads go out together (zeros past an instance's end)
    const uint4 gq = row_raw(q, cb.qi, cb.qa, row, c0);
    const uint4 gk = row_raw(k, cb.ki, cb.ka, row, c0);
    const uint4 gv = PV != PV_FP8 ? row_raw(v, cb.ki, cb.ka, row, c0) : make_uint4(0, 0, 0, 0);
    float xq[8], xv[8];
    unpack8<DT>(gq, xq);
    unpack8<DT>(gk, xk[p]);
    unpack8<DT>(gv, xv);
    // branch-free: rows past an instance's end are zeros, and the 0/1 factors keep them zero
    // after smoothing (so their codes, cs and ds are all 0)
    const float fq = qv ? 1.0f : 0.0f, fk = kv ? 1.0f : 0.0f;
    double cs = 0.0, ds = 0.0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      cs += (double)xq[i] * (double)mkq[c0 + i];
      xq[i] = xq[i] - fq * s_mq[c0 + i];
      xk[p][i] = xk[p][i] - fk * s_mk[c0 + i];
      if (!QB && grp == 1) ds += (double)s_mq[c0 + i] * (double)xk[p][i];
    }
    // one MX block = 32 channels = 4 neighbouring threads
    uint32_t aq = 0, ak = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      aq = max(aq, __float_as_uint(fabsf(xq[i])));
      ak = max(ak, __float_as_uint(fabsf(xk[p][i])));
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
      aq = max(aq, (uint32_t)__shfl_xor((int)aq, o));
      ak = max(ak, (uint32_t)__shfl_xor((int)ak, o));
    }
#pragma unroll
    for (int o = 1; o < C8; o <<= 1) {
      cs += __shfl_xor(cs, o);
      ds += __shfl_xor(ds, o);
    }
    if (cb.qa) {
      const unsigned bq = mx_fp4_scale_byte(__uint_as_float(aq));
      const float sq = bq == 0 ? 1.0f : e8m0_to_float(bq);
      *reinterpret_cast<uint32_t*>(qp.q_codes + (cb.qi.tok0 + row) * (D / 2) + c0 / 2) = pack_fp4x8(xq, sq);
      if ((c0 % 32) == 0) qe[(cb.qi.tok0 + row) * (D / 32) + c0 / 32] = (uint8_t)bq;
      if ((tid % C8) == 0 && qv) qp.lse_corr[cb.qi.row0 + row] = (float)(sm * cs);
    }
    if (cb.ka) {
      const unsigned bk = mx_fp4_scale_byte(__uint_as_float(ak));
      const float sk = bk == 0 ? 1.0f : e8m0_to_float(bk);
      *reinterpret_cast<uint32_t*>(qp.k_codes + (cb.ki.tok0 + row) * (D / 2) + c0 / 2) = pack_fp4x8(xk[p], sk);
      if ((c0 % 32) == 0) ke[(cb.ki.tok0 + row) * (D / 32) + c0 / 32] = (uint8_t)bk;
      if (!QB && grp == 1 && (tid % C8) == 0) qp.delta_s[ds_own + row] = kv ? (float)ds : 0.0f;
      if (PV != PV_FP8) {
#pragma unroll
        for (int i = 0; i < 8; i++) s_vf[rl][c0 + i] = xv[i];
      }
    }
  }
  if (!cb.ka) return;
  // grouped heads: dS for each query head of the group, with its own mu_q
  if (!QB && grp > 1) {
    const Inst qg = q_inst(g, cb.bk, cb.hk * grp, D);   // the group's query sequence
    for (int r = 0; r < grp; r++) {
      const int hq = cb.hk * grp + r, iq = cb.bk * g.H + hq;
      __syncthreads();
      if (tid < D) s_mq[tid] = chunk_mean(qp.sums, 1, BHm, iq, D, tid, qg.len);
      __syncthreads();
      const size_t ds0 = ds_base(g, cb.bk, hq);
#pragma unroll
      for (int p = 0; p < NP; p++) {
        const int row = t0 + r0 + p * RP;
        double ds = 0.0;
#pragma unroll
        for (int i = 0; i < 8; i++) ds += (double)s_mq[c0 + i] * (double)xk[p][i];
#pragma unroll
        for (int o = 1; o < C8; o <<= 1) ds += __shfl_xor(ds, o);
        if ((tid % C8) == 0) qp.delta_s[ds0 + row] = row < cb.ki.len ? (float)ds : 0.0f;
      }
    }
  }
  const size_t vt0 = cb.ki.tok0 / 64 + blk;   // the instance's V tile
  if (PV == PV_FP8) {
    auto row8 = [&](int jr, float* x) { unpack8<DT>(row_raw(v, cb.ki, true, t0 + NP * r0 + jr, c0), x); };
    v_block_fp8_rows<D>(row8, c0, r0, dv, rv, s_vt, qp.v_codes + vt0 * D * 64);
  } else {
    __syncthreads();
    // one thread per (channel, 32-token group)
    for (int w = tid; w < D * 2; w += 256) {
      const int ch = w % D, gi = w / D;
      float x[32];
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        x[i] = s_vf[32 * gi + i][ch];
        a = max(a, __float_as_uint(fabsf(x[i])));
      }
      uint8_t* vsb = reinterpret_cast<uint8_t*>(qp.v_scales) + (cb.ki.tok0 / 32 + 2 * blk + gi) * D + ch;
      if (PV == PV_MXFP4) {
        const unsigned b = mx_fp4_scale_byte(__uint_as_float(a));
        const float sc = b == 0 ? 1.0f : e8m0_to_float(b);
        uint4 pk;
        pk.x = pack_fp4x8(x, sc);
        pk.y = pack_fp4x8(x + 8, sc);
        pk.z = pack_fp4x8(x + 16, sc);
        pk.w = pack_fp4x8(x + 24, sc);
        *reinterpret_cast<uint4*>(qp.v_codes + (vt0 * D + ch) * 32 + 16 * gi) = pk;
        *vsb = (uint8_t)b;
      } else {
        // E4M3 elements: v * 2^-e is exact (b <= 246, so the factor 2^(127-b) is a normal
        // float); the floor rule can put the block max up to 512, so saturate at 448 first
        const unsigned b = mx_scale_byte<8>(__uint_as_float(a));
        const float inv = __uint_as_float((254u - b) << 23);
        float y[32];
#pragma unroll
        for (int i = 0; i < 32; i++) y[i] = fminf(fmaxf(x[i] * inv, -448.0f), 448.0f);
        uint4 pk[2];
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          pk[hh].x = pack_fp8x4(y[16 * hh], y[16 * hh + 1], y[16 * hh + 2], y[16 * hh + 3]);
          pk[hh].y = pack_fp8x4(y[16 * hh + 4], y[16 * hh + 5], y[16 * hh + 6], y[16 * hh + 7]);
          pk[hh].z = pack_fp8x4(y[16 * hh + 8], y[16 * hh + 9], y[16 * hh + 10], y[16 * hh + 11]);
          pk[hh].w = pack_fp8x4(y[16 * hh + 12], y[16 * hh + 13], y[16 * hh + 14], y[16 * hh + 15]);
        }
        uint4* dst = reinterpret_cast<uint4*>(qp.v_codes + (vt0 * D + ch) * 64 + 32 * gi);
        dst[0] = pk[0];
        dst[1] = pk[1];
        *vsb = (uint8_t)b;
      }
    }
  }
}

// grid (table capacity, H): workgroup (e, h) takes the table's item e for query head h.
template <int DT, int D, int PV, bool QB>
__global__ __launch_bounds__(256) void quant_mxfp4_seq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, SeqGeo g, float sm,
                                                          QuantPtrs qp) {
  const int2* tab = reinterpret_cast<const int2*>(qp.blocks);
  const int n = tab[0].x;
  const int e = blockIdx.x;
  if (e >= n) return;
  const int2 it = tab[1 + e];
  seq_mxfp4_item<DT, D, PV, QB>(q, k, v, g, sm, qp, it.x, it.y, blockIdx.y);
}

template <int DT, int D>
static hipError_t prologue_dispatch(const void* q, const void* k, const void* v, const Shape& s, const QuantPtrs& qp,
                                    hipStream_t st) {
  const SeqGeo& g = s.g;
  const int BHm = g.B * g.H;
  const uint16_t *Q = (const uint16_t*)q, *K = (const uint16_t*)k, *V = (const uint16_t*)v;
  // fixed length without grouped heads: the streamlined codes kernels (N, Np per instance)
  const bool plain = g.cu_q == nullptr && g.Hkv == g.H;
  const dim3 sg(kChunks, BHm), qg(max(g.nbq, g.nbk), BHm);
  // packed sequences: one codes workgroup per entry of a table of the batch's (sequence, block)
  // pairs and query head; the grid covers the table's capacity, and the workgroups past its
  // count return at once
  const dim3 pg(plain ? 1 : seq_block_capacity(g), g.H);
  if (!plain) seq_blocks_kernel<<<1, 256, 0, st>>>(g, reinterpret_cast<int2*>(qp.blocks), seq_block_capacity(g));
  // Q and K only (the backward's quantization; fixed length, INT8 with 64-token steps)
  if (s.pv_fmt == PV_NONE) {
    if (!plain || s.qk_fmt != QK_INT8) return hipErrorInvalidValue;
    stats_kernel<DT, D, false, false><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
    quant_int8_fp8_kernel<DT, D, PV_NONE, false><<<qg, 256, 0, st>>>(Q, K, V, s.N, s.Np, BHm, s.sm_scale, qp);
    return hipGetLastError();
  }
  // else INT8 (QK_INT8, or QK_INT8T with finer steps)
  const bool mx = s.qk_fmt == QK_MXFP4 || s.qk_fmt == QK_MXFP4B;
  if (!mx) {
    auto codes = [&](auto pv, auto fine) {
      constexpr int PV = decltype(pv)::value;
      constexpr bool FINE = decltype(fine)::value;
      // fp16 V needs no channel maxima
      stats_kernel<DT, D, false, PV == PV_FP8><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
      if (plain)
        quant_int8_fp8_kernel<DT, D, PV, FINE><<<qg, 256, 0, st>>>(Q, K, V, s.N, s.Np, BHm, s.sm_scale, qp);
      else
        quant_int8_fp8_seq_kernel<DT, D, PV, FINE><<<pg, 256, 0, st>>>(Q, K, V, g, s.sm_scale, qp);
    };
    auto with_pv = [&](auto fine) {
      if (s.pv_fmt == PV_F16) codes(std::integral_constant<int, PV_F16>{}, fine);
      else codes(std::integral_constant<int, PV_FP8>{}, fine);
    };
    if (s.qk_fmt == QK_INT8T) with_pv(std::true_type{});
    else with_pv(std::false_type{});
    return hipGetLastError();
  }
  // QB (per-128-query-block Q smoothing): block means replace the Q sums
  const bool qb = s.qk_fmt == QK_MXFP4B;
  // QB: the fp64 copy of the block means follows the fp32 ones in the mu_q region (fixed
  // length: per instance, padded to whole 16-block groups; packed: by slot, 16 rows of padding)
  const int nbp = plain ? qblock_padded(s.Np / 128) : 0;
  double* muD = reinterpret_cast<double*>(qp.mu_q + qblock_slots(g) * D);
  const int2* tab = reinterpret_cast<const int2*>(qp.blocks);
  if (qb) {
    if (s.pv_fmt == PV_FP8)
      stats_kernel<DT, D, false, true><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
    else
      stats_kernel<DT, D, false, false><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
    if (plain)
      qblock_mean_kernel<DT, D><<<dim3(s.Np / 128, BHm), 256, 0, st>>>(Q, s.N, s.Np, qp.mu_q, muD, nbp);
    else
      seq_qblock_mean_kernel<DT, D><<<pg, 256, 0, st>>>(Q, g, qp.mu_q, muD, tab);
  } else if (s.pv_fmt == PV_FP8) {
    stats_kernel<DT, D, true, true><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
  } else {
    stats_kernel<DT, D, true, false><<<sg, 256, 0, st>>>(Q, K, V, g, qp.sums, qp.amax_v);
  }
  auto codes = [&](auto pv) {
    constexpr int PV = decltype(pv)::value;
    if (plain && qb)
      quant_mxfp4_kernel<DT, D, PV, true><<<qg, 256, 0, st>>>(Q, K, V, s.N, s.Np, BHm, s.sm_scale, qp);
    else if (plain)
      quant_mxfp4_kernel<DT, D, PV, false><<<qg, 256, 0, st>>>(Q, K, V, s.N, s.Np, BHm, s.sm_scale, qp);
    else if (qb)
      quant_mxfp4_seq_kernel<DT, D, PV, true><<<pg, 256, 0, st>>>(Q, K, V, g, s.sm_scale, qp);
    else
      quant_mxfp4_seq_kernel<DT, D, PV, false><<<pg, 256, 0, st>>>(Q, K, V, g, s.sm_scale, qp);
  };
  if (s.pv_fmt == PV_FP8) codes(std::integral_constant<int, PV_FP8>{});
  else if (s.pv_fmt == PV_MXFP8) codes(std::integral_constant<int, PV_MXFP8>{});
  else codes(std::integral_constant<int, PV_MXFP4>{});
  // QB: dS per (query block, key), after the codes kernel has written mu_k
  if (qb && plain)
    qblock_ds_kernel<DT, D><<<dim3(s.Np / 64, BHm), 256, 0, st>>>(K, s.N, s.Np, qp.mu_k, muD, nbp, qp.delta_s);
  else if (qb)
    seq_qblock_ds_kernel<DT, D><<<dim3(pg.x, g.Hkv), 256, 0, st>>>(K, g, qp.mu_k, muD, qblock_strip(g), qp.delta_s,
                                                                   tab);
  return hipGetLastError();
}

hipError_t launch_prologue(const void* q, const void* k, const void* v, const Shape& s, const QuantPtrs& qp,
                           hipStream_t st) {
  if (s.io_dtype == 0)
    return s.d == 64 ? prologue_dispatch<0, 64>(q, k, v, s, qp, st) : prologue_dispatch<0, 128>(q, k, v, s, qp, st);
  return s.d == 64 ? prologue_dispatch<1, 64>(q, k, v, s, qp, st) : prologue_dispatch<1, 128>(q, k, v, s, qp, st);
}

}  // namespace sage
