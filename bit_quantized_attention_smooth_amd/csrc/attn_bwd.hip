// attn_bwd.hip -- 8-bit attention backward (dQ, dK, dV) for gfx950.
//
// The pages name an accurate and efficient 8-bit attention for both forward and
// backward propagation (SageAttention3 abstract) and a trainable INT8 attention
// (SageBwd, related-papers page of SageAttention2++), without the recipe.  This
// backward keeps the forward's quantization of QK^T and runs every product on
// 8-bit MFMA with fp32 accumulation:
//   S   = Q K_s^T        INT8 (the forward's codes: per-64-token steps, K smoothed)
//   P   = exp(S sm - (LSE - c))      c = sm q.mu_k, the row shift smoothing removed
//   dP  = dO V^T         FP8, per-64-token-block steps of dO and V (they factor out of
//                        the channel sum)
//   dS  = P o (dP - D),  D_i = sum_c dO_ic O_ic
//   dV  = P~^T dO        FP8: P~ = E4M3(448 P), dO^T with per-channel steps (they factor
//                        out of the query sum)
//   dK  = sm dS^T Q      FP8: Q^T with per-channel steps; dS in E4M3 with one power-of-two
//                        scale per 32-element block (an MX block), applied by the scaled MFMA
//   dQ  = sm (dS K_s - rowsum(dS) P K_s)  FP8 the same way, K_s^T with per-channel steps.
//                        With quantized dP the rows of dS no longer sum to 0: rowsum(dS) =
//                        D^ - D, where D^ = sum_j P dP^ is the value consistent with the
//                        quantized dP.  Replacing D by D^ turns dS into dS - P rowsum(dS); for
//                        dQ that is the second term (the mu_k part of K = K_s + mu_k cancels
//                        since sum_j P = 1), and the dQ kernel runs first and hands D^ to the
//                        dK/dV kernel.
// Every step that varies from tile to tile is either a power of two taken by the scaled
// MFMA or factors out of the whole contraction, so the accumulators never need a per-tile
// rescale on the vector unit.  Two kernels, both forward-shaped, so every operand reaches
// the MFMA straight from registers or LDS: a key-stationary kernel (a wave owns 32 keys,
// loops over query tiles, accumulates dK^T and dV^T) and a query-stationary kernel (a wave
// owns 32 queries, loops over key tiles, accumulates dQ^T).  A prologue writes the operand
// layouts they need: dO and V in FP8 token-major with block steps, dO^T, Q^T and K_s^T in
// FP8 with channel steps, D and the smoothed-domain LSE in log2 units.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

namespace {

constexpr int kNT = 3;   // channel-step tensors: dO, Q, K_s

// Row of the 64-row operand tile fed to MFMA A-row m in subtile s, so that output lane
// half h holds tile positions 32h + 16s + r (r = register index).
__device__ __forceinline__ int tile_perm(int m, int s) { return 32 * ((m >> 2) & 1) + 16 * s + 4 * (m >> 3) + (m & 3); }

// 16-byte chunk swizzles (see the forward kernel): token-major 64-byte rows read by
// tile_perm lanes, and 64-byte transposed (channel) rows read by 16 consecutive lanes.
__device__ __forceinline__ int swz_row64(int r) { return ((r >> 2) & 1) | (((r >> 5) & 1) << 1); }
__device__ __forceinline__ int swz_t64(int r) { return (r >> 2) & 3; }

struct BwdPtrs {
  // forward quantization (INT8 Q, K_s; mu_k; lse correction)
  const int8_t* q_codes;
  const float* q_step;
  const int8_t* k_codes;
  const float* k_step;
  const float* mu_k;
  const float* lse_corr;
  // backward prologue outputs
  uint32_t* amax_part;    // [3, kStatChunks, BH, d] max |x| per token chunk and channel (bit patterns)
  float* chan_step;       // [3, BH, d] channel steps of dO^T, Q^T, K_s^T codes
  float* Dvec;            // [BH, Np]
  float* lse2;            // [BH, Np] (LSE - c) log2 e - log2 448; +inf for padding queries
  uint8_t* do_codes;      // [BH, Np, d] E4M3, token-major
  float* do_step;         // [BH, nb]
  uint8_t* v_codes;       // [BH, Np, d] E4M3, token-major
  float* v_step;          // [BH, nb]
  uint8_t* doT_codes;     // [BH, Np/64, d, 64] E4M3 of dO / channel step
  uint8_t* qT_codes;      // [BH, Np/64, d, 64] E4M3 of Q / channel step
  uint8_t* kT_codes;      // [BH, Np/64, d, 64] E4M3 of (K - mu_k) / channel step
};

template <int DT>
__device__ __forceinline__ void load8io(const uint16_t* p, float* x) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = DT == 0 ? bf16_to_f32(w[i] & 0xffff) : f16_to_f32(w[i] & 0xffff);
    x[2 * i + 1] = DT == 0 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
  }
}

// max |dO|, |Q|, |K - mu_k| per channel over one of kStatChunks token chunks of a head;
// partials, so no buffer needs clearing first.  grid (kStatChunks, BH), 256 threads.
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, const float* __restrict__ mu_k,
                                                        int N, uint32_t* __restrict__ part) {
  constexpr int C8 = D / 8, RP = 256 / C8;
  const int bh = blockIdx.y, ch = blockIdx.x, BH = gridDim.y, tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  const int len = (N + kStatChunks - 1) / kStatChunks, t0 = ch * len, t1 = min(N, t0 + len);
  float mu[8];
#pragma unroll
  for (int i = 0; i < 8; i++) mu[i] = mu_k[(size_t)bh * D + c0 + i];
  uint32_t a[kNT][8] = {};
  for (int r = t0 + r0; r < t1; r += RP) {
    const size_t off = ((size_t)bh * N + r) * D + c0;
    float x[kNT][8];
    load8io<DT>(dout + off, x[0]);
    load8io<DT>(q + off, x[1]);
    load8io<DT>(k + off, x[2]);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      a[0][i] = max(a[0][i], __float_as_uint(fabsf(x[0][i])));
      a[1][i] = max(a[1][i], __float_as_uint(fabsf(x[1][i])));
      a[2][i] = max(a[2][i], __float_as_uint(fabsf(x[2][i] - mu[i])));
    }
  }
  __shared__ uint32_t s_a[kNT][RP][D];
#pragma unroll
  for (int t = 0; t < kNT; t++)
#pragma unroll
    for (int i = 0; i < 8; i++) s_a[t][r0][c0 + i] = a[t][i];
  __syncthreads();
  for (int j = tid; j < kNT * D; j += 256) {
    const int t = j / D, c = j % D;
    uint32_t m = 0;
    for (int r = 0; r < RP; r++) m = max(m, s_a[t][r][c]);
    part[(((size_t)t * kStatChunks + ch) * BH + bh) * D + c] = m;
  }
}

// Unpack 8 16-bit inputs (one 16-byte load) to fp32.
template <int DT>
__device__ __forceinline__ void unpack8io(const uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = DT == 0 ? bf16_to_f32(w[i] & 0xffff) : f16_to_f32(w[i] & 0xffff);
    x[2 * i + 1] = DT == 0 ? bf16_to_f32(w[i] >> 16) : f16_to_f32(w[i] >> 16);
  }
}

// Per 64-token block: D, lse2, dO / V token-major FP8 with block steps, dO^T / Q^T / K_s^T
// FP8 with channel steps.  grid (Np/64, BH), 2*D threads.  A thread holds channels
// 8 cidx .. 8 cidx + 7 of the block's rows 4 rg .. 4 rg + 3, so one channel's four codes are
// one dword of the transposed [channel][token] layout; a wave covers 8 channel groups x 8
// row groups (8 rows of 128 contiguous bytes per load).  The transposed dwords pass through
// LDS rows of 17 dwords (one pad dword), which puts the 64 lanes of a write on 64 distinct
// banks, and leave as 16-byte stores of whole token rows.
template <int DT, int D>
__global__ __launch_bounds__(2 * D) void bwd_prep_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                         const uint16_t* __restrict__ v, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k, const float* __restrict__ lse,
                                                         int N, int Np, BwdPtrs bp) {
  constexpr int NTH = 2 * D, CG = D / 64, NW = NTH / 64, RS = 17;
  const int bh = blockIdx.y, blk = blockIdx.x, t0 = blk * 64, BH = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cidx = 8 * (w % CG) + (lane & 7), rg = 8 * (w / CG) + (lane >> 3), c0 = 8 * cidx;
  const int nb = Np / 64;
  __shared__ float s_inv[kNT][D];
  __shared__ uint32_t s_red[2][NW];
  __shared__ float s_dsum[CG][64];
  __shared__ uint32_t s_T[kNT][D * RS];
  // the thread's raw inputs, all loads issued first (rows past N read as zero)
  uint4 rd[4], ro[4], rv[4], rq[4], rk[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int row = t0 + 4 * rg + r;
    rd[r] = ro[r] = rv[r] = rq[r] = rk[r] = make_uint4(0, 0, 0, 0);
    if (row < N) {
      const size_t off = ((size_t)bh * N + row) * D + c0;
      rd[r] = *reinterpret_cast<const uint4*>(dout + off);
      ro[r] = *reinterpret_cast<const uint4*>(o + off);
      rv[r] = *reinterpret_cast<const uint4*>(v + off);
      rq[r] = *reinterpret_cast<const uint4*>(q + off);
      rk[r] = *reinterpret_cast<const uint4*>(k + off);
    }
  }
  // channel steps from the chunk partials: code = x * 448 / amax
  for (int j = tid; j < kNT * D; j += NTH) {
    const int t = j / D, c = j % D;
    uint32_t m = 0;
#pragma unroll
    for (int ch = 0; ch < kStatChunks; ch++) m = max(m, bp.amax_part[(((size_t)t * kStatChunks + ch) * BH + bh) * D + c]);
    const float am = __uint_as_float(m);
    s_inv[t][c] = am == 0.0f ? 0.0f : 448.0f / am;
    if (blk == 0) bp.chan_step[((size_t)t * BH + bh) * D + c] = am / 448.0f;
  }
  float mu[8];
#pragma unroll
  for (int i = 0; i < 8; i++) mu[i] = bp.mu_k[(size_t)bh * D + c0 + i];
  __syncthreads();
  // row sums dO.O, max |dO| and |V|, and the channel-step codes, two rows at a time
  uint32_t tw[kNT][8];
  uint32_t ad = 0, av = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
#pragma unroll
    for (int r2 = 0; r2 < 2; r2++) {
      const int r = 2 * h + r2;
      float xd[8], xo[8], xv[8];
      unpack8io<DT>(rd[r], xd);
      unpack8io<DT>(ro[r], xo);
      unpack8io<DT>(rv[r], xv);
      float dsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        dsum += xd[i] * xo[i];
        ad = max(ad, __float_as_uint(fabsf(xd[i])));
        av = max(av, __float_as_uint(fabsf(xv[i])));
      }
      // sum over the 8 lanes of this wave that share the row
#pragma unroll
      for (int o2 = 1; o2 < 8; o2 <<= 1) dsum += __shfl_xor(dsum, o2);
      if ((lane & 7) == 0) s_dsum[w % CG][4 * rg + r] = dsum;
    }
    const int r0 = 2 * h;
    float xd[2][8], xq[2][8], xk[2][8];
#pragma unroll
    for (int r2 = 0; r2 < 2; r2++) {
      unpack8io<DT>(rd[r0 + r2], xd[r2]);
      unpack8io<DT>(rq[r0 + r2], xq[r2]);
      unpack8io<DT>(rk[r0 + r2], xk[r2]);
      const bool in = t0 + 4 * rg + r0 + r2 < N;   // padding rows stay zero (not -mu_k)
#pragma unroll
      for (int i = 0; i < 8; i++) xk[r2][i] = in ? xk[r2][i] - mu[i] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float s0 = s_inv[0][c0 + i], s1 = s_inv[1][c0 + i], s2 = s_inv[2][c0 + i];
      if (h == 0) {   // rows 0, 1 -> bytes 0, 1
        tw[0][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xd[0][i] * s0, xd[1][i] * s0, 0, false);
        tw[1][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xq[0][i] * s1, xq[1][i] * s1, 0, false);
        tw[2][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xk[0][i] * s2, xk[1][i] * s2, 0, false);
      } else {        // rows 2, 3 -> bytes 2, 3
        tw[0][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xd[0][i] * s0, xd[1][i] * s0, tw[0][i], true);
        tw[1][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xq[0][i] * s1, xq[1][i] * s1, tw[1][i], true);
        tw[2][i] = __builtin_amdgcn_cvt_pk_fp8_f32(xk[0][i] * s2, xk[1][i] * s2, tw[2][i], true);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kNT; t++)
#pragma unroll
    for (int i = 0; i < 8; i++) s_T[t][(c0 + i) * RS + rg] = tw[t][i];
  // block max |dO|, |V|
#pragma unroll
  for (int o2 = 1; o2 < 64; o2 <<= 1) {
    ad = max(ad, (uint32_t)__shfl_xor((int)ad, o2));
    av = max(av, (uint32_t)__shfl_xor((int)av, o2));
  }
  if (lane == 0) {
    s_red[0][w] = ad;
    s_red[1][w] = av;
  }
  __syncthreads();
  uint32_t amd = 0, amv = 0;
#pragma unroll
  for (int j = 0; j < NW; j++) {
    amd = max(amd, s_red[0][j]);
    amv = max(amv, s_red[1][j]);
  }
  const float id = amd == 0 ? 0.0f : 448.0f / __uint_as_float(amd), iv = amv == 0 ? 0.0f : 448.0f / __uint_as_float(amv);
  if (tid < 64) {
    const int row = t0 + tid;
    float dsum = s_dsum[0][tid];
    if (CG == 2) dsum += s_dsum[CG - 1][tid];
    bp.Dvec[(size_t)bh * Np + row] = dsum;
    bp.lse2[(size_t)bh * Np + row] =
        row < N ? (lse[(size_t)bh * N + row] - bp.lse_corr[(size_t)bh * N + row]) * kLog2e - kLog2_448 : INFINITY;
    if (tid == 0) {
      bp.do_step[(size_t)bh * nb + blk] = __uint_as_float(amd) / 448.0f;
      bp.v_step[(size_t)bh * nb + blk] = __uint_as_float(amv) / 448.0f;
    }
  }
  // token-major dO and V codes with the block steps
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float xd[8], xv[8];
    unpack8io<DT>(rd[r], xd);
    unpack8io<DT>(rv[r], xv);
    uint32_t wd[2], wv[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      wd[j] = __builtin_amdgcn_cvt_pk_fp8_f32(xd[4 * j] * id, xd[4 * j + 1] * id, 0, false);
      wd[j] = __builtin_amdgcn_cvt_pk_fp8_f32(xd[4 * j + 2] * id, xd[4 * j + 3] * id, wd[j], true);
      wv[j] = __builtin_amdgcn_cvt_pk_fp8_f32(xv[4 * j] * iv, xv[4 * j + 1] * iv, 0, false);
      wv[j] = __builtin_amdgcn_cvt_pk_fp8_f32(xv[4 * j + 2] * iv, xv[4 * j + 3] * iv, wv[j], true);
    }
    const size_t off = ((size_t)bh * Np + t0 + 4 * rg + r) * D + c0;
    *reinterpret_cast<uint2*>(bp.do_codes + off) = make_uint2(wd[0], wd[1]);
    *reinterpret_cast<uint2*>(bp.v_codes + off) = make_uint2(wv[0], wv[1]);
  }
  // transposed codes: 16-byte chunks e (channel e/4, tokens 16(e%4) ..) of the [D][64] tile
  const size_t tb = ((size_t)bh * nb + blk) * D * 64;
  uint8_t* const dstT[kNT] = {bp.doT_codes, bp.qT_codes, bp.kT_codes};
#pragma unroll
  for (int t = 0; t < kNT; t++)
#pragma unroll
    for (int e = tid; e < D * 4; e += NTH) {
      const uint32_t* src = &s_T[t][(e >> 2) * RS + 4 * (e & 3)];
      *reinterpret_cast<uint4*>(dstT[t] + tb + (size_t)e * 16) = make_uint4(src[0], src[1], src[2], src[3]);
    }
}

// ---- shared pieces of the two main kernels ----

// Work item of a workgroup: the dispatcher deals workgroups round-robin to the 8 XCDs; each
// XCD takes whole heads (their tiles then share its L2) and, within its heads, item 0 (the
// heaviest under a causal mask) first, so the long items do not trail at the end.
__device__ __forceinline__ void work_item(int hw_id, int BH, int nt, int& bh, int& t) {
  constexpr int X = 8;
  if (BH % X == 0) {
    const int hpx = BH / X, local = hw_id / X;
    t = local / hpx;
    bh = (hw_id % X) * hpx + local % hpx;
  } else {
    bh = hw_id / nt;
    t = hw_id % nt;
  }
}

// Direct loads of one 64-row token-major tile (64 x D bytes) into LDS with the row swizzle.
template <int D>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const uint8_t* g, int w, int lane) {
  constexpr int CH = D / 16, CHUNKS = 64 * CH;
#pragma unroll
  for (int i = 0; i < (CHUNKS + 255) / 256; i++) {
    const int pbase = 256 * i + 64 * w;
    if (pbase < CHUNKS) {
      const int P = pbase + lane, row = P / CH, col = (P % CH) ^ (D == 64 ? swz_row64(row) : (((row >> 1) & 3) | (((row >> 5) & 1) << 2)));
      load_lds16(g + row * D + col * 16, lds + pbase * 16);
    }
  }
}
// Direct loads of one transposed tile (D rows x 64 bytes) into LDS with the channel-row swizzle.
template <int D>
__device__ __forceinline__ void stage_cols(uint8_t* lds, const uint8_t* g, int w, int lane) {
  constexpr int CHUNKS = D * 4;
#pragma unroll
  for (int i = 0; i < (CHUNKS + 255) / 256; i++) {
    const int pbase = 256 * i + 64 * w;
    if (pbase < CHUNKS) {
      const int P = pbase + lane, row = P >> 2, col = (P & 3) ^ swz_t64(row);
      load_lds16(g + row * 64 + col * 16, lds + pbase * 16);
    }
  }
}
template <int D>
__device__ __forceinline__ int rowoff(int row, int chunk) {
  return row * D + ((chunk ^ (D == 64 ? swz_row64(row) : (((row >> 1) & 3) | (((row >> 5) & 1) << 2)))) << 4);
}
__device__ __forceinline__ int coloff(int row, int chunk) { return row * 64 + ((chunk ^ swz_t64(row)) << 4); }

__device__ __forceinline__ v8i lds_v8i(const uint8_t* p0, const uint8_t* p1) {
  const v4i x0 = *reinterpret_cast<const v4i*>(p0), x1 = *reinterpret_cast<const v4i*>(p1);
  return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// O^T[32 x 32] += A[32 x 64] B[64 x 32] in E4M3, B scaled per 32-element K block by the
// E8M0 byte `sb` (A unscaled).  The two K blocks of the scaled form are bytes 0-15 and
// 16-31 of both lane halves; block b takes its scale from the lanes of half b.
__device__ __forceinline__ v16f mfma_f8_sb(v8i a, v8i b, v16f c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// E8M0 byte of the smallest power of two s with amax / s <= 448 (the E4M3 maximum), at
// least 1 so that the scale is a normal float.  amax = 2^(E-127) (1 + f): E - 8 suffices
// when 1 + f <= 1.75, else E - 7.
__device__ __forceinline__ int e4m3_scale_byte(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 23) - 8 + ((amax_bits & 0x7fffff) > 0x600000 ? 1 : 0);
  return max(e, 1);
}

// A lane's 32 dS values (bytes 0-15: subtile 0, bytes 16-31: subtile 1) -> E4M3 B operand
// with per-block scales.  a0 / a1: the lane's max |x| over each subtile.  Returns the
// E8M0 byte this lane supplies to the MFMA (block hh of its column).
__device__ __forceinline__ int quant_ds(const float* x, float a0, float a1, int hh, v8i& out) {
  // block b spans both halves' subtile b: lane l < 32 gets block 0's max, lane l >= 32 block 1's
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  const uint32_t mine = max((uint32_t)sw[0], (uint32_t)sw[1]);
  const uint32_t other = __float_as_uint(other_half(__uint_as_float(mine)));
  const int bm = e4m3_scale_byte(mine), bo = e4m3_scale_byte(other);
  const float sc0 = __uint_as_float((uint32_t)(hh ? bo : bm) << 23), sc1 = __uint_as_float((uint32_t)(hh ? bm : bo) << 23);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float sc = i < 4 ? sc0 : sc1;
    typedef short v2s __attribute__((ext_vector_type(2)));
    v2s w = __builtin_bit_cast(v2s, __float_as_int(x[4 * i]));   // high half overwritten below
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[4 * i], x[4 * i + 1], sc, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[4 * i + 2], x[4 * i + 3], sc, true);
    out[i] = __builtin_bit_cast(int, w);
  }
  return bm;
}

// ---- key-stationary kernel: dK and dV ----
// Workgroup: 128 keys (4 waves x 32), loops over 64-query tiles.  LDS per stage:
// Q rows, dO rows (token-major), dO^T and Q^T (channel rows), lse2 and D (64 floats each).
// d = 128 doubles the accumulators (dK^T, dV^T: 128 registers) and the operand tiles, so one
// workgroup runs per CU there, with the accumulators in the AGPR half of the register file.
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdPtrs bp, void* dk, void* dv, int N, int Np, int BH, float sm) {
  constexpr int TB = 64 * D;                          // one tile of 64 x D bytes
  constexpr int STAGE = 4 * TB + 2 * 64 * 4 + 16;   // + the tile's Q step and dO step
  constexpr int NCB = D / 32;
  __shared__ __align__(16) uint8_t lds[2][STAGE];
  const int nkt = Np / 128;
  int bh, kt;
  work_item(blockIdx.x, BH, nkt, bh, kt);
  const int kbase = kt * 128;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int kw = kbase + 32 * w, key = kw + n;
  const int nb = Np / 64;
  const float smlog2e = sm * kLog2e;

  // resident B operands: K_s codes (for S) and V FP8 (for dP) of this wave's 32 keys
  v4i kf[D / 32];
  v8i vf[D / 64];
  {
    const int8_t* kp = bp.k_codes + ((size_t)bh * Np + key) * D + 16 * hh;
#pragma unroll
    for (int c = 0; c < D / 32; c++) kf[c] = *reinterpret_cast<const v4i*>(kp + 32 * c);
    const uint8_t* vp = bp.v_codes + ((size_t)bh * Np + key) * D + 32 * hh;
#pragma unroll
    for (int c = 0; c < D / 64; c++) vf[c] = lds_v8i(vp + 64 * c, vp + 64 * c + 16);
  }
  const float kstep = bp.k_step[(size_t)bh * nb + kw / 64];
  const float vstep = bp.v_step[(size_t)bh * nb + kw / 64];

  v16f dV[NCB], dK[NCB];
#pragma unroll
  for (int c = 0; c < NCB; c++) dV[c] = dK[c] = v16f{};

  const int qt0 = CAUSAL ? kbase / 64 : 0;
  const int nqt = (N + 63) / 64;
  auto stage = [&](int buf, int qt) {
    uint8_t* L = lds[buf];
    const size_t rb = ((size_t)bh * Np + (size_t)qt * 64) * D;
    const size_t tb = ((size_t)bh * nb + qt) * TB;
    stage_rows<D>(L, reinterpret_cast<const uint8_t*>(bp.q_codes) + rb, w, lane);
    stage_rows<D>(L + TB, bp.do_codes + rb, w, lane);
    stage_cols<D>(L + 2 * TB, bp.doT_codes + tb, w, lane);
    stage_cols<D>(L + 3 * TB, bp.qT_codes + tb, w, lane);
    if (w == 0 && lane < 16) load_lds16(bp.lse2 + (size_t)bh * Np + qt * 64 + 4 * lane, L + 4 * TB + 16 * lane);
    if (w == 1 && lane < 16) load_lds16(bp.Dvec + (size_t)bh * Np + qt * 64 + 4 * lane, L + 4 * TB + 256 + 16 * lane);
    if (w == 2 && lane < 2) load_lds4((lane ? bp.do_step : bp.q_step) + (size_t)bh * nb + qt, L + 4 * TB + 512);
  };
  // one query tile: S, dP on MFMA; P~ and dS on the vector unit; dV^T, dK^T on MFMA
  auto tile = [&](const uint8_t* L, int qt, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int qb = qt * 64;
    const float qstep = reinterpret_cast<const float*>(L + 4 * TB + 512)[0];
    const float dostep = reinterpret_cast<const float*>(L + 4 * TB + 512)[1];
    v16i S[2];
    v16f G[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int row = tile_perm(n, s);
      v16i a = v16i{};
#pragma unroll
      for (int c = 0; c < D / 32; c++) a = mfma_i8(*reinterpret_cast<const v4i*>(L + rowoff<D>(row, 2 * c + hh)), kf[c], a);
      S[s] = a;
      v16f b = v16f{};
#pragma unroll
      for (int c = 0; c < D / 64; c++)
        b = mfma_f8(lds_v8i(L + TB + rowoff<D>(row, 4 * c + 2 * hh), L + TB + rowoff<D>(row, 4 * c + 2 * hh + 1)), vf[c], b);
      G[s] = b;
    }
    // element r of subtile s: query qb + 32 hh + 16 s + r, key = this lane's key.
    // p = 448 P (lse2 carries -log2 448); ds = p (dP - D) = 448 dS.
    const float cS = qstep * kstep * smlog2e, cP = dostep * vstep;
    const float* l2 = reinterpret_cast<const float*>(L + 4 * TB) + 32 * hh;
    const float* Dv = reinterpret_cast<const float*>(L + 4 * TB + 256) + 32 * hh;
    float p[32], ds[32], am[2] = {0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const v4f lv = *reinterpret_cast<const v4f*>(l2 + 16 * s + r);
        const v4f dvv = *reinterpret_cast<const v4f*>(Dv + 16 * s + r);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float x = fmaf((float)S[s][r + i], cS, -lv[i]);
          if (MASKED) x = key <= qb + 32 * hh + 16 * s + r + i ? x : -INFINITY;
          const float e = fast_exp2(x);
          const float d = e * fmaf(G[s][r + i], cP, -dvv[i]);
          p[16 * s + r + i] = e;
          ds[16 * s + r + i] = d;
          am[s] = fmaxf(am[s], fabsf(d));
        }
      }
    // dV^T += dO^T P~ (FP8, K = 64 queries)
    v8i pb;
#pragma unroll
    for (int i = 0; i < 32; i += 4) pb[i / 4] = pack_fp8x4(p[i], p[i + 1], p[i + 2], p[i + 3]);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) {
      const int row = 32 * cb + n;
      dV[cb] = mfma_f8(lds_v8i(L + 2 * TB + coloff(row, 2 * hh), L + 2 * TB + coloff(row, 2 * hh + 1)), pb, dV[cb]);
    }
    // dK^T += Q^T dS~ (dS in E4M3 with per-block power-of-two scales)
    v8i db;
    const int sb = quant_ds(ds, am[0], am[1], hh, db);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) {
      const int row = 32 * cb + n;
      dK[cb] = mfma_f8_sb(lds_v8i(L + 3 * TB + coloff(row, 2 * hh), L + 3 * TB + coloff(row, 2 * hh + 1)), db, dK[cb], sb);
    }
  };
  // per-wave phases over the query tiles (wave-uniform bounds, so the accumulators never meet
  // a branch join inside a loop): tiles whose queries all precede this wave's keys add nothing,
  // then the diagonal tiles need the causal mask, then every pair is visible.  Keys >= N need
  // no mask: their columns only reach their own (unstored) dK, dV rows.
  const int qt_first = kw >= N ? nqt : (CAUSAL ? max(qt0, kw / 64) : qt0);
  const int qt_open = kw >= N ? nqt : (CAUSAL ? max(qt_first, (kw + 94) / 64) : qt0);
  auto iter = [&](int qt, auto mode) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) stage(buf ^ 1, qt + 1);
    if constexpr (decltype(mode)::value >= 0) tile(lds[buf], qt, std::bool_constant<decltype(mode)::value == 1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  if (qt0 < nqt) stage(0, qt0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  int qt = qt0;
  for (; qt < min(qt_first, nqt); qt++) iter(qt, std::integral_constant<int, -1>{});
  for (; qt < min(qt_open, nqt); qt++) iter(qt, std::integral_constant<int, 1>{});
  for (; qt < nqt; qt++) iter(qt, std::integral_constant<int, 0>{});
  // epilogue: dK = sm qT_step dK^T / 448, dV = doT_step dV^T / 448; lane holds channels
  // 32 cb + 8 g + 4 hh + {0..3} of its key.  All factors are loaded before the first store.
  if (key < N) {
    uint16_t* dkr = reinterpret_cast<uint16_t*>(dk) + ((size_t)bh * N + key) * D;
    uint16_t* dvr = reinterpret_cast<uint16_t*>(dv) + ((size_t)bh * N + key) * D;
    const float* cdo = bp.chan_step + (size_t)bh * D + 4 * hh;
    const float* cq = bp.chan_step + ((size_t)BH + bh) * D + 4 * hh;
    v4f fk[NCB][4], fv[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        fk[cb][g] = *reinterpret_cast<const v4f*>(cq + 32 * cb + 8 * g);
        fv[cb][g] = *reinterpret_cast<const v4f*>(cdo + 32 * cb + 8 * g);
      }
    const float kf448 = sm * (1.0f / 448.0f);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * cb + 8 * g + 4 * hh;
        uint32_t k2[2], v2[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const int i0 = 2 * t, i1 = 2 * t + 1;
          k2[t] = (uint32_t)to_io<DT>(dK[cb][4 * g + i0] * (fk[cb][g][i0] * kf448)) |
                  ((uint32_t)to_io<DT>(dK[cb][4 * g + i1] * (fk[cb][g][i1] * kf448)) << 16);
          v2[t] = (uint32_t)to_io<DT>(dV[cb][4 * g + i0] * (fv[cb][g][i0] * (1.0f / 448.0f))) |
                  ((uint32_t)to_io<DT>(dV[cb][4 * g + i1] * (fv[cb][g][i1] * (1.0f / 448.0f))) << 16);
        }
        *reinterpret_cast<uint2*>(dkr + ch) = make_uint2(k2[0], k2[1]);
        *reinterpret_cast<uint2*>(dvr + ch) = make_uint2(v2[0], v2[1]);
      }
  }
}

// ---- query-stationary kernel: dQ ----
// Workgroup: 128 queries (4 waves x 32), loops over 64-key tiles.  LDS per stage:
// K_s rows (INT8), V rows (FP8), K_s^T (channel rows, FP8).  One workgroup per CU at d = 128,
// as for the dK/dV kernel.
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dq_kernel(BwdPtrs bp, void* dq, int N, int Np, int BH, float sm) {
  constexpr int TB = 64 * D;
  constexpr int STAGE = 3 * TB + 16;   // + the tile's K step and V step
  constexpr int NCB = D / 32;
  __shared__ __align__(16) uint8_t lds[2][STAGE];
  const int nqt = Np / 128;
  int bh, t;
  work_item(blockIdx.x, BH, nqt, bh, t);
  const int qt = CAUSAL ? nqt - 1 - t : t;   // causal: the longest rows first
  const int qbase = qt * 128;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int qw = qbase + 32 * w, q = qw + n;
  const int nb = Np / 64;
  const float smlog2e = sm * kLog2e;

  // resident B operands: Q codes (for S^T) and dO FP8 (for dP^T) of this wave's queries
  v4i qf[D / 32];
  v8i df[D / 64];
  {
    const int8_t* qp = bp.q_codes + ((size_t)bh * Np + q) * D + 16 * hh;
#pragma unroll
    for (int c = 0; c < D / 32; c++) qf[c] = *reinterpret_cast<const v4i*>(qp + 32 * c);
    const uint8_t* dp = bp.do_codes + ((size_t)bh * Np + q) * D + 32 * hh;
#pragma unroll
    for (int c = 0; c < D / 64; c++) df[c] = lds_v8i(dp + 64 * c, dp + 64 * c + 16);
  }
  const float qstep = bp.q_step[(size_t)bh * nb + q / 64];
  const float dostep = bp.do_step[(size_t)bh * nb + q / 64];
  const float l2 = bp.lse2[(size_t)bh * Np + q];
  const float Dq = bp.Dvec[(size_t)bh * Np + q];

  v16f dQ[NCB], PK[NCB];
#pragma unroll
  for (int c = 0; c < NCB; c++) dQ[c] = PK[c] = v16f{};
  float rsum = 0.0f;

  int nkt = (N + 63) / 64;
  if (CAUSAL) nkt = min(nkt, (qbase + 127) / 64 + 1);
  auto stage = [&](int buf, int kt) {
    uint8_t* L = lds[buf];
    const size_t rb = ((size_t)bh * Np + (size_t)kt * 64) * D;
    const size_t tb = ((size_t)bh * nb + kt) * TB;
    stage_rows<D>(L, reinterpret_cast<const uint8_t*>(bp.k_codes) + rb, w, lane);
    stage_rows<D>(L + TB, bp.v_codes + rb, w, lane);
    stage_cols<D>(L + 2 * TB, bp.kT_codes + tb, w, lane);
    if (w == 0 && lane < 2) load_lds4((lane ? bp.v_step : bp.k_step) + (size_t)bh * nb + kt, L + 3 * TB);
  };
  auto tile = [&](const uint8_t* L, int kt, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kb = kt * 64;
    const float kstep = reinterpret_cast<const float*>(L + 3 * TB)[0];
    const float vstep = reinterpret_cast<const float*>(L + 3 * TB)[1];
    v16i S[2];
    v16f G[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const int row = tile_perm(n, s);
      v16i a = v16i{};
#pragma unroll
      for (int c = 0; c < D / 32; c++) a = mfma_i8(*reinterpret_cast<const v4i*>(L + rowoff<D>(row, 2 * c + hh)), qf[c], a);
      S[s] = a;
      v16f b = v16f{};
#pragma unroll
      for (int c = 0; c < D / 64; c++)
        b = mfma_f8(lds_v8i(L + TB + rowoff<D>(row, 4 * c + 2 * hh), L + TB + rowoff<D>(row, 4 * c + 2 * hh + 1)), df[c], b);
      G[s] = b;
    }
    // element r of subtile s: key kb + 32 hh + 16 s + r, query = this lane's query
    const float cS = qstep * kstep * smlog2e, cP = dostep * vstep;
    const int lim = min(N, CAUSAL ? q + 1 : N) - (kb + 32 * hh);   // keys i < lim are visible
    float p[32], ds[32], am[2] = {0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float x = fmaf((float)S[s][r], cS, -l2);
        if (MASKED) x = 16 * s + r < lim ? x : -INFINITY;
        const float e = fast_exp2(x);
        const float d = e * fmaf(G[s][r], cP, -Dq);
        p[16 * s + r] = e;
        ds[16 * s + r] = d;
        rsum += d;
        am[s] = fmaxf(am[s], fabsf(d));
      }
    v8i pb, db;
#pragma unroll
    for (int i = 0; i < 32; i += 4) pb[i / 4] = pack_fp8x4(p[i], p[i + 1], p[i + 2], p[i + 3]);
    const int sb = quant_ds(ds, am[0], am[1], hh, db);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) {
      const int row = 32 * cb + n;
      const v8i a = lds_v8i(L + 2 * TB + coloff(row, 2 * hh), L + 2 * TB + coloff(row, 2 * hh + 1));
      dQ[cb] = mfma_f8_sb(a, db, dQ[cb], sb);
      PK[cb] = mfma_f8(a, pb, PK[cb]);   // P K_s for the rowsum correction
    }
  };
  // per-wave phases over the key tiles (wave-uniform bounds): fully visible tiles, then the
  // diagonal / ragged-end tiles that need the mask, then tiles past this wave's last query
  const int nkt_n = (N + 63) / 64;
  const int nvis = CAUSAL ? min(nkt_n, (qw + 31) / 64 + 1) : nkt_n;
  const int nfull = min(N / 64, CAUSAL ? (qw + 1) / 64 : nkt_n);
  auto iter = [&](int kt, auto mode) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) stage(buf ^ 1, kt + 1);
    if constexpr (decltype(mode)::value >= 0) tile(lds[buf], kt, std::bool_constant<decltype(mode)::value == 1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  int kt = 0;
  for (; kt < min(nfull, nkt); kt++) iter(kt, std::integral_constant<int, 0>{});
  for (; kt < min(nvis, nkt); kt++) iter(kt, std::integral_constant<int, 1>{});
  for (; kt < nkt; kt++) iter(kt, std::integral_constant<int, -1>{});
  // epilogue: dQ = sm kT_step (dQ^T - rs PK^T) / 448 with rs = rowsum(dS); hand D^ = D + rs
  // to the dK/dV kernel
  const float rs = half_sum(rsum) * (1.0f / 448.0f);
  if (q < N) {
    uint16_t* dqr = reinterpret_cast<uint16_t*>(dq) + ((size_t)bh * N + q) * D;
    const float* ck = bp.chan_step + ((size_t)2 * BH + bh) * D + 4 * hh;
    v4f fq[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) fq[cb][g] = *reinterpret_cast<const v4f*>(ck + 32 * cb + 8 * g);
    const float f448 = sm * (1.0f / 448.0f);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * cb + 8 * g + 4 * hh;
        uint32_t w2[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; t2++) {
          const int i0 = 2 * t2, i1 = 2 * t2 + 1;
          w2[t2] = (uint32_t)to_io<DT>(fq[cb][g][i0] * f448 * fmaf(-rs, PK[cb][4 * g + i0], dQ[cb][4 * g + i0])) |
                   ((uint32_t)to_io<DT>(fq[cb][g][i1] * f448 * fmaf(-rs, PK[cb][4 * g + i1], dQ[cb][4 * g + i1])) << 16);
        }
        *reinterpret_cast<uint2*>(dqr + ch) = make_uint2(w2[0], w2[1]);
      }
    if (hh == 0) bp.Dvec[(size_t)bh * Np + q] = Dq + rs;
  }
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct BwdLayout {
  size_t amax_part, chan_step, Dvec, lse2, do_codes, do_step, v_codes, v_step, doT, qT, kT, total;
};

BwdLayout bwd_layout(const Shape& s) {
  const size_t BH = (size_t)s.B * s.H, d = s.d, Np = s.Np, nb = Np / 64;
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off = round256(off + b); return o; };
  L.amax_part = take((size_t)kNT * kStatChunks * BH * d * 4);
  L.chan_step = take((size_t)kNT * BH * d * 4);
  L.Dvec = take(BH * Np * 4);
  L.lse2 = take(BH * Np * 4);
  L.do_codes = take(BH * Np * d);
  L.do_step = take(BH * nb * 4);
  L.v_codes = take(BH * Np * d);
  L.v_step = take(BH * nb * 4);
  L.doT = take(BH * Np * d);
  L.qT = take(BH * Np * d);
  L.kT = take(BH * Np * d);
  L.total = off;
  return L;
}

template <int DT, int D>
hipError_t bwd_run(const Shape& s, const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, uint8_t* ws, size_t qbytes, const QuantPtrs& qp,
                   hipStream_t st) {
  const int BH = s.B * s.H;
  const BwdLayout L = bwd_layout(s);
  uint8_t* b = ws + qbytes;
  BwdPtrs bp;
  bp.q_codes = reinterpret_cast<const int8_t*>(qp.q_codes);
  bp.q_step = reinterpret_cast<const float*>(qp.q_scales);
  bp.k_codes = reinterpret_cast<const int8_t*>(qp.k_codes);
  bp.k_step = reinterpret_cast<const float*>(qp.k_scales);
  bp.mu_k = qp.mu_k;
  bp.lse_corr = qp.lse_corr;
  bp.amax_part = reinterpret_cast<uint32_t*>(b + L.amax_part);
  bp.chan_step = reinterpret_cast<float*>(b + L.chan_step);
  bp.Dvec = reinterpret_cast<float*>(b + L.Dvec);
  bp.lse2 = reinterpret_cast<float*>(b + L.lse2);
  bp.do_codes = b + L.do_codes;
  bp.do_step = reinterpret_cast<float*>(b + L.do_step);
  bp.v_codes = b + L.v_codes;
  bp.v_step = reinterpret_cast<float*>(b + L.v_step);
  bp.doT_codes = b + L.doT;
  bp.qT_codes = b + L.qT;
  bp.kT_codes = b + L.kT;
  // forward quantization of Q, K (the codes the forward used; V's are not needed), then the
  // backward prologue
  Shape sqk = s;
  sqk.pv_fmt = PV_NONE;
  hipError_t e = launch_prologue(q, k, v, sqk, qp, st);
  if (e != hipSuccess) return e;
  bwd_stats_kernel<DT, D><<<dim3(kStatChunks, BH), 256, 0, st>>>((const uint16_t*)dout, (const uint16_t*)q,
                                                                (const uint16_t*)k, qp.mu_k, s.N, bp.amax_part);
  bwd_prep_kernel<DT, D><<<dim3(s.Np / 64, BH), 2 * D, 0, st>>>((const uint16_t*)o, (const uint16_t*)dout,
                                                             (const uint16_t*)v, (const uint16_t*)q,
                                                             (const uint16_t*)k, lse, s.N, s.Np, bp);
  const int grid = BH * (s.Np / 128);
  // dQ first: it turns D into D^ = D + rowsum(dS), which the dK/dV kernel then uses
  if (s.causal) {
    bwd_dq_kernel<D, true, DT><<<grid, 256, 0, st>>>(bp, dq, s.N, s.Np, BH, s.sm_scale);
    bwd_dkdv_kernel<D, true, DT><<<grid, 256, 0, st>>>(bp, dk, dv, s.N, s.Np, BH, s.sm_scale);
  } else {
    bwd_dq_kernel<D, false, DT><<<grid, 256, 0, st>>>(bp, dq, s.N, s.Np, BH, s.sm_scale);
    bwd_dkdv_kernel<D, false, DT><<<grid, 256, 0, st>>>(bp, dk, dv, s.N, s.Np, BH, s.sm_scale);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_ws_bytes(const Shape& s) { return bwd_layout(s).total; }

hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                           size_t qbytes, const QuantPtrs& qp, hipStream_t stream) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (s.d == 64)
    return s.io_dtype == 0 ? bwd_run<0, 64>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream)
                           : bwd_run<1, 64>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream);
  return s.io_dtype == 0 ? bwd_run<0, 128>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream)
                         : bwd_run<1, 128>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream);
}

}  // namespace sage
