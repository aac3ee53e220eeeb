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
//   dV  = P~^T dO        FP8: P~ = E4M3(448 P), dO per-channel steps (factor out of the
//                        query sum)
//   dK  = sm dS~^T Q     INT8: dS~ = INT8 codes of dS with one step per wave tile
//   dQ  = sm (dS~ K_s - rowsum(dS) P K_s)  INT8.  With quantized dP the rows of dS no
//                        longer sum to 0: rowsum(dS) = D^ - D, where D^ = sum_j P dP^ is
//                        the value consistent with the quantized dP.  Replacing D by D^
//                        turns dS into dS - P rowsum(dS); for dQ that is the second term
//                        (the mu_k part of K = K_s + mu_k cancels since sum_j P = 1), and
//                        the dQ kernel runs first and hands D^ to the dK/dV kernel.
// Two kernels, both forward-shaped, so every operand reaches the MFMA straight from
// registers or LDS: a key-stationary kernel (a wave owns 32 keys, loops over query
// tiles, accumulates dK^T and dV^T) and a query-stationary kernel (a wave owns 32
// queries, loops over key tiles, accumulates dQ^T).  A prologue writes the operand
// layouts they need: dO and V in FP8 token-major with block steps, dO^T in FP8 with
// channel steps, Q^T and K_s^T INT8 tiles, D and the smoothed-domain LSE in log2 units.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

namespace {

constexpr int kT = 64;   // query / key tile (= INT8 and FP8 block)

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
  uint32_t* amax_do;      // [BH, d] max |dO| per channel (bit patterns)
  float* Dvec;            // [BH, Np]
  float* lse2;            // [BH, Np] (LSE - c) log2 e; +inf for padding queries
  uint8_t* do_codes;      // [BH, Np, d] E4M3, token-major
  float* do_step;         // [BH, nb]
  uint8_t* doT_codes;     // [BH, Np/64, d, 64] E4M3 of dO / channel step
  float* doT_step;        // [BH, d]
  uint8_t* v_codes;       // [BH, Np, d] E4M3, token-major
  float* v_step;          // [BH, nb]
  int8_t* qT_codes;       // [BH, Np/64, d, 64]
  int8_t* kT_codes;       // [BH, Np/64, d, 64]
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

__global__ void bwd_zero_kernel(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// max |dO| per channel.  grid (ceil(N/256), BH), 256 threads.
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const uint16_t* __restrict__ dout, int N, uint32_t* amax) {
  constexpr int C8 = D / 8, RP = 256 / C8;
  const int bh = blockIdx.y, t0 = blockIdx.x * 256, tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  uint32_t a[8] = {};
  for (int r = t0 + r0; r < t0 + 256 && r < N; r += RP) {
    float x[8];
    load8io<DT>(dout + ((size_t)bh * N + r) * D + c0, x);
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = max(a[i], __float_as_uint(fabsf(x[i])));
  }
  __shared__ uint32_t s_a[RP][D];
#pragma unroll
  for (int i = 0; i < 8; i++) s_a[r0][c0 + i] = a[i];
  __syncthreads();
  if (tid < D) {
    uint32_t m = 0;
    for (int r = 0; r < RP; r++) m = max(m, s_a[r][tid]);
    atomicMax(&amax[(size_t)bh * D + tid], m);
  }
}

__device__ __forceinline__ uint32_t block_umax4(uint32_t x, uint32_t* red) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return x;
}

// Per 64-token block: D, lse2, dO / V token-major FP8 with block steps, dO^T FP8 with
// channel steps, Q^T and K_s^T INT8 tiles.  grid (Np/64, BH), 256 threads.
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                       const uint16_t* __restrict__ v, const float* __restrict__ lse,
                                                       int N, int Np, BwdPtrs bp) {
  constexpr int C8 = D / 8, RP = 256 / C8, NP = 64 / RP;
  const int bh = blockIdx.y, blk = blockIdx.x, t0 = blk * 64;
  const int tid = threadIdx.x, c0 = (tid % C8) * 8, r0 = tid / C8;
  const int nb = Np / 64;
  __shared__ uint32_t s_red[4];
  __shared__ __align__(16) uint8_t s_doT[D * 64];
  __shared__ __align__(16) int8_t s_qT[D * 64];
  __shared__ __align__(16) int8_t s_kT[D * 64];
  float dcs[8];
#pragma unroll
  for (int i = 0; i < 8; i++) dcs[i] = __uint_as_float(bp.amax_do[(size_t)bh * D + c0 + i]) / 448.0f;
  float xd[NP][8], xv[NP][8];
  uint32_t ad = 0, av = 0;
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int rl = r0 + p * RP, row = t0 + rl;
    float dsum = 0.0f;
    if (row < N) {
      float xo[8];
      const size_t off = ((size_t)bh * N + row) * D + c0;
      load8io<DT>(dout + off, xd[p]);
      load8io<DT>(o + off, xo);
      load8io<DT>(v + off, xv[p]);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        dsum += xd[p][i] * xo[i];
        ad = max(ad, __float_as_uint(fabsf(xd[p][i])));
        av = max(av, __float_as_uint(fabsf(xv[p][i])));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) xd[p][i] = xv[p][i] = 0.0f;
    }
#pragma unroll
    for (int o2 = 1; o2 < C8; o2 <<= 1) dsum += __shfl_xor(dsum, o2);
    if ((tid % C8) == 0) {
      bp.Dvec[(size_t)bh * Np + row] = dsum;
      bp.lse2[(size_t)bh * Np + row] =
          row < N ? (lse[(size_t)bh * N + row] - bp.lse_corr[(size_t)bh * N + row]) * kLog2e : INFINITY;
    }
    // dO^T with per-channel steps, and the Q^T / K_s^T transposes, through LDS
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float a0 = dcs[i] == 0.0f ? 0.0f : xd[p][i] / dcs[i];
      const float a1 = dcs[i + 1] == 0.0f ? 0.0f : xd[p][i + 1] / dcs[i + 1];
      const int w2 = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      s_doT[(c0 + i) * 64 + rl] = (uint8_t)(w2 & 0xff);
      s_doT[(c0 + i + 1) * 64 + rl] = (uint8_t)((w2 >> 8) & 0xff);
    }
    const uint2 qc = *reinterpret_cast<const uint2*>(bp.q_codes + ((size_t)bh * Np + row) * D + c0);
    const uint2 kc = *reinterpret_cast<const uint2*>(bp.k_codes + ((size_t)bh * Np + row) * D + c0);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      s_qT[(c0 + i) * 64 + rl] = (int8_t)(((i < 4 ? qc.x : qc.y) >> (8 * (i % 4))) & 0xff);
      s_kT[(c0 + i) * 64 + rl] = (int8_t)(((i < 4 ? kc.x : kc.y) >> (8 * (i % 4))) & 0xff);
    }
  }
  const float sd = __uint_as_float(block_umax4(ad, s_red)) / 448.0f;
  const float sv = __uint_as_float(block_umax4(av, s_red)) / 448.0f;
  if (tid == 0) {
    bp.do_step[(size_t)bh * nb + blk] = sd;
    bp.v_step[(size_t)bh * nb + blk] = sv;
  }
  if (blk == 0 && tid < D) bp.doT_step[(size_t)bh * D + tid] = __uint_as_float(bp.amax_do[(size_t)bh * D + tid]) / 448.0f;
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int row = t0 + r0 + p * RP;
    uint32_t wd[2] = {0, 0}, wv[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float d0 = sd == 0.0f ? 0.0f : xd[p][i] / sd, d1 = sd == 0.0f ? 0.0f : xd[p][i + 1] / sd;
      const float v0 = sv == 0.0f ? 0.0f : xv[p][i] / sv, v1 = sv == 0.0f ? 0.0f : xv[p][i + 1] / sv;
      wd[i / 4] |= (uint32_t)(__builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false) & 0xffff) << (8 * (i % 4));
      wv[i / 4] |= (uint32_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false) & 0xffff) << (8 * (i % 4));
    }
    const size_t off = ((size_t)bh * Np + row) * D + c0;
    *reinterpret_cast<uint2*>(bp.do_codes + off) = make_uint2(wd[0], wd[1]);
    *reinterpret_cast<uint2*>(bp.v_codes + off) = make_uint2(wv[0], wv[1]);
  }
  __syncthreads();
  const size_t tb = ((size_t)bh * nb + blk) * D * 64;
  for (int c = tid; c < D * 4; c += 256) {
    *reinterpret_cast<uint4*>(bp.doT_codes + tb + c * 16) = *reinterpret_cast<const uint4*>(s_doT + c * 16);
    *reinterpret_cast<uint4*>(bp.qT_codes + tb + c * 16) = *reinterpret_cast<const uint4*>(s_qT + c * 16);
    *reinterpret_cast<uint4*>(bp.kT_codes + tb + c * 16) = *reinterpret_cast<const uint4*>(s_kT + c * 16);
  }
}

// ---- shared pieces of the two main kernels ----

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

__device__ __forceinline__ float wave_absmax(float x) {
  uint32_t u = __float_as_uint(fabsf(x));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o));
  return __uint_as_float(u);
}

__device__ __forceinline__ int q8(float x, float inv) {
  return (int)fminf(fmaxf(rintf(x * inv), -127.0f), 127.0f);
}
__device__ __forceinline__ int pack_i8x4(int a, int b, int c, int d) {
  return (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | ((d & 0xff) << 24);
}

// ---- key-stationary kernel: dK and dV ----
// Workgroup: 128 keys (4 waves x 32), loops over 64-query tiles.  LDS per stage:
// Q rows, dO rows (token-major), dO^T and Q^T (channel rows), lse2 and D (64 floats each).
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdPtrs bp, void* dk, void* dv, int N, int Np, float sm) {
  constexpr int TB = 64 * D;                          // one tile of 64 x D bytes
  constexpr int STAGE = 4 * TB + 2 * 64 * 4;
  constexpr int NCB = D / 32;
  __shared__ __align__(16) uint8_t lds[2][STAGE];
  const int nkt = Np / 128;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / nkt, kt = id % nkt;
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
    for (int c = 0; c < D / 64; c++) {
      const v4i a0 = *reinterpret_cast<const v4i*>(vp + 64 * c), a1 = *reinterpret_cast<const v4i*>(vp + 64 * c + 16);
      vf[c] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  }
  const float kstep = bp.k_step[(size_t)bh * nb + kw / 64];
  const float vstep = bp.v_step[(size_t)bh * nb + kw / 64];

  v16f dV[NCB], dK[NCB];
#pragma unroll
  for (int c = 0; c < NCB; c++) dV[c] = dK[c] = v16f{};

  int qt0 = CAUSAL ? kbase / 64 : 0;
  const int nqt = (N + 63) / 64;
  auto stage = [&](int buf, int qt) {
    uint8_t* L = lds[buf];
    const size_t rb = ((size_t)bh * Np + (size_t)qt * 64) * D;
    const size_t tb = ((size_t)bh * nb + qt) * TB;
    stage_rows<D>(L, reinterpret_cast<const uint8_t*>(bp.q_codes) + rb, w, lane);
    stage_rows<D>(L + TB, bp.do_codes + rb, w, lane);
    stage_cols<D>(L + 2 * TB, bp.doT_codes + tb, w, lane);
    stage_cols<D>(L + 3 * TB, reinterpret_cast<const uint8_t*>(bp.qT_codes) + tb, w, lane);
    if (w == 0 && lane < 16) load_lds16(bp.lse2 + (size_t)bh * Np + qt * 64 + 4 * lane, L + 4 * TB + 16 * lane);
    if (w == 1 && lane < 16) load_lds16(bp.Dvec + (size_t)bh * Np + qt * 64 + 4 * lane, L + 4 * TB + 256 + 16 * lane);
  };
  if (qt0 < nqt) stage(0, qt0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int qt = qt0; qt < nqt; qt++) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) stage(buf ^ 1, qt + 1);
    const uint8_t* L = lds[buf];
    const int qb = qt * 64;
    // causal: this wave's keys all exceed the tile's queries -> nothing to add
    if (!(CAUSAL && kw > qb + 63) && kw < N) {
      const float qstep = bp.q_step[(size_t)bh * nb + qt];
      const float dostep = bp.do_step[(size_t)bh * nb + qt];
      // S = Q K^T and dP = dO V^T (rows: tile queries in tile_perm order, cols: the wave's keys)
      v16i S[2];
      v16f P[2];
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const int row = tile_perm(n, s);
        v16i a = v16i{};
#pragma unroll
        for (int c = 0; c < D / 32; c++)
          a = mfma_i8(*reinterpret_cast<const v4i*>(L + rowoff<D>(row, 2 * c + hh)), kf[c], a);
        S[s] = a;
        v16f b = v16f{};
#pragma unroll
        for (int c = 0; c < D / 64; c++) {
          const v4i x0 = *reinterpret_cast<const v4i*>(L + TB + rowoff<D>(row, 4 * c + 2 * hh));
          const v4i x1 = *reinterpret_cast<const v4i*>(L + TB + rowoff<D>(row, 4 * c + 2 * hh + 1));
          b = mfma_f8(v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}, vf[c], b);
        }
        P[s] = b;   // dP accumulator for now
      }
      // P, dS (element r of subtile s = query qb + 32 hh + 16 s + r, key = this lane's key)
      const float cS = qstep * kstep * smlog2e, cP = dostep * vstep;
      const float* l2 = reinterpret_cast<const float*>(L + 4 * TB) + 32 * hh;
      const float* Dv = reinterpret_cast<const float*>(L + 4 * TB + 256) + 32 * hh;
      float pf[32], ds[32];
      float amax = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const v4f lv = *reinterpret_cast<const v4f*>(l2 + 16 * s + r);
          const v4f dv = *reinterpret_cast<const v4f*>(Dv + 16 * s + r);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int q = qb + 32 * hh + 16 * s + r + i;
            const bool ok = key < N && (!CAUSAL || key <= q);
            const float p = ok ? fast_exp2(fmaf((float)S[s][r + i], cS, -lv[i])) : 0.0f;
            const float d = p * fmaf(P[s][r + i], cP, -dv[i]);
            pf[16 * s + r + i] = p;
            ds[16 * s + r + i] = d;
            amax = fmaxf(amax, fabsf(d));
          }
        }
      // dV^T += dO^T P~ (FP8, K = 64 queries)
      v8i pb;
#pragma unroll
      for (int i = 0; i < 32; i += 4)
        pb[i / 4] = pack_fp8x4(448.0f * pf[i], 448.0f * pf[i + 1], 448.0f * pf[i + 2], 448.0f * pf[i + 3]);
#pragma unroll
      for (int cb = 0; cb < NCB; cb++) {
        const int row = 32 * cb + n;
        const v4i x0 = *reinterpret_cast<const v4i*>(L + 2 * TB + coloff(row, 2 * hh));
        const v4i x1 = *reinterpret_cast<const v4i*>(L + 2 * TB + coloff(row, 2 * hh + 1));
        dV[cb] = mfma_f8(v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}, pb, dV[cb]);
      }
      // dS~ (INT8, one step per wave tile), dK^T += Q^T dS~ (INT8, K = 32 queries per subtile)
      const float am = wave_absmax(amax);
      const float step = am / 127.0f, inv = am == 0.0f ? 0.0f : 127.0f / am;
      const float kscale = step * qstep;
#pragma unroll
      for (int cb = 0; cb < NCB; cb++) {
        const int row = 32 * cb + n;
        v16i acc = v16i{};
#pragma unroll
        for (int s = 0; s < 2; s++) {
          v4i db;
#pragma unroll
          for (int k = 0; k < 4; k++)
            db[k] = pack_i8x4(q8(ds[16 * s + 4 * k], inv), q8(ds[16 * s + 4 * k + 1], inv), q8(ds[16 * s + 4 * k + 2], inv),
                              q8(ds[16 * s + 4 * k + 3], inv));
          acc = mfma_i8(*reinterpret_cast<const v4i*>(L + 3 * TB + coloff(row, 2 * hh + s)), db, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) dK[cb][r] = fmaf((float)acc[r], kscale, dK[cb][r]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  // epilogue: dK = sm dK^T, dV = dV^T * doT_step / 448; lane holds channels of its key
  if (key < N) {
    uint16_t* dkr = reinterpret_cast<uint16_t*>(dk) + ((size_t)bh * N + key) * D;
    uint16_t* dvr = reinterpret_cast<uint16_t*>(dv) + ((size_t)bh * N + key) * D;
    const float* dcs = bp.doT_step + (size_t)bh * D;
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * cb + 8 * g + 4 * hh;
        uint32_t k2[2], v2[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          k2[t] = (uint32_t)to_io<DT>(dK[cb][4 * g + 2 * t] * sm) | ((uint32_t)to_io<DT>(dK[cb][4 * g + 2 * t + 1] * sm) << 16);
          v2[t] = (uint32_t)to_io<DT>(dV[cb][4 * g + 2 * t] * (dcs[ch + 2 * t] * (1.0f / 448.0f))) |
                  ((uint32_t)to_io<DT>(dV[cb][4 * g + 2 * t + 1] * (dcs[ch + 2 * t + 1] * (1.0f / 448.0f))) << 16);
        }
        *reinterpret_cast<uint2*>(dkr + ch) = make_uint2(k2[0], k2[1]);
        *reinterpret_cast<uint2*>(dvr + ch) = make_uint2(v2[0], v2[1]);
      }
  }
}

// ---- query-stationary kernel: dQ ----
// Workgroup: 128 queries (4 waves x 32), loops over 64-key tiles.  LDS per stage:
// K_s rows (INT8), V rows (FP8), K_s^T (channel rows, INT8).
template <int D, bool CAUSAL, int DT>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdPtrs bp, void* dq, int N, int Np, float sm) {
  constexpr int TB = 64 * D;
  constexpr int STAGE = 3 * TB;
  constexpr int NCB = D / 32;
  __shared__ __align__(16) uint8_t lds[2][STAGE];
  const int nqt = Np / 128;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / nqt;
  const int qt = CAUSAL ? nqt - 1 - id % nqt : id % nqt;
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
    for (int c = 0; c < D / 64; c++) {
      const v4i a0 = *reinterpret_cast<const v4i*>(dp + 64 * c), a1 = *reinterpret_cast<const v4i*>(dp + 64 * c + 16);
      df[c] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
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
    stage_cols<D>(L + 2 * TB, reinterpret_cast<const uint8_t*>(bp.kT_codes) + tb, w, lane);
  };
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kt = 0; kt < nkt; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) stage(buf ^ 1, kt + 1);
    const uint8_t* L = lds[buf];
    const int kb = kt * 64;
    if (!(CAUSAL && kb > qw + 31)) {
      const float kstep = bp.k_step[(size_t)bh * nb + kt];
      const float vstep = bp.v_step[(size_t)bh * nb + kt];
      v16i S[2];
      v16f G[2];
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const int row = tile_perm(n, s);
        v16i a = v16i{};
#pragma unroll
        for (int c = 0; c < D / 32; c++)
          a = mfma_i8(*reinterpret_cast<const v4i*>(L + rowoff<D>(row, 2 * c + hh)), qf[c], a);
        S[s] = a;
        v16f b = v16f{};
#pragma unroll
        for (int c = 0; c < D / 64; c++) {
          const v4i x0 = *reinterpret_cast<const v4i*>(L + TB + rowoff<D>(row, 4 * c + 2 * hh));
          const v4i x1 = *reinterpret_cast<const v4i*>(L + TB + rowoff<D>(row, 4 * c + 2 * hh + 1));
          b = mfma_f8(v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}, df[c], b);
        }
        G[s] = b;
      }
      const float cS = qstep * kstep * smlog2e, cP = dostep * vstep;
      float ds[32];
      int pc[32];
      float amax = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int k = kb + 32 * hh + 16 * s + r;
          const bool ok = k < N && (!CAUSAL || k <= q);
          const float p = ok ? fast_exp2(fmaf((float)S[s][r], cS, -l2)) : 0.0f;
          const float d = p * fmaf(G[s][r], cP, -Dq);
          ds[16 * s + r] = d;
          pc[16 * s + r] = (int)rintf(p * 127.0f);   // P in [0, 1] as INT8 codes of step 1/127
          rsum += d;
          amax = fmaxf(amax, fabsf(d));
        }
      const float am = wave_absmax(amax);
      const float step = am / 127.0f, inv = am == 0.0f ? 0.0f : 127.0f / am;
      const float qscale = step * kstep;
#pragma unroll
      for (int cb = 0; cb < NCB; cb++) {
        const int row = 32 * cb + n;
        v16i acc = v16i{};
#pragma unroll
        for (int s = 0; s < 2; s++) {
          v4i db;
#pragma unroll
          for (int k = 0; k < 4; k++)
            db[k] = pack_i8x4(q8(ds[16 * s + 4 * k], inv), q8(ds[16 * s + 4 * k + 1], inv), q8(ds[16 * s + 4 * k + 2], inv),
                              q8(ds[16 * s + 4 * k + 3], inv));
          acc = mfma_i8(*reinterpret_cast<const v4i*>(L + 2 * TB + coloff(row, 2 * hh + s)), db, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) dQ[cb][r] = fmaf((float)acc[r], qscale, dQ[cb][r]);
        // P K_s for the rowsum correction
        v16i accp = v16i{};
#pragma unroll
        for (int s = 0; s < 2; s++) {
          v4i pb;
#pragma unroll
          for (int k = 0; k < 4; k++)
            pb[k] = pack_i8x4(pc[16 * s + 4 * k], pc[16 * s + 4 * k + 1], pc[16 * s + 4 * k + 2], pc[16 * s + 4 * k + 3]);
          accp = mfma_i8(*reinterpret_cast<const v4i*>(L + 2 * TB + coloff(row, 2 * hh + s)), pb, accp);
        }
        const float pscale = kstep * (1.0f / 127.0f);
#pragma unroll
        for (int r = 0; r < 16; r++) PK[cb][r] = fmaf((float)accp[r], pscale, PK[cb][r]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  // epilogue: dQ = sm (dS K_s - rowsum(dS) P K_s); hand D^ = D + rowsum(dS) to the dK/dV kernel
  const float rs = half_sum(rsum);
  if (q < N) {
    uint16_t* dqr = reinterpret_cast<uint16_t*>(dq) + ((size_t)bh * N + q) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * cb + 8 * g + 4 * hh;
        uint32_t w2[2];
#pragma unroll
        for (int t = 0; t < 2; t++)
          w2[t] = (uint32_t)to_io<DT>(sm * fmaf(-rs, PK[cb][4 * g + 2 * t], dQ[cb][4 * g + 2 * t])) |
                  ((uint32_t)to_io<DT>(sm * fmaf(-rs, PK[cb][4 * g + 2 * t + 1], dQ[cb][4 * g + 2 * t + 1])) << 16);
        *reinterpret_cast<uint2*>(dqr + ch) = make_uint2(w2[0], w2[1]);
      }
    if (hh == 0) bp.Dvec[(size_t)bh * Np + q] = Dq + rs;
  }
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct BwdLayout {
  size_t amax_do, Dvec, lse2, do_codes, do_step, doT_codes, doT_step, v_codes, v_step, qT, kT, total;
};

BwdLayout bwd_layout(const Shape& s) {
  const size_t BH = (size_t)s.B * s.H, d = s.d, Np = s.Np, nb = Np / 64;
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off = round256(off + b); return o; };
  L.amax_do = take(BH * d * 4);
  L.Dvec = take(BH * Np * 4);
  L.lse2 = take(BH * Np * 4);
  L.do_codes = take(BH * Np * d);
  L.do_step = take(BH * nb * 4);
  L.doT_codes = take(BH * Np * d);
  L.doT_step = take(BH * d * 4);
  L.v_codes = take(BH * Np * d);
  L.v_step = take(BH * nb * 4);
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
  bp.amax_do = reinterpret_cast<uint32_t*>(b + L.amax_do);
  bp.Dvec = reinterpret_cast<float*>(b + L.Dvec);
  bp.lse2 = reinterpret_cast<float*>(b + L.lse2);
  bp.do_codes = b + L.do_codes;
  bp.do_step = reinterpret_cast<float*>(b + L.do_step);
  bp.doT_codes = b + L.doT_codes;
  bp.doT_step = reinterpret_cast<float*>(b + L.doT_step);
  bp.v_codes = b + L.v_codes;
  bp.v_step = reinterpret_cast<float*>(b + L.v_step);
  bp.qT_codes = reinterpret_cast<int8_t*>(b + L.qT);
  bp.kT_codes = reinterpret_cast<int8_t*>(b + L.kT);
  // forward quantization of Q, K (the codes the forward used), then the backward prologue
  hipError_t e = launch_prologue(q, k, v, s, qp, st);
  if (e != hipSuccess) return e;
  bwd_zero_kernel<<<(BH * D + 255) / 256, 256, 0, st>>>(bp.amax_do, BH * D);
  bwd_stats_kernel<DT, D><<<dim3((s.N + 255) / 256, BH), 256, 0, st>>>((const uint16_t*)dout, s.N, bp.amax_do);
  bwd_prep_kernel<DT, D><<<dim3(s.Np / 64, BH), 256, 0, st>>>((const uint16_t*)o, (const uint16_t*)dout,
                                                             (const uint16_t*)v, lse, s.N, s.Np, bp);
  const int grid = BH * (s.Np / 128);
  // dQ first: it turns D into D^ = D + rowsum(dS), which the dK/dV kernel then uses
  if (s.causal) {
    bwd_dq_kernel<D, true, DT><<<grid, 256, 0, st>>>(bp, dq, s.N, s.Np, s.sm_scale);
    bwd_dkdv_kernel<D, true, DT><<<grid, 256, 0, st>>>(bp, dk, dv, s.N, s.Np, s.sm_scale);
  } else {
    bwd_dq_kernel<D, false, DT><<<grid, 256, 0, st>>>(bp, dq, s.N, s.Np, s.sm_scale);
    bwd_dkdv_kernel<D, false, DT><<<grid, 256, 0, st>>>(bp, dk, dv, s.N, s.Np, s.sm_scale);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_ws_bytes(const Shape& s) { return bwd_layout(s).total; }

hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, void* ws,
                           size_t qbytes, const QuantPtrs& qp, hipStream_t stream) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (s.d != 64) return hipErrorNotSupported;
  return s.io_dtype == 0 ? bwd_run<0, 64>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream)
                         : bwd_run<1, 64>(s, q, k, v, o, dout, lse, dq, dk, dv, w, qbytes, qp, stream);
}

}  // namespace sage
