// attn_fwd.hip -- fused quantized attention forward for gfx950.
//
// FlashAttention-style: one workgroup owns a 128-query tile of one (b,h) head
// and streams 64-key tiles of K and V codes through LDS; per tile it forms the
// score tile with MFMA, applies the online-softmax update (running max m and
// row sum l, rescale of the running output by exp(m_old - m_new)), quantizes
// P to FP8 and accumulates P~V with MFMA; normalisation by l happens once,
// after the last tile (SageAttention review thread: online softmax, reply to
// reviewer xY6z Q3; deferred normalisation, reply to Q2).  QK^T runs on INT8
// (SageAttention contributions, reply to reviewer wwcu W1) or on microscaled
// FP4 (SageAttention3 abstract); P~ and V are FP8 (SageAttention2 abstract).
//
// Dequantization is folded into the softmax: t = S_int * (dQ_row * dK_tile *
// sm * log2 e) for INT8, t = (S + dS_key) * sm * log2 e for MXFP4, and
// p~ = E4M3(exp2(t - m + log2 448)) = E4M3(448 p).  l accumulates the
// unquantized 448 p and the epilogue divides by it and multiplies by the
// per-channel V step.
//
// Two-level P~V accumulation (SageAttention2 abstract): the pages accumulate
// each tile's P~V in the matrix unit and add it to an fp32 running output.  On
// gfx950 the FP8 MFMA rounds only inside each group of 8 products and adds the
// group sums into its fp32 C operand at full fp32 precision, so the running O
// is kept directly as the MFMA accumulator (rescaled by alpha before each tile):
// the second level is the accumulator itself.
//
// Layout per wave (4 waves, 32 queries each).  The QK MFMA computes
// S^T = K Q^T: A rows are keys, B columns are the wave's 32 queries, so lane l
// owns query l%32 and, across the two 32-key subtiles, the 32 keys
// 32*(l/32) + [0, 32) of the 64-key tile (A rows are fed in the permuted key
// order pi_s(m) that makes this true).  Row max and row sum are therefore
// in-lane plus one exchange between wave halves, and the lane's 32 P~ bytes
// are already the B operand of the PV MFMA O^T = V^T P~^T (A = V^T, rows =
// channels, K = the same 32 keys).
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

struct FwdArgs {
  const uint8_t* q_codes;
  const void* q_scales;
  const uint8_t* k_codes;
  const void* k_scales;
  const float* delta_s;
  const uint8_t* v_codes;
  const float* v_scales;
  const float* lse_corr;
  void* o;
  float* lse;
  int N, Np;
  float sm_log2e;
};

constexpr int kTK = 64;      // keys per tile (= the INT8 K block)
constexpr int kQT = 128;     // queries per workgroup

template <int D, int QK>
struct TileGeom {
  static constexpr int KROW = QK == QK_INT8 ? D : D / 2;   // bytes per key row
  static constexpr int KCH = KROW / 16;                      // 16-byte chunks per key row
  static constexpr int KBYTES = kTK * KROW;
  static constexpr int SBYTES = QK == QK_MXFP4 ? kTK * (D / 32) : 0;   // E8M0 bytes per tile
  static constexpr int DSBYTES = QK == QK_MXFP4 ? kTK * 4 : 0;         // dS floats per tile
  static constexpr int VBYTES = D * kTK;                               // FP8 V^T tile
  static constexpr int STAGE = KBYTES + SBYTES + DSBYTES + VBYTES;
  static constexpr int KLOADS = (KBYTES / 16 + 255) / 256;
  static constexpr int VLOADS = VBYTES / 16 / 256;
};

// Key row fed to A-row m of subtile s, so that output lane half h holds keys 32h + 16s + r.
__device__ __forceinline__ int key_perm(int m, int s) { return 32 * ((m >> 2) & 1) + 16 * s + 4 * (m >> 3) + (m & 3); }

template <int D, int QK>
struct Stage {
  using G = TileGeom<D, QK>;
  uint4 k[G::KLOADS];
  uint4 v[G::VLOADS];
  uint4 sd;   // MXFP4: scales (threads 0..15) or dS (threads 16..31)

  __device__ __forceinline__ void load(const FwdArgs& a, int bh, int j) {
    const int tid = threadIdx.x;
    const uint8_t* kg = a.k_codes + ((size_t)bh * a.Np + (size_t)j * kTK) * G::KROW;
#pragma unroll
    for (int i = 0; i < G::KLOADS; i++) {
      int c = tid + 256 * i;
      if (c < G::KBYTES / 16) k[i] = reinterpret_cast<const uint4*>(kg)[c];
    }
    const uint8_t* vg = a.v_codes + ((size_t)bh * (a.Np / kTK) + j) * G::VBYTES;
#pragma unroll
    for (int i = 0; i < G::VLOADS; i++) v[i] = reinterpret_cast<const uint4*>(vg)[tid + 256 * i];
    if (QK == QK_MXFP4) {
      if (tid < G::SBYTES / 16) {
        const uint8_t* sg = reinterpret_cast<const uint8_t*>(a.k_scales) + ((size_t)bh * a.Np + (size_t)j * kTK) * (D / 32);
        sd = reinterpret_cast<const uint4*>(sg)[tid];
      } else if (tid >= 64 && tid < 64 + G::DSBYTES / 16) {
        const float* dg = a.delta_s + (size_t)bh * a.Np + (size_t)j * kTK;
        sd = reinterpret_cast<const uint4*>(dg)[tid - 64];
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::KLOADS; i++) {
      int c = tid + 256 * i;
      if (c < G::KBYTES / 16) {
        int row = c / G::KCH, col = c % G::KCH;
        *reinterpret_cast<uint4*>(lds + row * G::KROW + ((col ^ (row & (G::KCH - 1))) << 4)) = k[i];
      }
    }
    uint8_t* lv = lds + G::KBYTES + G::SBYTES + G::DSBYTES;
#pragma unroll
    for (int i = 0; i < G::VLOADS; i++) {
      int c = tid + 256 * i;
      int row = c >> 2, col = c & 3;
      *reinterpret_cast<uint4*>(lv + row * 64 + ((col ^ (row & 3)) << 4)) = v[i];
    }
    if (QK == QK_MXFP4) {
      if (tid < G::SBYTES / 16)
        reinterpret_cast<uint4*>(lds + G::KBYTES)[tid] = sd;
      else if (tid >= 64 && tid < 64 + G::DSBYTES / 16)
        reinterpret_cast<uint4*>(lds + G::KBYTES + G::SBYTES)[tid - 64] = sd;
    }
  }
};

template <int D, int QK, bool CAUSAL, int DT>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  using G = TileGeom<D, QK>;
  constexpr int NCB = D / 32;                          // 32-channel output blocks
  constexpr int NQF = QK == QK_INT8 ? D / 32 : D / 64; // QK MFMAs per 32-key subtile
  __shared__ __align__(16) uint8_t smem[2][G::STAGE];

  const int nqt = a.Np / kQT;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / nqt;
  const int qt = CAUSAL ? nqt - 1 - id % nqt : id % nqt;   // causal: longest rows first
  const int qbase = qt * kQT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int qw = qbase + 32 * w;          // first query of this wave
  const int qrow = qw + n;                // this lane's query

  // Q fragments (B operand), resident for the whole loop
  v4i qf[QK == QK_INT8 ? NQF : 1];
  v8i qf4[QK == QK_MXFP4 ? NQF : 1];
  int qsc[QK == QK_MXFP4 ? NQF : 1];
  float qstep = 0.0f;
  if (QK == QK_INT8) {
    const uint8_t* qp = a.q_codes + ((size_t)bh * a.Np + qrow) * D + 16 * hh;
#pragma unroll
    for (int c = 0; c < NQF; c++) qf[c] = *reinterpret_cast<const v4i*>(qp + 32 * c);
    qstep = reinterpret_cast<const float*>(a.q_scales)[(size_t)bh * (a.Np / kTK) + qrow / kTK] * a.sm_log2e;
  } else {
    const uint8_t* qp = a.q_codes + ((size_t)bh * a.Np + qrow) * (D / 2) + 16 * hh;
    const uint8_t* qe = reinterpret_cast<const uint8_t*>(a.q_scales) + ((size_t)bh * a.Np + qrow) * (D / 32) + hh;
#pragma unroll
    for (int c = 0; c < NQF; c++) {
      v4i lo = *reinterpret_cast<const v4i*>(qp + 32 * c);
      qf4[c] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      qsc[c] = qe[2 * c];
    }
  }
  const float* kstep = reinterpret_cast<const float*>(a.k_scales) + (size_t)bh * (a.Np / kTK);

  int ntiles = (a.N + kTK - 1) / kTK;
  if (CAUSAL) ntiles = min(ntiles, (qbase + kQT - 1) / kTK + 1);

  v16f O[NCB];
#pragma unroll
  for (int c = 0; c < NCB; c++) O[c] = v16f{};
  float m = -INFINITY, l = 0.0f;

  Stage<D, QK> st;
  st.load(a, bh, 0);
  st.store(smem[0]);
  __syncthreads();

  for (int j = 0; j < ntiles; j++) {
    const bool more = j + 1 < ntiles;
    if (more) st.load(a, bh, j + 1);
    const uint8_t* lds = smem[j & 1];
    const int kbase = j * kTK;
    // waves whose queries all precede this tile have nothing to do here
    if (!(CAUSAL && kbase > qw + 31)) {
      // ---- S^T = K Q^T for two 32-key subtiles ----
      float t[32];
      if (QK == QK_INT8) {
        v16i S[2] = {v16i{}, v16i{}};
#pragma unroll
        for (int s = 0; s < 2; s++) {
          const int row = key_perm(n, s);
#pragma unroll
          for (int c = 0; c < NQF; c++) {
            const int col = 2 * c + hh;
            v4i ka = *reinterpret_cast<const v4i*>(lds + row * G::KROW + ((col ^ (row & (G::KCH - 1))) << 4));
            S[s] = mfma_i8(ka, qf[c], S[s]);
          }
        }
        const float cst = qstep * kstep[j];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
          for (int r = 0; r < 16; r++) t[16 * s + r] = (float)S[s][r] * cst;
      } else {
        v16f S[2] = {v16f{}, v16f{}};
        const uint8_t* lsc = lds + G::KBYTES;
#pragma unroll
        for (int s = 0; s < 2; s++) {
          const int row = key_perm(n, s);
#pragma unroll
          for (int c = 0; c < NQF; c++) {
            const int col = 2 * c + hh;
            v4i lo = *reinterpret_cast<const v4i*>(lds + row * G::KROW + ((col ^ (row & (G::KCH - 1))) << 4));
            v8i ka = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
            const int ksc = lsc[row * (D / 32) + col];
            S[s] = mfma_mxfp4(ka, qf4[c], S[s], ksc, qsc[c]);
          }
        }
        const float* lds_ds = reinterpret_cast<const float*>(lds + G::KBYTES + G::SBYTES) + 32 * hh;
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            v4f dsv = *reinterpret_cast<const v4f*>(lds_ds + 16 * s + r);
#pragma unroll
            for (int i = 0; i < 4; i++) t[16 * s + r + i] = (S[s][r + i] + dsv[i]) * a.sm_log2e;
          }
      }
      // ---- masking (tail tile, causal diagonal) ----
      const bool need_mask = kbase + kTK > a.N || (CAUSAL && kbase + kTK - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
          const int key = kbase + 32 * hh + i;
          if (key >= a.N || (CAUSAL && key > qrow)) t[i] = -INFINITY;
        }
      }
      // ---- online softmax ----
      float mt = t[0];
#pragma unroll
      for (int i = 1; i < 32; i++) mt = fmaxf(mt, t[i]);
      mt = half_max(mt);
      const float mnew = fmaxf(m, mt);
      const float mref = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = fast_exp2(m - mref);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < NCB; c++) O[c] *= alpha;
      const float off = kLog2_448 - mref;
      v8i pb;
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float p0 = fast_exp2(t[i] + off), p1 = fast_exp2(t[i + 1] + off);
        const float p2 = fast_exp2(t[i + 2] + off), p3 = fast_exp2(t[i + 3] + off);
        ps += (p0 + p1) + (p2 + p3);
        pb[i / 4] = pack_fp8x4(p0, p1, p2, p3);
      }
      l += ps;
      m = mnew;
      // ---- O^T += V^T P~^T ----
      const uint8_t* lv = lds + G::KBYTES + G::SBYTES + G::DSBYTES;
#pragma unroll
      for (int c = 0; c < NCB; c++) {
        const int row = 32 * c + n;
        const uint8_t* rp = lv + row * 64;
        v4i v0 = *reinterpret_cast<const v4i*>(rp + (((2 * hh) ^ (row & 3)) << 4));
        v4i v1 = *reinterpret_cast<const v4i*>(rp + (((2 * hh + 1) ^ (row & 3)) << 4));
        v8i va = v8i{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        O[c] = mfma_f8(va, pb, O[c]);
      }
    }
    if (more) st.store(smem[(j + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: O / l * dV, LSE ----
  const float lt = half_sum(l);
  if (qrow < a.N) {
    const float inv = 1.0f / lt;
    const float* vs = a.v_scales + (size_t)bh * D;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + ((size_t)bh * a.N + qrow) * D;
#pragma unroll
    for (int c = 0; c < NCB; c++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * c + 8 * g + 4 * hh;
        v4f sc = *reinterpret_cast<const v4f*>(vs + ch);
        uint32_t lo = (uint32_t)to_io<DT>(O[c][4 * g] * sc[0] * inv) | ((uint32_t)to_io<DT>(O[c][4 * g + 1] * sc[1] * inv) << 16);
        uint32_t hi = (uint32_t)to_io<DT>(O[c][4 * g + 2] * sc[2] * inv) | ((uint32_t)to_io<DT>(O[c][4 * g + 3] * sc[3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + ch) = make_uint2(lo, hi);
      }
    if (a.lse && hh == 0)
      a.lse[(size_t)bh * a.N + qrow] = (m + __log2f(lt) - kLog2_448) * kLn2 + a.lse_corr[(size_t)bh * a.N + qrow];
  }
}

template <int D, int QK, int DT>
static hipError_t fwd_dispatch(const Shape& s, const FwdArgs& a, hipStream_t st) {
  const int grid = s.B * s.H * (s.Np / kQT);
  if (s.causal)
    attn_fwd_kernel<D, QK, true, DT><<<grid, 256, 0, st>>>(a);
  else
    attn_fwd_kernel<D, QK, false, DT><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int QK, int DT>
static hipError_t fwd_dispatch_d(const Shape& s, const FwdArgs& a, hipStream_t st) {
  return s.d == 64 ? fwd_dispatch<64, QK, DT>(s, a, st) : fwd_dispatch<128, QK, DT>(s, a, st);
}

hipError_t launch_attn_fwd(const Shape& s, const QuantPtrs& qp, void* o, float* lse, hipStream_t st) {
  FwdArgs a;
  a.q_codes = qp.q_codes;
  a.q_scales = qp.q_scales;
  a.k_codes = qp.k_codes;
  a.k_scales = qp.k_scales;
  a.delta_s = qp.delta_s;
  a.v_codes = qp.v_codes;
  a.v_scales = reinterpret_cast<const float*>(qp.v_scales);
  a.lse_corr = qp.lse_corr;
  a.o = o;
  a.lse = lse;
  a.N = s.N;
  a.Np = s.Np;
  a.sm_log2e = s.sm_scale * kLog2e;
  if (s.pv_fmt != PV_FP8) return hipErrorInvalidValue;   // MXFP4 P~V: not in this kernel
  if (s.qk_fmt == QK_INT8)
    return s.io_dtype == 0 ? fwd_dispatch_d<QK_INT8, 0>(s, a, st) : fwd_dispatch_d<QK_INT8, 1>(s, a, st);
  return s.io_dtype == 0 ? fwd_dispatch_d<QK_MXFP4, 0>(s, a, st) : fwd_dispatch_d<QK_MXFP4, 1>(s, a, st);
}

}  // namespace sage
