// attn_fwd.hip -- fused quantized attention forward for gfx950.
//
// FlashAttention-style: a workgroup owns a 128-query tile of one (b,h) head and
// streams 64-key tiles of K and V codes through LDS; per tile it forms the
// score tile with MFMA, applies the online-softmax update (running max m and
// row sum l, rescale of the running output by exp(m_old - m_new)), quantizes
// P to FP8 and accumulates P~V with MFMA; normalisation by l happens once,
// after the last tile (SageAttention review thread: online softmax, reply to
// reviewer xY6z Q3; deferred normalisation, reply to Q2).  QK^T runs on INT8
// (SageAttention contributions, reply to reviewer wwcu W1) or on microscaled
// FP4 (SageAttention3 abstract); P~ and V are FP8 (SageAttention2 abstract).
//
// Dequantization is folded into the softmax: t = S_int * (dQ_row * dK_tile *
// sm * log2 e) for INT8, t = (S + dS_key) * sm * log2 e for MXFP4 (dS enters as
// the QK MFMA's initial accumulator in the one-buffer kernels), and
// p~ = E4M3(exp2(t - m + log2 448)) = E4M3(448 p).  l accumulates the
// unquantized 448 p; the epilogue divides by it and applies the per-channel V
// step.
//
// Two-level P~V accumulation (SageAttention2 abstract): the pages accumulate
// each tile's P~V in the matrix unit and add it to an fp32 running output.  On
// gfx950 the FP8 MFMA rounds only inside each group of 8 products and adds the
// group sums into its fp32 C operand at full fp32 precision, so the running O
// is kept directly as the MFMA accumulator (rescaled by alpha before a tile's
// product is added): the second level is the accumulator itself.
//
// Layout per wave (4 waves, 32 queries each).  The QK MFMA computes
// S^T = K Q^T: A rows are keys, B columns are the wave's 32 queries, so lane l
// owns query l%32 and, across the two 32-key subtiles, the 32 keys
// 32*(l/32) + [0, 32) of the 64-key tile (A rows are fed in the permuted key
// order key_perm(m, s) that makes this true).  Row max and row sum are
// in-lane plus one exchange between wave halves, and the lane's 32 P~ bytes
// are already the B operand of the PV MFMA O^T = V^T P~^T (A = V^T, rows =
// channels, K = the same 32 keys).
//
// Pipeline, one barrier per tile.  At d = 128 (kOneBuf: every pair but fp16 P~V) a wave
// holds one score tile: tile j issues its own QK MFMAs, with K and V loaded one tile ahead
// into two LDS buffers, and the registers saved fit three workgroups per CU, so other waves
// fill the matrix and vector units while one waits.  The others (d = 64, fp16 P~V; two
// workgroups per CU) hold two: the QK MFMAs of tile j+1 overlap the softmax of tile j
// (issued before it, or spread through its exp / pack stream where that measured faster),
// with K one tile ahead of V.
// Causal: one query tile per workgroup, longest first (see attn_fwd_kernel).
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
  SeqGeo g;
  int nqt;            // query tiles per instance in the grid
  int qbs;            // MXFP4 with per-block Q smoothing: keys per dS strip (one strip per query tile,
                      // at qblock_slot); else 0
  float sm_log2e;
};

#ifndef MFMA_IL_D128
#define MFMA_IL_D128 0
#endif
#ifndef FWD_ONEBUF_D128
#define FWD_ONEBUF_D128 1
#endif
// One score buffer per wave (QK(j) issued in tile j itself), which frees the registers of the
// second buffer so that three workgroups (three waves per SIMD) fit on a CU: at head dim 128 with
// INT8 QK and FP8 P~V the kernel is bound by vector issue, and a lone wave issues vector work at
// half the SIMD's rate, so a third wave that keeps two of them ready pays more than the overlap
// of the next tile's QK products inside one wave.  Measured: N = 8192 non-causal 712 -> 666 us,
// the causal 4096-token prefill 110 -> 102 us; MXFP4 QK and P~V at N = 8192 2724 -> 2629 us.
// (fp16 P~V keeps two buffers: its 16-bit P~ operands do not fit three waves.)
template <int D, int QK, int PV>
constexpr bool kOneBuf = FWD_ONEBUF_D128 && D == 128 &&
                         ((QK == QK_INT8 && PV == PV_FP8) ||
                          (QK == QK_MXFP4 && (PV == PV_FP8 || PV == PV_MXFP8 || PV == PV_MXFP4)));
// MXFP4 QK in the one-buffer kernels: the per-key smoothing term dS is the initial accumulator
// of the QK products (S^T = dS + K Q^T: the C operand of the first MFMA holds each output row's
// dS), so a score takes one FMA (p = exp2(S' sm log2 e + off)) instead of two, and the row max
// is taken on S' before scaling.  The only new rounding, of S + dS in the matrix core's fp32
// accumulation, is bounded by 2^-24 (|S| + |dS|), which the P~ decision's admissible window
// covers sixteen times over.  (The two-buffer kernels issue QK(j+1) before tile j+1's dS is in
// LDS, so they keep the FMA.)
template <int D, int QK, int PV>
constexpr bool kDsAcc = QK == QK_MXFP4 && kOneBuf<D, QK, PV>;
constexpr int kTK = 64;      // keys per tile (= the INT8 K block)
constexpr int kQT = 128;     // queries per workgroup pass

template <int D, int QK, int PV = PV_FP8>
struct Geo {
  static constexpr int KROW = QK == QK_INT8 ? D : D / 2;               // bytes per key row
  static constexpr int KCH = KROW / 16;                                 // 16-byte chunks per key row
  static constexpr int KBYTES = kTK * KROW;
  static constexpr int SBYTES = QK == QK_MXFP4 ? kTK * (D / 32) : 0;    // E8M0 bytes per tile
  static constexpr int DSBYTES = QK == QK_MXFP4 ? kTK * 4 : 0;          // scaled dS floats per tile
  static constexpr int KSTAGE = KBYTES + SBYTES;
  // V^T tile: FP8 / MXFP8 (64 bytes per channel), MXFP4 (32 bytes per channel) or fp16 (128
  // bytes per channel); the MX formats then carry one E8M0 byte per channel for each of the
  // two 32-key groups
  static constexpr int VBYTES = PV == PV_MXFP4 ? D * kTK / 2 : PV == PV_F16 ? D * kTK * 2 : D * kTK;
  static constexpr int VSB = PV == PV_MXFP4 || PV == PV_MXFP8 ? 2 * D : 0;
  static constexpr int VOPS = PV == PV_F16 ? 4 : 2;                    // V operand reads per block
  static constexpr int PVM = PV == PV_F16 ? 4 : 1;                     // PV MFMAs per block and tile
  // log2 of the static P~ scale folded into exp2: 448 fills E4M3; fp16 takes p itself
  static constexpr float PLOG2 = PV == PV_F16 ? 0.0f : kLog2_448;
  static constexpr int DSOFF = VBYTES + VSB;                            // scaled dS after V
  static constexpr int VSTAGE = DSOFF + DSBYTES;
  static constexpr int KCHUNKS = KBYTES / 16;                           // 16-byte chunks per K tile
  static constexpr int VCHUNKS = VBYTES / 16;                           // 16-byte chunks per V^T tile
  template <int NT> static constexpr int kloads() { return (KCHUNKS + NT - 1) / NT; }   // per lane, NT threads
  template <int NT> static constexpr int vloads() { return (VCHUNKS + NT - 1) / NT; }
  static constexpr int NCB = D / 32;                                    // 32-channel output blocks
  static constexpr int NQF = QK == QK_INT8 ? D / 32 : D / 64;           // QK MFMAs per 32-key subtile
};

// Which keys of a 64-key tile a lane's scores hold: lane half h, subtile s, register r holds
// key KH h + KS s + r.  The default gives each half 32 consecutive keys.  MXFP8 V needs the
// scaled FP8 MFMA's two 32-element K blocks (bytes [0, 16) and [16, 32) of both halves) to
// be the tile's two 32-token scale groups, so there subtile s carries keys [32 s, 32 s + 32).
template <int PV> struct KeyMap {
  static constexpr int KH = PV == PV_MXFP8 ? 16 : 32;
  static constexpr int KS = PV == PV_MXFP8 ? 32 : 16;
  // key in-lane score i (= 16 s + r) of half h
  static constexpr int lane_key(int i) { return (i / 16) * KS + (i % 16); }
};
// Key row fed to A-row m of subtile s: the output row of register r in half h is
// 8 (r / 4) + 4 h + r % 4, so this puts key KH h + KS s + r there.
template <int PV>
__device__ __forceinline__ int key_perm(int m, int s) {
  return KeyMap<PV>::KH * ((m >> 2) & 1) + KeyMap<PV>::KS * s + 4 * (m >> 3) + (m & 3);
}

// LDS swizzles: the 16-byte chunk c of row r is stored at chunk c ^ swz(r).  One ds_read_b128
// serves 16 lanes per LDS cycle; with 64 banks of 4 bytes a chunk's bank group is fixed by
// (row bits below the 256-byte period, chunk).  The K operand read by lanes 0-15 touches rows
// {0..3, 32..35, 4..7, 36..39} (+8, +16, ... for the other lane groups and subtiles); the V^T
// read touches 16 consecutive rows.  Each swizzle makes those 16 bank groups distinct.
template <int ROWBYTES>
__device__ __forceinline__ int swz(int r) {
  if (ROWBYTES == 128) return ((r >> 1) & 3) | (((r >> 5) & 1) << 2);   // 8 chunks, bank period 2 rows
  if (ROWBYTES == 64) return ((r >> 2) & 1) | (((r >> 5) & 1) << 1);    // 4 chunks, period 4 rows
  return (r >> 5) & 1;                                                   // 32-byte rows, 2 chunks
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 2) & 3; }     // V^T rows of 64 bytes
__device__ __forceinline__ int swz_v4(int r) { return (r >> 3) & 1; }    // MXFP4 V^T rows of 32 bytes
__device__ __forceinline__ int swz_v16(int r) { return (r >> 1) & 7; }   // fp16 V^T rows of 128 bytes

template <int DT>
__device__ __forceinline__ uint32_t pack2_io(float a, float b) {
  if (DT == 0) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    bf2 r = __builtin_convertvector(f2{a, b}, bf2);
    return __builtin_bit_cast(uint32_t, r);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    h2 r = __builtin_convertvector(f2{a, b}, h2);
    return __builtin_bit_cast(uint32_t, r);
  }
}

// ---- K / V tile staging: direct global -> LDS loads (no staging registers) ----
// A wave's 16-byte direct load puts lane L's data at LDS base + 16 L, so the XOR
// swizzle of the 16-byte chunks within a row (which spreads the MFMA operand reads
// over all LDS banks) is applied to the global source address instead.
// K stage: codes (+ E8M0 scales).  V stage: V^T codes (+ dS * sm * log2 e, staged through
// registers because it is rescaled on the way), read one step later than K.
// Per-lane byte offsets, computed once per query-tile pass and pinned in registers (the
// tile base addresses are wave-uniform, so every access is uniform base + lane offset).
template <int D, int QK, int NT = 256, int PV = PV_FP8>
struct LaneOffs {
  using G = Geo<D, QK, PV>;
  static constexpr int NTHREADS = NT;
  static constexpr int KL = G::template kloads<NT>(), VL = G::template vloads<NT>();
  uint32_t kld[KL];                 // direct-load source offsets inside a K tile
  uint32_t vld[VL];                 // direct-load source offsets inside a V^T tile
  // Subtile 1's K rows are subtile 0's plus KS (16 rows, except MXFP8 V), and V^T block c's rows
  // are block 0's plus 32 c; the swizzles below do not depend on those row bits, so the later
  // offsets are the first ones plus a constant (an immediate of the LDS read), and only the
  // first ones occupy registers.
  static constexpr bool KOP_IMM = KeyMap<PV>::KS == 16;
  static constexpr int VROWB = PV == PV_MXFP4 ? 32 : PV == PV_F16 ? 128 : 64;   // bytes per V^T row
  uint32_t kop[KOP_IMM ? 1 : 2][G::NQF];   // LDS offsets of the K operand reads (subtile, chunk)
  uint32_t ksc[G::NQF];             // MXFP4: LDS offsets of the K scale bytes (subtile 0)
  uint32_t vop[G::VOPS];            // LDS offsets of the V^T operand reads of block 0: FP8 / MXFP8 /
                                    // fp16 (16-byte chunk); MXFP4 ({codes, scale byte})
  uint32_t vsc;                     // MXFP8: LDS offset of block 0's E8M0 byte (+32 per block)

  __device__ __forceinline__ uint32_t kop_at(int s, int c) const {
    return KOP_IMM ? kop[0][c] + s * KeyMap<PV>::KS * G::KROW : kop[KOP_IMM ? 0 : s][c];
  }
  __device__ __forceinline__ uint32_t ksc_at(int s, int c) const { return ksc[c] + s * KeyMap<PV>::KS * (D / 32); }
  // block c, read t: MXFP4's scale byte (t = 1) advances 32 bytes per block
  __device__ __forceinline__ uint32_t vop_at(int c, int t) const {
    return vop[t] + c * (PV == PV_MXFP4 && t == 1 ? 32 : 32 * VROWB);
  }

  __device__ __forceinline__ void init(int w, int lane, int n, int hh) {
#pragma unroll
    for (int i = 0; i < KL; i++) {
      const int P = (NT * i + 64 * w + lane) % G::KCHUNKS;
      const int row = P / G::KCH, col = (P % G::KCH) ^ swz<G::KROW>(row);
      kld[i] = row * G::KROW + col * 16;
    }
#pragma unroll
    for (int i = 0; i < VL; i++) {
      const int P = (NT * i + 64 * w + lane) % G::VCHUNKS;
      if (PV == PV_MXFP4) {
        const int row = P >> 1, col = (P & 1) ^ swz_v4(row);
        vld[i] = row * 32 + col * 16;
      } else if (PV == PV_F16) {
        const int row = P >> 3, col = (P & 7) ^ swz_v16(row);
        vld[i] = row * 128 + col * 16;
      } else {
        const int row = P >> 2, col = (P & 3) ^ swz_v(row);
        vld[i] = row * 64 + col * 16;
      }
    }
#pragma unroll
    for (int s = 0; s < (KOP_IMM ? 1 : 2); s++) {
      const int row = key_perm<PV>(n, s);
#pragma unroll
      for (int c = 0; c < G::NQF; c++) {
        const int col = 2 * c + hh;
        kop[s][c] = row * G::KROW + ((col ^ swz<G::KROW>(row)) << 4);
        if (s == 0) ksc[c] = G::KBYTES + row * (D / 32) + col;
      }
    }
    {
      const int row = n;   // V^T block 0
      if (PV == PV_MXFP4) {
        vop[0] = row * 32 + ((hh ^ swz_v4(row)) << 4);
        vop[1] = G::VBYTES + hh * D + row;
      } else if (PV == PV_MXFP8) {
        // half hh: keys 16 hh + [0, 16) (block 0), then 32 + 16 hh + [0, 16) (block 1)
        vop[0] = row * 64 + ((hh ^ swz_v(row)) << 4);
        vop[1] = row * 64 + (((2 + hh) ^ swz_v(row)) << 4);
      } else if (PV == PV_F16) {
        // half hh: keys 32 hh + 8 t + [0, 8) for the t-th K = 16 product
#pragma unroll
        for (int t = 0; t < G::VOPS; t++) vop[t] = row * 128 + (((4 * hh + t) ^ swz_v16(row)) << 4);
      } else {
        vop[0] = row * 64 + (((2 * hh) ^ swz_v(row)) << 4);
        vop[1] = row * 64 + (((2 * hh + 1) ^ swz_v(row)) << 4);
      }
    }
    // the scale byte of (channel 32 c + n, key block hh), supplied by lane n + 32 hh
    vsc = G::VBYTES + hh * D + n;
    // opaque to the optimizer: keep these in registers instead of recomputing them every tile
#pragma unroll
    for (int i = 0; i < KL; i++) asm volatile("" : "+v"(kld[i]));
#pragma unroll
    for (int i = 0; i < VL; i++) asm volatile("" : "+v"(vld[i]));
#pragma unroll
    for (int s = 0; s < (KOP_IMM ? 1 : 2); s++)
#pragma unroll
      for (int c = 0; c < G::NQF; c++) asm volatile("" : "+v"(kop[s][c]));
#pragma unroll
    for (int c = 0; c < G::NQF; c++)
      if (QK == QK_MXFP4) asm volatile("" : "+v"(ksc[c]));
#pragma unroll
    for (int t = 0; t < G::VOPS; t++) asm volatile("" : "+v"(vop[t]));
  }
};

// ---- K / V tile staging: direct global -> LDS loads (no staging registers) ----
// A wave's 16-byte direct load puts lane L's data at LDS base + 16 L, so the swizzle is
// applied to the global source offset instead.  K stage: codes (+ E8M0 scales).  V stage:
// V^T codes (+ dS * sm * log2 e, staged through registers because it is rescaled on the
// way), read one step later than K.
template <int D, int QK, typename LO>
__device__ __forceinline__ void issue_k(uint8_t* lds, const FwdArgs& a, size_t kt0, int j, const LO& lo, int w, int lane) {
  using G = Geo<D, QK>;
  const uint8_t* kg = a.k_codes + (kt0 + (size_t)j * kTK) * G::KROW;
#pragma unroll
  for (int i = 0; i < LO::KL; i++) {
    const int pbase = LO::NTHREADS * i + 64 * w;
    if (pbase < G::KCHUNKS) load_lds16_async_so(kg, lo.kld[i], lds + pbase * 16);
  }
  if (QK == QK_MXFP4 && w == 0 && lane < G::SBYTES / 16) {
    const uint8_t* sg = reinterpret_cast<const uint8_t*>(a.k_scales) + (kt0 + (size_t)j * kTK) * (D / 32);
    load_lds16_async_so(sg, lane * 16, lds + G::KBYTES);
  }
}

template <int D, int QK, int NT, int PV>
__device__ __forceinline__ void issue_v(uint8_t* lds, const FwdArgs& a, size_t kt0, int j,
                                        const LaneOffs<D, QK, NT, PV>& lo, int w, int lane) {
  using G = Geo<D, QK, PV>;
  const uint8_t* vg = a.v_codes + (kt0 / kTK + j) * G::VBYTES;
#pragma unroll
  for (int i = 0; i < LaneOffs<D, QK, NT, PV>::VL; i++) {
    const int pbase = NT * i + 64 * w;
    if (pbase < G::VCHUNKS) load_lds16_async_so(vg, lo.vld[i], lds + pbase * 16);
  }
  if (PV != PV_FP8 && w == NT / 64 - 1 && lane < G::VSB / 16) {
    // E8M0 bytes of the tile's two 32-key groups: [group][channel], contiguous in the buffer
    const uint8_t* sg = reinterpret_cast<const uint8_t*>(a.v_scales) + (kt0 / 32 + 2 * j) * D;
    load_lds16_async_so(sg, 16 * lane, lds + G::VBYTES + 16 * lane);
  }
}

// MXFP4 dS strip of one tile (64 floats): fetched into registers, stored scaled.
__device__ __forceinline__ uint4 load_ds(const FwdArgs& a, size_t ds0, int j) {
  return reinterpret_cast<const uint4*>(a.delta_s + ds0 + (size_t)j * kTK)[threadIdx.x & 15];
}
template <int D, int QK, int PV>
__device__ __forceinline__ void store_ds(uint4 r, uint8_t* lds, float c) {
  const v4f f = {__uint_as_float(r.x) * c, __uint_as_float(r.y) * c, __uint_as_float(r.z) * c, __uint_as_float(r.w) * c};
  reinterpret_cast<v4f*>(lds + Geo<D, QK, PV>::DSOFF)[threadIdx.x & 15] = f;
}

// Wait for this wave's outstanding global loads (the direct-to-LDS tiles) before a barrier.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- score tile: S^T = K Q^T for the two 32-key subtiles of a 64-key tile ----
template <int D, int QK>
struct Score {
  v16i si[QK == QK_INT8 ? 2 : 1];
  v16f sf[QK == QK_MXFP4 ? 2 : 1];
};

// dsl (MXFP4 with kDsAcc): this lane's dS values in LDS (the tile's dS floats from the lane
// half's first key), the initial accumulator of each subtile; null otherwise.
template <int D, int QK, typename LO, int KS = 16>
__device__ __forceinline__ void qk_tile(Score<D, QK>& S, const uint8_t* lk, const v4i* qf, const v8i* qf4,
                                        const int* qsc, const LO& lo, const float* dsl = nullptr) {
  using G = Geo<D, QK>;
#pragma unroll
  for (int s = 0; s < 2; s++) {
    if (QK == QK_INT8) {
      v16i acc = v16i{};
#pragma unroll
      for (int c = 0; c < G::NQF; c++) {
        const v4i ka = *reinterpret_cast<const v4i*>(lk + lo.kop_at(s, c));
        acc = mfma_i8(ka, qf[c], acc);
      }
      S.si[s] = acc;
    } else {
      v16f acc = v16f{};
      if (dsl) {
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const v4f dv = *reinterpret_cast<const v4f*>(dsl + KS * s + r);
#pragma unroll
          for (int i = 0; i < 4; i++) acc[r + i] = dv[i];
        }
      }
#pragma unroll
      for (int c = 0; c < G::NQF; c++) {
        const v4i k4 = *reinterpret_cast<const v4i*>(lk + lo.kop_at(s, c));
        const v8i ka = v8i{k4[0], k4[1], k4[2], k4[3], 0, 0, 0, 0};
        acc = mfma_mxfp4(ka, qf4[c], acc, lk[lo.ksc_at(s, c)], qsc[c]);
      }
      S.sf[s] = acc;
    }
  }
}

// Reductions of a lane's values as balanced trees: a wave issues a vector instruction that
// depends on the previous one only after that one's latency, so a long chain (a running max
// or sum) leaves the lane idle; a tree of 32 is 5 deep.  Measured 2 % faster on the MXFP4
// kernels.  The fp32 row sum is not a quantization decision, so its order is free.
template <int N>
__device__ __forceinline__ float tree_max_f(float* x) {
#pragma unroll
  for (int w = N / 2; w >= 1; w /= 2)
#pragma unroll
    for (int r = 0; r < w; r++) x[r] = fmaxf(x[r], x[r + w]);
  return x[0];
}
// The maximum of 32 values as a tree of three-operand maxima (v_max3_f32): 11, then 4, 2 and 1
// values, 17 instructions against 31 two-operand ones, still only four deep.
__device__ __forceinline__ float tree_max3_32(const float* x) {
  float a[11], b[4];
#pragma unroll
  for (int k = 0; k < 10; k++) a[k] = fmaxf(fmaxf(x[3 * k], x[3 * k + 1]), x[3 * k + 2]);
  a[10] = fmaxf(x[30], x[31]);
#pragma unroll
  for (int k = 0; k < 3; k++) b[k] = fmaxf(fmaxf(a[3 * k], a[3 * k + 1]), a[3 * k + 2]);
  b[3] = fmaxf(a[9], a[10]);
  return fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3]));
}
template <int N>
__device__ __forceinline__ float tree_sum_f(float* x) {
#pragma unroll
  for (int w = N / 2; w >= 1; w /= 2)
#pragma unroll
    for (int r = 0; r < w; r++) x[r] = x[r] + x[r + w];
  return x[0];
}

// Online-softmax state of one wave's 32 queries.
template <int D>
struct RowState {
  v16f O[D / 32];
  float m, l;
  float mt;   // MXFP4 P~: the tile max that fixes the frame of O (see softmax_max)
  float um;   // MXFP4 P~: the largest of this lane's scaled scores in the current tile
};

// Softmax of tile j from its score registers, then O^T += V^T P~^T.
//   u_i = S_i (INT8: converted to fp32) or S_i + dS_i / c (MXFP4), with c = the positive
//   log2-domain scale; masked entries are set to -inf; the row max is taken on u, and
//   p448_i = exp2(u_i * c + (log2 448 - m)) comes out of one FMA and one exp2 per element.
template <int D, int QK, bool CAUSAL, int PV, bool FINE>
__device__ __forceinline__ void softmax_max(RowState<D>& st, const Score<D, QK>& Sc, const uint8_t* vstage,
                                            float kstep, float qstep, float sm_log2e, int j, int N, int qw,
                                            int qrow, int hh, float* u, float& c, float& off, float& lsc) {
  using G = Geo<D, QK, PV>;
  constexpr int NCB = G::NCB;
  const int kbase = j * kTK;
  const bool need_mask = kbase + kTK > N || (CAUSAL && kbase + kTK - 1 > qw);
  float mt;
  if (QK == QK_INT8) {
    // kstep: this tile's K step (FINE: the step of the 32-key group hh this lane's half holds)
    c = qstep * kstep;
    // c must stay positive so that masked entries (-inf) stay -inf after scaling.  A zero
    // step (an all-zero block: every code 0) or a product of tiny steps that underflows
    // binary32 is raised to the smallest normal float: a score times it is below 2^-100, as
    // negligible as the true one, so tiny inputs keep near-uniform weights.  A NaN step
    // fails the comparison and stays NaN.
    c = c < __FLT_MIN__ ? __FLT_MIN__ : c;
    int im;
    if (need_mask) {
      asm volatile("" ::: "memory");   // a real branch: the rare masked tiles must not cost every tile
      // in-lane key offsets below lim are visible
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - (kbase + KeyMap<PV>::KH * hh);
      im = INT_MIN;
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int i = 16 * s + r;
          const bool ok = KeyMap<PV>::lane_key(i) < lim;
          im = ok ? max(im, Sc.si[s][r]) : im;
          u[i] = ok ? (float)Sc.si[s][r] : -INFINITY;
        }
      if (FINE) {
        // the halves scale differently: the row max is taken on the scaled scores
        const float mo = im == INT_MIN ? -INFINITY : (float)im * c;
        mt = fmaxf(mo, other_half(mo));
      } else {
        const int imo = __builtin_bit_cast(int, other_half(__builtin_bit_cast(float, im)));
        im = max(im, imo);
        mt = im == INT_MIN ? -INFINITY : (float)im * c;
      }
    } else {
      // the row max on the integer scores (c > 0): exact, no NaN handling
      // (a running max here: the hardware hides its chain under the converts, and a tree
      // measured no faster while it costs 7 more instructions)
      im = Sc.si[0][0];
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          im = max(im, Sc.si[s][r]);
          u[16 * s + r] = (float)Sc.si[s][r];
        }
      if (FINE) {
        const float mo = (float)im * c;
        mt = fmaxf(mo, other_half(mo));
      } else {
        const int imo = __builtin_bit_cast(int, other_half(__builtin_bit_cast(float, im)));
        mt = (float)max(im, imo) * c;
      }
    }
  } else {
    if (kDsAcc<D, QK, PV>) {
      // the scores already hold dS (the QK accumulator's initial value): u = S + dS, and the
      // positive scale c = sm log2 e applies with the exp's offset, as c does on the INT8 path
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r++) u[16 * s + r] = Sc.sf[s][r];
      c = sm_log2e;
    } else {
      // dS arrives pre-multiplied by sm * log2 e; u = S * sm * log2 e + dS * sm * log2 e, c = 1
      const float* dsl = reinterpret_cast<const float*>(vstage + G::DSOFF) + KeyMap<PV>::KH * hh;
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const v4f dv = *reinterpret_cast<const v4f*>(dsl + KeyMap<PV>::KS * s + r);
#pragma unroll
          for (int i = 0; i < 4; i++) u[16 * s + r + i] = fmaf(Sc.sf[s][r + i], sm_log2e, dv[i]);
        }
      c = 1.0f;
    }
    if (need_mask) {
      asm volatile("" ::: "memory");
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - (kbase + KeyMap<PV>::KH * hh);
#pragma unroll
      for (int i = 0; i < 32; i++) u[i] = KeyMap<PV>::lane_key(i) < lim ? u[i] : -INFINITY;
    }
    // lane max of u (MXFP4 P~ takes its block scale from it with the same c and offset as the
    // weights); the tile max in the scaled units (c > 0 keeps the order; c = 1 without kDsAcc)
    st.um = tree_max3_32(u);
    mt = half_max(st.um) * c;
  }
  const float mnew = fmaxf(st.m, mt);
  const float mref = mnew == -INFINITY ? 0.0f : mnew;
  if (PV != PV_MXFP4) {
    if (__any(mnew > st.m)) {
      const float alpha = fast_exp2(st.m - mref);
      st.l *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; cb++) st.O[cb] *= alpha;
    }
    off = G::PLOG2 - mref;
    lsc = 1.0f;
  } else {
    // MXFP4 P~: p' = sigma p with sigma = 6 / max_tile(p) = 6 exp2(m - mt), so p' = exp2(t - mt +
    // log2 6) needs only the tile max mt.  O is kept as O' = sigma O (the frame of the last
    // tile's sigma), so P~V accumulates into it directly and the frame moves by
    // beta = sigma_j alpha_j / sigma_{j-1} = exp2(mt_{j-1} - mt_j).  A row whose tile is fully
    // masked keeps its frame; mt is held within 64 of m (p' of such a tile is then < 6, its
    // share of O < 2^-64, and the frame cannot overflow).  l' = 6 sum p = exp2(mt - m) sum p'.
    const float mte = mt == -INFINITY ? st.mt : fmaxf(mt, mnew - 64.0f);
    st.l *= fast_exp2(st.m - mref);
    const float beta = mte == -INFINITY ? 1.0f : fast_exp2(st.mt - mte);
    if (__any(beta != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < NCB; cb++) st.O[cb] *= beta;
    }
    st.mt = mte;
    const float mter = mte == -INFINITY ? 0.0f : mte;
    off = kLog2_6 - mter;
    lsc = fast_exp2(mter - mref);
  }
  st.m = mnew;
}

// Second half of tile j's softmax: p = exp2(u c + off) (FP8: 448 P; MXFP4: sigma P), the row
// sum and the P~ pack, sharing one basic block with the QK MFMAs of tile j+1 (into Sn) and the
// PV MFMAs of tile j.  The issue order is pinned: the K operand reads, then the QK MFMAs one at
// a time between slices of the exp / pack stream (so the matrix core runs under the vector
// work of the same wave instead of stalling its issue), then the V operand reads and the PV
// MFMAs.  MXFP4 P~: each lane's 32 keys are one MX block (E8M0 from the block max, floor rule;
// E2M1 RNE with saturation), and the scaled FP4 MFMA applies both operands' block scales.
template <int D, int QK, int PV, bool IL, typename LO>
__device__ __forceinline__ void softmax_body_pv(RowState<D>& st, const float* u, float c, float off, float lsc,
                                                Score<D, QK>& Sn, const uint8_t* lk_next, const uint8_t* vstage,
                                                const v4i* qf, const v8i* qf4, const int* qsc, const LO& lo) {
  using G = Geo<D, QK, PV>;
  constexpr int NCB = G::NCB;
  constexpr int NQK = 2 * G::NQF;                          // QK MFMAs of one tile
  constexpr int KREADS = NQK * (QK == QK_MXFP4 ? 2 : 1);   // their LDS reads (+ scale bytes)
  constexpr int VSLOT = 112 / NQK;                         // vector instructions per MFMA slot
  if (IL) qk_tile<D, QK>(Sn, lk_next, qf, qf4, qsc, lo);
  float ps[8];   // row-sum partials of 4 keys each, summed as a tree
  if (PV == PV_F16) {
    // fp16 P~ = p (RNE), eight keys per K = 16 product, fp32 accumulation
    v4i ph[4];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float p0 = fast_exp2(fmaf(u[i], c, off)), p1 = fast_exp2(fmaf(u[i + 1], c, off));
      const float p2 = fast_exp2(fmaf(u[i + 2], c, off)), p3 = fast_exp2(fmaf(u[i + 3], c, off));
      ps[i / 4] = (p0 + p1) + (p2 + p3);
      ph[i / 8][(i % 8) / 2] = pack_f16x2(p0, p1);
      ph[i / 8][(i % 8) / 2 + 1] = pack_f16x2(p2, p3);
    }
    st.l += tree_sum_f<8>(ps);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
      for (int t = 0; t < 4; t++)
        st.O[cb] = mfma_f16(*reinterpret_cast<const v4i*>(vstage + lo.vop_at(cb, t)), ph[t], st.O[cb]);
  } else if (PV != PV_MXFP4) {
    v8i pb;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float p0 = fast_exp2(fmaf(u[i], c, off)), p1 = fast_exp2(fmaf(u[i + 1], c, off));
      const float p2 = fast_exp2(fmaf(u[i + 2], c, off)), p3 = fast_exp2(fmaf(u[i + 3], c, off));
      ps[i / 4] = (p0 + p1) + (p2 + p3);
      pb[i / 4] = pack_fp8x4(p0, p1, p2, p3);
    }
    st.l += tree_sum_f<8>(ps);
    // O^T += V^T P~^T
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) {
      const v4i v0 = *reinterpret_cast<const v4i*>(vstage + lo.vop_at(cb, 0));
      const v4i v1 = *reinterpret_cast<const v4i*>(vstage + lo.vop_at(cb, 1));
      const v8i va = v8i{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if (PV == PV_MXFP8)
        st.O[cb] = mfma_f8_sa(va, pb, st.O[cb], vstage[lo.vsc + 32 * cb]);
      else
        st.O[cb] = mfma_f8(va, pb, st.O[cb]);
    }
  } else {
    // the block maximum of the lane's 32 weights is the weight of its largest score (the FMA
    // and exp2 do not decrease), so the E8M0 scale is fixed before any weight is formed and
    // the weights are packed eight at a time
    const int sb = (int)mx_fp4_scale_byte(fast_exp2(fmaf(st.um, c, off)));
    // byte 0 (an all-zero block, e.g. keys past the causal diagonal): codes 0 under any scale,
    // so convert with 1 rather than the subnormal 2^-127
    const float scl = sb == 0 ? 1.0f : e8m0_to_float((unsigned)sb);
    v8i pb = v8i{};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float pf[8];
#pragma unroll
      for (int i = 0; i < 8; i++) pf[i] = fast_exp2(fmaf(u[8 * k + i], c, off));
      ps[2 * k] = (pf[0] + pf[1]) + (pf[2] + pf[3]);
      ps[2 * k + 1] = (pf[4] + pf[5]) + (pf[6] + pf[7]);
      pb[k] = (int)pack_fp4x8(pf, scl);
    }
    st.l = fmaf(lsc, tree_sum_f<8>(ps), st.l);
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) {
      const v4i v0 = *reinterpret_cast<const v4i*>(vstage + lo.vop_at(cb, 0));
      const int sa = vstage[lo.vop_at(cb, 1)];
      const v8i va = v8i{v0[0], v0[1], v0[2], v0[3], 0, 0, 0, 0};
      st.O[cb] = mfma_mxfp4(va, pb, st.O[cb], sa, sb);
    }
  }
  if (IL) {
    __builtin_amdgcn_sched_group_barrier(0x100, KREADS, 0);     // DS reads: K operands
#pragma unroll
    for (int i = 0; i < NQK; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one QK MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VSLOT, 0);    // vector work of tile j
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);         // the rest of it
    __builtin_amdgcn_sched_group_barrier(0x100, G::VOPS * NCB, 0);   // DS reads: V operands
    __builtin_amdgcn_sched_group_barrier(0x008, G::PVM * NCB, 0);    // PV MFMAs
  }
}

// ---- epilogue: O / l (FP8: times the V channel step), LSE ----
//   FP8 P~ (V in FP8 or MXFP8): O and l both carry the factor 448; MXFP8's V block scales are
//   applied inside the MFMA.  MXFP4 P~: O' = sigma O with sigma = 6 exp2(m - mt) and
//   l' = 6 sum p, so O / l = O' exp2(mt - m) / l'.
template <int D, int QK, bool CAUSAL, int DT, int PV>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, const RowState<D>& st, const Inst& qi, int qrow, int hh,
                                             const float* vsc) {
  using G = Geo<D, QK, PV>;
  constexpr int NCB = G::NCB;
  const float lt = half_sum(st.l);
  if (qrow < qi.len) {
    const float inv = PV != PV_MXFP4 ? 1.0f / lt : fast_exp2(st.mt - st.m) / lt;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + qi.io0 + (size_t)qrow * qi.ios;
#pragma unroll
    for (int c = 0; c < NCB; c++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int ch = 32 * c + 8 * g + 4 * hh;
        const v4f sc = PV == PV_FP8 ? *reinterpret_cast<const v4f*>(vsc + ch) * inv
                                    : v4f{inv, inv, inv, inv};
        const uint32_t lo = pack2_io<DT>(st.O[c][4 * g] * sc[0], st.O[c][4 * g + 1] * sc[1]);
        const uint32_t hi = pack2_io<DT>(st.O[c][4 * g + 2] * sc[2], st.O[c][4 * g + 3] * sc[3]);
        *reinterpret_cast<uint2*>(orow + ch) = make_uint2(lo, hi);
      }
    if (a.lse && hh == 0)
      a.lse[qi.lse0 + qrow] =
          (st.m + __log2f(lt) - (PV != PV_MXFP4 ? G::PLOG2 : kLog2_6)) * kLn2 + a.lse_corr[qi.row0 + qrow];
  }
}

template <int D, int QK, bool CAUSAL, int DT, int PV, bool FINE>
__device__ __forceinline__ void run_qtile(const FwdArgs& a, int b, int h, int qt, uint8_t (*lk)[Geo<D, QK, PV>::KSTAGE],
                                          uint8_t (*lv)[Geo<D, QK, PV>::VSTAGE], float* vsc) {
  using G = Geo<D, QK, PV>;
  constexpr int NCB = G::NCB, NQF = G::NQF;
  const int qbase = qt * kQT;
  // this query tile's instance, the KV instance its head reads, and its dS strip
  const Inst qi = q_inst(a.g, b, h, D);
  if (qbase >= qi.len) return;   // packed sequences: a tile past this sequence's end
  const int hk = h / (a.g.H / a.g.Hkv);
  const Inst ki = k_inst(a.g, b, hk, D);
  const size_t kt0 = ki.tok0, kvid = (size_t)b * a.g.Hkv + hk;
  // dS strip: per key, or (per-block Q smoothing) the row of this query tile's block
  const size_t ds0 = QK != QK_MXFP4 ? 0
                     : a.qbs ? qblock_slot(a.g, b, h, qt) * a.qbs : ds_base(a.g, b, h);
  const int NK = ki.len;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int n = lane & 31, hh = lane >> 5;
  const int qw = qbase + 32 * w;          // first query of this wave
  const int qrow = qw + n;                // this lane's query
  LaneOffs<D, QK, 256, PV> lo;
  lo.init(w, lane, n, hh);

  // Q fragments (B operand), resident for the whole pass
  v4i qf[QK == QK_INT8 ? NQF : 1];
  v8i qf4[QK == QK_MXFP4 ? NQF : 1];
  int qsc[QK == QK_MXFP4 ? NQF : 1];
  float qstep = 0.0f;
  if (QK == QK_INT8) {
    const uint8_t* qp = a.q_codes + (qi.tok0 + qrow) * D + 16 * hh;
#pragma unroll
    for (int c = 0; c < NQF; c++) qf[c] = *reinterpret_cast<const v4i*>(qp + 32 * c);
    // FINE: a step per query token; else one per 64-token block, the same for the whole wave
    // (its 32 queries lie in one block): a scalar register, not a vector one
    if (FINE) {
      qstep = reinterpret_cast<const float*>(a.q_scales)[qi.tok0 + qrow] * a.sm_log2e;
    } else {
      const float qs = reinterpret_cast<const float*>(a.q_scales)[qi.tok0 / kTK + qw / kTK] * a.sm_log2e;
      qstep = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, qs)));
    }
  } else {
    const uint8_t* qp = a.q_codes + (qi.tok0 + qrow) * (D / 2) + 16 * hh;
    const uint8_t* qe = reinterpret_cast<const uint8_t*>(a.q_scales) + (qi.tok0 + qrow) * (D / 32) + hh;
#pragma unroll
    for (int c = 0; c < NQF; c++) {
      const v4i lo = *reinterpret_cast<const v4i*>(qp + 32 * c);
      qf4[c] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      qsc[c] = qe[2 * c];
    }
  }
  // K steps: one per 64-key tile, or (FINE) one per 32 keys; a lane takes its half's step.  They
  // are read-only during the kernel and the same for the whole wave (FINE: per lane half), so
  // they come through the scalar cache (the constant address space) instead of as vector-memory
  // loads, each tile's one tile ahead.
  typedef __attribute__((address_space(4))) const float cfloat;
  cfloat* kstep = (cfloat*)(uintptr_t)(reinterpret_cast<const float*>(a.k_scales) + (FINE ? kt0 / 32 : kt0 / kTK));
  auto kstep_of = [&](int t) -> float {
    if (QK != QK_INT8) return 0.0f;
    if (!FINE) return kstep[t];
    const float k0 = kstep[2 * t], k1 = kstep[2 * t + 1];
    return hh ? k1 : k0;
  };

  int ntiles = (NK + kTK - 1) / kTK;
  if (CAUSAL) ntiles = min(ntiles, (qbase + kQT - 1) / kTK + 1);
  // tiles holding keys this wave may see (causal: later tiles are fully masked for it)
  const int wtiles = CAUSAL ? min(ntiles, (qw + 31) / kTK + 1) : ntiles;

  RowState<D> st;
#pragma unroll
  for (int c = 0; c < NCB; c++) st.O[c] = v16f{};
  st.m = -INFINITY;
  st.l = 0.0f;
  st.mt = -INFINITY;

  // prologue: K0, K1, V0 -> LDS in one round trip; QK(0); a barrier before the loop's first
  // prefetch overwrites K0
  if (ntiles == 0) {
    // no key in this sequence: a zero output and LSE -inf (the softmax over an empty set)
    if (qrow < qi.len) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + qi.io0 + (size_t)qrow * qi.ios;
#pragma unroll
      for (int c = 0; c < NCB; c++)
#pragma unroll
        for (int g4 = 0; g4 < 4; g4++) *reinterpret_cast<uint2*>(orow + 32 * c + 8 * g4 + 4 * hh) = make_uint2(0, 0);
      if (a.lse && hh == 0) a.lse[qi.lse0 + qrow] = -INFINITY;
    }
    return;
  }
  float ks_cur = kstep_of(0);
  // FP8 V: the KV head's channel steps, staged in LDS for the epilogue (visible after the
  // prologue's barrier), so the output stores do not wait on global loads one by one
  if (PV == PV_FP8 && threadIdx.x < D) vsc[threadIdx.x] = a.v_scales[kvid * D + threadIdx.x];
  const int last = ntiles - 1;
  if constexpr (kOneBuf<D, QK, PV>) {
    // K and V one tile ahead; tile j: prefetch K(j+1), V(j+1) into the buffers tile j-1 used,
    // then QK(j), softmax and PV(j) from this tile's buffers; barrier
    issue_k<D, QK>(lk[0], a, kt0, 0, lo, w, lane);
    issue_v<D, QK>(lv[0], a, kt0, 0, lo, w, lane);
    // kDsAcc: dS unscaled (the QK accumulator adds it to S before the scale)
    const float ds_scale = kDsAcc<D, QK, PV> ? 1.0f : a.sm_log2e;
    if (QK == QK_MXFP4) store_ds<D, QK, PV>(load_ds(a, ds0, 0), lv[0], ds_scale);
    wait_vmem();
    __syncthreads();
    auto step1 = [&](int j) {
      const float ks = ks_cur;
      ks_cur = kstep_of(min(j + 1, last));
      issue_k<D, QK>(lk[(j + 1) & 1], a, kt0, min(j + 1, last), lo, w, lane);
      issue_v<D, QK>(lv[(j + 1) & 1], a, kt0, min(j + 1, last), lo, w, lane);
      uint4 dsr;
      if (QK == QK_MXFP4) dsr = load_ds(a, ds0, min(j + 1, last));
      if (j < wtiles) {
        Score<D, QK> Sc;
        qk_tile<D, QK, decltype(lo), KeyMap<PV>::KS>(
            Sc, lk[j & 1], qf, qf4, qsc, lo,
            kDsAcc<D, QK, PV> ? reinterpret_cast<const float*>(lv[j & 1] + G::DSOFF) + KeyMap<PV>::KH * hh : nullptr);
        float u[32], c, off, lsc;
        softmax_max<D, QK, CAUSAL, PV, FINE>(st, Sc, lv[j & 1], ks, qstep, a.sm_log2e, j, NK, qw, qrow, hh, u, c, off,
                                             lsc);
        softmax_body_pv<D, QK, PV, false>(st, u, c, off, lsc, Sc, lk[(j + 1) & 1], lv[j & 1], qf, qf4, qsc, lo);
      }
      if (QK == QK_MXFP4) store_ds<D, QK, PV>(dsr, lv[(j + 1) & 1], ds_scale);
      wait_vmem();
      __syncthreads();
    };
    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
      step1(j);
      step1(j + 1);
    }
    if (j < ntiles) step1(j);
    fwd_epilogue<D, QK, CAUSAL, DT, PV>(a, st, qi, qrow, hh, vsc);
    return;
  }
  issue_k<D, QK>(lk[0], a, kt0, 0, lo, w, lane);
  issue_k<D, QK>(lk[1], a, kt0, min(1, ntiles - 1), lo, w, lane);
  issue_v<D, QK>(lv[0], a, kt0, 0, lo, w, lane);
  if (QK == QK_MXFP4) store_ds<D, QK, PV>(load_ds(a, ds0, 0), lv[0], a.sm_log2e);
  wait_vmem();
  __syncthreads();
  Score<D, QK> Sa, Sb;
  qk_tile<D, QK>(Sa, lk[0], qf, qf4, qsc, lo);
  __syncthreads();

  // One tile: prefetch K(j+2) into lk[j&1] and V(j+1) into lv[(j+1)&1] (both already
  // consumed: tile j's K by QK(j) and tile j-1's V by PV(j-1), before the last barrier);
  // issue QK(j+1) into Sn; softmax + PV of tile j from Sc; barrier.  Prefetch indices are
  // clamped to the last tile, so the loads are unconditional.  Unrolled twice so Sa/Sb
  // alternate without copies.
  constexpr bool IL = !(D == 128 && QK == QK_INT8 && MFMA_IL_D128 == 0);
  auto step = [&](int j, const Score<D, QK>& Sc, Score<D, QK>& Sn) {
    const float ks = ks_cur;
    ks_cur = kstep_of(min(j + 1, last));
    issue_k<D, QK>(lk[j & 1], a, kt0, min(j + 2, last), lo, w, lane);
    issue_v<D, QK>(lv[(j + 1) & 1], a, kt0, min(j + 1, last), lo, w, lane);
    uint4 dsr;
    if (QK == QK_MXFP4) dsr = load_ds(a, ds0, min(j + 1, last));
    // tiles past this wave's last visible one need neither softmax nor the next scores.  With
    // IL the next tile's QK MFMAs are spread through the exp / pack stream (the last tile then
    // computes scores of an already-loaded tile that nothing reads); otherwise they are all
    // issued before the softmax, whose vector work then runs under them.  Measured: IL is
    // ahead at d = 64 (fewer, shorter QK MFMAs per tile), behind at d = 128 INT8.
    if (!IL) {
      if (j + 1 < wtiles) qk_tile<D, QK>(Sn, lk[(j + 1) & 1], qf, qf4, qsc, lo);
      // keep the phases apart: QK(j+1)'s operands die before the softmax starts
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j < wtiles) {
      float u[32], c, off, lsc;
      softmax_max<D, QK, CAUSAL, PV, FINE>(st, Sc, lv[j & 1], ks, qstep, a.sm_log2e, j, NK, qw, qrow, hh, u, c, off, lsc);
      softmax_body_pv<D, QK, PV, IL>(st, u, c, off, lsc, Sn, lk[(j + 1) & 1], lv[j & 1], qf, qf4, qsc, lo);
    }
    if (QK == QK_MXFP4) store_ds<D, QK, PV>(dsr, lv[(j + 1) & 1], a.sm_log2e);
    wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, Sa, Sb);
    step(j + 1, Sb, Sa);
  }
  if (j < ntiles) step(j, Sa, Sb);

  fwd_epilogue<D, QK, CAUSAL, DT, PV>(a, st, qi, qrow, hh, vsc);
}

// One 128-query tile per workgroup.  Causal tiles differ in length, so they are dealt longest
// first: the dispatcher starts workgroups in id order as slots free up, which makes this a
// longest-first greedy schedule (a slot that runs faster, e.g. the older of the two
// workgroups sharing a CU, simply takes more of the short tiles at the end).  Each XCD takes
// whole heads, so a head's K/V tiles stay in one L2 (packed sequences: whole KV groups,
// dealt round-robin so that every XCD gets a share of every sequence).
template <int D, int QK, bool CAUSAL, int DT, int PV, bool FINE>
__global__ __launch_bounds__(256, (kOneBuf<D, QK, PV> ? 3 : 2)) void attn_fwd_kernel(FwdArgs a) {
  using G = Geo<D, QK, PV>;
  __shared__ __align__(16) uint8_t lk[2][G::KSTAGE];
  __shared__ __align__(16) uint8_t lv[2][G::VSTAGE];
  __shared__ __align__(16) float vsc[PV == PV_FP8 ? D : 4];
  const int nqt = a.nqt, BH = a.g.B * a.g.H;
  int bh, qt;
  const int nkv = a.g.B * a.g.Hkv;
  if (a.g.cu_q && nkv % 8 == 0) {
    // packed sequences differ in length, so an XCD must not take whole sequences: KV instance
    // x + 8 m goes to XCD x (each XCD gets one KV group of every sequence, and the query heads
    // sharing a KV head stay in one L2); tiles run longest (highest) first
    constexpr int X = 8;
    const int hw = blockIdx.x, x = hw % X, local = hw / X, per = BH / X, grp = a.g.H / a.g.Hkv;
    qt = nqt - 1 - local / per;
    const int j = local % per, kv = x + X * (j / grp);
    bh = (kv / a.g.Hkv) * a.g.H + (kv % a.g.Hkv) * grp + j % grp;
  } else if (CAUSAL) {
    constexpr int X = 8;
    const int hw = blockIdx.x;
    if (BH % X == 0) {
      const int hpx = BH / X, local = hw / X;
      bh = (hw % X) * hpx + local % hpx;
      qt = nqt - 1 - local / hpx;
    } else {
      bh = hw % BH;
      qt = nqt - 1 - hw / BH;
    }
  } else {
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    bh = id / nqt;
    qt = id % nqt;
  }
  run_qtile<D, QK, CAUSAL, DT, PV, FINE>(a, bh / a.g.H, bh % a.g.H, qt, lk, lv, vsc);
}

template <int D, int QK, int DT, int PV, bool FINE>
static hipError_t fwd_dispatch(const Shape& s, const FwdArgs& a, hipStream_t st) {
  const int grid = s.g.B * s.g.H * a.nqt;
  if (s.causal)
    attn_fwd_kernel<D, QK, true, DT, PV, FINE>
        <<<grid, 256, debug_lds_pad(attn_fwd_kernel<D, QK, true, DT, PV, FINE>), st>>>(a);
  else
    attn_fwd_kernel<D, QK, false, DT, PV, FINE>
        <<<grid, 256, debug_lds_pad(attn_fwd_kernel<D, QK, false, DT, PV, FINE>), st>>>(a);
  return hipGetLastError();
}

template <int QK, int DT, int PV, bool FINE = false>
static hipError_t fwd_dispatch_d(const Shape& s, const FwdArgs& a, hipStream_t st) {
  return s.d == 64 ? fwd_dispatch<64, QK, DT, PV, FINE>(s, a, st) : fwd_dispatch<128, QK, DT, PV, FINE>(s, a, st);
}
// INT8 QK: per-64-token steps (QK_INT8) or per-token / per-32-key steps (QK_INT8T)
template <int DT, int PV>
static hipError_t fwd_dispatch_int8(const Shape& s, const FwdArgs& a, hipStream_t st) {
  return s.qk_fmt == QK_INT8T ? fwd_dispatch_d<QK_INT8, DT, PV, true>(s, a, st) : fwd_dispatch_d<QK_INT8, DT, PV>(s, a, st);
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
  a.g = s.g;
  a.nqt = (s.g.nbq * 64) / kQT;   // tiles of 128 queries covering the longest query instance
  a.qbs = s.qk_fmt == QK_MXFP4B ? (int)qblock_strip(s.g) : 0;
  a.sm_log2e = s.sm_scale * kLog2e;
  if (s.qk_fmt == QK_INT8 || s.qk_fmt == QK_INT8T) {
    if (s.pv_fmt == PV_F16)
      return s.io_dtype == 0 ? fwd_dispatch_int8<0, PV_F16>(s, a, st) : fwd_dispatch_int8<1, PV_F16>(s, a, st);
    if (s.pv_fmt != PV_FP8) return hipErrorInvalidValue;
    return s.io_dtype == 0 ? fwd_dispatch_int8<0, PV_FP8>(s, a, st) : fwd_dispatch_int8<1, PV_FP8>(s, a, st);
  }
  if (s.qk_fmt != QK_MXFP4 && s.qk_fmt != QK_MXFP4B) return hipErrorInvalidValue;
  if (s.pv_fmt == PV_MXFP4)
    return s.io_dtype == 0 ? fwd_dispatch_d<QK_MXFP4, 0, PV_MXFP4>(s, a, st)
                           : fwd_dispatch_d<QK_MXFP4, 1, PV_MXFP4>(s, a, st);
  if (s.pv_fmt == PV_MXFP8)
    return s.io_dtype == 0 ? fwd_dispatch_d<QK_MXFP4, 0, PV_MXFP8>(s, a, st)
                           : fwd_dispatch_d<QK_MXFP4, 1, PV_MXFP8>(s, a, st);
  return s.io_dtype == 0 ? fwd_dispatch_d<QK_MXFP4, 0, PV_FP8>(s, a, st) : fwd_dispatch_d<QK_MXFP4, 1, PV_FP8>(s, a, st);
}

}  // namespace sage
