// chunk.hip -- fused chunkwise KDA prefill for gfx950 (MI355X).
//
// Algebra: "Kimi Unveils Delta Attention and K3 Architecture Updates",
// section 6 (Chunkwise KDA), in the key-by-value orientation (S is d_k x d_v,
// decay multiplies key rows).  For one chunk of C = 64 tokens with incoming
// state S_c, let Gamma_i = prod_{m<=i} alpha_m (chunk-local cumulative decay,
// section 6.1/6.6 -- kept as a running product instead of exp of a prefix
// sum), Gamma_L the decay over the whole chunk, and
//
//   QG_i = s q_i * Gamma_i          KG_i = beta_i k_i * Gamma_i
//   KI_i = k_i / Gamma_i            KE_i = k_i * Gamma_L / Gamma_i   (K_end)
//   BV_i = beta_i v_i
//
// (products per key channel).  Then (section 6.3) R = strict_tril(KG KI^T)
// holds rho_ij = beta_i <k_j, D_{j+1:i} k_i>, (section 6.5)
// Aqk = tril(QG KI^T) holds chi_ij, and with T = (I + R)^{-1} the WY factors
// W = T KG and U = T BV give the resolved errors E = U - W S_c (section 6.2 +
// 6.3: E = T (BV - KG S_c)).  Finally (6.4, 6.5)
//
//   O_c     = QG S_c + Aqk E
//   S_{c+1} = Diag(Gamma_L) S_c + KE^T E.
//
// Design (one workgroup of 4 waves per (sequence, head) chain, all of d_v):
//  * the fp32 state never leaves the chip: each wave keeps its d_v/4 value
//    columns of S in MFMA accumulator registers for the whole sequence, and
//    only the chunk's S-independent operands are shared through LDS;
//  * S and E are consumed straight from the accumulator layout: two stacked
//    16-row accumulator tiles are one 32-deep MFMA operand once the k index is
//    relabelled (k = 4g + e for e < 4, 16 + 4g + e - 4 for e >= 4, g = lane/16);
//    every other operand is read from LDS in that same k order;
//  * operands contracted over tokens are stored row-major and read with
//    ds_read_b64_tr_b16 (gfx950 LDS transpose read);
//  * T is never formed off the diagonal: the four 16x16 diagonal blocks are
//    inverted by forward substitution, and W, U come from block forward
//    substitution X_I = T_II (B_I - sum_{J<I} R_IJ X_J);
//  * the next chunk's inputs are loaded into registers while this chunk is
//    computed.
//  * Exactness guard: the single chunk-start reference of KI = k / Gamma needs
//    Gamma_L >= 2^-100 in every key channel.  A chunk that decays more than
//    that in any channel is processed token by token (the recurrence itself)
//    on the same on-chip state instead; outputs are identical up to rounding.
#include "common.h"

namespace kda {

// ============================================================ operand policies
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <class P>
__device__ __forceinline__ __attribute__((address_space(3))) P* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) P*)(p);
}

// bf16 operands, fp32 accumulation: v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16.
struct OpBf16 {
  typedef uint16_t T;
  static constexpr int PAD_RM = 8;    // row padding (elements) of buffers read row-wise
  static constexpr int PAD_TR = 16;   // row padding of buffers read with the transpose read
  static constexpr int PAD_64 = 16;   // row padding of 64-wide buffers
  typedef i16x4 F16;                  // 16-deep operand fragment
  struct F32 { i16x4 lo, hi; };       // 32-deep operand fragment

  static __device__ __forceinline__ T cvt(float x) { return f32_to_bf16_bits(x); }
  static __device__ __forceinline__ F16 pack(f32x4 t) {
    u32x2 w;
    w[0] = pack_bf16x2(t[0], t[1]);
    w[1] = pack_bf16x2(t[2], t[3]);
    return __builtin_bit_cast(F16, w);
  }
  static __device__ __forceinline__ f32x4 unpack(F16 f) {
    u32x2 w = __builtin_bit_cast(u32x2, f);
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
  }
  static __device__ __forceinline__ f32x4 mma16(F16 a, F16 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma32(F32 a, F32 b, f32x4 c) {
    i16x8 a8 = __builtin_shufflevector(a.lo, a.hi, 0, 1, 2, 3, 4, 5, 6, 7);
    i16x8 b8 = __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a8),
                                                    __builtin_bit_cast(bf16x8, b8), c, 0, 0, 0);
  }
  // X row-major (ld elements per row): lane gets X[row0 + l%16][k0 + 4g + e], e < 4
  static __device__ __forceinline__ F16 ld16_rm(const T* X, int ld, int row0, int k0) {
    const int l = lane_id();
    return *lds_ptr<const F16>(X + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  // X row-major: lane gets X[k0 + 4g + e][m0 + l%16] (transpose read)
  static __device__ __forceinline__ F16 ld16_tr(const T* X, int ld, int k0, int m0) {
    const int l = lane_id();
    const int j = l & 15;
    const T* p = X + (k0 + 4 * (l >> 4) + (j >> 2)) * ld + m0 + 4 * (j & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  }
  static __device__ __forceinline__ F32 ld32_rm(const T* X, int ld, int row0, int k0) {
    return F32{ld16_rm(X, ld, row0, k0), ld16_rm(X, ld, row0, k0 + 16)};
  }
  static __device__ __forceinline__ F32 ld32_tr(const T* X, int ld, int k0, int m0) {
    return F32{ld16_tr(X, ld, k0, m0), ld16_tr(X, ld, k0 + 16, m0)};
  }
  // write accumulator tile t (rows row0 + 4g + r, column col0 + l%16) transposed:
  // Xt[col0 + l%16][row0 + 4g + r] for r = 0..3 (four contiguous elements)
  static __device__ __forceinline__ void st_ct(T* Xt, int ld, int col0, int row0, f32x4 t) {
    const int l = lane_id();
    *lds_ptr<F16>(Xt + (col0 + (l & 15)) * ld + row0 + 4 * (l >> 4)) = pack(t);
  }
};

// fp32 operands: v_mfma_f32_16x16x4_f32, four (or eight) per fragment.
struct OpF32 {
  typedef float T;
  static constexpr int PAD_RM = 4;
  static constexpr int PAD_TR = 4;
  static constexpr int PAD_64 = 4;
  typedef f32x4 F16;
  struct F32 { f32x4 lo, hi; };

  static __device__ __forceinline__ T cvt(float x) { return x; }
  static __device__ __forceinline__ F16 pack(f32x4 t) { return t; }
  static __device__ __forceinline__ f32x4 unpack(F16 f) { return f; }
  static __device__ __forceinline__ f32x4 mma16(F16 a, F16 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 mma32(F32 a, F32 b, f32x4 c) {
    return mma16(a.hi, b.hi, mma16(a.lo, b.lo, c));
  }
  static __device__ __forceinline__ F16 ld16_rm(const T* X, int ld, int row0, int k0) {
    const int l = lane_id();
    return *lds_ptr<const F16>(X + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  static __device__ __forceinline__ F16 ld16_tr(const T* X, int ld, int k0, int m0) {
    const int l = lane_id();
    const T* p = X + (k0 + 4 * (l >> 4)) * ld + m0 + (l & 15);
    F16 r;
    r[0] = *lds_ptr<const T>(p);
    r[1] = *lds_ptr<const T>(p + ld);
    r[2] = *lds_ptr<const T>(p + 2 * ld);
    r[3] = *lds_ptr<const T>(p + 3 * ld);
    return r;
  }
  static __device__ __forceinline__ F32 ld32_rm(const T* X, int ld, int row0, int k0) {
    return F32{ld16_rm(X, ld, row0, k0), ld16_rm(X, ld, row0, k0 + 16)};
  }
  static __device__ __forceinline__ F32 ld32_tr(const T* X, int ld, int k0, int m0) {
    return F32{ld16_tr(X, ld, k0, m0), ld16_tr(X, ld, k0 + 16, m0)};
  }
  static __device__ __forceinline__ void st_ct(T* Xt, int ld, int col0, int row0, f32x4 t) {
    const int l = lane_id();
    *lds_ptr<F16>(Xt + (col0 + (l & 15)) * ld + row0 + 4 * (l >> 4)) = t;
  }
};

// ============================================================ raw input vectors
// N consecutive I/O elements kept in their storage form, so that a prefetch
// stays in flight until the next chunk unpacks it.
template <class Io, int N> struct RawVec;
template <> struct RawVec<IoBf16, 4> {
  typedef u32x2 type;
  __device__ static type load(const void* p, size_t i) {
    return *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p) + i);
  }
  __device__ static void unpack(type w, float* o) {
    o[0] = __uint_as_float(w[0] << 16); o[1] = __uint_as_float(w[0] & 0xffff0000u);
    o[2] = __uint_as_float(w[1] << 16); o[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
};
template <> struct RawVec<IoBf16, 2> {
  typedef uint32_t type;
  __device__ static type load(const void* p, size_t i) {
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(p) + i);
  }
  __device__ static void unpack(type w, float* o) {
    o[0] = __uint_as_float(w << 16); o[1] = __uint_as_float(w & 0xffff0000u);
  }
};
template <> struct RawVec<IoF32, 4> {
  typedef f32x4 type;
  __device__ static type load(const void* p, size_t i) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i);
  }
  __device__ static void unpack(type w, float* o) { o[0] = w[0]; o[1] = w[1]; o[2] = w[2]; o[3] = w[3]; }
};
template <> struct RawVec<IoF32, 2> {
  typedef f32x2 type;
  __device__ static type load(const void* p, size_t i) {
    return *reinterpret_cast<const f32x2*>(reinterpret_cast<const float*>(p) + i);
  }
  __device__ static void unpack(type w, float* o) { o[0] = w[0]; o[1] = w[1]; }
};
template <int N> struct RawG;
template <> struct RawG<4> {
  typedef f32x4 type;
  __device__ static type load(const float* p, size_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
  __device__ static void unpack(type w, float* o) { o[0] = w[0]; o[1] = w[1]; o[2] = w[2]; o[3] = w[3]; }
};
template <> struct RawG<2> {
  typedef f32x2 type;
  __device__ static type load(const float* p, size_t i) { return *reinterpret_cast<const f32x2*>(p + i); }
  __device__ static void unpack(type w, float* o) { o[0] = w[0]; o[1] = w[1]; }
};

// ============================================================ configuration
template <int DK_, int DV_, class Io_, class Op_>
struct ChunkCfg {
  static constexpr int DK = DK_, DV = DV_;
  typedef Io_ Io;
  typedef Op_ Op;
  typedef typename Op::T T;
  static constexpr int C = 64;          // tokens per chunk
  static constexpr int NB = 4;          // 16-token blocks per chunk
  static constexpr int NW = 4;          // waves per workgroup
  static constexpr int CPL = DK / 32;   // key channels per lane in the prep layout
  static constexpr int VPL = DV / 32;   // value channels per lane in the prep layout
  static constexpr int NKS = DK / 32;   // 32-deep steps over key channels
  static constexpr int MTK = DK / 16;   // 16-row tiles over key channels
  static constexpr int NVT = DV / 64;   // 16-column value tiles per wave
  static constexpr int NKT = DK / 64;   // 16-column W tiles per wave
  static constexpr int NT = NKT + NVT;  // tiles per wave in the block substitution
  // LDS leading dimensions (elements)
  static constexpr int LD_K = DK + Op::PAD_RM;   // QG, KG, KI  [C][LD_K]
  static constexpr int LD_E = DK + Op::PAD_TR;   // KE          [C][LD_E]
  static constexpr int LD_V = DV + Op::PAD_TR;   // BV          [C][LD_V]
  static constexpr int LD_64 = C + Op::PAD_64;   // RTn, AQT [C][LD_64], WTn [DK][LD_64]
  // LDS byte offsets
  static constexpr int SZ = sizeof(T);
  static constexpr int OFF_QG = 0;
  static constexpr int OFF_KG = OFF_QG + C * LD_K * SZ;
  static constexpr int OFF_KI = OFF_KG + C * LD_K * SZ;
  static constexpr int OFF_KE = OFF_KI + C * LD_K * SZ;
  static constexpr int OFF_BV = OFF_KE + C * LD_E * SZ;
  static constexpr int OFF_RT = OFF_BV + C * LD_V * SZ;
  static constexpr int OFF_AQ = OFF_RT + C * LD_64 * SZ;
  static constexpr int OFF_WT = OFF_AQ + C * LD_64 * SZ;
  static constexpr int OFF_TD = OFF_WT + DK * LD_64 * SZ;
  static constexpr int OFF_RD = OFF_TD + NB * 16 * 16 * SZ;
  static constexpr int OFF_GL = OFF_RD + NB * 16 * 16 * 4;
  static constexpr int OFF_FL = OFF_GL + DK * 4;
  static constexpr int LDS_BYTES = OFF_FL + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(OFF_KG % 16 == 0 && OFF_KE % 16 == 0 && OFF_BV % 16 == 0 && OFF_RT % 16 == 0 &&
                OFF_AQ % 16 == 0 && OFF_WT % 16 == 0 && OFF_TD % 16 == 0 && OFF_RD % 16 == 0,
                "LDS alignment");
};

// Threshold below which a channel's chunk decay Gamma_L makes k / Gamma unsafe.
#define KDA_GAMMA_MIN 7.888609052210118e-31f /* 2^-100 */

// ============================================================ the kernel
template <class Cfg>
struct ChunkKernel {
  typedef typename Cfg::Io Io;
  typedef typename Cfg::Op Op;
  typedef typename Cfg::T T;
  static constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C;
  static constexpr int CPL = Cfg::CPL, VPL = Cfg::VPL;
  static constexpr int NKS = Cfg::NKS, MTK = Cfg::MTK, NVT = Cfg::NVT, NKT = Cfg::NKT,
                       NT = Cfg::NT;

  typedef typename RawVec<Io, CPL>::type RK;
  typedef typename RawVec<Io, VPL>::type RV;
  typedef typename RawG<CPL>::type RG;

  struct Raw {
    RG g[8];
    RK q[8], k[8];
    RV v[8];
    float beta;
  };

  // ---------------------------------------------------------------- loads
  // Prep layout: wave w, lane l: token group tg = l / 8 (tokens 8tg .. 8tg+7),
  // key channels kc0 .. kc0 + CPL - 1 with kc0 = w * DK/4 + (l % 8) * CPL,
  // value channels vc0 .. vc0 + VPL - 1 with vc0 = w * DV/4 + (l % 8) * VPL.
  static __device__ __forceinline__ void load_raw(Raw& r, const void* q, const void* k,
                                                  const void* v, const float* g,
                                                  const float* beta, size_t row_base, int H,
                                                  int h, int clen) {
    const int w = threadIdx.x >> 6, l = lane_id();
    const int tg = l >> 3, cq = l & 7;
    const int kc0 = w * (DK / 4) + cq * CPL;
    const int vc0 = w * (DV / 4) + cq * VPL;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = 8 * tg + t;
      if (i < clen) {
        const size_t row = (row_base + i) * H + h;
        r.g[t] = RawG<CPL>::load(g, row * DK + kc0);
        r.q[t] = RawVec<Io, CPL>::load(q, row * DK + kc0);
        r.k[t] = RawVec<Io, CPL>::load(k, row * DK + kc0);
        r.v[t] = RawVec<Io, VPL>::load(v, row * DV + vc0);
      } else {
        r.g[t] = RG{};
        r.q[t] = RK{};
        r.k[t] = RK{};
        r.v[t] = RV{};
      }
    }
    // lane l fetches beta of token l
    r.beta = (l < clen) ? beta[(row_base + l) * H + h] : 0.f;
  }

  // N contiguous LDS elements written as one vector store
  template <int N>
  static __device__ __forceinline__ void st_vec(T* p, const T (&x)[N]) {
    typedef T vec __attribute__((ext_vector_type(N)));
    vec v;
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = x[c];
    *lds_ptr<vec>(p) = v;
  }

  // ---------------------------------------------------------------- prep
  // Cumulative decay and the five gate-scaled operands; returns the chunk's
  // guard flag (1 = some channel decays below KDA_GAMMA_MIN).
  static __device__ __forceinline__ int prep(const Raw& r, char* smem, float scale) {
    const int w = threadIdx.x >> 6, l = lane_id();
    const int tg = l >> 3, cq = l & 7;
    const int kc0 = w * (DK / 4) + cq * CPL;
    const int vc0 = w * (DV / 4) + cq * VPL;
    T* QG = reinterpret_cast<T*>(smem + Cfg::OFF_QG);
    T* KG = reinterpret_cast<T*>(smem + Cfg::OFF_KG);
    T* KI = reinterpret_cast<T*>(smem + Cfg::OFF_KI);
    T* KE = reinterpret_cast<T*>(smem + Cfg::OFF_KE);
    T* BV = reinterpret_cast<T*>(smem + Cfg::OFF_BV);
    float* GL = reinterpret_cast<float*>(smem + Cfg::OFF_GL);

    // in-lane running products of alpha over the lane's 8 tokens
    float cp[8][CPL];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float gv[CPL];
      RawG<CPL>::unpack(r.g[t], gv);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float a = __expf(gv[c]);
        cp[t][c] = (t == 0) ? a : cp[t - 1][c] * a;
      }
    }
    // exclusive product over the 8 token groups (lanes cq + 8 tg)
    float ex[CPL], tot[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float x = cp[7][c];
#pragma unroll
      for (int d = 8; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d);
        if (l >= d) x *= y;
      }
      tot[c] = __shfl(x, 56 + cq);          // Gamma_L
      const float y = __shfl_up(x, 8);
      ex[c] = (l >= 8) ? y : 1.f;
    }
    int bad = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) bad |= !(tot[c] >= KDA_GAMMA_MIN);
    if (tg == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) GL[kc0 + c] = tot[c];
    }
    // betas of this lane's tokens
    float bt[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) bt[t] = __shfl(r.beta, 8 * tg + t);

#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = 8 * tg + t;
      float qv[CPL], kv[CPL];
      RawVec<Io, CPL>::unpack(r.q[t], qv);
      RawVec<Io, CPL>::unpack(r.k[t], kv);
      T qg[CPL], kg[CPL], ki[CPL], ke[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float gam = ex[c] * cp[t][c];
        const float inv = __builtin_amdgcn_rcpf(gam);
        qg[c] = Op::cvt(scale * qv[c] * gam);
        kg[c] = Op::cvt(bt[t] * kv[c] * gam);
        ki[c] = Op::cvt(kv[c] * inv);
        ke[c] = Op::cvt(kv[c] * (tot[c] * inv));
      }
      st_vec(QG + i * Cfg::LD_K + kc0, qg);
      st_vec(KG + i * Cfg::LD_K + kc0, kg);
      st_vec(KI + i * Cfg::LD_K + kc0, ki);
      st_vec(KE + i * Cfg::LD_E + kc0, ke);
      float vv[VPL];
      RawVec<Io, VPL>::unpack(r.v[t], vv);
      T bv[VPL];
#pragma unroll
      for (int c = 0; c < VPL; ++c) bv[c] = Op::cvt(bt[t] * vv[c]);
      st_vec(BV + i * Cfg::LD_V + vc0, bv);
    }
    return bad;
  }

  // ---------------------------------------------------------------- phase A
  // R = strict_tril(KG KI^T) and Aqk = tril(QG KI^T) by 16x16 tiles.
  // Off-diagonal R tiles go negated and transposed to RTn (bf16/f32), diagonal
  // R tiles to RD (fp32, transposed) for the inverse, Aqk transposed to AQT.
  static __device__ __forceinline__ void tile_qk(char* smem, int I, int J) {
    const T* QG = reinterpret_cast<const T*>(smem + Cfg::OFF_QG);
    const T* KG = reinterpret_cast<const T*>(smem + Cfg::OFF_KG);
    const T* KI = reinterpret_cast<const T*>(smem + Cfg::OFF_KI);
    T* RTn = reinterpret_cast<T*>(smem + Cfg::OFF_RT);
    T* AQT = reinterpret_cast<T*>(smem + Cfg::OFF_AQ);
    float* RD = reinterpret_cast<float*>(smem + Cfg::OFF_RD);
    f32x4 accR = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const typename Op::F32 b = Op::ld32_rm(KI, Cfg::LD_K, 16 * J, 32 * ks);
      const typename Op::F32 ak = Op::ld32_rm(KG, Cfg::LD_K, 16 * I, 32 * ks);
      const typename Op::F32 aq = Op::ld32_rm(QG, Cfg::LD_K, 16 * I, 32 * ks);
      accR = Op::mma32(ak, b, accR);
      accA = Op::mma32(aq, b, accA);
    }
    const int l = lane_id();
    const int n = l & 15, g4 = 4 * (l >> 4);
    if (I == J) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!(n < g4 + r)) accR[r] = 0.f;    // strictly lower
        if (!(n <= g4 + r)) accA[r] = 0.f;   // lower with diagonal
      }
      // RD[I][m][i] = R[16I + i][16I + m]  (column m of the block, contiguous over i)
      *lds_ptr<f32x4>(RD + I * 256 + n * 16 + g4) = accR;
    } else {
      Op::st_ct(RTn, Cfg::LD_64, 16 * J, 16 * I, -accR);
    }
    Op::st_ct(AQT, Cfg::LD_64, 16 * J, 16 * I, accA);
  }

  // ---------------------------------------------------------------- phase T
  // T_II = (I + R_II)^{-1} for block I = wave id, by column forward
  // substitution; lane l%16 = column.  Written transposed (TD[I][col][i]).
  static __device__ __forceinline__ void invert_diag(char* smem) {
    const int w = threadIdx.x >> 6, l = lane_id();
    const int col = l & 15;
    const float* RD = reinterpret_cast<const float*>(smem + Cfg::OFF_RD) + w * 256;
    T* TD = reinterpret_cast<T*>(smem + Cfg::OFF_TD) + w * 256;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
      const float xm = x[m];
      // column m of N: N[i][m] = RD[m][i]
#pragma unroll
      for (int i4 = (m + 1) / 4; i4 < 4; ++i4) {
        const f32x4 nv = *lds_ptr<const f32x4>(RD + m * 16 + 4 * i4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          if (i > m) x[i] -= nv[e] * xm;
        }
      }
    }
    if (l < 16) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 t = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
        *lds_ptr<typename Op::F16>(TD + col * 16 + 4 * i4) = Op::pack(t);
      }
    }
  }

  // ---------------------------------------------------------------- phase S1
  // Block forward substitution for this wave's W channels and U columns:
  //   Y_I = [KG | BV]_I - sum_{J<I} R_IJ X_J,  X_I = T_II Y_I.
  // The W part is written negated and transposed to WTn; U stays in registers.
  static __device__ __forceinline__ void wy_factors(char* smem, f32x4 (&U)[4][NVT]) {
    const int w = threadIdx.x >> 6;
    const T* KG = reinterpret_cast<const T*>(smem + Cfg::OFF_KG);
    const T* BV = reinterpret_cast<const T*>(smem + Cfg::OFF_BV);
    const T* RTn = reinterpret_cast<const T*>(smem + Cfg::OFF_RT);
    const T* TD = reinterpret_cast<const T*>(smem + Cfg::OFF_TD);
    T* WTn = reinterpret_cast<T*>(smem + Cfg::OFF_WT);
    const int cw0 = w * (DK / 4), vw0 = w * (DV / 4);
    f32x4 X[4][NT];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 Y[NT];
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) Y[nt] = Op::unpack(Op::ld16_tr(KG, Cfg::LD_K, 16 * I, cw0 + 16 * nt));
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
        Y[NKT + nt] = Op::unpack(Op::ld16_tr(BV, Cfg::LD_V, 16 * I, vw0 + 16 * nt));
#pragma unroll
      for (int J = 0; J < I; ++J) {
        // A[m = i][k = j] = -R[16I + m][16J + k] = RTn[16J + k][16I + m]
        const typename Op::F16 a = Op::ld16_tr(RTn, Cfg::LD_64, 16 * J, 16 * I);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Y[nt] = Op::mma16(a, Op::pack(X[J][nt]), Y[nt]);
      }
      // A[m = i][k = i'] = T_II[m][k] = TD[I][k][m]
      const typename Op::F16 a = Op::ld16_tr(TD + I * 256, 16, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        X[I][nt] = Op::mma16(a, Op::pack(Y[nt]), z);
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) Op::st_ct(WTn, Cfg::LD_64, cw0 + 16 * nt, 16 * I, -X[I][nt]);
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) U[I][nt] = X[I][NKT + nt];
    }
  }

  // ---------------------------------------------------------------- phase S2
  // E = U - W S, O = QG S + Aqk E, S <- Diag(Gamma_L) S + KE^T E.
  static __device__ __forceinline__ void scan_step(char* smem, f32x4 (&S)[MTK][NVT],
                                                   const f32x4 (&U)[4][NVT], void* out,
                                                   size_t row_base, int H, int h, int clen) {
    const int w = threadIdx.x >> 6, l = lane_id();
    const T* QG = reinterpret_cast<const T*>(smem + Cfg::OFF_QG);
    const T* KE = reinterpret_cast<const T*>(smem + Cfg::OFF_KE);
    const T* AQT = reinterpret_cast<const T*>(smem + Cfg::OFF_AQ);
    const T* WTn = reinterpret_cast<const T*>(smem + Cfg::OFF_WT);
    const float* GL = reinterpret_cast<const float*>(smem + Cfg::OFF_GL);
    const int vw0 = w * (DV / 4);

    // S as 32-deep B operands over key channels
    typename Op::F32 SB[NKS][NVT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
        SB[ks][nt] = typename Op::F32{Op::pack(S[2 * ks][nt]), Op::pack(S[2 * ks + 1][nt])};

    f32x4 E[4][NVT], O[4][NVT];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        E[I][nt] = U[I][nt];
        O[I][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename Op::F32 aw = Op::ld32_tr(WTn, Cfg::LD_64, 32 * ks, 16 * I);
        const typename Op::F32 aq = Op::ld32_rm(QG, Cfg::LD_K, 16 * I, 32 * ks);
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) {
          E[I][nt] = Op::mma32(aw, SB[ks][nt], E[I][nt]);
          O[I][nt] = Op::mma32(aq, SB[ks][nt], O[I][nt]);
        }
      }
    }
    // E as 32-deep B operands over tokens
    typename Op::F32 EB[2][NVT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
        EB[kt][nt] = typename Op::F32{Op::pack(E[2 * kt][nt]), Op::pack(E[2 * kt + 1][nt])};
    // causal in-chunk part of the outputs
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
      for (int kt = 0; kt <= I / 2; ++kt) {
        const typename Op::F32 a = Op::ld32_tr(AQT, Cfg::LD_64, 32 * kt, 16 * I);
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) O[I][nt] = Op::mma32(a, EB[kt][nt], O[I][nt]);
      }
    }
    // store outputs: rows i = 16I + 4g + r, column vw0 + 16nt + l%16
    const int n = l & 15, g4 = 4 * (l >> 4);
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + g4 + r;
        if (i < clen) {
          const size_t base = ((row_base + i) * H + h) * DV + vw0 + n;
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) Io::store(out, base + 16 * nt, O[I][nt][r]);
        }
      }
    // state update
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) {
      const f32x4 gl = *lds_ptr<const f32x4>(GL + 16 * mt + g4);
      typename Op::F32 a[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) a[kt] = Op::ld32_tr(KE, Cfg::LD_E, 32 * kt, 16 * mt);
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        f32x4 s = S[mt][nt] * gl;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s = Op::mma32(a[kt], EB[kt][nt], s);
        S[mt][nt] = s;
      }
    }
  }

  // ---------------------------------------------------------------- guard path
  // The recurrence itself, token by token, on the on-chip state (each wave its
  // own value columns; reductions over key rows stay inside the wave).
  static __device__ void recurrent_chunk(f32x4 (&S)[MTK][NVT], const void* q, const void* k,
                                         const void* v, const float* g, const float* beta,
                                         void* out, size_t row_base, int H, int h, int clen,
                                         float scale) {
    const int w = threadIdx.x >> 6, l = lane_id();
    const int n = l & 15, g4 = 4 * (l >> 4);
    const int vw0 = w * (DV / 4);
    for (int t = 0; t < clen; ++t) {
      const size_t row = (row_base + t) * H + h;
      float p[NVT], o[NVT];
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) p[nt] = 0.f;
      float kk[MTK][4], qq[MTK][4];
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt) {
        const size_t ci = row * DK + 16 * mt + g4;
        const f32x4 gv = *reinterpret_cast<const f32x4*>(g + ci);
        const f32x4 kv = Io::load4(k, ci);
        const f32x4 qv = Io::load4(q, ci);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = __expf(gv[r]);
          kk[mt][r] = kv[r];
          qq[mt][r] = scale * qv[r];
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) {
            S[mt][nt][r] *= a;
            p[nt] += S[mt][nt][r] * kv[r];
          }
        }
      }
      const float b = beta[row];
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        p[nt] += __shfl_xor(p[nt], 16);
        p[nt] += __shfl_xor(p[nt], 32);
        const float e = b * (Io::load(v, row * DV + vw0 + 16 * nt + n) - p[nt]);
        o[nt] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            S[mt][nt][r] += kk[mt][r] * e;
            o[nt] += S[mt][nt][r] * qq[mt][r];
          }
        o[nt] += __shfl_xor(o[nt], 16);
        o[nt] += __shfl_xor(o[nt], 32);
        if (l < 16) Io::store(out, row * DV + vw0 + 16 * nt + n, o[nt]);
      }
    }
  }

  // ---------------------------------------------------------------- driver
  static __device__ void run(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* S0, void* out, float* S_final,
                             size_t row_base, int len, int H, int h, size_t chain, float scale) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int w = threadIdx.x >> 6, l = lane_id();
    const int n = l & 15, g4 = 4 * (l >> 4);
    const int vw0 = w * (DV / 4);
    int* FL = reinterpret_cast<int*>(smem + Cfg::OFF_FL);

    // Aqk^T tiles above the diagonal are never written: zero the buffer once.
    {
      T* AQT = reinterpret_cast<T*>(smem + Cfg::OFF_AQ);
      for (int i = threadIdx.x; i < C * Cfg::LD_64; i += 256) AQT[i] = Op::cvt(0.f);
    }
    // state tiles: S[16mt + 4g + r][vw0 + 16nt + n]
    f32x4 S[MTK][NVT];
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[mt][nt][r] = S0 ? S0[(chain * DK + 16 * mt + g4 + r) * DV + vw0 + 16 * nt + n] : 0.f;

    Raw nxt;
    if (len > 0) load_raw(nxt, q, k, v, g, beta, row_base, H, h, len < C ? len : C);
    for (int c0 = 0; c0 < len; c0 += C) {
      const int clen = (len - c0) < C ? (len - c0) : C;
      Raw cur = nxt;
      if (c0 + C < len) {
        const int nlen = (len - c0 - C) < C ? (len - c0 - C) : C;
        load_raw(nxt, q, k, v, g, beta, row_base + c0 + C, H, h, nlen);
      }
      const int bad = prep(cur, smem, scale);
      const bool wave_bad = __any(bad);
      if (l == 0) FL[w] = wave_bad ? 1 : 0;
      __syncthreads();                                           // B1
      const bool guard = (FL[0] | FL[1] | FL[2] | FL[3]) != 0;
      if (!guard) {
        // balanced tile lists: 3, 3, 2, 2 tile pairs per wave
        if (w == 0) { tile_qk(smem, 0, 0); tile_qk(smem, 1, 0); tile_qk(smem, 1, 1); }
        if (w == 1) { tile_qk(smem, 2, 0); tile_qk(smem, 2, 1); tile_qk(smem, 2, 2); }
        if (w == 2) { tile_qk(smem, 3, 0); tile_qk(smem, 3, 1); }
        if (w == 3) { tile_qk(smem, 3, 2); tile_qk(smem, 3, 3); }
        __syncthreads();                                         // B2
        invert_diag(smem);
        __syncthreads();                                         // B3
        f32x4 U[4][NVT];
        wy_factors(smem, U);
        __syncthreads();                                         // B4
        scan_step(smem, S, U, out, row_base + c0, H, h, clen);
      } else {
        recurrent_chunk(S, q, k, v, g, beta, out, row_base + c0, H, h, clen, scale);
      }
      __syncthreads();                                           // LDS reuse
    }
    if (S_final) {
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S_final[(chain * DK + 16 * mt + g4 + r) * DV + vw0 + 16 * nt + n] = S[mt][nt][r];
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, int T, int H, float scale) {
  const int chain = blockIdx.x;   // b * H + h
  const int b = chain / H, h = chain % H;
  ChunkKernel<Cfg>::run(q, k, v, g, beta, S0, out, S_final, (size_t)b * T, T, H, h,
                        (size_t)chain, scale);
}

template <class Cfg>
__global__ __launch_bounds__(256, 1) void chunk_fwd_varlen_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, const int32_t* __restrict__ cu_seqlens, int H, float scale) {
  const int chain = blockIdx.x;   // n * H + h
  const int n = chain / H, h = chain % H;
  const int b0 = cu_seqlens[n], b1 = cu_seqlens[n + 1];
  ChunkKernel<Cfg>::run(q, k, v, g, beta, S0, out, S_final, (size_t)b0, b1 - b0, H, h,
                        (size_t)chain, scale);
}

template <class Cfg>
static hipError_t launch_chunk_t(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* S0, void* out, float* S_final,
                                 const int32_t* cu, int n_seq, int T, int H, float scale,
                                 hipStream_t stream) {
  const int bytes = Cfg::LDS_BYTES;
  if (cu) {
    auto kern = chunk_fwd_varlen_kernel<Cfg>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(256), bytes, stream, q, k, v, g, beta, S0, out,
                       S_final, cu, H, scale);
  } else {
    auto kern = chunk_fwd_kernel<Cfg>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(256), bytes, stream, q, k, v, g, beta, S0, out,
                       S_final, T, H, scale);
  }
  return hipGetLastError();
}

// Supported (d_k, d_v, io) combinations; fp32 I/O keeps fp32 operands and
// fits the LDS budget only for d_k = d_v = 64.
bool chunk_supported(int dk, int dv, bool bf16) {
  if (bf16) return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
  return dk == 64 && dv == 64;
}

hipError_t launch_chunk(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, void* out, float* S_final,
                        const int32_t* cu_seqlens, int n_seq, int T, int H, int dk, int dv,
                        float scale, bool bf16, hipStream_t stream) {
#define KDA_CH(DK, DV, IO, OP)                                                            \
  return launch_chunk_t<ChunkCfg<DK, DV, IO, OP>>(q, k, v, g, beta, S0, out, S_final,     \
                                                  cu_seqlens, n_seq, T, H, scale, stream);
  if (bf16) {
    if (dk == 128 && dv == 128) { KDA_CH(128, 128, IoBf16, OpBf16) }
    if (dk == 128 && dv == 64) { KDA_CH(128, 64, IoBf16, OpBf16) }
    if (dk == 64 && dv == 128) { KDA_CH(64, 128, IoBf16, OpBf16) }
    if (dk == 64 && dv == 64) { KDA_CH(64, 64, IoBf16, OpBf16) }
  } else {
    if (dk == 64 && dv == 64) { KDA_CH(64, 64, IoF32, OpF32) }
  }
#undef KDA_CH
  return hipErrorInvalidValue;
}

}  // namespace kda
